// Activation rotation: xr_g = H . x_g for every 128-group of every row, with
// H = S/sqrt(128) and S the Sylvester-Hadamard matrix ("cact-format" post,
// "How the kernel reads it": a fast Walsh-Hadamard butterfly per 128-lane
// group, computed once and shared by all output rows).
//
// Layout: 16 lanes own one group, each lane holds 8 consecutive elements, so a
// 64-lane wave rotates 4 groups (the butterfly is cq_fwht.h's, shared with the
// products that rotate their own activations).  Memory-bound: one read of x
// and one write of xr.
#include "cq_fwht.h"
#include "cq_internal.h"

namespace {

using cqdev::kInvSqrt128;

__device__ inline float load_elem(const float *p) { return *p; }
__device__ inline float load_elem(const _Float16 *p) { return static_cast<float>(*p); }
__device__ inline float load_elem(const uint16_t *p) {  // bf16 bits
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

__device__ inline void load8_vec(const float *p, float v[8]) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0];
  const float4 b = reinterpret_cast<const float4 *>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ inline void load8_vec(const _Float16 *p, float v[8]) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const h8 a = *reinterpret_cast<const h8 *>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = static_cast<float>(a[i]);
}
__device__ inline void load8_vec(const uint16_t *p, float v[8]) {
  const uint4 a = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Round to nearest even bf16 (NaN stays NaN).
__device__ inline uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

template <typename TIn, bool VEC, bool OUT_BF16>
__global__ __launch_bounds__(256) void rotate_kernel(const TIn *__restrict__ x, int64_t batch,
                                                    int64_t cols, int64_t kpad, void *__restrict__ xr) {
  const int64_t ngroups = kpad / CQ_GROUP;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  const bool valid = gid < batch * ngroups;  // all lanes take part in the exchanges
  const int64_t b = valid ? gid / ngroups : 0;
  const int64_t col0 = valid ? (gid - b * ngroups) * CQ_GROUP + j * 8 : 0;

  float v[8];
  const TIn *src = x + b * cols + col0;
  if (VEC && valid && col0 + 8 <= cols) {
    load8_vec(src, v);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (valid && col0 + i < cols) ? load_elem(src + i) : 0.0f;
  }

  cqdev::fwht128_unscaled(v, j);
  if (!valid) return;
  const int64_t out = b * kpad + col0;
  if (OUT_BF16) {
    uint4 o;
    o.x = bf16_bits(v[0] * kInvSqrt128) | (bf16_bits(v[1] * kInvSqrt128) << 16);
    o.y = bf16_bits(v[2] * kInvSqrt128) | (bf16_bits(v[3] * kInvSqrt128) << 16);
    o.z = bf16_bits(v[4] * kInvSqrt128) | (bf16_bits(v[5] * kInvSqrt128) << 16);
    o.w = bf16_bits(v[6] * kInvSqrt128) | (bf16_bits(v[7] * kInvSqrt128) << 16);
    reinterpret_cast<uint4 *>(static_cast<uint16_t *>(xr) + out)[0] = o;
  } else {
    float4 *dst = reinterpret_cast<float4 *>(static_cast<float *>(xr) + out);
    dst[0] = make_float4(v[0] * kInvSqrt128, v[1] * kInvSqrt128, v[2] * kInvSqrt128, v[3] * kInvSqrt128);
    dst[1] = make_float4(v[4] * kInvSqrt128, v[5] * kInvSqrt128, v[6] * kInvSqrt128, v[7] * kInvSqrt128);
  }
}

template <typename TIn, bool OUT_BF16>
hipError_t launch_typed(const void *x, int64_t batch, int64_t cols, int64_t kpad, void *xr, bool vec,
                        hipStream_t s) {
  const int64_t groups = batch * (kpad / CQ_GROUP);
  const int64_t blocks = (groups + 15) / 16;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  const TIn *xp = static_cast<const TIn *>(x);
  if (vec)
    rotate_kernel<TIn, true, OUT_BF16><<<grid, 256, 0, s>>>(xp, batch, cols, kpad, xr);
  else
    rotate_kernel<TIn, false, OUT_BF16><<<grid, 256, 0, s>>>(xp, batch, cols, kpad, xr);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_kernel(float *__restrict__ p, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) p[i] = 0.0f;
}

}  // namespace

namespace cq {

hipError_t launch_rotate(const void *x, int x_dtype, int64_t batch, int64_t cols, int64_t kpad, void *xr,
                         int xr_dtype, hipStream_t s) {
  // Vector loads need every group's 8-element run to be contiguous and aligned.
  const size_t esz = x_dtype == CQ_F32 ? 4 : 2;
  const bool vec = (cols % 8 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0) && (esz * 8 >= 16);
  const bool bf = xr_dtype == CQ_BF16;
  switch (x_dtype) {
    case CQ_F32:
      return bf ? launch_typed<float, true>(x, batch, cols, kpad, xr, vec, s)
                : launch_typed<float, false>(x, batch, cols, kpad, xr, vec, s);
    case CQ_F16:
      return bf ? launch_typed<_Float16, true>(x, batch, cols, kpad, xr, vec, s)
                : launch_typed<_Float16, false>(x, batch, cols, kpad, xr, vec, s);
    default:
      return bf ? launch_typed<uint16_t, true>(x, batch, cols, kpad, xr, vec, s)
                : launch_typed<uint16_t, false>(x, batch, cols, kpad, xr, vec, s);
  }
}

hipError_t launch_zero_f32(float *p, int64_t n, hipStream_t s) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const dim3 grid(static_cast<unsigned>(blocks));
  zero_kernel<<<grid, 256, 0, s>>>(p, n);
  return hipGetLastError();
}

}  // namespace cq
