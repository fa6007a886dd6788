// Row gather: the dense reconstruction of the indexed rows only,
//
//   out[i][k] = w_hat[ids[i]][k],  w_hat group = (c[q] * float(norm)) . H
//
// (needle.js tutorial, "Reconstructing one group": a row gather, for
// embeddings and engram tables, reconstructs the dense group; "Keep the
// quantized views": dequantise only the rows you need; OpenNeedle reference
// notes, engine notes: embedding and engram lookups decode only the indexed
// rows).
//
// Sixteen lanes own one (gathered row, group), 8 consecutive codes per lane:
// the codes are looked up in an LDS copy of the level table, scaled by the
// fp32 norm, and rotated back with the butterfly every rotating kernel uses
// (H is its own inverse).  An id outside [0, rows) gives a row of NaN; a
// valid id never reads outside its row.
#include <type_traits>

#include "cq_decode.h"
#include "cq_fwht.h"
#include "cq_internal.h"

namespace {

using namespace cqdev;

constexpr int kThreads = 256;  // 16 (row, group) tasks

struct GArgs {
  const uint8_t *packed;
  const uint16_t *norms;  // fp16 bits [rows][ngroups]
  const int64_t *ids;     // [n]
  void *out;              // [n][cols] of the output type
  int64_t rows, cols, n, row_bytes, ngroups;
  int32_t vec;            // out rows allow 16-byte stores of 8 elements
  cq::CodeLevels lev;
};

// OUT: 0 fp32, 1 fp16, 2 bf16 (the cq_dtype values).
template <int SB, int OUT>
__global__ __launch_bounds__(kThreads) void gather_kernel(GArgs a) {
  __shared__ float lev[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (static_cast<int>(threadIdx.x) == i) lev[i] = a.lev.v[i];
  __syncthreads();

  const int64_t task = static_cast<int64_t>(blockIdx.x) * (kThreads / 16) + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  const bool valid = task < a.n * a.ngroups;  // every lane runs the exchanges
  const int64_t i = valid ? task / a.ngroups : 0;
  const int64_t g = valid ? task - i * a.ngroups : 0;
  const int64_t id = valid ? a.ids[i] : 0;
  const bool ok = valid && id >= 0 && id < a.rows;

  // codes 8j..8j+7 of the group: 8 * SB bits at byte (16 g + j) * SB of the
  // row, read as two aligned dwords of a buffer over the row (bytes past the
  // row read zero)
  const __amdgpu_buffer_rsrc_t rb =
      buffer_rsrc(a.packed + (ok ? id : 0) * a.row_bytes, ok ? static_cast<uint32_t>(a.row_bytes) : 0u);
  const uint32_t off = static_cast<uint32_t>((16 * g + j) * SB);
  const uint32_t d0 = __builtin_amdgcn_raw_buffer_load_b32(rb, off & ~3u, 0, 0);
  const uint32_t d1 = __builtin_amdgcn_raw_buffer_load_b32(rb, (off & ~3u) + 4, 0, 0);
  const uint32_t f = __builtin_amdgcn_alignbit(d1, d0, (off & 3u) * 8);
  const __amdgpu_buffer_rsrc_t nb =
      buffer_rsrc(a.norms + (ok ? id : 0) * a.ngroups, ok ? static_cast<uint32_t>(a.ngroups * 2) : 0u);
  const uint16_t nraw = __builtin_amdgcn_raw_buffer_load_b16(nb, static_cast<uint32_t>(g * 2), 0, 0);
  const float nrm = static_cast<float>(__builtin_bit_cast(_Float16, nraw));

  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = lev[(f >> (SB * e)) & ((1u << SB) - 1)] * nrm;
  fwht128_unscaled(v, j);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = ok ? v[e] * kInvSqrt128 : __builtin_nanf("");
  if (!valid) return;

  const int64_t col0 = g * CQ_GROUP + 8 * j;
  const int64_t base = i * a.cols + col0;
  if constexpr (OUT == CQ_F32) {
    float *o = static_cast<float *>(a.out) + base;
    if (a.vec && col0 + 8 <= a.cols) {
      reinterpret_cast<float4 *>(o)[0] = make_float4(v[0], v[1], v[2], v[3]);
      reinterpret_cast<float4 *>(o)[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col0 + e < a.cols) o[e] = v[e];
    }
  } else {
    typedef typename std::conditional<OUT == CQ_F16, _Float16, __bf16>::type T;
    T *o = static_cast<T *>(a.out) + base;
    if (a.vec && col0 + 8 <= a.cols) {
      uint32_t w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const T lo = static_cast<T>(v[2 * t]), hi = static_cast<T>(v[2 * t + 1]);
        w[t] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
      }
      *reinterpret_cast<uint4 *>(o) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col0 + e < a.cols) o[e] = static_cast<T>(v[e]);
    }
  }
}

typedef void (*GKernel)(GArgs);

template <int OUT>
GKernel pick_sb(int sb) {
  return sb == 1 ? gather_kernel<1, OUT>
                 : (sb == 2 ? gather_kernel<2, OUT> : (sb == 3 ? gather_kernel<3, OUT> : gather_kernel<4, OUT>));
}

}  // namespace

namespace cq {

hipError_t launch_gather(const uint8_t *blob, int bits, int64_t rows, int64_t cols, int64_t kpad,
                         const CodeLevels &lev, const int64_t *ids, int64_t n, void *out, int out_dtype,
                         hipStream_t s) {
  const int sb = storage_bits(bits);
  GArgs a;
  a.packed = blob;
  a.row_bytes = kpad * sb / 8;
  a.norms = reinterpret_cast<const uint16_t *>(blob + rows * a.row_bytes);
  a.ids = ids;
  a.out = out;
  a.rows = rows;
  a.cols = cols;
  a.n = n;
  a.ngroups = kpad / CQ_GROUP;
  const int esize = out_dtype == CQ_F32 ? 4 : 2;
  a.vec = (cols * esize) % 16 == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  a.lev = lev;
  // 32-bit offsets within a row; row_bytes < 2^31 for any valid shape
  if (a.row_bytes >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  const int64_t tasks = n * a.ngroups;
  const int64_t wgs = (tasks + kThreads / 16 - 1) / (kThreads / 16);
  if (wgs >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  const GKernel k = out_dtype == CQ_F32 ? pick_sb<CQ_F32>(sb) : (out_dtype == CQ_F16 ? pick_sb<CQ_F16>(sb) : pick_sb<CQ_BF16>(sb));
  k<<<dim3(static_cast<unsigned>(wgs)), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace cq
