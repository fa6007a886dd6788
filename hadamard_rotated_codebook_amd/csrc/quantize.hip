// Encoder: fp32 [rows][cols] master -> CQ blob (OpenNeedle reference notes,
// CQ quantisation steps; bit packing per the file-layout note: every 8 codes
// form the word sum(code[i] << (i*b)), written as b little-endian bytes).
//
// Layout: 16 lanes own one (row, group); each lane holds 8 consecutive
// weights, i.e. exactly one 8-code word of the packed row.
//
// Numerics (fixed so that every decision is reproducible):
//   w . S is summed in double by the butterfly (exact for fp32 inputs that do
//   not span more than ~2^22 in magnitude), scaled by sqrt(1/128) in double and
//   rounded once to the fp32 coordinate r; the norm is the double norm of the
//   fp32 r rounded to fp32; u is the IEEE fp32 quotient (formed in double --
//   as r times the group's double reciprocal, see below -- and rounded once,
//   which is exact rounding for fp32 operands); the nearest level
//   is decided by exact comparison against the midpoints of adjacent levels,
//   ties to the smaller index; the stored norm is fp16, round to nearest even.
//   The comparison runs as a bucket lookup (cq::EncodeTable: one fp32
//   threshold per bucket, compared by order keys of the bit patterns, the
//   same decisions) or, for code books whose thresholds are too close for
//   the buckets, as a count of the midpoints.
// The 16 lanes of a group exchange values with DPP (two 32-bit moves per
// double), not through LDS.
#include "cq_fwht.h"
#include "cq_internal.h"

namespace {

constexpr double kSqrtInv128 = 0.08838834764831845;  // sqrt(1/128) in double

// The double of lane j ^ D within each 16-lane row, both halves moved by DPP.
template <int D>
__device__ inline double xor_lane_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __float_as_uint(cqdev::xor_lane<D>(__uint_as_float(static_cast<uint32_t>(b))));
  const uint32_t hi = __float_as_uint(cqdev::xor_lane<D>(__uint_as_float(static_cast<uint32_t>(b >> 32))));
  return __builtin_bit_cast(double, static_cast<uint64_t>(hi) << 32 | lo);
}
// -v for the upper lane of a pair (sign flip, exact), v otherwise
__device__ inline double signed_f64(double v, bool upper) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v) ^ (upper ? 0x8000000000000000ull : 0ull);
  return __builtin_bit_cast(double, b);
}
template <int D>
__device__ inline void lane_stage_f64(double (&t)[8], int j) {
  const bool upper = (j & D) != 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = xor_lane_f64<D>(t[i]) + signed_f64(t[i], upper);
}

// packed: the first output row's codes (rows of kpad * SB / 8 bytes follow);
// norms: its fp16 norms (rows of kpad / 128 follow) -- the rows of a whole
// blob, or a row range of a larger one.
template <int SB, bool VEC, bool LUT>
__global__ __launch_bounds__(256) void quantize_kernel(const float *__restrict__ w, int64_t rows,
                                                      int64_t cols, int64_t kpad, cq::EncodeTable tab,
                                                      uint8_t *__restrict__ packed, uint16_t *__restrict__ norms) {
  __shared__ int32_t lut_key[cq::kLutBuckets];
  __shared__ int32_t lut_base[cq::kLutBuckets];
  if constexpr (LUT) {
    if (threadIdx.x < cq::kLutBuckets) {
      lut_key[threadIdx.x] = tab.lut_key[threadIdx.x];
      lut_base[threadIdx.x] = tab.lut_base[threadIdx.x];
    }
    __syncthreads();
  }
  const int64_t ngroups = kpad / CQ_GROUP;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  const bool valid = gid < rows * ngroups;
  const int64_t r = valid ? gid / ngroups : 0;
  const int64_t g = valid ? gid - r * ngroups : 0;
  const int64_t col0 = g * CQ_GROUP + j * 8;

  double t[8];
  const float *src = w + r * cols + col0;
  if (VEC && valid && col0 + 8 <= cols) {
    const float4 a = reinterpret_cast<const float4 *>(src)[0];
    const float4 b = reinterpret_cast<const float4 *>(src)[1];
    t[0] = a.x; t[1] = a.y; t[2] = a.z; t[3] = a.w;
    t[4] = b.x; t[5] = b.y; t[6] = b.z; t[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = (valid && col0 + i < cols) ? static_cast<double>(src[i]) : 0.0;
  }

  // Unnormalised Walsh-Hadamard butterfly (natural Sylvester order).
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
      const double a = t[i], c = t[i + h];
      t[i] = a + c;
      t[i + h] = a - c;
    }
  }
  lane_stage_f64<1>(t, j);
  lane_stage_f64<2>(t, j);
  lane_stage_f64<4>(t, j);
  lane_stage_f64<8>(t, j);

  float r32[8];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    r32[i] = static_cast<float>(t[i] * kSqrtInv128);
    const double rd = static_cast<double>(r32[i]);
    ss += rd * rd;  // each square is exact in double
  }
  ss += xor_lane_f64<1>(ss);
  ss += xor_lane_f64<2>(ss);
  ss += xor_lane_f64<4>(ss);
  ss += xor_lane_f64<8>(ss);
  const float n32 = static_cast<float>(sqrt(ss));
  const double den = static_cast<double>(fmaxf(n32, 1e-12f));

  // u = fp32(r / den): r * (1 / den) in double rounds to the same fp32.  The
  // double product is within ~2^-52 of the quotient, and a quotient of two
  // fp32 values lies at least ~2^-49 (relative) from an fp32 rounding
  // boundary unless it is exactly one -- impossible for a normal result (it
  // would need 25 significant bits in r), possible among subnormal results,
  // so a wave with such a quotient divides exactly.
  const double inv = 1.0 / den;
  float uq[8];
  bool sub = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double ud = static_cast<double>(r32[i]) * inv;
    uq[i] = static_cast<float>(ud);
    sub |= ud != 0.0 && fabs(ud) < 1.1754943508222875e-38;  // below the smallest normal fp32
  }
  if (__builtin_amdgcn_ballot_w64(sub) != 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) uq[i] = static_cast<float>(static_cast<double>(r32[i]) / den);
  }

  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float u32 = uq[i];
    int q = 0;
    if constexpr (LUT) {
      const float x = fminf(fmaxf(u32 * tab.lut_scale, -1e6f), 1e6f);
      const int b = min(max(static_cast<int>(floorf(x)) + tab.lut_off, 0), cq::kLutBuckets - 1);
      q = lut_base[b] + (cq::float_key(__float_as_uint(u32)) >= lut_key[b] ? 1 : 0);
      q = u32 == u32 ? q : 0;  // NaN: no midpoint is below it
    } else {
      const double u = static_cast<double>(u32);
      for (int m = 0; m + 1 < tab.nlevels; ++m) q += (u > tab.mid[m]) ? 1 : 0;
    }
    word |= tab.code_of_index[q] << (i * SB);
  }
  if (!valid) return;

  const int64_t row_bytes = kpad * SB / 8;
  uint8_t *dst = packed + r * row_bytes + g * (16 * SB) + j * SB;
  if (SB == 1) {
    dst[0] = static_cast<uint8_t>(word);
  } else if (SB == 2) {
    *reinterpret_cast<uint16_t *>(dst) = static_cast<uint16_t>(word);
  } else if (SB == 4) {
    *reinterpret_cast<uint32_t *>(dst) = word;
  } else {
    dst[0] = static_cast<uint8_t>(word);
    dst[1] = static_cast<uint8_t>(word >> 8);
    dst[2] = static_cast<uint8_t>(word >> 16);
  }
  if (j == 0) norms[r * ngroups + g] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(n32));
}

template <int SB>
hipError_t launch_sb(const float *w, int64_t rows, int64_t cols, int64_t kpad, const cq::EncodeTable &tab,
                     uint8_t *packed, uint16_t *norms, hipStream_t s) {
  const int64_t groups = rows * (kpad / CQ_GROUP);
  const int64_t blocks = (groups + 15) / 16;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const bool vec = (cols % 4 == 0) && ((reinterpret_cast<uintptr_t>(w) & 15) == 0);
  const dim3 grid(static_cast<unsigned>(blocks));
  if (tab.lut) {
    if (vec)
      quantize_kernel<SB, true, true><<<grid, 256, 0, s>>>(w, rows, cols, kpad, tab, packed, norms);
    else
      quantize_kernel<SB, false, true><<<grid, 256, 0, s>>>(w, rows, cols, kpad, tab, packed, norms);
  } else {
    if (vec)
      quantize_kernel<SB, true, false><<<grid, 256, 0, s>>>(w, rows, cols, kpad, tab, packed, norms);
    else
      quantize_kernel<SB, false, false><<<grid, 256, 0, s>>>(w, rows, cols, kpad, tab, packed, norms);
  }
  return hipGetLastError();
}

}  // namespace

namespace cq {

hipError_t launch_quantize(const float *w, int64_t rows, int64_t cols, int64_t kpad, int bits,
                           const EncodeTable &tab, uint8_t *packed, uint16_t *norms, hipStream_t s) {
  switch (storage_bits(bits)) {
    case 1: return launch_sb<1>(w, rows, cols, kpad, tab, packed, norms, s);
    case 2: return launch_sb<2>(w, rows, cols, kpad, tab, packed, norms, s);
    case 3: return launch_sb<3>(w, rows, cols, kpad, tab, packed, norms, s);
    default: return launch_sb<4>(w, rows, cols, kpad, tab, packed, norms, s);
  }
}

}  // namespace cq
