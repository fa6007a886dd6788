// Encoder: fp32 [rows][cols] master -> CQ blob (OpenNeedle reference notes,
// CQ quantisation steps; bit packing per the file-layout note: every 8 codes
// form the word sum(code[i] << (i*b)), written as b little-endian bytes).
//
// Layout: 4 lanes own one (row, group); lane j holds the 32 consecutive
// weights 32j .. 32j+31, i.e. four 8-code words of the packed row, which it
// stores with one 4-, 8-, 12- or 16-byte write.  Five of the seven butterfly
// stages stay in the lane, two cross lanes (quad DPP).
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
//   The comparison runs as a bucket lookup (cq::EncodeTable: at most one
//   fp32 threshold per bucket, the same decisions) or, for binary, ternary
//   and code books whose thresholds are too close for the buckets, as a
//   count of the midpoints.
#include <algorithm>

#include "cq_fwht.h"
#include "cq_internal.h"

namespace {

constexpr double kSqrtInv128 = 0.08838834764831845;  // sqrt(1/128) in double
constexpr int kLanes = 4;                            // lanes per group
constexpr int kPer = CQ_GROUP / kLanes;              // weights per lane
constexpr int kThreads = 256;
constexpr int kGroupsPerBlock = kThreads / kLanes;

// The double of lane j ^ D (D = 1 or 2) within each quad, both halves moved by DPP.
template <int D>
__device__ inline double xor_lane_f64(double v) {
  static_assert(D == 1 || D == 2, "quad exchanges only");
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __float_as_uint(cqdev::xor_lane<D>(__uint_as_float(static_cast<uint32_t>(b))));
  const uint32_t hi = __float_as_uint(cqdev::xor_lane<D>(__uint_as_float(static_cast<uint32_t>(b >> 32))));
  return __builtin_bit_cast(double, static_cast<uint64_t>(hi) << 32 | lo);
}

// Butterfly stage across lanes at distance D: the lower lane of a pair keeps
// partner + self, the upper one partner - self, as one fused multiply-add by
// +-1 (rounded once, the same as the add).
template <int D>
__device__ inline void lane_stage_f64(double (&t)[kPer], int j) {
  const double sgn = (j & D) ? -1.0 : 1.0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) t[i] = __builtin_fma(t[i], sgn, xor_lane_f64<D>(t[i]));
}

// Job blockIdx.y of one launch (a launch may encode two matrices' rows with
// one code book, e.g. a new key and value row of a KV cache): job.packed is the first output
// row's codes (rows of kpad * SB / 8 bytes follow), job.norms its fp16 norms
// (rows of kpad / 128 follow) -- the rows of a whole blob, or a row range of
// a larger one.  16-byte aligned (blob layout).
// Both jobs use the one code book of `tab` (a by-value table chosen per
// block would be copied to scratch).
template <int SB, bool VEC, bool LUT>
__global__ __launch_bounds__(kThreads) void quantize_kernel(cq::QuantizeJob j0, cq::QuantizeJob j1,
                                                           cq::EncodeTable tab) {
  const bool second = blockIdx.y != 0;
  const float *__restrict__ w = second ? j1.w : j0.w;
  const int64_t rows = second ? j1.rows : j0.rows, cols = second ? j1.cols : j0.cols;
  const int64_t kpad = second ? j1.kpad : j0.kpad;
  uint8_t *__restrict__ packed = second ? j1.packed : j0.packed;
  uint16_t *__restrict__ norms = second ? j1.norms : j0.norms;
  __shared__ float lut_thr[cq::kLutBuckets];
  __shared__ int32_t lut_base[cq::kLutBuckets];
  if constexpr (LUT) {
    if (threadIdx.x < cq::kLutBuckets) {
      lut_thr[threadIdx.x] = tab.lut_thr[threadIdx.x];
      lut_base[threadIdx.x] = tab.lut_base[threadIdx.x];
    }
    __syncthreads();
  }
  const int64_t ngroups = kpad / CQ_GROUP;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kGroupsPerBlock + (threadIdx.x / kLanes);
  const int j = threadIdx.x % kLanes;
  const bool valid = gid < rows * ngroups;
  const int64_t r = valid ? gid / ngroups : 0;
  const int64_t g = valid ? gid - r * ngroups : 0;
  const int64_t col0 = g * CQ_GROUP + j * kPer;

  double t[kPer];
  const float *src = w + r * cols + col0;
  if (VEC && valid && col0 + kPer <= cols) {
#pragma unroll
    for (int c = 0; c < kPer / 4; ++c) {
      const float4 a = reinterpret_cast<const float4 *>(src)[c];
      t[4 * c] = a.x; t[4 * c + 1] = a.y; t[4 * c + 2] = a.z; t[4 * c + 3] = a.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i) t[i] = (valid && col0 + i < cols) ? static_cast<double>(src[i]) : 0.0;
  }

  // Unnormalised Walsh-Hadamard butterfly (natural Sylvester order): index
  // bits 0..4 within the lane, bits 5..6 across the quad.
#pragma unroll
  for (int h = 1; h < kPer; h <<= 1) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (i & h) continue;
      const double a = t[i], c = t[i + h];
      t[i] = a + c;
      t[i + h] = a - c;
    }
  }
  lane_stage_f64<1>(t, j);
  lane_stage_f64<2>(t, j);

  float r32[kPer];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    r32[i] = static_cast<float>(t[i] * kSqrtInv128);
    const double rd = static_cast<double>(r32[i]);
    ss += rd * rd;  // each square is exact in double
  }
  ss += xor_lane_f64<1>(ss);
  ss += xor_lane_f64<2>(ss);
  const float n32 = static_cast<float>(sqrt(ss));
  const double den = static_cast<double>(fmaxf(n32, 1e-12f));

  // u = fp32(r / den): r * (1 / den) in double rounds to the same fp32.  The
  // double product is within ~2^-52 of the quotient, and a quotient of two
  // fp32 values lies at least ~2^-49 (relative) from an fp32 rounding
  // boundary unless it is exactly one -- impossible for a normal result (it
  // would need 25 significant bits in r), possible among subnormal results.
  // Those matter only to a code book with a threshold near zero (counted
  // midpoints: binary's is zero), so there a wave with a subnormal or zero
  // quotient in a non-zero group divides exactly.
  const double inv = 1.0 / den;
  float uq[kPer];
  bool sub = false;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    uq[i] = static_cast<float>(static_cast<double>(r32[i]) * inv);
    if constexpr (!LUT) sub |= __builtin_amdgcn_classf(uq[i], 0xf0);  // -subnormal, -0, +0, +subnormal
  }
  if (!LUT && __builtin_amdgcn_ballot_w64(sub && ss != 0.0) != 0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) uq[i] = static_cast<float>(static_cast<double>(r32[i]) / den);
  }

  // The nearest level index of each u, stored as its code; a non-finite
  // group (ss NaN or +inf, the only way a u can be NaN) also maps NaN to
  // index 0: no midpoint is below it.
  uint32_t word[SB] = {};
  auto decide = [&](auto nan_c, auto ident_c) {
    constexpr bool NAN_CHECK = decltype(nan_c)::value;
    constexpr bool IDENT = decltype(ident_c)::value;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const float u32 = uq[i];
      uint32_t q;
      if constexpr (LUT) {
        const int32_t yb = __float_as_int(__builtin_fmaf(u32, tab.lut_scale, tab.lut_bias));
        const int b = min(max(yb, cq::kLutMagicBits), cq::kLutMagicBits + cq::kLutBuckets - 1) - cq::kLutMagicBits;
        q = static_cast<uint32_t>(lut_base[b]) + (u32 >= lut_thr[b] ? 1u : 0u);
        if constexpr (NAN_CHECK) q = u32 == u32 ? q : 0u;
      } else {  // NaN compares false: index 0 by itself
        const double u = static_cast<double>(u32);
        q = 0;
        for (int m = 0; m + 1 < tab.nlevels; ++m) q += (u > tab.mid[m]) ? 1u : 0u;
        if constexpr (!IDENT) q = __builtin_amdgcn_perm(0u, tab.code_bytes, 0x0c0c0c00u | q);
      }
      const int bit = i * SB, wd = bit / 32, sh = bit % 32;
      word[wd] |= q << sh;
      if (sh + SB > 32) word[wd + 1] |= q >> (32 - sh);
    }
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  if constexpr (LUT) {  // (codes are level indices whenever the lookup is used)
    if (__builtin_amdgcn_ballot_w64(!(ss <= 1.7976931348623157e308)) != 0)
      decide(yes(), yes());
    else
      decide(no(), yes());
  } else if (tab.code_ident) {
    decide(no(), yes());
  } else {
    decide(no(), no());
  }
  if (!valid) return;

  // Lane j's 32 codes: bytes 4 j SB .. of the group's 16 SB bytes.
  uint8_t *dst = packed + r * (kpad * SB / 8) + g * (16 * SB) + j * (4 * SB);
  if constexpr (SB == 4) {
    *reinterpret_cast<uint4 *>(dst) = make_uint4(word[0], word[1], word[2], word[3]);
  } else if constexpr (SB == 3) {
    uint32_t *d = reinterpret_cast<uint32_t *>(dst);
    d[0] = word[0];
    d[1] = word[1];
    d[2] = word[2];
  } else if constexpr (SB == 2) {
    *reinterpret_cast<uint2 *>(dst) = make_uint2(word[0], word[1]);
  } else {
    *reinterpret_cast<uint32_t *>(dst) = word[0];
  }
  if (j == 0) norms[r * ngroups + g] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(n32));
}

template <int SB>
hipError_t launch_sb(const cq::QuantizeJob &a, const cq::QuantizeJob *b, const cq::EncodeTable &tab, hipStream_t s) {
  auto blocks_of = [](const cq::QuantizeJob &j) {
    return (j.rows * (j.kpad / CQ_GROUP) + kGroupsPerBlock - 1) / kGroupsPerBlock;
  };
  auto vec_of = [](const cq::QuantizeJob &j) {
    return (j.cols % 4 == 0) && ((reinterpret_cast<uintptr_t>(j.w) & 15) == 0);
  };
  const int64_t blocks = b ? std::max(blocks_of(a), blocks_of(*b)) : blocks_of(a);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (blocks == 0) return hipSuccess;
  const bool vec = vec_of(a) && (!b || vec_of(*b));
  const dim3 grid(static_cast<unsigned>(blocks), b ? 2u : 1u);
  const cq::QuantizeJob &jb = b ? *b : a;
  if (tab.lut) {
    if (vec)
      quantize_kernel<SB, true, true><<<grid, kThreads, 0, s>>>(a, jb, tab);
    else
      quantize_kernel<SB, false, true><<<grid, kThreads, 0, s>>>(a, jb, tab);
  } else {
    if (vec)
      quantize_kernel<SB, true, false><<<grid, kThreads, 0, s>>>(a, jb, tab);
    else
      quantize_kernel<SB, false, false><<<grid, kThreads, 0, s>>>(a, jb, tab);
  }
  return hipGetLastError();
}

}  // namespace

namespace cq {

hipError_t launch_quantize(const QuantizeJob &a, const QuantizeJob *b, const EncodeTable &tab, int bits, hipStream_t s) {
  switch (storage_bits(bits)) {
    case 1: return launch_sb<1>(a, b, tab, s);
    case 2: return launch_sb<2>(a, b, tab, s);
    case 3: return launch_sb<3>(a, b, tab, s);
    default: return launch_sb<4>(a, b, tab, s);
  }
}

}  // namespace cq
