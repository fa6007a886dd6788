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
//   fp32 r rounded to fp32; u is the IEEE fp32 quotient (formed in double and
//   rounded once, which is exact rounding for fp32 operands); the nearest level
//   is decided by exact comparison against the midpoints of adjacent levels,
//   ties to the smaller index; the stored norm is fp16, round to nearest even.
#include "cq_internal.h"

namespace {

constexpr double kSqrtInv128 = 0.08838834764831845;  // sqrt(1/128) in double

// packed: the first output row's codes (rows of kpad * SB / 8 bytes follow);
// norms: its fp16 norms (rows of kpad / 128 follow) -- the rows of a whole
// blob, or a row range of a larger one.
template <int SB, bool VEC>
__global__ __launch_bounds__(256) void quantize_kernel(const float *__restrict__ w, int64_t rows,
                                                      int64_t cols, int64_t kpad, cq::EncodeTable tab,
                                                      uint8_t *__restrict__ packed, uint16_t *__restrict__ norms) {
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
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) {
    const bool upper = (j & d) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double p = __shfl_xor(t[i], d, 16);
      t[i] = upper ? (p - t[i]) : (t[i] + p);
    }
  }

  float r32[8];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    r32[i] = static_cast<float>(t[i] * kSqrtInv128);
    const double rd = static_cast<double>(r32[i]);
    ss += rd * rd;  // each square is exact in double
  }
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) ss += __shfl_xor(ss, d, 16);
  const float n32 = static_cast<float>(sqrt(ss));
  const double den = static_cast<double>(fmaxf(n32, 1e-12f));

  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double u = static_cast<double>(static_cast<float>(static_cast<double>(r32[i]) / den));
    int q = 0;
    for (int m = 0; m + 1 < tab.nlevels; ++m) q += (u > tab.mid[m]) ? 1 : 0;
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
  if (vec)
    quantize_kernel<SB, true><<<dim3(static_cast<unsigned>(blocks)), 256, 0, s>>>(w, rows, cols, kpad, tab, packed, norms);
  else
    quantize_kernel<SB, false><<<dim3(static_cast<unsigned>(blocks)), 256, 0, s>>>(w, rows, cols, kpad, tab, packed, norms);
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
