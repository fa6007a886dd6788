// The CQ-W2A8 decode product: int8 activations, int8 codebook, integer dot
// products, one float multiply per group:
//
//   y[b][r] = sum_g (float(norm[r][g]) * sx[b][g] * sc) * sum_k c8[q[r][g][k]] * xq[b][g][k]
//
// (".cact" format post, "How the kernel reads it": the rotated activation
// group is quantised to int8 with one scale per group, the int8 centroids are
// looked up by the packed indices and dotted with the activation, and one
// multiply per group applies the weight norm, the activation scale and the
// codebook scale; OpenNeedle reference notes, Cactus 2-bit kernel: absmax/127
// per group for the activation, maxabs/127 for the codebook.)
//
// Numerics (the same decisions as the oracle's, in the same precision):
//   xr   = the fp32 butterfly of every rotating kernel (cq_fwht.h);
//   sx   = fp32(absmax of the group's xr / 127), an IEEE division;
//   xq   = clamp(round-half-even(fp32(xr / sx)), -128, 127); 0 when sx == 0;
//   c8   = round-half-even(fp32(c / sc)), sc = fp32(max|c| / 127), computed on
//          the host; ternary crumbs use their sign-extended integers, sc = a;
//          binary codes +-127.
// The integer dots are exact; the per-group scaling and the sums are fp32.
//
// Three kernels:
//  * quant_acts_kernel rotates and quantises the activation once (int8 in
//    column order and the group scales, in global memory);
//  * w2a8_row_kernel (batch 1-2, 3 at two bits, and what the next kernel's
//    LDS cannot hold) streams whole stretches of rows through v_dot4_i32_i8
//    (its own notes are below);
//  * w2a8_kernel (larger batches): per workgroup of 256 threads (4 waves), a
//    wave owns a 16-row block; v_mfma_i32_16x16x64_i8 with A = the batch
//    (padding lanes read a zero row) and B = 16 rows x 64 codes of one group,
//    two steps per group, so the i32 accumulator holds one group and is
//    scaled into the fp32 sum before the next.  Lane (row n, quarter q) owns
//    codes 32q..32q+31 of every group of its row (4 to 16 contiguous bytes)
//    and decodes them with byte permutes of the int8 codebook held in
//    registers.  Each workgroup copies the quantised activation into LDS in
//    the decoders' slot order, then loops over row tiles (a grid of about as
//    many workgroups as fit the chip).  Chunks of 4 groups, two in flight per
//    wave; with 2+ chunks, 2 or 4 waves split a block's K and add their
//    accumulators through LDS in wave order.
// Both product kernels load the packed codes of matrices of
// cq::kStreamMinBytes and more with the nt (streaming) cache hint: 3-10 %
// faster on the 285 and 554 MB matrices than plain loads, which smaller
// matrices keep (they may stay in the Infinity Cache between calls).
#include <atomic>
#include <mutex>

#include "cq_decode.h"
#include "cq_fwht.h"
#include "cq_internal.h"

namespace {

using namespace cqdev;

typedef int int32x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // 4 waves
constexpr int kWaves = kThreads / 64;
constexpr int kBlockRows = 16;  // one MFMA block
// Groups per chunk (two chunks in flight per wave).  Larger chunks measured
// slower: the per-group address work, not the bytes in flight, bounds the
// kernel on large matrices.
template <int SB>
constexpr int chunk_groups() { return 4; }
constexpr int kMaxBatch = 8;
constexpr uint32_t kOutOfRange = 0xffff0000u;  // a buffer offset past any range

struct W8Args {
  const uint8_t *packed;
  const uint16_t *norms;  // fp16 bits [rows][ngroups]
  const int8_t *xq;       // [batch][kpad], column order
  const float *sx;        // [batch][ngroups]
  float *y;               // [batch][rows]
  int64_t rows, row_bytes;
  int32_t ngroups, batch, ks_shift;
  int32_t ntiles;  // row tiles (16 << (2 - ks_shift) rows each); workgroups loop over them
  uint32_t c8[4];  // int8 value of stored code c in byte c % 4 of c8[c / 4]
  float sc;
};

// Slot of code c of a decoder block (16 codes; 32 at one bit) in the
// decoders' output order.
template <int SB>
__device__ constexpr int code_slot(int c) {
  return SB == 1 ? 4 * (c & 7) + (c >> 3)                          // dword k: codes k, 8+k, 16+k, 24+k
       : SB == 2 ? 4 * (c & 3) + (c >> 2)                          // dword i: codes i, 4+i, 8+i, 12+i
       : SB == 4 ? 4 * (2 * (c >> 3) + (c & 1)) + ((c & 7) >> 1)  // dwords: even codes, odd codes of each 8
                 : c;                                              // 3-bit: natural order
}
template <int SB>
constexpr int slot_block() { return SB == 1 ? 32 : 16; }

// Decoders: 16 codes -> 4 dwords of int8 (slot order code_slot).
// 1-bit: the 32 codes of dword d -> 8 dwords; selector k takes bit k of each
// byte, which picks byte 0 (code 0) or byte 1 (code 1) of the table.
__device__ inline void decode1_i8(uint32_t t, uint32_t d, int32x4 &o0, int32x4 &o1) {
#pragma unroll
  for (int k = 0; k < 4; ++k) o0[k] = static_cast<int>(perm(0u, t, (d >> k) & 0x01010101u));
#pragma unroll
  for (int k = 0; k < 4; ++k) o1[k] = static_cast<int>(perm(0u, t, (d >> (k + 4)) & 0x01010101u));
}
// 2-bit: the 16 codes of dword d.
__device__ inline void decode2_i8(uint32_t t, uint32_t d, int32x4 &o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = static_cast<int>(perm(0u, t, (d >> (2 * i)) & 0x03030303u));
}
// 4-bit: the 8 codes of each of d0, d1 (tables t0..t3 hold the 16 int8 values).
__device__ inline uint32_t nib_lookup(const uint32_t (&t)[4], uint32_t sel) {
  const uint32_t lo = sel & 0x07070707u;
  const uint32_t hi = ((sel >> 3) & 0x01010101u) * 0xffu;
  return select(hi, perm(t[3], t[2], lo), perm(t[1], t[0], lo));
}
__device__ inline void decode4_i8(const uint32_t (&t)[4], uint32_t d0, uint32_t d1, int32x4 &o) {
  o[0] = static_cast<int>(nib_lookup(t, d0 & 0x0f0f0f0fu));
  o[1] = static_cast<int>(nib_lookup(t, (d0 >> 4) & 0x0f0f0f0fu));
  o[2] = static_cast<int>(nib_lookup(t, d1 & 0x0f0f0f0fu));
  o[3] = static_cast<int>(nib_lookup(t, (d1 >> 4) & 0x0f0f0f0fu));
}
// 3-bit: two 24-bit fields (8 codes each) -> codes in natural order.
__device__ inline uint32_t three_bit_4(const uint32_t (&t)[4], uint32_t f) {
  const uint32_t s = (f & 7u) | ((f << 5) & 0x700u) | ((f << 10) & 0x70000u) | ((f << 15) & 0x7000000u);
  return perm(t[1], t[0], s);
}
__device__ inline void decode3_i8(const uint32_t (&t)[4], uint32_t f0, uint32_t f1, int32x4 &o) {
  o[0] = static_cast<int>(three_bit_4(t, f0));
  o[1] = static_cast<int>(three_bit_4(t, f0 >> 12));
  o[2] = static_cast<int>(three_bit_4(t, f1));
  o[3] = static_cast<int>(three_bit_4(t, f1 >> 12));
}

// Row max of |v| over the 16 lanes of a row (DPP within the row; exact).
__device__ inline float row16_max(float m) {
  m = fmaxf(m, dpp_f32<0xb1>(m));   // quad_perm 1,0,3,2
  m = fmaxf(m, dpp_f32<0x4e>(m));   // quad_perm 2,3,0,1
  m = fmaxf(m, dpp_f32<0x141>(m));  // row_half_mirror
  m = fmaxf(m, dpp_f32<0x128>(m));  // row_ror:8
  return m;
}

// The rotated activation quantised to int8, one (batch row, group) per 16
// lanes: the shared butterfly, the group's absmax, sx = absmax / 127 and
// q = clamp(rint(xr / sx)) (IEEE division, round half to even), written in
// column order (8 bytes per lane) with the scale at sx[b][g].
__global__ __launch_bounds__(kThreads) void quant_acts_kernel(const float *x, int64_t cols, int32_t xvec,
                                                              int64_t tasks, int32_t ngroups, int8_t *xq, float *sxo) {
  const int j = threadIdx.x & 15;
  const int64_t task = static_cast<int64_t>(blockIdx.x) * (kThreads / 16) + (threadIdx.x >> 4);
  const bool valid = task < tasks;  // every lane runs the exchanges
  const int64_t b = valid ? task / ngroups : 0, g = valid ? task - b * ngroups : 0;
  float v[8];
  load8_f32(x + b * cols, g * CQ_GROUP + 8 * j, valid ? cols : 0, xvec != 0, v);
  fwht128_unscaled(v, j);
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] *= kInvSqrt128;
    m = fmaxf(m, fabsf(v[i]));
  }
  m = row16_max(m);
  const float sx = m / 127.0f;
  if (!valid) return;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int qv = 0;
    if (sx > 0.0f) qv = static_cast<int>(fminf(fmaxf(rintf(v[i] / sx), -128.0f), 127.0f));
    w[i >> 2] |= (static_cast<uint32_t>(qv) & 0xffu) << (8 * (i & 3));
  }
  const int64_t kpad = static_cast<int64_t>(ngroups) * CQ_GROUP;
  *reinterpret_cast<uint2 *>(xq + b * kpad + g * CQ_GROUP + 8 * j) = make_uint2(w[0], w[1]);
  if (j == 0) sxo[task] = sx;
}

// The activation bytes of one decoder block (N = 16 or 32 codes, N / 16
// uint4), column order -> slot order.
template <int SB>
__device__ inline void to_slot_order(const uint4 *src, uint4 *dst) {
  constexpr int N = slot_block<SB>();
  if constexpr (SB == 3) {
    dst[0] = src[0];
  } else {
    uint32_t in[N / 4], out[N / 4];
#pragma unroll
    for (int q = 0; q < N / 16; ++q) {
      const uint4 v = src[q];
      in[4 * q] = v.x, in[4 * q + 1] = v.y, in[4 * q + 2] = v.z, in[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < N / 4; ++i) out[i] = 0u;
#pragma unroll
    for (int c = 0; c < N; ++c) {
      const uint32_t byte = (in[c >> 2] >> (8 * (c & 3))) & 0xffu;
      const int sl = code_slot<SB>(c);
      out[sl >> 2] |= byte << (8 * (sl & 3));
    }
#pragma unroll
    for (int q = 0; q < N / 16; ++q) dst[q] = make_uint4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
  }
}

// The quantised activation into LDS: xq [batch][kpad] in slot order and the
// scales at sxs[g * 8 + b].  All threads of the workgroup call it.
// Bit planes of a 32-code binary block (two uint4 of int8 in column order):
// plane p (dword p of the output) has bit i = bit p of activation i, so that
// sum_i bit_i * x_i = sum_p (p < 7 ? 2^p : -2^7) * popcount(bits & plane_p).
// Each 8 bytes are one 8 x 8 bit transpose (three delta swaps: byte p of the
// result holds bit p of bytes 0..7).
__device__ inline uint64_t transpose8x8(uint64_t x) {
  uint64_t t = (x ^ (x >> 7)) & 0x00AA00AA00AA00AAull;
  x = x ^ t ^ (t << 7);
  t = (x ^ (x >> 14)) & 0x0000CCCC0000CCCCull;
  x = x ^ t ^ (t << 14);
  t = (x ^ (x >> 28)) & 0x00000000F0F0F0F0ull;
  return x ^ t ^ (t << 28);
}
__device__ inline void to_planes(const uint4 *src, uint4 *dst) {
  const uint4 lo = src[0], hi = src[1];
  const uint64_t w[4] = {lo.x | static_cast<uint64_t>(lo.y) << 32, lo.z | static_cast<uint64_t>(lo.w) << 32,
                         hi.x | static_cast<uint64_t>(hi.y) << 32, hi.z | static_cast<uint64_t>(hi.w) << 32};
  uint64_t t[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) t[a] = transpose8x8(w[a]);
  uint32_t pl[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {  // byte a of plane q: byte q of t[a]
    pl[q] = 0u;
#pragma unroll
    for (int a = 0; a < 4; ++a) pl[q] |= static_cast<uint32_t>((t[a] >> (8 * q)) & 0xffu) << (8 * a);
  }
  dst[0] = make_uint4(pl[0], pl[1], pl[2], pl[3]);
  dst[1] = make_uint4(pl[4], pl[5], pl[6], pl[7]);
}

template <int SB, int NT, bool PLANES = false>
__device__ inline void fill_int8(const int8_t *xq, const float *sx, int batch, int ngroups, uint8_t *lxq,
                                 float *sxs) {
  static_assert(!PLANES || SB == 1, "bit planes: binary blocks");
  const int tid = threadIdx.x;
  constexpr int Q = slot_block<SB>() / 16;  // uint4 per decoder block
  const int blocks = batch * ngroups * (CQ_GROUP / slot_block<SB>());
  const uint4 *src = reinterpret_cast<const uint4 *>(xq);
  uint4 *dst = reinterpret_cast<uint4 *>(lxq);
  for (int t = tid; t < blocks; t += NT) {
    if constexpr (PLANES)
      to_planes(src + Q * t, dst + Q * t);
    else
      to_slot_order<SB>(src + Q * t, dst + Q * t);
  }
  for (int t = tid; t < batch * ngroups; t += NT) {
    const int b = t / ngroups, g = t - b * ngroups;
    sxs[g * 8 + b] = sx[t];
  }
}

// LDS: int8 activations [kMaxBatch + 1 rows][kpad] (row `batch` is zero for
// the padding lanes), then the group scales [ngroups][8] (fp32).
template <int SB, int POL>
__global__ __launch_bounds__(kThreads) void w2a8_kernel(W8Args a) {
  constexpr int GROUP_BYTES = CQ_GROUP * SB / 8;  // 16, 32, 48, 64
  constexpr int QB = GROUP_BYTES / 4;              // a quarter's bytes: 4, 8, 12, 16
  constexpr int QDW = QB / 4;                      // 1, 2, 3, 4
  extern __shared__ __align__(16) uint8_t lds[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ngroups = a.ngroups;
  const int64_t kpad = static_cast<int64_t>(ngroups) * CQ_GROUP;
  const int batch = a.batch;
  uint8_t *xq = lds;                                                        // [(batch + 1)][kpad]
  float *sxs = reinterpret_cast<float *>(lds + (batch + 1) * kpad);        // [ngroups][8]

  const int ks = a.ks_shift, ksplit = 1 << ks;
  const int blk = wave >> ks, part = wave & (ksplit - 1);
  const int64_t rows = a.rows;
  constexpr int CG = chunk_groups<SB>();
  const int nchunks = (ngroups + CG - 1) / CG;
  const int c_lo = part * nchunks >> ks, c_hi = (part + 1) * nchunks >> ks;
  const int n = lane & 15, q = lane >> 4;
  __amdgpu_buffer_rsrc_t wbuf, nbuf;
  int64_t r0 = 0;
  auto set_tile = [&](int tile) {
    r0 = ((static_cast<int64_t>(tile) << (2 - ks)) + blk) * kBlockRows;
    const int64_t live_rows = rows - r0 < kBlockRows ? (rows - r0 > 0 ? rows - r0 : 0) : kBlockRows;
    wbuf = buffer_rsrc(a.packed + r0 * a.row_bytes, static_cast<uint32_t>(live_rows * a.row_bytes));
    nbuf = buffer_rsrc(a.norms + r0 * ngroups, static_cast<uint32_t>(live_rows * ngroups * 2));
  };
  int tile = blockIdx.x;
  set_tile(tile);

  // ---- codes and norms of a chunk: 4 groups, this lane's quarter of each,
  // and the row's norms of those groups (groups past K read zeros)
  uint32_t codes[2][CG][QDW];
  uint16_t nrm[2][CG];
  auto load_chunk = [&](int c, auto set_c) {
    constexpr int S = decltype(set_c)::value;
    const bool live = c < c_hi;
#pragma unroll
    for (int gi = 0; gi < CG; ++gi) {
      const int g = CG * c + gi;
      const uint32_t off = live && g < ngroups ? static_cast<uint32_t>(n * a.row_bytes + g * GROUP_BYTES + q * QB)
                                               : kOutOfRange;
      load_dwords<QDW, POL>(wbuf, off, codes[S][gi]);
      const uint32_t noff = live && g < ngroups ? static_cast<uint32_t>((n * ngroups + g) * 2) : kOutOfRange;
      nrm[S][gi] = __builtin_amdgcn_raw_buffer_load_b16(nbuf, noff, 0, 0);
    }
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  load_chunk(c_lo, Set0{});

  // ---- the activation (and the zero row the padding lanes read)
  for (int64_t k = tid * 16; k < kpad; k += kThreads * 16)
    *reinterpret_cast<uint4 *>(xq + batch * kpad + k) = make_uint4(0u, 0u, 0u, 0u);
  fill_int8<SB, kThreads>(a.xq, a.sx, batch, ngroups, xq, sxs);
  __syncthreads();

  // ---- the product
  const int m_a = (lane & 15) < batch ? (lane & 15) : batch;  // padding lanes read the zero row
  const uint8_t *a_row = xq + static_cast<int64_t>(m_a) * kpad + q * 32;
  uint32_t tab[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) tab[i] = a.c8[i];

  floatx4 acc;
  auto compute_chunk = [&](int c, auto set_c) {
    constexpr int S = decltype(set_c)::value;
#pragma unroll
    for (int gi = 0; gi < CG; ++gi) {
      const int g = CG * c + gi;
      if (g >= ngroups) break;  // a partial last chunk (uniform)
      const uint32_t *cd = codes[S][gi];
      int32x4 bq[2];
      if constexpr (SB == 1) {  // one 32-code slot block
        decode1_i8(tab[0], cd[0], bq[0], bq[1]);
      } else if constexpr (SB == 2) {
        decode2_i8(tab[0], cd[0], bq[0]);
        decode2_i8(tab[0], cd[1], bq[1]);
      } else if constexpr (SB == 4) {
        decode4_i8(tab, cd[0], cd[1], bq[0]);
        decode4_i8(tab, cd[2], cd[3], bq[1]);
      } else {
        // 32 codes in 3 dwords: fields of 24 bits at bit 0, 24, 48, 72
        const uint32_t f1 = __builtin_amdgcn_alignbit(cd[1], cd[0], 24);
        const uint32_t f2 = __builtin_amdgcn_alignbit(cd[2], cd[1], 16);
        const uint32_t f3 = cd[2] >> 8;
        decode3_i8(tab, cd[0], f1, bq[0]);
        decode3_i8(tab, f2, f3, bq[1]);
      }
      const uint8_t *ap = a_row + static_cast<int64_t>(g) * CQ_GROUP;
      const int32x4 a0 = *reinterpret_cast<const int32x4 *>(ap);
      const int32x4 a1 = *reinterpret_cast<const int32x4 *>(ap + 16);
      int32x4 d = {0, 0, 0, 0};
      d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bq[0], d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bq[1], d, 0, 0, 0);
      // D layout: lane l, register e -> batch row 4 (l / 16) + e, weight row l % 16
      const floatx4 s = *reinterpret_cast<const floatx4 *>(sxs + g * 8 + 4 * q);
      const float nn = static_cast<float>(__builtin_bit_cast(_Float16, nrm[S][gi]));
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(static_cast<float>(d[e]), s[e] * nn, acc[e]);
    }
  };
  __shared__ floatx4 red[kWaves][64];
  for (;;) {  // tiles blockIdx.x, + gridDim.x, ... (the bound is the same for the whole workgroup)
    acc = floatx4{0.f, 0.f, 0.f, 0.f};
    int c = c_lo;
    for (; c + 2 <= c_hi; c += 2) {
      load_chunk(c + 1, Set1{});
      compute_chunk(c, Set0{});
      load_chunk(c + 2, Set0{});
      compute_chunk(c + 1, Set1{});
    }
    if (c < c_hi) compute_chunk(c, Set0{});
    const int64_t r = r0 + n;
    const int next = tile + static_cast<int>(gridDim.x);
    if (next < a.ntiles) {  // the next tile's first chunk goes out before the sums are stored
      set_tile(next);
      load_chunk(c_lo, Set0{});
    }

    // ---- the K-split waves of a block add their sums in wave order
    if (ksplit > 1) {
      red[wave][lane] = acc;
      __syncthreads();
      if (part == 0) {
#pragma unroll
        for (int p = 1; p < 4; ++p)
          if (p < ksplit) acc += red[wave + p][lane];
      }
      __syncthreads();  // red is free again
    }
    if (part == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 4 * q + e;
        if (m < batch && r < rows) a.y[static_cast<int64_t>(m) * rows + r] = acc[e] * a.sc;
      }
    }
    if (next >= a.ntiles) break;
    tile = next;
  }
}

// ---- the row-streaming kernel: batch 1 or 2 and batch x cols_pad <= 16384.
// A wave reads whole stretches of a row (16-byte pieces, 1 KB per load
// instruction at full width), decodes each piece with byte permutes and
// accumulates it with v_dot4_i32_i8 against the lane's int8 activations,
// which it holds in registers for the whole kernel.  The pieces of one group
// sit in adjacent lanes: their integer dots are added across those lanes
// (exact), and the group's first lane scales the group's dot by norm x
// activation scale, so every group is rounded once, as in the MFMA kernel.
// Short rows share a wave: 2^lpr_shift lanes per row, a segmented reduction
// at the end of each step of rows.  A workgroup copies the quantised
// activation into LDS once (slot order), each lane takes its pieces' bytes
// into registers, and the waves then take steps of rows from an LDS counter
// over the workgroup's contiguous range, two steps in flight per wave.
template <int SB>
struct RowGeom {
  static constexpr int PB = SB == 3 ? 12 : 16;  // code bytes per piece (one load)
  static constexpr int PDW = PB / 4;            // 4, 4, 3, 4
  static constexpr int CP = PB * 8 / SB;        // codes per piece: 128, 64, 32, 32
  static constexpr int XDW = CP / 4;            // int8 activation dwords per piece
  static constexpr int PPG = CQ_GROUP / CP;     // pieces per group: 1, 2, 4, 4
};
constexpr int kRowThreads = 256;
constexpr int kRowMaxXdw = 64;  // activation dwords a lane holds, all batch rows

struct W8RowArgs {
  const uint8_t *packed;
  const uint16_t *norms;
  const int8_t *xq;  // [B][kpad], column order
  const float *sx;   // [B][ngroups]
  float *y;
  int64_t rows, row_bytes;
  int32_t ngroups, npieces, lpr_shift, npl, nsteps;
  uint32_t c8[4];
  float sc;
};

// XREG: the lane's activation bytes live in registers (B * NPL * XDW <= 64
// dwords); otherwise each piece reads them from LDS.
template <int SB, int B, int NPL, bool XREG, int POL>
__global__ __launch_bounds__(kRowThreads) void w2a8_row_kernel(W8RowArgs a) {
  using G = RowGeom<SB>;
  static_assert(!XREG || B * NPL * G::XDW <= kRowMaxXdw, "activation registers");
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int next_step;
  const int tid = threadIdx.x, lane = tid & 63;
  const int ngroups = a.ngroups, npieces = a.npieces;
  const int64_t kpad = static_cast<int64_t>(ngroups) * CQ_GROUP;
  uint8_t *xq = lds;                                             // [B][kpad]
  float *sxs = reinterpret_cast<float *>(lds + B * kpad);       // [ngroups][8]

  // steps of rows: this workgroup's contiguous range, handed out to its waves
  const int spw = (a.nsteps + static_cast<int>(gridDim.x) - 1) / static_cast<int>(gridDim.x);
  const int s_begin = static_cast<int>(blockIdx.x) * spw;
  const int s_end = min(s_begin + spw, a.nsteps);
  if (tid == 0) next_step = s_begin;
  // Binary at batch 1 with the activations in registers: the lane holds the
  // activations' bit planes instead of their bytes (the same 32 dwords per
  // piece), and a group's masked sum is 32 popcounts of code & plane.
  constexpr bool PLANES = SB == 1 && XREG && B == 1;
  fill_int8<SB, kRowThreads, PLANES>(a.xq, a.sx, B, ngroups, xq, sxs);
  __syncthreads();

  const int lps = a.lpr_shift, lpr = 1 << lps, li = lane & (lpr - 1), rsub = lane >> lps;
  const int rs = 64 >> lps;  // rows per step
  // ---- this lane's activations (pieces li + lpr * i) and their group scales
  uint32_t xr8[XREG ? B : 1][XREG ? NPL : 1][G::XDW];
  float sxv[B][NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int p = li + lpr * i;
    const bool live = i < a.npl && p < npieces;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if constexpr (XREG) {
        const uint32_t *src =
            reinterpret_cast<const uint32_t *>(xq + b * kpad + static_cast<int64_t>(live ? p : 0) * G::CP);
#pragma unroll
        for (int w = 0; w < G::XDW; ++w) xr8[b][i][w] = live ? src[w] : 0u;
      }
      // only the group's first lane scales the group's summed dot
      sxv[b][i] = live && (p % G::PPG) == 0 ? sxs[(p / G::PPG) * 8 + b] : 0.0f;
    }
  }
  uint32_t tab[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) tab[i] = a.c8[i];
  // Binary with the activations in registers: c8[bit] = c0 + (c1 - c0) * bit,
  // so a group's dot is c0 * sum(x) + (c1 - c0) * sum(bit * x), exactly; the
  // masked sums take the bit bytes straight into v_dot4 (no table permute),
  // and sum(x) of each of the lane's groups is taken once here.
  constexpr bool MASKED = SB == 1 && XREG;
  const int c0 = static_cast<int8_t>(tab[0] & 0xffu), dc = static_cast<int8_t>((tab[0] >> 8) & 0xffu) - c0;
  int xsum[MASKED ? B : 1][MASKED ? NPL : 1];
  // sum_p (p < 7 ? 2^p : -2^7) * cnt[p]: the signed int8 sum the planes encode
  auto plane_sum = [](const int (&cnt)[8]) {
    int v = -(cnt[7] << 7);
#pragma unroll
    for (int q = 0; q < 7; ++q) v += cnt[q] << q;
    return v;
  };
  if constexpr (MASKED) {
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        int t = 0;
        if constexpr (PLANES) {
          int cnt[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
          for (int w = 0; w < G::XDW; ++w) cnt[w & 7] += __builtin_popcount(xr8[b][i][w]);
          t = plane_sum(cnt);
        } else {
#pragma unroll
          for (int w = 0; w < G::XDW; ++w)
            t = __builtin_amdgcn_sdot4(0x01010101, static_cast<int>(xr8[b][i][w]), t, false);
        }
        xsum[b][i] = t;
      }
  }

  // this lane's byte offsets in a step's code and norm buffers
  uint32_t coff[NPL], noff[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const uint32_t p = static_cast<uint32_t>(li + lpr * i);
    const bool live = i < a.npl && p < static_cast<uint32_t>(npieces);
    coff[i] = live ? static_cast<uint32_t>(rsub * a.row_bytes) + p * G::PB : kOutOfRange;
    noff[i] = live ? (static_cast<uint32_t>(rsub * ngroups) + p / G::PPG) * 2u : kOutOfRange;
  }
  uint32_t codes[2][NPL][G::PDW];  // two steps in flight per wave
  uint16_t nrm[2][NPL];
  auto grab = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(&next_step, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  auto load_step = [&](int st, auto set_c) {
    constexpr int S = decltype(set_c)::value;
    const int64_t r0 = static_cast<int64_t>(st) * rs;
    const int64_t live_rows = st < s_end ? (a.rows - r0 < rs ? a.rows - r0 : rs) : 0;
    const __amdgpu_buffer_rsrc_t rb =
        buffer_rsrc(a.packed + r0 * a.row_bytes, static_cast<uint32_t>(live_rows * a.row_bytes));
    const __amdgpu_buffer_rsrc_t nb =
        buffer_rsrc(a.norms + r0 * ngroups, static_cast<uint32_t>(live_rows * ngroups * 2));
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      load_dwords<G::PDW, POL>(rb, coff[i], codes[S][i]);
      nrm[S][i] = __builtin_amdgcn_raw_buffer_load_b16(nb, noff[i], 0, 0);
    }
  };
  auto compute_step = [&](int st, auto set_c) {
    constexpr int S = decltype(set_c)::value;
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.0f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      if (i >= a.npl) break;  // uniform
      const uint32_t *cd = codes[S][i];
      int32x4 dq[G::XDW / 4];
      if constexpr (PLANES) {
        // (the planes' dot replaces the bit bytes below)
      } else if constexpr (MASKED) {
        // bit bytes: selector k of code dword w is slot dword 8w + k
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
          for (int k = 0; k < 8; ++k) dq[(8 * w + k) >> 2][k & 3] = static_cast<int>((cd[w] >> k) & 0x01010101u);
      } else if constexpr (SB == 1) {
#pragma unroll
        for (int w = 0; w < 4; ++w) decode1_i8(tab[0], cd[w], dq[2 * w], dq[2 * w + 1]);
      } else if constexpr (SB == 2) {
#pragma unroll
        for (int w = 0; w < 4; ++w) decode2_i8(tab[0], cd[w], dq[w]);
      } else if constexpr (SB == 4) {
        decode4_i8(tab, cd[0], cd[1], dq[0]);
        decode4_i8(tab, cd[2], cd[3], dq[1]);
      } else {
        const uint32_t f1 = __builtin_amdgcn_alignbit(cd[1], cd[0], 24);
        const uint32_t f2 = __builtin_amdgcn_alignbit(cd[2], cd[1], 16);
        decode3_i8(tab, cd[0], f1, dq[0]);
        decode3_i8(tab, f2, cd[2] >> 8, dq[1]);
      }
      const float nn = static_cast<float>(__builtin_bit_cast(_Float16, nrm[S][i]));
#pragma unroll
      for (int b = 0; b < B; ++b) {
        int dot = 0;
        if constexpr (PLANES) {  // code dword w against planes 8w .. 8w + 7
          int cnt[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
          for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int q = 0; q < 8; ++q) cnt[q] += __builtin_popcount(cd[w] & xr8[b][i][8 * w + q]);
          dot = plane_sum(cnt);
        } else if constexpr (XREG) {
#pragma unroll
          for (int w = 0; w < G::XDW; ++w)
            dot = __builtin_amdgcn_sdot4(dq[w >> 2][w & 3], static_cast<int>(xr8[b][i][w]), dot, false);
        } else {
          // a group's lanes are all live or all past K; the latter read piece 0
          const int p = li + lpr * i;
          const int32x4 *src = reinterpret_cast<const int32x4 *>(xq + b * kpad + (p < npieces ? p : 0) * G::CP);
#pragma unroll
          for (int w4 = 0; w4 < G::XDW / 4; ++w4) {
            const int32x4 xv = src[w4];
#pragma unroll
            for (int w = 0; w < 4; ++w) dot = __builtin_amdgcn_sdot4(dq[w4][w], xv[w], dot, false);
          }
        }
        if constexpr (MASKED) dot = c0 * xsum[b][i] + dc * dot;
        if constexpr (G::PPG >= 2) dot += __builtin_amdgcn_mov_dpp(dot, 0xb1, 0xf, 0xf, false);  // xor 1: 2 pieces
        if constexpr (G::PPG == 4) dot += __builtin_amdgcn_mov_dpp(dot, 0x4e, 0xf, 0xf, false);  // xor 2: its 4
        acc[b] = fmaf(static_cast<float>(dot), sxv[b][i] * nn, acc[b]);
      }
    }
    // segmented sum over the row's lanes (every lane of the segment gets it)
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float v = acc[b];
      if (lps >= 1) v += xor_lane<1>(v);
      if (lps >= 2) v += xor_lane<2>(v);
      if (lps >= 3) v += xor_lane<4>(v);
      if (lps >= 4) v += xor_lane<8>(v);
      if (lps >= 5) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      }
      if (lps >= 6) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      }
      acc[b] = v;
    }
    const int64_t r = static_cast<int64_t>(st) * rs + rsub;
    if (li == 0 && st < s_end && r < a.rows) {
#pragma unroll
      for (int b = 0; b < B; ++b) a.y[static_cast<int64_t>(b) * a.rows + r] = acc[b] * a.sc;
    }
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  int s0 = grab();
  load_step(s0, Set0{});
  int s1 = grab();
  load_step(s1, Set1{});
  // grabs only grow: the loop ends once both sets are past the range (a set
  // past it loads nothing and stores nothing)
  while (s0 < s_end || s1 < s_end) {
    compute_step(s0, Set0{});
    s0 = grab();
    load_step(s0, Set0{});
    compute_step(s1, Set1{});
    s1 = grab();
    load_step(s1, Set1{});
  }
}

typedef void (*W8RowKernel)(W8RowArgs);

// Pieces per lane: with the activation in registers, as many as 64 dwords
// hold; from LDS, enough for 16384 columns.
template <int SB, int B>
constexpr int row_npl_reg() { return kRowMaxXdw / (B * RowGeom<SB>::XDW); }
template <int SB>
constexpr int row_npl_lds() { return 16384 * SB / 8 / RowGeom<SB>::PB / 64; }

constexpr int kRowMaxBatch = 4;

// The row kernel for (storage bits, batch, pieces per lane): registers when
// they hold the lane's activations, else LDS; nullptr past its limits.
template <int SB, int POL>
W8RowKernel pick_row_sb(int batch, int npl) {
  if (batch == 1 && npl <= row_npl_reg<SB, 1>()) return w2a8_row_kernel<SB, 1, row_npl_reg<SB, 1>(), true, POL>;
  if (batch == 2 && npl <= row_npl_reg<SB, 2>()) return w2a8_row_kernel<SB, 2, row_npl_reg<SB, 2>(), true, POL>;
  if (npl > row_npl_lds<SB>()) return nullptr;
  switch (batch) {  // batch 1 always fits registers
    case 2: return w2a8_row_kernel<SB, 2, row_npl_lds<SB>(), false, POL>;
    case 3: return w2a8_row_kernel<SB, 3, row_npl_lds<SB>(), false, POL>;
    case 4: return w2a8_row_kernel<SB, 4, row_npl_lds<SB>(), false, POL>;
    default: return nullptr;
  }
}

template <int POL>
W8RowKernel pick_row_pol(int sb, int batch, int npl) {
  return sb == 1 ? pick_row_sb<1, POL>(batch, npl)
                 : (sb == 2 ? pick_row_sb<2, POL>(batch, npl)
                            : (sb == 3 ? pick_row_sb<3, POL>(batch, npl) : pick_row_sb<4, POL>(batch, npl)));
}

// stream: the packed codes' loads carry the nt hint (cq::kStreamLoad)
W8RowKernel pick_row(int sb, int batch, int npl, bool stream) {
  return stream ? pick_row_pol<cq::kStreamLoad>(sb, batch, npl) : pick_row_pol<0>(sb, batch, npl);
}

// Resident workgroups per CU of a row kernel at an LDS size, cached per
// device (a handful of (kernel, size) pairs occur in a process).
int row_occupancy(const void *k, size_t lds, int dev) {
  struct Entry { const void *k; size_t lds; int dev, per_cu; };
  static Entry cache[32];
  static int used = 0;
  static std::mutex mu;  // host threads may launch concurrently
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].k == k && cache[i].lds == lds && cache[i].dev == dev) return cache[i].per_cu;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kRowThreads, lds) != hipSuccess || per_cu < 1) per_cu = 1;
  if (used < 32) cache[used++] = Entry{k, lds, dev, per_cu};
  return per_cu;
}

typedef void (*W8Kernel)(W8Args);

template <int POL>
W8Kernel pick_pol(int sb) {
  return sb == 1 ? w2a8_kernel<1, POL>
                 : (sb == 2 ? w2a8_kernel<2, POL> : (sb == 3 ? w2a8_kernel<3, POL> : w2a8_kernel<4, POL>));
}

W8Kernel pick(int sb, bool stream) { return stream ? pick_pol<cq::kStreamLoad>(sb) : pick_pol<0>(sb); }

}  // namespace

namespace cq {

uint64_t w2a8_lds_bytes(int64_t kpad, int64_t batch) {
  return static_cast<uint64_t>(batch + 1) * kpad + static_cast<uint64_t>(kpad / CQ_GROUP) * 32;
}

// LDS of a row-kernel workgroup: the batch's int8 activations and the scales.
static uint64_t row_lds_bytes(int64_t kpad, int64_t batch) {
  return static_cast<uint64_t>(batch) * kpad + static_cast<uint64_t>(kpad / CQ_GROUP) * 32;
}

static bool use_row_kernel(int64_t kpad, int64_t batch) {
  return batch <= kRowMaxBatch && kpad <= 16384 && row_lds_bytes(kpad, batch) <= kW2a8MaxLds;
}

bool w2a8_fits(int bits, int64_t kpad, int64_t batch) {
  (void)bits;  // every width has both kernels
  if (kpad > 0 && kpad % CQ_GROUP == 0 && batch >= 1 && use_row_kernel(kpad, batch)) return true;
  return kpad > 0 && kpad % CQ_GROUP == 0 && batch >= 1 && batch <= kMaxBatch &&
         w2a8_lds_bytes(kpad, batch) <= kW2a8MaxLds;
}

uint64_t w2a8_workspace_bytes(int64_t kpad, int64_t batch) {
  const uint64_t q = (static_cast<uint64_t>(batch) * kpad + 255) / 256 * 256;
  return q + static_cast<uint64_t>(batch) * (kpad / CQ_GROUP) * 4;
}

hipError_t launch_quant_acts_int8(const float *x, int64_t batch, int64_t cols, int64_t kpad, int8_t *xq, float *sx,
                                  hipStream_t s) {
  const int64_t ngroups = kpad / CQ_GROUP;
  const int64_t tasks = batch * ngroups;
  const int64_t wgs = (tasks + kThreads / 16 - 1) / (kThreads / 16);
  if (wgs >= (int64_t{1} << 31) || ngroups >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  const int32_t xvec = cols % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  quant_acts_kernel<<<dim3(static_cast<unsigned>(wgs)), kThreads, 0, s>>>(x, cols, xvec, tasks,
                                                                          static_cast<int32_t>(ngroups), xq, sx);
  return hipGetLastError();
}

hipError_t launch_w2a8(const uint8_t *blob, int bits, int64_t rows, int64_t kpad, const Int8Codebook &cb,
                       const int8_t *xq, const float *sx, int64_t batch, float *y, hipStream_t s) {
  if (!w2a8_fits(bits, kpad, batch) || rows <= 0) return hipErrorInvalidValue;
  const int sb = storage_bits(bits);
  static std::atomic<int> cu_cache[64];  // CUs per device, 0 until asked
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int cus = cu_cache[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    cu_cache[dev].store(cus, std::memory_order_relaxed);
  }
  // Batch 1-2 and 3 at two bits stream rows (measured faster at 65536 x
  // 16384 and 131072 x 8192); larger batches share the decode over the
  // matrix cores unless their activation does not fit that kernel's LDS.
  const bool mfma_fits = batch <= kMaxBatch && w2a8_lds_bytes(kpad, batch) <= kW2a8MaxLds;
  if (use_row_kernel(kpad, batch) && (batch <= 2 || (batch == 3 && sb == 2) || !mfma_fits)) {
    W8RowArgs r;
    r.packed = blob;
    r.row_bytes = kpad * sb / 8;
    r.norms = reinterpret_cast<const uint16_t *>(blob + rows * r.row_bytes);
    r.xq = xq;
    r.sx = sx;
    r.y = y;
    r.rows = rows;
    r.ngroups = static_cast<int32_t>(kpad / CQ_GROUP);
    const int pb = sb == 3 ? 12 : 16;
    r.npieces = static_cast<int32_t>(r.row_bytes / pb);
    int lps = 0;
    while ((1 << lps) < r.npieces && lps < 6) ++lps;
    r.lpr_shift = lps;
    r.npl = (r.npieces + 63) >> 6;
    if (r.npl < 1) r.npl = 1;
    const int64_t rs = 64 >> lps;
    const int64_t nsteps = (rows + rs - 1) / rs;
    if (nsteps >= (int64_t{1} << 31) || static_cast<int64_t>(rs) * r.row_bytes >= (int64_t{1} << 31))
      return hipErrorInvalidValue;
    r.nsteps = static_cast<int32_t>(nsteps);
    for (int i = 0; i < 4; ++i) r.c8[i] = cb.c8[i];
    r.sc = cb.sc;
    const size_t lds = static_cast<size_t>(row_lds_bytes(kpad, batch));
    const W8RowKernel k = pick_row(sb, static_cast<int>(batch), r.npl, rows * (r.row_bytes + 2 * r.ngroups) >= kStreamMinBytes);
    if (!k) return hipErrorInvalidValue;
    // one wave of workgroups: as many as the CUs hold at once (registers and
    // LDS), each over a contiguous range of row steps
    const int per_cu = row_occupancy(reinterpret_cast<const void *>(k), lds, dev);
    const int64_t grid = nsteps < int64_t{per_cu} * cus ? nsteps : int64_t{per_cu} * cus;
    k<<<dim3(static_cast<unsigned>(grid)), kRowThreads, lds, s>>>(r);
    return hipGetLastError();
  }
  W8Args a;
  a.packed = blob;
  a.row_bytes = kpad * sb / 8;
  a.norms = reinterpret_cast<const uint16_t *>(blob + rows * a.row_bytes);
  a.xq = xq;
  a.sx = sx;
  a.y = y;
  a.rows = rows;
  a.ngroups = static_cast<int32_t>(kpad / CQ_GROUP);
  a.batch = static_cast<int32_t>(batch);
  const int cg = sb == 2 ? chunk_groups<2>() : chunk_groups<4>();
  const int nchunks = (a.ngroups + cg - 1) / cg;
  a.ks_shift = nchunks >= 4 ? 2 : (nchunks >= 2 ? 1 : 0);
  for (int i = 0; i < 4; ++i) a.c8[i] = cb.c8[i];
  a.sc = cb.sc;
  // 32-bit tile-relative offsets: 16 rows of packed bytes or norms.
  if (static_cast<int64_t>(kBlockRows) * a.row_bytes >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  const int64_t wg_rows = static_cast<int64_t>(kBlockRows) * (kWaves >> a.ks_shift);
  const int64_t ntiles = (rows + wg_rows - 1) / wg_rows;
  if (ntiles >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  a.ntiles = static_cast<int32_t>(ntiles);
  const size_t lds = static_cast<size_t>(w2a8_lds_bytes(kpad, batch));
  // about as many workgroups as the CUs hold at once (by LDS, at most 8 per
  // CU): each stages the activation once and loops over tiles
  int64_t per_cu = static_cast<int64_t>(160 * 1024) / static_cast<int64_t>(lds + sizeof(float) * 4 * kThreads);
  per_cu = per_cu < 1 ? 1 : (per_cu > 8 ? 8 : per_cu);
  const int64_t grid = ntiles < per_cu * cus ? ntiles : per_cu * cus;
  const W8Kernel k = pick(sb, rows * (a.row_bytes + 2 * a.ngroups) >= kStreamMinBytes);
  if (!k) return hipErrorInvalidValue;
  k<<<dim3(static_cast<unsigned>(grid)), kThreads, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace cq
