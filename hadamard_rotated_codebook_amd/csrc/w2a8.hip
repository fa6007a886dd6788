// The CQ-W2A8 decode product: int8 activations, int8 codebook, integer dot
// products on the matrix cores, one float multiply per group:
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
//          the host; ternary crumbs use their sign-extended integers, sc = a.
// The integer dots are exact; the per-group scaling and the sums are fp32.
//
// Design, per workgroup of 256 threads (4 waves):
//  * a wave owns a 16-row block; v_mfma_i32_16x16x64_i8 with A = the batch
//    (padding lanes read a zero row) and B = 16 rows x 64 codes of one group,
//    two steps per group, so the i32 accumulator holds one group and is
//    scaled into the fp32 sum before the next;
//  * lane (row n, quarter q) owns codes 32q..32q+31 of every group of its row
//    (8, 12 or 16 contiguous bytes) and decodes them with byte permutes of
//    the int8 codebook held in registers;
//  * the workgroup first rotates and quantises the whole activation into LDS
//    (int8, stored in the decoders' slot order) and the group scales, then
//    loops over row tiles (a grid of about as many workgroups as fit the
//    chip, so the staging is paid once per workgroup, not per tile);
//  * chunks of 4 groups, two in flight per wave; with 2+ chunks, 2 or 4 waves
//    split a block's K and add their accumulators through LDS in wave order.
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
  const float *x;         // [batch][cols], not rotated
  float *y;               // [batch][rows]
  int64_t rows, cols, row_bytes;
  int32_t ngroups, batch, xvec, ks_shift;
  int32_t ntiles;  // row tiles (16 << (2 - ks_shift) rows each); workgroups loop over them
  uint32_t c8[4];  // int8 value of stored code c in byte c % 4 of c8[c / 4]
  float sc;
};

// Slot of code c (0..15) of a 16-code step in the decoders' output order.
template <int SB>
__device__ constexpr int code_slot(int c) {
  return SB == 2 ? 4 * (c & 3) + (c >> 2)                          // dword i: codes i, 4+i, 8+i, 12+i
       : SB == 4 ? 4 * (2 * (c >> 3) + (c & 1)) + ((c & 7) >> 1)  // dwords: even codes, odd codes of each 8
                 : c;                                              // 3-bit: natural order
}

// Decoders: 16 codes -> 4 dwords of int8 (slot order code_slot).
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

// LDS: int8 activations [kMaxBatch + 1 rows][kpad] (row `batch` is zero for
// the padding lanes), then the group scales [ngroups][8] (fp32).
template <int SB>
__global__ __launch_bounds__(kThreads) void w2a8_kernel(W8Args a) {
  constexpr int GROUP_BYTES = CQ_GROUP * SB / 8;  // 32, 48, 64
  constexpr int QB = GROUP_BYTES / 4;              // a quarter's bytes: 8, 12, 16
  constexpr int QDW = QB / 4;                      // 2, 3, 4
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
      load_dwords<QDW>(wbuf, off, codes[S][gi]);
      const uint32_t noff = live && g < ngroups ? static_cast<uint32_t>((n * ngroups + g) * 2) : kOutOfRange;
      nrm[S][gi] = __builtin_amdgcn_raw_buffer_load_b16(nbuf, noff, 0, 0);
    }
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  load_chunk(c_lo, Set0{});

  // ---- the activation: rotate each (batch row, group) with 16 lanes, find
  // the group's absmax, quantise, store the int8 codes in slot order and the
  // scale.  The zero row first.
  for (int64_t k = tid * 16; k < kpad; k += kThreads * 16)
    *reinterpret_cast<uint4 *>(xq + batch * kpad + k) = make_uint4(0u, 0u, 0u, 0u);
  {
    const int j = lane & 15;
    const int tasks = batch * ngroups;
    for (int t0 = 0; t0 < tasks; t0 += kThreads / 16) {  // uniform trip count: all lanes run the exchanges
      const int task = t0 + (tid >> 4);
      const bool valid = task < tasks;
      const int b = valid ? task / ngroups : 0, g = valid ? task % ngroups : 0;
      float v[8];
      load8_f32(a.x + static_cast<int64_t>(b) * a.cols, static_cast<int64_t>(g) * CQ_GROUP + 8 * j, valid ? a.cols : 0,
                a.xvec != 0, v);
      fwht128_unscaled(v, j);
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[i] *= kInvSqrt128;
        m = fmaxf(m, fabsf(v[i]));
      }
      m = row16_max(m);
      const float sx = m / 127.0f;
      if (valid) {
        uint8_t *dst = xq + static_cast<int64_t>(b) * kpad + static_cast<int64_t>(g) * CQ_GROUP;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int e = 8 * j + i;  // element of the group
          int qv = 0;
          if (sx > 0.0f) qv = static_cast<int>(fminf(fmaxf(rintf(v[i] / sx), -128.0f), 127.0f));
          dst[(e & ~15) + code_slot<SB>(e & 15)] = static_cast<uint8_t>(qv);
        }
        if (j == 0) sxs[g * 8 + b] = sx;
      }
    }
  }
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
      if constexpr (SB == 2) {
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

typedef void (*W8Kernel)(W8Args);

W8Kernel pick(int sb) {
  return sb == 2 ? w2a8_kernel<2> : (sb == 3 ? w2a8_kernel<3> : w2a8_kernel<4>);
}

}  // namespace

namespace cq {

uint64_t w2a8_lds_bytes(int64_t kpad, int64_t batch) {
  return static_cast<uint64_t>(batch + 1) * kpad + static_cast<uint64_t>(kpad / CQ_GROUP) * 32;
}

bool w2a8_fits(int64_t kpad, int64_t batch) {
  return kpad > 0 && kpad % CQ_GROUP == 0 && batch >= 1 && batch <= kMaxBatch &&
         w2a8_lds_bytes(kpad, batch) <= kW2a8MaxLds;
}

hipError_t launch_w2a8(const uint8_t *blob, int bits, int64_t rows, int64_t cols, int64_t kpad, const Int8Codebook &cb,
                       const float *x, int64_t batch, float *y, hipStream_t s) {
  if (!w2a8_fits(kpad, batch) || rows <= 0) return hipErrorInvalidValue;
  const int sb = storage_bits(bits);
  W8Args a;
  a.packed = blob;
  a.row_bytes = kpad * sb / 8;
  a.norms = reinterpret_cast<const uint16_t *>(blob + rows * a.row_bytes);
  a.x = x;
  a.y = y;
  a.rows = rows;
  a.cols = cols;
  a.ngroups = static_cast<int32_t>(kpad / CQ_GROUP);
  a.batch = static_cast<int32_t>(batch);
  a.xvec = cols % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
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
  static int cu_cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cu_cache[dev] == 0) {
    int cus = 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    cu_cache[dev] = cus;
  }
  int64_t per_cu = static_cast<int64_t>(160 * 1024) / static_cast<int64_t>(lds + sizeof(float) * 4 * kThreads);
  per_cu = per_cu < 1 ? 1 : (per_cu > 8 ? 8 : per_cu);
  const int64_t grid = ntiles < per_cu * cu_cache[dev] ? ntiles : per_cu * cu_cache[dev];
  pick(sb)<<<dim3(static_cast<unsigned>(grid)), kThreads, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace cq
