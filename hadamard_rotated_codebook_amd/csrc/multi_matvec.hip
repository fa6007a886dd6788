// Decode products of small matrices, several per launch, optionally
// rotating the activation inside the kernel:
//
//   y_i[b][r] = sum_g float(norm_i[r][g]) * sum_j c_i[q_i[r][g*128+j]] * xr[b][g*128+j]
//
// with xr = H x per 128-group computed by each workgroup from x (ROT), or
// read as written by the rotation kernel.  Up to kMaxMats matrices W_i of one
// storage width and one column count share the activation: the rotated
// group is computed once per workgroup and serves every row it reads
// (".cact" format post, "How the kernel reads it": rotate each 128-group once
// and reuse it for all rows; OpenNeedle reference notes, rotated-activation
// identity).  This is the path of a decode step's projections -- Q, K, V and
// gate read the same normalised activation -- and of every matrix up to
// kSmallMaxWeights: there launches and latencies, not bytes, set the time.
//
// Limits (checked by the host): batch 1..8, cols_pad <= 4096 (no partial
// sums in memory, no workspace).
//
// Precision: the product is an fp32 computation with two fp16 matrix-core
// operands that each carry 22 significant bits.  The activation a (times a
// power of two per batch row) is held as fp16 hi + lo parts in MFMA rows 0..7
// and 8..15; the level operand is fp16(level / lscale) plus, in a second MFMA,
// its low part (cq::MmaLevels; binary and ternary levels are exact with one
// operand).  The products of fp16 values are exact in fp32, each group's sum
// is a separate fp32 accumulation, and the fp16 group norm times lscale
// multiplies it in fp32.  Nothing is rounded to fp16 with a coherent error
// that would add up over a row: an activation lined up with a weight row, a
// group norm in fp16's subnormal range or a row of 128 columns all stay at
// fp32 accuracy.
//
// Design, per workgroup of 256 threads (4 waves):
//  * the unit of work is a 16-row block; ksplit (1, 2 or 4) waves share a
//    block, each taking a contiguous range of its groups, so a workgroup
//    covers 64, 32 or 16 rows (a 512-wide matrix: one group per wave).  The waves' fp32 accumulators are
//    added in wave order through LDS: results do not depend on scheduling;
//  * K order: every MFMA k step of 32 covers one group, so the group's sum
//    stays apart from the others until its norm is applied.  The 16-lane
//    quarter q of a wave owns codes 32q..32q+31 of each group of its row
//    (a 4/8/12/16-byte piece), k step t its codes 8t..8t+7;
//  * each wave requests its batch row of the activation first, then its
//    first group's codes and norms, so the code latency overlaps the
//    rotation; the row is rotated with the butterfly every rotating kernel
//    uses (cq_fwht.h), held in registers until its largest |xr| is known,
//    scaled by the power of two that puts that value in [2^14, 2^15) and
//    stored to LDS as the fp16 hi and lo rows in the decoders' slot order.
//    With or without ROT the staged values are identical, so both give the
//    same results;
//  * the product: v_mfma_f32_16x16x32_f16 with A = the hi and lo rows of the
//    batch (padding lanes read a zero row) and B = 16 rows x 32 k of levels
//    decoded in registers from tables that depend only on the code book;
//    groups in pairs with the next group's loads in flight, and an odd last
//    group on its own; the products with the levels' hi and lo parts are
//    two independent chains.  Out-of-range rows and groups read zeros through the
//    buffer range (their norms are zero).
#include <mutex>

#include "cq_decode.h"
#include "cq_fwht.h"
#include "cq_internal.h"

namespace {

using namespace cqdev;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;                     // 4 waves
constexpr int kWaves = kThreads / 64;
constexpr int kBlockRows = 16;                    // one MFMA block
constexpr int kMaxCols = 4096;
constexpr int kChunkCols = 4 * CQ_GROUP;          // 512: four groups
constexpr int kMaxChunks = kMaxCols / kChunkCols;
constexpr int kMaxBatch = 8;
constexpr int kMaxMats = 8;
constexpr int kXPad = 8;                          // fp16 elements of padding per LDS row
constexpr uint32_t kOutOfRange = 0xffff0000u;     // a buffer offset past any range

struct SmallMat {
  const uint8_t *packed;  // packed rows; the fp16 norms [rows][ngroups] follow
  float *y;               // [batch][rows]
  int64_t rows;
  int64_t wgs;            // workgroups of this matrix
};

// Grid: x = row tiles (the largest matrix's count), y = matrix.
struct SmallArgs {
  SmallMat mat[kMaxMats];
  cq::MmaLevels lev[kMaxMats];
};

__device__ inline uint32_t pack_h2(_Float16 a, _Float16 b) { return __builtin_bit_cast(uint32_t, f16x2{a, b}); }

// Dynamic LDS of one launch: the hi rows, the lo rows and a zero row of the
// staged activation, each kpad (rounded up to a chunk) + kXPad fp16 values.
size_t small_lds_bytes(int64_t kpad, int64_t batch) {
  const int64_t nchunks = (kpad + kChunkCols - 1) / kChunkCols;
  return static_cast<size_t>((2 * batch + 1) * (nchunks * kChunkCols + kXPad) * 2);
}

// The scalar arguments come first: the compiler asks the dispatcher to
// preload them into SGPRs (-amdgpu-kernarg-preload-count=6), so the
// activation loads go out before any argument load returns.
//   x         ROT: x [batch][cols]; otherwise xr [batch][kpad]
//   xstride   cols (ROT) or kpad, in floats
//   xvec      ROT: x rows allow 16-byte loads (cols % 8 == 0, x 16-byte aligned)
//   ks_shift  ksplit = 1 << ks_shift waves per 16-row block
// SPLIT: the level operand has a low part (a second MFMA per k step).
template <int SB, bool ROT, bool SPLIT>
__global__ __launch_bounds__(kThreads) void small_matvec_kernel(const float *x, int32_t xstride, int32_t ngroups,
                                                                int32_t batch, int32_t xvec, int32_t ks_shift,
                                                                SmallArgs a) {
  constexpr int GROUP_BYTES = CQ_GROUP * SB / 8;  // 16, 32, 48, 64
  constexpr int PIECE_BYTES = 4 * SB;             // a lane's 32 codes of a group
  extern __shared__ __align__(16) _Float16 xs[];  // [2 * batch + 1][xsr]: hi rows, lo rows, zero row
  __shared__ float unscale[kMaxBatch];
  __shared__ floatx4 red[kWaves][64];             // the K-split waves' accumulators

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = blockIdx.x, mi = blockIdx.y;

  // ---- lane roles: row n of the block, quarter q (codes 32q..32q+31 of
  // each group in the product; group 4c+q of chunk c in the staging)
  const int n = lane & 15, q = lane >> 4;
  const int nchunks = (ngroups + 3) / 4;
  const int xsr = nchunks * kChunkCols + kXPad;  // LDS row stride (fp16 elements)

  // ---- activation loads of the wave's first batch row, before anything
  // that depends on the matrix (a wave without a row loads row 0 and
  // discards it, so that the loads are unconditional).  Every chunk slot is
  // loaded, in straight-line code (slots at or past nchunks, and elements
  // past the row, read zeros through the buffer range), so that the wait
  // before the rotation covers only these loads and not the codes requested
  // after them.
  float v[kMaxChunks][8];
  auto load_x = [&](int m) {
    const __amdgpu_buffer_rsrc_t xb = buffer_rsrc(x + static_cast<int64_t>(m) * xstride,
                                                  static_cast<uint32_t>(xstride) * 4u);
    if (!ROT || xvec) {
      // whole 8-element blocks: xr rows are 16-byte aligned; x rows are when
      // xvec (cols % 8 == 0 and x 16-byte aligned)
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c) {
        const int g = 4 * c + q;
        const uint32_t off = c < nchunks && g < ngroups ? static_cast<uint32_t>((g * CQ_GROUP + 8 * n) * 4) : kOutOfRange;
        // (whole vectors are bit-cast: a bit-cast of one vector component
        // does not compile to that component)
        const floatx4 lo = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(xb, off, 0, 0));
        const floatx4 hi = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(xb, off + 16, 0, 0));
        v[c][0] = lo.x, v[c][1] = lo.y, v[c][2] = lo.z, v[c][3] = lo.w;
        v[c][4] = hi.x, v[c][5] = hi.y, v[c][6] = hi.z, v[c][7] = hi.w;
      }
    } else {
      // element by element: zero past cols
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c) {
        const int64_t col0 = static_cast<int64_t>(4 * c + q) * CQ_GROUP + 8 * n;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t off = c < nchunks && col0 + i < xstride ? static_cast<uint32_t>((col0 + i) * 4) : kOutOfRange;
          v[c][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xb, off, 0, 0));
        }
      }
    }
  };
  load_x(wave < batch ? wave : 0);

  // ---- this workgroup's matrix and row tile (a tile past the matrix's end
  // reads nothing through its empty buffer ranges and leaves once its
  // requests are out, so that no argument load waits behind a branch)
  const SmallMat &mat = a.mat[mi];
  const uint8_t *packed = mat.packed;
  float *y = mat.y;
  const int64_t rows = mat.rows;
  const int64_t row_bytes = static_cast<int64_t>(ngroups) * GROUP_BYTES;
  const uint16_t *norms = reinterpret_cast<const uint16_t *>(packed + rows * row_bytes);
  const int ks = ks_shift, ksplit = 1 << ks;
  const int blk = wave >> ks, part = wave & (ksplit - 1);
  const int64_t r0 = ((static_cast<int64_t>(wg) << (2 - ks)) + blk) * kBlockRows;
  const int64_t live_rows = rows - r0 < kBlockRows ? (rows - r0 > 0 ? rows - r0 : 0) : kBlockRows;
  const __amdgpu_buffer_rsrc_t wbuf =
      buffer_rsrc(packed + r0 * row_bytes, static_cast<uint32_t>(live_rows * row_bytes));
  const __amdgpu_buffer_rsrc_t nbuf =
      buffer_rsrc(norms + r0 * ngroups, static_cast<uint32_t>(live_rows * ngroups * 2));
  const int g_lo = part * ngroups >> ks, g_hi = (part + 1) * ngroups >> ks;

  uint32_t codes[2][SB];  // [set][dword of the lane's piece]
  uint16_t nrm[2];
  auto load_group = [&](int g, auto set_c) {
    constexpr int S = decltype(set_c)::value;
    const bool g_live = g < g_hi;
    const uint32_t woff = static_cast<uint32_t>(n * row_bytes + g * GROUP_BYTES + q * PIECE_BYTES);
    load_dwords<SB>(wbuf, g_live ? woff : kOutOfRange, codes[S]);
    const uint32_t noff = static_cast<uint32_t>((n * ngroups + g) * 2);
    nrm[S] = __builtin_amdgcn_raw_buffer_load_b16(nbuf, g_live ? noff : kOutOfRange, 0, 0);
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  load_group(g_lo, Set0{});
  if (wg >= mat.wgs) return;

  // ---- the activation in LDS: hi row m and lo row batch + m of batch row
  // m.  Wave w stages batch rows w and w + 4; lane j of quarter q holds
  // elements 8j..8j+7 of group 4c+q.  Groups past K (up to the chunk
  // boundary) hold zeros, so every column the product reads is written.
  _Float16 *const zrow = xs + 2 * batch * xsr;
  for (int k = tid * 4; k < nchunks * kChunkCols; k += kThreads * 4)
    *reinterpret_cast<uint2 *>(zrow + k) = make_uint2(0u, 0u);
  for (int m = wave; m < batch; m += kWaves) {
    if (m != wave) load_x(m);
    float mx = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      if (c < nchunks) {
        if constexpr (ROT) {
          fwht128_unscaled(v[c], n);
#pragma unroll
          for (int i = 0; i < 8; ++i) v[c][i] *= kInvSqrt128;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(v[c][i]));
      }
    }
    mx = wave_max(mx);
    int e = 0;
    if (mx > 0.0f && mx <= 3.0e38f) {
      (void)frexpf(mx, &e);  // mx < 2^e
      e = max(-100, min(100, 15 - e));
    } else {
      e = 0;
    }
    const float scale = ldexpf(1.0f, e);
    if (lane == 0) unscale[m] = ldexpf(1.0f, -e);
    _Float16 *dhi = xs + m * xsr + q * CQ_GROUP + 8 * n;
    _Float16 *dlo = xs + (batch + m) * xsr + q * CQ_GROUP + 8 * n;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      if (c < nchunks) {
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          _Float16 h0, l0, h1, l1;
          split_f16(v[c][perm_code<SB>(2 * t)] * scale, h0, l0);
          split_f16(v[c][perm_code<SB>(2 * t + 1)] * scale, h1, l1);
          wh[t] = pack_h2(h0, h1);
          wl[t] = pack_h2(l0, l1);
        }
        *reinterpret_cast<uint4 *>(dhi + c * kChunkCols) = make_uint4(wh[0], wh[1], wh[2], wh[3]);
        *reinterpret_cast<uint4 *>(dlo + c * kChunkCols) = make_uint4(wl[0], wl[1], wl[2], wl[3]);
      }
    }
  }
  __syncthreads();

  // ---- the product.  A operand: MFMA row ma = lane % 16 reads the hi row
  // of batch row ma (ma < 8) or the lo row of batch row ma - 8, the zero row
  // past the batch; quarter q reads the 32 elements of a group that go with
  // its codes.
  const int ma = lane & 15;
  const int arow = ma < 8 ? (ma < batch ? ma : 2 * batch) : (ma - 8 < batch ? batch + ma - 8 : 2 * batch);
  const uint32_t a_base = static_cast<uint32_t>(arow * xsr + q * 32) * 2u;  // bytes
  const cq::MmaLevels &lev = a.lev[mi];
  MmaTable<SB> thi, tlo;
  thi.load(lev.hi);
  if constexpr (SPLIT) tlo.load(lev.lo);
  const float lscale = lev.lscale;

  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  auto compute_group = [&](int g, auto set_c) {
    constexpr int S = decltype(set_c)::value;
    const uint8_t *a_grp = reinterpret_cast<const uint8_t *>(xs) + a_base + g * CQ_GROUP * 2;
    // the products with the levels' hi and lo parts: two independent chains
    floatx4 gh = {0.f, 0.f, 0.f, 0.f}, gl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f16x8 af = *reinterpret_cast<const f16x8 *>(a_grp + t * 16);
      uint32_t o[4], ol[4];
      if constexpr (SPLIT)
        decode_piece2<SB>(thi, tlo, codes[S], t, o, ol);
      else
        decode_piece<SB>(thi, codes[S], t, o);
      gh = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, __builtin_bit_cast(f16x8, make_uint4(o[0], o[1], o[2], o[3])), gh,
                                                  0, 0, 0);
      if constexpr (SPLIT)
        gl = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            af, __builtin_bit_cast(f16x8, make_uint4(ol[0], ol[1], ol[2], ol[3])), gl, 0, 0, 0);
    }
    // the group's sum times its norm (times lscale), in fp32
    const float nf = static_cast<float>(__builtin_bit_cast(_Float16, nrm[S])) * lscale;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(nf, SPLIT ? gh[e] + gl[e] : gh[e], acc[e]);
  };
  // groups in pairs with unconditional loads (the load past the wave's range
  // reads zeros), then an odd last group
  int g = g_lo;
  for (; g + 2 <= g_hi; g += 2) {
    load_group(g + 1, Set1{});
    compute_group(g, Set0{});
    load_group(g + 2, Set0{});
    compute_group(g + 1, Set1{});
  }
  if (g < g_hi) compute_group(g, Set0{});

  // ---- the K-split waves of a block add their sums in wave order
  if (ksplit > 1) {
    red[wave][lane] = acc;
    __syncthreads();
    if (part == 0) {
#pragma unroll
      for (int p = 1; p < 4; ++p)
        if (p < ksplit) acc += red[wave + p][lane];
    }
  }
  if (part != 0) return;

  // D layout: lane l, register e -> MFMA row 4 (l / 16) + e, weight row
  // l % 16.  Rows 8..15 (lanes 32..63) are the lo parts' products: lane l
  // < 32 adds lane l + 32's sum to its own (the lane-half swap).
  const int64_t r = r0 + n;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[e]), __float_as_uint(acc[e]), false, false);
    const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const int m = 4 * q + e;
    if (q < 2 && m < batch && r < rows) y[static_cast<int64_t>(m) * rows + r] = tot * unscale[m];
  }
}

typedef void (*SmallKernel)(const float *, int32_t, int32_t, int32_t, int32_t, int32_t, SmallArgs);

template <bool ROT, bool SPLIT>
SmallKernel pick_rs(int sb) {
  if constexpr (SPLIT)
    return sb == 2 ? small_matvec_kernel<2, ROT, true>
                   : (sb == 3 ? small_matvec_kernel<3, ROT, true> : small_matvec_kernel<4, ROT, true>);
  else
    return sb == 1 ? small_matvec_kernel<1, ROT, false>
                   : (sb == 2 ? small_matvec_kernel<2, ROT, false>
                              : (sb == 3 ? small_matvec_kernel<3, ROT, false> : small_matvec_kernel<4, ROT, false>));
}

SmallKernel pick(int sb, bool rot, bool split) {
  if (sb == 1) split = false;  // binary levels are always exact
  return rot ? (split ? pick_rs<true, true>(sb) : pick_rs<true, false>(sb))
             : (split ? pick_rs<false, true>(sb) : pick_rs<false, false>(sb));
}

// Lets every variant take the largest dynamic LDS a launch asks for (once
// per process; the attribute is per kernel, not per device).
void allow_large_lds() {
  static std::once_flag once;
  std::call_once(once, [] {
    const size_t most = small_lds_bytes(kMaxCols, kMaxBatch);
    for (int sb = 1; sb <= 4; ++sb)
      for (int r = 0; r < 2; ++r)
        for (int sp = 0; sp < 2; ++sp)
          (void)hipFuncSetAttribute(reinterpret_cast<const void *>(pick(sb, r != 0, sp != 0)),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(most));
  });
}

}  // namespace

namespace cq {

bool small_matvec_fits(int64_t kpad, int64_t batch) {
  return kpad > 0 && kpad <= kMaxCols && kpad % CQ_GROUP == 0 && batch >= 1 && batch <= kMaxBatch;
}

hipError_t launch_small_matvec(const MultiItem *items, int n, const float *x, bool rotate, int64_t cols,
                               int64_t kpad, int64_t batch, hipStream_t s) {
  if (!small_matvec_fits(kpad, batch) || n < 0) return hipErrorInvalidValue;
  allow_large_lds();
  const int64_t ngroups = kpad / CQ_GROUP;
  const int ks_shift = ngroups >= 4 ? 2 : (ngroups >= 2 ? 1 : 0);
  const int64_t wg_rows = static_cast<int64_t>(kBlockRows) * (kWaves >> ks_shift);
  const size_t lds = small_lds_bytes(kpad, batch);
  // one launch per (storage width, low part or not), at most kMaxMats
  // matrices each, in order
  for (int sb = 1; sb <= 4; ++sb) {
    for (int sp = 0; sp < 2; ++sp) {
      SmallArgs a;
      int count = 0;
      int64_t max_wgs = 0;
      auto flush = [&]() -> hipError_t {
        if (count == 0) return hipSuccess;
        for (int i = count; i < kMaxMats; ++i) a.mat[i] = a.mat[count - 1], a.lev[i] = a.lev[count - 1];
        const int32_t xvec = cols % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
        pick(sb, rotate, sp != 0)<<<dim3(static_cast<unsigned>(max_wgs), static_cast<unsigned>(count)), kThreads,
                                    lds, s>>>(x, static_cast<int32_t>(rotate ? cols : kpad),
                                              static_cast<int32_t>(kpad / CQ_GROUP), static_cast<int32_t>(batch),
                                              xvec, ks_shift, a);
        count = 0;
        max_wgs = 0;
        return hipGetLastError();
      };
      for (int i = 0; i < n; ++i) {
        const MultiItem &it = items[i];
        if (storage_bits(it.bits) != sb || it.rows <= 0) continue;
        const MmaLevels lev = mma_levels(it.bits, it.lev);
        if ((lev.split != 0) != (sp != 0)) continue;
        const int64_t t = (it.rows + wg_rows - 1) / wg_rows;
        if (t >= (int64_t{1} << 31)) return hipErrorInvalidValue;
        a.mat[count] = SmallMat{it.blob, it.y, it.rows, t};
        a.lev[count] = lev;
        if (t > max_wgs) max_wgs = t;
        if (++count == kMaxMats) {
          const hipError_t e = flush();
          if (e != hipSuccess) return e;
        }
      }
      const hipError_t e = flush();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace cq
