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
// Design, per workgroup of 256 threads (4 waves):
//  * the unit of work is a 16-row block; ksplit (1, 2 or 4) waves share a
//    block, each taking a contiguous range of its 512-column chunks, so a
//    workgroup covers 64, 32 or 16 rows.  The waves' fp32 accumulators are
//    added in wave order through LDS: results do not depend on scheduling;
//  * each wave requests its batch row of the activation first, then its
//    first chunk's codes and norms, so the code latency overlaps the
//    rotation; the row is rotated with the butterfly every rotating kernel
//    uses (cq_fwht.h), held in registers until its largest |xr| is known,
//    scaled by the power of two that puts that value in [2^14, 2^15) and
//    stored to LDS as fp16 in the decoders' slot order.  With or without
//    ROT the staged values are identical, so both give the same results;
//  * the product: v_mfma_f32_16x16x32_f16 with A = the batch (padding lanes
//    read a zero row) and B = 16 rows x 32 k of fp16(level * norm) decoded in
//    registers; chunks in pairs with the next chunk's loads in flight, and an
//    odd last chunk on its own.  Out-of-range rows and groups read zeros
//    through the buffer range.
#include "cq_decode.h"
#include "cq_fwht.h"
#include "cq_internal.h"

namespace {

using namespace cqdev;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;                     // 4 waves
constexpr int kWaves = kThreads / 64;
constexpr int kBlockRows = 16;                    // one MFMA block
constexpr int kMaxCols = 4096;
constexpr int kChunkCols = 4 * CQ_GROUP;          // 512: one group per 16-lane quarter
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
  cq::CodeLevels lev[kMaxMats];
};

// The scalar arguments come first: the compiler asks the dispatcher to
// preload them into SGPRs (-amdgpu-kernarg-preload-count=6), so the
// activation loads go out before any argument load returns.
//   x         ROT: x [batch][cols]; otherwise xr [batch][kpad]
//   xstride   cols (ROT) or kpad, in floats
//   xvec      ROT: x rows allow 16-byte loads (cols % 8 == 0, x 16-byte aligned)
//   ks_shift  ksplit = 1 << ks_shift waves per 16-row block
template <int SB, bool ROT>
__global__ __launch_bounds__(kThreads) void small_matvec_kernel(const float *x, int32_t xstride, int32_t ngroups,
                                                                int32_t batch, int32_t xvec, int32_t ks_shift,
                                                                SmallArgs a) {
  constexpr int GROUP_BYTES = CQ_GROUP * SB / 8;  // 32, 48, 64
  constexpr int GROUP_DW = GROUP_BYTES / 4;
  constexpr int XS = kMaxCols + kXPad;            // LDS row stride (fp16 elements)
  __shared__ __align__(16) _Float16 xs[(kMaxBatch + 1) * XS];  // row kMaxBatch stays zero
  __shared__ float unscale[kMaxBatch];
  __shared__ floatx4 red[kWaves][64];            // the K-split waves' accumulators

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = blockIdx.x, mi = blockIdx.y;

  // ---- lane roles: row n of the block; quarter q = group 4c+q of chunk c
  // (for the product and for the staging)
  const int n = lane & 15, q = lane >> 4;
  const int nchunks = (ngroups + 3) / 4;

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
  const int c_lo = part * nchunks >> ks, c_hi = (part + 1) * nchunks >> ks;

  uint32_t codes[2][GROUP_DW];  // [set][dword]
  uint16_t nrm[2];
  auto load_chunk = [&](int c, auto set_c) {
    constexpr int S = decltype(set_c)::value;
    const int g = 4 * c + q;  // this lane's group
    const bool g_live = g < ngroups && c < c_hi;
    const uint32_t woff = static_cast<uint32_t>(n * row_bytes + g * GROUP_BYTES);
    load_dwords<GROUP_DW>(wbuf, g_live ? woff : kOutOfRange, codes[S]);
    const uint32_t noff = static_cast<uint32_t>((n * ngroups + g) * 2);
    nrm[S] = __builtin_amdgcn_raw_buffer_load_b16(nbuf, g_live ? noff : kOutOfRange, 0, 0);
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  load_chunk(c_lo, Set0{});
  if (wg >= mat.wgs) return;

  // ---- the activation, fp16 in LDS.  Wave w stages batch rows w and w + 4;
  // lane j of quarter q holds elements 8j..8j+7 of group 4c+q.  Groups past
  // K (up to the chunk boundary) hold zeros, so every column the product
  // reads is written.
  for (int k = tid * 4; k < nchunks * kChunkCols; k += kThreads * 4)
    *reinterpret_cast<uint2 *>(xs + kMaxBatch * XS + k) = make_uint2(0u, 0u);
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
    _Float16 *dst = xs + m * XS + q * CQ_GROUP + 8 * n;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      if (c < nchunks) {
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          w[t] = pack2<_Float16>(v[c][perm_code<SB>(2 * t)] * scale, v[c][perm_code<SB>(2 * t + 1)] * scale);
        *reinterpret_cast<uint4 *>(dst + c * kChunkCols) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
  __syncthreads();

  // ---- the product; for the A operand, batch row m = lane % 16 (the zero
  // row when m >= batch)
  const int m_a = (lane & 15) < batch ? (lane & 15) : kMaxBatch;
  const uint32_t a_base = static_cast<uint32_t>(m_a * XS + q * CQ_GROUP) * 2u;  // bytes
  const cq::CodeLevels &lev = a.lev[mi];

  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  auto compute_chunk = [&](int c, auto set_c) {
    constexpr int S = decltype(set_c)::value;
    MmaTable<SB> tab;
    tab.build(lev, static_cast<float>(__builtin_bit_cast(_Float16, nrm[S])));
    const uint8_t *a_chunk = reinterpret_cast<const uint8_t *>(xs) + a_base + c * kChunkCols * 2;
    f16x8 af[CQ_GROUP / 8];
#pragma unroll
    for (int s = 0; s < CQ_GROUP / 8; ++s) af[s] = *reinterpret_cast<const f16x8 *>(a_chunk + s * 16);
#pragma unroll
    for (int s = 0; s < CQ_GROUP / 8; ++s) {
      uint32_t o[4];
      decode_step<SB>(tab, codes[S], s, o);
      const f16x8 bv = __builtin_bit_cast(f16x8, make_uint4(o[0], o[1], o[2], o[3]));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[s], bv, acc, 0, 0, 0);
    }
  };
  // chunk pairs with unconditional loads (the load past the wave's range
  // reads zeros), then an odd last chunk
  int c = c_lo;
  for (; c + 2 <= c_hi; c += 2) {
    load_chunk(c + 1, Set1{});
    compute_chunk(c, Set0{});
    load_chunk(c + 2, Set0{});
    compute_chunk(c + 1, Set1{});
  }
  if (c < c_hi) compute_chunk(c, Set0{});

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

  // D layout: lane l, register e -> batch row 4 (l / 16) + e, weight row l % 16
  const int64_t r = r0 + n;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m = 4 * q + e;
    if (m < batch && r < rows) y[static_cast<int64_t>(m) * rows + r] = acc[e] * unscale[m];
  }
}

typedef void (*SmallKernel)(const float *, int32_t, int32_t, int32_t, int32_t, int32_t, SmallArgs);

template <bool ROT>
SmallKernel pick_rot(int sb) {
  return sb == 1 ? small_matvec_kernel<1, ROT>
                 : (sb == 2 ? small_matvec_kernel<2, ROT>
                            : (sb == 3 ? small_matvec_kernel<3, ROT> : small_matvec_kernel<4, ROT>));
}

SmallKernel pick(int sb, bool rot) { return rot ? pick_rot<true>(sb) : pick_rot<false>(sb); }

}  // namespace

namespace cq {

bool small_matvec_fits(int64_t kpad, int64_t batch) {
  return kpad > 0 && kpad <= kMaxCols && kpad % CQ_GROUP == 0 && batch >= 1 && batch <= kMaxBatch;
}

hipError_t launch_small_matvec(const MultiItem *items, int n, const float *x, bool rotate, int64_t cols,
                               int64_t kpad, int64_t batch, hipStream_t s) {
  if (!small_matvec_fits(kpad, batch) || n < 0) return hipErrorInvalidValue;
  const int nchunks = static_cast<int>((kpad + kChunkCols - 1) / kChunkCols);
  const int ks_shift = nchunks >= 4 ? 2 : (nchunks >= 2 ? 1 : 0);
  const int64_t wg_rows = static_cast<int64_t>(kBlockRows) * (kWaves >> ks_shift);
  // one launch per storage width, at most kMaxMats matrices each, in order
  for (int sb = 1; sb <= 4; ++sb) {
    SmallArgs a;
    int count = 0;
    int64_t max_wgs = 0;
    auto flush = [&]() -> hipError_t {
      if (count == 0) return hipSuccess;
      for (int i = count; i < kMaxMats; ++i) a.mat[i] = a.mat[count - 1], a.lev[i] = a.lev[count - 1];
      const int32_t xvec = cols % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
      pick(sb, rotate)<<<dim3(static_cast<unsigned>(max_wgs), static_cast<unsigned>(count)), kThreads, 0, s>>>(
          x, static_cast<int32_t>(rotate ? cols : kpad), static_cast<int32_t>(kpad / CQ_GROUP),
          static_cast<int32_t>(batch), xvec, ks_shift, a);
      count = 0;
      max_wgs = 0;
      return hipGetLastError();
    };
    for (int i = 0; i < n; ++i) {
      const MultiItem &it = items[i];
      if (storage_bits(it.bits) != sb || it.rows <= 0) continue;
      const int64_t t = (it.rows + wg_rows - 1) / wg_rows;
      if (t >= (int64_t{1} << 31)) return hipErrorInvalidValue;
      a.mat[count] = SmallMat{it.blob, it.y, it.rows, t};
      a.lev[count] = it.lev;
      if (t > max_wgs) max_wgs = t;
      if (++count == kMaxMats) {
        const hipError_t e = flush();
        if (e != hipSuccess) return e;
      }
    }
    const hipError_t e = flush();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace cq
