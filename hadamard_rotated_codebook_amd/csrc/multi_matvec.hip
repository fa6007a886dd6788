// Several decode products that share one activation, in one launch, with the
// rotation done inside the kernel:
//
//   y_i[b][r] = sum_g float(norm_i[r][g]) * sum_j c_i[q_i[r][g*128+j]] * (H x[b])[g*128+j]
//
// for up to kMaxMats matrices W_i of one storage width and one column count.
// The rotated activation is computed once per workgroup and serves every row
// the workgroup reads (".cact" format post, "How the kernel reads it": rotate
// each 128-group once and reuse it for all rows; OpenNeedle reference notes,
// rotated-activation identity).  This is the path of a decode step's small
// projections -- Q, K, V and gate read the same normalised activation --
// where the number of launches and their latencies, not bytes, set the time.
//
// Limits (checked by the host): batch 1..8, cols_pad <= 4096 (one K slice,
// so there are no partial sums and no workspace).
//
// Design, per workgroup of 256 threads (4 waves, 32 rows each):
//  * the first chunk's codes and norms are requested before anything else,
//    so their HBM latency overlaps the activation's;
//  * each wave rotates whole batch rows of x with the butterfly every
//    rotating kernel uses (cq_fwht.h), keeping the row in registers until
//    its largest |xr| is known; the row is then scaled by the power of two
//    that puts that value in [2^14, 2^15) and stored to LDS as fp16, in the
//    decoders' slot order -- the same values, scale and order the
//    batched matrix-core kernel stages from a rotated xr, so the two paths
//    give identical results;
//  * the product is that kernel's: v_mfma_f32_16x16x32_f16 with A = the
//    batch (padding lanes read a zero row) and B = 16 rows x 32 k of
//    fp16(level * norm) decoded in registers, chunks of 512 columns in pairs
//    with the next chunk's loads in flight; out-of-range rows and groups
//    read zeros through the buffer range.
#include "cq_decode.h"
#include "cq_fwht.h"
#include "cq_internal.h"

namespace {

using namespace cqdev;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;                     // 4 waves
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerWave = 32;                  // two 16-row MFMA blocks
constexpr int kTileRows = kWaves * kRowsPerWave;  // 128
constexpr int kMaxCols = 4096;
constexpr int kChunkCols = 4 * CQ_GROUP;          // 512: one group per 16-lane quarter
constexpr int kMaxChunks = kMaxCols / kChunkCols;
constexpr int kMaxBatch = 8;
constexpr int kMaxMats = 8;
constexpr int kXPad = 8;                          // fp16 elements of padding per LDS row
constexpr uint32_t kOutOfRange = 0xffff0000u;     // a buffer offset past any range

struct MultiMat {
  const uint8_t *packed;
  const uint16_t *norms;  // fp16 bits [rows][ngroups]
  float *y;               // [batch][rows]
  int64_t rows;
  int32_t tile0;          // first workgroup (128-row tile) of this matrix
  int32_t unused;
};

struct MultiArgs {
  MultiMat mat[kMaxMats];
  cq::CodeLevels lev[kMaxMats];
  const float *x;  // [batch][cols], not rotated
  int64_t cols, kpad, row_bytes, ngroups;
  int32_t nmat, batch, xvec;
};

template <int SB>
__global__ __launch_bounds__(kThreads) void multi_matvec_kernel(MultiArgs a) {
  constexpr int GROUP_BYTES = CQ_GROUP * SB / 8;  // 32, 48, 64
  constexpr int GROUP_DW = GROUP_BYTES / 4;
  constexpr int XS = kMaxCols + kXPad;            // LDS row stride (fp16 elements)
  __shared__ __align__(16) _Float16 xs[(kMaxBatch + 1) * XS];  // row kMaxBatch stays zero
  __shared__ float unscale[kMaxBatch];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = blockIdx.x;

  // ---- this workgroup's matrix: the last one whose first tile is <= tile
  int mi = 0;
#pragma unroll
  for (int i = 1; i < kMaxMats; ++i)
    if (i < a.nmat && tile >= a.mat[i].tile0) mi = i;
  mi = __builtin_amdgcn_readfirstlane(mi);
  const MultiMat &M = a.mat[mi];
  const int64_t rows = M.rows;
  const int64_t r0 = static_cast<int64_t>(tile - M.tile0) * kTileRows + wave * kRowsPerWave;
  const int64_t live_rows = rows - r0 < kRowsPerWave ? (rows - r0 > 0 ? rows - r0 : 0) : kRowsPerWave;
  const __amdgpu_buffer_rsrc_t wbuf =
      buffer_rsrc(M.packed + r0 * a.row_bytes, static_cast<uint32_t>(live_rows * a.row_bytes));
  const __amdgpu_buffer_rsrc_t nbuf =
      buffer_rsrc(M.norms + r0 * a.ngroups, static_cast<uint32_t>(live_rows * a.ngroups * 2));
  const int ngroups = static_cast<int>(a.ngroups);
  const int nchunks = (ngroups + 3) / 4;

  // ---- lane roles: row n of each 16-row block; quarter q = group 4c+q of
  // chunk c (for the product) or of rotation round c (for the staging)
  const int n = lane & 15, q = lane >> 4;

  uint32_t codes[2][2][GROUP_DW];  // [set][block][dword]
  uint16_t nrm[2][2];
  auto load_chunk = [&](int c, auto set_c) {
    constexpr int S = decltype(set_c)::value;
    const int g = 4 * c + q;  // this lane's group
    const bool g_live = g < ngroups;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int row = 16 * b + n;
      const uint32_t woff = static_cast<uint32_t>(row * a.row_bytes + g * GROUP_BYTES);
      load_dwords<GROUP_DW>(wbuf, g_live ? woff : kOutOfRange, codes[S][b]);
      const uint32_t noff = static_cast<uint32_t>((row * ngroups + g) * 2);
      nrm[S][b] = __builtin_amdgcn_raw_buffer_load_b16(nbuf, g_live ? noff : kOutOfRange, 0, 0);
    }
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  load_chunk(0, Set0{});

  // ---- the rotated activation, fp16 in LDS.  Wave w owns batch rows w and
  // w + 4; round c rotates groups 4c..4c+3, one per 16-lane quarter, lane j
  // of the quarter holding elements 8j..8j+7 of its group.  Groups past K
  // (up to the chunk boundary) rotate zeros, so every column the product
  // reads is written.
  for (int k = tid * 4; k < nchunks * kChunkCols; k += kThreads * 4)
    *reinterpret_cast<uint2 *>(xs + kMaxBatch * XS + k) = make_uint2(0u, 0u);
  for (int m = wave; m < a.batch; m += kWaves) {
    const float *row = a.x + static_cast<int64_t>(m) * a.cols;
    float v[kMaxChunks][8];
    float mx = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      if (c < nchunks) {
        load8_f32(row, static_cast<int64_t>(4 * c + q) * CQ_GROUP + 8 * n, a.cols, a.xvec != 0, v[c]);
        fwht128_unscaled(v[c], n);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[c][i] *= kInvSqrt128;
          mx = fmaxf(mx, fabsf(v[c][i]));
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
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
  const int m_a = (lane & 15) < a.batch ? (lane & 15) : kMaxBatch;
  const uint32_t a_base = static_cast<uint32_t>(m_a * XS + q * CQ_GROUP) * 2u;  // bytes
  const cq::CodeLevels &lev = a.lev[mi];

  floatx4 acc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
  auto compute_chunk = [&](int c, auto set_c) {
    constexpr int S = decltype(set_c)::value;
    MmaTable<SB> tab[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) tab[b].build(lev, static_cast<float>(__builtin_bit_cast(_Float16, nrm[S][b])));
    // a chunk past the end (the odd one of the last pair) rereads the last
    // chunk's activations; its weights are zero
    const int cc = c < nchunks ? c : nchunks - 1;
    const uint8_t *a_chunk = reinterpret_cast<const uint8_t *>(xs) + a_base + cc * kChunkCols * 2;
    f16x8 af[CQ_GROUP / 8];
#pragma unroll
    for (int s = 0; s < CQ_GROUP / 8; ++s) af[s] = *reinterpret_cast<const f16x8 *>(a_chunk + s * 16);
#pragma unroll
    for (int s = 0; s < CQ_GROUP / 8; ++s) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        uint32_t o[4];
        decode_step<SB>(tab[b], codes[S][b], s, o);
        const f16x8 bv = __builtin_bit_cast(f16x8, make_uint4(o[0], o[1], o[2], o[3]));
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[s], bv, acc[b], 0, 0, 0);
      }
    }
  };
  // chunk pairs with unconditional loads: chunks at or past nchunks load
  // zero norms and add nothing
  for (int c = 0; c < nchunks; c += 2) {
    load_chunk(c + 1, Set1{});
    compute_chunk(c, Set0{});
    load_chunk(c + 2, Set0{});
    compute_chunk(c + 1, Set1{});
  }

  // D layout: lane l, register e -> batch row 4 (l / 16) + e, weight row l % 16
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int64_t r = r0 + 16 * b + n;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * q + e;
      if (m < a.batch && r < rows) M.y[static_cast<int64_t>(m) * rows + r] = acc[b][e] * unscale[m];
    }
  }
}

}  // namespace

namespace cq {

bool multi_matvec_fits(int64_t kpad, int64_t batch) {
  return kpad > 0 && kpad <= kMaxCols && kpad % CQ_GROUP == 0 && batch >= 1 && batch <= kMaxBatch;
}

hipError_t launch_multi_matvec(const MultiItem *items, int n, const float *x, int64_t cols, int64_t kpad,
                               int64_t batch, hipStream_t s) {
  if (!multi_matvec_fits(kpad, batch) || n < 0) return hipErrorInvalidValue;
  // One launch per storage width, at most kMaxMats matrices each, in order.
  for (int sb = 2; sb <= 4; ++sb) {
    MultiArgs a;
    int count = 0, tiles = 0;
    auto flush = [&]() -> hipError_t {
      if (count == 0) return hipSuccess;
      a.nmat = count;
      a.x = x;
      a.cols = cols;
      a.kpad = kpad;
      a.row_bytes = kpad * sb / 8;
      a.ngroups = kpad / CQ_GROUP;
      a.batch = static_cast<int32_t>(batch);
      a.xvec = cols % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
      for (int i = count; i < kMaxMats; ++i) a.mat[i] = a.mat[count - 1], a.lev[i] = a.lev[count - 1];
      const dim3 grid(static_cast<unsigned>(tiles));
      switch (sb) {
        case 2: multi_matvec_kernel<2><<<grid, kThreads, 0, s>>>(a); break;
        case 3: multi_matvec_kernel<3><<<grid, kThreads, 0, s>>>(a); break;
        default: multi_matvec_kernel<4><<<grid, kThreads, 0, s>>>(a); break;
      }
      count = 0;
      tiles = 0;
      return hipGetLastError();
    };
    for (int i = 0; i < n; ++i) {
      const MultiItem &it = items[i];
      if (storage_bits(it.bits) != sb || it.rows <= 0) continue;
      const int64_t t = (it.rows + kTileRows - 1) / kTileRows;
      if (t > (int64_t{1} << 30) - tiles) return hipErrorInvalidValue;
      MultiMat &m = a.mat[count];
      m.packed = it.blob;
      m.norms = reinterpret_cast<const uint16_t *>(it.blob + it.rows * (kpad * sb / 8));
      m.y = it.y;
      m.rows = it.rows;
      m.tile0 = tiles;
      m.unused = 0;
      a.lev[count] = it.lev;
      tiles += static_cast<int>(t);
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
