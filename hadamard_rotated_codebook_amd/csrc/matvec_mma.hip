// Decode product on the fp16 matrix cores, for batches of 2..8 vectors and
// for small matrices at batch 1 (where the lookup tables' prologue dominates):
//
//   y[b][r] = sum_g float(norm[r][g]) * sum_j c[q[r][g*128+j]] * xr[b][g*128+j]
//
// computed as a thin product Xr . V^T with V[r][g*128+j] = fp16(c[q] * norm),
// i.e. by the rotated-activation identity (OpenNeedle reference notes) the
// product with the dequantised matrix, reading every packed byte of W once
// for the whole batch (".cact" format post, "How the kernel reads it": the
// indices are decoded in registers, no weight is written to memory).
//
// Why not the lookup tables of the batch-1 kernel: their entries depend on
// the activation, so a batch of B vectors needs B tables (B times the LDS) or
// B passes over W.  Here the decoded weights are shared by the batch and the
// per-vector work is one MFMA operand.
//
// Design:
//  * v_mfma_f32_16x16x32_f16: A = activations (batch rows padded to 16, the
//    padding lanes read zeros), B = 16 weight rows x 32 k.  A wave owns 32
//    rows (two 16-row blocks sharing each A fragment); a 256-thread workgroup
//    owns a K slice of up to 4096 columns and walks 128-row tiles.
//  * K order inside a 512-column chunk: the 16-lane quarter q of a wave takes
//    group 4c+q whole, so each lane loads the 128 codes of one (row, group)
//    -- 32/48/64 contiguous bytes -- and builds one decode table (level *
//    norm, fp16) for them; the A operand uses the same k order.  The sum over
//    k is unchanged by the permutation.
//  * The slice's activations are staged once per workgroup in LDS as fp16,
//    scaled per batch row by a power of two that puts the slice's largest
//    |xr| in [2^14, 2^15); the scale is undone exactly on the fp32 result.
//  * Codes and norms of the next chunk are loaded while the current one is
//    decoded and multiplied.  Rows past the end, and groups past K, read
//    zeros through the buffer range (a zero norm makes a zero table).
//  * With more than one K slice the slices' partial sums go to the caller's
//    workspace and are added in slice order by the combine kernel.
#include <type_traits>

#include "cq_decode.h"
#include "cq_internal.h"

namespace {

using namespace cqdev;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;                  // 4 waves
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerWave = 32;               // two 16-row MFMA blocks
constexpr int kTileRows = kWaves * kRowsPerWave;  // 128
constexpr int kMaxSliceCols = 4096;
constexpr int kChunkCols = 4 * CQ_GROUP;       // 512: one group per 16-lane quarter
constexpr int kMaxBatch = 8;
constexpr int kXPad = 8;                       // fp16 elements of padding per LDS activation row
constexpr uint32_t kOutOfRange = 0xffff0000u;  // a buffer offset past any range (ranges are < 2^31)

struct MmArgs {
  const uint8_t *packed;
  const uint16_t *norms;  // fp16 bits [rows][ngroups]
  const float *xr;        // [batch][kpad]
  float *out;             // y [batch][rows] (one slice) or partial [nslice][batch][rows]
  int64_t rows, kpad, row_bytes, ngroups;
  int32_t batch, slice_cols, nslice, per_slice, ntiles;
  cq::CodeLevels lev;
};

template <int SB>
__global__ __launch_bounds__(kThreads) void matvec_mma_kernel(MmArgs a) {
  constexpr int GROUP_BYTES = CQ_GROUP * SB / 8;  // 32, 48, 64
  constexpr int GROUP_DW = GROUP_BYTES / 4;
  constexpr int XS = kMaxSliceCols + kXPad;      // LDS row stride (fp16 elements)
  __shared__ __align__(16) _Float16 xs[(kMaxBatch + 1) * XS];  // row kMaxBatch stays zero
  __shared__ float unscale[kMaxBatch];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slice = blockIdx.x % a.nslice;
  const int first_tile = blockIdx.x / a.nslice;
  const int64_t c0 = static_cast<int64_t>(slice) * a.slice_cols;  // first column of the slice
  const int ncols = static_cast<int>(a.kpad - c0 < a.slice_cols ? a.kpad - c0 : a.slice_cols);

  // ---- the slice's activations: max |xr| per batch row, then fp16 copies.
  // Thread t covers batch row t / 32 (kMaxBatch rows of 32 threads).
  {
    const int m = tid >> 5, part = tid & 31;
    const bool live = m < a.batch;
    // only the chunks the products read are staged (and zeroed in the zero row)
    const int staged = (ncols + kChunkCols - 1) / kChunkCols * kChunkCols;
    for (int k = tid * 4; k < staged; k += kThreads * 4)
      *reinterpret_cast<uint2 *>(xs + kMaxBatch * XS + k) = make_uint2(0u, 0u);
    const float *src = a.xr + static_cast<int64_t>(live ? m : 0) * a.kpad + c0;
    float mx = 0.0f;
    for (int k = part * 4; k < ncols; k += 32 * 4) {
      const float4 v = *reinterpret_cast<const float4 *>(src + k);
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 32));
    int e = 0;
    if (mx > 0.0f && mx <= 3.0e38f) {
      (void)frexpf(mx, &e);  // mx < 2^e
      e = max(-100, min(100, 15 - e));
    } else {
      e = 0;
    }
    const float scale = ldexpf(1.0f, e);
    if (part == 0 && m < kMaxBatch) unscale[m] = ldexpf(1.0f, -e);
    // Each block of 8 columns is stored in the decoder's slot order, so that
    // A and B pair the same k in every MFMA slot.
    _Float16 *dst = xs + m * XS;
    for (int k = part * 8; k < staged; k += 32 * 8) {
      float v[8];
      float4 u0 = make_float4(0.f, 0.f, 0.f, 0.f), u1 = u0;
      if (live && k < ncols) {
        u0 = *reinterpret_cast<const float4 *>(src + k);
        u1 = *reinterpret_cast<const float4 *>(src + k + 4);
      }
      v[0] = u0.x, v[1] = u0.y, v[2] = u0.z, v[3] = u0.w, v[4] = u1.x, v[5] = u1.y, v[6] = u1.z, v[7] = u1.w;
      uint32_t w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        w[t] = pack2<_Float16>(v[perm_code<SB>(2 * t)] * scale, v[perm_code<SB>(2 * t + 1)] * scale);
      *reinterpret_cast<uint4 *>(dst + k) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  __syncthreads();

  // ---- lane roles: row n of each 16-row block, quarter q = group 4c+q of a
  // chunk; for the A operand, batch row m = lane % 16 (zero when m >= batch).
  const int n = lane & 15, q = lane >> 4;
  const int m_a = (lane & 15) < a.batch ? (lane & 15) : kMaxBatch;  // padding lanes read the zero row
  const uint32_t a_base = static_cast<uint32_t>(m_a * XS + q * CQ_GROUP) * 2u;  // bytes
  const int slice_groups = a.slice_cols / CQ_GROUP;
  const int nchunks = (ncols + kChunkCols - 1) / kChunkCols;

  for (int tile = first_tile; tile < a.ntiles; tile += a.per_slice) {
    const int64_t r0 = static_cast<int64_t>(tile) * kTileRows + wave * kRowsPerWave;
    const int64_t live_rows = a.rows - r0 < kRowsPerWave ? (a.rows - r0 > 0 ? a.rows - r0 : 0) : kRowsPerWave;
    const __amdgpu_buffer_rsrc_t wbuf =
        buffer_rsrc(a.packed + r0 * a.row_bytes, static_cast<uint32_t>(live_rows * a.row_bytes));
    const __amdgpu_buffer_rsrc_t nbuf =
        buffer_rsrc(a.norms + r0 * a.ngroups, static_cast<uint32_t>(live_rows * a.ngroups * 2));

    uint32_t codes[2][2][GROUP_DW];  // [set][block][dword]
    uint16_t nrm[2][2];
    auto load_chunk = [&](int c, auto set_c) {
      constexpr int S = decltype(set_c)::value;
      const int64_t g = static_cast<int64_t>(slice) * slice_groups + 4 * c + q;  // this lane's group
      const bool g_live = g < a.ngroups && 4 * c + q < slice_groups;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int row = 16 * b + n;
        const uint32_t woff = static_cast<uint32_t>(row * a.row_bytes + g * GROUP_BYTES);
        load_dwords<GROUP_DW>(wbuf, g_live ? woff : kOutOfRange, codes[S][b]);
        const uint32_t noff = static_cast<uint32_t>((row * a.ngroups + g) * 2);
        nrm[S][b] = __builtin_amdgcn_raw_buffer_load_b16(nbuf, g_live ? noff : kOutOfRange, 0, 0);
      }
    };

    floatx4 acc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    auto compute_chunk = [&](int c, auto set_c) {
      constexpr int S = decltype(set_c)::value;
      // byte-plane tables and the permuted decoders at 2 and 4 bits
      MmaTable<SB> tab[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) tab[b].build(a.lev, static_cast<float>(__builtin_bit_cast(_Float16, nrm[S][b])));
      // A fragments of the chunk's 16 k steps, all read up front (a chunk
      // past the slice -- the odd one of the last pair -- rereads the last
      // chunk; its weights are zero).
      const int cc = c < nchunks ? c : nchunks - 1;
      const uint8_t *a_chunk = reinterpret_cast<const uint8_t *>(xs) + a_base + cc * kChunkCols * 2;
      f16x8 af[CQ_GROUP / 8];
#pragma unroll
      for (int s = 0; s < CQ_GROUP / 8; ++s) af[s] = *reinterpret_cast<const f16x8 *>(a_chunk + s * 16);
      // 16 k steps of 8 codes per lane
#pragma unroll
      for (int s = 0; s < CQ_GROUP / 8; ++s) {
        const f16x8 av = af[s];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          uint32_t o[4];
          decode_step<SB>(tab[b], codes[S][b], s, o);
          const f16x8 bv = __builtin_bit_cast(f16x8, make_uint4(o[0], o[1], o[2], o[3]));
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[b], 0, 0, 0);
        }
      }
    };

    using Set0 = std::integral_constant<int, 0>;
    using Set1 = std::integral_constant<int, 1>;
    // Chunks in pairs, every load and product unconditional (a load on only
    // some paths makes the compiler wait for all outstanding loads): chunks
    // at or past nchunks load zero norms and add nothing.
    load_chunk(0, Set0{});
    for (int c = 0; c < nchunks; c += 2) {
      load_chunk(c + 1, Set1{});
      compute_chunk(c, Set0{});
      load_chunk(c + 2, Set0{});
      compute_chunk(c + 1, Set1{});
    }

    // D layout: lane l, register e -> batch row 4 (l / 16) + e, weight row l % 16.
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t row = r0 + 16 * b + n;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 4 * q + e;
        if (m < a.batch && row < a.rows) {
          const float v = acc[b][e] * unscale[m];
          const int64_t at = (static_cast<int64_t>(slice) * a.batch + m) * a.rows + row;
          a.out[at] = v;
        }
      }
    }
  }
}

struct MmShape {
  int slice_cols, nslice, ntiles, per_slice;
};

MmShape mm_shape(int64_t rows, int64_t kpad) {
  MmShape s;
  const int64_t chunks = (kpad + kChunkCols - 1) / kChunkCols;
  const int64_t chunks_per_slice = kMaxSliceCols / kChunkCols;
  s.nslice = static_cast<int>((chunks + chunks_per_slice - 1) / chunks_per_slice);
  // spread the columns evenly over the slices, in whole chunks
  s.slice_cols = static_cast<int>((chunks + s.nslice - 1) / s.nslice) * kChunkCols;
  s.ntiles = static_cast<int>((rows + kTileRows - 1) / kTileRows);
  constexpr int kTargetGroups = 512;  // about two workgroups per CU
  int per = kTargetGroups / s.nslice;
  if (per < 1) per = 1;
  if (per > s.ntiles) per = s.ntiles;
  s.per_slice = per;
  return s;
}

}  // namespace

namespace cq {

uint64_t matvec_mma_workspace_bytes(int64_t rows, int64_t kpad, int64_t batch) {
  if (rows <= 0 || kpad <= 0 || batch <= 0) return 0;
  const MmShape s = mm_shape(rows, kpad);
  if (s.nslice <= 1) return 0;
  return static_cast<uint64_t>(s.nslice) * batch * rows * 4;
}

hipError_t launch_matvec_mma(const uint8_t *blob, int bits, int64_t rows, int64_t kpad, const CodeLevels &lev,
                             const float *xr, int64_t batch, float *y, void *workspace, hipStream_t s) {
  if (batch < 1 || batch > kMaxBatch || kpad % CQ_GROUP != 0) return hipErrorInvalidValue;
  const int sb = storage_bits(bits);
  const MmShape sh = mm_shape(rows, kpad);
  MmArgs a;
  a.packed = blob;
  a.row_bytes = kpad * sb / 8;
  a.norms = reinterpret_cast<const uint16_t *>(blob + rows * a.row_bytes);
  a.xr = xr;
  a.rows = rows;
  a.kpad = kpad;
  a.ngroups = kpad / CQ_GROUP;
  a.batch = static_cast<int32_t>(batch);
  a.slice_cols = sh.slice_cols;
  a.nslice = sh.nslice;
  a.per_slice = sh.per_slice;
  a.ntiles = sh.ntiles;
  a.lev = lev;
  a.out = sh.nslice > 1 ? static_cast<float *>(workspace) : y;
  // 32-bit tile-relative offsets: 32 rows of packed bytes or norms.
  if (static_cast<int64_t>(kRowsPerWave) * a.row_bytes >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(sh.nslice) * sh.per_slice));
  switch (sb) {
    case 1: matvec_mma_kernel<1><<<grid, kThreads, 0, s>>>(a); break;
    case 2: matvec_mma_kernel<2><<<grid, kThreads, 0, s>>>(a); break;
    case 3: matvec_mma_kernel<3><<<grid, kThreads, 0, s>>>(a); break;
    default: matvec_mma_kernel<4><<<grid, kThreads, 0, s>>>(a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sh.nslice <= 1) return e;
  return launch_combine(a.out, batch * rows, sh.nslice, y, s);
}

}  // namespace cq
