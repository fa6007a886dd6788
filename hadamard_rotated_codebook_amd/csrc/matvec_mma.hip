// Decode product on the fp16 matrix cores, for batches of 2..8 vectors and
// for matrices at batch 1 too small for the lookup tables but too wide for
// the small-matrix kernel:
//
//   y[b][r] = sum_g float(norm[r][g]) * sum_j c[q[r][g*128+j]] * xr[b][g*128+j]
//
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
// Precision (the same scheme as the small-matrix kernel): both MFMA operands
// carry 22 significant bits as fp16 hi + lo parts -- the activation's parts
// in MFMA rows 0..7 and 8..15 (a batch of at most 8), the level's parts in two
// MFMAs per k step (cq::MmaLevels; one for binary and ternary levels, which
// are exact) -- every product is exact in fp32, each group is summed on its
// own and multiplied by its fp16 norm (times lscale) in fp32.
//
// Design:
//  * v_mfma_f32_16x16x32_f16: A = the hi and lo rows of the batch (the rows
//    past the batch read a zero row), B = 16 weight rows x 32 k.  A wave owns
//    32 rows (two 16-row blocks sharing each A fragment); a 512-thread
//    workgroup owns a K slice of up to 4096 columns, stages its activations
//    once, and walks 256-row tiles.
//  * K order: every k step of 32 covers one group.  The 16-lane quarter q of
//    a wave owns codes 32q..32q+31 of each group of its row (a 4/8/12/16-byte
//    piece), k step t its codes 8t..8t+7; the A operand follows the same
//    order.  Four groups (a 512-column chunk) are in flight at a time, their
//    sums independent chains.  The loads are of whole groups (a lane reads
//    group 4c+q of its rows, 16 bytes per load), and the quarters trade the
//    pieces with lane swaps: loads of 8-byte pieces and single norms made
//    the texture addresser the bound.
//  * The slice's activations are staged once per workgroup in LDS, scaled
//    per batch row by a power of two that puts the slice's largest |xr| in
//    [2^14, 2^15); the scale is undone exactly on the fp32 result.
//  * Codes and norms of the next chunk are loaded while the current one is
//    decoded and multiplied.  Rows past the end, and groups past K, read
//    zeros through the buffer range (their norms are zero).
//  * With more than one K slice the slices' partial sums go to the caller's
//    workspace and are added in slice order by the combine kernel.
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "cq_decode.h"
#include "cq_fwht.h"
#include "cq_internal.h"

namespace {

using namespace cqdev;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;                  // 8 waves
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerWave = 32;               // two 16-row MFMA blocks
constexpr int kTileRows = kWaves * kRowsPerWave;  // 256
constexpr int kMaxSliceCols = 4096;
constexpr int kChunkCols = 4 * CQ_GROUP;       // 512: four groups
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
  cq::MmaLevels lev;
};

__device__ inline uint32_t pack_h2(_Float16 a, _Float16 b) { return __builtin_bit_cast(uint32_t, f16x2{a, b}); }

// Dynamic LDS: hi rows [batch], lo rows [batch] and a zero row, each
// slice_cols + kXPad fp16 values.
size_t mm_lds_bytes(int64_t slice_cols, int64_t batch) {
  return static_cast<size_t>((2 * batch + 1) * (slice_cols + kXPad) * 2);
}

template <int SB, bool SPLIT>
__global__ __launch_bounds__(kThreads) void matvec_mma_kernel(MmArgs a) {
  constexpr int GROUP_BYTES = CQ_GROUP * SB / 8;  // 16, 32, 48, 64
  constexpr int PIECE_BYTES = 4 * SB;             // a lane's 32 codes of a group
  extern __shared__ __align__(16) _Float16 xs[];  // [2 * batch + 1][xsr]
  __shared__ float unscale[kMaxBatch];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slice = blockIdx.x % a.nslice;
  const int first_tile = blockIdx.x / a.nslice;
  const int64_t c0 = static_cast<int64_t>(slice) * a.slice_cols;  // first column of the slice
  const int ncols = static_cast<int>(a.kpad - c0 < a.slice_cols ? a.kpad - c0 : a.slice_cols);
  const int nchunks = (ncols + kChunkCols - 1) / kChunkCols;
  const int staged = nchunks * kChunkCols;  // the columns the products read
  const int xsr = a.slice_cols + kXPad;     // LDS row stride (fp16 elements)
  const int batch = a.batch;

  // ---- the slice's activations: wave m stages batch row m (hi row m, lo
  // row batch + m), every thread zeroes part of the zero row.  Each block of
  // 8 columns is stored in the decoder's slot order, so that A and B pair the
  // same k in every MFMA slot.
  {
    _Float16 *const zrow = xs + 2 * batch * xsr;
    for (int k = tid * 4; k < staged; k += kThreads * 4) *reinterpret_cast<uint2 *>(zrow + k) = make_uint2(0u, 0u);
    if (wave < batch) {
      const int m = wave;
      const float *src = a.xr + static_cast<int64_t>(m) * a.kpad + c0;
      float mx = 0.0f;
      for (int k = lane * 4; k < ncols; k += 64 * 4) {
        const float4 v = *reinterpret_cast<const float4 *>(src + k);
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
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
      _Float16 *dhi = xs + m * xsr, *dlo = xs + (batch + m) * xsr;
      for (int k = lane * 8; k < staged; k += 64 * 8) {
        // v: the block's 8 slots in the decoder's order.  Binary: slots
        // 2u, 2u + 1 of block t of a 32-column piece are columns 4t + u and
        // 4t + u + 16 (decode1_sign); otherwise perm_code within the block.
        float v[8];
        float4 u0 = make_float4(0.f, 0.f, 0.f, 0.f), u1 = u0;
        if (k < ncols) {
          if constexpr (SB == 1) {
            const int pc = (k & ~31) + 4 * ((k >> 3) & 3);
            u0 = *reinterpret_cast<const float4 *>(src + pc);
            u1 = *reinterpret_cast<const float4 *>(src + pc + 16);
          } else {
            u0 = *reinterpret_cast<const float4 *>(src + k);
            u1 = *reinterpret_cast<const float4 *>(src + k + 4);
          }
        }
        if constexpr (SB == 1) {
          v[0] = u0.x, v[1] = u1.x, v[2] = u0.y, v[3] = u1.y, v[4] = u0.z, v[5] = u1.z, v[6] = u0.w, v[7] = u1.w;
        } else {
          const float n8[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = n8[perm_code<SB>(e)];
        }
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          _Float16 h0, l0, h1, l1;
          split_f16(v[2 * t] * scale, h0, l0);
          split_f16(v[2 * t + 1] * scale, h1, l1);
          wh[t] = pack_h2(h0, h1);
          wl[t] = pack_h2(l0, l1);
        }
        *reinterpret_cast<uint4 *>(dhi + k) = make_uint4(wh[0], wh[1], wh[2], wh[3]);
        *reinterpret_cast<uint4 *>(dlo + k) = make_uint4(wl[0], wl[1], wl[2], wl[3]);
      }
    }
  }
  __syncthreads();

  // ---- lane roles: row n of each 16-row block, quarter q (codes
  // 32q..32q+31 of every group); for the A operand, MFMA row ma = lane % 16
  // reads the hi row of batch row ma (ma < 8) or the lo row of batch row
  // ma - 8, the zero row past the batch.
  const int n = lane & 15, q = lane >> 4;
  const int ma = lane & 15;
  const int arow = ma < 8 ? (ma < batch ? ma : 2 * batch) : (ma - 8 < batch ? batch + ma - 8 : 2 * batch);
  const uint32_t a_base = static_cast<uint32_t>(arow * xsr + q * 32) * 2u;  // bytes
  const int slice_groups = a.slice_cols / CQ_GROUP;
  MmaTable<SB> thi, tlo;
  thi.load(a.lev.hi);
  if constexpr (SPLIT) tlo.load(a.lev.lo);
  const float lscale = a.lev.lscale;

  for (int tile = first_tile; tile < a.ntiles; tile += a.per_slice) {
    const int64_t r0 = static_cast<int64_t>(tile) * kTileRows + wave * kRowsPerWave;
    const int64_t live_rows = a.rows - r0 < kRowsPerWave ? (a.rows - r0 > 0 ? a.rows - r0 : 0) : kRowsPerWave;
    const __amdgpu_buffer_rsrc_t wbuf =
        buffer_rsrc(a.packed + r0 * a.row_bytes, static_cast<uint32_t>(live_rows * a.row_bytes));
    const __amdgpu_buffer_rsrc_t nbuf =
        buffer_rsrc(a.norms + r0 * a.ngroups, static_cast<uint32_t>(live_rows * a.ngroups * 2));

    // Lane (n, q) loads group 4c+q of rows n and 16 + n whole (16-byte
    // loads: few requests per instruction) and its norm; the quarters then
    // trade pieces (quarter_transpose) and norms (quarter_gather).
    uint32_t codes[2][2][4 * SB];  // [set][block][dword]: group q, then piece q of each group
    uint16_t nrm[2][2];
    auto load_chunk = [&](int c, auto set_c) {
      constexpr int S = decltype(set_c)::value;
      const int64_t g = static_cast<int64_t>(slice) * slice_groups + 4 * c + q;  // this lane's group
      const bool g_live = g < a.ngroups && 4 * c + q < slice_groups;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int row = 16 * b + n;
        const uint32_t woff = static_cast<uint32_t>(row * a.row_bytes + g * GROUP_BYTES);
        load_dwords<4 * SB>(wbuf, g_live ? woff : kOutOfRange, codes[S][b]);
        const uint32_t noff = static_cast<uint32_t>((row * a.ngroups + g) * 2);
        nrm[S][b] = __builtin_amdgcn_raw_buffer_load_b16(nbuf, g_live ? noff : kOutOfRange, 0, 0);
      }
    };

    floatx4 acc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    auto compute_chunk = [&](int c, auto set_c) {
      constexpr int S = decltype(set_c)::value;
      // (a chunk past the slice -- the odd one of the last pair -- rereads
      // the last chunk's activations; its norms are zero)
      const int cc = c < nchunks ? c : nchunks - 1;
      const uint8_t *a_chunk = reinterpret_cast<const uint8_t *>(xs) + a_base + cc * kChunkCols * 2;
#pragma unroll
      for (int b = 0; b < 2; ++b) quarter_transpose<SB>(codes[S][b]);
      uint32_t nq[4];  // norms of the chunk's groups: block 0 low half, block 1 high half
      quarter_gather(static_cast<uint32_t>(nrm[S][0]) | static_cast<uint32_t>(nrm[S][1]) << 16, nq);
      floatx4 gs[2][4];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) gs[b][j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f16x8 af = *reinterpret_cast<const f16x8 *>(a_chunk + j * CQ_GROUP * 2 + t * 16);
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            uint32_t o[4], ol[4];
            if constexpr (SPLIT)
              decode_piece2<SB>(thi, tlo, codes[S][b] + j * SB, t, o, ol);
            else if constexpr (SB == 1)
              decode1_sign(codes[S][b][j], t, o);
            else
              decode_piece<SB>(thi, codes[S][b] + j * SB, t, o);
            gs[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                af, __builtin_bit_cast(f16x8, make_uint4(o[0], o[1], o[2], o[3])), gs[b][j], 0, 0, 0);
            if constexpr (SPLIT)
              gs[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  af, __builtin_bit_cast(f16x8, make_uint4(ol[0], ol[1], ol[2], ol[3])), gs[b][j], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint16_t nb = static_cast<uint16_t>(nq[j] >> (16 * b));
          const float nf = static_cast<float>(__builtin_bit_cast(_Float16, nb)) * lscale;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[b][e] = __builtin_fmaf(nf, gs[b][j][e], acc[b][e]);
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

    // D layout: lane l, register e -> MFMA row 4 (l / 16) + e, weight row
    // l % 16.  Rows 8..15 (lanes 32..63) are the lo parts' products: lane l
    // < 32 adds lane l + 32's sum to its own (the lane-half swap).
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t row = r0 + 16 * b + n;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto sw =
            __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[b][e]), __float_as_uint(acc[b][e]), false, false);
        const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const int m = 4 * q + e;
        if (q < 2 && m < batch && row < a.rows) {
          const int64_t at = (static_cast<int64_t>(slice) * batch + m) * a.rows + row;
          a.out[at] = tot * unscale[m];
        }
      }
    }
  }
}

typedef void (*MmKernel)(MmArgs);

MmKernel pick_kernel(int sb, bool split) {
  if (sb == 1) return matvec_mma_kernel<1, false>;  // binary levels are always exact
  if (split) return sb == 2 ? matvec_mma_kernel<2, true> : (sb == 3 ? matvec_mma_kernel<3, true> : matvec_mma_kernel<4, true>);
  return sb == 2 ? matvec_mma_kernel<2, false> : (sb == 3 ? matvec_mma_kernel<3, false> : matvec_mma_kernel<4, false>);
}

// Lets every variant take the largest dynamic LDS a launch asks for (once
// per process; the attribute is per kernel).
void allow_large_lds() {
  static std::once_flag once;
  std::call_once(once, [] {
    const size_t most = mm_lds_bytes(kMaxSliceCols, kMaxBatch);
    for (int sb = 1; sb <= 4; ++sb)
      for (int sp = 0; sp < 2; ++sp)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(pick_kernel(sb, sp != 0)),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(most));
  });
}

// Resident workgroups of one launch on the current device: the LDS (rounded
// up to 4 KB), not the registers, limits the larger batches.  Cached per
// device, width class and LDS size.
int resident_groups(int sb, bool split, size_t lds) {
  constexpr int kBuckets = 41;  // up to 160 KB
  static std::atomic<int> cache[64][2][2][kBuckets];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int bucket = static_cast<int>((lds + 4095) / 4096);
  if (bucket >= kBuckets) bucket = kBuckets - 1;
  std::atomic<int> &slot = cache[dev][sb == 1 ? 0 : 1][split ? 1 : 0][bucket];
  int c = slot.load(std::memory_order_relaxed);
  if (c == 0) {
    int per_cu = 1, cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(pick_kernel(sb, split)),
                                                     kThreads, static_cast<size_t>(bucket) * 4096) != hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    c = per_cu * cus;
    slot.store(c, std::memory_order_relaxed);
  }
  return c;
}

struct MmShape {
  int slice_cols, nslice, ntiles, per_slice;
};

MmShape mm_shape(int64_t rows, int64_t kpad, int target) {
  MmShape s;
  const int64_t chunks = (kpad + kChunkCols - 1) / kChunkCols;
  const int64_t chunks_per_slice = kMaxSliceCols / kChunkCols;
  s.nslice = static_cast<int>((chunks + chunks_per_slice - 1) / chunks_per_slice);
  // spread the columns evenly over the slices, in whole chunks
  s.slice_cols = static_cast<int>((chunks + s.nslice - 1) / s.nslice) * kChunkCols;
  s.ntiles = static_cast<int>((rows + kTileRows - 1) / kTileRows);
  int per = target / s.nslice;
  if (per < 1) per = 1;
  if (per > s.ntiles) per = s.ntiles;
  s.per_slice = per;
  return s;
}

}  // namespace

namespace cq {

MmaLevels mma_levels(int bits, const CodeLevels &lev) {
  MmaLevels m;
  std::memset(&m, 0, sizeof m);
  const int sb = storage_bits(bits);
  const int nlev = 1 << sb;
  uint16_t hi[16] = {0}, lo[16] = {0};
  auto f16_bits = [](float f) {
    const _Float16 h = static_cast<_Float16>(f);  // round to nearest even
    uint16_t b;
    std::memcpy(&b, &h, 2);
    return b;
  };
  if (bits == 1 || bits == 5) {
    // integer multiples of one level: binary codes -1, +1 times c; ternary
    // crumbs 0, 1, -2, -1 times a (both exact in fp16)
    static const float kBinary[2] = {-1.0f, 1.0f}, kTernary[4] = {0.0f, 1.0f, -2.0f, -1.0f};
    m.lscale = lev.v[1];
    for (int i = 0; i < nlev; ++i) hi[i] = f16_bits(bits == 1 ? kBinary[i] : kTernary[i]);
  } else {
    float mx = 0.0f;
    for (int i = 0; i < nlev; ++i) mx = std::fmax(mx, std::fabs(lev.v[i]));
    int e = 0, sl = 0;
    if (mx > 0.0f) {
      (void)std::frexp(mx, &e);  // mx < 2^e
      sl = std::max(-100, std::min(100, 15 - e));  // largest level times 2^sl in [2^14, 2^15)
    }
    m.lscale = std::ldexp(1.0f, -sl);
    for (int i = 0; i < nlev; ++i) {
      const float s = std::ldexp(lev.v[i], sl);  // exact: a power of two
      const _Float16 h = static_cast<_Float16>(s);
      hi[i] = f16_bits(s);
      lo[i] = f16_bits(s - static_cast<float>(h));  // exact in fp32
      if ((lo[i] & 0x7fffu) != 0) m.split = 1;
    }
  }
  if (sb == 1) {
    // BinTable: the two values' high bytes and their common low byte
    m.hi[0] = static_cast<uint32_t>(hi[0] >> 8) | static_cast<uint32_t>(hi[1] >> 8) << 8 |
              static_cast<uint32_t>(hi[0] & 0xffu) << 16;
  } else {
    for (int k = 0; k < nlev / 4; ++k)
      for (int i = 0; i < 4; ++i) {
        m.hi[k] |= static_cast<uint32_t>(hi[4 * k + i] & 0xffu) << (8 * i);
        m.hi[nlev / 4 + k] |= static_cast<uint32_t>(hi[4 * k + i] >> 8) << (8 * i);
        m.lo[k] |= static_cast<uint32_t>(lo[4 * k + i] & 0xffu) << (8 * i);
        m.lo[nlev / 4 + k] |= static_cast<uint32_t>(lo[4 * k + i] >> 8) << (8 * i);
      }
  }
  return m;
}

uint64_t matvec_mma_workspace_bytes(int64_t rows, int64_t kpad, int64_t batch) {
  if (rows <= 0 || kpad <= 0 || batch <= 0) return 0;
  const MmShape s = mm_shape(rows, kpad, 1);
  if (s.nslice <= 1) return 0;
  return static_cast<uint64_t>(s.nslice) * batch * rows * 4;
}

hipError_t launch_matvec_mma(const uint8_t *blob, int bits, int64_t rows, int64_t kpad, const CodeLevels &lev,
                             const float *xr, int64_t batch, float *y, void *workspace, hipStream_t s) {
  if (batch < 1 || batch > kMaxBatch || kpad % CQ_GROUP != 0) return hipErrorInvalidValue;
  allow_large_lds();
  const int sb = storage_bits(bits);
  MmArgs a;
  a.lev = mma_levels(bits, lev);
  const bool split = sb != 1 && a.lev.split != 0;
  const MmShape probe = mm_shape(rows, kpad, 1);
  const size_t lds = mm_lds_bytes(probe.slice_cols, batch);
  const MmShape sh = mm_shape(rows, kpad, resident_groups(sb, split, lds));
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
  a.out = sh.nslice > 1 ? static_cast<float *>(workspace) : y;
  // 32-bit tile-relative offsets: 32 rows of packed bytes or norms.
  if (static_cast<int64_t>(kRowsPerWave) * a.row_bytes >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(sh.nslice) * sh.per_slice));
  pick_kernel(sb, split)<<<grid, kThreads, lds, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sh.nslice <= 1) return e;
  return launch_combine(a.out, batch * rows, sh.nslice, y, s);
}

}  // namespace cq
