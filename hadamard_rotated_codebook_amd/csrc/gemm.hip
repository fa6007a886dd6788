// Prefill product C = Xr . V^T on the bf16 matrix cores, where Xr is the
// rotated activation (bf16, from cq_rotate_acts) and V is the CQ matrix
// dequantised in the rotated domain, V[r][g*128+j] = bf16(c[q] * norm[r][g]).
// By the rotated-activation identity (OpenNeedle reference notes) this is the
// product with the dense dequantised matrix, without ever applying H to the
// weights or writing them to memory (".cact" format post, "How the kernel
// reads it": no weight is materialised outside the tile being multiplied).
//
// Design (MFMA-bound at M = 4096, N = K = 16384 on MI355X):
//  * A 512-thread workgroup (8 waves, 2 along M x 4 along N) computes a
//    256 x 256 tile of C, 128 x 64 per wave: 8 x 4 blocks of
//    v_mfma_f32_16x16x32_bf16 with fp32 accumulators (128 VGPRs per lane), two
//    waves per SIMD so that one's barrier waits and decode hide behind the
//    other's matrix work.
//  * K advances 64 columns per stage through double-buffered LDS (2 x 64 KB).
//    At the start of stage s every thread issues the Xr tile of stage s+1 as
//    buffer loads straight into LDS (16 bytes per lane, no registers, into the
//    buffer stage s-1 used) and the loads of stage s+2's W codes (and, at
//    group starts, the norm) into one of two register sets; while the matrix
//    cores work on stage s it decodes stage s+1's W into the other LDS
//    buffer, the decode interleaved among the MFMAs (sched_group_barrier) so
//    that VALU and matrix cores overlap; the stage ends waiting for its direct
//    loads, then one barrier.  All loads are unconditional buffer loads; rows
//    past the end of Xr or W fall outside the tile's buffer range and read as
//    zeros, so no select ties a load to its issue point.
//  * Decode: a pair of threads owns a row of the W tile.  Per (row, group) it
//    builds the table bf16(level[c] * norm) for every code c
//    (v_cvt_pk_bf16_f32, round to nearest even) as byte planes, and turns
//    packed codes into bf16 pairs with v_perm_b32 lookups: 1.9 VALU per weight
//    at 2 bits, 2.5 at 3 bits, 3.6 at 4 bits (two 8-entry halves selected by
//    the code's top bit).
//  * LDS rows are 64 bf16 (128 B); 16-byte chunks are XOR-swizzled by row so
//    that the fragment reads of 16 consecutive rows fall in distinct banks.
//  * Tiles are ordered in groups of 4 M-tiles, and the ids are renumbered so
//    that each XCD runs consecutive groups: the 32 workgroups of an XCD share
//    4 Xr tiles and 8 W tiles through its L2.
#include <type_traits>

#include "cq_decode.h"
#include "cq_internal.h"

namespace {

using namespace cqdev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int BK = 64;
constexpr int kWavesM = 2;  // waves along M; the waves along N are a template parameter
constexpr int kGroupM = 4;  // M-tiles per tile group
constexpr int kValuPerMfma = 2;  // VALU slots after each MFMA in the interleave
#ifndef CQ_GEMM_WN
#define CQ_GEMM_WN 4
#endif

struct GemmArgs {
  const uint8_t *packed;
  const uint16_t *norms;  // fp16 bits [rows][ngroups]
  const uint16_t *xr;     // bf16 bits [m][kpad]
  float *c;               // [m][rows]
  int64_t m, rows, kpad, row_bytes, ngroups;
  int32_t tiles_m, tiles_n;
  cq::CodeLevels lev;
};

__device__ inline int swz(int row, int chunk) { return chunk ^ (row & 7); }

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}
typedef __attribute__((address_space(3))) void *lds_ptr_t;

// T: the workgroup's tile is T x T (256, or 128 for products too small to
// give every CU a 256 x 256 tile); WN waves along N.
template <int SB, int WN, int T>
__global__ __launch_bounds__(64 * kWavesM * WN, 1) void gemm_kernel(GemmArgs a) {
  constexpr int BM = T, BN = T;
  constexpr int kThreads = 64 * kWavesM * WN;
  constexpr int WTM = BM / kWavesM;            // wave tile: WTM x TN
  constexpr int TN = BN / WN;
  constexpr int FI = WTM / 16, FJ = TN / 16;   // 16 x 16 blocks per wave
  constexpr int XPT = BM * 8 / kThreads;       // Xr chunks per thread per stage
  constexpr int TPR = kThreads / BN;           // threads per W row
  constexpr int CODES = BK / TPR;              // codes a thread decodes per stage
  constexpr int CODE_DW = CODES * SB / 32;     // their packed dwords
  // the two stage buffers of the Xr tile as separate arrays: a direct load
  // into one then provably does not alias reads of the other
  __shared__ uint4 As0[BM * 8], As1[BM * 8];   // [row][chunk], 16-byte chunks
  auto as_buf = [&](auto b_c) -> uint4 * {
    if constexpr (decltype(b_c)::value == 0) return As0; else return As1;
  };
  __shared__ uint4 Bs[2][BN * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // Tile order: groups of kGroupM M-tiles walk all N-tiles; ids renumbered so
  // that consecutive tiles run on one XCD (ids are dispatched round-robin).
  const int total = a.tiles_m * a.tiles_n;
  int t = blockIdx.x;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
  const int per_group = kGroupM * a.tiles_n;
  const int first_m = (t / per_group) * kGroupM;
  const int gsize = min(kGroupM, a.tiles_m - first_m);
  const int tm = first_m + (t % per_group) % gsize;
  const int tn = (t % per_group) / gsize;
  const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;

  // Global sources of this thread: part `half` of row `wr` of the W tile (the
  // Xr tile goes straight to LDS, below).  Offsets are relative to the tile's
  // first row and fit 32 bits (the host bounds kpad).
  const int wr = tid / TPR, half = tid % TPR;
  const int64_t mrows = a.m - m0 < BM ? a.m - m0 : BM, nrows = a.rows - n0 < BN ? a.rows - n0 : BN;
  const __amdgpu_buffer_rsrc_t xbuf = buffer_rsrc(a.xr + m0 * a.kpad, static_cast<uint32_t>(mrows * a.kpad * 2));
  const __amdgpu_buffer_rsrc_t wbuf =
      buffer_rsrc(a.packed + n0 * a.row_bytes, static_cast<uint32_t>(nrows * a.row_bytes));
  const __amdgpu_buffer_rsrc_t nbuf =
      buffer_rsrc(a.norms + n0 * a.ngroups, static_cast<uint32_t>(nrows * a.ngroups * 2));
  const uint32_t woff = static_cast<uint32_t>(wr * a.row_bytes + half * (CODES * SB / 8));
  const uint32_t noff = static_cast<uint32_t>(wr * a.ngroups * 2);

  // The W codes of stage s+2 (from HBM) are loaded while stage s is
  // multiplied, into one of two register sets.  Even stages start a group
  // (BK is half a group), so only set 0 carries a norm and only its stores
  // build a table.  Rows past the end load zeros: an Xr row directly, a W
  // row through a zero norm (an all-zero decode table).
  uint32_t wc[2][CODE_DW];
  uint16_t wn16 = 0;
  auto load = [&](int64_t k0, auto set_c) {
    constexpr int S = decltype(set_c)::value;
    load_dwords<CODE_DW>(wbuf, woff + static_cast<uint32_t>(k0 * SB / 8), wc[S]);
    if constexpr (S == 0)
      wn16 = __builtin_amdgcn_raw_buffer_load_b16(nbuf, noff + static_cast<uint32_t>(k0 / CQ_GROUP * 2), 0, 0);
  };
  // Xr tile of a stage straight into LDS: instruction p of wave w fills rows
  // 8 (w XPT + p) .. +7 (1 KB), lane -> row + lane / 8, physical chunk
  // lane % 8, i.e. logical chunk (lane % 8) ^ (row & 7).
  const int dwave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t dma_off = static_cast<uint32_t>((lane >> 3) * a.kpad * 2 + (((lane & 7) ^ ((lane >> 3) & 7)) * 16));
  auto dma = [&](int64_t k0, auto buf_c) {
#pragma unroll
    for (int p = 0; p < XPT; ++p) {
      const int row0 = 8 * (dwave * XPT + p);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xbuf, (lds_ptr_t)(as_buf(buf_c) + row0 * 8), 16, dma_off,
          static_cast<uint32_t>(row0 * a.kpad * 2 + k0 * 2), 0, 0);
    }
  };

  // Writing the W stage held in register set S into LDS buffer buf, in two
  // parts: part 0 builds the group's table (set 0: even stages start a group)
  // and decodes the first half of this thread's codes; part 1 decodes the
  // second half.  Each half is two 16-byte chunks of W.
  typename std::conditional<SB == 1, BinTable<__bf16>, Table<SB, __bf16>>::type tab;
  auto store_part = [&](int buf, auto set_c, auto part_c) {
    constexpr int S = decltype(set_c)::value, PART = decltype(part_c)::value;
    const uint32_t *wcs = wc[S];
    if constexpr (PART == 0) {
      if constexpr (S == 0) tab.build(a.lev, static_cast<float>(__builtin_bit_cast(_Float16, wn16)));
    }
    static_assert(CODES / 8 == 4, "four 8-code chunks per thread and stage");
    uint32_t o[8];
    if constexpr (SB == 1) {  // 16 codes: bytes 2 PART and 2 PART + 1 of the stage's dword
      decode1(tab, (wcs[0] >> (16 * PART)) & 0xffu, o);
      decode1(tab, (wcs[0] >> (16 * PART + 8)) & 0xffu, o + 4);
    } else if constexpr (SB == 4) {
      decode4(tab, wcs[2 * PART], o);
      decode4(tab, wcs[2 * PART + 1], o + 4);
    } else if constexpr (SB == 3) {
#pragma unroll
      for (int q = 2 * PART; q < 2 * PART + 2; ++q) {  // 24 bits per 8 codes: byte offset 3 q
        const int bit = 24 * q, w = bit >> 5, sh = bit & 31;
        const uint32_t b = sh <= 8 ? (wcs[w] >> sh) : __builtin_amdgcn_alignbit(wcs[(w + 1) % CODE_DW], wcs[w], sh);
        decode3(tab, b, o + 4 * (q - 2 * PART));
      }
    } else {
      decode2(tab, wcs[PART], o);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int ch = half * (CODES / 8) + 2 * PART + c;
      Bs[buf][wr * 8 + swz(wr, ch)] = make_uint4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
    }
  };

  floatx4 acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // One 32-wide k step on LDS buffer cur: the fragment reads, then part PART
  // of writing the next stage (register set S) into the other buffer, then
  // the 32 MFMAs, with the decode and its LDS writes interleaved among them
  // so that the matrix cores and the VALU work at the same time.
  auto kstep = [&](auto cur_c, auto kk_c, auto set_c) {
    constexpr int cur = decltype(cur_c)::value, kk = decltype(kk_c)::value;
    const int ch = kk * 4 + (lane >> 4);
    bf16x8 af[FI], bfr[FJ];
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int row = wn * TN + j * 16 + (lane & 15);
      bfr[j] = __builtin_bit_cast(bf16x8, Bs[cur][row * 8 + swz(row, ch)]);
    }
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int row = wm * WTM + i * 16 + (lane & 15);
      af[i] = __builtin_bit_cast(bf16x8, as_buf(cur_c)[row * 8 + swz(row, ch)]);
    }
    store_part(cur ^ 1, set_c, kk_c);
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    // Order: the B fragments and the first A fragment, then per A fragment
    // the read of the next one and its FJ MFMAs, each MFMA followed by a few
    // VALU instructions and every fourth by an LDS write.  A fragments are
    // read one ahead of use, which keeps few of them live.
    __builtin_amdgcn_sched_group_barrier(0x100, FJ + 1, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      if (i + 1 < FI) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);  // VALU
        if ((i * FJ + j) % 4 == 3) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
      }
    }
    // Fence: without it the scheduler loads the next step's fragments while
    // this step's are live, and the 3- and 4-bit kernels spill past 256 VGPRs.
    __builtin_amdgcn_sched_barrier(0);
  };

  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  using Part0 = std::integral_constant<int, 0>;
  using Part1 = std::integral_constant<int, 1>;
  // kpad is a multiple of the group size, so the stage count is even.
  const int nstages = static_cast<int>(a.kpad / BK);
  dma(0, std::integral_constant<int, 0>{});
  load(0, Set0{});
  load(BK, Set1{});
  store_part(0, Set0{}, Part0{});
  store_part(0, Set0{}, Part1{});
  wait_vmcnt<0>();
  __syncthreads();
  // Stage s: loads of stage s+2 into register set s%2, then the matrix cores
  // on LDS buffer s%2 while stage s+1 (register set (s+1)%2) is written into
  // buffer (s+1)%2.  The loads are unconditional (past the end they reload
  // the last stage, unused), and so are the writes (after the last stage
  // they fill the idle buffer): a load or a use on only some paths would make
  // the compiler wait for the newer loads too, or sink the loads to the use.
  auto stage = [&](int s, auto par_c) {
    constexpr int P = decltype(par_c)::value;  // s % 2
    // Xr of stage s+1 into the buffer stage s-1 used (every wave is past it)
    dma(static_cast<int64_t>(s + 1 < nstages ? s + 1 : nstages - 1) * BK, std::integral_constant<int, 1 - P>{});
    load(static_cast<int64_t>(s + 2 < nstages ? s + 2 : nstages - 1) * BK, par_c);
    __builtin_amdgcn_sched_barrier(0);
    using Cur = std::integral_constant<int, P>;
    using Next = std::integral_constant<int, 1 - P>;
    kstep(Cur{}, Part0{}, Next{});
    kstep(Cur{}, Part1{}, Next{});
    // the direct loads of stage s+1 have landed (only this stage's W loads,
    // issued after them, may still be in flight)
    wait_vmcnt<P == 0 ? 2 : 1>();
    __syncthreads();
  };
  for (int s = 0; s < nstages; s += 2) {
    stage(s, Set0{});
    stage(s + 1, Set1{});
  }
  wait_vmcnt<0>();

  // C fragment layout: lane l, register e -> row 4*(l/16) + e, column l%16.
#pragma unroll
  for (int i = 0; i < FI; ++i) {
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int64_t col = n0 + wn * TN + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + wm * WTM + i * 16 + 4 * (lane >> 4) + e;
        if (row < a.m && col < a.rows) a.c[row * a.rows + col] = acc[i][j][e];
      }
    }
  }
}

}  // namespace

namespace cq {

hipError_t launch_gemm(const uint8_t *blob, int bits, int64_t rows, int64_t kpad, const CodeLevels &lev,
                       const void *xr, int64_t m, float *c, hipStream_t s) {
  // The stage loop needs whole groups; tile-relative buffer offsets need
  // 257 rows of Xr (2 kpad bytes each) to fit 32 bits.
  if (kpad <= 0 || kpad % CQ_GROUP != 0 || kpad > (int64_t{1} << 22)) return hipErrorInvalidValue;
  const int sb = storage_bits(bits);
  GemmArgs a;
  a.packed = blob;
  a.row_bytes = kpad * sb / 8;
  a.norms = reinterpret_cast<const uint16_t *>(blob + rows * a.row_bytes);
  a.xr = static_cast<const uint16_t *>(xr);
  a.c = c;
  a.m = m;
  a.rows = rows;
  a.kpad = kpad;
  a.ngroups = kpad / CQ_GROUP;
  a.lev = lev;
  // 256 x 256 tiles when they give at least one per CU; otherwise 128 x 128
  // tiles (4 waves, 64 x 64 each), four times as many workgroups.
  const int64_t tm256 = (m + 255) / 256, tn256 = (rows + 255) / 256;
  const bool big = tm256 * tn256 >= 256;
  const int64_t tile = big ? 256 : 128;
  const int64_t tm = (m + tile - 1) / tile, tn = (rows + tile - 1) / tile;
  if (tm * tn > 0x7fffffff) return hipErrorInvalidConfiguration;
  a.tiles_m = static_cast<int32_t>(tm);
  a.tiles_n = static_cast<int32_t>(tn);
  const dim3 grid(static_cast<unsigned>(tm * tn));
  if (big) {
    constexpr int threads = 64 * kWavesM * CQ_GEMM_WN;
    switch (sb) {
      case 1: gemm_kernel<1, CQ_GEMM_WN, 256><<<grid, threads, 0, s>>>(a); break;
      case 2: gemm_kernel<2, CQ_GEMM_WN, 256><<<grid, threads, 0, s>>>(a); break;
      case 3: gemm_kernel<3, CQ_GEMM_WN, 256><<<grid, threads, 0, s>>>(a); break;
      default: gemm_kernel<4, CQ_GEMM_WN, 256><<<grid, threads, 0, s>>>(a); break;
    }
  } else {
    constexpr int threads = 64 * kWavesM * 2;
    switch (sb) {
      case 1: gemm_kernel<1, 2, 128><<<grid, threads, 0, s>>>(a); break;
      case 2: gemm_kernel<2, 2, 128><<<grid, threads, 0, s>>>(a); break;
      case 3: gemm_kernel<3, 2, 128><<<grid, threads, 0, s>>>(a); break;
      default: gemm_kernel<4, 2, 128><<<grid, threads, 0, s>>>(a); break;
    }
  }
  return hipGetLastError();
}

}  // namespace cq
