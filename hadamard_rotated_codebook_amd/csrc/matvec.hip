// Decode matrix-vector product y = W . x for a CQ matrix (equation (1) of
// include/cq.h), computed as sum_g norm_g * <c[q_g], H x_g> on the rotated
// activation xr (OpenNeedle reference notes, rotated-activation identity; the
// ".cact" format post, "How the kernel reads it": the stored indices are looked
// up, never expanded, and no weight is materialised).
//
// Design (HBM-bound at batch 1 on MI355X):
//  * Lookup tables are indexed by a whole packed field: one byte for 2-bit rows
//    (CQ2 and ternary crumbs, 4 weights per lookup) and for 4-bit rows (2
//    weights), one 6-bit field (2 codes) for 3-bit rows.  An entry is the sum
//    over the field's codes of level * xr, computed in fp32 and stored as fp16
//    after scaling by a power of two chosen per K-slice (the largest possible
//    entry lands in [2^14, 2^15)).  Each entry is rounded once; the product with
//    the fp16 group norm and every sum are fp32 (v_fma_mix), and the scale is
//    undone exactly after the row reduction.  Compared with 16-entry tables per
//    pair of columns this halves the LDS reads per weight, which together with
//    the VALU work bounded the kernel below HBM speed.
//  * A 1024-thread workgroup (one per CU: the tables take 128 KB of LDS) owns
//    one K-slice -- the columns whose tables fill 128 KB: 1024 columns at CQ2,
//    512 at CQ4, 2048 at CQ3 -- builds its tables once, and streams that slice
//    of every row of its row blocks.  Each lane owns a fixed run of columns and
//    a private 4-byte slot in every table row (two fp16 positions per slot), so
//    the 64 lookups of a wave never collide in an LDS bank.
//  * Table address: one v_perm_b32 for byte fields (the data byte lands next to
//    the lane slot and the region bit), v_bfe + v_lshl_or for 6-bit fields; the
//    half of the slot rides in the LDS instruction's immediate offset.  At CQ2 a
//    lane spends 4 v_perm, 4 LDS reads and 4 v_fma_mix on 16 weights of a row.
//  * The group norms of a wave's unit of 32 rows (16 bytes per row at 2 bits,
//    4 KB apart) come in a few 2-byte loads per lane when the loads move on
//    to the unit, and are staged in a per-wave LDS buffer: one load per row
//    cost 11 % of the kernel's time, the unit loads cut that by a third.  The
//    buffer holds each group's 32 norms side by side, so one 16-byte LDS read
//    serves 8 rows (v_fma_mix selects the half).
//  * Matrices of cq::kStreamMinBytes and more load their code rows with the nt
//    (streaming) cache hint: each byte is read once per call, and such a
//    matrix does not stay in the 256 MB Infinity Cache between calls.  11 %
//    faster at CQ2 and 14 % at CQ4 on the 65536 x 16384 matrices than plain
//    loads; smaller matrices keep plain loads, which let a matrix that fits
//    the cache be read from it on the next call (nt measured up to 10 %
//    slower there).  The norms, which the K-slices of a row share through
//    L2, always take plain loads (nt on them measured slower).
//  * Rows are read through buffer descriptors rebased per row in scalar
//    registers.  A row past the end of its block or of the matrix gets a
//    zero-length descriptor and reads zeros, as do lanes past the end of K (their
//    offsets are out of range): no clamping and no branches, so the loads can run
//    AHEAD rows ahead of the arithmetic without the compiler draining them.
//  * The per-lane partial sums of a wave's 32 row slots are reduced across the 64
//    lanes with the lane-swap instructions (32- and 16-lane halves) and three DPP
//    halving steps: VALU only, no LDS traffic.
//  * Workgroup id -> (slice, row blocks) is XCD-aware.  Consecutive workgroup ids
//    are dispatched to different XCDs; the mapping gives each XCD every slice of
//    its row blocks, so all of a row's bytes and its norms (a 128-byte line of
//    norms spans several slices) go through one L2.
//  * With more than one slice, the workgroups write per-slice partial sums of
//    each row to the caller's workspace with plain stores, and a second small
//    kernel adds the slices of each row in slice order: the result does not
//    depend on scheduling.  (An in-kernel combine -- agent-scope partial stores
//    and per-block completion counters, the last arrival adding up -- cost
//    more than this kernel boundary: the counter protocol stalls the waves and
//    the coherent stores go to memory one 4-byte write at a time.)
#include <atomic>

#include "cq_fwht.h"
#include "cq_internal.h"

namespace {

#ifndef CQ_MV_AHEAD
#define CQ_MV_AHEAD 16
#endif
constexpr int kThreads = 1024;                        // one workgroup per CU
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerWave = 32;                      // row slots per wave (fully unrolled)
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;  // rows of a full row block (512)
constexpr uint32_t kRawBufferWord3 = 0x00020000u;     // buffer descriptor: raw, 32-bit data format
constexpr uint32_t kOutOfRange = 0x7ffff000u;         // a buffer offset past any descriptor's length

// Geometry of a storage width SB (1: binary, 2: CQ2 and ternary crumbs,
// 3: CQ3, 4: CQ4).
template <int SB>
struct Geom {
  static constexpr int LANE_BYTES = SB == 3 ? 12 : 4;            // packed bytes per lane and row
  static constexpr int LANE_COLS = LANE_BYTES * 8 / SB;          // 32, 16, 32, 8 columns per lane
  static constexpr int IDX_BITS = SB == 3 ? 6 : 8;               // bits of a table index
  static constexpr int ENTRIES = 1 << IDX_BITS;                  // entries per table
  static constexpr int CODES = IDX_BITS / SB;                    // codes per table index
  static constexpr int POSITIONS = LANE_COLS / CODES;            // tables per lane: 4, 16, 4
  static constexpr int REGION = ENTRIES * 256;                   // bytes per pair of positions
  static constexpr int LDS_BYTES = POSITIONS / 2 * REGION;       // 128 KB
  static constexpr int SLICE_COLS = 64 * LANE_COLS;              // 1024, 2048, 512
  static constexpr int SLICE_BYTES = 64 * LANE_BYTES;            // 256, 768, 256
  static constexpr int SLICE_GROUPS = SLICE_COLS / CQ_GROUP;     // 8, 16, 4
  static constexpr int LANES_PER_GROUP = CQ_GROUP / LANE_COLS;   // 8, 4, 16
  // rows of loads in flight per wave (measured per width: 32 helps binary by ~4 %, not CQ2/CQ4)
  static constexpr int AHEAD = SB == 3 ? 8 : (SB == 1 ? kRowsPerWave : CQ_MV_AHEAD);
  static constexpr int DWORDS = LANE_BYTES / 4;
  static constexpr int LOOKUPS = LANE_BYTES * 8 / IDX_BITS;     // table reads per lane and row
  static constexpr int NORM_BYTES = SLICE_GROUPS * 2;            // a row chunk's norms: 16, 32, 8 (32 at 1 bit)
  static constexpr int NORM_H = kRowsPerWave * SLICE_GROUPS / 64;  // a lane's norms of a unit: 4, 8, 2 (8)
  static_assert(LDS_BYTES == 128 * 1024, "tables fill 128 KB");
  static_assert(kRowsPerWave % AHEAD == 0 && AHEAD <= kRowsPerWave, "prefetch ring: divides the row slots");
};

struct MvArgs {
  const uint8_t *packed;
  const uint16_t *norms;  // fp16 bits, [rows][ngroups]
  const float *xr;        // [kpad], rotated (unused when the kernel rotates)
  const float *x;         // [cols], not rotated (used when the kernel rotates)
  int64_t cols;
  int32_t xvec;           // x rows may be read 8 floats at a time
  float *y;               // [rows]
  float *partial;         // [nslice][rows] (nslice > 1)
  int64_t rows, kpad, row_bytes, ngroups;
  int32_t rows_per_block;  // multiple of kWaves, <= kRowsPerBlock
  int32_t nblocks;         // row blocks
  int32_t nslice;          // K slices
  int32_t per_slice;       // workgroups per slice (grid = nslice * per_slice)
  float lev_absmax;        // largest |level| of the code book
  cq::CodeLevels lev;
};

__device__ inline _Float16 lds_half(const uint8_t *lds, uint32_t byte_addr) {
  return *reinterpret_cast<const _Float16 *>(lds + byte_addr);
}

// Two floats rounded to nearest-even fp16, a in the low half.
__device__ inline uint32_t pack_half2(float a, float b) {
  // one v_cvt_pk_f16_f32 (round to nearest even, as two scalar conversions)
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

__device__ inline __amdgpu_buffer_rsrc_t buffer(uint64_t addr, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(addr), 0, static_cast<int>(nbytes),
                                           static_cast<int>(kRawBufferWord3));
}

template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Bitwise select (one v_bfi_b32): a where mask is 0, b where it is all ones.
__device__ inline float pick(float a, float b, uint32_t mask) {
  return __uint_as_float((__float_as_uint(a) & ~mask) | (__float_as_uint(b) & mask));
}

// One halving step: values i and H+i of each lane pair up with a partner lane
// (DPP pattern CTRL, partner in the other half selected by `upper`); the lower
// lanes keep value i, the upper lanes value H+i, each adding the partner's
// copy of it.
template <int H, int CTRL>
__device__ inline void halve(float *v, uint32_t upper) {
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float keep = pick(v[i], v[H + i], upper);
    const float send = pick(v[H + i], v[i], upper);
    v[i] = keep + dpp<CTRL>(send);
  }
}

// Sum each of the 32 row-slot partials over the 64 lanes of the wave.  After
// it, lanes 2m and 2m+1 hold the total of row slot m.
__device__ inline float reduce_rows(float (&v)[kRowsPerWave], int lane) {
  static_assert(kRowsPerWave == 32, "the swap/DPP schedule is written for 32 row slots");
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // lanes 0-31 <-> 32-63: rows i (low half) and 16+i (high half)
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[16 + i]), false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {  // 16-lane rows within each half
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[8 + i]), false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  halve<4, 0x128>(v, (lane & 8) ? ~0u : 0u);  // row_ror:8        pairs lane k with k^8 in a row
  halve<2, 0x141>(v, (lane & 4) ? ~0u : 0u);  // row_half_mirror  pairs k with 7-k in 8 lanes
  halve<1, 0x4e>(v, (lane & 2) ? ~0u : 0u);   // quad_perm 2301   pairs k with k^2
  return v[0] + dpp<0xb1>(v[0]);              // quad_perm 1032   pairs k with k^1
}

// Store a unit's per-row totals: straight to y with one slice, else to this
// slice's partial sums [slice][row] in the workspace.
__device__ inline void store_block(const MvArgs &a, int slice, int64_t r0, int64_t r1, int slot, int lane, float t) {
  const int64_t r = r0 + slot + static_cast<int64_t>(kWaves) * (lane >> 1);
  if ((lane & 1) || r >= r1) return;
  if (a.nslice == 1)
    a.y[r] = t;
  else
    a.partial[static_cast<int64_t>(slice) * a.rows + r] = t;
}

// Power-of-two scale that puts the largest possible table entry of this slice
// in [2^14, 2^15): the exponent k of 2^k (0 when the slice's activations are
// all zero or not finite; clamped so both 2^k and 2^-k are normal floats).
__device__ inline int table_exponent(float bound) {
  if (!(bound > 0.0f) || !(bound <= 3.0e38f)) return 0;
  int e;
  (void)frexpf(bound, &e);  // bound < 2^e
  return max(-100, min(100, 15 - e));
}

// ROT: the kernel rotates its slice of x itself (the fused call) instead of
// reading the rotated activation xr.
template <int SB, bool ROT, int POL>
__global__ __launch_bounds__(kThreads) void matvec_kernel(MvArgs a) {
  using G = Geom<SB>;
  __shared__ __align__(16) uint8_t lds[G::LDS_BYTES];
  __shared__ __align__(16) float xrot[ROT ? G::SLICE_COLS : 4];  // the slice's rotated activations
  constexpr int NBS = kRowsPerWave + 8;  // halves per group row of the norm buffer (padded)
  __shared__ __align__(16) uint16_t nbuf[kWaves][G::SLICE_GROUPS * NBS];  // each wave's unit norms, [group][row]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps row addressing scalar
  // XCD-aware id: consecutive ids go to different XCDs (8 of them); renumber so
  // that each XCD's ids are contiguous, then slices vary fastest.
  int j = blockIdx.x;
  if ((gridDim.x & 7) == 0) j = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int slice = j % a.nslice;
  const int first_blk = j / a.nslice;
  const int my_blocks = first_blk < a.nblocks ? (a.nblocks - 1 - first_blk) / a.per_slice + 1 : 0;

  // Slice geometry.  Lanes past the end of K (only in the last slice) read
  // zeros and own all-zero tables.
  const int64_t c_lane = static_cast<int64_t>(slice) * G::SLICE_COLS + lane * G::LANE_COLS;
  const bool lane_active = c_lane < a.kpad;
  const uint32_t chunk_bytes = static_cast<uint32_t>(
      min(static_cast<int64_t>(G::SLICE_BYTES), a.row_bytes - static_cast<int64_t>(slice) * G::SLICE_BYTES));
  const uint32_t chunk_norm_bytes = static_cast<uint32_t>(
      2 * min(static_cast<int64_t>(G::SLICE_GROUPS), a.ngroups - static_cast<int64_t>(slice) * G::SLICE_GROUPS));
  const uint32_t voff_data = lane_active ? static_cast<uint32_t>(lane * G::LANE_BYTES) : kOutOfRange;
  const uint64_t slice_packed = reinterpret_cast<uint64_t>(a.packed) + static_cast<uint64_t>(slice) * G::SLICE_BYTES;
  const uint64_t slice_norms =
      reinterpret_cast<uint64_t>(a.norms) + static_cast<uint64_t>(slice) * G::SLICE_GROUPS * 2;

  // Work units: unit g of a slice is the 32 rows r0 + (g % kWaves) + kWaves*m,
  // m < 32, of row block g / kWaves.  Wave w starts with unit first_blk *
  // kWaves + w; further units of the workgroup's row blocks (first_blk,
  // first_blk + per_slice, ...) come from an LDS counter, taken one unit ahead
  // so the loads can run on into them.  The issue arbiter favours older waves;
  // with a fixed share per wave the youngest waves of a CU finished far behind
  // the others, and now they simply do fewer units.  (A per-slice counter in
  // memory shared by all workgroups of a slice measured no better.)  The loads
  // walk the rows of the current unit and then of the next one AHEAD rows
  // ahead of the arithmetic, with scalar bookkeeping: rows left in the unit and
  // the two row addresses.
  const int nunits = a.nblocks * kWaves;
  __shared__ int next_local;
  auto unit_of = [&](int grab) {  // the unit a grab stands for, nunits when none is left
    const int64_t blk = first_blk + static_cast<int64_t>(grab / kWaves) * a.per_slice;
    return blk < a.nblocks ? static_cast<int>(blk * kWaves + grab % kWaves) : nunits;
  };
  const uint64_t row_step = static_cast<uint64_t>(kWaves) * a.row_bytes;
  const uint64_t nrow_step = static_cast<uint64_t>(kWaves) * a.ngroups * 2;
  int lk = 0, nlive = 0;  // loads issued in the current unit, live rows in it
  uint64_t lp = 0;
  // The norms of a unit's 32 row chunks come in NORM_H 2-byte loads per lane
  // when the loads move on to the unit (norm j of the unit: row j /
  // SLICE_GROUPS, group j % SLICE_GROUPS; lane l takes j = 64 h + l), each
  // checked against the buffer range on its own, so groups past K read zeros.
  uint32_t nun[G::NORM_H];
  auto start_unit = [&](int uu) {
    const int64_t r0 = static_cast<int64_t>(uu / kWaves) * a.rows_per_block;
    const int64_t lrow = r0 + uu % kWaves;
    const int64_t lend = uu < nunits ? min(r0 + a.rows_per_block, a.rows) : 0;
    nlive = __builtin_amdgcn_readfirstlane(lend > lrow ? static_cast<int>((lend - lrow + kWaves - 1) / kWaves) : 0);
    lk = 0;
    lp = slice_packed + static_cast<uint64_t>(lrow) * a.row_bytes;
    const uint64_t lq = slice_norms + static_cast<uint64_t>(lrow) * a.ngroups * 2;
    const uint32_t range = nlive > 0 ? static_cast<uint32_t>((nlive - 1) * nrow_step) + chunk_norm_bytes : 0u;
    const __amdgpu_buffer_rsrc_t rq = buffer(lq, range);
#pragma unroll
    for (int h = 0; h < G::NORM_H; ++h) {
      const int j = 64 * h + lane, m = j / G::SLICE_GROUPS, gq = j % G::SLICE_GROUPS;
      const uint32_t off = 2 * gq < static_cast<int>(chunk_norm_bytes) ? static_cast<uint32_t>(m * nrow_step + 2 * gq)
                                                                       : kOutOfRange;
      nun[h] = __builtin_amdgcn_raw_buffer_load_b16(rq, off, 0, 0);
    }
  };
  auto load_next = [&](uint32_t (&d)[G::DWORDS]) {
    const bool live = lk < nlive;
    const __amdgpu_buffer_rsrc_t rd = buffer(lp, live ? chunk_bytes : 0u);
    // Keep every row's two loads in one fixed order, in the prologue as in the
    // loop: the wait counts at the loop header are merged over both paths, and
    // a different order there makes the compiler drain the prefetch ring.
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (SB == 3) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b96(rd, voff_data, 0, POL);
      d[0] = v[0];
      d[1 % G::DWORDS] = v[1];
      d[2 % G::DWORDS] = v[2];
    } else {
      d[0] = __builtin_amdgcn_raw_buffer_load_b32(rd, voff_data, 0, POL);
    }
    __builtin_amdgcn_sched_barrier(0);
    ++lk;
    lp += row_step;
  };

  // ---- tables: entry (position p, index v, lane) at byte
  //      (p >> 1) * REGION + v * 256 + lane * 4 + (p & 1) * 2.
  // The activation loads go out first and are waited for (the slice's max)
  // before the first rows are requested.
  // Fused call: the first SLICE_GROUPS * 16 threads (whole waves) rotate the
  // slice's groups into LDS with the same butterfly as cq_rotate_acts.
  if constexpr (ROT) {
    constexpr int NG = G::SLICE_GROUPS;
    static_assert((NG * 16) % 64 == 0, "whole waves rotate");
    if (tid < NG * 16) {
      const int g = tid >> 4, j = tid & 15;
      float v[8];
      cqdev::load8_f32(a.x, static_cast<int64_t>(slice) * G::SLICE_COLS + g * CQ_GROUP + j * 8, a.cols,
                       a.xvec != 0, v);
      cqdev::fwht128_unscaled(v, j);
      float4 *dst = reinterpret_cast<float4 *>(xrot + g * CQ_GROUP + j * 8);
      dst[0] = make_float4(v[0] * cqdev::kInvSqrt128, v[1] * cqdev::kInvSqrt128, v[2] * cqdev::kInvSqrt128,
                           v[3] * cqdev::kInvSqrt128);
      dst[1] = make_float4(v[4] * cqdev::kInvSqrt128, v[5] * cqdev::kInvSqrt128, v[6] * cqdev::kInvSqrt128,
                           v[7] * cqdev::kInvSqrt128);
    }
    __syncthreads();
  }
  // Four rotated activations at column `col` of the slice.
  auto xr4 = [&](int col) -> float4 {
    if constexpr (ROT)
      return *reinterpret_cast<const float4 *>(xrot + col);
    else
      return *reinterpret_cast<const float4 *>(a.xr + static_cast<int64_t>(slice) * G::SLICE_COLS + col);
  };
  const int lane_col = lane * G::LANE_COLS;  // c_lane within the slice
  float4 xv[G::LANE_COLS / 4];
#pragma unroll
  for (int c = 0; c < G::LANE_COLS / 4; ++c) {
    xv[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane_active) xv[c] = xr4(lane_col + 4 * c);
  }
  // Thread (wave w, lane) builds 32 slots of its lane: the pair of positions
  // q = w / (16 / PAIRS) (both halves of a slot) at indices v = vb + i, i < 32.
  constexpr int PAIRS = G::POSITIONS / 2;               // 2, 8, 2 pairs of positions
  constexpr int XQ = 2 * G::CODES;                      // activations of a pair of positions
  const int q = wave / (kWaves / PAIRS);
  const int vb = (wave % (kWaves / PAIRS)) * 32;
  float xq[XQ];
#pragma unroll
  for (int c = 0; c < XQ; c += 4) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane_active) v = xr4(lane_col + XQ * q + c);
    xq[c] = v.x, xq[c + 1] = v.y, xq[c + 2] = v.z, xq[c + 3] = v.w;
  }
  if (tid == 0) next_local = kWaves;

  float mx = 0.0f;
#pragma unroll
  for (int c = 0; c < G::LANE_COLS / 4; ++c)
    mx = fmaxf(fmaxf(mx, fmaxf(fabsf(xv[c].x), fabsf(xv[c].y))), fmaxf(fabsf(xv[c].z), fabsf(xv[c].w)));
  // The slice's max |xr|: DPP within 16-lane rows, then the two lane swaps.
  mx = fmaxf(mx, dpp<0xb1>(mx));   // quad_perm 1032
  mx = fmaxf(mx, dpp<0x4e>(mx));   // quad_perm 2301
  mx = fmaxf(mx, dpp<0x141>(mx));  // row_half_mirror
  mx = fmaxf(mx, dpp<0x128>(mx));  // row_ror:8
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  // Only now the first AHEAD rows: issued together with the activations, the
  // whole chip's burst of row loads held the activations back by several us.
  constexpr int AH = G::AHEAD;
  uint32_t dw[AH][G::DWORDS];
  const int first_unit = my_blocks > 0 ? first_blk * kWaves + wave : nunits;
  start_unit(first_unit);
#pragma unroll
  for (int u = 0; u < AH; ++u) load_next(dw[u]);  // in flight while the tables are built
  const int kexp = table_exponent(static_cast<float>(G::CODES) * a.lev_absmax * mx);
  const float scale = ldexpf(1.0f, kexp), unscale = ldexpf(1.0f, -kexp);
  {
#pragma unroll
    for (int c = 0; c < XQ; ++c) xq[c] *= scale;  // exact: a power of two
    uint32_t *const out = reinterpret_cast<uint32_t *>(lds + q * G::REGION + vb * 256 + lane * 4);
    const float *lev = a.lev.v;
    if constexpr (SB == 1) {
      // position h of the pair: bit m of v selects -c or +c for column 8h + m;
      // bits 5..7 are fixed for this thread, bits 0..1 and 2..4 are summed
      // from small tables, each sum in a fixed order (one rounded product,
      // then fused multiply-adds)
      float a2[2][4], b3[2][8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float fixed = __builtin_fmaf(lev[(vb >> 7) & 1], xq[8 * h + 7],
                                           __builtin_fmaf(lev[(vb >> 6) & 1], xq[8 * h + 6], lev[(vb >> 5) & 1] * xq[8 * h + 5]));
#pragma unroll
        for (int t = 0; t < 4; ++t) a2[h][t] = __builtin_fmaf(lev[(t >> 1) & 1], xq[8 * h + 1], lev[t & 1] * xq[8 * h]);
#pragma unroll
        for (int t = 0; t < 8; ++t)
          b3[h][t] = __builtin_fmaf(lev[(t >> 2) & 1], xq[8 * h + 4],
                                    __builtin_fmaf(lev[(t >> 1) & 1], xq[8 * h + 3], __builtin_fmaf(lev[t & 1], xq[8 * h + 2], fixed)));
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) out[i * 64] = pack_half2(a2[0][i & 3] + b3[0][i >> 2], a2[1][i & 3] + b3[1][i >> 2]);
    } else if constexpr (SB == 2) {
      // position h of the pair: codes (v&3, v>>2&3, v>>4&3, v>>6) of columns 4h..4h+3.
      // entry = lo[v & 15] + hi[bit 4 of v], each half summed in a fixed order
      // (one rounded product, then a fused multiply-add); bits 5..7 of v are
      // fixed for this thread.
      const int c2hi = (vb >> 5) & 1, c3 = vb >> 6;
      float lo[2][16], hi[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int c = 0; c < 16; ++c) lo[h][c] = __builtin_fmaf(lev[c >> 2], xq[4 * h + 1], lev[c & 3] * xq[4 * h]);
#pragma unroll
        for (int b = 0; b < 2; ++b) hi[h][b] = __builtin_fmaf(lev[c3], xq[4 * h + 3], lev[2 * c2hi + b] * xq[4 * h + 2]);
      }
#pragma unroll
      for (int i = 0; i < 32; ++i)
        out[i * 64] = pack_half2(lo[0][i & 15] + hi[0][i >> 4], lo[1][i & 15] + hi[1][i >> 4]);
    } else if constexpr (SB == 4) {
      // position h: codes (v&15, v>>4) of columns 2h, 2h+1 (the high code's
      // rounded product, then a fused multiply-add with the low code's level)
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int v = vb + i;
        const float t0 = __builtin_fmaf(lev[v & 15], xq[0], lev[v >> 4] * xq[1]);
        const float t1 = __builtin_fmaf(lev[v & 15], xq[2], lev[v >> 4] * xq[3]);
        out[i * 64] = pack_half2(t0, t1);
      }
    } else {
      // position h: codes (v&7, v>>3) of columns 2h, 2h+1, as at 4 bits
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int v = vb + i;
        const float t0 = __builtin_fmaf(lev[v & 7], xq[0], lev[v >> 3] * xq[1]);
        const float t1 = __builtin_fmaf(lev[v & 7], xq[2], lev[v >> 3] * xq[3]);
        out[i * 64] = pack_half2(t0, t1);
      }
    }
  }
  __syncthreads();

  const uint32_t base0 = static_cast<uint32_t>(lane) * 4u;
  const uint32_t base1 = base0 + 0x10000u;
  const int norm_group = lane / G::LANES_PER_GROUP;  // this lane's group within the slice
  int u = first_unit, un = nunits;
  uint32_t grabbed = 0;  // lane 0: the grab for the unit after this one
  while (u < nunits) {
    const int64_t r0 = static_cast<int64_t>(u / kWaves) * a.rows_per_block;
    const int64_t r1 = min(r0 + static_cast<int64_t>(a.rows_per_block), a.rows);
    // Lookups of row m are issued before the accumulation of row m-1, so the
    // LDS latency of a row is covered by the next row's address and load work.
    float racc[kRowsPerWave];
    _Float16 tv[2][G::LOOKUPS];
    _Float16 nv[2];
    uint4 nb8;
    auto accumulate = [&](int m) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < G::LOOKUPS; ++k)
        acc = fmaf(static_cast<float>(tv[m & 1][k]), static_cast<float>(nv[m & 1]), acc);
      asm volatile("" : "+v"(acc));  // keep the sums here: sunk to the unit's end they hold every lookup live
      racc[m] = acc;
    };
#pragma unroll
    for (int m = 0; m < kRowsPerWave; ++m) {
      const int slot = m % AH;
      uint32_t cur[G::DWORDS];
#pragma unroll
      for (int d = 0; d < G::DWORDS; ++d) cur[d] = dw[slot][d];
      if (m == 0) {  // this unit's norms into the wave's buffer (written and read as uint16_t)
#pragma unroll
        for (int h = 0; h < G::NORM_H; ++h) {
          const int jn = 64 * h + lane;
          nbuf[wave][(jn % G::SLICE_GROUPS) * NBS + jn / G::SLICE_GROUPS] = static_cast<uint16_t>(nun[h]);
        }
      }
      // one 16-byte read brings the norms of 8 rows; the fma picks its half
      if (m % 8 == 0) nb8 = *reinterpret_cast<const uint4 *>(&nbuf[wave][norm_group * NBS + m]);
      {
        const uint32_t d = (m % 8) / 2 == 0 ? nb8.x : ((m % 8) / 2 == 1 ? nb8.y : ((m % 8) / 2 == 2 ? nb8.z : nb8.w));
        nv[m & 1] = __builtin_bit_cast(_Float16, static_cast<uint16_t>(d >> (16 * (m % 2))));
      }
      if (m == 0 && lane == 0) grabbed = static_cast<uint32_t>(atomicAdd(&next_local, 1));
      // the loads move on to the next unit (with AH = kRowsPerWave at row 0,
      // right after the grab and after this unit's norms went to the buffer)
      if (m + AH == kRowsPerWave) {
        un = unit_of(static_cast<int>(__builtin_amdgcn_readfirstlane(grabbed)));
        start_unit(un);
      }
      load_next(dw[slot]);
      if constexpr (SB == 3) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {  // 6-bit field k: codes 2k, 2k+1
          const int bit = 6 * k, w = bit >> 5, sh = bit & 31;
          const uint32_t f = sh <= 26 ? __builtin_amdgcn_ubfe(cur[w], sh, 6)
                                      : (__builtin_amdgcn_alignbit(cur[(w + 1) % G::DWORDS], cur[w], sh) & 63u);
          const uint32_t addr = (f << 8) | (k < 8 ? base0 : base1);
          tv[m & 1][k] = lds_half(lds, addr + ((k >> 1) & 3) * G::REGION + (k & 1) * 2);
        }
      } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) {  // byte p of the lane's dword
          const uint32_t addr = __builtin_amdgcn_perm(cur[0], p < 2 ? base0 : base1, 0x0C020400u + (p << 8));
          tv[m & 1][p] = lds_half(lds, addr + (p & 1) * 2);
        }
      }
      if (m > 0) accumulate(m - 1);
    }
    accumulate(kRowsPerWave - 1);
    const float t = reduce_rows(racc, lane) * unscale;
    store_block(a, slice, r0, r1, u % kWaves, lane, t);
    u = un;
  }
}

// y[r] = sum over slices, in slice order, of partial[slice][r].
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ partial, int64_t rows, int nslice,
                                                      float *__restrict__ y) {
  constexpr int CH = 16;  // loads in flight per thread
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; r < rows; r += stride) {
    float acc = 0.0f;
    for (int s0 = 0; s0 < nslice; s0 += CH) {
      float v[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) v[c] = s0 + c < nslice ? partial[static_cast<int64_t>(s0 + c) * rows + r] : 0.0f;
#pragma unroll
      for (int c = 0; c < CH; ++c) acc += v[c];  // slice order (the padding adds +0)
    }
    y[r] = acc;
  }
}

// Shape of one launch: slices of K, row blocks and persistent workgroups.
struct MvShape {
  int32_t nslice, rows_per_block, nblocks, per_slice;
};

int slice_cols(int sb) {
  return sb == 1 ? Geom<1>::SLICE_COLS
                 : (sb == 2 ? Geom<2>::SLICE_COLS : (sb == 3 ? Geom<3>::SLICE_COLS : Geom<4>::SLICE_COLS));
}

typedef void (*MvKernel)(MvArgs);

template <bool ROT, int POL>
MvKernel pick_sb(int sb) {
  return sb == 1 ? matvec_kernel<1, ROT, POL>
                 : (sb == 2 ? matvec_kernel<2, ROT, POL> : (sb == 3 ? matvec_kernel<3, ROT, POL> : matvec_kernel<4, ROT, POL>));
}

// stream: the code rows' loads carry the nt hint (cq::kStreamLoad)
MvKernel pick_kernel(int sb, bool rot = false, bool stream = false) {
  if (stream) return rot ? pick_sb<true, cq::kStreamLoad>(sb) : pick_sb<false, cq::kStreamLoad>(sb);
  return rot ? pick_sb<true, 0>(sb) : pick_sb<false, 0>(sb);
}

int max_grid(int sb) {
  // Resident workgroups per CU for this kernel, times the CU count of the
  // current device; computed once per (device, width).
  // (atomic: host threads may launch concurrently; a racing first call only
  // computes the same value twice)
  static std::atomic<int> cache[64][4];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int c = cache[dev][sb - 1].load(std::memory_order_relaxed);
  if (c == 0) {
    int per_cu = 1, cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(pick_kernel(sb)),
                                                     kThreads, 0) != hipSuccess || per_cu < 1)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    c = per_cu * cus;
    cache[dev][sb - 1].store(c, std::memory_order_relaxed);
  }
  return c;
}

MvShape mv_shape(int sb, int64_t rows, int64_t kpad) {
  MvShape s;
  const int64_t sc = slice_cols(sb);
  const int grid_max = max_grid(sb);
  s.nslice = static_cast<int32_t>((kpad + sc - 1) / sc);
  // Aim at grid_max busy workgroups: small matrices get small row blocks.
  int64_t rpb = (rows * s.nslice + grid_max - 1) / grid_max;
  rpb = (rpb + kWaves - 1) / kWaves * kWaves;
  if (rpb < kWaves) rpb = kWaves;
  if (rpb > kRowsPerBlock) rpb = kRowsPerBlock;
  s.rows_per_block = static_cast<int32_t>(rpb);
  s.nblocks = static_cast<int32_t>((rows + rpb - 1) / rpb);
  int64_t ps = s.nslice >= grid_max ? 1 : grid_max / s.nslice;
  if (ps > s.nblocks) ps = s.nblocks;
  s.per_slice = static_cast<int32_t>(ps);
  return s;
}

float lev_absmax(int sb, const cq::CodeLevels &lev) {
  float m = 0.0f;
  for (int i = 0; i < (1 << sb); ++i) m = fmaxf(m, fabsf(lev.v[i]));
  return m;
}

}  // namespace

namespace cq {

#ifndef CQ_LUT_MIN_WEIGHTS
#define CQ_LUT_MIN_WEIGHTS (int64_t{1} << 23)
#endif
// Kernel choice, from batch-1 and batch-8 timings on MI355X.  With
// cols_pad <= 4096 the small-matrix kernel is faster up to 64 M weights
// (batch 1: 8.0 us at 512 x 512 and 14.2 us at 16384 x 4096, against 13.0
// and 16.4 us on the lookup tables) and slower from 128 M.  With more
// columns, batch 1 takes the lookup tables from 2^23 weights and the batched
// matrix-core kernel below (every width, binary included).
static bool use_small(int bits, int64_t rows, int64_t kpad, int64_t batch) {
  (void)bits;
  return rows * kpad <= kSmallMaxWeights && small_matvec_fits(kpad, batch);
}

static bool use_lut(int bits, int64_t rows, int64_t kpad, int64_t batch) {
  (void)bits;
  // the unit norm offsets (32 rows 16 rows apart) are 32-bit: K below 2^28
  return batch == 1 && rows * kpad >= static_cast<int64_t>(CQ_LUT_MIN_WEIGHTS) && kpad < (int64_t{1} << 28);
}

// Workspace of one call: the per-slice partial sums, [nslice][rows] (fp32)
// for the lookup-table kernel, [nslice][batch][rows] for the matrix-core one.
uint64_t matvec_workspace_bytes(int bits, int64_t rows, int64_t kpad, int64_t batch) {
  if (rows <= 0 || kpad <= 0 || batch <= 0) return 0;  // nothing is launched
  if (use_small(bits, rows, kpad, batch)) return 0;
  if (!use_lut(bits, rows, kpad, batch)) return matvec_mma_workspace_bytes(rows, kpad, batch);
  const MvShape s = mv_shape(storage_bits(bits), rows, kpad);  // one [nslice][rows] reused by each batch row
  if (s.nslice <= 1) return 0;
  return static_cast<uint64_t>(s.nslice) * rows * 4;
}

uint64_t rotate_matvec_workspace_bytes(int bits, int64_t rows, int64_t kpad, int64_t batch) {
  if (rows <= 0 || kpad <= 0 || batch <= 0) return 0;
  if (use_small(bits, rows, kpad, batch)) return 0;
  if (use_lut(bits, rows, kpad, batch)) return matvec_workspace_bytes(bits, rows, kpad, 1);
  return (matvec_mma_workspace_bytes(rows, kpad, batch) + 15) / 16 * 16 + static_cast<uint64_t>(batch) * kpad * 4;
}

hipError_t launch_combine(const float *partial, int64_t n, int nslice, float *y, hipStream_t s) {
  const int64_t cblocks = (n + 255) / 256;
  const unsigned cgrid = static_cast<unsigned>(cblocks < 65536 ? cblocks : 65536);
  combine_kernel<<<cgrid, 256, 0, s>>>(partial, n, nslice, y);
  return hipGetLastError();
}

namespace {

// One lookup-table pass (batch 1): from the rotated xr, or (x != nullptr)
// rotating x in the kernel.
hipError_t launch_lut(const uint8_t *blob, int bits, int64_t rows, int64_t kpad, const CodeLevels &lev,
                      const float *xr, const float *x, int64_t cols, float *y, void *workspace, hipStream_t s) {
  const int sb = storage_bits(bits);
  const MvShape sh = mv_shape(sb, rows, kpad);
  MvArgs a;
  a.packed = blob;
  a.row_bytes = kpad * sb / 8;
  a.norms = reinterpret_cast<const uint16_t *>(blob + rows * a.row_bytes);
  a.xr = xr;
  a.x = x;
  a.cols = cols;
  a.xvec = x != nullptr && cols % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  a.y = y;
  a.rows = rows;
  a.kpad = kpad;
  a.ngroups = kpad / CQ_GROUP;
  a.lev = lev;
  a.lev_absmax = lev_absmax(sb, lev);
  a.nslice = sh.nslice;
  a.rows_per_block = sh.rows_per_block;
  a.nblocks = sh.nblocks;
  a.per_slice = sh.per_slice;
  a.partial = sh.nslice > 1 ? static_cast<float *>(workspace) : nullptr;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(sh.nslice) * sh.per_slice));
  const bool stream = rows * (a.row_bytes + 2 * a.ngroups) >= cq::kStreamMinBytes;
  pick_kernel(sb, x != nullptr, stream)<<<grid, kThreads, 0, s>>>(a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || sh.nslice <= 1) return e;
  return launch_combine(a.partial, rows, sh.nslice, y, s);
}

}  // namespace

hipError_t launch_matvec(const uint8_t *blob, int bits, int64_t rows, int64_t kpad, const CodeLevels &lev,
                         const float *xr, int64_t batch, float *y, void *workspace, hipStream_t s) {
  if (use_small(bits, rows, kpad, batch)) {
    const MultiItem item = {blob, bits, rows, lev, y};
    return launch_small_matvec(&item, 1, xr, false, kpad, kpad, batch, s);
  }
  if (!use_lut(bits, rows, kpad, batch)) return launch_matvec_mma(blob, bits, rows, kpad, lev, xr, batch, y, workspace, s);
  hipError_t e = hipSuccess;
  for (int64_t b = 0; b < batch && e == hipSuccess; ++b)  // stream order: the partial sums are reused
    e = launch_lut(blob, bits, rows, kpad, lev, xr + b * kpad, nullptr, 0, y + b * rows, workspace, s);
  return e;
}

hipError_t launch_rotate_matvec(const uint8_t *blob, int bits, int64_t rows, int64_t kpad, const CodeLevels &lev,
                                const float *x, int64_t cols, int64_t batch, float *y, void *workspace,
                                hipStream_t s) {
  if (use_small(bits, rows, kpad, batch)) {
    const MultiItem item = {blob, bits, rows, lev, y};
    return launch_small_matvec(&item, 1, x, true, cols, kpad, batch, s);
  }
  if (use_lut(bits, rows, kpad, batch)) {
    hipError_t e = hipSuccess;
    for (int64_t b = 0; b < batch && e == hipSuccess; ++b)
      e = launch_lut(blob, bits, rows, kpad, lev, nullptr, x + b * cols, cols, y + b * rows, workspace, s);
    return e;
  }
  // Batches: every workgroup of a K slice would redo the slice's rotation, so
  // it runs once, into the workspace after the partial sums.
  const uint64_t part = matvec_mma_workspace_bytes(rows, kpad, batch);
  float *xr = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + (part + 15) / 16 * 16);
  const hipError_t e = launch_rotate(x, CQ_F32, batch, cols, kpad, xr, CQ_F32, s);
  if (e != hipSuccess) return e;
  return launch_matvec_mma(blob, bits, rows, kpad, lev, xr, batch, y, part ? workspace : nullptr, s);
}

uint64_t rotate_multi_workspace_bytes(const MultiItem *items, int n, int64_t kpad, int64_t batch) {
  if (kpad <= 0 || batch <= 0) return 0;
  uint64_t part = 0;
  bool shared = false;
  for (int i = 0; i < n; ++i) {
    if (items[i].rows <= 0 || use_small(items[i].bits, items[i].rows, kpad, batch)) continue;
    shared = true;
    const uint64_t p = matvec_workspace_bytes(items[i].bits, items[i].rows, kpad, batch);
    if (p > part) part = p;
  }
  if (!shared) return 0;
  return (part + 15) / 16 * 16 + static_cast<uint64_t>(batch) * kpad * 4;
}

hipError_t launch_rotate_multi_matvec(const MultiItem *items, int n, const float *x, int64_t cols, int64_t kpad,
                                      int64_t batch, void *workspace, hipStream_t s) {
  MultiItem small[64];
  int nsmall = 0;
  bool shared = false;
  uint64_t part = 0;
  for (int i = 0; i < n; ++i) {
    if (items[i].rows <= 0) continue;
    if (use_small(items[i].bits, items[i].rows, kpad, batch)) {
      if (nsmall == 64) return hipErrorInvalidValue;
      small[nsmall++] = items[i];
    } else {
      shared = true;
      const uint64_t p = matvec_workspace_bytes(items[i].bits, items[i].rows, kpad, batch);
      if (p > part) part = p;
    }
  }
  if (nsmall) {
    const hipError_t e = launch_small_matvec(small, nsmall, x, true, cols, kpad, batch, s);
    if (e != hipSuccess) return e;
  }
  if (!shared) return hipSuccess;
  // the larger matrices: one rotation, shared through the workspace
  float *xr = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + (part + 15) / 16 * 16);
  hipError_t e = launch_rotate(x, CQ_F32, batch, cols, kpad, xr, CQ_F32, s);
  for (int i = 0; i < n && e == hipSuccess; ++i) {
    const MultiItem &it = items[i];
    if (it.rows <= 0 || use_small(it.bits, it.rows, kpad, batch)) continue;
    e = launch_matvec(it.blob, it.bits, it.rows, kpad, it.lev, xr, batch, it.y, part ? workspace : nullptr, s);
  }
  return e;
}

}  // namespace cq
