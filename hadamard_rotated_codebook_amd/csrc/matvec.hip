// Decode matrix-vector product y = W . x for a CQ matrix (equation (1) of
// include/cq.h), computed as sum_g norm_g * <c[q_g], H x_g> on the rotated
// activation xr (OpenNeedle reference notes, rotated-activation identity; the
// ".cact" format post, "How the kernel reads it": the kernel never expands the
// stored indices and no weight is materialised).
//
// Design (HBM-bound at batch 1):
//  * K is cut into slices whose lookup tables fill 128 KB of LDS.  A
//    persistent 512-thread workgroup per CU owns one slice, builds its tables
//    once from the rotated activation, and then streams its slice of the packed
//    bytes of several 256-row blocks.  The workgroups of the other slices run
//    at the same time on other CUs and read the other parts of the same rows,
//    so every packed row is fetched whole from HBM within a short window (a
//    slice-by-slice walk of K inside one workgroup leaves 1 KB holes in each
//    4 KB row and measured ~35 % slower).
//  * 2-bit rows (CQ2 and ternary crumbs): one 16-entry table per pair of
//    columns, T[v] = lev[v & 3] * x0 + lev[v >> 2] * x1, so one nibble of
//    packed data (two weights) costs one LDS read and one add.
//    4-bit rows: one 16-entry table per column, T[v] = lev[v] * x.
//  * A lane reads 16 consecutive packed bytes of a row (dwordx4, coalesced).
//    The nibble -> table address is one v_perm_b32 that drops the data byte
//    next to a per-lane slot: address = value*stride + lane*4 + block*blk_stride,
//    so in every LDS read the 64 lanes hit 64 different 4-byte slots (one
//    table per lane) and the access is bank-conflict free.
//  * Low nibbles index region 0 (stride 256 B per value), high nibbles region
//    1 (their value already sits at bits 4..7, so stride 4096 B); both masks
//    take one AND per dword.
//  * 3-bit rows: one 8-entry table per column; the 3-bit field is extracted
//    with v_bfe (indices cross byte boundaries) and placed next to the lane
//    slot with one shift-or.
//  * Every lane keeps one partial per row slot; the group norm scales it once
//    per row, and a halving exchange reduces all row slots of a wave at the
//    end of a row block.  Loads run kAhead rows ahead of the arithmetic, across
//    row-block boundaries, from clamped in-bounds addresses (no branches, so
//    the compiler never has to drain the load queue).
//  * With more than one slice, each workgroup writes its per-row partials to
//    the caller's workspace; the last of the slices to finish a row block
//    (an agent-scope counter, release/acquire fences) adds the partials in
//    slice order and writes y, then resets the counter: the result does not
//    depend on which workgroup finishes first.
#include "cq_internal.h"

namespace {

#ifndef CQ_MV_THREADS
#define CQ_MV_THREADS 512
#endif
#ifndef CQ_MV_ROWS_PER_WAVE
#define CQ_MV_ROWS_PER_WAVE 32
#endif
#ifndef CQ_MV_AHEAD
#define CQ_MV_AHEAD 8
#endif
constexpr int kThreads = CQ_MV_THREADS;     // one workgroup per CU (128 KB LDS)
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerWave = CQ_MV_ROWS_PER_WAVE;     // row slots per wave (fully unrolled)
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;  // rows of one row block (256)
constexpr int kAhead = CQ_MV_AHEAD;         // rows whose loads are in flight ahead of the arithmetic
static_assert((kRowsPerWave & (kRowsPerWave - 1)) == 0 && kRowsPerWave <= 64, "row slots: power of two");
static_assert(kRowsPerWave % kAhead == 0, "prefetch ring must divide the row slots");

struct MvArgs {
  const uint8_t *packed;
  const uint16_t *norms;  // fp16 bits, [rows][ngroups]
  const float *xr;        // [nb][kpad]
  float *y;               // [nb][rows]
  float *partial;         // [nslice][nb][rows] (nslice > 1)
  uint32_t *counter;      // [nblocks] (nslice > 1), zero between calls
  int64_t rows, kpad, row_bytes, ngroups;
  int32_t rows_per_block;  // multiple of kWaves, <= kRowsPerBlock
  int32_t nblocks;         // row blocks
  int32_t nslice;          // K slices
  int32_t per_slice;       // workgroups per slice (grid = nslice * per_slice)
  cq::CodeLevels lev;
};

__device__ inline float half_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ inline float lds_at(const float *lds, uint32_t byte_addr) {
  return *reinterpret_cast<const float *>(reinterpret_cast<const char *>(lds) + byte_addr);
}

// Lanes that hold row slot m after reduce_rows: lanes kLanesPerRow*m ... +kLanesPerRow-1.
constexpr int kLanesPerRow = 64 / kRowsPerWave;

// Bitwise select (one v_bfi_b32): a where mask is 0, b where it is all ones.
__device__ inline float pick(float a, float b, uint32_t mask) {
  return __uint_as_float((__float_as_uint(a) & ~mask) | (__float_as_uint(b) & mask));
}

// Sum kRowsPerWave per-lane partials over the 64 lanes of a wave.  Halving
// exchange: at lane distance 32, 16, ... each lane keeps half of its values
// (upper lanes the upper half) and adds the partner's copy of them; the rest of
// the lane distances then sum the remaining single value.  Afterwards the
// lanes kLanesPerRow*m .. +kLanesPerRow-1 hold the total of row slot m.
__device__ inline float reduce_rows(float (&v)[kRowsPerWave], int lane) {
#pragma unroll
  for (int half = kRowsPerWave / 2, dist = 32; half >= 1; half >>= 1, dist >>= 1) {
    const uint32_t upper = (lane & dist) ? 0xffffffffu : 0u;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float keep = pick(v[i], v[half + i], upper);
      const float send = pick(v[half + i], v[i], upper);
      v[i] = keep + __shfl_xor(send, dist);
    }
  }
  float t = v[0];
#pragma unroll
  for (int dist = kLanesPerRow / 2; dist >= 1; dist >>= 1) t += __shfl_xor(t, dist);
  return t;
}

// Write a row block's per-row totals: directly to y with one slice, else via
// the workspace, where the last slice to arrive adds the partials in slice
// order.  All threads of the workgroup call this (it contains barriers).
//
// The partials cross CUs (and XCDs, whose L2s are not coherent with each
// other for plain stores): they are written and read with agent-scope atomic
// stores/loads, which bypass the non-coherent cache levels.  Each thread waits
// for its stores to complete (workgroup-scope release: a counter wait, no
// cache flush) before the barrier; only then does one thread bump the row
// block's counter.  The last arriver reads the partials, writes y, and clears
// the partials and the counter, so the workspace is all zeros between calls.
template <int NB>
__device__ void finish_block(const MvArgs &a, int slice, int blk, int64_t r0, int64_t r1, int wave, int lane,
                             const float (&t)[NB]) {
  const int64_t r = r0 + wave + static_cast<int64_t>(kWaves) * (lane / kLanesPerRow);
  const bool writer = lane % kLanesPerRow == 0 && r < r1;
  if (a.nslice == 1) {
    if (writer)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) a.y[nb * a.rows + r] = t[nb];
    return;
  }
  if (writer)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      __hip_atomic_store(a.partial + (static_cast<int64_t>(slice) * NB + nb) * a.rows + r, t[nb], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  __shared__ int is_last;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.counter + blk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = old == static_cast<uint32_t>(a.nslice - 1);
  }
  __syncthreads();
  if (is_last) {
    const int n = static_cast<int>(r1 - r0);
    for (int i = threadIdx.x; i < NB * n; i += kThreads) {
      const int nb = i / n;
      const int64_t rr = r0 + (i - nb * n);
      float acc = 0.0f;
      for (int sl = 0; sl < a.nslice; ++sl) {
        float *p = a.partial + (static_cast<int64_t>(sl) * NB + nb) * a.rows + rr;
        acc += __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p, 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      a.y[nb * a.rows + rr] = acc;
    }
    if (threadIdx.x == 0) __hip_atomic_store(a.counter + blk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// One kernel for all widths.  SB = 2 or 4: nibble tables; SB = 3: column tables
// (one batch vector).  NB batch vectors share each packed byte.
// Table layouts (per lane slot s = lane*4 bytes, nibble value v):
//  * wide (D*NB == 4, 128 KB): low nibbles at v*256 + s + blk*4096, high nibbles
//    left in place (value*16) at 64 KB + v*4096 + s + blk*256;
//  * compact (D*NB <= 2, 32*D*NB KB): both nibbles at v*256 + s + blk*4096, the
//    high nibble shifted down first (one extra shift per dword).
template <int SB, int NB, int D>
__global__ __launch_bounds__(kThreads) void matvec_kernel(MvArgs a) {
  static_assert(SB != 3 || (NB == 1 && D == 3), "3-bit rows: one batch vector, 12 bytes per lane");
  static_assert(SB == 3 || D * NB <= 4, "nibble tables fit 128 KB");
  constexpr bool WIDE = SB != 3 && D * NB == 4;
  constexpr int LDS_FLOATS = SB == 3 ? 16384 : 8192 * D * NB;
  __shared__ float lds[LDS_FLOATS];
  constexpr int LANE_COLS = SB == 3 ? 32 : 4 * D * (8 / SB);  // columns per lane
  constexpr int SLICE_COLS = 64 * LANE_COLS;
  constexpr int SLICE_BYTES = SLICE_COLS * SB / 8;
  constexpr int BLOCKS = 4 * D;                      // nibble tables per lane, region, batch vector
  constexpr int TPT = SB == 3 ? (LANE_COLS + kWaves - 1) / kWaves : (2 * NB * BLOCKS + kWaves - 1) / kWaves;
  constexpr int NTAB = SB == 3 ? LANE_COLS : 2 * NB * BLOCKS;  // tables per lane slot
  constexpr int XPT = SB == 2 ? 2 : 1;               // activations per table

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps row addressing scalar
  const int slice = blockIdx.x % a.nslice;
  const int first_blk = blockIdx.x / a.nslice;
  const int64_t c_lane = static_cast<int64_t>(slice) * SLICE_COLS + lane * LANE_COLS;  // lane's first column
  const bool lane_active = c_lane < a.kpad;
  const uint32_t lane_byte = lane_active ? static_cast<uint32_t>(lane * (LANE_COLS * SB / 8)) : 0u;
  const uint32_t lane_group = lane_active ? static_cast<uint32_t>(lane * LANE_COLS) >> 7 : 0u;
  const uint8_t *slice_packed = a.packed + static_cast<int64_t>(slice) * SLICE_BYTES;
  const uint16_t *slice_norms = a.norms + static_cast<int64_t>(slice) * (SLICE_COLS / 128);

  // Lanes past the end of K in the last slice read table slots that nothing
  // writes; their partials are multiplied by a zero norm, so clear LDS once to
  // keep those reads finite.
  for (int i = tid; i < LDS_FLOATS / 4; i += kThreads)
    reinterpret_cast<float4 *>(lds)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  __syncthreads();

  // Build this slice's tables.  Thread (wave, lane) builds tables
  // t = wave + kWaves*i in its lane's slot.
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int t = wave + kWaves * i;
    if (t >= NTAB) break;
    if (SB == 3) {
      const int64_t c = c_lane + t;
      const float x0 = c < a.kpad ? a.xr[c] : 0.0f;
#pragma unroll
      for (int v = 0; v < 8; ++v) lds[(v * 256u + lane * 4u + t * 2048u) >> 2] = a.lev.v[v] * x0;
    } else {
      const int hi = t & 1, blk = t >> 1, nb = blk / BLOCKS, beta = blk - nb * BLOCKS;
      const int64_t c = c_lane + (SB == 2 ? 4 * beta + 2 * hi : 2 * beta + hi);
      float x[XPT];
#pragma unroll
      for (int e = 0; e < XPT; ++e) x[e] = c < a.kpad ? a.xr[nb * a.kpad + c + e] : 0.0f;
      float e16[16];
      if (SB == 2) {
#pragma unroll
        for (int v = 0; v < 16; ++v) e16[v] = a.lev.v[v & 3] * x[0] + a.lev.v[v >> 2] * x[XPT - 1];
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) e16[v] = a.lev.v[v] * x[0];
      }
      uint32_t off, stride;
      if (WIDE) {
        off = hi ? 0x10000u + blk * 256u + lane * 4u : blk * 4096u + lane * 4u;
        stride = hi ? 4096u : 256u;
      } else {
        off = (hi * BLOCKS * NB + blk) * 4096u + lane * 4u;
        stride = 256u;
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) lds[(off + v * stride) >> 2] = e16[v];
    }
  }
  __syncthreads();

  // Row streams: this workgroup's row blocks are first_blk, first_blk +
  // per_slice, ...; row slot m of a block is row r0 + wave + kWaves*m.  Loads
  // walk that sequence kAhead rows ahead of the arithmetic with wave-uniform
  // pointers: +kWaves rows per slot, a jump per row block, and a clamp to the
  // last row (the clamped rows past the end are computed and discarded).
  const int my_blocks = (a.nblocks - 1 - first_blk) / a.per_slice + 1;  // >= 1: first_blk < nblocks
  const int64_t slot_stride = static_cast<int64_t>(kWaves) * a.row_bytes;
  const int64_t nslot_stride = static_cast<int64_t>(kWaves) * a.ngroups;
  const uint8_t *const last_row = slice_packed + (a.rows - 1) * a.row_bytes;
  const uint16_t *const last_nrow = slice_norms + (a.rows - 1) * a.ngroups;
  auto block_row = [&](int bi) {  // row of slot 0 of this wave in the bi-th block
    return (first_blk + static_cast<int64_t>(bi) * a.per_slice) * a.rows_per_block + wave;
  };
  const uint8_t *lp = slice_packed + block_row(0) * a.row_bytes;  // next row to load
  const uint16_t *lq = slice_norms + block_row(0) * a.ngroups;
  auto load_next = [&](uint32_t (&dw)[D], uint32_t &nraw) {
    const uint8_t *p = lp < last_row ? lp : last_row;
    const uint16_t *q = lq < last_nrow ? lq : last_nrow;
    const uint8_t *src = p + lane_byte;
    if (D == 4) {
      const uint4 v = *reinterpret_cast<const uint4 *>(src);
      dw[0] = v.x; dw[1 % D] = v.y; dw[2 % D] = v.z; dw[3 % D] = v.w;
    } else if (D == 3) {
      const uint32_t *w = reinterpret_cast<const uint32_t *>(src);
      dw[0] = w[0]; dw[1 % D] = w[1 % D]; dw[2 % D] = w[2 % D];
    } else if (D == 2) {
      const uint2 v = *reinterpret_cast<const uint2 *>(src);
      dw[0] = v.x; dw[1 % D] = v.y;
    } else {
      dw[0] = *reinterpret_cast<const uint32_t *>(src);
    }
    nraw = q[lane_group];
    lp += slot_stride;
    lq += nslot_stride;
  };

  const uint32_t base_lo = static_cast<uint32_t>(lane) * 4u;
  const uint32_t base_hi = static_cast<uint32_t>(lane) * 4u + 0x10000u;
  uint32_t dw[kAhead][D];
  uint32_t nraw[kAhead];
#pragma unroll
  for (int u = 0; u < kAhead; ++u) load_next(dw[u], nraw[u]);

  for (int bi = 0; bi < my_blocks; ++bi) {
    const int blk = first_blk + bi * a.per_slice;
    const int64_t r0 = static_cast<int64_t>(blk) * a.rows_per_block;
    const int64_t r1 = min(r0 + static_cast<int64_t>(a.rows_per_block), a.rows);
    float racc[NB][kRowsPerWave];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int m = 0; m < kRowsPerWave; ++m) racc[nb][m] = 0.0f;

#pragma unroll
    for (int m = 0; m < kRowsPerWave; ++m) {
      const int slot = m % kAhead;
      uint32_t cur[D];
#pragma unroll
      for (int d = 0; d < D; ++d) cur[d] = dw[slot][d];
      const uint32_t ncur = nraw[slot];
      if (m + kAhead == kRowsPerWave) {  // the loads move on to the next row block
        lp = slice_packed + block_row(bi + 1) * a.row_bytes;
        lq = slice_norms + block_row(bi + 1) * a.ngroups;
      }
      load_next(dw[slot], nraw[slot]);
      {
        const float n = lane_active ? half_to_float(static_cast<uint16_t>(ncur)) : 0.0f;
        if (SB == 3) {
          float tv[32];
#pragma unroll
          for (int k = 0; k < 32; ++k) {
            const int bit = 3 * k, w = bit >> 5, sh = bit & 31;
            const uint32_t code = sh <= 29 ? __builtin_amdgcn_ubfe(cur[w % D], sh, 3)
                                           : (__builtin_amdgcn_alignbit(cur[(w + 1) % D], cur[w % D], sh) & 7u);
            tv[k] = lds_at(lds, ((code << 8) | base_lo) + k * 2048u);
          }
#pragma unroll
          for (int w = 1; w < 32; w <<= 1)
#pragma unroll
            for (int i = 0; i + w < 32; i += 2 * w) tv[i] += tv[i + w];
          racc[0][m] = fmaf(tv[0], n, racc[0][m]);
        } else {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            // All LDS reads of the row first, then a pairwise sum.
            float tv[8 * D];
#pragma unroll
            for (int d = 0; d < D; ++d) {
              const uint32_t lo = cur[d] & 0x0F0F0F0Fu;
              const uint32_t hi = WIDE ? (cur[d] & 0xF0F0F0F0u) : ((cur[d] >> 4) & 0x0F0F0F0Fu);
#pragma unroll
              for (int jb = 0; jb < 4; ++jb) {
                const uint32_t sel = 0x0C020400u + (static_cast<uint32_t>(jb) << 8);
                const uint32_t tb = nb * BLOCKS + 4 * d + jb;
                tv[8 * d + 2 * jb] = lds_at(lds, __builtin_amdgcn_perm(lo, base_lo, sel) + tb * 4096u);
                if (WIDE)
                  tv[8 * d + 2 * jb + 1] = lds_at(lds, __builtin_amdgcn_perm(hi, base_hi, sel) + tb * 256u);
                else
                  tv[8 * d + 2 * jb + 1] = lds_at(lds, __builtin_amdgcn_perm(hi, base_lo, sel) + (BLOCKS * NB + tb) * 4096u);
              }
            }
#pragma unroll
            for (int w = 1; w < 8 * D; w <<= 1)
#pragma unroll
              for (int i = 0; i + w < 8 * D; i += 2 * w) tv[i] += tv[i + w];
            racc[nb][m] = fmaf(tv[0], n, racc[nb][m]);
          }
        }
      }
    }
    float t[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) t[nb] = reduce_rows(racc[nb], lane);
    finish_block<NB>(a, slice, blk, r0, r1, wave, lane, t);
  }
}

#ifndef CQ_MV_D1
#define CQ_MV_D1 4  // packed dwords per lane and row for one batch vector
#endif

// Packed dwords per lane and row for a chunk of nb batch vectors.
int lane_dwords(int sb, int nb) { return sb == 3 ? 3 : (nb == 1 ? CQ_MV_D1 : 4 / nb); }

// Shape of one launch: slices of K, row blocks and persistent workgroups.
struct MvShape {
  int32_t nslice, rows_per_block, nblocks, per_slice;
};

int slice_cols(int sb, int nb) {
  if (sb == 3) return 64 * 32;
  return 64 * 4 * lane_dwords(sb, nb) * (8 / sb);
}

// Workgroups that fit on the device at once (persistent grid size).
int max_grid(int sb, int nb);

MvShape mv_shape(int sb, int nb, int64_t rows, int64_t kpad) {
  MvShape s;
  const int64_t sc = slice_cols(sb, nb);
  const int grid_max = max_grid(sb, nb);
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

typedef void (*MvKernel)(MvArgs);

MvKernel pick_kernel(int sb, int nb) {
  const int d = lane_dwords(sb, nb);
  if (sb == 3) return matvec_kernel<3, 1, 3>;
  if (sb == 2) {
    if (nb == 4) return matvec_kernel<2, 4, 1>;
    if (nb == 2) return matvec_kernel<2, 2, 2>;
    return d == 4 ? matvec_kernel<2, 1, 4> : (d == 2 ? matvec_kernel<2, 1, 2> : matvec_kernel<2, 1, 1>);
  }
  if (nb == 4) return matvec_kernel<4, 4, 1>;
  if (nb == 2) return matvec_kernel<4, 2, 2>;
  return d == 4 ? matvec_kernel<4, 1, 4> : (d == 2 ? matvec_kernel<4, 1, 2> : matvec_kernel<4, 1, 1>);
}

int max_grid(int sb, int nb) {
  // Resident workgroups per CU for this kernel, times the CU count of the
  // current device; computed once per (device, width, batch chunk).
  static int cache[64][3][3];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  const int si = sb == 2 ? 0 : (sb == 3 ? 1 : 2), ni = nb == 1 ? 0 : (nb == 2 ? 1 : 2);
  int &c = cache[dev][si][ni];
  if (c == 0) {
    int per_cu = 1, cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(pick_kernel(sb, nb)),
                                                     kThreads, 0) != hipSuccess || per_cu < 1)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    c = per_cu * cus;
  }
  return c;
}

int nb_chunk(int sb, int64_t left) {
  if (sb == 3) return 1;
  return left >= 4 ? 4 : (left >= 2 ? 2 : 1);
}

}  // namespace

namespace cq {

// Workspace of one launch: [counters: nblocks x u32, padded to 256 B][partials: nslice x nb x rows f32].
uint64_t chunk_workspace_bytes(const MvShape &s, int nb, int64_t rows) {
  if (s.nslice <= 1) return 0;
  const uint64_t counters = (static_cast<uint64_t>(s.nblocks) * 4 + 255) / 256 * 256;
  return counters + static_cast<uint64_t>(s.nslice) * nb * rows * 4;
}

uint64_t matvec_workspace_bytes(int bits, int64_t rows, int64_t kpad, int64_t batch) {
  const int sb = storage_bits(bits);
  uint64_t need = 0;
  if (rows <= 0 || kpad <= 0) return 0;  // nothing is launched
  for (int64_t b = 0; b < batch;) {
    const int nb = nb_chunk(sb, batch - b);
    const uint64_t bytes = chunk_workspace_bytes(mv_shape(sb, nb, rows, kpad), nb, rows);
    if (bytes > need) need = bytes;
    b += nb;
  }
  return need;
}

hipError_t launch_matvec(const uint8_t *blob, int bits, int64_t rows, int64_t kpad, const CodeLevels &lev,
                         const float *xr, int64_t batch, float *y, void *workspace, hipStream_t s) {
  const int sb = storage_bits(bits);
  MvArgs a;
  a.packed = blob;
  a.row_bytes = kpad * sb / 8;
  a.norms = reinterpret_cast<const uint16_t *>(blob + rows * a.row_bytes);
  a.rows = rows;
  a.kpad = kpad;
  a.ngroups = kpad / CQ_GROUP;
  a.lev = lev;
  for (int64_t b = 0; b < batch;) {
    const int nb = nb_chunk(sb, batch - b);
    const MvShape sh = mv_shape(sb, nb, rows, kpad);
    a.xr = xr + b * kpad;
    a.y = y + b * rows;
    a.nslice = sh.nslice;
    a.rows_per_block = sh.rows_per_block;
    a.nblocks = sh.nblocks;
    a.per_slice = sh.per_slice;
    if (sh.nslice > 1) {
      const uint64_t counters = (static_cast<uint64_t>(sh.nblocks) * 4 + 255) / 256 * 256;
      a.counter = static_cast<uint32_t *>(workspace);
      a.partial = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + counters);
    } else {
      a.partial = nullptr;
      a.counter = nullptr;
    }
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(sh.nslice) * sh.per_slice));
    pick_kernel(sb, nb)<<<grid, kThreads, 0, s>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    b += nb;
  }
  return hipSuccess;
}

}  // namespace cq
