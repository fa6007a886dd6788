// Decode matrix-vector product y = W . x for a CQ matrix (equation (1) of
// include/cq.h), computed as sum_g norm_g * <c[q_g], H x_g> on the rotated
// activation xr (OpenNeedle reference notes, rotated-activation identity; the
// ".cact" format post, "How the kernel reads it": the kernel never expands the
// stored indices and no weight is materialised).
//
// Design (HBM-bound at batch 1):
//  * One 512-thread workgroup per CU owns a block of rows and all of K.  K is
//    walked in phases; for each phase the workgroup builds lookup tables from
//    the rotated activation in LDS (128 KB) and then streams its rows' packed
//    bytes for that phase from HBM exactly once.
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
//  * Per row: the lane's partial is scaled by its group's fp16 norm, summed
//    across 16 lanes with DPP, and accumulated in registers across phases.
//  * 3-bit rows: one 8-entry table per column; the 3-bit field is extracted
//    with v_bfe (indices cross byte boundaries) and placed next to the lane
//    slot with one shift-or.
#include "cq_internal.h"

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxRowsPerWave = 32;
constexpr int kMaxRowsPerBlock = kWaves * kMaxRowsPerWave;  // 256
constexpr int kUnroll = 4;  // rows whose loads are in flight per wave

struct MvArgs {
  const uint8_t *packed;
  const uint16_t *norms;  // fp16 bits, [rows][ngroups]
  const float *xr;        // [nb][kpad]
  float *y;               // [nb][rows]
  int64_t rows, kpad, row_bytes, ngroups;
  int32_t rows_per_block;
  cq::CodeLevels lev;
};

template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over each row of 16 lanes; every lane of the row receives the sum.
__device__ inline float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

__device__ inline float half_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ inline float lds_at(const float *lds, uint32_t byte_addr) {
  return *reinterpret_cast<const float *>(reinterpret_cast<const char *>(lds) + byte_addr);
}

// Accumulate v into the lane that keeps row m: lane (16k + m%16), register m/16.
__device__ inline void keep_row(float &acc0, float &acc1, float v, int lane, int m) {
  const bool mine = (lane & 15) == (m & 15);
  acc0 += (mine && m < 16) ? v : 0.0f;
  acc1 += (mine && m >= 16) ? v : 0.0f;
}

// Final cross-row reduction and store of the per-row accumulators.
__device__ inline void store_rows(float acc0, float acc1, int lane, int wave, int64_t r0, int64_t r1,
                                  float *y) {
  acc0 += __shfl_xor(acc0, 16);
  acc0 += __shfl_xor(acc0, 32);
  acc1 += __shfl_xor(acc1, 16);
  acc1 += __shfl_xor(acc1, 32);
  if (lane < 16) {
    const int64_t ra = r0 + wave + static_cast<int64_t>(kWaves) * lane;
    const int64_t rb = r0 + wave + static_cast<int64_t>(kWaves) * (lane + 16);
    if (ra < r1) y[ra] = acc0;
    if (rb < r1) y[rb] = acc1;
  }
}

// ---------------------------------------------------------------------------
// Storage widths 2 and 4, NB batch vectors (1, 2 or 4).
template <int SB, int NB>
__global__ __launch_bounds__(kThreads) void matvec_nibble_kernel(MvArgs a) {
  __shared__ float lds[32768];  // two 64 KB table regions
  constexpr int D = 4 / NB;                  // packed dwords per lane, row and phase
  constexpr int CPB = 8 / SB;                // codes per byte
  constexpr int LANE_COLS = 4 * D * CPB;     // columns per lane and phase
  constexpr int PHASE_COLS = 64 * LANE_COLS;
  constexpr int BLOCKS = 4 * D;              // tables per lane, region and batch vector

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * a.rows_per_block;
  const int64_t r1 = min(r0 + static_cast<int64_t>(a.rows_per_block), a.rows);
  const uint32_t base_lo = static_cast<uint32_t>(lane) * 4u;
  const uint32_t base_hi = static_cast<uint32_t>(lane) * 4u + 0x10000u;

  float acc[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb][0] = acc[nb][1] = 0.0f;

  for (int64_t p0 = 0; p0 < a.kpad; p0 += PHASE_COLS) {
    __syncthreads();
    // Build this phase's tables: per lane slot, 2 regions x NB x BLOCKS tables.
    for (int t = wave; t < 2 * NB * BLOCKS; t += kWaves) {
      const int hi = t & 1, blk = t >> 1;
      const int nb = blk / BLOCKS, beta = blk - nb * BLOCKS;
      const int64_t c = p0 + static_cast<int64_t>(lane) * LANE_COLS + (SB == 2 ? 4 * beta + 2 * hi : 2 * beta + hi);
      if (c >= a.kpad) continue;
      const float *xb = a.xr + nb * a.kpad + c;
      float e[16];
      if (SB == 2) {
        const float x0 = xb[0], x1 = xb[1];
        float p[4], q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = a.lev.v[i] * x0;
          q[i] = a.lev.v[i] * x1;
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) e[v] = p[v & 3] + q[v >> 2];
      } else {
        const float x0 = xb[0];
#pragma unroll
        for (int v = 0; v < 16; ++v) e[v] = a.lev.v[v] * x0;
      }
      const uint32_t off = hi ? 0x10000u + blk * 256u + lane * 4u : blk * 4096u + lane * 4u;
      const uint32_t stride = hi ? 4096u : 256u;
#pragma unroll
      for (int v = 0; v < 16; ++v) lds[(off + v * stride) >> 2] = e[v];
    }
    __syncthreads();

    const int64_t lc0 = p0 + static_cast<int64_t>(lane) * LANE_COLS;
    const bool active = lc0 < a.kpad;
    const int64_t g = lc0 >> 7;
    const uint8_t *colp = a.packed + p0 * SB / 8 + lane * (4 * D);
    int m = 0;
    for (int64_t rb = r0 + wave; rb < r1; rb += kUnroll * kWaves, m += kUnroll) {
      // Issue the loads of kUnroll rows before any arithmetic.
      uint32_t dw[kUnroll][D];
      float n[kUnroll];
      bool ok[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t r = rb + u * kWaves;
        ok[u] = active && r < r1;
        n[u] = 0.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) dw[u][d] = 0;
        if (ok[u]) {
          const uint8_t *src = colp + r * a.row_bytes;
          if (D == 4) {
            const uint4 v = *reinterpret_cast<const uint4 *>(src);
            dw[u][0] = v.x; dw[u][1 % D] = v.y; dw[u][2 % D] = v.z; dw[u][3 % D] = v.w;
          } else if (D == 2) {
            const uint2 v = *reinterpret_cast<const uint2 *>(src);
            dw[u][0] = v.x; dw[u][1 % D] = v.y;
          } else {
            dw[u][0] = *reinterpret_cast<const uint32_t *>(src);
          }
          n[u] = half_to_float(a.norms[r * a.ngroups + g]);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float s[NB][2];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[nb][0] = s[nb][1] = 0.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const uint32_t lo = dw[u][d] & 0x0F0F0F0Fu;
          const uint32_t hi = dw[u][d] & 0xF0F0F0F0u;
#pragma unroll
          for (int jb = 0; jb < 4; ++jb) {
            const uint32_t sel = 0x0C020400u + (static_cast<uint32_t>(jb) << 8);
            const uint32_t alo = __builtin_amdgcn_perm(lo, base_lo, sel);
            const uint32_t ahi = __builtin_amdgcn_perm(hi, base_hi, sel);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              const uint32_t blk = nb * BLOCKS + 4 * d + jb;
              s[nb][jb & 1] += lds_at(lds, alo + blk * 4096u);
              s[nb][jb & 1] += lds_at(lds, ahi + blk * 256u);
            }
          }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const float v = ok[u] ? (s[nb][0] + s[nb][1]) * n[u] : 0.0f;
          keep_row(acc[nb][0], acc[nb][1], row16_sum(v), lane, m + u);
        }
      }
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) store_rows(acc[nb][0], acc[nb][1], lane, wave, r0, r1, a.y + nb * a.rows);
}

// ---------------------------------------------------------------------------
// Storage width 3, one batch vector.  A lane reads 12 bytes = 32 codes.
__device__ inline uint32_t code3(const uint32_t dw[3], int k) {
  const int bit = 3 * k;
  const int w = bit >> 5, sh = bit & 31;
  if (sh <= 29) return __builtin_amdgcn_ubfe(dw[w], sh, 3);
  return __builtin_amdgcn_alignbit(dw[w + 1], dw[w], sh) & 7u;
}

__global__ __launch_bounds__(kThreads) void matvec_b3_kernel(MvArgs a) {
  __shared__ float lds[16384];  // 64 KB: 32 columns per lane x 8 values x 64 lanes
  constexpr int LANE_COLS = 32;
  constexpr int PHASE_COLS = 64 * LANE_COLS;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * a.rows_per_block;
  const int64_t r1 = min(r0 + static_cast<int64_t>(a.rows_per_block), a.rows);
  const uint32_t base = static_cast<uint32_t>(lane) * 4u;
  float acc0 = 0.0f, acc1 = 0.0f;

  for (int64_t p0 = 0; p0 < a.kpad; p0 += PHASE_COLS) {
    __syncthreads();
    for (int cl = wave; cl < LANE_COLS; cl += kWaves) {
      const int64_t c = p0 + static_cast<int64_t>(lane) * LANE_COLS + cl;
      if (c >= a.kpad) continue;
      const float x0 = a.xr[c];
#pragma unroll
      for (int v = 0; v < 8; ++v) lds[(v * 256u + base + cl * 2048u) >> 2] = a.lev.v[v] * x0;
    }
    __syncthreads();

    const int64_t lc0 = p0 + static_cast<int64_t>(lane) * LANE_COLS;
    const bool active = lc0 < a.kpad;
    const int64_t g = lc0 >> 7;
    const uint8_t *colp = a.packed + p0 * 3 / 8 + lane * 12;
    int m = 0;
    for (int64_t rb = r0 + wave; rb < r1; rb += kUnroll * kWaves, m += kUnroll) {
      uint32_t dw[kUnroll][3];
      float n[kUnroll];
      bool ok[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t r = rb + u * kWaves;
        ok[u] = active && r < r1;
        dw[u][0] = dw[u][1] = dw[u][2] = 0;
        n[u] = 0.0f;
        if (ok[u]) {
          const uint32_t *src = reinterpret_cast<const uint32_t *>(colp + r * a.row_bytes);
          dw[u][0] = src[0];
          dw[u][1] = src[1];
          dw[u][2] = src[2];
          n[u] = half_to_float(a.norms[r * a.ngroups + g]);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          const uint32_t addr = (code3(dw[u], k) << 8) | base;
          if (k & 1)
            s1 += lds_at(lds, addr + k * 2048u);
          else
            s0 += lds_at(lds, addr + k * 2048u);
        }
        const float v = ok[u] ? (s0 + s1) * n[u] : 0.0f;
        keep_row(acc0, acc1, row16_sum(v), lane, m + u);
      }
    }
  }
  store_rows(acc0, acc1, lane, wave, r0, r1, a.y);
}

int rows_per_block(int64_t rows) {
  int64_t r = (rows + 255) / 256;        // aim at one block per CU
  r = (r + kWaves - 1) / kWaves * kWaves;
  if (r < kWaves) r = kWaves;
  if (r > kMaxRowsPerBlock) r = kMaxRowsPerBlock;
  return static_cast<int>(r);
}

}  // namespace

namespace cq {

hipError_t launch_matvec(const uint8_t *blob, int bits, int64_t rows, int64_t kpad, const CodeLevels &lev,
                         const float *xr, int64_t batch, float *y, hipStream_t s) {
  const int sb = storage_bits(bits);
  MvArgs a;
  a.packed = blob;
  a.row_bytes = kpad * sb / 8;
  a.norms = reinterpret_cast<const uint16_t *>(blob + rows * a.row_bytes);
  a.rows = rows;
  a.kpad = kpad;
  a.ngroups = kpad / CQ_GROUP;
  a.rows_per_block = rows_per_block(rows);
  a.lev = lev;
  const int64_t blocks = (rows + a.rows_per_block - 1) / a.rows_per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  for (int64_t b = 0; b < batch;) {
    a.xr = xr + b * kpad;
    a.y = y + b * rows;
    const int64_t left = batch - b;
    if (sb == 3) {
      matvec_b3_kernel<<<grid, kThreads, 0, s>>>(a);
      b += 1;
    } else if (left >= 4) {
      if (sb == 2) matvec_nibble_kernel<2, 4><<<grid, kThreads, 0, s>>>(a);
      else matvec_nibble_kernel<4, 4><<<grid, kThreads, 0, s>>>(a);
      b += 4;
    } else if (left >= 2) {
      if (sb == 2) matvec_nibble_kernel<2, 2><<<grid, kThreads, 0, s>>>(a);
      else matvec_nibble_kernel<4, 2><<<grid, kThreads, 0, s>>>(a);
      b += 2;
    } else {
      if (sb == 2) matvec_nibble_kernel<2, 1><<<grid, kThreads, 0, s>>>(a);
      else matvec_nibble_kernel<4, 1><<<grid, kThreads, 0, s>>>(a);
      b += 1;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace cq
