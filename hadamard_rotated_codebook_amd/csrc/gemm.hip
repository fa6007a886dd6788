// Prefill product C = Xr . V^T on the bf16 matrix cores, where Xr is the
// rotated activation (bf16, from cq_rotate_acts) and V is the CQ matrix
// dequantised in the rotated domain, V[r][g*128+j] = bf16(c[q] * norm[r][g]).
// By the rotated-activation identity (OpenNeedle reference notes) this is the
// product with the dense dequantised matrix, without ever applying H to the
// weights or writing them to memory.
//
// Tiling: a 256-thread workgroup (4 waves, 2 x 2) computes a 128 x 128 tile of
// C.  The K loop steps 64 columns (half a quantisation group).  Each step
// stages the Xr tile (global -> LDS) and decodes the packed W tile to bf16
// straight into LDS (8 codes per thread per word), then every wave runs
// 2 x 4 x 4 v_mfma_f32_16x16x32_bf16 on its 64 x 64 sub-tile, fp32 accumulate.
// LDS rows are 64 bf16 (128 B); 16-byte chunks are XOR-swizzled by row so
// that the fragment reads of 16 consecutive rows fall in distinct banks.
#include "cq_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;

struct GemmArgs {
  const uint8_t *packed;
  const uint16_t *norms;  // fp16 bits [rows][ngroups]
  const uint16_t *xr;     // bf16 bits [m][kpad]
  float *c;               // [m][rows]
  int64_t m, rows, kpad, row_bytes, ngroups;
  cq::CodeLevels lev;
};

__device__ inline uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline int swz(int row, int chunk) { return chunk ^ (row & 7); }

template <int SB>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs a) {
  __shared__ uint4 As[BM * BK / 8];  // [row][chunk] 16-byte chunks
  __shared__ uint4 Vs[BN * BK / 8];
  __shared__ float lev[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
  if (tid < 16) lev[tid] = a.lev.v[tid];

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  constexpr uint32_t mask = (1u << SB) - 1u;
  for (int64_t k0 = 0; k0 < a.kpad; k0 += BK) {
    __syncthreads();
    // Stage Xr: 128 rows x 8 chunks.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + kThreads * i;
      const int row = id >> 3, ch = id & 7;
      const int64_t gm = m0 + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (gm < a.m) v = *reinterpret_cast<const uint4 *>(a.xr + gm * a.kpad + k0 + ch * 8);
      As[row * 8 + swz(row, ch)] = v;
    }
    // Decode W: 128 rows x 8 words of 8 codes.
    const int64_t g = k0 >> 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + kThreads * i;
      const int row = id >> 3, wd = id & 7;
      const int64_t gr = n0 + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (gr < a.rows) {
        const uint8_t *src = a.packed + gr * a.row_bytes + ((k0 >> 3) + wd) * SB;
        uint32_t word;
        if (SB == 2) word = *reinterpret_cast<const uint16_t *>(src);
        else if (SB == 4) word = *reinterpret_cast<const uint32_t *>(src);
        else word = src[0] | (static_cast<uint32_t>(src[1]) << 8) | (static_cast<uint32_t>(src[2]) << 16);
        const float n = static_cast<float>(__builtin_bit_cast(_Float16, a.norms[gr * a.ngroups + g]));
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = bf16_bits(lev[(word >> (e * SB)) & mask] * n);
        v = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
      }
      Vs[row * 8 + swz(row, wd)] = v;
    }
    __syncthreads();

#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      const int ch = kk * 4 + (lane >> 4);
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 64 + i * 16 + (lane & 15);
        af[i] = __builtin_bit_cast(bf16x8, As[row * 8 + swz(row, ch)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wn * 64 + j * 16 + (lane & 15);
        bfr[j] = __builtin_bit_cast(bf16x8, Vs[row * 8 + swz(row, ch)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // C fragment layout: lane l, register e -> row 4*(l/16) + e, column l%16.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + e;
        if (row < a.m && col < a.rows) a.c[row * a.rows + col] = acc[i][j][e];
      }
    }
  }
}

}  // namespace

namespace cq {

hipError_t launch_gemm(const uint8_t *blob, int bits, int64_t rows, int64_t kpad, const CodeLevels &lev,
                       const void *xr, int64_t m, float *c, hipStream_t s) {
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
  const int64_t gx = (rows + BN - 1) / BN, gy = (m + BM - 1) / BM;
  if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
  switch (sb) {
    case 2: gemm_kernel<2><<<grid, kThreads, 0, s>>>(a); break;
    case 3: gemm_kernel<3><<<grid, kThreads, 0, s>>>(a); break;
    default: gemm_kernel<4><<<grid, kThreads, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace cq
