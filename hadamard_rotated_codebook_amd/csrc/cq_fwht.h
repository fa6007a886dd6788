// The per-group rotation xr_g = H . x_g (H = S/sqrt(128), S Sylvester) as it
// runs on the GPU: 16 lanes own one 128-group, each lane 8 consecutive
// elements.  Stages of element distance 1, 2, 4 run inside a lane; distances
// 8..64 are lane distances 1..8, exchanged with DPP ("cact-format" post, "How
// the kernel reads it": a fast Walsh-Hadamard butterfly per group).  Every
// kernel that rotates activations (or rotates sums back) uses this one
// routine, so they all produce the same fp32 values; the encoder rotates
// weights in double with a butterfly of its own (quantize.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cqdev {

constexpr float kInvSqrt128 = 0.08838834764831845f;

// A lane's value moved by the DPP pattern CTRL (every lane enabled).
template <int CTRL>
__device__ inline float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// The value of lane j ^ D within each 16-lane row, through the VALU's data
// path (no LDS round trip): quad permutations for 1 and 2, the half-row
// mirror (j ^ 7) then the quad reversal (^ 3) for 4, a rotation by 8 for 8.
template <int D>
__device__ inline float xor_lane(float v) {
  if constexpr (D == 1) return dpp_f32<0xb1>(v);  // quad_perm 1,0,3,2
  else if constexpr (D == 2) return dpp_f32<0x4e>(v);  // quad_perm 2,3,0,1
  else if constexpr (D == 4) return dpp_f32<0x1b>(dpp_f32<0x141>(v));  // row_half_mirror, quad_perm 3,2,1,0
  else return dpp_f32<0x128>(v);  // row_ror:8
}

// One butterfly stage at lane distance D: the lower lane of each pair keeps
// v + p, the upper one p - v (p = the partner's value), written p + (+-v)
// so that one add serves both (negation is exact).
template <int D>
__device__ inline void lane_stage(float (&v)[8], int j) {
  const float s = (j & D) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = xor_lane<D>(v[i]) + s * v[i];
}

// v: this lane's 8 elements of the group; j: the lane's index in its 16-lane
// group (lane % 16).  All 64 lanes of the wave must execute it.  Returns
// S . x; the caller applies 1/sqrt(128).
__device__ inline void fwht128_unscaled(float (&v)[8], int j) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
      const float a = v[i], c = v[i + h];
      v[i] = a + c;
      v[i + h] = a - c;
    }
  }
  lane_stage<1>(v, j);
  lane_stage<2>(v, j);
  lane_stage<4>(v, j);
  lane_stage<8>(v, j);
}

// Largest value over the 64 lanes of the wave, in every lane (max is exact,
// so the order does not matter): DPP within 16-lane rows, then the two
// half-swaps.
__device__ inline float wave_max(float m) {
  m = fmaxf(m, dpp_f32<0xb1>(m));   // quad_perm 1,0,3,2
  m = fmaxf(m, dpp_f32<0x4e>(m));   // quad_perm 2,3,0,1
  m = fmaxf(m, dpp_f32<0x141>(m));  // row_half_mirror
  m = fmaxf(m, dpp_f32<0x128>(m));  // row_ror:8
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return m;
}

// Elements [col0, col0 + 8) of an fp32 row of `cols` values, zeros past cols.
__device__ inline void load8_f32(const float *row, int64_t col0, int64_t cols, bool vec, float (&v)[8]) {
  if (vec && col0 + 8 <= cols) {
    const float4 a = *reinterpret_cast<const float4 *>(row + col0);
    const float4 b = *reinterpret_cast<const float4 *>(row + col0 + 4);
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = col0 + i < cols ? row[col0 + i] : 0.0f;
  }
}

}  // namespace cqdev
