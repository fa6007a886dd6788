// The per-group rotation xr_g = H . x_g (H = S/sqrt(128), S Sylvester) as it
// runs on the GPU: 16 lanes own one 128-group, each lane 8 consecutive
// elements.  Stages of element distance 1, 2, 4 run inside a lane; distances
// 8..64 are lane distances 1..8 ("cact-format" post, "How the kernel reads
// it": a fast Walsh-Hadamard butterfly per group).  Every kernel that rotates
// uses this one routine, so they all produce the same fp32 values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cqdev {

constexpr float kInvSqrt128 = 0.08838834764831845f;

// v: this lane's 8 elements of the group; j: the lane's index in its 16-lane
// group.  All 64 lanes of the wave must execute it (the exchanges are
// shuffles within 16 lanes).  Returns S . x; the caller applies 1/sqrt(128).
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
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) {
    const bool upper = (j & d) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = __shfl_xor(v[i], d, 16);
      v[i] = upper ? (p - v[i]) : (v[i] + p);
    }
  }
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
