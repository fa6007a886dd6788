// Products with a CQ-quantised KV cache (".cact" format post, "Five regions":
// the header's kv_bits is the cache precision the model was trained for, 8
// or 2, 3, 4; "How the kernel reads it": the same path serves the KV cache).
// A cache is a CQ matrix [tokens][n_kv_heads * head_dim]: one token's whole
// key (or value) vector per row, quantised in 128-groups like a weight row,
// so a group may hold several heads.
//
// Scores: query head h against every cached key, restricted to its KV head's
// columns, is the decode matvec of the cache with the query written into a
// zero row of the cache's width (launch_kv_pad_queries, then the matvec
// kernels, up to 8 heads per launch).
//
// Values: out[b][k] = sum_r p[b][r] * w_hat[r][k], the product with the
// transposed matrix (launch_matvec_t).  By the rotated-activation identity
// (OpenNeedle reference notes) sum_r p_r w_hat[r, g] = (sum_r p_r n[r, g]
// c[q[r, g]]) . H: the kernel sums the weighted levels of the codes in the
// rotated domain and rotates each group back once with the shared butterfly.
//
// Attention step (launch_kv_attention): scores, softmax and values of one
// query head in one workgroup; a head whose width divides 128 lies inside one
// group g of both caches, so the step needs only that group's codes and norms.
#include "cq_decode.h"
#include "cq_fwht.h"
#include "cq_internal.h"

namespace {

using namespace cqdev;

__global__ __launch_bounds__(256) void kv_pad_kernel(const float *__restrict__ q, int nq, int n_kv, int head_dim,
                                                    float *__restrict__ x) {
  const int cols = n_kv * head_dim;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(nq) * cols) return;
  const int h = static_cast<int>(i / cols), c = static_cast<int>(i % cols);
  const int kvh = h / (nq / n_kv);  // consecutive query heads share a KV head
  const int d = c - kvh * head_dim;
  x[i] = (d >= 0 && d < head_dim) ? q[static_cast<int64_t>(h) * head_dim + d] : 0.0f;
}

constexpr int kTThreads = 1024;  // 128 columns of a group x 8 row phases
constexpr int kTPhases = kTThreads / CQ_GROUP;
constexpr int kTChunk = 1024;     // rows per workgroup (a cache of up to 1024 rows needs no combine)
constexpr int kTInFlight = 8;     // rows whose loads a thread has in flight
constexpr int kTMaxBatch = 8;

struct TArgs {
  const uint8_t *packed;
  const uint16_t *norms;  // fp16 bits [rows][ngroups]
  const float *p;         // [batch][rows]
  float *out;             // [batch][cols] (one chunk) or partial [nchunk][batch][cols]
  int64_t rows, cols, kpad, row_bytes, ngroups;
  int32_t batch, nchunk;
  cq::CodeLevels lev;
};

// Workgroup (group g, row chunk c): thread (phase ph, column j) adds
// p[b][r] * (float(norm[r][g]) * level(code[r][g*128+j])) over the chunk's
// rows r = c*1024 + 8i + ph, in order of i; the eight phases are added in
// order through LDS and the group's 128 sums of each batch row are rotated
// back with the register butterfly of the rotation (times 1/sqrt(128)).
template <int SB>
__global__ __launch_bounds__(kTThreads) void matvec_t_kernel(TArgs a) {
  __shared__ float lev[16];
  __shared__ float4 pch[kTChunk][2];                       // p of the chunk's rows, [row][batch]
  __shared__ float red[kTPhases][kTMaxBatch][CQ_GROUP];
  const int tid = threadIdx.x, j = tid % CQ_GROUP, ph = tid / CQ_GROUP;
  const int64_t g = blockIdx.x;
  const int chunk = blockIdx.y;
  const int64_t r0 = static_cast<int64_t>(chunk) * kTChunk;
  const int nr = static_cast<int>(a.rows - r0 < kTChunk ? a.rows - r0 : kTChunk);
  if (tid < 16) lev[tid] = a.lev.v[tid];
  for (int rl = tid; rl < kTChunk; rl += kTThreads) {
    float v[kTMaxBatch];
#pragma unroll
    for (int b = 0; b < kTMaxBatch; ++b)
      v[b] = (rl < nr && b < a.batch) ? a.p[static_cast<int64_t>(b) * a.rows + r0 + rl] : 0.0f;
    pch[rl][0] = make_float4(v[0], v[1], v[2], v[3]);
    pch[rl][1] = make_float4(v[4], v[5], v[6], v[7]);
  }
  __syncthreads();

  // the code of column j of group g: bits [SB*j, SB*j + SB) of the group's
  // bytes, read from the dword holding the first bit (and, for 3-bit codes,
  // the next one; bytes past the packed region read as zero)
  const uint32_t bit = static_cast<uint32_t>(SB * j);
  const uint32_t goff = static_cast<uint32_t>(g * (CQ_GROUP * SB / 8)) + (bit >> 5) * 4;
  const __amdgpu_buffer_rsrc_t pk = buffer_rsrc(a.packed, static_cast<uint32_t>(a.rows * a.row_bytes));
  const __amdgpu_buffer_rsrc_t nb = buffer_rsrc(a.norms, static_cast<uint32_t>(a.rows * a.ngroups * 2));
  float acc[kTMaxBatch];
#pragma unroll
  for (int b = 0; b < kTMaxBatch; ++b) acc[b] = 0.0f;
  const int steps = (nr + kTPhases - 1) / kTPhases;  // rows per thread, the last ones possibly past the chunk
  for (int i0 = 0; i0 < steps; i0 += kTInFlight) {
    uint32_t w0[kTInFlight], w1[kTInFlight];
    uint16_t nrm[kTInFlight];
#pragma unroll
    for (int u = 0; u < kTInFlight; ++u) {
      const int rl = kTPhases * (i0 + u) + ph;
      const bool live = rl < nr;
      const int64_t r = r0 + rl;
      const uint32_t off = live ? static_cast<uint32_t>(r * a.row_bytes) + goff : 0xffff0000u;
      w0[u] = __builtin_amdgcn_raw_buffer_load_b32(pk, off, 0, 0);
      w1[u] = SB == 3 ? __builtin_amdgcn_raw_buffer_load_b32(pk, off + 4, 0, 0) : 0u;
      nrm[u] = __builtin_amdgcn_raw_buffer_load_b16(
          nb, live ? static_cast<uint32_t>((r * a.ngroups + g) * 2) : 0xffff0000u, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kTInFlight; ++u) {
      const int rl = kTPhases * (i0 + u) + ph;
      const uint32_t code = static_cast<uint32_t>(
          ((static_cast<uint64_t>(w1[u]) << 32 | w0[u]) >> (bit & 31)) & ((1u << SB) - 1));
      const float w = static_cast<float>(__builtin_bit_cast(_Float16, nrm[u])) * lev[code];
      // rows past the chunk: p reads the zero padding of pch (rl < kTChunk) or
      // is skipped
      if (rl < kTChunk) {
        const float4 pa = pch[rl][0], pb = pch[rl][1];
        acc[0] = __builtin_fmaf(pa.x, w, acc[0]);
        acc[1] = __builtin_fmaf(pa.y, w, acc[1]);
        acc[2] = __builtin_fmaf(pa.z, w, acc[2]);
        acc[3] = __builtin_fmaf(pa.w, w, acc[3]);
        acc[4] = __builtin_fmaf(pb.x, w, acc[4]);
        acc[5] = __builtin_fmaf(pb.y, w, acc[5]);
        acc[6] = __builtin_fmaf(pb.z, w, acc[6]);
        acc[7] = __builtin_fmaf(pb.w, w, acc[7]);
      }
    }
  }

  // the phases in order, then the rotation back: waves 0 and 1, 16 lanes per
  // batch row, lane jj holding sums 8 jj .. 8 jj + 7
#pragma unroll
  for (int b = 0; b < kTMaxBatch; ++b) red[ph][b][j] = acc[b];
  __syncthreads();
  if (tid < 2 * 64) {
    const int b = tid >> 4, jj = tid & 15;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float s = red[0][b][8 * jj + e];
#pragma unroll
      for (int k = 1; k < kTPhases; ++k) s += red[k][b][8 * jj + e];
      v[e] = s;
    }
    fwht128_unscaled(v, jj);
    if (b < a.batch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t k = g * CQ_GROUP + 8 * jj + e;
        if (k < a.cols) a.out[(static_cast<int64_t>(chunk) * a.batch + b) * a.cols + k] = v[e] * kInvSqrt128;
      }
    }
  }
}

// ---- one decode attention step, a workgroup per query head --------------

constexpr int kAThreads = 1024;
constexpr int kASlots = kAThreads / 4;  // tokens scored at once: 4 threads per token
constexpr int kABlocks = 4;             // token blocks whose loads a thread has in flight
constexpr int kAQuads = CQ_GROUP / 4;   // value side: threads per row, 4 codes each
constexpr int kAPhases = kAThreads / kAQuads;  // row phases (32)
constexpr int kAVRows = 8;              // rows per value batch per thread

struct AArgs {
  const uint8_t *kpacked, *vpacked;
  const uint16_t *knorms, *vnorms;  // fp16 bits [rows][ngroups]
  const float *q;                   // [nq][hd]
  float *out;                       // [nq][hd]
  int64_t row_bytes, ngroups;
  int32_t tokens, nq, nkv, hd;
  float scale;
  cq::CodeLevels klev, vlev;
};

// v combined over the 64 lanes with op (every lane gets the same value: the
// lane exchanges pair each lane with one partner per step, in a fixed order).
template <typename Op>
__device__ inline float wave_all(float v, Op op) {
  v = op(v, xor_lane<1>(v));
  v = op(v, xor_lane<2>(v));
  v = op(v, xor_lane<4>(v));
  v = op(v, xor_lane<8>(v));
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return v;
}

// Query head h = blockIdx.x, KV head kv(h), columns c0 .. c0 + hd - 1 of
// group g at offset off.
//  1. x = the query written into a zero 128-vector at off, rotated (the
//     butterfly of cq_rotate_acts times 1/sqrt(128)).
//  2. scores: thread (slot, quarter qj) takes codes 32 qj .. 32 qj + 31 of
//     group g of key row t = blk * 256 + slot: sum of level(code) * x in
//     order, the four quarters added pairwise, times float(norm) and scale
//     (R25 by the rotated-activation identity).
//  3. softmax weights e_t = exp(z_t - max z) and their sum S, in LDS.
//  4. values: thread (phase ph, column j) adds e_t * (float(norm) *
//     level(code j)) over rows t = ph, ph + 8, ... in order; the phases are
//     added in order, the group is rotated back and scaled by 1/(sqrt(128) S);
//     columns off .. off + hd - 1 are the head's output (R26, R27).
template <int SB>
__global__ __launch_bounds__(kAThreads) void kv_attention_kernel(AArgs a) {
  __shared__ float z[cq::kMaxKvTokens];  // scaled scores, then their exp weights
  __shared__ float xr[CQ_GROUP];
  __shared__ float klv[16], vlv[16];
  __shared__ float wred[kAThreads / 64];
  __shared__ float vph[kAPhases][CQ_GROUP];
  __shared__ float vsum[kAThreads / CQ_GROUP][CQ_GROUP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x;
  const int c0 = (h / (a.nq / a.nkv)) * a.hd;
  const int64_t g = c0 / CQ_GROUP;
  const int off = c0 % CQ_GROUP;
  const int n = a.tokens;

  // The first key and value loads go out before anything waits: none of
  // them depends on the query.
  const __amdgpu_buffer_rsrc_t kb = buffer_rsrc(a.kpacked, static_cast<uint32_t>(n * a.row_bytes));
  const __amdgpu_buffer_rsrc_t kn = buffer_rsrc(a.knorms, static_cast<uint32_t>(n * a.ngroups * 2));
  const __amdgpu_buffer_rsrc_t vb = buffer_rsrc(a.vpacked, static_cast<uint32_t>(n * a.row_bytes));
  const __amdgpu_buffer_rsrc_t vn = buffer_rsrc(a.vnorms, static_cast<uint32_t>(n * a.ngroups * 2));
  const int qj = tid & 3, slot = tid >> 2;
  const uint32_t qoff = static_cast<uint32_t>(g * (16 * SB) + qj * (4 * SB));
  uint32_t d[kABlocks][SB];
  uint16_t nn[kABlocks];
  auto kload = [&](int b0) {
#pragma unroll
    for (int u = 0; u < kABlocks; ++u) {
      const int t = b0 + u * kASlots + slot;
      const bool live = t < n;
      load_dwords<SB>(kb, live ? static_cast<uint32_t>(t * a.row_bytes) + qoff : 0xffff0000u, d[u]);
      nn[u] = __builtin_amdgcn_raw_buffer_load_b16(
          kn, live ? static_cast<uint32_t>((t * a.ngroups + g) * 2) : 0xffff0000u, 0, 0);
    }
  };
  // value side: thread (phase vp, code quad vq) takes codes 4 vq .. 4 vq + 3
  // of rows vp, vp + 32, ..., kAVRows rows per batch
  const int vq = tid % kAQuads, vp = tid / kAQuads;
  const uint32_t vbit = static_cast<uint32_t>(4 * SB * vq);
  const uint32_t goff = static_cast<uint32_t>(g * (CQ_GROUP * SB / 8)) + (vbit >> 5) * 4;
  uint32_t w0[kAVRows], w1[kAVRows];
  uint16_t nrm[kAVRows];
  auto vload = [&](int t0) {  // rows t0, t0 + 32, ...
#pragma unroll
    for (int u = 0; u < kAVRows; ++u) {
      const int t = t0 + kAPhases * u;
      const bool live = t < n;
      const uint32_t o = live ? static_cast<uint32_t>(t * a.row_bytes) + goff : 0xffff0000u;
      w0[u] = __builtin_amdgcn_raw_buffer_load_b32(vb, o, 0, 0);
      w1[u] = SB == 3 ? __builtin_amdgcn_raw_buffer_load_b32(vb, o + 4, 0, 0) : 0u;
      nrm[u] = __builtin_amdgcn_raw_buffer_load_b16(
          vn, live ? static_cast<uint32_t>((t * a.ngroups + g) * 2) : 0xffff0000u, 0, 0);
    }
  };
  kload(0);
  vload(vp);

  if (tid < 16) {
    klv[tid] = a.klev.v[tid];
    vlv[tid] = a.vlev.v[tid];
  }
  if (wave == 0) {  // lanes 0..15 hold elements 8 jj .. 8 jj + 7; the other rows rotate zeros
    const int jj = lane & 15;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int dd = 8 * jj + e - off;
      v[e] = (lane < 16 && dd >= 0 && dd < a.hd) ? a.q[static_cast<int64_t>(h) * a.hd + dd] : 0.0f;
    }
    fwht128_unscaled(v, jj);
    if (lane < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xr[8 * jj + e] = v[e] * kInvSqrt128;
    }
  }
  __syncthreads();

  // ---- scores (blocks of 256 tokens; a block past the end is skipped by
  // the whole workgroup)
  {
    const float *xq = xr + 32 * qj;  // read in the loop (a broadcast LDS read), not held
    for (int b0 = 0; b0 < n; b0 += kABlocks * kASlots) {
      if (b0 > 0) kload(b0);
#pragma unroll
      for (int u = 0; u < kABlocks; ++u) {
        if (b0 + u * kASlots >= n) break;
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int bit = SB * i, w = bit / 32, sh = bit % 32;
          uint32_t c = d[u][w] >> sh;
          if (sh + SB > 32) c |= d[u][(w + 1) % SB] << (32 - sh);
          part = __builtin_fmaf(klv[c & ((1u << SB) - 1)], xq[i], part);
        }
        part += xor_lane<1>(part);
        part += xor_lane<2>(part);
        const int t = b0 + u * kASlots + slot;
        if (qj == 0 && t < n) z[t] = a.scale * (part * static_cast<float>(__builtin_bit_cast(_Float16, nn[u])));
      }
    }
  }
  __syncthreads();

  // ---- softmax weights
  float mx = -__builtin_inff();
  for (int t = tid; t < n; t += kAThreads) mx = fmaxf(mx, z[t]);
  mx = wave_all(mx, [](float x, float y) { return fmaxf(x, y); });
  if (lane == 0) wred[wave] = mx;
  __syncthreads();
  mx = wred[0];
#pragma unroll
  for (int w = 1; w < kAThreads / 64; ++w) mx = fmaxf(mx, wred[w]);
  __syncthreads();  // every wave has read wred
  float se = 0.0f;
  for (int t = tid; t < n; t += kAThreads) {
    const float e = expf(z[t] - mx);
    z[t] = e;
    se += e;
  }
  se = wave_all(se, [](float x, float y) { return x + y; });
  if (lane == 0) wred[wave] = se;
  __syncthreads();
  se = wred[0];
#pragma unroll
  for (int w = 1; w < kAThreads / 64; ++w) se += wred[w];

  // ---- values: thread (phase vp, quad vq) adds e_t * (float(norm) *
  // level(code)) for its 4 codes over rows vp, vp + 32, ... in order (a
  // cache of up to 256 rows is one batch, loaded at the start)
  {
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int kStep = kAPhases * kAVRows;
    for (int t0 = vp; t0 < n; t0 += kStep) {
      if (t0 != vp) vload(t0);
#pragma unroll
      for (int u = 0; u < kAVRows; ++u) {
        const int t = t0 + kAPhases * u;
        if (t < n) {
          const uint64_t bits = (static_cast<uint64_t>(w1[u]) << 32 | w0[u]) >> (vbit & 31);
          const float nv = static_cast<float>(__builtin_bit_cast(_Float16, nrm[u]));
          const float p = z[t];
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc[c] = __builtin_fmaf(p, nv * vlv[(bits >> (SB * c)) & ((1u << SB) - 1)], acc[c]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) vph[vp][4 * vq + c] = acc[c];
  }
  __syncthreads();
  {  // the phases in order, in two levels: 8 parts of 4 phases, then the parts
    const int k = tid % CQ_GROUP, part = tid / CQ_GROUP;
    float s4 = vph[4 * part][k];
#pragma unroll
    for (int i = 1; i < 4; ++i) s4 += vph[4 * part + i][k];
    vsum[part][k] = s4;
  }
  __syncthreads();
  if (wave == 0) {
    const int jj = lane & 15;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float sum = vsum[0][8 * jj + e];
#pragma unroll
      for (int k = 1; k < kAThreads / CQ_GROUP; ++k) sum += vsum[k][8 * jj + e];
      v[e] = sum;
    }
    fwht128_unscaled(v, jj);
    const float f = kInvSqrt128 / se;
    if (lane < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dd = 8 * jj + e - off;
        if (dd >= 0 && dd < a.hd) a.out[static_cast<int64_t>(h) * a.hd + dd] = v[e] * f;
      }
    }
  }
}

}  // namespace

namespace cq {

hipError_t launch_kv_pad_queries(const float *q, int nq, int n_kv, int head_dim, float *x, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(nq) * n_kv * head_dim;
  kv_pad_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), 256, 0, s>>>(q, nq, n_kv, head_dim, x);
  return hipGetLastError();
}

uint64_t matvec_t_workspace_bytes(int64_t rows, int64_t cols, int64_t batch) {
  const int64_t nchunk = (rows + kTChunk - 1) / kTChunk;
  if (nchunk <= 1 || cols <= 0 || batch <= 0) return 0;
  return static_cast<uint64_t>(nchunk) * batch * cols * 4;
}

hipError_t launch_matvec_t(const uint8_t *blob, int bits, int64_t rows, int64_t cols, int64_t kpad,
                           const CodeLevels &lev, const float *p, int64_t batch, float *out, void *workspace,
                           hipStream_t s) {
  if (batch < 1 || batch > kTMaxBatch || rows < 1 || kpad % CQ_GROUP != 0) return hipErrorInvalidValue;
  const int sb = storage_bits(bits);
  TArgs a;
  a.row_bytes = kpad * sb / 8;
  a.packed = blob;
  a.norms = reinterpret_cast<const uint16_t *>(blob + rows * a.row_bytes);
  a.p = p;
  a.rows = rows;
  a.cols = cols;
  a.kpad = kpad;
  a.ngroups = kpad / CQ_GROUP;
  a.batch = static_cast<int32_t>(batch);
  a.nchunk = static_cast<int32_t>((rows + kTChunk - 1) / kTChunk);
  a.lev = lev;
  a.out = a.nchunk > 1 ? static_cast<float *>(workspace) : out;
  // 32-bit buffer offsets over the packed region and the norms
  if (rows * a.row_bytes >= (int64_t{1} << 31) || a.nchunk > 65535) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(a.ngroups), static_cast<unsigned>(a.nchunk));
  switch (sb) {
    case 1: matvec_t_kernel<1><<<grid, kTThreads, 0, s>>>(a); break;
    case 2: matvec_t_kernel<2><<<grid, kTThreads, 0, s>>>(a); break;
    case 3: matvec_t_kernel<3><<<grid, kTThreads, 0, s>>>(a); break;
    default: matvec_t_kernel<4><<<grid, kTThreads, 0, s>>>(a); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nchunk <= 1) return e;
  return launch_combine(a.out, batch * cols, a.nchunk, out, s);
}

hipError_t launch_kv_attention(const uint8_t *kblob, const uint8_t *vblob, int bits, int64_t rows, int64_t kpad,
                               const CodeLevels &klev, const CodeLevels &vlev, int64_t tokens, const float *q,
                               int nq, int n_kv, int head_dim, float scale, float *out, hipStream_t s) {
  const int sb = storage_bits(bits);
  AArgs a;
  a.row_bytes = kpad * sb / 8;
  a.ngroups = kpad / CQ_GROUP;
  if (tokens < 1 || tokens > kMaxKvTokens || tokens > rows || nq < 1 || n_kv < 1 || nq % n_kv != 0 ||
      head_dim < 1 || CQ_GROUP % head_dim != 0 || kpad % CQ_GROUP != 0 ||
      tokens * a.row_bytes >= (int64_t{1} << 31) || tokens * a.ngroups * 2 >= (int64_t{1} << 31))
    return hipErrorInvalidValue;
  a.kpacked = kblob;
  a.vpacked = vblob;
  a.knorms = reinterpret_cast<const uint16_t *>(kblob + rows * a.row_bytes);
  a.vnorms = reinterpret_cast<const uint16_t *>(vblob + rows * a.row_bytes);
  a.q = q;
  a.out = out;
  a.tokens = static_cast<int32_t>(tokens);
  a.nq = nq;
  a.nkv = n_kv;
  a.hd = head_dim;
  a.scale = scale;
  a.klev = klev;
  a.vlev = vlev;
  const dim3 grid(static_cast<unsigned>(nq));
  switch (sb) {
    case 1: kv_attention_kernel<1><<<grid, kAThreads, 0, s>>>(a); break;
    case 2: kv_attention_kernel<2><<<grid, kAThreads, 0, s>>>(a); break;
    case 3: kv_attention_kernel<3><<<grid, kAThreads, 0, s>>>(a); break;
    default: kv_attention_kernel<4><<<grid, kAThreads, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace cq
