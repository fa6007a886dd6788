// Internal declarations shared by the HIP translation units of libcq.
// Not part of the public ABI (that is include/cq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cq.h"

namespace cq {

// Cache-policy operand of the buffer-load builtins with the nt (non-temporal)
// bit set.  A batch-1 product reads each packed code once per call, and a
// large matrix is gone from every cache before the next call reaches it; the
// nt hint marks such loads as streaming data for L2 and the Infinity Cache.
// Measured on the table kernel (CQ2, 65536 x 16384, batch 1): 65.2 -> 57.9 us
// per call, outputs unchanged.
constexpr int kStreamLoad = 2;
// Blob size from which the batch-1 products (table and W2A8 kernels) load
// the packed codes with kStreamLoad: half the 256 MB Infinity Cache.  A
// smaller matrix may stay in that cache from one call to the next, which nt
// loads forgo: per call at CQ2 (plain / nt), 71 MB 18.2 / 18.8 us; 143 MB
// 28.8 / 31.7 us on one matrix called again and again but 36.0 / 31.9 us on
// three matrices in turn; 285 MB 68.3 / 58.2 us on three in turn.
constexpr int64_t kStreamMinBytes = int64_t{128} << 20;

// Level selected by each *stored* code: levels[code] for 2/3/4-bit matrices;
// for the ternary marker the crumb's sign extension times a, i.e.
// {0, a, -2a, -a} for crumbs 00, 01, 10, 11.  Passed to kernels by value.
struct CodeLevels {
  float v[16];
};

// Decision thresholds of the encoder: exact midpoints of adjacent ascending
// levels (held exactly in double), and the stored code of each level index.
// The decision q = #{m : u > mid[m]} for an fp32 u equals #{m : u >= T[m]}
// with T[m] the smallest fp32 above mid[m].  With at least 3 thresholds, all
// of magnitude >= 2^-125 (so an fp32 compare with them is exact in any
// denormal mode, and a u anywhere in the subnormal range lies on the same
// side of each), and codes equal to level indices, the encoder looks the
// decision up (lut = 1): bucket b(u) = clamp(bits(fma(u, lut_scale,
// lut_bias)) - bits(1.5 * 2^23), 0, 127) (one fp32 fused multiply-add
// rounded to nearest, whose result's low bits hold round(u * lut_scale +
// off) in [2^23, 2^24); monotone in u), at most one threshold per bucket, and
// q = lut_base[b] + (u >= lut_thr[b]) (NaN for a bucket without one).
// Otherwise it counts the midpoints in double and stores code byte q of
// code_bytes (up to 4 levels) or q itself (codes are level indices).
constexpr int kLutBuckets = 128;
constexpr int32_t kLutMagicBits = 0x4b400000;  // bits of 1.5 * 2^23
struct EncodeTable {
  double mid[15];
  uint32_t code_bytes;  // byte q: the stored code of level index q (nlevels <= 4)
  int32_t code_ident;   // 1 when every code is its level index
  int32_t nlevels;
  int32_t lut;
  float lut_scale;
  float lut_bias;                  // 1.5 * 2^23 + an integer offset
  float lut_thr[kLutBuckets];      // the bucket's threshold, NaN if none
  uint8_t lut_base[kLutBuckets];   // thresholds below the bucket
};

// Storage width of one index: 2 for ternary crumbs, else bits (1 for binary).
inline int storage_bits(int bits) { return bits == 5 ? 2 : bits; }

// Code levels of the fp16 matrix-core matvec kernels.  The weight operand is
// the level of each code alone (the group norm is applied in fp32 to each
// group's sum), scaled by 1 / lscale and held as the sum of two fp16 values,
// hi = fp16(level / lscale) and lo = fp16(level / lscale - hi), so that the
// operand carries 22 significant bits.  Binary and ternary levels are
// integer multiples of one level (+-1; 0, 1, -2, -1), exact in fp16 with
// lscale = that level, and need no low part.  hi / lo hold the decode tables
// of the 16-bit values as cq_decode.h's MmaTable loads them (byte planes).
struct MmaLevels {
  uint32_t hi[8];
  uint32_t lo[8];
  float lscale;
  int32_t split;  // 1 when some low part is non-zero
};
MmaLevels mma_levels(int bits, const CodeLevels &lev);

// fp32 ternary level: a / sqrt(128) with a = 1.2240064, divided in double and
// rounded once (needle.js tutorial, "Shared codebooks").
float ternary_level_f32();

// fp32 binary level sqrt(2/pi) / sqrt(128), computed in double and rounded
// once; binary code 0 selects -c, code 1 +c.
float binary_level_f32();

// Launchers.  Arguments are already validated; sizes are non-zero unless a
// launcher documents otherwise.
hipError_t launch_rotate(const void *x, int x_dtype, int64_t batch, int64_t cols, int64_t kpad,
                         void *xr, int xr_dtype, hipStream_t s);

// Workspace the matvec needs (0 when K fits one slice): the per-slice partial
// sums, any contents on entry.
uint64_t matvec_workspace_bytes(int bits, int64_t rows, int64_t kpad, int64_t batch);

// Small matrices (see kSmallMaxWeights): launch_small_matvec; otherwise
// batch 1 from 2^23 weights up: the lookup-table kernel; otherwise the
// batched matrix-core kernel.
hipError_t launch_matvec(const uint8_t *blob, int bits, int64_t rows, int64_t kpad,
                         const CodeLevels &lev, const float *xr, int64_t batch, float *y,
                         void *workspace, hipStream_t s);

// The same product from the activation before rotation (x fp32
// [batch][cols]), results equal to launch_rotate + launch_matvec.  Small
// matrices: launch_small_matvec rotating x itself.  Batch 1 on the tables:
// the lookup-table kernel rotates its slice of x itself, with the butterfly
// of launch_rotate.  Otherwise launch_rotate into the workspace (after the
// partial sums), then the batched matrix-core kernel.
uint64_t rotate_matvec_workspace_bytes(int bits, int64_t rows, int64_t kpad, int64_t batch);
hipError_t launch_rotate_matvec(const uint8_t *blob, int bits, int64_t rows, int64_t kpad,
                                const CodeLevels &lev, const float *x, int64_t cols, int64_t batch,
                                float *y, void *workspace, hipStream_t s);

// The batched matrix-core kernel (batch 2..8 beyond the small-matrix
// kernel's limits; also batch 1 with cols_pad > 4096 under 2^23 weights).
uint64_t matvec_mma_workspace_bytes(int64_t rows, int64_t kpad, int64_t batch);
hipError_t launch_matvec_mma(const uint8_t *blob, int bits, int64_t rows, int64_t kpad,
                             const CodeLevels &lev, const float *xr, int64_t batch, float *y,
                             void *workspace, hipStream_t s);

// One matrix of a shared-activation product: its blob, width, rows, code
// levels and output y [batch][rows].
struct MultiItem {
  const uint8_t *blob;
  int bits;
  int64_t rows;
  CodeLevels lev;
  float *y;
};

// Matrices of at most this many weights (rows x cols_pad) with cols_pad <=
// 4096 take the small-matrix kernel.
#ifndef CQ_SMALL_MAX_WEIGHTS
#define CQ_SMALL_MAX_WEIGHTS (int64_t{1} << 26)
#endif
constexpr int64_t kSmallMaxWeights = CQ_SMALL_MAX_WEIGHTS;

// The small-matrix kernel, one launch per storage width for up to 8
// matrices sharing x: batch 1..8, cols_pad <= 4096.  rotate: x is the
// activation [batch][cols] and each workgroup rotates it; otherwise x is xr
// [batch][kpad] (16-byte aligned) as launch_rotate writes it.  Both give the
// same values.
bool small_matvec_fits(int64_t kpad, int64_t batch);
hipError_t launch_small_matvec(const MultiItem *items, int n, const float *x, bool rotate, int64_t cols,
                               int64_t kpad, int64_t batch, hipStream_t s);

// Products of several matrices with one activation x (fp32 [batch][cols],
// not rotated).  Small matrices go to launch_small_matvec (rotating x
// themselves); the others share one rotation into the workspace (after the
// largest partial-sum region) and take launch_matvec each.
uint64_t rotate_multi_workspace_bytes(const MultiItem *items, int n, int64_t kpad, int64_t batch);
hipError_t launch_rotate_multi_matvec(const MultiItem *items, int n, const float *x, int64_t cols, int64_t kpad,
                                      int64_t batch, void *workspace, hipStream_t s);

// The CQ-W2A8 product: int8 code book (byte c % 4 of c8[c / 4] is the int8
// value of stored code c) and its scale.
struct Int8Codebook {
  uint32_t c8[4];
  float sc;
};
// LDS of one W2A8 workgroup: (batch + 1) x cols_pad int8 activations and the
// group scales; the kernel takes at most kW2a8MaxLds.
constexpr uint64_t kW2a8MaxLds = 60 * 1024;
uint64_t w2a8_lds_bytes(int64_t kpad, int64_t batch);
bool w2a8_fits(int bits, int64_t kpad, int64_t batch);
// Quantised activations of cq_matvec_w2a8: int8 [batch][kpad] (column order)
// then, 256 bytes aligned, the scales fp32 [batch][kpad / 128].
uint64_t w2a8_workspace_bytes(int64_t kpad, int64_t batch);
hipError_t launch_quant_acts_int8(const float *x, int64_t batch, int64_t cols, int64_t kpad, int8_t *xq, float *sx,
                                  hipStream_t s);
hipError_t launch_w2a8(const uint8_t *blob, int bits, int64_t rows, int64_t kpad, const Int8Codebook &cb,
                       const int8_t *xq, const float *sx, int64_t batch, float *y, hipStream_t s);

// Row gather: out[i][k] = w_hat[ids[i]][k] (k < cols) in out_dtype; NaN rows
// for ids outside [0, rows).
hipError_t launch_gather(const uint8_t *blob, int bits, int64_t rows, int64_t cols, int64_t kpad,
                         const CodeLevels &lev, const int64_t *ids, int64_t n, void *out, int out_dtype,
                         hipStream_t s);

// y[i] = sum over s < nslice, in order, of partial[s * n + i].
hipError_t launch_combine(const float *partial, int64_t n, int nslice, float *y, hipStream_t s);

hipError_t launch_gemm(const uint8_t *blob, int bits, int64_t rows, int64_t kpad,
                       const CodeLevels &lev, const void *xr, int64_t m, float *c, hipStream_t s);

// Encoding job: rows x cols of w into the codes at packed (rows of kpad * b'
// / 8 bytes) and the fp16 norms at norms ([rows][kpad / 128]).
struct QuantizeJob {
  const float *w;
  int64_t rows, cols, kpad;
  uint8_t *packed;
  uint16_t *norms;
};
// Encodes job a, and job b if not null, in one launch with one code book.
hipError_t launch_quantize(const QuantizeJob &a, const QuantizeJob *b, const EncodeTable &tab, int bits, hipStream_t s);

// KV-cache products (csrc/kv.hip).  Query padding: x[h][c] = q[h][c - c0(h)]
// for c in the columns of query head h's KV head, 0 elsewhere (x [nq][cols]).
hipError_t launch_kv_pad_queries(const float *q, int nq, int n_kv, int head_dim, float *x, hipStream_t s);
// Transposed product out[b][k] = sum_r p[b][r] w_hat[r][k] (k < cols); the
// workspace holds the row chunks' partial sums when there is more than one.
uint64_t matvec_t_workspace_bytes(int64_t rows, int64_t cols, int64_t batch);
hipError_t launch_matvec_t(const uint8_t *blob, int bits, int64_t rows, int64_t cols, int64_t kpad,
                           const CodeLevels &lev, const float *p, int64_t batch, float *out, void *workspace,
                           hipStream_t s);

// One decode attention step (csrc/kv.hip): per query head, softmax over the
// first `tokens` rows of the scaled scores against K, then the weighted rows
// of V (both caches [rows][n_kv * head_dim] at width `bits`, head_dim
// dividing 128, tokens <= kMaxKvTokens).
constexpr int kMaxKvTokens = 16384;
hipError_t launch_kv_attention(const uint8_t *kblob, const uint8_t *vblob, int bits, int64_t rows, int64_t kpad,
                               const CodeLevels &klev, const CodeLevels &vlev, int64_t tokens, const float *q,
                               int nq, int n_kv, int head_dim, float scale, float *out, hipStream_t s);

// Fills n floats with +0.0 (a kernel, so that it can sit in a captured graph).
hipError_t launch_zero_f32(float *p, int64_t n, hipStream_t s);

}  // namespace cq
