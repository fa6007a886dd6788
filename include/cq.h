/*
 * cq.h -- C ABI of the Cactus Quants (CQ) matrix-product library for one
 * AMD Instinct MI355X (gfx950).
 *
 * A CQ matrix W is stored [rows = out, cols = in] in groups of 128 weights
 * along the input axis.  Each group is an fp16 L2 norm times a unit direction
 * in the normalised Walsh-Hadamard domain whose coordinates index a codebook,
 * so that for every output row
 *
 *     y[r] = sum_g norm[r][g] * < c[q[r][g]], H . x_g >            (1)
 *
 * with H the order-128 Sylvester-Hadamard matrix divided by sqrt(128).
 * Sources: the Needle ".cact" format post ("Cactus Quants", "How the kernel
 * reads it"), the needle.js tutorial "The .cact archive and Cactus Quants"
 * ("Anatomy of a CQ matrix", "Reconstructing one group") and the OpenNeedle
 * reference notes (CQ quantisation steps; rotated-activation identity).
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Pointers named "device" are HIP device pointers owned by the caller; the
 *    library never frees, keeps or allocates memory, and keeps no state.
 *  - Pointers named "host" are read during the call only.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued on
 *    it and the call returns; results are valid once the stream has reached
 *    that point.
 *  - Every argument is validated before anything is enqueued.  On an error
 *    nothing is launched and no output byte is written.  A failed HIP launch
 *    returns CQ_ERR_HIP.  Nothing aborts the process.
 *  - All arrays are dense and row-major; sizes are element counts.
 *  - Calls that share an output buffer on one stream are ordered by it; two
 *    calls on different streams writing the same buffer race.
 */
#ifndef CQ_H
#define CQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum cq_status {
  CQ_OK = 0,
  CQ_ERR_NULL = 1,      /* a required pointer is NULL                           */
  CQ_ERR_BITS = 2,      /* bits is not 1, 2, 3, 4 or 5                          */
  CQ_ERR_GROUP = 3,     /* group is not 128                                     */
  CQ_ERR_SHAPE = 4,     /* a dimension is negative or above its limit          */
  CQ_ERR_LENGTH = 5,    /* blob_bytes differs from cq_blob_bytes():
                           "Inconsistent CQ matrix length"                     */
  CQ_ERR_CODEBOOK = 6,  /* levels missing, not finite or not strictly
                           ascending; or levels given for binary or ternary    */
  CQ_ERR_DTYPE = 7,     /* unsupported element type                             */
  CQ_ERR_WORKSPACE = 8, /* workspace smaller than cq_workspace_bytes()          */
  CQ_ERR_ALIGN = 9,     /* a device pointer is not aligned as documented        */
  CQ_ERR_HIP = 10,      /* a HIP runtime call or kernel launch failed           */
  CQ_ERR_OVERLAP = 11,  /* an output buffer overlaps an input buffer            */
  CQ_ERR_SCRATCH = 12   /* the call needs more than the static scratch
                           (CQ_NOALLOC_SCRATCH_BYTES) of the no-allocation
                           entry point                                        */
} cq_status;

/* Element types of activation buffers. */
typedef enum cq_dtype { CQ_F32 = 0, CQ_F16 = 1, CQ_BF16 = 2 } cq_dtype;

/* Largest accepted dimensions (rows, cols, batch of a GEMM). */
#define CQ_MAX_DIM ((int64_t)1 << 30)
/* Largest batch of cq_matvec; larger batches are prefill: use cq_gemm. */
#define CQ_MAX_MATVEC_BATCH 8
/* The only supported quantisation group. */
#define CQ_GROUP 128
/* Most matrices in one cq_rotate_multi_matvec call. */
#define CQ_MAX_MULTI 64
/* Widest cols_pad of the matvec calls (cq_matvec, cq_rotate_matvec,
 * cq_rotate_multi_matvec, their workspace queries) and of cq_gemm: the
 * kernels address a tile of rows with 32-bit offsets.  Wider matrices are
 * refused with CQ_ERR_SHAPE before anything is launched. */
#define CQ_MAX_MATVEC_COLS ((int64_t)1 << 24)
#define CQ_MAX_GEMM_COLS ((int64_t)1 << 22)
/* Most query heads of one cq_kv_scores call; most rows of cq_matvec_t (whose
 * packed rows must also stay below 2 GiB). */
#define CQ_MAX_KV_HEADS 256
/* Most cached tokens one cq_kv_attention call attends to. */
#define CQ_MAX_KV_TOKENS 16384
#define CQ_MAX_MATVEC_T_ROWS ((int64_t)1 << 20)
/* Size of the static device scratch of cq_rotate_matvec_noalloc (16 MiB). */
#define CQ_NOALLOC_SCRATCH_BYTES ((uint64_t)16 << 20)

/*
 * A CQ matrix as the ".cact" blob stores it (needle.js tutorial, "Anatomy of a
 * CQ matrix"; OpenNeedle reference notes, file layout):
 *
 *   blob = packed index rows, then fp16 norms
 *   packed row r: cols_pad * b / 8 bytes, cols_pad = ceil(cols/128) * 128,
 *                 one continuous LSB-first bitstream: index k occupies bits
 *                 [k*b, (k+1)*b) (2-bit: four per byte, first column in the
 *                 lowest bits; 4-bit: low nibble first; 3-bit: indices cross
 *                 byte boundaries; 1-bit: eight per byte, first column in
 *                 the lowest bit)
 *   norms:        rows * (cols_pad/128) little-endian fp16, [row][group],
 *                 directly after the last packed row
 *
 * b is `bits` for 2/3/4.  bits == 5 is the ternary marker: b = 2 and each
 * 2-bit crumb sign-extends (00 -> 0, 01 -> +1, 11 -> -1; 10 -> -2, never
 * written by cq_quantize) and scales the analytic level
 * a = fp32(1.2240064 / sqrt(128)) (needle.js tutorial, "Shared codebooks").
 * bits == 1 is binary: b = 1, code 0 selects -c and code 1 selects +c with
 * the closed-form level c = fp32(sqrt(2/pi) / sqrt(128)), the mean of the
 * positive half of N(0, 1/128) (".cact" format post, "Cactus Quants": binary
 * weights pack eight per byte and their centroid is analytic; the marker and
 * the sign convention are this library's reading).
 */
typedef struct cq_matrix {
  int32_t bits;          /* 1 (binary), 2, 3, 4, or 5 (ternary marker)            */
  int32_t group;         /* must be 128                                           */
  int64_t rows;          /* output dimension, 0 <= rows <= CQ_MAX_DIM             */
  int64_t cols;          /* input dimension, 0 <= cols <= CQ_MAX_DIM              */
  const void *blob;      /* device, 16-byte aligned; NULL allowed if blob_bytes==0*/
  uint64_t blob_bytes;   /* must equal cq_blob_bytes(bits, group, rows, cols)     */
  const float *levels;   /* host: 2^bits strictly ascending finite fp32 levels,
                            already divided by sqrt(128) (the file's embedded
                            codebook); must be NULL when bits is 1 or 5          */
} cq_matrix;

/* Version of this ABI (major * 10000 + minor * 100 + patch). */
int32_t cq_version(void);

/* Static description of a status code; never NULL. */
const char *cq_status_string(cq_status status);

/*
 * Byte length of a CQ blob: rows * (cols_pad*b/8 + 2*cols_pad/128)
 * (needle.js tutorial, "Anatomy of a CQ matrix"; ternary uses b = 2, binary
 * b = 1).  Writes *bytes and returns CQ_OK, or returns an error and leaves *bytes.
 * Host-only; launches nothing.
 */
cq_status cq_blob_bytes(int32_t bits, int32_t group, int64_t rows, int64_t cols,
                        uint64_t *bytes);

/* Operations that may take a workspace. */
typedef enum cq_op {
  CQ_OP_MATVEC = 0,
  CQ_OP_GEMM = 1,
  CQ_OP_ROTATE_MATVEC = 2,
  CQ_OP_W2A8 = 3,
  CQ_OP_MATVEC_T = 4
} cq_op;

/*
 * Device workspace (bytes) that `op` needs for `W` and the given batch (M for
 * the GEMM).  Host-only.  0 means the call takes workspace = NULL.
 *
 * A workspace is device memory owned by the caller, 16-byte aligned.  Its
 * contents on entry do not matter and are left unspecified (it holds the
 * per-call partial sums of the K slices and, for CQ_OP_ROTATE_MATVEC at batch
 * 2..8, the rotated activation; for CQ_OP_W2A8 the int8 activation and its
 * group scales).  Calls that may run at the same time
 * must not share a workspace; calls on one stream may, whatever their shapes.
 */
cq_status cq_workspace_bytes(int32_t op, const cq_matrix *W, int64_t batch,
                             uint64_t *bytes);

/*
 * Rotate activations once per 128-group (the ".cact" format post, "How the
 * kernel reads it": each 128-lane group of the activation is rotated with the
 * same Hadamard transform, shared by all output rows; OpenNeedle reference
 * notes, rotated-activation identity: dot(w_hat, x) = n * dot(c[q], H x)).
 *
 *   xr[b][g*128 + j] = sum_k H[j][k] * x[b][g*128 + k],  x zero-padded
 *
 *   x      device [batch][cols] of x_dtype (CQ_F32, CQ_F16, CQ_BF16),
 *          aligned to its element size
 *   xr     device [batch][cols_pad] of xr_dtype (CQ_F32 for cq_matvec,
 *          CQ_BF16 for cq_gemm), 16-byte aligned; must not overlap x
 *   Computed in fp32 (seven butterfly stages, then one multiply by
 *   1/sqrt(128)); bf16 output is rounded to nearest even.
 *   batch, cols in [0, CQ_MAX_DIM]; nothing is launched when either is 0
 *   (then xr is untouched: it has no elements when batch or cols_pad is 0).
 */
cq_status cq_rotate_acts(const void *x, int32_t x_dtype, int64_t batch, int64_t cols,
                         void *xr, int32_t xr_dtype, void *stream);

/*
 * Decode matrix-vector product, equation (1):
 *
 *   y[b][r] = sum_g float(norm[r][g]) * sum_j c[q[r][g*128+j]] * xr[b][g*128+j]
 *
 *   W        matrix descriptor (its blob is read, never expanded);
 *            W.cols_pad <= CQ_MAX_MATVEC_COLS, else CQ_ERR_SHAPE
 *   xr       device fp32 [batch][W.cols_pad], 16-byte aligned, as written by
 *            cq_rotate_acts(..., CQ_F32, ...)
 *   batch    0 <= batch <= CQ_MAX_MATVEC_BATCH
 *   y        device fp32 [batch][W.rows], 4-byte aligned, must not overlap
 *            xr or the blob; fully overwritten (0 where cols == 0)
 *   workspace, workspace_bytes: at least cq_workspace_bytes(CQ_OP_MATVEC),
 *            see cq_workspace_bytes (NULL, 0 when that is 0); must not
 *            overlap any other buffer of the call
 *   Kernels: a matrix with cols_pad <= 4096 and at most 2^26 weights
 *   (rows * cols_pad) takes the small-matrix kernel at every batch; otherwise
 *   batch 1 from 2^23 weights takes the lookup tables, and the rest the
 *   batched matrix-core kernel.
 *   Arithmetic of the lookup tables: the inner sum is read from tables
 *   indexed by a packed field (8 codes at 1 bit, 4 codes at 2-bit widths, 2
 *   codes at 3- and 4-bit widths); an entry, the sum of its codes' level * xr products, is
 *   computed in fp32, scaled by a power of two per slice of 512-2048 columns
 *   and rounded once to fp16 (relative error <= 2^-11 per entry).  Products
 *   with the fp16 norm and all sums are fp32.
 *   Arithmetic of the matrix-core kernels (W read once for the batch; the
 *   fp16 matrix cores with two-part operands): the activation a = xr * 2^e
 *   (2^e a power of two per batch vector and slice of up to 4096 columns
 *   that puts the slice's largest |xr| in [2^14, 2^15)) is held as
 *   hi = fp16(a) plus lo = fp16(a - hi); each code's level, scaled by 2^sl
 *   (largest |level| in [2^14, 2^15)), is held the same way (binary and
 *   ternary levels are exact multiples of one level and need no low part);
 *   the products of the fp16 parts are exact in fp32, each 128-group is
 *   summed on its own in fp32 and multiplied in fp32 by float(norm) * 2^-sl
 *   (or by norm * level), and the scales are undone exactly.  Operands
 *   thus carry 22 significant bits, and no rounding is shared by all weights
 *   of one code: activations lined up with a weight row, group norms in
 *   fp16's subnormal range and rows of one group keep fp32 accuracy.
 *   Results do not depend on scheduling: partial sums (of K slices, or of
 *   the waves that share a row block) are added in a fixed order.
 */
cq_status cq_matvec(const cq_matrix *W, const float *xr, int64_t batch, float *y,
                    void *workspace, uint64_t workspace_bytes, void *stream);

/*
 * Decode product from the activation before rotation: the same result as
 * cq_rotate_acts(x, CQ_F32, ..., xr, CQ_F32) followed by cq_matvec(W, xr, ...),
 * bit for bit, in one call.  Where the product kernel allows it, each of its
 * workgroups rotates the part of x it needs (the butterfly of
 * cq_rotate_acts) and no rotated activation is written to memory: the
 * small-matrix kernel (one launch, any batch, no workspace) and the lookup
 * tables.  Otherwise the rotation runs once into the workspace, then the
 * product.
 *
 *   W, batch, y, stream: as for cq_matvec
 *   x        device fp32 [batch][W.cols], 4-byte aligned (16-byte alignment
 *            and W.cols % 8 == 0 allow vector loads), must not overlap y or
 *            the workspace; not modified
 *   workspace, workspace_bytes: at least cq_workspace_bytes(CQ_OP_ROTATE_MATVEC)
 *            (it may also hold the rotated activation)
 *   Errors as cq_matvec.
 */
cq_status cq_rotate_matvec(const cq_matrix *W, const float *x, int64_t batch, float *y,
                           void *workspace, uint64_t workspace_bytes, void *stream);

/*
 * cq_rotate_matvec without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The call allocates nothing (no hipMalloc,
 * no hipFree, no allocating library routine); its scratch is a static device
 * array of CQ_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on until the process ends.
 *
 *   W, x, batch, y, stream: as cq_rotate_matvec (same results, bit for bit)
 *   Errors: those of cq_rotate_matvec; CQ_ERR_SCRATCH when
 *   cq_workspace_bytes(CQ_OP_ROTATE_MATVEC, W, batch) exceeds
 *   CQ_NOALLOC_SCRATCH_BYTES (16 MiB covers 65536 x 16384 at batch 1..8);
 *   nothing is launched then.
 *   Every call on one GPU uses the same array and leaves its contents there;
 *   no call reads what another wrote.  Calls that run at the same time on one
 *   GPU (several streams or host threads) race on the array: serialise them.
 */
cq_status cq_rotate_matvec_noalloc(const cq_matrix *W, const float *x, int64_t batch, float *y, void *stream);

/*
 * Several decode products with one activation: for i < n,
 *
 *   y[i] = cq_rotate_matvec(W[i], x)      (same values, bit for bit)
 *
 * with the rotation of x shared by all of them (".cact" format post, "How
 * the kernel reads it": each 128-group of the activation is rotated once and
 * reused by every row that reads it; OpenNeedle reference notes: Q, K, V and
 * the gate read the same normalised activation).  Matrices that take the
 * small-matrix kernel (see cq_matvec) run in one launch per storage width
 * (up to 8 matrices a launch), each workgroup rotating x itself; the others
 * share a single rotation into the workspace and take one product each.
 *
 *   W        host array of n descriptors, all with the same cols
 *   n        0 <= n <= CQ_MAX_MULTI (0: nothing is done)
 *   x        device fp32 [batch][cols], as for cq_rotate_matvec
 *   batch    0 <= batch <= CQ_MAX_MATVEC_BATCH
 *   y        host array of n device pointers; y[i] is fp32 [batch][W[i].rows],
 *            4-byte aligned, fully overwritten; the y[i] must not overlap one
 *            another, x, any blob or the workspace (y[i] may be NULL when
 *            W[i].rows == 0)
 *   workspace, workspace_bytes: at least cq_rotate_multi_workspace_bytes(W, n,
 *            batch) (NULL, 0 when that is 0; it is 0 when every matrix takes
 *            the one-launch path)
 *   Errors: those of cq_rotate_matvec for any W[i]; CQ_ERR_SHAPE for n out of
 *   range or unequal cols.  Nothing is launched unless every check passes.
 */
cq_status cq_rotate_multi_matvec(const cq_matrix *W, int32_t n, const float *x, int64_t batch,
                                 float *const *y, void *workspace, uint64_t workspace_bytes,
                                 void *stream);

/* Workspace (bytes) of cq_rotate_multi_matvec for these matrices and batch;
   checks W, n and batch as that call does.  Host-only. */
cq_status cq_rotate_multi_workspace_bytes(const cq_matrix *W, int32_t n, int64_t batch,
                                          uint64_t *bytes);

/*
 * The activation side of CQ-W2A8 (".cact" format post, "How the kernel reads
 * it": each rotated 128-group of the activation is quantised to int8 with one
 * scale; OpenNeedle reference notes, Cactus 2-bit kernel: the scale is the
 * group's absmax / 127):
 *
 *   xr  = H . x per group, fp32 (the butterfly of cq_rotate_acts)
 *   sx[b][g]  = fp32(max |xr| over the group / 127)
 *   xq[b][k]  = clamp(round_half_even(fp32(xr / sx)), -128, 127)  (0 where sx == 0)
 *
 *   x      device fp32 [batch][cols], not rotated, 4-byte aligned (16-byte
 *          alignment and cols % 8 == 0 allow vector loads); not modified
 *   batch, cols   0 <= each <= CQ_MAX_DIM (0: nothing is done)
 *   xq     device int8 [batch][cols_pad], 16-byte aligned, column order
 *          (the padding columns hold their quantised rotated values)
 *   sx     device fp32 [batch][cols_pad / 128], 4-byte aligned
 *   Outputs fully overwritten; none may overlap x or each other
 *   (CQ_ERR_OVERLAP).  CQ_ERR_SHAPE, CQ_ERR_NULL, CQ_ERR_ALIGN, CQ_ERR_HIP.
 */
cq_status cq_quantize_acts_int8(const float *x, int64_t batch, int64_t cols, int8_t *xq, float *sx, void *stream);

/*
 * CQ-W2A8 decode product from quantised activations: int8 activations and an
 * int8 code book, integer dot products, one float multiply per group
 * (".cact" format post, "How the kernel reads it": int8 centroids are looked
 * up by the packed indices, and each group's dot is multiplied by the weight
 * norm, the activation scale and the codebook scale; OpenNeedle reference
 * notes, Cactus 2-bit kernel: the codebook scale is maxabs / 127):
 *
 *   sc  = fp32(max |level| / 127), c8 = round_half_even(fp32(level / sc));
 *         ternary: c8 = the crumb's integer (0, 1, -2, -1), sc = the level a
 *   y[b][r] = sum_g (float(norm[r][g]) * sx[b][g] * sc) * sum_j c8[q] * xq
 *
 * The integer sums are exact; the per-group products and the sum over groups
 * are fp32.  This is the pages' deployment arithmetic, not the fp32-accurate
 * product of cq_matvec: its error against that product is the int8
 * quantisation of the activation and the code book (about 1 % of |y|).
 *
 *   W        matrix descriptor
 *   xq, sx   as written by cq_quantize_acts_int8 for W.cols columns (any
 *            int8 values and finite scales are accepted); not modified
 *   batch    0 <= batch <= CQ_MAX_MATVEC_BATCH, and one workgroup holds
 *            the whole quantised activation: with P = 32 * cols_pad / 128,
 *            batch * cols_pad + P <= 61440 for batch <= 4 and cols_pad <=
 *            16384, or (batch + 1) * cols_pad + P <= 61440; e.g. cols_pad up
 *            to 27264 at batch 1, 16384 at batch 2 and 3, 14336 at batch 4,
 *            6528 at batch 8; CQ_ERR_SHAPE otherwise
 *   y        device fp32 [batch][W.rows], 4-byte aligned, must not overlap
 *            xq, sx or the blob; fully overwritten (0 where cols == 0)
 *   Errors as cq_matvec.
 */
cq_status cq_matvec_w2a8_quantized(const cq_matrix *W, const int8_t *xq, const float *sx, int64_t batch, float *y,
                                   void *stream);

/*
 * CQ-W2A8 from the fp32 activation: cq_quantize_acts_int8 into the workspace,
 * then cq_matvec_w2a8_quantized (two kernels on the stream).
 *
 *   x        device fp32 [batch][W.cols], not rotated, 4-byte aligned; not
 *            modified
 *   batch, y as cq_matvec_w2a8_quantized; y must not overlap x
 *   workspace, workspace_bytes: at least cq_workspace_bytes(CQ_OP_W2A8), not
 *            overlapping x, y or the blob
 *   Errors as cq_matvec.
 */
cq_status cq_matvec_w2a8(const cq_matrix *W, const float *x, int64_t batch, float *y, void *workspace,
                         uint64_t workspace_bytes, void *stream);

/*
 * Row gather: the dense reconstruction of the indexed rows only (needle.js
 * tutorial, "Reconstructing one group": a row gather, for embeddings and
 * engram tables, reconstructs the dense group; "Keep the quantized views":
 * dequantise only the rows you need):
 *
 *   out[i][k] = w_hat[ids[i]][k],  k < W.cols,
 *   w_hat group = (c[q] * float(norm)) . H   (fp32: the level times the
 *                 norm, the butterfly of cq_rotate_acts, H being its own inverse)
 *
 *   W          matrix descriptor
 *   ids        device int64 [n], 8-byte aligned; an id outside [0, W.rows)
 *              gives a row of NaN (nothing outside the blob is read)
 *   n          0 <= n <= CQ_MAX_DIM (0: nothing is done)
 *   out        device [n][W.cols] of out_dtype (CQ_F32, CQ_F16 or CQ_BF16,
 *              rounded to nearest even), aligned to its element size; must not
 *              overlap ids or the blob; fully overwritten
 *   Errors as cq_matvec, and CQ_ERR_DTYPE for another out_dtype.
 */
cq_status cq_gather_rows(const cq_matrix *W, const int64_t *ids, int64_t n, void *out, int32_t out_dtype,
                         void *stream);

/*
 * Prefill product on the bf16 matrix cores, fp32 accumulation:
 *
 *   C[m][r] = sum_k Xr[m][k] * V[r][k],  V[r][g*128+j] = bf16(c[q] * float(norm[r][g]))
 *
 * (the product c*norm in fp32, then rounded to nearest even bf16; the
 * dequantised tile is never written to memory).
 *
 *   W        matrix descriptor
 *   xr       device bf16 [m][W.cols_pad], 16-byte aligned, as written by
 *            cq_rotate_acts(..., CQ_BF16, ...)
 *   m        0 <= m <= CQ_MAX_DIM
 *   c        device fp32 [m][W.rows], 4-byte aligned, must not overlap xr
 *            or the blob; fully overwritten (0 where cols == 0)
 *   workspace, workspace_bytes: unused -- the product needs no scratch and
 *            cq_workspace_bytes(CQ_OP_GEMM) reports 0; pass NULL, 0 (any
 *            value is accepted and ignored)
 *   Errors as cq_matvec; CQ_ERR_SHAPE also for cols_pad > CQ_MAX_GEMM_COLS.
 */
cq_status cq_gemm(const cq_matrix *W, const void *xr, int64_t m, float *c,
                  void *workspace, uint64_t workspace_bytes, void *stream);

/*
 * Encoder (OpenNeedle reference notes, CQ quantisation steps; the porting
 * post's "cq_quantize rounds each group of 128 weights exactly as the
 * exporter does").  Per row and per 128-group w (zero-padded):
 *
 *   r = w . H                     fp32: fp32 rounding of (w . S) * sqrt(1/128)
 *                                 with w . S summed exactly and one double
 *                                 multiply (S = +-1 Sylvester matrix)
 *   n = ||r||_2                   fp32 rounding of the double norm of r
 *   u = r / max(n, 1e-12f)        IEEE fp32 division
 *   q_i = argmin_j |u_i - c_j|    ties to the smaller index (exact compare)
 *   norm = fp16(n)                round to nearest even; > 65504 -> +inf
 *   ternary (bits 5): q over (-a, 0, +a) stored as crumbs 11, 00, 01
 *   binary (bits 1): q over (-c, +c), i.e. the sign of r (0 -> code 0)
 *
 *   w          device fp32 [rows][cols], 4-byte aligned
 *   bits       1, 2, 3, 4 or 5;   group: 128
 *   levels     host, as in cq_matrix (NULL for bits 1 and 5)
 *   blob       device, 16-byte aligned, blob_bytes == cq_blob_bytes(...);
 *              fully overwritten; must not overlap w
 */
cq_status cq_quantize(const float *w, int64_t rows, int64_t cols, int32_t bits, int32_t group,
                      const float *levels, void *blob, uint64_t blob_bytes, void *stream);

/*
 * ---- CQ-quantised KV cache ------------------------------------------------
 *
 * The header's kv_bits is the precision the KV cache was post-trained for:
 * 8 (int8), else 2, 3 or 4 (".cact" format post, "Five regions"), and the CQ
 * path serves the cache at that width (".cact" format post, "How the kernel
 * reads it"; OpenNeedle reference notes: below 8 bits the cache is simulated
 * by CQ fake quantisation).  Reading taken here: a cached key or value row
 * is one token's whole KV vector (n_kv_heads * head_dim values) quantised
 * like a weight row, in 128-groups along it -- so a group can hold several
 * heads (Needle 2: four KV heads of 64, two per group) -- and the cache is a
 * CQ matrix [tokens][n_kv_heads * head_dim] of any storage width.  A sliding
 * window of W tokens is a matrix of W rows used as a ring.
 */

/*
 * Encodes n rows (fp32 [n][dst.cols], 4-byte aligned) into rows row0 ..
 * row0 + n - 1 of an existing matrix, exactly as cq_quantize would encode
 * them (rows are encoded on their own: OpenNeedle reference notes, CQ
 * quantisation steps).  The codes and fp16 norms of those rows in dst.blob
 * are overwritten; nothing else is touched.  This is the append of new
 * tokens' keys or values to a cache.
 *   dst      the matrix (rows = its capacity); its blob is written although
 *            the descriptor holds a const pointer
 *   Errors: those of cq_matvec's descriptor checks; CQ_ERR_SHAPE unless
 *   0 <= row0 and row0 + n <= dst.rows; CQ_ERR_NULL, CQ_ERR_ALIGN,
 *   CQ_ERR_OVERLAP (w inside the blob), CQ_ERR_HIP.  A norm above the fp16
 *   range is stored as +inf, as by cq_quantize.
 */
cq_status cq_quantize_rows(const float *w, int64_t n, const cq_matrix *dst, int64_t row0, void *stream);

/*
 * Attention scores against a CQ key cache K [tokens][n_kv_heads * head_dim]:
 *
 *   scores[h][t] = sum_{d < head_dim} q[h][d] * k_hat[t][kv(h) * head_dim + d]
 *
 * with kv(h) = h / (n_q_heads / n_kv_heads) (consecutive query heads share a
 * KV head; OpenNeedle reference notes, attention: two query heads map to one
 * KV head).  No 1/sqrt(head_dim) factor and no mask: those belong to the
 * attention around it.  Computed as the decode matvec (cq_rotate_matvec) of
 * K with each query head written into a zero row of K's width: the same
 * kernels and the same fp32 arithmetic, at most 8 heads per launch.
 *   q        device fp32 [n_q_heads][head_dim], 4-byte aligned
 *   n_q_heads 1 <= n_q_heads <= CQ_MAX_KV_HEADS, a multiple of n_kv_heads;
 *            n_kv_heads * head_dim == K.cols
 *   scores   device fp32 [n_q_heads][K.rows], 4-byte aligned, must not
 *            overlap q, the blob or the workspace
 *   workspace 256-byte aligned, at least cq_kv_scores_workspace_bytes(): the
 *            padded queries, then the matvec's scratch (any contents on entry)
 *   Errors: the descriptor checks of cq_matvec, CQ_ERR_SHAPE for head counts
 *   or widths that do not fit, CQ_ERR_NULL, CQ_ERR_ALIGN, CQ_ERR_WORKSPACE,
 *   CQ_ERR_OVERLAP, CQ_ERR_HIP.  K.rows == 0 does nothing.
 */
cq_status cq_kv_scores_workspace_bytes(const cq_matrix *K, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                       uint64_t *bytes);
cq_status cq_kv_scores(const cq_matrix *K, const float *q, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                       float *scores, void *workspace, uint64_t workspace_bytes, void *stream);

/*
 * Product with the transposed matrix (the value side of attention over a CQ
 * value cache: o = sum_t p_t v_hat_t):
 *
 *   out[b][k] = sum_r p[b][r] * w_hat[r][k],   k < W.cols
 *
 * By the rotated-activation identity (OpenNeedle reference notes) the
 * weighted sum is taken on the codes in the rotated domain,
 * sum_r p[b][r] * float(norm[r][g]) * c[q[r][g*128+j]], and each group is
 * rotated back once (the butterfly of cq_rotate_acts, times 1/sqrt(128)).
 * fp32 throughout: each term is fp32(float(norm) * c) times p, summed over
 * chunks of 1024 rows in a fixed order, the chunks added in order (a
 * matrix of at most 1024 rows needs no workspace).
 *   p        device fp32 [batch][W.rows], 4-byte aligned
 *   batch    0 <= batch <= CQ_MAX_MATVEC_BATCH
 *   out      device fp32 [batch][W.cols], 4-byte aligned, must not overlap
 *            p, the blob or the workspace; fully overwritten (0 where W.rows
 *            == 0)
 *   workspace, workspace_bytes: at least cq_workspace_bytes(CQ_OP_MATVEC_T)
 *            (the row chunks' partial sums; NULL, 0 when that is 0)
 *   W.rows <= CQ_MAX_MATVEC_T_ROWS with the packed rows below 2 GiB, and
 *   W.cols <= CQ_MAX_MATVEC_COLS, else CQ_ERR_SHAPE.  Other errors as
 *   cq_matvec.
 */
cq_status cq_matvec_t(const cq_matrix *W, const float *p, int64_t batch, float *out, void *workspace,
                      uint64_t workspace_bytes, void *stream);

/*
 * The append of n new tokens to a key cache K and a value cache V at once:
 * k (fp32 [n][K.cols]) into rows row0 .. row0 + n - 1 of K and v (fp32
 * [n][V.cols]) into the same rows of V, each exactly as cq_quantize_rows
 * encodes them, in one launch when K and V share the code book (same width
 * and levels; else one launch each).
 *   Errors: those of cq_quantize_rows on either cache; CQ_ERR_SHAPE when
 *   the widths differ or the rows do not fit either cache; CQ_ERR_OVERLAP
 *   when the blobs overlap each other or an input.
 */
cq_status cq_kv_append(const cq_matrix *K, const cq_matrix *V, const float *k, const float *v, int64_t n,
                       int64_t row0, void *stream);

/*
 * One decode attention step over a CQ key cache K and value cache V, both
 * [rows][n_kv_heads * head_dim] at the same width, reading their first
 * n_tokens rows (the rows filled so far; a full ring is every row):
 *
 *   out[h] = sum_{t < n_tokens} p[h][t] * v_hat[t][kv(h) * head_dim + d],
 *   p[h]   = softmax_t(scale * scores[h][t]),   d < head_dim,
 *
 * scores and kv(h) as in cq_kv_scores, no mask (OpenNeedle reference notes,
 * attention: the softmax of the scaled scores of the cached keys weighs the
 * cached values).  One launch: each query head's workgroup rotates its
 * zero-padded query once, scores every token on the codes of its group
 * (fp32 sums of level * rotated query, times the fp32 norm and scale), takes
 * the softmax in fp32 (expf; the weights' sum added in a fixed order), sums
 * the weighted levels of the value codes in the rotated domain and rotates
 * them back (the rotated-activation identity), as cq_matvec_t.
 *   q        device fp32 [n_q_heads][head_dim], 4-byte aligned
 *   head_dim divides 128 (a head lies inside one 128-group); n_q_heads a
 *            multiple of n_kv_heads, at most CQ_MAX_KV_HEADS; n_kv_heads *
 *            head_dim == K.cols == V.cols; K.rows == V.rows
 *   n_tokens 1 <= n_tokens <= min(K.rows, CQ_MAX_KV_TOKENS)
 *   scale    factor on the scores (e.g. 1/sqrt(head_dim))
 *   out      device fp32 [n_q_heads][head_dim], 4-byte aligned, must not
 *            overlap q or either blob; fully overwritten
 *   Errors: the descriptor checks of cq_matvec on K and V, CQ_ERR_SHAPE for
 *   shapes outside the above (the composed cq_kv_scores + softmax +
 *   cq_matvec_t path takes any head_dim), CQ_ERR_NULL, CQ_ERR_ALIGN,
 *   CQ_ERR_OVERLAP, CQ_ERR_HIP.  No workspace.
 */
cq_status cq_kv_attention(const cq_matrix *K, const cq_matrix *V, int64_t n_tokens, const float *q,
                          int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale, float *out,
                          void *stream);

/*
 * Measurement helper (not part of the product): reads `bytes` bytes at p once
 * with the widest loads, nt (streaming) cache hint as the products' code
 * loads have it (32 KB contiguous tiles per workgroup), and
 * writes one checksum word per thread to sink.  Its rate is the streaming-read
 * ceiling the HBM-bound products are reported against beside the published
 * peak.  sink_words / 256 workgroups are launched (at most 65535), so sink
 * must hold a multiple of 256 words; CQ_ERR_WORKSPACE when it holds fewer
 * than 256.
 */
cq_status cq_read_probe(const void *p, uint64_t bytes, uint32_t *sink, uint64_t sink_words, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CQ_H */
