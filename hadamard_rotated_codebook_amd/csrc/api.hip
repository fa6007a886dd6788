// Host side of libcq: argument validation and kernel dispatch for the C ABI
// declared in include/cq.h.  Every check runs before anything is enqueued, so
// a rejected call launches nothing and writes nothing.
#include <cmath>
#include <cstring>
#include <limits>

#include "cq_internal.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
  if (!na || !nb) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

cq_status hip_status(hipError_t e) { return e == hipSuccess ? CQ_OK : CQ_ERR_HIP; }

int64_t padded(int64_t cols) { return (cols + CQ_GROUP - 1) / CQ_GROUP * CQ_GROUP; }

// Blob length rows * (cols_pad*b/8 + 2*cols_pad/128) (needle.js tutorial,
// "Anatomy of a CQ matrix"; the ternary marker stores 2-bit crumbs, binary
// one bit per weight).
cq_status blob_bytes_impl(int32_t bits, int32_t group, int64_t rows, int64_t cols, uint64_t *out) {
  if (bits < 1 || bits > 5) return CQ_ERR_BITS;
  if (group != CQ_GROUP) return CQ_ERR_GROUP;
  if (rows < 0 || cols < 0 || rows > CQ_MAX_DIM || cols > CQ_MAX_DIM) return CQ_ERR_SHAPE;
  const uint64_t kpad = static_cast<uint64_t>(padded(cols));
  const uint64_t row_bytes = kpad * cq::storage_bits(bits) / 8 + kpad / CQ_GROUP * 2;
  *out = static_cast<uint64_t>(rows) * row_bytes;  // < 2^61 within the limits
  return CQ_OK;
}

// Levels of the stored codes; see cq::CodeLevels.
cq_status code_levels(int bits, const float *levels, cq::CodeLevels *lev) {
  std::memset(lev, 0, sizeof *lev);
  if (bits == 5) {
    if (levels) return CQ_ERR_CODEBOOK;
    const float a = cq::ternary_level_f32();
    lev->v[0] = 0.0f;
    lev->v[1] = a;
    lev->v[2] = -2.0f * a;
    lev->v[3] = -a;
    return CQ_OK;
  }
  if (bits == 1) {  // code 0 -> -c, code 1 -> +c
    if (levels) return CQ_ERR_CODEBOOK;
    const float c = cq::binary_level_f32();
    lev->v[0] = -c;
    lev->v[1] = c;
    return CQ_OK;
  }
  if (!levels) return CQ_ERR_CODEBOOK;
  const int n = 1 << bits;
  for (int i = 0; i < n; ++i) {
    if (!std::isfinite(levels[i])) return CQ_ERR_CODEBOOK;
    if (i && !(levels[i] > levels[i - 1])) return CQ_ERR_CODEBOOK;
    lev->v[i] = levels[i];
  }
  return CQ_OK;
}

cq_status check_matrix(const cq_matrix *W, cq::CodeLevels *lev) {
  if (!W) return CQ_ERR_NULL;
  uint64_t need = 0;
  cq_status st = blob_bytes_impl(W->bits, W->group, W->rows, W->cols, &need);
  if (st != CQ_OK) return st;
  if (W->blob_bytes != need) return CQ_ERR_LENGTH;
  if (need && !W->blob) return CQ_ERR_NULL;
  if (W->blob && !aligned(W->blob, 16)) return CQ_ERR_ALIGN;
  return code_levels(W->bits, W->levels, lev);
}

// Decision table of the encoder: exact midpoints of adjacent ascending
// levels.  For fp32 levels whose magnitudes are within 2^29 of each other the
// double sum is exact, so "u > mid" is the exact "nearer to the upper level"
// test and a tie keeps the smaller index (OpenNeedle reference notes, CQ
// quantisation steps).  levels are valid (code_levels accepted them).
// The bucket lookup of the encoder's decision (cq::EncodeTable): fp32
// thresholds, a scale and bias that spread them over the buckets, and a
// check that no bucket holds two of them.  The bucket map is evaluated here
// with the same fp32 operation as in the kernel (one fused multiply-add,
// correctly rounded on both sides, then integer clamps of its bit pattern);
// it is monotone in u, so a u in bucket b lies above every threshold of a
// lower bucket and below every one of a higher.  Only for code books whose
// codes are their level indices; up to two midpoints are counted instead.
void build_decision_lut(cq::EncodeTable &tab, bool codes_are_indices) {
  tab.lut = 0;
  const int nt = tab.nlevels - 1;
  if (nt < 3 || !codes_are_indices) return;
  float thr[15];
  for (int m = 0; m < nt; ++m) {
    float f = static_cast<float>(tab.mid[m]);
    if (!(static_cast<double>(f) > tab.mid[m])) f = std::nextafter(f, std::numeric_limits<float>::infinity());
    // finite and clear of the subnormal range (a tiny threshold: the kernel's
    // u may then be off by a subnormal step where it matters)
    if (!std::isfinite(f) || !(std::fabs(f) >= 0x1p-125f)) return;
    thr[m] = f;
  }
  const double span = static_cast<double>(thr[nt - 1]) - static_cast<double>(thr[0]);
  const float scale = span > 0.0 ? static_cast<float>((cq::kLutBuckets - 4) / span) : 1.0f;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return;
  // the lowest threshold near bucket 2
  const double lo = std::floor(static_cast<double>(thr[0]) * static_cast<double>(scale));
  if (!(std::fabs(lo) < 1e6)) return;
  const float bias = static_cast<float>(0x1.8p23 + (2.0 - lo));  // exact: an integer below 2^24
  auto bucket = [&](float u) {
    const float y = std::fmaf(u, scale, bias);
    int32_t yb;
    std::memcpy(&yb, &y, sizeof yb);
    const int32_t b = std::min(std::max(yb, cq::kLutMagicBits), cq::kLutMagicBits + cq::kLutBuckets - 1);
    return static_cast<int>(b - cq::kLutMagicBits);
  };
  int bm[15];
  for (int m = 0; m < nt; ++m) {
    bm[m] = bucket(thr[m]);
    if (m > 0 && bm[m] <= bm[m - 1]) return;  // two thresholds in one bucket
  }
  for (int b = 0; b < cq::kLutBuckets; ++b) {
    int below = 0;
    float t = std::numeric_limits<float>::quiet_NaN();
    for (int m = 0; m < nt; ++m) {
      if (bm[m] < b) ++below;
      if (bm[m] == b) t = thr[m];
    }
    tab.lut_base[b] = static_cast<uint8_t>(below);
    tab.lut_thr[b] = t;
  }
  tab.lut_scale = scale;
  tab.lut_bias = bias;
  tab.lut = 1;
}

cq::EncodeTable encode_table(int32_t bits, const float *levels) {
  cq::EncodeTable tab;
  std::memset(&tab, 0, sizeof tab);
  uint32_t code_of_index[16] = {};
  if (bits == 5) {
    const double a = static_cast<double>(cq::ternary_level_f32());
    tab.nlevels = 3;
    tab.mid[0] = -a * 0.5;
    tab.mid[1] = a * 0.5;
    code_of_index[0] = 3;  // -a -> crumb 11
    code_of_index[1] = 0;  //  0 -> crumb 00
    code_of_index[2] = 1;  // +a -> crumb 01
  } else if (bits == 1) {
    tab.nlevels = 2;
    tab.mid[0] = 0.0;  // the midpoint of -c and +c
    code_of_index[0] = 0;
    code_of_index[1] = 1;
  } else {
    tab.nlevels = 1 << bits;
    for (int j = 0; j + 1 < tab.nlevels; ++j)
      tab.mid[j] = (static_cast<double>(levels[j]) + static_cast<double>(levels[j + 1])) * 0.5;
    for (int j = 0; j < tab.nlevels; ++j) code_of_index[j] = static_cast<uint32_t>(j);
  }
  bool ident = true;
  for (int j = 0; j < tab.nlevels; ++j) {
    ident = ident && code_of_index[j] == static_cast<uint32_t>(j);
    if (j < 4) tab.code_bytes |= code_of_index[j] << (8 * j);
  }
  tab.code_ident = ident ? 1 : 0;
  build_decision_lut(tab, ident);
  return tab;
}

size_t dtype_size(int32_t dt) { return dt == CQ_F32 ? 4 : 2; }

// Sizes of cq_matvec_t: its kernel addresses the packed rows with 32-bit
// offsets.
bool matvec_t_shape_ok(const cq_matrix *W) {
  if (W->rows > CQ_MAX_MATVEC_T_ROWS || W->cols > CQ_MAX_MATVEC_COLS) return false;
  const int64_t row_bytes = padded(W->cols) * cq::storage_bits(W->bits) / 8;
  return W->rows * row_bytes < (int64_t{1} << 31);
}

// The matvec kernels' 32-bit tile offsets bound cols_pad.
cq_status check_matvec_cols(const cq_matrix *W) {
  return padded(W->cols) > CQ_MAX_MATVEC_COLS ? CQ_ERR_SHAPE : CQ_OK;
}

}  // namespace

namespace cq {

float ternary_level_f32() { return static_cast<float>(1.2240064 / std::sqrt(128.0)); }

// sqrt(2/pi) / sqrt(128), the mean of the positive half of N(0, 1/128),
// rounded once to fp32.
float binary_level_f32() { return static_cast<float>(std::sqrt(2.0 / 3.14159265358979323846) / std::sqrt(128.0)); }

}  // namespace cq

extern "C" {

int32_t cq_version(void) { return 10000; }

const char *cq_status_string(cq_status status) {
  switch (status) {
    case CQ_OK: return "ok";
    case CQ_ERR_NULL: return "a required pointer is NULL";
    case CQ_ERR_BITS: return "bits must be 1 (binary), 2, 3, 4 or 5 (ternary marker)";
    case CQ_ERR_GROUP: return "group must be 128";
    case CQ_ERR_SHAPE: return "a dimension is negative or above its limit";
    case CQ_ERR_LENGTH: return "Inconsistent CQ matrix length";
    case CQ_ERR_CODEBOOK: return "levels must be 2^bits strictly ascending finite floats (NULL for binary and ternary)";
    case CQ_ERR_DTYPE: return "unsupported element type";
    case CQ_ERR_WORKSPACE: return "workspace smaller than cq_workspace_bytes()";
    case CQ_ERR_ALIGN: return "a device pointer is not aligned as documented";
    case CQ_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case CQ_ERR_OVERLAP: return "an output buffer overlaps an input buffer";
    case CQ_ERR_SCRATCH: return "the call needs more than the static scratch of the no-allocation entry point";
  }
  return "unknown status";
}

cq_status cq_blob_bytes(int32_t bits, int32_t group, int64_t rows, int64_t cols, uint64_t *bytes) {
  if (!bytes) return CQ_ERR_NULL;
  uint64_t n = 0;
  cq_status st = blob_bytes_impl(bits, group, rows, cols, &n);
  if (st == CQ_OK) *bytes = n;
  return st;
}

cq_status cq_workspace_bytes(int32_t op, const cq_matrix *W, int64_t batch, uint64_t *bytes) {
  if (!bytes) return CQ_ERR_NULL;
  cq::CodeLevels lev;
  cq_status st = check_matrix(W, &lev);
  if (st != CQ_OK) return st;
  if (op == CQ_OP_MATVEC) {
    if (batch < 0 || batch > CQ_MAX_MATVEC_BATCH || check_matvec_cols(W) != CQ_OK) return CQ_ERR_SHAPE;
    *bytes = W->rows ? cq::matvec_workspace_bytes(W->bits, W->rows, padded(W->cols), batch) : 0;
  } else if (op == CQ_OP_ROTATE_MATVEC) {
    if (batch < 0 || batch > CQ_MAX_MATVEC_BATCH || check_matvec_cols(W) != CQ_OK) return CQ_ERR_SHAPE;
    *bytes = W->rows ? cq::rotate_matvec_workspace_bytes(W->bits, W->rows, padded(W->cols), batch) : 0;
  } else if (op == CQ_OP_MATVEC_T) {
    if (batch < 0 || batch > CQ_MAX_MATVEC_BATCH || !matvec_t_shape_ok(W)) return CQ_ERR_SHAPE;
    *bytes = W->rows && W->cols && batch ? cq::matvec_t_workspace_bytes(W->rows, W->cols, batch) : 0;
  } else if (op == CQ_OP_GEMM) {
    if (batch < 0 || batch > CQ_MAX_DIM || padded(W->cols) > CQ_MAX_GEMM_COLS) return CQ_ERR_SHAPE;
    *bytes = 0;
  } else if (op == CQ_OP_W2A8) {
    if (batch < 0 || batch > CQ_MAX_MATVEC_BATCH) return CQ_ERR_SHAPE;
    const int64_t kpad = padded(W->cols);
    if (kpad > 0 && batch > 0 && !cq::w2a8_fits(W->bits, kpad, batch)) return CQ_ERR_SHAPE;
    *bytes = W->rows && kpad && batch ? cq::w2a8_workspace_bytes(kpad, batch) : 0;
  } else {
    return CQ_ERR_SHAPE;
  }
  return CQ_OK;
}

cq_status cq_rotate_acts(const void *x, int32_t x_dtype, int64_t batch, int64_t cols, void *xr,
                         int32_t xr_dtype, void *stream) {
  if (x_dtype != CQ_F32 && x_dtype != CQ_F16 && x_dtype != CQ_BF16) return CQ_ERR_DTYPE;
  if (xr_dtype != CQ_F32 && xr_dtype != CQ_BF16) return CQ_ERR_DTYPE;
  if (batch < 0 || cols < 0 || batch > CQ_MAX_DIM || cols > CQ_MAX_DIM) return CQ_ERR_SHAPE;
  if (batch == 0 || cols == 0) return CQ_OK;
  if (!x || !xr) return CQ_ERR_NULL;
  if (!aligned(x, dtype_size(x_dtype)) || !aligned(xr, 16)) return CQ_ERR_ALIGN;
  const int64_t kpad = padded(cols);
  if (overlaps(x, static_cast<uint64_t>(batch) * cols * dtype_size(x_dtype), xr,
               static_cast<uint64_t>(batch) * kpad * dtype_size(xr_dtype)))
    return CQ_ERR_OVERLAP;
  return hip_status(cq::launch_rotate(x, x_dtype, batch, cols, kpad, xr, xr_dtype,
                                      static_cast<hipStream_t>(stream)));
}

cq_status cq_matvec(const cq_matrix *W, const float *xr, int64_t batch, float *y, void *workspace,
                    uint64_t workspace_bytes, void *stream) {
  cq::CodeLevels lev;
  cq_status st = check_matrix(W, &lev);
  if (st != CQ_OK) return st;
  if (batch < 0 || batch > CQ_MAX_MATVEC_BATCH) return CQ_ERR_SHAPE;
  if ((st = check_matvec_cols(W)) != CQ_OK) return st;
  if (batch == 0 || W->rows == 0) return CQ_OK;
  if (!y) return CQ_ERR_NULL;
  if (!aligned(y, 4)) return CQ_ERR_ALIGN;
  const uint64_t ybytes = static_cast<uint64_t>(batch) * W->rows * 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t kpad = padded(W->cols);
  if (kpad == 0) return hip_status(cq::launch_zero_f32(y, batch * W->rows, s));
  if (!xr) return CQ_ERR_NULL;
  if (!aligned(xr, 16)) return CQ_ERR_ALIGN;
  const uint64_t need = cq::matvec_workspace_bytes(W->bits, W->rows, kpad, batch);
  if (need) {
    if (!workspace || workspace_bytes < need) return CQ_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return CQ_ERR_ALIGN;
  }
  const uint64_t xbytes = static_cast<uint64_t>(batch) * kpad * 4;
  if (overlaps(y, ybytes, xr, xbytes) || overlaps(y, ybytes, W->blob, W->blob_bytes) ||
      overlaps(workspace, need, y, ybytes) || overlaps(workspace, need, xr, xbytes) ||
      overlaps(workspace, need, W->blob, W->blob_bytes))
    return CQ_ERR_OVERLAP;
  return hip_status(cq::launch_matvec(static_cast<const uint8_t *>(W->blob), W->bits, W->rows, kpad,
                                      lev, xr, batch, y, need ? workspace : nullptr, s));
}

cq_status cq_rotate_matvec(const cq_matrix *W, const float *x, int64_t batch, float *y, void *workspace,
                           uint64_t workspace_bytes, void *stream) {
  cq::CodeLevels lev;
  cq_status st = check_matrix(W, &lev);
  if (st != CQ_OK) return st;
  if (batch < 0 || batch > CQ_MAX_MATVEC_BATCH) return CQ_ERR_SHAPE;
  if ((st = check_matvec_cols(W)) != CQ_OK) return st;
  if (batch == 0 || W->rows == 0) return CQ_OK;
  if (!y) return CQ_ERR_NULL;
  if (!aligned(y, 4)) return CQ_ERR_ALIGN;
  const uint64_t ybytes = static_cast<uint64_t>(batch) * W->rows * 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t kpad = padded(W->cols);
  if (kpad == 0) return hip_status(cq::launch_zero_f32(y, batch * W->rows, s));
  if (!x) return CQ_ERR_NULL;
  if (!aligned(x, 4)) return CQ_ERR_ALIGN;
  const uint64_t need = cq::rotate_matvec_workspace_bytes(W->bits, W->rows, kpad, batch);
  if (need) {
    if (!workspace || workspace_bytes < need) return CQ_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return CQ_ERR_ALIGN;
  }
  const uint64_t xbytes = static_cast<uint64_t>(batch) * W->cols * 4;
  if (overlaps(y, ybytes, x, xbytes) || overlaps(y, ybytes, W->blob, W->blob_bytes) ||
      overlaps(workspace, need, y, ybytes) || overlaps(workspace, need, x, xbytes) ||
      overlaps(workspace, need, W->blob, W->blob_bytes))
    return CQ_ERR_OVERLAP;
  return hip_status(cq::launch_rotate_matvec(static_cast<const uint8_t *>(W->blob), W->bits, W->rows, kpad, lev,
                                             x, W->cols, batch, y, need ? workspace : nullptr, s));
}

}  // extern "C"

namespace {

// Checks the matrices of a shared-activation call and fills items (y left
// NULL); returns the common cols_pad through *kpad.
cq_status check_multi(const cq_matrix *W, int32_t n, int64_t batch, cq::MultiItem *items, int64_t *kpad) {
  if (n < 0 || n > CQ_MAX_MULTI) return CQ_ERR_SHAPE;
  if (batch < 0 || batch > CQ_MAX_MATVEC_BATCH) return CQ_ERR_SHAPE;
  if (n > 0 && !W) return CQ_ERR_NULL;
  for (int i = 0; i < n; ++i) {
    cq_status st = check_matrix(&W[i], &items[i].lev);
    if (st != CQ_OK) return st;
    if (W[i].cols != W[0].cols || check_matvec_cols(&W[i]) != CQ_OK) return CQ_ERR_SHAPE;
    items[i].blob = static_cast<const uint8_t *>(W[i].blob);
    items[i].bits = W[i].bits;
    items[i].rows = W[i].rows;
    items[i].y = nullptr;
  }
  *kpad = n > 0 ? padded(W[0].cols) : 0;
  return CQ_OK;
}

}  // namespace

extern "C" {

cq_status cq_rotate_multi_workspace_bytes(const cq_matrix *W, int32_t n, int64_t batch, uint64_t *bytes) {
  if (!bytes) return CQ_ERR_NULL;
  cq::MultiItem items[CQ_MAX_MULTI];
  int64_t kpad = 0;
  cq_status st = check_multi(W, n, batch, items, &kpad);
  if (st != CQ_OK) return st;
  *bytes = cq::rotate_multi_workspace_bytes(items, n, kpad, batch);
  return CQ_OK;
}

cq_status cq_rotate_multi_matvec(const cq_matrix *W, int32_t n, const float *x, int64_t batch, float *const *y,
                                 void *workspace, uint64_t workspace_bytes, void *stream) {
  cq::MultiItem items[CQ_MAX_MULTI];
  int64_t kpad = 0;
  cq_status st = check_multi(W, n, batch, items, &kpad);
  if (st != CQ_OK) return st;
  if (n == 0 || batch == 0) return CQ_OK;
  if (!y) return CQ_ERR_NULL;
  for (int i = 0; i < n; ++i) {
    if (W[i].rows == 0) continue;
    if (!y[i]) return CQ_ERR_NULL;
    if (!aligned(y[i], 4)) return CQ_ERR_ALIGN;
    items[i].y = y[i];
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kpad == 0) {
    for (int i = 0; i < n; ++i) {
      if (W[i].rows == 0) continue;
      const hipError_t e = cq::launch_zero_f32(y[i], batch * W[i].rows, s);
      if (e != hipSuccess) return CQ_ERR_HIP;
    }
    return CQ_OK;
  }
  if (!x) return CQ_ERR_NULL;
  if (!aligned(x, 4)) return CQ_ERR_ALIGN;
  const uint64_t need = cq::rotate_multi_workspace_bytes(items, n, kpad, batch);
  if (need) {
    if (!workspace || workspace_bytes < need) return CQ_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return CQ_ERR_ALIGN;
  }
  const uint64_t xbytes = static_cast<uint64_t>(batch) * W[0].cols * 4;
  if (overlaps(workspace, need, x, xbytes)) return CQ_ERR_OVERLAP;
  for (int i = 0; i < n; ++i) {
    if (overlaps(workspace, need, W[i].blob, W[i].blob_bytes)) return CQ_ERR_OVERLAP;
    if (W[i].rows == 0) continue;
    const uint64_t yb = static_cast<uint64_t>(batch) * W[i].rows * 4;
    if (overlaps(y[i], yb, x, xbytes) || overlaps(y[i], yb, workspace, need)) return CQ_ERR_OVERLAP;
    for (int j = 0; j < n; ++j) {
      if (overlaps(y[i], yb, W[j].blob, W[j].blob_bytes)) return CQ_ERR_OVERLAP;
      if (j != i && W[j].rows && overlaps(y[i], yb, y[j], static_cast<uint64_t>(batch) * W[j].rows * 4))
        return CQ_ERR_OVERLAP;
    }
  }
  return hip_status(cq::launch_rotate_multi_matvec(items, n, x, W[0].cols, kpad, batch,
                                                   need ? workspace : nullptr, s));
}

// The int8 code book of W: maxabs / 127 and round half to even, in fp32 (the
// ternary crumbs keep their sign-extended integers, scale a).
static cq::Int8Codebook int8_codebook(const cq_matrix *W, const cq::CodeLevels &lev) {
  cq::Int8Codebook cb;
  std::memset(&cb, 0, sizeof cb);
  const int nlev = W->bits == 5 ? 4 : 1 << W->bits;
  int8_t c8[16] = {0};
  if (W->bits == 5) {
    c8[0] = 0, c8[1] = 1, c8[2] = -2, c8[3] = -1;
    cb.sc = cq::ternary_level_f32();
  } else {
    float mx = 0.0f;
    for (int i = 0; i < nlev; ++i) mx = std::fmax(mx, std::fabs(lev.v[i]));
    cb.sc = mx / 127.0f;
    for (int i = 0; i < nlev; ++i) c8[i] = static_cast<int8_t>(std::nearbyint(lev.v[i] / cb.sc));
  }
  for (int i = 0; i < 16; ++i) cb.c8[i / 4] |= static_cast<uint32_t>(static_cast<uint8_t>(c8[i])) << (8 * (i % 4));
  return cb;
}

cq_status cq_quantize_acts_int8(const float *x, int64_t batch, int64_t cols, int8_t *xq, float *sx, void *stream) {
  if (batch < 0 || cols < 0 || batch > CQ_MAX_DIM || cols > CQ_MAX_DIM) return CQ_ERR_SHAPE;
  if (batch == 0 || cols == 0) return CQ_OK;
  if (!x || !xq || !sx) return CQ_ERR_NULL;
  if (!aligned(x, 4) || !aligned(xq, 16) || !aligned(sx, 4)) return CQ_ERR_ALIGN;
  const int64_t kpad = padded(cols);
  const uint64_t xbytes = static_cast<uint64_t>(batch) * cols * 4;
  const uint64_t qbytes = static_cast<uint64_t>(batch) * kpad;
  const uint64_t sbytes = static_cast<uint64_t>(batch) * (kpad / CQ_GROUP) * 4;
  if (overlaps(xq, qbytes, x, xbytes) || overlaps(sx, sbytes, x, xbytes) || overlaps(xq, qbytes, sx, sbytes))
    return CQ_ERR_OVERLAP;
  return hip_status(cq::launch_quant_acts_int8(x, batch, cols, kpad, xq, sx, static_cast<hipStream_t>(stream)));
}

// Checks shared by the two W2A8 products; CQ_OK with *done set when there is
// nothing to launch (or only the zero fill of y).
static cq_status check_w2a8(const cq_matrix *W, int64_t batch, float *y, cq::CodeLevels *lev, int64_t *kpad,
                            bool *done, hipStream_t s) {
  *done = true;
  cq_status st = check_matrix(W, lev);
  if (st != CQ_OK) return st;
  if (batch < 0 || batch > CQ_MAX_MATVEC_BATCH) return CQ_ERR_SHAPE;
  if ((st = check_matvec_cols(W)) != CQ_OK) return st;
  if (batch == 0 || W->rows == 0) return CQ_OK;
  *kpad = padded(W->cols);
  if (*kpad > 0 && !cq::w2a8_fits(W->bits, *kpad, batch)) return CQ_ERR_SHAPE;
  if (!y) return CQ_ERR_NULL;
  if (!aligned(y, 4)) return CQ_ERR_ALIGN;
  if (overlaps(y, static_cast<uint64_t>(batch) * W->rows * 4, W->blob, W->blob_bytes)) return CQ_ERR_OVERLAP;
  if (*kpad == 0) return hip_status(cq::launch_zero_f32(y, batch * W->rows, s));
  *done = false;
  return CQ_OK;
}

cq_status cq_matvec_w2a8_quantized(const cq_matrix *W, const int8_t *xq, const float *sx, int64_t batch, float *y,
                                   void *stream) {
  cq::CodeLevels lev;
  int64_t kpad = 0;
  bool done = true;
  hipStream_t s = static_cast<hipStream_t>(stream);
  cq_status st = check_w2a8(W, batch, y, &lev, &kpad, &done, s);
  if (st != CQ_OK || done) return st;
  if (!xq || !sx) return CQ_ERR_NULL;
  if (!aligned(xq, 16) || !aligned(sx, 4)) return CQ_ERR_ALIGN;
  const uint64_t ybytes = static_cast<uint64_t>(batch) * W->rows * 4;
  if (overlaps(y, ybytes, xq, static_cast<uint64_t>(batch) * kpad) ||
      overlaps(y, ybytes, sx, static_cast<uint64_t>(batch) * (kpad / CQ_GROUP) * 4))
    return CQ_ERR_OVERLAP;
  return hip_status(cq::launch_w2a8(static_cast<const uint8_t *>(W->blob), W->bits, W->rows, kpad,
                                    int8_codebook(W, lev), xq, sx, batch, y, s));
}

cq_status cq_matvec_w2a8(const cq_matrix *W, const float *x, int64_t batch, float *y, void *workspace,
                         uint64_t workspace_bytes, void *stream) {
  cq::CodeLevels lev;
  int64_t kpad = 0;
  bool done = true;
  hipStream_t s = static_cast<hipStream_t>(stream);
  cq_status st = check_w2a8(W, batch, y, &lev, &kpad, &done, s);
  if (st != CQ_OK || done) return st;
  if (!x) return CQ_ERR_NULL;
  if (!aligned(x, 4)) return CQ_ERR_ALIGN;
  const uint64_t need = cq::w2a8_workspace_bytes(kpad, batch);
  if (!workspace || workspace_bytes < need) return CQ_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return CQ_ERR_ALIGN;
  const uint64_t ybytes = static_cast<uint64_t>(batch) * W->rows * 4;
  const uint64_t xbytes = static_cast<uint64_t>(batch) * W->cols * 4;
  if (overlaps(y, ybytes, x, xbytes) || overlaps(workspace, need, y, ybytes) ||
      overlaps(workspace, need, x, xbytes) || overlaps(workspace, need, W->blob, W->blob_bytes))
    return CQ_ERR_OVERLAP;
  int8_t *xq = static_cast<int8_t *>(workspace);
  float *sx = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + (need - static_cast<uint64_t>(batch) *
                                                                                        (kpad / CQ_GROUP) * 4));
  hipError_t e = cq::launch_quant_acts_int8(x, batch, W->cols, kpad, xq, sx, s);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(cq::launch_w2a8(static_cast<const uint8_t *>(W->blob), W->bits, W->rows, kpad,
                                    int8_codebook(W, lev), xq, sx, batch, y, s));
}

cq_status cq_gather_rows(const cq_matrix *W, const int64_t *ids, int64_t n, void *out, int32_t out_dtype,
                         void *stream) {
  cq::CodeLevels lev;
  cq_status st = check_matrix(W, &lev);
  if (st != CQ_OK) return st;
  if (out_dtype != CQ_F32 && out_dtype != CQ_F16 && out_dtype != CQ_BF16) return CQ_ERR_DTYPE;
  if (n < 0 || n > CQ_MAX_DIM) return CQ_ERR_SHAPE;
  if (n == 0 || W->cols == 0) return CQ_OK;
  if (!ids || !out) return CQ_ERR_NULL;
  if (!aligned(ids, 8) || !aligned(out, dtype_size(out_dtype))) return CQ_ERR_ALIGN;
  const uint64_t obytes = static_cast<uint64_t>(n) * W->cols * dtype_size(out_dtype);
  if (overlaps(out, obytes, ids, static_cast<uint64_t>(n) * 8) || overlaps(out, obytes, W->blob, W->blob_bytes))
    return CQ_ERR_OVERLAP;
  return hip_status(cq::launch_gather(static_cast<const uint8_t *>(W->blob), W->bits, W->rows, W->cols,
                                      padded(W->cols), lev, ids, n, out, out_dtype,
                                      static_cast<hipStream_t>(stream)));
}

cq_status cq_gemm(const cq_matrix *W, const void *xr, int64_t m, float *c, void *workspace,
                  uint64_t workspace_bytes, void *stream) {
  (void)workspace;  // no scratch: cq_workspace_bytes(CQ_OP_GEMM) is 0
  (void)workspace_bytes;
  cq::CodeLevels lev;
  cq_status st = check_matrix(W, &lev);
  if (st != CQ_OK) return st;
  if (m < 0 || m > CQ_MAX_DIM) return CQ_ERR_SHAPE;
  if (m == 0 || W->rows == 0) return CQ_OK;
  if (!c) return CQ_ERR_NULL;
  if (!aligned(c, 4)) return CQ_ERR_ALIGN;
  const uint64_t cbytes = static_cast<uint64_t>(m) * W->rows * 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t kpad = padded(W->cols);
  if (kpad > CQ_MAX_GEMM_COLS) return CQ_ERR_SHAPE;
  if (kpad == 0) return hip_status(cq::launch_zero_f32(c, m * W->rows, s));
  if (!xr) return CQ_ERR_NULL;
  if (!aligned(xr, 16)) return CQ_ERR_ALIGN;
  if (overlaps(c, cbytes, xr, static_cast<uint64_t>(m) * kpad * 2) ||
      overlaps(c, cbytes, W->blob, W->blob_bytes))
    return CQ_ERR_OVERLAP;
  return hip_status(cq::launch_gemm(static_cast<const uint8_t *>(W->blob), W->bits, W->rows, kpad,
                                    lev, xr, m, c, s));
}

cq_status cq_quantize(const float *w, int64_t rows, int64_t cols, int32_t bits, int32_t group,
                      const float *levels, void *blob, uint64_t blob_bytes, void *stream) {
  uint64_t need = 0;
  cq_status st = blob_bytes_impl(bits, group, rows, cols, &need);
  if (st != CQ_OK) return st;
  cq::CodeLevels lev;
  st = code_levels(bits, levels, &lev);
  if (st != CQ_OK) return st;
  if (blob_bytes != need) return CQ_ERR_LENGTH;
  if (need == 0) return CQ_OK;
  if (!w || !blob) return CQ_ERR_NULL;
  if (!aligned(w, 4) || !aligned(blob, 16)) return CQ_ERR_ALIGN;
  if (overlaps(blob, need, w, static_cast<uint64_t>(rows) * cols * 4)) return CQ_ERR_OVERLAP;

  const cq::EncodeTable tab = encode_table(bits, levels);
  const int64_t kpad = padded(cols);
  uint8_t *packed = static_cast<uint8_t *>(blob);
  uint16_t *norms = reinterpret_cast<uint16_t *>(packed + rows * (kpad * cq::storage_bits(bits) / 8));
  const cq::QuantizeJob job{w, rows, cols, kpad, packed, norms};
  return hip_status(cq::launch_quantize(job, nullptr, tab, bits, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

extern "C" {

cq_status cq_quantize_rows(const float *w, int64_t n, const cq_matrix *dst, int64_t row0, void *stream) {
  cq::CodeLevels lev;
  cq_status st = check_matrix(dst, &lev);
  if (st != CQ_OK) return st;
  if (n < 0 || row0 < 0 || n > dst->rows || row0 > dst->rows - n) return CQ_ERR_SHAPE;
  if (n == 0 || dst->cols == 0) return CQ_OK;
  if (!w) return CQ_ERR_NULL;
  if (!aligned(w, 4)) return CQ_ERR_ALIGN;
  if (overlaps(dst->blob, dst->blob_bytes, w, static_cast<uint64_t>(n) * dst->cols * 4)) return CQ_ERR_OVERLAP;
  const int64_t kpad = padded(dst->cols);
  const int64_t row_bytes = kpad * cq::storage_bits(dst->bits) / 8;
  uint8_t *blob = static_cast<uint8_t *>(const_cast<void *>(dst->blob));
  uint8_t *packed = blob + row0 * row_bytes;
  uint16_t *norms = reinterpret_cast<uint16_t *>(blob + dst->rows * row_bytes) + row0 * (kpad / CQ_GROUP);
  const cq::QuantizeJob job{w, n, dst->cols, kpad, packed, norms};
  return hip_status(cq::launch_quantize(job, nullptr, encode_table(dst->bits, dst->levels), dst->bits,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Checks of a score call; *xbytes: the padded queries' bytes.
cq_status check_kv(const cq_matrix *K, int32_t nq, int32_t n_kv, int32_t head_dim, cq::CodeLevels *lev) {
  cq_status st = check_matrix(K, lev);
  if (st != CQ_OK) return st;
  if ((st = check_matvec_cols(K)) != CQ_OK) return st;
  if (nq < 1 || n_kv < 1 || head_dim < 1 || nq > CQ_MAX_KV_HEADS || nq % n_kv != 0 ||
      static_cast<int64_t>(n_kv) * head_dim != K->cols)
    return CQ_ERR_SHAPE;
  return CQ_OK;
}

uint64_t kv_scores_ws(const cq_matrix *K, int32_t nq) {
  const int64_t b = nq < CQ_MAX_MATVEC_BATCH ? nq : CQ_MAX_MATVEC_BATCH;
  const uint64_t x = (static_cast<uint64_t>(nq) * K->cols * 4 + 255) / 256 * 256;
  return x + cq::rotate_matvec_workspace_bytes(K->bits, K->rows, padded(K->cols), b);
}

}  // namespace

extern "C" {

cq_status cq_kv_scores_workspace_bytes(const cq_matrix *K, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                       uint64_t *bytes) {
  if (!bytes) return CQ_ERR_NULL;
  cq::CodeLevels lev;
  cq_status st = check_kv(K, n_q_heads, n_kv_heads, head_dim, &lev);
  if (st != CQ_OK) return st;
  *bytes = K->rows ? kv_scores_ws(K, n_q_heads) : 0;
  return CQ_OK;
}

cq_status cq_kv_scores(const cq_matrix *K, const float *q, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                       float *scores, void *workspace, uint64_t workspace_bytes, void *stream) {
  cq::CodeLevels lev;
  cq_status st = check_kv(K, n_q_heads, n_kv_heads, head_dim, &lev);
  if (st != CQ_OK) return st;
  if (K->rows == 0) return CQ_OK;
  if (!q || !scores) return CQ_ERR_NULL;
  if (!aligned(q, 4) || !aligned(scores, 4)) return CQ_ERR_ALIGN;
  const uint64_t need = kv_scores_ws(K, n_q_heads);
  if (!workspace || workspace_bytes < need) return CQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return CQ_ERR_ALIGN;
  const uint64_t qbytes = static_cast<uint64_t>(n_q_heads) * head_dim * 4;
  const uint64_t sbytes = static_cast<uint64_t>(n_q_heads) * K->rows * 4;
  if (overlaps(scores, sbytes, q, qbytes) || overlaps(scores, sbytes, K->blob, K->blob_bytes) ||
      overlaps(workspace, need, scores, sbytes) || overlaps(workspace, need, q, qbytes) ||
      overlaps(workspace, need, K->blob, K->blob_bytes))
    return CQ_ERR_OVERLAP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float *x = static_cast<float *>(workspace);
  const uint64_t xb = (static_cast<uint64_t>(n_q_heads) * K->cols * 4 + 255) / 256 * 256;
  void *ws = static_cast<uint8_t *>(workspace) + xb;
  hipError_t e = cq::launch_kv_pad_queries(q, n_q_heads, n_kv_heads, head_dim, x, s);
  const int64_t kpad = padded(K->cols);
  for (int32_t h0 = 0; h0 < n_q_heads && e == hipSuccess; h0 += CQ_MAX_MATVEC_BATCH) {
    const int64_t b = n_q_heads - h0 < CQ_MAX_MATVEC_BATCH ? n_q_heads - h0 : CQ_MAX_MATVEC_BATCH;
    const bool need_ws = cq::rotate_matvec_workspace_bytes(K->bits, K->rows, kpad, b) > 0;
    e = cq::launch_rotate_matvec(static_cast<const uint8_t *>(K->blob), K->bits, K->rows, kpad, lev,
                                 x + static_cast<int64_t>(h0) * K->cols, K->cols, b,
                                 scores + static_cast<int64_t>(h0) * K->rows, need_ws ? ws : nullptr, s);
  }
  return hip_status(e);
}

cq_status cq_kv_append(const cq_matrix *K, const cq_matrix *V, const float *k, const float *v, int64_t n,
                       int64_t row0, void *stream) {
  cq::CodeLevels klev, vlev;
  cq_status st = check_matrix(K, &klev);
  if (st != CQ_OK) return st;
  if ((st = check_matrix(V, &vlev)) != CQ_OK) return st;
  if (V->bits != K->bits) return CQ_ERR_SHAPE;
  if (n < 0 || row0 < 0 || n > K->rows || row0 > K->rows - n || n > V->rows || row0 > V->rows - n)
    return CQ_ERR_SHAPE;
  if (n == 0) return CQ_OK;
  if (!k || !v) return CQ_ERR_NULL;
  if (!aligned(k, 4) || !aligned(v, 4)) return CQ_ERR_ALIGN;
  if (overlaps(K->blob, K->blob_bytes, V->blob, V->blob_bytes) ||
      overlaps(K->blob, K->blob_bytes, k, static_cast<uint64_t>(n) * K->cols * 4) ||
      overlaps(K->blob, K->blob_bytes, v, static_cast<uint64_t>(n) * V->cols * 4) ||
      overlaps(V->blob, V->blob_bytes, k, static_cast<uint64_t>(n) * K->cols * 4) ||
      overlaps(V->blob, V->blob_bytes, v, static_cast<uint64_t>(n) * V->cols * 4))
    return CQ_ERR_OVERLAP;
  auto job = [&](const cq_matrix *M, const float *w) {
    const int64_t kpad = padded(M->cols);
    const int64_t row_bytes = kpad * cq::storage_bits(M->bits) / 8;
    uint8_t *blob = static_cast<uint8_t *>(const_cast<void *>(M->blob));
    return cq::QuantizeJob{w, n, M->cols, kpad, blob + row0 * row_bytes,
                           reinterpret_cast<uint16_t *>(blob + M->rows * row_bytes) + row0 * (kpad / CQ_GROUP)};
  };
  const cq::QuantizeJob jk = job(K, k), jv = job(V, v);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool same_book = std::memcmp(&klev, &vlev, sizeof klev) == 0;
  if (same_book && K->cols > 0 && V->cols > 0)
    return hip_status(cq::launch_quantize(jk, &jv, encode_table(K->bits, K->levels), K->bits, s));
  hipError_t e = K->cols > 0 ? cq::launch_quantize(jk, nullptr, encode_table(K->bits, K->levels), K->bits, s)
                             : hipSuccess;
  if (e == hipSuccess && V->cols > 0) e = cq::launch_quantize(jv, nullptr, encode_table(V->bits, V->levels), V->bits, s);
  return hip_status(e);
}

cq_status cq_kv_attention(const cq_matrix *K, const cq_matrix *V, int64_t n_tokens, const float *q,
                          int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale, float *out,
                          void *stream) {
  cq::CodeLevels klev, vlev;
  cq_status st = check_kv(K, n_q_heads, n_kv_heads, head_dim, &klev);
  if (st != CQ_OK) return st;
  if ((st = check_kv(V, n_q_heads, n_kv_heads, head_dim, &vlev)) != CQ_OK) return st;
  if (V->bits != K->bits || V->rows != K->rows || head_dim > 128 || 128 % head_dim != 0 || n_tokens < 1 ||
      n_tokens > K->rows || n_tokens > CQ_MAX_KV_TOKENS)
    return CQ_ERR_SHAPE;
  const int64_t row_bytes = padded(K->cols) * cq::storage_bits(K->bits) / 8;
  if (n_tokens * row_bytes >= (int64_t{1} << 31)) return CQ_ERR_SHAPE;
  if (!q || !out) return CQ_ERR_NULL;
  if (!aligned(q, 4) || !aligned(out, 4)) return CQ_ERR_ALIGN;
  const uint64_t qbytes = static_cast<uint64_t>(n_q_heads) * head_dim * 4;
  if (overlaps(out, qbytes, q, qbytes) || overlaps(out, qbytes, K->blob, K->blob_bytes) ||
      overlaps(out, qbytes, V->blob, V->blob_bytes))
    return CQ_ERR_OVERLAP;
  return hip_status(cq::launch_kv_attention(static_cast<const uint8_t *>(K->blob), static_cast<const uint8_t *>(V->blob),
                                            K->bits, K->rows, padded(K->cols), klev, vlev, n_tokens, q, n_q_heads,
                                            n_kv_heads, head_dim, scale, out, static_cast<hipStream_t>(stream)));
}

cq_status cq_matvec_t(const cq_matrix *W, const float *p, int64_t batch, float *out, void *workspace,
                      uint64_t workspace_bytes, void *stream) {
  cq::CodeLevels lev;
  cq_status st = check_matrix(W, &lev);
  if (st != CQ_OK) return st;
  if (batch < 0 || batch > CQ_MAX_MATVEC_BATCH) return CQ_ERR_SHAPE;
  if (!matvec_t_shape_ok(W)) return CQ_ERR_SHAPE;
  if (batch == 0 || W->cols == 0) return CQ_OK;
  if (!out) return CQ_ERR_NULL;
  if (!aligned(out, 4)) return CQ_ERR_ALIGN;
  const uint64_t obytes = static_cast<uint64_t>(batch) * W->cols * 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (W->rows == 0) return hip_status(cq::launch_zero_f32(out, batch * W->cols, s));
  if (!p) return CQ_ERR_NULL;
  if (!aligned(p, 4)) return CQ_ERR_ALIGN;
  const uint64_t need = cq::matvec_t_workspace_bytes(W->rows, W->cols, batch);
  if (need) {
    if (!workspace || workspace_bytes < need) return CQ_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return CQ_ERR_ALIGN;
  }
  const uint64_t pbytes = static_cast<uint64_t>(batch) * W->rows * 4;
  if (overlaps(out, obytes, p, pbytes) || overlaps(out, obytes, W->blob, W->blob_bytes) ||
      overlaps(workspace, need, out, obytes) || overlaps(workspace, need, p, pbytes) ||
      overlaps(workspace, need, W->blob, W->blob_bytes))
    return CQ_ERR_OVERLAP;
  return hip_status(cq::launch_matvec_t(static_cast<const uint8_t *>(W->blob), W->bits, W->rows, W->cols,
                                        padded(W->cols), lev, p, batch, out, need ? workspace : nullptr, s));
}

}  // extern "C"
