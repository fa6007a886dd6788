/*
 * A plain C99 client of libcq: the boundary used without Python or PyTorch.
 * Device memory comes from the HIP runtime, everything else through the
 * entry points of include/cq.h.
 *
 *   c_client <dir>
 *
 * reads <dir>/in.bin (int64 rows, cols, batch; fp32 levels[4]; fp32 w[rows]
 * [cols]; fp32 x[batch][cols]), encodes w at 2 bits with cq_quantize, rotates
 * x with cq_rotate_acts, runs cq_matvec (with the workspace it asks for) and
 * writes <dir>/blob.bin and <dir>/y.bin.  Exit status 0 on success; any
 * failing call prints its status string and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>

#include "cq.h"

#define CHECK_CQ(call)                                                    \
  do {                                                                    \
    cq_status st_ = (call);                                               \
    if (st_ != CQ_OK) {                                                   \
      fprintf(stderr, "%s: %s\n", #call, cq_status_string(st_));          \
      return 1;                                                           \
    }                                                                     \
  } while (0)
#define CHECK_HIP(call)                                                   \
  do {                                                                    \
    if ((call) != hipSuccess) {                                           \
      fprintf(stderr, "%s failed\n", #call);                              \
      return 1;                                                           \
    }                                                                     \
  } while (0)

static int read_all(const char *path, void *dst, size_t n, long offset) {
  FILE *f = fopen(path, "rb");
  if (!f) return 1;
  int bad = fseek(f, offset, SEEK_SET) != 0 || fread(dst, 1, n, f) != n;
  fclose(f);
  return bad;
}

static int write_all(const char *path, const void *src, size_t n) {
  FILE *f = fopen(path, "wb");
  if (!f) return 1;
  int bad = fwrite(src, 1, n, f) != n;
  fclose(f);
  return bad;
}

int main(int argc, char **argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: c_client <dir>\n");
    return 2;
  }
  char in_path[4096], blob_path[4096], y_path[4096];
  snprintf(in_path, sizeof in_path, "%s/in.bin", argv[1]);
  snprintf(blob_path, sizeof blob_path, "%s/blob.bin", argv[1]);
  snprintf(y_path, sizeof y_path, "%s/y.bin", argv[1]);

  int64_t dims[3];
  float levels[4];
  if (read_all(in_path, dims, sizeof dims, 0) || read_all(in_path, levels, sizeof levels, sizeof dims)) return 1;
  const int64_t rows = dims[0], cols = dims[1], batch = dims[2];
  if (rows <= 0 || cols <= 0 || batch <= 0 || batch > CQ_MAX_MATVEC_BATCH || rows * cols > (1 << 24)) return 1;
  const int64_t kpad = (cols + CQ_GROUP - 1) / CQ_GROUP * CQ_GROUP;
  const size_t wn = (size_t)(rows * cols), xn = (size_t)(batch * cols);
  float *w = malloc(wn * sizeof(float)), *x = malloc(xn * sizeof(float));
  float *y = malloc((size_t)(batch * rows) * sizeof(float));
  if (!w || !x || !y) return 1;
  const long off = (long)(sizeof dims + sizeof levels);
  if (read_all(in_path, w, wn * sizeof(float), off) ||
      read_all(in_path, x, xn * sizeof(float), off + (long)(wn * sizeof(float))))
    return 1;

  uint64_t blob_bytes = 0;
  CHECK_CQ(cq_blob_bytes(2, CQ_GROUP, rows, cols, &blob_bytes));
  /* a call that must fail: bits 6 is no CQ width */
  uint64_t unused = 0;
  if (cq_blob_bytes(6, CQ_GROUP, rows, cols, &unused) != CQ_ERR_BITS) return 1;

  void *d_w = NULL, *d_x = NULL, *d_xr = NULL, *d_y = NULL, *d_blob = NULL, *d_ws = NULL;
  CHECK_HIP(hipMalloc(&d_w, wn * sizeof(float)));
  CHECK_HIP(hipMalloc(&d_x, xn * sizeof(float)));
  CHECK_HIP(hipMalloc(&d_xr, (size_t)(batch * kpad) * sizeof(float)));
  CHECK_HIP(hipMalloc(&d_y, (size_t)(batch * rows) * sizeof(float)));
  CHECK_HIP(hipMalloc(&d_blob, blob_bytes));
  CHECK_HIP(hipMemcpy(d_w, w, wn * sizeof(float), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_x, x, xn * sizeof(float), hipMemcpyHostToDevice));

  CHECK_CQ(cq_quantize(d_w, rows, cols, 2, CQ_GROUP, levels, d_blob, blob_bytes, NULL));
  const cq_matrix W = {2, CQ_GROUP, rows, cols, d_blob, blob_bytes, levels};
  CHECK_CQ(cq_rotate_acts(d_x, CQ_F32, batch, cols, d_xr, CQ_F32, NULL));
  uint64_t ws_bytes = 0;
  CHECK_CQ(cq_workspace_bytes(CQ_OP_MATVEC, &W, batch, &ws_bytes));
  if (ws_bytes) CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
  CHECK_CQ(cq_matvec(&W, d_xr, batch, d_y, d_ws, ws_bytes, NULL));
  CHECK_HIP(hipDeviceSynchronize());

  unsigned char *blob = malloc(blob_bytes);
  if (!blob) return 1;
  CHECK_HIP(hipMemcpy(blob, d_blob, blob_bytes, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(y, d_y, (size_t)(batch * rows) * sizeof(float), hipMemcpyDeviceToHost));
  if (write_all(blob_path, blob, blob_bytes) || write_all(y_path, y, (size_t)(batch * rows) * sizeof(float))) return 1;

  hipFree(d_w), hipFree(d_x), hipFree(d_xr), hipFree(d_y), hipFree(d_blob);
  if (d_ws) hipFree(d_ws);
  free(w), free(x), free(y), free(blob);
  printf("c_client ok: %lld x %lld, batch %lld, %llu blob bytes\n", (long long)rows, (long long)cols,
         (long long)batch, (unsigned long long)blob_bytes);
  return 0;
}
