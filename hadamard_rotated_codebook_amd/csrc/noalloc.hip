// cq_rotate_matvec_noalloc: the decode product from the activation before
// rotation with no workspace argument and no allocation, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The call's scratch (the K-slice partial sums, and for batches the rotated
// activation) lives in `scratch`, a file-scope device array of
// CQ_NOALLOC_SCRATCH_BYTES.  Each GPU the library runs on holds its own copy
// from module load until the process ends.  In host code the array's name
// stands for a host-side shadow, not a device address, so it is never passed
// to a kernel: the first call on a device, with that device current, asks
// the runtime for that device's address (hipGetSymbolAddress) and keeps it;
// every later call on the device uses the kept address.
//
// Every call on one GPU uses the same array and leaves its contents behind.
// Nothing needs clearing: the kernels write every partial sum and every
// rotated value they read within the same call.  Calls that run at the same
// time on one GPU (several streams, several host threads) share the array
// and race.
#include <atomic>
#include <mutex>

#include "cq_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[CQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch`.
cq_status device_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CQ_ERR_HIP;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void *addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return CQ_ERR_HIP;
      g_scratch[dev].store(addr, std::memory_order_release);
      p = addr;
    }
  }
  *out = p;
  return CQ_OK;
}

}  // namespace

extern "C" cq_status cq_rotate_matvec_noalloc(const cq_matrix *W, const float *x, int64_t batch, float *y,
                                              void *stream) {
  uint64_t need = 0;
  cq_status st = cq_workspace_bytes(CQ_OP_ROTATE_MATVEC, W, batch, &need);
  if (st != CQ_OK) return st;
  if (need > CQ_NOALLOC_SCRATCH_BYTES) return CQ_ERR_SCRATCH;
  void *ws = nullptr;
  if (need && batch > 0 && W->rows > 0 && W->cols > 0) {
    st = device_scratch(&ws);
    if (st != CQ_OK) return st;
  }
  return cq_rotate_matvec(W, x, batch, y, ws, need, stream);
}
