// Streaming-read probe: the rate at which one kernel can read a buffer from
// HBM with the widest loads, the ceiling the HBM-bound products are measured
// against beside the published peak.  Each workgroup reads 32 KB tiles (256
// threads x 8 loads of 16 bytes, contiguous), tiles dealt out round robin;
// loads past the end read zeros through the buffer range.  The loads carry
// the nt (streaming) cache hint, as the products' code loads do: on the
// 285 MB CQ2 blob it reads ~6.4 TB/s against ~5.8 TB/s with plain loads.
#include "cq_decode.h"
#include "cq_internal.h"

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeLoads = 8;
constexpr uint64_t kTile = static_cast<uint64_t>(kProbeThreads) * kProbeLoads * 16;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint8_t *p, uint64_t bytes, uint32_t *sink) {
  const uint64_t ntiles = (bytes + kTile - 1) / kTile;
  uint32_t acc = 0;
  for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const uint64_t base = t * kTile;
    const uint64_t left = bytes - base;
    const __amdgpu_buffer_rsrc_t r =
        cqdev::buffer_rsrc(p + base, static_cast<uint32_t>(left < kTile ? left : kTile));
    cqdev::u32x4 v[kProbeLoads];
#pragma unroll
    for (int l = 0; l < kProbeLoads; ++l)
      v[l] = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<uint32_t>((l * kProbeThreads + threadIdx.x) * 16), 0, cq::kStreamLoad);
#pragma unroll
    for (int l = 0; l < kProbeLoads; ++l) acc ^= v[l].x ^ v[l].y ^ v[l].z ^ v[l].w;
  }
  sink[static_cast<uint64_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" cq_status cq_read_probe(const void *p, uint64_t bytes, uint32_t *sink, uint64_t sink_words, void *stream) {
  if (bytes == 0) return CQ_OK;
  if (!p || !sink) return CQ_ERR_NULL;
  const uint64_t grid = sink_words / kProbeThreads;
  if (grid < 1) return CQ_ERR_WORKSPACE;
  const uint64_t g = grid < 65535 ? grid : 65535;
  read_probe_kernel<<<dim3(static_cast<unsigned>(g)), kProbeThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint8_t *>(p), bytes, sink);
  return hipGetLastError() == hipSuccess ? CQ_OK : CQ_ERR_HIP;
}
