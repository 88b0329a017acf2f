// Memory-system probe for measurement: a read-only stream over a device
// buffer.  The decode passes of the library are HBM-bound reads, so the
// rate this kernel reaches (large buffers) and its time per launch (buffers
// of the kept-token passes' size, 1-64 MB) are the platform's own ceiling and
// floor for them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fastocr.h"

namespace fastocr {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;  // 16-byte loads in flight per thread per iteration

// Every thread folds the 16-byte pieces it reads into one word; a word equal
// to `never` (a value the host picks so that it does not occur) would be
// stored, so the loads are live but nothing is written in practice.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* __restrict__ src, int64_t n16,
                                                                   uint32_t never, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == never) sink[blockIdx.x & 63] = acc;
}

}  // namespace
}  // namespace fastocr

extern "C" int fastocr_probe_read(const void* buf, int64_t bytes, int32_t workgroups, uint32_t* sink,
                                  void* hip_stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 || workgroups < 1) return FASTOCR_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(buf) % 16) return FASTOCR_ERR_INVALID_ARG;
  fastocr::read_probe_kernel<<<workgroups, fastocr::kProbeThreads, 0, reinterpret_cast<hipStream_t>(hip_stream)>>>(
      reinterpret_cast<const uint4*>(buf), bytes / 16, 0x9e3779b9u, sink);
  return hipGetLastError() == hipSuccess ? FASTOCR_OK : FASTOCR_ERR_HIP;
}
