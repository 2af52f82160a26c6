// Read-only HBM streaming probe: the read bandwidth this device achieves with
// the access the batch-1 kernels use (16-byte non-temporal loads from every
// lane), as context for the fraction of the nameplate peak.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "qbl_device.h"
#include "qbl_kernels.h"

namespace qbl {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // loads in flight per lane

// Workgroup g reads 16-byte words g*256 + tid + i*stride (stride = grid * 256)
// for i = 0, 1, ...: every word once.  Each workgroup writes the XOR of its
// words to sink[g], so a caller can check that every word was read exactly
// once (a word read twice would cancel).
__global__ __launch_bounds__(kProbeThreads) void hbm_probe_kernel(const uint4* p, int64_t n16, uint32_t* sink) {
  __shared__ uint32_t red[kProbeThreads / 64];
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = stream_load16(reinterpret_cast<const uint8_t*>(p + i + u * stride));
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = stream_load16(reinterpret_cast<const uint8_t*>(p + i));
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / 64; ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

}  // namespace

// 8 workgroups per compute unit (enough loads in flight to cover the latency),
// at most one per sink word
int probe_workgroups(int sink_words) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  return std::max(1, std::min(sink_words, 8 * cus));
}

hipError_t launch_hbm_probe(const void* buf, int64_t bytes, uint32_t* sink, int sink_words, const LaunchCtx& lc) {
  (void)hipGetLastError();  // drop errors left by earlier, unrelated calls
  if (!buf || !sink || bytes < 16 || bytes % 16 || sink_words < 1 || reinterpret_cast<uintptr_t>(buf) % 16)
    return hipErrorInvalidValue;
  const int grid = probe_workgroups(sink_words);
  QBL_LAUNCH(hbm_probe_kernel, dim3(grid), dim3(kProbeThreads), 0, lc, static_cast<const uint4*>(buf), bytes / 16,
             sink);
  return hipGetLastError();
}

}  // namespace qbl
