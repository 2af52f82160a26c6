// The scratch of qbl_linear_static: one file-scope device array per GPU, for
// callers that cannot allocate device memory.  Internal to the library.
//
// In host code the array's name is a host-side stand-in for the symbol, not a
// device address: the address comes from hipGetSymbolAddress, called once per
// device with that device current (each GPU holds its own copy of the array at
// its own address), and only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qbl_kernels.h"

namespace qbl {
namespace {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// Zeroes n 16-byte words (grid-stride; n fits the array by construction).
__global__ __launch_bounds__(256) void clear_scratch_kernel(uint4* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of the array per device, null until set up

}  // namespace

hipError_t static_scratch(hipStream_t st, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_ptr[dev]) {
    // Set-up on this device's first call: it enqueues the clear, which must not
    // land in a graph being captured.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(st, &cs);
    if (e != hipSuccess) return e;
    if (cs != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // the batch-1 hand-off needs its words zeroed once before first use
    const int64_t words = kStaticScratchBytes / 16;
    hipLaunchKernelGGL(clear_scratch_kernel, dim3(1024), dim3(256), 0, st, static_cast<uint4*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace qbl
