// Test double of the HIP runtime (see hip/hip_runtime.h here) and of the
// library's kernel launchers, so that the unchanged host runtime source builds
// with g++ into a CPU-only library for lifecycle tests.  Device allocations are
// host allocations that the double tracks: every copy must stay inside one live
// allocation, frees must match allocations, and a capacity can be set so that
// allocations fail like a full device.  Kernel launches fail with
// hipErrorNoDevice: run calls cannot fall back to the CPU.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>

#include "../../quantized_base_linear_amd/csrc/qbl_kernels.h"

namespace {

struct Sim {
  std::mutex mu;
  std::map<uintptr_t, size_t> live;  // base address -> bytes
  int64_t live_bytes = 0;
  int64_t capacity = 0;              // 0 = unlimited
  int64_t allocations = 0, frees = 0, bad_copies = 0, bad_frees = 0;
  void* last = nullptr;              // most recent allocation
};

Sim& sim() {
  static Sim s;
  return s;
}

// True when [p, p + n) lies inside one live allocation.
bool inside(const void* p, size_t n) {
  Sim& s = sim();
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  auto it = s.live.upper_bound(a);
  if (it == s.live.begin()) return false;
  --it;
  return a >= it->first && a + n <= it->first + it->second;
}

thread_local int t_device = 0;

}  // namespace

hipError_t hipGetDevice(int* device) {
  if (!device) return hipErrorInvalidValue;
  *device = t_device;
  return hipSuccess;
}

hipError_t hipSetDevice(int device) {
  if (device != 0) return hipErrorInvalidDevice;
  t_device = device;
  return hipSuccess;
}

hipError_t hipMalloc(void** ptr, size_t size) {
  if (!ptr) return hipErrorInvalidValue;
  *ptr = nullptr;
  Sim& s = sim();
  std::lock_guard<std::mutex> g(s.mu);
  const size_t bytes = size ? (size + 255) / 256 * 256 : 256;
  if (s.capacity > 0 && s.live_bytes + (int64_t)bytes > s.capacity) return hipErrorOutOfMemory;
  void* p = std::aligned_alloc(256, bytes);
  if (!p) return hipErrorOutOfMemory;
  std::memset(p, 0xA5, bytes);  // like fresh device memory, not zero
  s.live[reinterpret_cast<uintptr_t>(p)] = size;
  s.live_bytes += (int64_t)bytes;
  ++s.allocations;
  s.last = p;
  *ptr = p;
  return hipSuccess;
}

hipError_t hipFree(void* ptr) {
  if (!ptr) return hipSuccess;
  Sim& s = sim();
  std::lock_guard<std::mutex> g(s.mu);
  auto it = s.live.find(reinterpret_cast<uintptr_t>(ptr));
  if (it == s.live.end()) {
    ++s.bad_frees;
    return hipErrorInvalidValue;
  }
  s.live_bytes -= (int64_t)(it->second ? (it->second + 255) / 256 * 256 : 256);
  s.live.erase(it);
  ++s.frees;
  std::free(ptr);
  return hipSuccess;
}

hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind kind) {
  if (n == 0) return hipSuccess;
  if (!dst || !src) return hipErrorInvalidValue;
  Sim& s = sim();
  {
    std::lock_guard<std::mutex> g(s.mu);
    const bool dev_dst = kind == hipMemcpyHostToDevice || kind == hipMemcpyDeviceToDevice;
    const bool dev_src = kind == hipMemcpyDeviceToHost || kind == hipMemcpyDeviceToDevice;
    if ((dev_dst && !inside(dst, n)) || (dev_src && !inside(src, n))) {
      ++s.bad_copies;
      return hipErrorInvalidValue;
    }
  }
  std::memmove(dst, src, n);
  return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

hipError_t hipEventCreate(hipEvent_t* event) { return hipEventCreateWithFlags(event, 0); }
hipError_t hipEventCreateWithFlags(hipEvent_t* event, unsigned) {
  if (!event) return hipErrorInvalidValue;
  *event = reinterpret_cast<hipEvent_t>(new char(0));
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  if (ms) *ms = 0.0f;
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t event) {
  delete reinterpret_cast<char*>(event);
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }

// Pinned host memory is ordinary host memory here, outside the device tally.
hipError_t hipHostMalloc(void** ptr, size_t size, unsigned) {
  if (!ptr) return hipErrorInvalidValue;
  *ptr = std::calloc(1, size ? size : 1);
  return *ptr ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t hipHostGetDevicePointer(void** dev, void* host, unsigned) {
  if (!dev || !host) return hipErrorInvalidValue;
  *dev = host;
  return hipSuccess;
}

hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* status) {
  if (!status) return hipErrorInvalidValue;
  *status = hipStreamCaptureStatusNone;
  return hipSuccess;
}

const char* hipGetErrorString(hipError_t error) {
  switch (error) {
    case hipSuccess: return "hipSuccess";
    case hipErrorInvalidValue: return "hipErrorInvalidValue";
    case hipErrorOutOfMemory: return "hipErrorOutOfMemory";
    case hipErrorNoDevice: return "hipErrorNoDevice";
    case hipErrorInvalidDevice: return "hipErrorInvalidDevice";
  }
  return "unknown error";
}

// The kernel launchers: no GPU here.
namespace qbl {
hipError_t launch_prep(const PrepArgs&, const LaunchCtx&) { return hipErrorNoDevice; }
hipError_t launch_rms(const float*, int, float*, const LaunchCtx&) { return hipErrorNoDevice; }
hipError_t launch_gemv(GemvArgs&, const LaunchCtx&) { return hipErrorNoDevice; }
int64_t mfma_stage_bytes(int64_t, int, int) { return 0; }
hipError_t launch_gemv_mfma(GemvArgs&, const PrepEntry*, int, int, void*, int, const LaunchCtx&, const LaunchCtx&) {
  return hipErrorNoDevice;
}
bool fused_supported(int, int) { return true; }
hipError_t launch_fused(FusedArgs&, const LaunchCtx&) { return hipErrorNoDevice; }
hipError_t launch_jit(const JitArgs&, const LaunchCtx&) { return hipErrorNoDevice; }
int64_t jit_workspace_bytes(int, int, int) { return 0; }
hipError_t launch_dar(const DarArgs&, const LaunchCtx&) { return hipErrorNoDevice; }
int probe_workgroups(int sink_words) { return sink_words < 2048 ? sink_words : 2048; }
hipError_t launch_hbm_probe(const void*, int64_t, uint32_t*, int, const LaunchCtx&) { return hipErrorNoDevice; }
hipError_t static_scratch(hipStream_t, void**) { return hipErrorNoDevice; }
}  // namespace qbl

// Inspection of the double, for the tests.
extern "C" int64_t qbl_sim_live_bytes(void) {
  std::lock_guard<std::mutex> g(sim().mu);
  return sim().live_bytes;
}
extern "C" int64_t qbl_sim_live_allocations(void) {
  std::lock_guard<std::mutex> g(sim().mu);
  return (int64_t)sim().live.size();
}
extern "C" int64_t qbl_sim_bad_calls(void) {
  std::lock_guard<std::mutex> g(sim().mu);
  return sim().bad_copies + sim().bad_frees;
}
extern "C" void* qbl_sim_last_allocation(void) {
  std::lock_guard<std::mutex> g(sim().mu);
  return sim().last;
}
extern "C" void qbl_sim_set_capacity(int64_t bytes) {
  std::lock_guard<std::mutex> g(sim().mu);
  sim().capacity = bytes;
}
// Changes one byte of simulated device memory, as a fault outside the library
// would (the base's later hash must notice).
extern "C" int qbl_sim_poke(void* device_ptr, uint8_t xor_mask) {
  std::lock_guard<std::mutex> g(sim().mu);
  if (!inside(device_ptr, 1)) return -1;
  *static_cast<uint8_t*>(device_ptr) ^= xor_mask;
  return 0;
}
