// Test double of the HIP runtime API for CPU-only tests of the library's host
// logic (the lifecycle of bases, adapters and compositions).  "Device" memory
// is host memory that the double allocates and bounds-checks; there is no GPU
// and no kernel: every launch reports hipErrorNoDevice.  Only the calls the
// host runtime makes are declared here.  Never part of the product library.
#pragma once
#include <cstddef>
#include <cstdint>

typedef enum hipError_t {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorOutOfMemory = 2,
  hipErrorNoDevice = 100,
  hipErrorInvalidDevice = 101,
  hipErrorStreamCaptureUnsupported = 900,
} hipError_t;

typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

typedef enum hipMemcpyKind {
  hipMemcpyHostToHost = 0,
  hipMemcpyHostToDevice = 1,
  hipMemcpyDeviceToHost = 2,
  hipMemcpyDeviceToDevice = 3,
  hipMemcpyDefault = 4,
} hipMemcpyKind;

#define hipEventDefault 0x0
#define hipEventDisableTiming 0x2
#define hipEventDisableSystemFence 0x20000000

hipError_t hipGetDevice(int* device);
hipError_t hipSetDevice(int device);
hipError_t hipMalloc(void** ptr, size_t size);
hipError_t hipFree(void* ptr);
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind kind);
hipError_t hipStreamSynchronize(hipStream_t stream);
hipError_t hipEventCreate(hipEvent_t* event);
hipError_t hipEventCreateWithFlags(hipEvent_t* event, unsigned flags);
hipError_t hipEventRecord(hipEvent_t event, hipStream_t stream);
hipError_t hipEventSynchronize(hipEvent_t event);
hipError_t hipEventElapsedTime(float* ms, hipEvent_t start, hipEvent_t stop);
hipError_t hipEventDestroy(hipEvent_t event);
hipError_t hipGetLastError(void);
const char* hipGetErrorString(hipError_t error);

// pinned host memory (plain host memory here) and stream capture (never active)
#define hipHostMallocDefault 0x0
#define hipHostMallocMapped 0x2
#define hipHostMallocCoherent 0x40000000
hipError_t hipHostMalloc(void** ptr, size_t size, unsigned flags);
hipError_t hipHostGetDevicePointer(void** dev, void* host, unsigned flags);
typedef enum hipStreamCaptureStatus {
  hipStreamCaptureStatusNone = 0,
  hipStreamCaptureStatusActive = 1,
  hipStreamCaptureStatusInvalidated = 2,
} hipStreamCaptureStatus;
hipError_t hipStreamIsCapturing(hipStream_t stream, hipStreamCaptureStatus* status);
