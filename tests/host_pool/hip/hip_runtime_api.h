/* Host-only stand-in for the HIP runtime API, for building the slot pool
 * (csrc/pool.cpp) and the error helpers (csrc/layout.cpp) with g++ on a
 * machine without a GPU: "device" memory is host memory, copies are
 * immediate memcpy, streams and events are bookkeeping objects (a copy is
 * complete when it returns, so every event is complete when recorded).
 * Declares only what those two files use.  Test infrastructure. */
#ifndef MOE_FAKE_HIP_RUNTIME_API_H
#define MOE_FAKE_HIP_RUNTIME_API_H

#include <stddef.h>

typedef enum hipError_t {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorOutOfMemory = 2,
  hipErrorNotReady = 600
} hipError_t;

typedef enum hipMemcpyKind {
  hipMemcpyHostToHost = 0,
  hipMemcpyHostToDevice = 1,
  hipMemcpyDeviceToHost = 2,
  hipMemcpyDeviceToDevice = 3,
  hipMemcpyDefault = 4
} hipMemcpyKind;

typedef struct fake_hip_stream* hipStream_t;
typedef struct fake_hip_event* hipEvent_t;

#define hipHostMallocDefault 0x0
#define hipEventDisableTiming 0x2
#define hipStreamNonBlocking 0x1

#ifdef __cplusplus
extern "C" {
#endif
hipError_t hipSetDevice(int device);
hipError_t hipMalloc(void** ptr, size_t size);
hipError_t hipFree(void* ptr);
hipError_t hipHostMalloc(void** ptr, size_t size, unsigned int flags);
hipError_t hipHostFree(void* ptr);
hipError_t hipMemset(void* dst, int value, size_t size);
hipError_t hipMemsetAsync(void* dst, int value, size_t size, hipStream_t stream);
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t size, hipMemcpyKind kind,
                          hipStream_t stream);
hipError_t hipStreamCreateWithFlags(hipStream_t* stream, unsigned int flags);
hipError_t hipStreamDestroy(hipStream_t stream);
hipError_t hipStreamSynchronize(hipStream_t stream);
hipError_t hipStreamWaitEvent(hipStream_t stream, hipEvent_t event, unsigned int flags);
hipError_t hipEventCreateWithFlags(hipEvent_t* event, unsigned int flags);
hipError_t hipEventDestroy(hipEvent_t event);
hipError_t hipEventRecord(hipEvent_t event, hipStream_t stream);
hipError_t hipEventQuery(hipEvent_t event);
hipError_t hipEventSynchronize(hipEvent_t event);
const char* hipGetErrorString(hipError_t error);

/* Test counters: host-to-device copies of exactly `bytes` bytes, and
 * stream waits on events, since the process started. */
long long fake_hip_copies_of(size_t bytes);
long long fake_hip_stream_waits(void);
#ifdef __cplusplus
}
#endif

#endif /* MOE_FAKE_HIP_RUNTIME_API_H */
