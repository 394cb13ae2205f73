// Host-only stand-in for the HIP runtime functions the slot pool uses (see
// hip/hip_runtime_api.h).  Test infrastructure: never linked into libmoe.
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>

#include "hip/hip_runtime_api.h"

struct fake_hip_stream {
  int id;
};
struct fake_hip_event {
  bool recorded;
};

namespace {
std::mutex g_mu;
std::map<size_t, long long> g_copies;
long long g_waits = 0;
}  // namespace

extern "C" {

hipError_t hipSetDevice(int device) { return device == 0 ? hipSuccess : hipErrorInvalidValue; }

hipError_t hipMalloc(void** ptr, size_t size) {
  *ptr = std::malloc(size ? size : 1);
  return *ptr ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* ptr) {
  std::free(ptr);
  return hipSuccess;
}
hipError_t hipHostMalloc(void** ptr, size_t size, unsigned int) {
  // page-aligned, as pinned allocations are (the pool checks it)
  *ptr = nullptr;
  if (posix_memalign(ptr, 4096, size ? size : 1) != 0) return hipErrorOutOfMemory;
  return hipSuccess;
}
hipError_t hipHostFree(void* ptr) {
  std::free(ptr);
  return hipSuccess;
}
hipError_t hipMemset(void* dst, int value, size_t size) {
  std::memset(dst, value, size);
  return hipSuccess;
}
hipError_t hipMemsetAsync(void* dst, int value, size_t size, hipStream_t) {
  std::memset(dst, value, size);
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t size, hipMemcpyKind kind,
                          hipStream_t) {
  std::memcpy(dst, src, size);
  if (kind == hipMemcpyHostToDevice) {
    std::lock_guard<std::mutex> lock(g_mu);
    g_copies[size] += 1;
  }
  return hipSuccess;
}
hipError_t hipStreamCreateWithFlags(hipStream_t* stream, unsigned int) {
  static int next = 1;
  *stream = new fake_hip_stream{next++};
  return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t stream) {
  delete stream;
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t event, unsigned int) {
  if (!event) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lock(g_mu);
  g_waits += 1;
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* event, unsigned int) {
  *event = new fake_hip_event{false};
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t event) {
  delete event;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t event, hipStream_t) {
  if (!event) return hipErrorInvalidValue;
  event->recorded = true;
  return hipSuccess;
}
hipError_t hipEventQuery(hipEvent_t event) { return event ? hipSuccess : hipErrorInvalidValue; }
hipError_t hipEventSynchronize(hipEvent_t event) {
  return event ? hipSuccess : hipErrorInvalidValue;
}
const char* hipGetErrorString(hipError_t error) {
  switch (error) {
    case hipSuccess: return "hipSuccess";
    case hipErrorInvalidValue: return "hipErrorInvalidValue";
    case hipErrorOutOfMemory: return "hipErrorOutOfMemory";
    case hipErrorNotReady: return "hipErrorNotReady";
  }
  return "unknown";
}

long long fake_hip_copies_of(size_t bytes) {
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_copies.find(bytes);
  return it == g_copies.end() ? 0 : it->second;
}
long long fake_hip_stream_waits(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  return g_waits;
}

}  // extern "C"
