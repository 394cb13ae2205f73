// Calibration kernel: the ceiling a batch-1 decode layer could reach.
//
// A decode layer streams its weight bytes once, but cannot stream the next
// layer's routed experts before the layer's own all-to-all hand-offs are
// done.  This kernel measures that shape with nothing else in it: the same
// grid as the persistent stack kernel (256 workgroups x 512 threads, all
// resident), a sequence of phases, each reading `bytes` of fresh memory
// (16-byte loads, every load of a workgroup in flight at once) and then
// `handoffs` dependent all-to-all exchanges through tagged words, exactly
// as the stack kernel exchanges y, logits and h (value and call tag in one
// write-through store, 8 copies, one per XCD; coherent polls, each polling
// wave on its own, one workgroup barrier after the wait).  Its time
// per phase is what streaming that many bytes plus that many hand-offs
// costs on this device.
#include "device.h"
#include "kernels.h"

namespace moe {
namespace {

using namespace dev;

constexpr int kCT = kStackThreads;
constexpr int kCG = kStackGrid;
constexpr int kCRep = kStackReplicas;

__global__ __launch_bounds__(kCT, 1) void stream_phases_kernel(const uint4* buf, int64_t n16,
                                                                int phases, int handoffs,
                                                                uint64_t* words, uint32_t* epochs,
                                                                float* sink, int32_t* err,
                                                                int64_t timeout_ticks) {
  const int blk = blockIdx.x, tid = threadIdx.x;
  const int rep = blk % kCRep;
  const uint32_t epoch = ld_dev(epochs + blk);
  const uint32_t tag = 2u * epoch + 1u;
  const int64_t deadline = wall_clock64() + timeout_ticks;
  // this workgroup's share of a phase's 16-byte units
  const int64_t per = (n16 + kCG - 1) / kCG;
  const int64_t u0 = (int64_t)blk * per, u1 = u0 + per < n16 ? u0 + per : n16;
  uint32_t acc = 0;
  bool failed = false;
  for (int p = 0; p < phases && !failed; ++p) {
    const uint4* base = buf + (size_t)p * n16;
    int64_t i = u0 + tid;
    // 8 loads per thread in flight per step
    for (; i + 7 * kCT < u1; i += 8 * kCT) {
      uint4 v[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) v[m] = ld16(base + i + m * kCT);
#pragma unroll
      for (int m = 0; m < 8; ++m) acc ^= v[m].x ^ v[m].y ^ v[m].z ^ v[m].w;
    }
    for (; i < u1; i += kCT) {
      const uint4 v = ld16(base + i);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int h = 0; h < handoffs && !failed; ++h) {
      // every workgroup publishes one word (depending on what it read) in
      // 8 copies, then waits for all 256 words of its XCD's copy
      // (every thread has used its loads before the barrier, so the word
      // goes out after all of the workgroup's loads have returned)
      uint64_t* w = words + ((size_t)(p * handoffs + h) * kCRep) * kCG;
      __syncthreads();
      if (tid < kCRep)
        st_dev(w + (size_t)tid * kCG + blk, (uint64_t)acc | ((uint64_t)tag << 32));
      // waves 0..3 poll one word per lane, each wave on its own until all
      // of its words are in; one barrier joins the workgroup
      const uint64_t* mine = w + (size_t)rep * kCG;
      uint32_t got = 0;
      bool to = false;
      if (tid < kCG) {
        bool have = false;
        for (;;) {
          if (!have) {
            const uint64_t e = ld_dev(mine + tid);
            if ((uint32_t)(e >> 32) == tag) {
              got = (uint32_t)e;
              have = true;
            }
          }
          if (__ballot(!have) == 0ull) break;
          if (wall_clock64() > deadline) {
            to = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      if (__syncthreads_or(to)) {
        failed = true;
        break;
      }
      acc += got;
    }
  }
  sink[(size_t)blk * kCT + tid] = __uint_as_float(acc);
  if (tid == 0) {
    if (failed) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    st_dev(epochs + blk, epoch + 1u);
  }
}

}  // namespace

hipError_t launch_stream_phases(const void* buf, int64_t bytes, int phases, int handoffs,
                                uint64_t* words, uint32_t* epochs, float* sink, int32_t* err,
                                int64_t timeout_ticks, hipStream_t s) {
  hipLaunchKernelGGL(stream_phases_kernel, dim3(kCG), dim3(kCT), 0, s,
                     static_cast<const uint4*>(buf), bytes / 16, phases, handoffs, words, epochs,
                     sink, err, timeout_ticks);
  return hipGetLastError();
}

}  // namespace moe
