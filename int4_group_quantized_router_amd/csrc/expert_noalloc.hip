// moe_expert_forward for callers that cannot allocate device memory (code
// under stream capture, tight serving loops, harnesses that forbid
// hipMalloc): the activations h live in a fixed array of the library instead
// of stream-ordered scratch.  The kernels are those of moe_expert_forward.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// Largest T * inter of a call: 8 tokens of the largest supported
// intermediate size (2048: 64 chunks of 32 int4 values).
constexpr int kNoAllocH = MOE_NOALLOC_MAX_H;

// h of the call in progress, bf16 [T][inter].  One copy per device, held
// until the process ends; every call on a device reuses it, so calls that
// overlap on one device (different streams, or threads) race.  gate/up
// writes every element a call's down projection reads, so nothing needs to
// start at zero.
static __device__ __align__(256) uint16_t scratch[kNoAllocH];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
uint16_t* g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per
// device, with that device current).  The host-side name of the array is
// not a device address and is never passed to a kernel.
int32_t scratch_ptr(uint16_t** out) {
  int dev = 0;
  MOE_HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_E_INVAL, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    MOE_HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(MOE_E_HIP, "hipGetSymbolAddress returned NULL");
    g_ptr[dev] = static_cast<uint16_t*>(p);
  }
  *out = g_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int32_t moe_expert_forward_noalloc(const uint16_t* x, int32_t T,
                                              const moe_qshape* shape, const void* blob,
                                              const float* coef, float* y_accum,
                                              hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(x && shape && blob && coef && y_accum, "null argument");
  MOE_REQUIRE(T >= 1 && T <= MOE_MAX_DECODE_T, "T must be in [1, %d]", MOE_MAX_DECODE_T);
  moe_blob_layout lay;
  if (!blob_layout(*shape, &lay)) return MOE_E_INVAL;
  MOE_REQUIRE(shape->hidden % 256 == 0 && shape->hidden <= 2048 &&
                  decode_shape_supported(shape->hidden, shape->inter, shape->inter, shape->bits),
              "unsupported expert shape H=%d I=%d bits=%d", shape->hidden, shape->inter,
              shape->bits);
  MOE_REQUIRE((int64_t)T * shape->inter <= kNoAllocH,
              "T * inter = %lld exceeds the fixed activation buffer (%d values)",
              (long long)T * shape->inter, kNoAllocH);
  uint16_t* h = nullptr;
  const int32_t st = scratch_ptr(&h);
  if (st != MOE_OK) return st;
  DecodeArgs d{};
  d.x = x;
  d.T = T;
  d.H = shape->hidden;
  d.I = shape->inter;
  d.Is = shape->inter;
  d.k = 0;
  d.bits = shape->bits;
  d.n_slot_max = 0;
  d.ls = to_qlayout(lay);
  d.lr = d.ls;
  d.shared_blob = static_cast<const uint8_t*>(blob);
  d.h = h;
  d.hI = shape->inter;
  d.gate = coef;
  d.y_f32 = y_accum;
  d.accumulate = 1;
  MOE_HIP_TRY(launch_gate_up(d, stream));
  MOE_HIP_TRY(launch_down(d, stream));
  return MOE_OK;
}
