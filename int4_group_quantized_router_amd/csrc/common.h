// Host-side helpers shared by every translation unit of libmoe.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "../../include/moe.h"

namespace moe {

// Records a formatted message for moe_last_error() and returns `code`.
int32_t fail(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Fills `out`; false (with the error set) if the shape is unsupported.
bool blob_layout(const moe_qshape& s, moe_blob_layout* out);

// Device-side copy of the few layout numbers the kernels need.
struct QLayout {
  int64_t q_off[3];
  int64_t sb_off[3];
  int64_t stride;
};

inline QLayout to_qlayout(const moe_blob_layout& l) {
  QLayout q;
  for (int i = 0; i < 3; ++i) {
    q.q_off[i] = l.q_off[i];
    q.sb_off[i] = l.sb_off[i];
  }
  q.stride = l.stride;
  return q;
}

// Slot pool internals the layer uses (pool.cpp): the device table row of
// `layer` ((expert) -> slot address, NULL when not resident), and the wait a
// stream needs before a kernel on it may read that table.
const uint8_t* const* pool_device_table(const slotpool* p, int32_t layer);
int32_t pool_before_lookup(slotpool* p, hipStream_t stream);
// MOE_OK if a layer with `experts` routed experts at store layer
// `layer_index`, blob stride `stride`, can draw on pool p's store; else
// MOE_E_INVAL with the mismatch in the error message.
int32_t pool_check_layer(const slotpool* p, int32_t layer_index, int32_t experts, int64_t stride);
// The policy updates of nl layer calls that found every expert resident
// (each acquire + release of experts[l*k .. l*k+k) of layers[l], all hits,
// in order), with one release point recorded on `stream` for all of them
// now.  The updates themselves are held in the pool and applied, in order,
// by pool_apply_pending, which every public pool call runs first: nothing
// can observe or change the policy before they are in.
int32_t pool_defer_hits(slotpool* p, const int32_t* layers, const int32_t* experts, int32_t nl,
                        int32_t k, hipStream_t stream);
int32_t pool_apply_pending(slotpool* p);

}  // namespace moe

#define MOE_HIP_TRY(expr)                                                        \
  do {                                                                           \
    hipError_t moe_err_ = (expr);                                                \
    if (moe_err_ != hipSuccess)                                                  \
      return ::moe::fail(MOE_E_HIP, "%s failed: %s (%s:%d)", #expr,              \
                         hipGetErrorString(moe_err_), __FILE__, __LINE__);       \
  } while (0)

#define MOE_REQUIRE(cond, ...)                                                   \
  do {                                                                           \
    if (!(cond)) return ::moe::fail(MOE_E_INVAL, __VA_ARGS__);                   \
  } while (0)
