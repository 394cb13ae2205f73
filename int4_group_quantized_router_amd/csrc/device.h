// Device-side helpers for the gfx950 kernels (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace moe {
namespace dev {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// c + a.lo*b.lo + a.hi*b.hi with bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// v_perm_b32: byte i of the result is byte sel[i] of {hi:lo} (0-3 from lo, 4-7 from hi).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64);
// every lane of a group ends with the same value (butterfly; addition order
// is the same for every lane up to commutativity, so the bits agree).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

template <int WIDTH>
__device__ __forceinline__ float group_sum_c(float v) {
#pragma unroll
  for (int off = WIDTH >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// 16-byte global load.
__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

}  // namespace dev
}  // namespace moe
