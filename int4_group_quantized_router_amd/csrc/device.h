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

namespace moe {
namespace dev {

// ---- device-coherent hand-off between workgroups (possibly on different
// XCDs, whose L2 caches are not coherent with each other).  Stores write
// through to the device coherence point and loads read from it, so no full
// L2 write-back/invalidate is needed; wait_stores() makes this thread's
// earlier stores complete before a later signal.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_dev(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ uint32_t ticket(uint32_t* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Order-preserving map float -> uint32 (larger float, larger key); 0 is
// below every finite float's key.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0: equal floats, equal keys
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// Top-k of up to 64*VPL logits held by one wave (value i of lane l is
// expert l + 64 i, invalid entries key 0), ordered by (logit desc, index
// asc).  k-th largest key by a 32-step bitwise search with ballot counts,
// then the k winners (ties at the threshold: lowest indices) are compacted
// to LDS and ranked.  Results: sel_e[j], sel_v[j] for j < k (LDS, wave's own
// scratch of >= k entries each).  All lanes must call it.
template <int VPL>
__device__ void wave_topk(const float* v, const uint32_t* key, int k, int* tmp_e, float* tmp_v,
                          int* sel_e, float* sel_v) {
  const int lane = threadIdx.x & 63;
  uint32_t thr = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = thr | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) cnt += __popcll(__ballot(key[i] >= cand));
    if (cnt >= k) thr = cand;
  }
  int n_gt = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) n_gt += __popcll(__ballot(key[i] > thr));
  int need_eq = k - n_gt;  // winners taken among keys == thr, lowest index first
  const uint64_t below = lanes_below();
  int base = 0, eq_before = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const uint64_t eq = __ballot(key[i] == thr);
    const bool is_eq = key[i] == thr;
    const int eq_rank = eq_before + __popcll(eq & below);
    const bool sel = key[i] > thr || (is_eq && eq_rank < need_eq);
    const uint64_t sm = __ballot(sel);
    if (sel) {
      const int pos = base + __popcll(sm & below);
      tmp_e[pos] = lane + 64 * i;
      tmp_v[pos] = v[i];
    }
    base += __popcll(sm);
    eq_before += __popcll(eq);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  if (lane < k) {
    const int e = tmp_e[lane];
    const float x = tmp_v[lane];
    const uint32_t kx = order_key(x);
    int r = 0;
    for (int m = 0; m < k; ++m) {
      const uint32_t km = order_key(tmp_v[m]);
      const int em = tmp_e[m];
      r += (km > kx) || (km == kx && em < e);
    }
    sel_e[r] = e;
    sel_v[r] = x;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

}  // namespace dev
}  // namespace moe
