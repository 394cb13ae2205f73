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

// Affine dequantisation s * q + b of packed integer fields without integer
// to float conversions.  A field of up to 8 bits placed in the low bits of a
// 16-bit half is an f16 subnormal, q * 2^-24 (f16 subnormals are kept: the
// kernels run with f16/f64 denormals enabled); v_fma_mix_f32 widens it
// exactly and computes fma(s * 2^24, q * 2^-24, b) = fma(s, q, b) with one
// rounding, bit for bit what fmaf(s, (float)q, b) gives.  A field at bits
// 4..7 of a half is q * 2^-20, taken with s * 2^20.
__device__ __forceinline__ float fma_mix_lo(float s, uint32_t h, float c) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,1,0]" : "=v"(d) : "v"(s), "v"(h), "v"(c));
  return d;
}
__device__ __forceinline__ float fma_mix_hi(float s, uint32_t h, float c) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
      : "=v"(d)
      : "v"(s), "v"(h), "v"(c));
  return d;
}
__device__ __forceinline__ uint32_t and_lit(uint32_t w, uint32_t m) { return w & m; }

// The 8 int4 fields of w (field i at bits 4i..4i+3), dequantised: f[i] =
// fmaf(s, q_i, b).  17 VALU operations.
__device__ __forceinline__ void dequant8_int4(uint32_t w, float s, float b, float* f) {
  const float s24 = s * 16777216.0f, s20 = s * 1048576.0f;  // exact: powers of two
  const uint32_t w8 = w >> 8;
  const uint32_t a0 = w & 0x000F000Fu, a1 = w & 0x00F000F0u;    // fields 0, 4 / 1, 5
  const uint32_t a2 = w8 & 0x000F000Fu, a3 = w8 & 0x00F000F0u;  // fields 2, 6 / 3, 7
  f[0] = fma_mix_lo(s24, a0, b);
  f[4] = fma_mix_hi(s24, a0, b);
  f[1] = fma_mix_lo(s20, a1, b);
  f[5] = fma_mix_hi(s20, a1, b);
  f[2] = fma_mix_lo(s24, a2, b);
  f[6] = fma_mix_hi(s24, a2, b);
  f[3] = fma_mix_lo(s20, a3, b);
  f[7] = fma_mix_hi(s20, a3, b);
}

// The 4 int8 fields of w (field i at bits 8i..8i+7): f[i] = fmaf(s, q_i, b).
__device__ __forceinline__ void dequant4_int8(uint32_t w, float s, float b, float* f) {
  const float s24 = s * 16777216.0f;
  const uint32_t a0 = w & 0x00FF00FFu, a1 = (w >> 8) & 0x00FF00FFu;  // fields 0, 2 / 1, 3
  f[0] = fma_mix_lo(s24, a0, b);
  f[2] = fma_mix_hi(s24, a0, b);
  f[1] = fma_mix_lo(s24, a1, b);
  f[3] = fma_mix_hi(s24, a1, b);
}

// v_perm_b32: byte i of the result is byte sel[i] of {hi:lo} (0-3 from lo, 4-7 from hi).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Cross-lane moves without LDS: DPP (data-parallel primitives) and readlane.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over aligned groups of `width` lanes (a power of two <= 64); every
// lane of a group ends with the same bits.  Inside 16 lanes a butterfly of
// DPP adds: lane^1, lane^2 (quad permutes), then the 8- and 16-lane mirrors,
// which pair lanes of the two halves once the halves are uniform.  The four
// 16-lane sums r0..r3 then meet through readlane as r0+r1 (width 32) or
// (r0+r1)+(r2+r3) (width 64).  Every wave-level reduction of the decode
// kernels uses this one order.  All lanes must be active.
__device__ __forceinline__ float group_sum(float v, int width) {
  if (width >= 2) v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  if (width >= 4) v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  if (width >= 8) v += dpp_f32<0x141>(v);  // row_half_mirror
  if (width >= 16) v += dpp_f32<0x140>(v); // row_mirror
  if (width >= 32) {
    const float r0 = readlane_f32(v, 0), r1 = readlane_f32(v, 16);
    const float r2 = readlane_f32(v, 32), r3 = readlane_f32(v, 48);
    if (width == 32)
      v = (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
    else
      v = (r0 + r1) + (r2 + r3);
  }
  return v;
}

// Loads through global-address-space pointers.  A pointer the compiler
// cannot prove global (read from a table, selected at run time) would be
// loaded with FLAT instructions, which also count against the LDS wait
// counter: every later LDS wait would then also wait for the HBM load.
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

// 16-byte global load as a native vector (stays in registers as-is).
__device__ __forceinline__ u32x4_v ld16v(const void* p) {
  return *(__attribute__((address_space(1))) const u32x4_v*)p;
}

// 16-byte global load.
__device__ __forceinline__ uint4 ld16(const void* p) {
  const u32x4_v v = *(__attribute__((address_space(1))) const u32x4_v*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ldf4(const void* p) {
  const f32x4_v v = *(__attribute__((address_space(1))) const f32x4_v*)p;
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ldu32(const void* p) {
  return *(__attribute__((address_space(1))) const uint32_t*)p;
}
__device__ __forceinline__ float ldf(const void* p) {
  return *(__attribute__((address_space(1))) const float*)p;
}

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct-to-LDS loads (global_load_lds): lane i's 16 (4) bytes at src go to
// LDS address m0 + 16 i (4 i); m0 must be wave-uniform.  Issued as plain
// instructions, they are invisible to the compiler's wait-count bookkeeping:
// the caller waits for them with wait_vm_n before reading the LDS they
// write.  Vector loads complete in issue order, so waiting until at most N
// loads are outstanding completes every load older than the last N issued.
__device__ __forceinline__ void dma16(const void* src, uint32_t m0) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t m0) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
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
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Lanes set in a wave mask, as a 32-bit count (two 32-bit popcounts keep
// later comparisons of the count on the scalar unit).
__device__ __forceinline__ uint32_t count_lanes(uint64_t m) {
  return (uint32_t)__builtin_popcount((uint32_t)m) + (uint32_t)__builtin_popcount((uint32_t)(m >> 32));
}

__device__ __forceinline__ uint64_t lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// Selection inside one wave: among the keys held one per lane-slot (slot i
// of lane l holds key[i] with index idx_of(l, i), invalid entries key 0),
// the k best by (key desc, index asc), given that the index order equals
// the (i, lane) order.  A bitwise search from the top bit finds a threshold
// key t with at least k keys >= t, stopping early as soon as exactly k are
// (then those k are the answer); otherwise it ends at the k-th largest key
// and ties at t go to the lowest indices.  The winners are compacted to
// tmp (k entries) and ranked by broadcasting each one's key (readlane).
template <int VPL, class IdxOf>
__device__ void select_k(const float* v, const uint32_t* key, int k, IdxOf idx_of, int* tmp_e,
                         float* tmp_v, int* sel_e, float* sel_v) {
  const int lane = threadIdx.x & 63;
  // (thr, cand and cnt are wave-uniform; readfirstlane keeps them scalar)
  uint32_t thr = 0;
  const uint32_t ku = (uint32_t)__builtin_amdgcn_readfirstlane(k);
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = (uint32_t)__builtin_amdgcn_readfirstlane(thr | (1u << b));
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) cnt += count_lanes(__ballot(key[i] >= cand));
    if (cnt >= ku) {
      thr = cand;
      if (cnt == ku) break;
    }
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
      tmp_e[pos] = idx_of(lane, i);
      tmp_v[pos] = v[i];
    }
    base += __popcll(sm);
    eq_before += __popcll(eq);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int e = lane < k ? tmp_e[lane] : 0;
  const float x = lane < k ? tmp_v[lane] : 0.f;
  const uint32_t kx = order_key(x);
  int r = 0;
#pragma unroll
  for (int m = 0; m < MOE_MAX_TOPK; ++m) {
    if (m < k) {
      const uint32_t km = (uint32_t)__builtin_amdgcn_readlane((int)kx, m);
      const int em = __builtin_amdgcn_readlane(e, m);
      r += (km > kx) || (km == kx && em < e);
    }
  }
  if (lane < k) {
    sel_e[r] = e;
    sel_v[r] = x;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Top-k of up to 64*VPL logits held by one wave (value i of lane l is
// expert l + 64 i, invalid entries key 0), ordered by (logit desc, index
// asc).  Results: sel_e[j], sel_v[j] for j < k (LDS).  tmp_e / tmp_v / tmp_k:
// the wave's own LDS scratch of >= 64 entries each.  All lanes must call it.
//
// With several keys per lane the selection runs on a pruned set: the k-th
// largest of the 64 per-lane maxima, t1, is found first (one key per lane,
// bitwise search); at least k lanes hold a key >= t1, so every one of the k
// best keys is >= t1.  The keys >= t1 -- usually few more than k -- are
// compacted one per lane with their expert index, and each one's place is
// its rank among them: the number of candidates whose (key, -index) is
// larger, counted by broadcasting each candidate in turn (one 64-bit
// comparison per candidate).  Ranks are distinct, so the lanes of rank < k
// write the result in order.  If more than 64 keys are >= t1 (many ties),
// the bitwise selection runs on all keys instead.  Either way the result is
// the unique top-k by (key desc, index asc).
template <int VPL>
__device__ void wave_topk(const float* v, const uint32_t* key, int k, int* tmp_e, float* tmp_v,
                          uint32_t* tmp_k, int* sel_e, float* sel_v) {
  auto natural = [](int l, int i) { return l + 64 * i; };
  if (VPL == 1) {
    select_k<VPL>(v, key, k, natural, tmp_e, tmp_v, sel_e, sel_v);
    return;
  }
  const int lane = threadIdx.x & 63;
  uint32_t mx = key[0];
#pragma unroll
  for (int i = 1; i < VPL; ++i) mx = mx > key[i] ? mx : key[i];
  uint32_t t1 = 0;
  const uint32_t ku = (uint32_t)__builtin_amdgcn_readfirstlane(k);
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = (uint32_t)__builtin_amdgcn_readfirstlane(t1 | (1u << b));
    const uint32_t cnt = count_lanes(__ballot(mx >= cand));
    if (cnt >= ku) {
      t1 = cand;
      if (cnt == ku) break;
    }
  }
  // candidates: keys >= t1 (t1 > 0 whenever any lane holds a valid key; the
  // floor of 1 keeps invalid entries out).  Their masks first (the total
  // decides the path), then the writes.
  const uint32_t tlo = t1 > 0u ? t1 : 1u;
  uint64_t cm[VPL];
  uint32_t n = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    cm[i] = __ballot(key[i] >= tlo);
    n += count_lanes(cm[i]);
  }
  n = (uint32_t)__builtin_amdgcn_readfirstlane(n);
  if (n > 64u || n < ku) {  // wave-uniform
    select_k<VPL>(v, key, k, natural, tmp_e, tmp_v, sel_e, sel_v);
    return;
  }
  uint32_t base = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    if (key[i] >= tlo) {
      const uint32_t pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(cm[i] >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)cm[i], 0u));
      tmp_k[pos] = key[i];
      tmp_e[pos] = lane + 64 * i;
    }
    base += count_lanes(cm[i]);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const bool have = (uint32_t)lane < n;
  const uint32_t ck = have ? tmp_k[lane] : 0u;
  const int ce = have ? tmp_e[lane] : 0;
  // the value back from its key (the inverse of order_key)
  const float cv = __uint_as_float((ck & 0x80000000u) ? (ck & 0x7FFFFFFFu) : ~ck);
  // (key, -index) as one 64-bit order: a larger key, then a lower index, wins
  const uint32_t nce = ~(uint32_t)ce;
  const uint64_t mine = ((uint64_t)ck << 32) | nce;
  uint32_t r = 0;
  // lanes >= n hold key 0, below every candidate: looping over them in
  // steps of 4 adds nothing to a candidate's rank
  const uint32_t n4 = (n + 3u) & ~3u;
  for (uint32_t m = 0; m < n4; m += 4) {
#pragma unroll
    for (uint32_t u = 0; u < 4; ++u) {
      const uint32_t km = (uint32_t)__builtin_amdgcn_readlane((int)ck, (int)(m + u));
      const uint32_t em = (uint32_t)__builtin_amdgcn_readlane((int)nce, (int)(m + u));
      r += (((uint64_t)km << 32) | em) > mine ? 1u : 0u;
    }
  }
  if (have && r < ku) {
    sel_e[r] = ce;
    sel_v[r] = cv;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

}  // namespace dev
}  // namespace moe
