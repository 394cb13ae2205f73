// Building blocks of the dequant-GEMV kernels (decode path), shared by the
// per-launch kernels and the persistent per-token kernel.
//
// Work unit = one 16-byte chunk of a weight row per lane (32 int4 or 16 int8
// values).  int4 -> bf16 pairs without converts: (w >> 4j) & 0x000F000F |
// 0x43004300 is the pair (128 + q_j, 128 + q_{j+4}); v_dot2_f32_bf16 takes it
// against the matching x pair; the 128 offset folds into the bias:
// sum (s q + b) x = s D + (b - 128 s) X with D = sum (128 + q) x, X = sum x.
// int8 fields convert exactly with v_cvt_f32_ubyte.
#pragma once

#include "device.h"

namespace moe {
namespace dev {

template <int BITS>
struct Fmt {
  static constexpr int kEpc = 128 / BITS;      // values per 16-byte chunk
  static constexpr int kPairs = kEpc / 2;      // bf16x2 registers per chunk
  static constexpr int kPerWord = 32 / BITS;   // values per uint32 word
};


// Position of intermediate index i inside h: for int4 the 8 values of each
// aligned block are stored as pairs (i, i+4) so the down kernel's lanes read
// ready-made bf16x2 operands matching the nibble pairing.
template <int BITS>
__device__ __forceinline__ int h_pos(int i) {
  if (BITS == 8) return i;
  const int j = i & 7;
  return (i & ~7) + (j < 4 ? 2 * j : 2 * (j - 4) + 1);
}

// Build the bf16x2 operand registers of one chunk from 16-byte loads of a
// bf16 vector in natural order (int4 pairing needs a byte permute).
template <int BITS>
__device__ __forceinline__ void pair_natural(const uint4* src, uint32_t* xp, float& xsum) {
  constexpr int P = Fmt<BITS>::kPairs;
  uint32_t d[P];
#pragma unroll
  for (int v = 0; v < P / 4; ++v) {
    const uint4 q = src[v];
    d[4 * v + 0] = q.x;
    d[4 * v + 1] = q.y;
    d[4 * v + 2] = q.z;
    d[4 * v + 3] = q.w;
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < P; ++i) s += bf16_lo(d[i]) + bf16_hi(d[i]);
  xsum = s;
  if (BITS == 8) {
#pragma unroll
    for (int i = 0; i < P; ++i) xp[i] = d[i];
  } else {
    // word m covers values 8m..8m+7 = dwords 4m..4m+3 (two values each)
#pragma unroll
    for (int m = 0; m < P / 4; ++m) {
      const uint32_t d0 = d[4 * m], d1 = d[4 * m + 1], d2 = d[4 * m + 2], d3 = d[4 * m + 3];
      xp[4 * m + 0] = perm(d2, d0, 0x05040100u);  // (v0, v4)
      xp[4 * m + 1] = perm(d2, d0, 0x07060302u);  // (v1, v5)
      xp[4 * m + 2] = perm(d3, d1, 0x05040100u);  // (v2, v6)
      xp[4 * m + 3] = perm(d3, d1, 0x07060302u);  // (v3, v7)
    }
  }
}

// (w & m) | c as one VALU op.  gfx950's three-operand encoding takes no
// 32-bit literal, so left to itself the compiler splits this into an AND and
// an OR with literals; here m sits in an SGPR and c in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(m), "v"(c));
  return r;
}

// sum over the chunk of (128 + q) * x (int4) or q * x (int8), f32.
template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint4 w4, const uint32_t* xp) {
  const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
  float d0 = 0.f, d1 = 0.f;
  if (BITS == 4) {
    constexpr uint32_t M = 0x000F000Fu, C = 0x43004300u;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      d0 = dot2(and_or(w[m], M, C), xp[4 * m + 0], d0);
      d1 = dot2(and_or(w[m] >> 4, M, C), xp[4 * m + 1], d1);
      d0 = dot2(and_or(w[m] >> 8, M, C), xp[4 * m + 2], d0);
      d1 = dot2(and_or(w[m] >> 12, M, C), xp[4 * m + 3], d1);
    }
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t f0 = __float_as_uint((float)(w[m] & 0xFFu));
      const uint32_t f1 = __float_as_uint((float)((w[m] >> 8) & 0xFFu));
      const uint32_t f2 = __float_as_uint((float)((w[m] >> 16) & 0xFFu));
      const uint32_t f3 = __float_as_uint((float)(w[m] >> 24));
      d0 = dot2(perm(f1, f0, 0x07060302u), xp[2 * m + 0], d0);
      d1 = dot2(perm(f3, f2, 0x07060302u), xp[2 * m + 1], d1);
    }
  }
  return d0 + d1;
}

// Add one chunk's dequantised dot product: s*D + (b - z*s)*X.
template <int BITS>
__device__ __forceinline__ float chunk_term(float acc, uint32_t sb, float D, float X) {
  const float s = bf16_lo(sb), b = bf16_hi(sb);
  const float bb = (BITS == 4) ? fmaf(-128.0f, s, b) : b;
  acc = fmaf(s, D, acc);
  return fmaf(bb, X, acc);
}

}  // namespace dev
}  // namespace moe
