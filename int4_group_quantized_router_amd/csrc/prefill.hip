// Many-token (prefill) path of the MoE layer on bf16 MFMA.
//
// The pages' decode loop is a per-token GEMV; a commenter points at prefill
// as the bottleneck ([digest] "Community Reactions"; [lens] community
// section).  With thousands of tokens each expert sees ~T*k/E rows, so the
// expert work becomes a dense contraction -- the one place on this path
// where matrix cores pay:
//
//   1. router: logits = x Wr^T + rb.  Wr is held as three bf16 planes with
//      hi + mid + lo == Wr exactly (8 + 8 + 8 significant bits), so bf16
//      MFMA with f32 accumulation computes exactly the products of the f32
//      router; each 64-wide K group is accumulated separately and then added
//      to the running total, which bounds the summation depth.
//   2. sort: per-expert counts (atomic integer adds in the top-k), a scan to
//      row offsets and a tile list, then a per-expert ballot compaction that
//      keeps token order (stable).  The shared expert is one more group whose
//      rows are all tokens.
//   3. gate/up grouped GEMM: one 128-row tile of an expert's rows x 64
//      intermediate columns of BOTH gate and up per workgroup; the 128 x 64
//      weight tile of each K group (one quantisation group) is dequantised
//      once by the workgroup into LDS as bf16 (s*q + b, then round to nearest
//      even) and read by four waves as MFMA 32x32x16 operands; token rows are
//      gathered straight from x in HBM; epilogue h = bf16(silu(g) * u).
//   4. down grouped GEMM: 128 rows x 128 output columns, same scheme; f32
//      outputs per (token, choice) row.
//   5. combine: y[t] = sum_j w[t,j] y_j + sigma_t y_shared, j in order.
//
// MFMA K order: for MFMA step s of a 64-wide group, lanes 0-31 supply
// K = 8s..8s+7 and lanes 32-63 supply K = 32+8s..32+8s+7, so each lane's A and
// B operands for the four steps are 64 contiguous bytes.  Both operands use
// the same order, so the product is unchanged.
//
// Blocks are numbered so that consecutive work items land on the same XCD
// (the dispatcher deals blocks round-robin over the 8 XCDs): the 16 or 8
// column tiles of one row tile then share its rows in that XCD's L2.
#include <algorithm>

#include "device.h"
#include "kernels.h"

namespace moe {
namespace {

using namespace dev;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int BM = kPrefillBM;
constexpr int KG = 64;                // K per step = one quantisation group
constexpr int kLdsRow = KG * 2 + 16;  // bytes per weight row in LDS (padded)

__device__ __forceinline__ f32x16_t mfma(const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_v r;
  r.x = (__bf16)lo;
  r.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// (tile, column tile) of this block.  Blocks are dealt round-robin to the 8
// XCDs; tile i runs on XCD i % 8 with all its column tiles, so the column
// tiles share the tile's rows in one L2 and the real tiles (a prefix of the
// padded grid's tile range) spread evenly over the XCDs.
__device__ __forceinline__ void tile_of_block(int nt_per_tile, int* tile, int* nt) {
  const int b = blockIdx.x;
  const int xcd = b & 7, j = b >> 3;
  *tile = (j / nt_per_tile) * 8 + xcd;
  *nt = j % nt_per_tile;
}

// Dequantise one 16-byte chunk of packed weights to bf16 (round to nearest
// even of the exact f32 value s*q + b) and store it in natural order.
template <int BITS>
__device__ __forceinline__ void dequant_chunk(const uint4 raw, uint32_t sb, uint8_t* dst) {
  const float s = bf16_lo(sb), b = bf16_hi(sb);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  if (BITS == 4) {
    uint32_t o[16];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // nibbles to bytes; the asm keeps the optimiser from folding the masks
      // into per-value bit-field extracts, so each byte converts with one
      // v_cvt_f32_ubyte{0..3}
      uint32_t lo, hi;
      asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(w[m]));
      asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(hi) : "v"(w[m] >> 4));
#pragma unroll
      for (int i = 0; i < 4; ++i)  // values 8m+2i (low nibble of byte i) and 8m+2i+1
        o[4 * m + i] = pack_bf16(fmaf(s, (float)((lo >> (8 * i)) & 0xFFu), b),
                                 fmaf(s, (float)((hi >> (8 * i)) & 0xFFu), b));
    }
    uint4* d = reinterpret_cast<uint4*>(dst);
#pragma unroll
    for (int v = 0; v < 4; ++v) d[v] = make_uint4(o[4 * v], o[4 * v + 1], o[4 * v + 2], o[4 * v + 3]);
  } else {
    uint32_t o[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        o[2 * m + i] = pack_bf16(fmaf(s, (float)((w[m] >> (16 * i)) & 0xFFu), b),
                                 fmaf(s, (float)((w[m] >> (16 * i + 8)) & 0xFFu), b));
    }
    uint4* d = reinterpret_cast<uint4*>(dst);
    d[0] = make_uint4(o[0], o[1], o[2], o[3]);
    d[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

// One packed word -> bf16 values in natural order: 8 (int4, as a uint4) or
// 4 (int8, low half of the uint4).
template <int BITS>
__device__ __forceinline__ uint4 dequant_word(uint32_t w, float s, float b) {
  if (BITS == 4) {
    uint32_t lo, hi;
    asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(w));
    asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(hi) : "v"(w >> 4));
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = pack_bf16(fmaf(s, (float)((lo >> (8 * i)) & 0xFFu), b),
                       fmaf(s, (float)((hi >> (8 * i)) & 0xFFu), b));
    return make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    const uint32_t o0 = pack_bf16(fmaf(s, (float)(w & 0xFFu), b), fmaf(s, (float)((w >> 8) & 0xFFu), b));
    const uint32_t o1 = pack_bf16(fmaf(s, (float)((w >> 16) & 0xFFu), b), fmaf(s, (float)(w >> 24), b));
    return make_uint4(o0, o1, 0u, 0u);
  }
}

__device__ __forceinline__ const uint8_t* group_blob(const PrefillArgs& a, int g) {
  if (g == a.E) return a.shared_blob;
  return a.routed_base ? a.routed_base + (int64_t)g * a.stride : a.slot_ptrs[g];
}

// ------------------------------------------------------------- router

__global__ __launch_bounds__(kThreads) void split_router_kernel(const float* Wr, const float* wsg,
                                                                int E, int H, uint16_t* wr3) {
  const int64_t n = (int64_t)(E + 1) * H;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const int64_t e = i / H;
  const float W = e < E ? Wr[i] : (wsg ? wsg[i - (int64_t)E * H] : 0.f);
  const uint32_t hi = f32_to_bf16(W);
  const float r1 = W - bf16_to_f32(hi);
  const uint32_t mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);
  wr3[i] = (uint16_t)hi;
  wr3[n + i] = (uint16_t)mid;
  wr3[2 * n + i] = (uint16_t)f32_to_bf16(r2);
}

// logits for a 128-token x 128-expert tile; row E of the planes is wsg
// (its result, wsg . x, goes to sigma_raw).
__global__ __launch_bounds__(kThreads, 2) void router_gemm_kernel(
    const uint16_t* x, int T, int H, const uint16_t* wr3, const float* bias, int E, int has_wsg,
    float* logits, float* sigma_raw) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mh = wave >> 1, nh = wave & 1, kh = lane >> 5, l32 = lane & 31;
  const int t0 = blockIdx.x * BM, e0 = blockIdx.y * BM;
  const int rows = E + (has_wsg ? 1 : 0);
  const int64_t plane = (int64_t)(E + 1) * H;
  const uint16_t* arow[2];
  bool av[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int t = t0 + mh * 64 + rb * 32 + l32;
    av[rb] = t < T;
    arow[rb] = x + (size_t)(av[rb] ? t : 0) * H + kh * 32;
  }
  const uint16_t* brow[2];
  bool bv[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int e = e0 + nh * 64 + cb * 32 + l32;
    bv[cb] = e < rows;
    brow[cb] = wr3 + (size_t)(bv[cb] ? e : 0) * H + kh * 32;
  }
  f32x16_t tot[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) tot[i][j] = f32x16_t{};
  // out-of-range rows / experts read row 0 (clamped above) and are never stored
  for (int kg = 0; kg < H / KG; ++kg) {
    uint4 af[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int s = 0; s < 4; ++s) af[rb][s] = ld16(arow[rb] + kg * KG + s * 8);
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      uint4 bf[2][4];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          bf[cb][s] = ld16(brow[cb] + p * plane + kg * KG + s * 8);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mfma(af[rb][s], bf[cb][s], acc[rb][cb]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) tot[i][j] += acc[i][j];
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = t0 + mh * 64 + rb * 32 + (v >> 2) * 8 + kh * 4 + (v & 3);
        const int e = e0 + nh * 64 + cb * 32 + l32;
        if (t >= T || e >= rows) continue;
        if (e < E)
          logits[(size_t)t * E + e] = tot[rb][cb][v] + (bias ? bias[e] : 0.f);
        else
          sigma_raw[t] = tot[rb][cb][v];
      }
}

// --------------------------------------------------------------- sort

// One block: group sizes (group E = shared expert = all tokens) -> row
// offsets and the tile list; resets the counts for the next call.
__global__ __launch_bounds__(kThreads) void prefill_scan_kernel(PrefillArgs a) {
  __shared__ int s_rows[1026];
  __shared__ int s_tiles[1026];
  const int G = a.E + 1;
  for (int g = threadIdx.x; g < G; g += kThreads) {
    const int c = g < a.E ? a.counts[g] : a.T;
    s_rows[g] = c;
    s_tiles[g] = (c + BM - 1) / BM;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int r = 0, tl = 0;
    for (int g = 0; g < G; ++g) {
      const int c = s_rows[g], n = s_tiles[g];
      s_rows[g] = r;
      s_tiles[g] = tl;
      r += c;
      tl += n;
    }
    s_rows[G] = r;
    s_tiles[G] = tl;
    a.row_off[G] = r;
    *a.n_tiles = tl;
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += kThreads) {
    a.row_off[g] = s_rows[g];
    const int n = s_tiles[g + 1] - s_tiles[g];
    for (int i = 0; i < n; ++i) {
      if (s_tiles[g] + i < a.max_tiles) {
        a.tile_group[s_tiles[g] + i] = g;
        a.tile_m0[s_tiles[g] + i] = i * BM;
      }
    }
    if (g < a.E) a.counts[g] = 0;
  }
}

// One block per group: the group's rows in token order (stable).
__global__ __launch_bounds__(kThreads) void prefill_compact_kernel(PrefillArgs a) {
  __shared__ int s_wcnt[kThreads / kWave];
  const int e = blockIdx.x;
  const int base = a.row_off[e];
  if (e == a.E) {
    for (int t = threadIdx.x; t < a.T; t += kThreads) a.perm_tok[base + t] = t;
    return;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int P = a.T * a.k;
  int running = 0;
  for (int p0 = 0; p0 < P; p0 += kThreads) {
    const int p = p0 + threadIdx.x;
    const bool match = p < P && a.idx[p] == e;
    const unsigned long long bal = __ballot(match);
    if (lane == 0) s_wcnt[wave] = __popcll(bal);
    __syncthreads();
    int before = running;
    for (int w = 0; w < wave; ++w) before += s_wcnt[w];
    if (match) {
      const int pos = base + before + __popcll(bal & lanes_below());
      a.perm_tok[pos] = p / a.k;
      a.inv[p] = pos;
    }
    for (int w = 0; w < kThreads / kWave; ++w) running += s_wcnt[w];
    __syncthreads();
  }
}

// ------------------------------------------------------ grouped GEMMs
//
// One kernel for both products.  Workgroup tile: 128 rows of one group x 256
// weight rows -- for gate/up, 128 intermediate columns of gate and the same
// 128 of up (so h = silu(g) * u is finished in registers); for down, 256
// output columns.  Per 64-wide K group the workgroup stages the 128 A rows
// (gathered token rows of x, or rows of h) and the 256 dequantised weight
// rows in LDS (double-buffered), with global loads issued two groups ahead
// through a ring of two register sets.  Eight waves (two per SIMD, so one
// wave's dequantisation overlaps the other's MFMAs); each owns a 64-row x
// 64-weight-row block = 2 x 2 MFMA 32x32x16 tiles, 64 f32 accumulators.

constexpr int BN = 256;                    // weight rows per tile
constexpr int kGemmThreads = 512;          // 8 waves
constexpr int kLdsA = BM * kLdsRow;        // bytes of one A stage
constexpr int kLdsB = BN * kLdsRow;        // bytes of one B stage

template <int BITS>
struct GemmRegs {
  static constexpr int CB = BN * (KG * BITS / 8) / 16 / kGemmThreads;  // B chunks per thread
  uint4 a[2];        // A: 2 x 16 bytes per thread per K group
  uint4 b[CB];       // B: packed weights
  uint32_t sb[CB];   // (scale, bias) word of each B chunk's row
};

template <int BITS, bool GU>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_gemm_kernel(PrefillArgs a,
                                                                       int nt_per_tile) {
  extern __shared__ __align__(16) uint8_t smem[];  // 2 x (A stage + B stage)
  using R = GemmRegs<BITS>;
  constexpr int CB = R::CB;
  constexpr int GBYTES = KG * BITS / 8;  // packed bytes of one weight row per K group
  constexpr int CPR = GBYTES / 16;       // 16-byte chunks per weight row per K group
  int tile, nt;
  tile_of_block(nt_per_tile, &tile, &nt);
  if (tile >= *a.n_tiles) return;
  const int g = a.tile_group[tile], m0 = a.tile_m0[tile];
  const bool shared = g == a.E;
  const int inner = shared ? a.Is : a.I;
  // gate/up: N = intermediate columns (128 per tile), K = H.  down: N = H, K = inner.
  const int c0 = nt * (GU ? BN / 2 : BN);
  if (GU && c0 >= inner) return;
  const int K = GU ? a.H : inner;
  const int r0 = a.row_off[g] + m0;
  const int mrows = min(BM, a.row_off[g + 1] - a.row_off[g] - m0);
  const uint8_t* blob = group_blob(a, g);
  const QLayout L = shared ? a.ls : a.lr;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // waves w and w+4 share a SIMD: give each SIMD one low-row and one
  // high-row wave, so skipped row blocks (below) shorten every SIMD's work
  const int mq = wave >> 2, nq = wave & 3, kh = lane >> 5, l32 = lane & 31;
  // row blocks of 32 entirely past the tile's rows do no MFMA work
  const bool rb_live0 = mq * 64 < mrows, rb_live1 = mq * 64 + 32 < mrows;

  // A rows this thread stages: row (tid >> 3) + 64 i, 16-byte part tid & 7.
  // Rows past the tile read a valid row and only feed rows never stored.
  const uint16_t* asrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rl = (tid >> 3) + 64 * i;
    const int rr = rl < mrows ? rl : 0;
    if (GU)
      asrc[i] = a.x + (size_t)a.perm_tok[r0 + rr] * a.H + (tid & 7) * 8;
    else
      asrc[i] = a.h + (size_t)(r0 + rr) * a.hI + (tid & 7) * 8;
  }
  // B chunks this thread dequantises: chunk c = tid + 512 j -> row c / CPR, part c % CPR
  const uint8_t* bsrc[CB];
  const uint32_t* sbsrc[CB];
  int bdst[CB];
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    const int c = tid + kGemmThreads * j;
    const int br = c / CPR, part = c % CPR;
    int m, wrow;
    if (GU) {
      m = br >= BN / 2 ? 1 : 0;
      wrow = c0 + (br & (BN / 2 - 1));
      if (wrow >= inner) wrow = 0;  // overhang of a small intermediate size: never stored
    } else {
      m = 2;
      wrow = c0 + br;
    }
    const uint8_t* qb = blob + (m == 0 ? L.q_off[0] : m == 1 ? L.q_off[1] : L.q_off[2]);
    const uint8_t* sbb = blob + (m == 0 ? L.sb_off[0] : m == 1 ? L.sb_off[1] : L.sb_off[2]);
    bsrc[j] = qb + (int64_t)wrow * (K * BITS / 8) + part * 16;
    sbsrc[j] = reinterpret_cast<const uint32_t*>(sbb) + (int64_t)wrow * (K / 64);
    bdst[j] = kLdsA + br * kLdsRow + part * (256 / BITS);
  }

  auto load = [&](R& r, int kg) {
#pragma unroll
    for (int i = 0; i < 2; ++i) r.a[i] = ld16(asrc[i] + kg * KG);
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      r.b[j] = ld16(bsrc[j] + kg * GBYTES);
      r.sb[j] = sbsrc[j][kg];
    }
  };
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
  // weight-row base (in the B stage) of the wave's 2 column blocks
  int bro[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
    bro[cb] = GU ? (cb * (BN / 2) + nq * 32) : (nq * 64 + cb * 32);

  auto read_frags = [&](const uint8_t* stage, int s, uint4* af, uint4* bf) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      af[rb] = *reinterpret_cast<const uint4*>(stage + (mq * 64 + rb * 32 + l32) * kLdsRow +
                                               kh * 64 + s * 16);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      bf[cb] = *reinterpret_cast<const uint4*>(stage + kLdsA + (bro[cb] + l32) * kLdsRow +
                                               kh * 64 + s * 16);
  };
  // Quarter `part` of staging a register set into LDS: the A rows (parts 0,
  // 1) and 4*CB/4 packed words of the weight chunks, dequantised.
  auto store_part = [&](const R& r, uint8_t* stage, int part) {
    if (part < 2)
      *reinterpret_cast<uint4*>(stage + ((tid >> 3) + 64 * part) * kLdsRow + (tid & 7) * 16) =
          r.a[part];
#pragma unroll
    for (int f = part * CB; f < (part + 1) * CB; ++f) {
      const int c = f / 4, m = f % 4;
      const uint32_t wrd = m == 0 ? r.b[c].x : m == 1 ? r.b[c].y : m == 2 ? r.b[c].z : r.b[c].w;
      const uint4 v = dequant_word<BITS>(wrd, bf16_lo(r.sb[c]), bf16_hi(r.sb[c]));
      if (BITS == 4) {
        *reinterpret_cast<uint4*>(stage + bdst[c] + m * 16) = v;
      } else {
        *reinterpret_cast<uint2*>(stage + bdst[c] + m * 8) = make_uint2(v.x, v.y);
      }
    }
  };
  // One K group: MFMAs on stage `sc` (already in LDS) interleaved with
  // staging register set `r` into `ss`: after each group of four MFMAs (which
  // run asynchronously on the matrix core) a quarter of the dequantisation
  // issues on the VALU.
  auto step = [&](const uint8_t* sc, const R& r, uint8_t* ss, bool do_store) {
    uint4 af[2][2], bf[2][2];
    read_frags(sc, 0, af[0], bf[0]);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      if (s4 < 3) read_frags(sc, s4 + 1, af[(s4 + 1) & 1], bf[(s4 + 1) & 1]);
      if (rb_live0) {
        acc[0][0] = mfma(af[s4 & 1][0], bf[s4 & 1][0], acc[0][0]);
        acc[0][1] = mfma(af[s4 & 1][0], bf[s4 & 1][1], acc[0][1]);
      }
      if (rb_live1) {
        acc[1][0] = mfma(af[s4 & 1][1], bf[s4 & 1][0], acc[1][0]);
        acc[1][1] = mfma(af[s4 & 1][1], bf[s4 & 1][1], acc[1][1]);
      }
      if (do_store) {
        __builtin_amdgcn_sched_barrier(0);
        store_part(r, ss, s4);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  const int NK = K / KG;
  uint8_t* st0 = smem;
  uint8_t* st1 = smem + kLdsA + kLdsB;
  R r0_, r1_;
  load(r0_, 0);
  if (NK > 1) load(r1_, 1);
#pragma unroll
  for (int part = 0; part < 4; ++part) store_part(r0_, st0, part);
  if (NK > 2) load(r0_, 2);
  __syncthreads();
  // step kg computes stage kg from LDS while staging kg+1 and loading kg+3
  int kg = 0;
  for (; kg + 4 < NK; kg += 2) {
    step(st0, r1_, st1, true);
    load(r1_, kg + 3);
    __syncthreads();
    step(st1, r0_, st0, true);
    load(r0_, kg + 4);
    __syncthreads();
  }
  for (; kg < NK; kg += 2) {
    step(st0, r1_, st1, kg + 1 < NK);
    if (kg + 3 < NK) load(r1_, kg + 3);
    __syncthreads();
    if (kg + 1 >= NK) break;
    step(st1, r0_, st0, kg + 2 < NK);
    if (kg + 4 < NK) load(r0_, kg + 4);
    __syncthreads();
  }

  if (GU) {
    // acc[rb][0] = gate, acc[rb][1] = up for the same rows and columns
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rl = mq * 64 + rb * 32 + (v >> 2) * 8 + kh * 4 + (v & 3);
        const int col = c0 + nq * 32 + l32;
        if (rl < mrows && col < inner) {
          const float gv = acc[rb][0][v], uv = acc[rb][1][v];
          const float hv = gv / (1.0f + __expf(-gv)) * uv;
          a.h[(size_t)(r0 + rl) * a.hI + col] = (uint16_t)f32_to_bf16(hv);
        }
      }
  } else {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rl = mq * 64 + rb * 32 + (v >> 2) * 8 + kh * 4 + (v & 3);
          if (rl < mrows)
            a.yd[(size_t)(r0 + rl) * a.H + c0 + nq * 64 + cb * 32 + l32] = acc[rb][cb][v];
        }
  }
}

// y[t] = sum_j w[t,j] * y_j[t] + sigma_t * y_shared[t]; one block per token.
__global__ __launch_bounds__(kThreads) void prefill_combine_kernel(PrefillArgs a) {
  const int t = blockIdx.x, H = a.H, k = a.k;
  const int shared_row = a.row_off[a.E] + t;
  int rows[MOE_MAX_TOPK];
  float wj[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    rows[j] = j < k ? a.inv[t * k + j] : 0;
    wj[j] = j < k ? a.w[t * k + j] : 0.f;
  }
  const float sg = a.sigma[t];
  for (int c = threadIdx.x * 4; c < H; c += kThreads * 4) {
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k) {
        const float4 v = *reinterpret_cast<const float4*>(a.yd + (size_t)rows[j] * H + c);
        y.x = fmaf(wj[j], v.x, y.x);
        y.y = fmaf(wj[j], v.y, y.y);
        y.z = fmaf(wj[j], v.z, y.z);
        y.w = fmaf(wj[j], v.w, y.w);
      }
    }
    const float4 v = *reinterpret_cast<const float4*>(a.yd + (size_t)shared_row * H + c);
    y.x = fmaf(sg, v.x, y.x);
    y.y = fmaf(sg, v.y, y.y);
    y.z = fmaf(sg, v.z, y.z);
    y.w = fmaf(sg, v.w, y.w);
    if (a.y_f32) *reinterpret_cast<float4*>(a.y_f32 + (size_t)t * H + c) = y;
    if (a.y_bf16) {
      const uint32_t lo = f32_to_bf16(y.x) | (f32_to_bf16(y.y) << 16);
      const uint32_t hi = f32_to_bf16(y.z) | (f32_to_bf16(y.w) << 16);
      *reinterpret_cast<uint2*>(a.y_bf16 + (size_t)t * H + c) = make_uint2(lo, hi);
    }
  }
}

int pad8(int n) { return (n + 7) / 8 * 8; }

}  // namespace

hipError_t launch_split_router(const float* Wr, const float* wsg, int E, int H, uint16_t* wr3,
                               hipStream_t s) {
  const int64_t n = (int64_t)(E + 1) * H;
  hipLaunchKernelGGL(split_router_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, Wr, wsg, E, H, wr3);
  return hipGetLastError();
}

hipError_t launch_router_gemm(const uint16_t* x, int T, int H, const uint16_t* wr3,
                              const float* bias, int has_wsg, int E, float* logits,
                              float* sigma_raw, hipStream_t s) {
  const dim3 grid((T + BM - 1) / BM, (E + (has_wsg ? 1 : 0) + BM - 1) / BM);
  hipLaunchKernelGGL(router_gemm_kernel, grid, dim3(kThreads), 0, s, x, T, H, wr3, bias, E,
                     has_wsg, logits, sigma_raw);
  return hipGetLastError();
}

hipError_t launch_prefill_sort(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(prefill_scan_kernel, dim3(1), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_compact_kernel, dim3(a.E + 1), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int BITS, bool GU>
hipError_t launch_grouped(const PrefillArgs& a, hipStream_t s) {
  const int nt = GU ? (std::max(a.I, a.Is) + BN / 2 - 1) / (BN / 2) : a.H / BN;
  const size_t lds = 2 * (size_t)(kLdsA + kLdsB);
  hipError_t e = allow_lds(grouped_gemm_kernel<BITS, GU>, lds);
  if (e != hipSuccess) return e;
  const int tiles8 = pad8(a.max_tiles);  // every XCD gets tiles8 / 8 tiles x nt blocks
  hipLaunchKernelGGL((grouped_gemm_kernel<BITS, GU>), dim3(tiles8 * nt), dim3(kGemmThreads), lds,
                     s, a, nt);
  return hipGetLastError();
}

hipError_t launch_prefill_gu(const PrefillArgs& a, hipStream_t s) {
  return a.bits == 4 ? launch_grouped<4, true>(a, s) : launch_grouped<8, true>(a, s);
}

hipError_t launch_prefill_down(const PrefillArgs& a, hipStream_t s) {
  return a.bits == 4 ? launch_grouped<4, false>(a, s) : launch_grouped<8, false>(a, s);
}

hipError_t launch_prefill_combine(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(prefill_combine_kernel, dim3(a.T), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
