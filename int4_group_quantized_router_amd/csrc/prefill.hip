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

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Work id with consecutive ids on the same XCD (grid padded to a multiple of 8).
__device__ __forceinline__ int xcd_work_id() {
  const int b = blockIdx.x;
  return (b & 7) * (gridDim.x >> 3) + (b >> 3);
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
      const uint32_t lo = w[m] & 0x0F0F0F0Fu, hi = (w[m] >> 4) & 0x0F0F0F0Fu;
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
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int kg = 0; kg < H / KG; ++kg) {
    uint4 af[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int s = 0; s < 4; ++s) af[rb][s] = av[rb] ? ld16(arow[rb] + kg * KG + s * 8) : z;
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
          bf[cb][s] = bv[cb] ? ld16(brow[cb] + p * plane + kg * KG + s * 8) : z;
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

// gate/up: tile = 128 rows of group g x 64 intermediate columns (gate and up).
template <int BITS>
__global__ __launch_bounds__(kThreads, 2) void gu_gemm_kernel(PrefillArgs a, int nt_per_tile) {
  __shared__ __align__(16) uint8_t Bs[2][BM * kLdsRow];
  const int wid = xcd_work_id();
  const int tile = wid / nt_per_tile, nt = wid % nt_per_tile;
  if (tile >= *a.n_tiles) return;
  const int g = a.tile_group[tile], m0 = a.tile_m0[tile];
  const bool shared = g == a.E;
  const int N = shared ? a.Is : a.I;
  const int c0 = nt * 64;
  if (c0 >= N) return;
  const int r0 = a.row_off[g] + m0;
  const int mrows = min(BM, a.row_off[g + 1] - a.row_off[g] - m0);
  const uint8_t* blob = group_blob(a, g);
  const QLayout L = shared ? a.ls : a.lr;
  const int H = a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mh = wave >> 1, nh = wave & 1, kh = lane >> 5, l32 = lane & 31;

  const uint16_t* arow[2];
  bool av[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int rl = mh * 64 + rb * 32 + l32;
    av[rb] = rl < mrows;
    arow[rb] = a.x + (size_t)(av[rb] ? a.perm_tok[r0 + rl] : 0) * H + kh * 32;
  }
  constexpr int CPT = BITS == 4 ? 1 : 2;     // 16-byte chunks per thread per K group
  constexpr int GB = KG * BITS / 8;          // packed bytes of one row in one K group
  const int br = tid >> 1;                   // tile row: 0..63 gate, 64..127 up
  const int wrow = c0 + (br & 63);
  const int64_t row_bytes = (int64_t)H * BITS / 8;
  const bool is_up = br >= 64;
  const uint8_t* qrow = blob + (is_up ? L.q_off[1] : L.q_off[0]) + wrow * row_bytes;
  const uint32_t* sbrow = reinterpret_cast<const uint32_t*>(
                              blob + (is_up ? L.sb_off[1] : L.sb_off[0])) + (int64_t)wrow * (H / 64);

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
  const uint4 z = make_uint4(0, 0, 0, 0);
  uint4 braw[CPT], araw[2][4];
  uint32_t bsb;
#pragma unroll
  for (int c = 0; c < CPT; ++c) braw[c] = ld16(qrow + ((tid & 1) * CPT + c) * 16);
  bsb = sbrow[0];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int s = 0; s < 4; ++s) araw[rb][s] = av[rb] ? ld16(arow[rb] + s * 8) : z;

  const int NK = H / KG;
  for (int kg = 0; kg < NK; ++kg) {
    uint8_t* buf = Bs[kg & 1];
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      dequant_chunk<BITS>(braw[c], bsb, buf + br * kLdsRow + ((tid & 1) * CPT + c) * (256 / BITS));
    uint4 braw_n[CPT], araw_n[2][4];
    uint32_t bsb_n = 0;
    if (kg + 1 < NK) {
#pragma unroll
      for (int c = 0; c < CPT; ++c)
        braw_n[c] = ld16(qrow + (kg + 1) * GB + ((tid & 1) * CPT + c) * 16);
      bsb_n = sbrow[kg + 1];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          araw_n[rb][s] = av[rb] ? ld16(arow[rb] + (kg + 1) * KG + s * 8) : z;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 bf[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        bf[cb] = *reinterpret_cast<const uint4*>(buf + (cb * 64 + nh * 32 + l32) * kLdsRow +
                                                 kh * 64 + s * 16);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mfma(araw[rb][s], bf[cb], acc[rb][cb]);
    }
    if (kg + 1 < NK) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) braw[c] = braw_n[c];
      bsb = bsb_n;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int s = 0; s < 4; ++s) araw[rb][s] = araw_n[rb][s];
    }
  }
  // acc[rb][0] = gate, acc[rb][1] = up for the same rows and columns
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rl = mh * 64 + rb * 32 + (v >> 2) * 8 + kh * 4 + (v & 3);
      if (rl < mrows) {
        const float gv = acc[rb][0][v], uv = acc[rb][1][v];
        const float hv = gv / (1.0f + __expf(-gv)) * uv;
        a.h[(size_t)(r0 + rl) * a.hI + c0 + nh * 32 + l32] = (uint16_t)f32_to_bf16(hv);
      }
    }
}

// down: tile = 128 rows of group g x 128 output columns.
template <int BITS>
__global__ __launch_bounds__(kThreads, 2) void down_gemm_kernel(PrefillArgs a, int nt_per_tile) {
  __shared__ __align__(16) uint8_t Bs[2][BM * kLdsRow];
  const int wid = xcd_work_id();
  const int tile = wid / nt_per_tile, nt = wid % nt_per_tile;
  if (tile >= *a.n_tiles) return;
  const int g = a.tile_group[tile], m0 = a.tile_m0[tile];
  const bool shared = g == a.E;
  const int K = shared ? a.Is : a.I;
  const int n0 = nt * BM;
  const int r0 = a.row_off[g] + m0;
  const int mrows = min(BM, a.row_off[g + 1] - a.row_off[g] - m0);
  const uint8_t* blob = group_blob(a, g);
  const QLayout L = shared ? a.ls : a.lr;
  const int H = a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mh = wave >> 1, nh = wave & 1, kh = lane >> 5, l32 = lane & 31;

  const uint16_t* arow[2];
  bool av[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int rl = mh * 64 + rb * 32 + l32;
    av[rb] = rl < mrows;
    arow[rb] = a.h + (size_t)(r0 + (av[rb] ? rl : 0)) * a.hI + kh * 32;
  }
  constexpr int CPT = BITS == 4 ? 1 : 2;
  constexpr int GB = KG * BITS / 8;
  const int br = tid >> 1;  // output column n0 + br
  const int64_t row_bytes = (int64_t)K * BITS / 8;
  const uint8_t* qrow = blob + L.q_off[2] + (int64_t)(n0 + br) * row_bytes;
  const uint32_t* sbrow =
      reinterpret_cast<const uint32_t*>(blob + L.sb_off[2]) + (int64_t)(n0 + br) * (K / 64);

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
  const uint4 z = make_uint4(0, 0, 0, 0);
  uint4 braw[CPT], araw[2][4];
  uint32_t bsb;
#pragma unroll
  for (int c = 0; c < CPT; ++c) braw[c] = ld16(qrow + ((tid & 1) * CPT + c) * 16);
  bsb = sbrow[0];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int s = 0; s < 4; ++s) araw[rb][s] = av[rb] ? ld16(arow[rb] + s * 8) : z;

  const int NK = K / KG;
  for (int kg = 0; kg < NK; ++kg) {
    uint8_t* buf = Bs[kg & 1];
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      dequant_chunk<BITS>(braw[c], bsb, buf + br * kLdsRow + ((tid & 1) * CPT + c) * (256 / BITS));
    uint4 braw_n[CPT], araw_n[2][4];
    uint32_t bsb_n = 0;
    if (kg + 1 < NK) {
#pragma unroll
      for (int c = 0; c < CPT; ++c)
        braw_n[c] = ld16(qrow + (kg + 1) * GB + ((tid & 1) * CPT + c) * 16);
      bsb_n = sbrow[kg + 1];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          araw_n[rb][s] = av[rb] ? ld16(arow[rb] + (kg + 1) * KG + s * 8) : z;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 bf[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        bf[cb] = *reinterpret_cast<const uint4*>(buf + (nh * 64 + cb * 32 + l32) * kLdsRow +
                                                 kh * 64 + s * 16);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mfma(araw[rb][s], bf[cb], acc[rb][cb]);
    }
    if (kg + 1 < NK) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) braw[c] = braw_n[c];
      bsb = bsb_n;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int s = 0; s < 4; ++s) araw[rb][s] = araw_n[rb][s];
    }
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rl = mh * 64 + rb * 32 + (v >> 2) * 8 + kh * 4 + (v & 3);
        if (rl < mrows)
          a.yd[(size_t)(r0 + rl) * H + n0 + nh * 64 + cb * 32 + l32] = acc[rb][cb][v];
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

hipError_t launch_prefill_gemms(const PrefillArgs& a, hipStream_t s) {
  const int nt_gu = std::max(a.I, a.Is) / 64;
  const int nt_dn = a.H / BM;
  hipError_t e;
  if (a.bits == 4)
    hipLaunchKernelGGL(gu_gemm_kernel<4>, dim3(pad8(a.max_tiles * nt_gu)), dim3(kThreads), 0, s,
                       a, nt_gu);
  else
    hipLaunchKernelGGL(gu_gemm_kernel<8>, dim3(pad8(a.max_tiles * nt_gu)), dim3(kThreads), 0, s,
                       a, nt_gu);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.bits == 4)
    hipLaunchKernelGGL(down_gemm_kernel<4>, dim3(pad8(a.max_tiles * nt_dn)), dim3(kThreads), 0,
                       s, a, nt_dn);
  else
    hipLaunchKernelGGL(down_gemm_kernel<8>, dim3(pad8(a.max_tiles * nt_dn)), dim3(kThreads), 0,
                       s, a, nt_dn);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_combine_kernel, dim3(a.T), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
