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
//      to the running total, which bounds the summation depth.  K is split
//      into up to 4 slices (enough workgroups for the chip); the top-k adds
//      the slices' partial sums in order, then rb.
//   2. sort: per-chunk expert histograms (LDS), one scan to row offsets, chunk
//      offsets and a tile list, a scatter at LDS cursors, then a per-expert
//      sort of each expert's pairs, so rows keep (token, choice) order.  The
//      shared expert is one more group whose rows are all tokens.
//   3. gate/up grouped GEMM: a tile of up to 96 rows of one group x 128
//      intermediate columns of BOTH gate and up per workgroup; operands reach
//      LDS by direct-to-LDS loads; each lane dequantises its own MFMA B
//      operands (s*q + b in f32, then round to nearest even); epilogue
//      h = bf16(silu(g) * u).
//   4. down grouped GEMM: up to 96 rows x 256 output columns, same scheme;
//      f32 outputs per (token, choice) row.
//   5. combine: y[t] = sum_j w[t,j] y_j + sigma_t y_shared, j in order.
//
// MFMA K order: for MFMA step s of a 64-wide group, lanes 0-31 supply
// K = 8s..8s+7 and lanes 32-63 supply K = 32+8s..32+8s+7, so each lane's A and
// B operands for the four steps are 64 contiguous bytes.  Both operands use
// the same order, so the product is unchanged.
//
// Blocks are numbered so that consecutive work items land on the same XCD
// (the dispatcher deals blocks round-robin over the 8 XCDs): the column
// tiles of one row tile then share its rows in that XCD's L2.
#include <algorithm>
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace moe {
namespace {

using namespace dev;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int BM = kPrefillBM;        // grouped-GEMM tile rows
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

// One packed word -> bf16 values in natural order: 8 (int4, as a uint4) or
// 4 (int8, low half of the uint4); each value is s * q + b in f32 (one
// rounding), then rounded to nearest even.  s24 = s * 2^24 and s20 = s * 2^20
// are hoisted by the caller (see dequant8_int4).
template <int BITS>
__device__ __forceinline__ uint4 dequant_word(uint32_t w, float s24, float s20, float b) {
  if (BITS == 4) {
    const uint32_t w8 = w >> 8;
    const uint32_t a0 = w & 0x000F000Fu, a1 = w & 0x00F000F0u;
    const uint32_t a2 = w8 & 0x000F000Fu, a3 = w8 & 0x00F000F0u;
    return make_uint4(pack_bf16(fma_mix_lo(s24, a0, b), fma_mix_lo(s20, a1, b)),
                      pack_bf16(fma_mix_lo(s24, a2, b), fma_mix_lo(s20, a3, b)),
                      pack_bf16(fma_mix_hi(s24, a0, b), fma_mix_hi(s20, a1, b)),
                      pack_bf16(fma_mix_hi(s24, a2, b), fma_mix_hi(s20, a3, b)));
  } else {
    const uint32_t a0 = w & 0x00FF00FFu, a1 = (w >> 8) & 0x00FF00FFu;
    return make_uint4(pack_bf16(fma_mix_lo(s24, a0, b), fma_mix_lo(s24, a1, b)),
                      pack_bf16(fma_mix_hi(s24, a0, b), fma_mix_hi(s24, a1, b)), 0u, 0u);
  }
}

__device__ __forceinline__ const uint8_t* group_blob(const PrefillArgs& a, int g) {
  if (g == a.E) return a.shared_blob;
  return a.routed_base ? a.routed_base + (int64_t)g * a.stride : a.slot_ptrs[g];
}

// ------------------------------------------------------------- router

__global__ __launch_bounds__(kThreads) void split_router_kernel(const float* Wr, int E, int H,
                                                                uint16_t* wr3) {
  const int64_t n = (int64_t)E * H;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const float W = Wr[i];
  const uint32_t hi = f32_to_bf16(W);
  const float r1 = W - bf16_to_f32(hi);
  const uint32_t mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);
  wr3[i] = (uint16_t)hi;
  wr3[n + i] = (uint16_t)mid;
  wr3[2 * n + i] = (uint16_t)f32_to_bf16(r2);
}

// Partial logits of a 128-token x 128-expert tile over one slice of the K
// groups: part[split][t][e] = sum over the slice of x[t] . (hi + mid + lo)[e].
// Each 64-wide K step is staged in LDS (x rows and the three planes' rows,
// 16-byte pieces, 8 threads per 128-byte row segment so every load
// instruction reads whole segments), one stage per workgroup so two
// workgroups share a CU; the next step's loads are in flight in registers
// during this step's MFMAs and go to LDS once every wave has read the stage.  Four waves, each 64 tokens x 64
// experts (2 x 2 MFMA 32x32x16 tiles).  Per step the products go to a fresh
// accumulator that is then added to the running total, so every f32 sum has
// a bounded depth.  Tokens / experts past the end read a valid row and are
// never stored.
constexpr int RT = 128;
constexpr int kRouterStage = 4 * RT * kLdsRow;  // x rows + three planes: 73,728 bytes

__global__ __launch_bounds__(kThreads, 2) void router_gemm_kernel(const uint16_t* x, int T, int H,
                                                                  const uint16_t* wr3, int E,
                                                                  int n_et, int ks, float* part) {
  extern __shared__ __align__(16) uint8_t smem[];
  int mt, inner;
  tile_of_block(n_et * ks, &mt, &inner);
  if (mt * RT >= T) return;
  const int et = inner / ks, sp = inner % ks;
  const int G = H / KG;
  const int g0 = sp * G / ks, nk = (sp + 1) * G / ks - g0;
  const int t0 = mt * RT, e0 = et * RT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mh = wave >> 1, nh = wave & 1, kh = lane >> 5, l32 = lane & 31;
  const int64_t plane = (int64_t)E * H;

  const int part8 = tid & 7, r8 = tid >> 3;
  uint32_t aoff[4], boff[4];  // element offsets: T * H and E * H are < 2^31
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    aoff[i] = (uint32_t)min(t0 + r8 + 32 * i, T - 1) * (uint32_t)H + part8 * 8;
    boff[i] = (uint32_t)min(e0 + r8 + 32 * i, E - 1) * (uint32_t)H + part8 * 8;
  }
  const int sdst = r8 * kLdsRow + part8 * 16;
  u32x4_v ra[4], rw[3][4];
  auto load = [&](int g) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = ld16v(x + g * KG + aoff[i]);
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) rw[p][i] = ld16v(wr3 + p * plane + g * KG + boff[i]);
  };
  auto store = [&]() __attribute__((always_inline)) {
    uint8_t* st = smem + sdst;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4_v*>(st + 32 * i * kLdsRow) = ra[i];
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4_v*>(st + ((p + 1) * RT + 32 * i) * kLdsRow) = rw[p][i];
  };

  f32x16_t tot[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) tot[i][j] = f32x16_t{};
  load(g0);
  store();
  __syncthreads();
  for (int i = 0; i < nk; ++i) {
    if (i + 1 < nk) load(g0 + i + 1);
    const uint8_t* st = smem + kh * 64;
    f32x16_t acc[2][2];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[r][c] = f32x16_t{};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      uint4 af[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        af[rb] = *reinterpret_cast<const uint4*>(st + (mh * 64 + rb * 32 + l32) * kLdsRow + s4 * 16);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        uint4 bf[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          bf[cb] = *reinterpret_cast<const uint4*>(
              st + ((p + 1) * RT + nh * 64 + cb * 32 + l32) * kLdsRow + s4 * 16);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mfma(af[rb], bf[cb], acc[rb][cb]);
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c) tot[r][c] += acc[r][c];
    if (i + 1 < nk) {
      __syncthreads();  // every wave has read the stage
      store();
      __syncthreads();
    }
  }
  float* out = part + (size_t)sp * T * E;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = t0 + mh * 64 + rb * 32 + (v >> 2) * 8 + kh * 4 + (v & 3);
        const int e = e0 + nh * 64 + cb * 32 + l32;
        if (t < T && e < E) out[(size_t)t * E + e] = tot[rb][cb][v];
      }
}

// --------------------------------------------------------------- sort

// Per-chunk expert histograms: the T * k (token, choice) pairs are cut into
// kSortChunks contiguous chunks; hist[c][e] = pairs of chunk c that chose e.
__device__ __forceinline__ void sort_chunk(const PrefillArgs& a, int c, int* p0, int* p1) {
  const int P = a.T * a.k, len = (P + kSortChunks - 1) / kSortChunks;
  *p0 = min(P, c * len);
  *p1 = min(P, *p0 + len);
}

__global__ __launch_bounds__(kThreads) void prefill_hist_kernel(PrefillArgs a) {
  __shared__ int h[1024];
  for (int e = threadIdx.x; e < a.E; e += kThreads) h[e] = 0;
  __syncthreads();
  int p0, p1;
  sort_chunk(a, blockIdx.x, &p0, &p1);
  for (int p = p0 + threadIdx.x; p < p1; p += kThreads) {
    const int e = a.idx[p];
    if ((unsigned)e < (unsigned)a.E) atomicAdd(&h[e], 1);  // other values: left out
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += kThreads) a.hist[blockIdx.x * a.E + e] = h[e];
}

// One block: per expert, counts over the chunks and each chunk's offset
// inside the expert's rows (hist rewritten in place as the exclusive prefix
// over chunks); then group sizes (group E = shared expert = all tokens) ->
// row offsets and the tile list.
constexpr int kScanThreads = 1024;

static_assert(kSortChunks % 16 == 0, "scan loads chunk counts 16 at a time");

__global__ __launch_bounds__(kScanThreads) void prefill_scan_kernel(PrefillArgs a) {
  constexpr int kPer = 2;  // groups per thread: up to 2048 groups
  __shared__ int s_cnt[kPer * kScanThreads];
  __shared__ int s_wr[kScanThreads / kWave], s_wt[kScanThreads / kWave];
  const int G = a.E + 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid < a.E) {
    int run = 0;
    for (int c0 = 0; c0 < kSortChunks; c0 += 16) {  // 16 loads in flight
      int v[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) v[c] = a.hist[(c0 + c) * a.E + tid];
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        a.hist[(c0 + c) * a.E + tid] = run;
        run += v[c];
      }
    }
    s_cnt[tid] = run;
  }
  if (tid == 0) s_cnt[a.E] = a.T;
  __syncthreads();
  const int g0 = tid * kPer;
  int c[kPer], r = 0, tl = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    c[i] = g0 + i < G ? s_cnt[g0 + i] : 0;
    r += c[i];
    tl += (c[i] + BM - 1) / BM;
  }
  // inclusive wave scan of (r, tl), then across the waves
  int ir = r, it = tl;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int yr = __shfl_up(ir, d), yt = __shfl_up(it, d);
    if (lane >= d) {
      ir += yr;
      it += yt;
    }
  }
  if (lane == kWave - 1) {
    s_wr[wave] = ir;
    s_wt[wave] = it;
  }
  __syncthreads();
  int br = ir - r, bt = it - tl;
  for (int w = 0; w < wave; ++w) {
    br += s_wr[w];
    bt += s_wt[w];
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int g = g0 + i;
    if (g < G) {
      a.row_off[g] = br;
      const int n = (c[i] + BM - 1) / BM;
      for (int j = 0; j < n; ++j) {
        if (bt + j < a.max_tiles) {
          a.tile_group[bt + j] = g;
          a.tile_m0[bt + j] = j * BM;
        }
      }
      if (g == G - 1) {
        a.row_off[G] = br + c[i];
        *a.n_tiles = bt + n;
      }
    }
    br += c[i];
    bt += (c[i] + BM - 1) / BM;
  }
}

// Scatter every (token, choice) pair p = t * k + j of a chunk to its
// expert's rows at an LDS cursor that starts at the chunk's offset (order
// inside a chunk's share arbitrary; fixed by the sort).  perm_tok
// temporarily holds p.
__global__ __launch_bounds__(kThreads) void prefill_scatter_kernel(PrefillArgs a) {
  __shared__ int cur[1024];
  for (int e = threadIdx.x; e < a.E; e += kThreads)
    cur[e] = a.row_off[e] + a.hist[blockIdx.x * a.E + e];
  __syncthreads();
  int p0, p1;
  sort_chunk(a, blockIdx.x, &p0, &p1);
  for (int p = p0 + threadIdx.x; p < p1; p += kThreads) {
    const int e = a.idx[p];
    if ((unsigned)e < (unsigned)a.E) a.perm_tok[atomicAdd(&cur[e], 1)] = p;
  }
}

// Sorted row -> pair index (t * k + j), from the inverse map the sort wrote.
__global__ __launch_bounds__(kThreads) void prefill_perm_kernel(PrefillArgs a, int32_t* perm) {
  const int P = a.T * a.k;
  for (int p = blockIdx.x * kThreads + threadIdx.x; p < P; p += gridDim.x * kThreads)
    if ((unsigned)a.idx[p] < (unsigned)a.E) perm[a.inv[p]] = p;
}

constexpr int kSortMax = 8192;  // longest segment sorted in LDS

// One block per group: its rows in (token, choice) order, i.e. p ascending
// (stable w.r.t. token order), then perm_tok = token, inv = row.  Segments
// up to kSortMax long are sorted in LDS (bitonic); a longer segment is
// rebuilt by a ballot compaction over all pairs.
__global__ __launch_bounds__(kThreads) void prefill_segsort_kernel(PrefillArgs a) {
  __shared__ int keys[kSortMax];
  __shared__ int s_wcnt[kThreads / kWave];
  const int e = blockIdx.x;
  const int base = a.row_off[e];
  if (e == a.E) {
    for (int t = threadIdx.x; t < a.T; t += kThreads) a.perm_tok[base + t] = t;
    return;
  }
  const int n = a.row_off[e + 1] - base;
  if (n <= kSortMax) {
    int N = 1;
    while (N < n) N <<= 1;
    for (int i = threadIdx.x; i < N; i += kThreads) keys[i] = i < n ? a.perm_tok[base + i] : 0x7fffffff;
    __syncthreads();
    for (int kk = 2; kk <= N; kk <<= 1) {
      for (int j = kk >> 1; j > 0; j >>= 1) {
        for (int i = threadIdx.x; i < N; i += kThreads) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const int x = keys[i], y = keys[ixj];
            if ((x > y) == ((i & kk) == 0)) {
              keys[i] = y;
              keys[ixj] = x;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int i = threadIdx.x; i < n; i += kThreads) {
      const int p = keys[i];
      a.perm_tok[base + i] = p / a.k;
      a.inv[p] = base + i;
    }
  } else {
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
}

// ------------------------------------------------------ grouped GEMMs
//
// One workgroup = one tile of up to 96 rows of a group x 256 weight rows:
// for gate/up, 128 intermediate columns of gate and the same 128 of up (so
// h = silu(g) * u is finished in registers); for down, 256 output columns.
// Four waves, one per SIMD, two workgroups per CU.  Wave w owns 64 weight
// rows (gate/up: 32 gate + the same 32 up; down: 64 outputs) for all rows of
// the tile: up to 3 x 2 MFMA 32x32x16 tiles.
//
// Every operand reaches LDS by direct-to-LDS loads (global_load_lds: lane i
// of an instruction writes 16 bytes at the instruction's LDS base + 16 i), so
// no staging registers and no LDS stores sit in the loop, and each load
// instruction reads whole row segments (the L1 and address units then see
// few distinct lines per instruction):
// * A, per K group (one quantisation group), three-slot ring: the tile's 96
//   rows (gathered token rows of x, or rows of h), 128 bytes each, 8 rows per
//   instruction; 16-byte piece p of row r sits in slot p ^ f(r) with
//   f(r) = (r ^ (r >> 3)) & 7, so the MFMA operand reads (32 rows, one piece
//   each) hit distinct banks.
// * B, per 64-byte slice of each weight row (two int4 groups or one int8
//   group), two-slot ring: 16 rows x 64 bytes per instruction; piece p of row
//   r in slot p ^ h(r), h(r) = ((r >> 1) ^ (r >> 3)) & 3, again conflict-free
//   for the operand reads (lane (l, k) reads weights 32k..32k+31 of row l).
// * (scale, bias) words, 16 bytes (four groups) of every weight row per
//   instruction, two-slot ring; when K is not a multiple of 256 one word per
//   row and group instead, three-slot ring.
// The A rows of group g + 2 and the weights of group g + 2 or beyond are in
// flight while group g computes.  Each lane dequantises its own weights to bf16 (s * q + b, round
// to nearest even) right before the MFMA step that uses them, overlapping
// the matrix core's previous step.  No weight is dequantised twice within a
// tile.

constexpr int kGemmThreads = 256;  // 4 waves
constexpr int kAStage = BM * 128;  // 12,288 bytes

template <int BITS>
struct GemmCfg {
  static constexpr int NQ = BITS == 4 ? 1 : 2;    // 16-byte pieces per lane per column block
  static constexpr int GPC = BITS == 4 ? 2 : 1;   // K groups per 64-byte weight slice
  static constexpr int kBOff = 3 * kAStage;       // A ring: 3 x 12,288
  static constexpr int kBSlot = 4 * 2 * 2048;     // 4 waves x 2 column blocks x 32 rows x 64 B
  static constexpr int kSbOff = kBOff + 2 * kBSlot;
  static constexpr int kLds = kSbOff + 2 * 4096;  // 77,824 bytes: two workgroups per CU
  static constexpr int kAOps = 3, kBOps = 4;      // load instructions per wave per A / B stage
};

template <int BITS>
struct BRaw {  // one K group of packed weights for the lane's two weight rows
  static constexpr int N = GemmCfg<BITS>::NQ;
  uint4 q[2][N];
  float s24[2], s20[2], bi[2];  // per column block: s * 2^24, s * 2^20, b
};

// (lds_addr, dma16, dma4 and wait_vm_n: device.h.)  The loop below waits
// for its direct-to-LDS loads itself.
// wait until at most N of this wave's LDS operations are outstanding
template <int N>
__device__ __forceinline__ void wait_lgkm_n() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int BITS, bool GU, bool SB4>
__global__ __launch_bounds__(kGemmThreads, 2) void grouped_gemm_kernel(PrefillArgs a,
                                                                       int nt_per_tile) {
  using C = GemmCfg<BITS>;
  using R = BRaw<BITS>;
  extern __shared__ __align__(16) uint8_t smem[];
  int tile, nt;
  tile_of_block(nt_per_tile, &tile, &nt);
  if (tile >= *a.n_tiles) return;
  const int g = a.tile_group[tile], m0 = a.tile_m0[tile];
  const bool shared = g == a.E;
  const int inner = shared ? a.Is : a.I;
  // gate/up: N = intermediate columns (128 per tile), K = H.  down: N = H, K = inner.
  const int c0 = nt * (GU ? 128 : 256);
  if (GU && c0 >= inner) return;
  const int K = GU ? a.H : inner;
  const int NK = K / KG;
  const int r0 = a.row_off[g] + m0;
  const int mrows = min(BM, a.row_off[g + 1] - a.row_off[g] - m0);
  const int nrb = min(BM / 32, (mrows + 31) / 32);  // row blocks of 32 with any live row
  const uint8_t* blob = group_blob(a, g);
  const QLayout L = shared ? a.ls : a.lr;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = lane >> 5, l32 = lane & 31;
  // gate/up waves whose 32 columns lie past a small intermediate size load
  // clamped rows and compute on them like the others, but store nothing
  const bool wave_live = !GU || c0 + 32 * wave < inner;
  const uint32_t lds0 = lds_addr(smem);

  // weight row of column block cb, row r (0..31) of this wave
  auto wrow = [&](int cb, int r) __attribute__((always_inline)) {
    return GU ? min(c0 + 32 * wave + r, inner - 1) : c0 + 64 * wave + 32 * cb + r;
  };
  auto qsec = [&](int cb) __attribute__((always_inline)) -> int64_t {
    const int m = GU ? cb : 2;
    return m == 0 ? L.q_off[0] : m == 1 ? L.q_off[1] : L.q_off[2];
  };
  auto sbsec = [&](int cb) __attribute__((always_inline)) -> int64_t {
    const int m = GU ? cb : 2;
    return m == 0 ? L.sb_off[0] : m == 1 ? L.sb_off[1] : L.sb_off[2];
  };

  // A loads: wave w fills 8-row chunks w, w + 4, w + 8; lane l takes row
  // 8c + l / 8 and stores slot l % 8, i.e. global piece (l % 8) ^ f(row).
  // Rows past the tile read the tile's first row and feed only accumulator
  // rows that are never stored.
  const uint8_t* asrc[3];
  {
    const uint16_t* abase = GU ? a.x : a.h;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int rl = 8 * (wave + 4 * i) + (lane >> 3);
      const int rr = rl < mrows ? rl : 0;
      const int piece = (lane & 7) ^ ((rl ^ (rl >> 3)) & 7);
      const int64_t row = GU ? (int64_t)a.perm_tok[r0 + rr] * a.H : (int64_t)(r0 + rr) * a.hI;
      asrc[i] = reinterpret_cast<const uint8_t*>(abase + row + piece * 8);
    }
  }
  // B loads: instruction i of column block cb covers rows 16i .. 16i + 15;
  // lane l takes row 16i + l / 4, slot l % 4 = global piece (l % 4) ^ h(row)
  // of the row's 64-byte slice.  A slice of an odd last int4 group reads 32
  // bytes past the row: the next row, or the next section of the blob.
  const uint8_t* bsrc[2][2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 16 * i + (lane >> 2);
      const int piece = (lane & 3) ^ (((r >> 1) ^ (r >> 3)) & 3);
      bsrc[cb][i] = blob + qsec(cb) + (int64_t)wrow(cb, r) * (K * BITS / 8) + piece * 16;
    }
  // (scale, bias) words: lane l loads those of column block l / 32, row l % 32
  const uint8_t* sbsrc = blob + sbsec(kh) + (int64_t)wrow(kh, l32) * NK * 4;

  const uint32_t ldsA = lds0, ldsB = lds0 + C::kBOff, ldsS = lds0 + C::kSbOff;
  auto issue_a = [&](int kg) __attribute__((always_inline)) {
    const uint32_t st = ldsA + (kg % 3) * kAStage;
#pragma unroll
    for (int i = 0; i < 3; ++i) dma16(asrc[i] + kg * (KG * 2), st + (wave + 4 * i) * 1024);
  };
  auto issue_b = [&](int c) __attribute__((always_inline)) {  // 64-byte slice c
    const uint32_t st = ldsB + (c & 1) * C::kBSlot + wave * 4096;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16(bsrc[cb][i] + c * 64, st + cb * 2048 + i * 1024);
  };
  auto issue_sb = [&](int d) __attribute__((always_inline)) {  // SB4: groups 4d..4d+3; else group d
    if (SB4)
      dma16(sbsrc + d * 16, ldsS + (d & 1) * 4096 + wave * 1024);
    else
      dma4(sbsrc + d * 4, ldsS + (d % 3) * 1024 + wave * 256);
  };

  // A operand rows: row rb * 32 + l32, piece kh * 4 + s at slot
  // (kh * 4 + s) ^ f(row) = ax[rb] ^ s
  int ax[3];
#pragma unroll
  for (int rb = 0; rb < 3; ++rb) {
    const int r = rb * 32 + l32;
    ax[rb] = (kh * 4) ^ ((r ^ (r >> 3)) & 7);
  }
  const int bh = ((l32 >> 1) ^ (l32 >> 3)) & 3;  // h(l32)
  auto a_frag = [&](const uint8_t* st, int rb, int s) __attribute__((always_inline)) -> uint4 {
    return *reinterpret_cast<const uint4*>(st + (rb * 32 + l32) * 128 + ((ax[rb] ^ s) << 4));
  };
  // bf16 B operand of MFMA step s for column block cb: weights 8s..8s+7 of
  // the lane's 32
  auto b_operand = [&](const R& r, int cb, int s) __attribute__((always_inline)) -> uint4 {
    const float s24 = r.s24[cb], s20 = r.s20[cb], bi = r.bi[cb];
    if (BITS == 4) {
      const uint4 q = r.q[cb][0];
      const uint32_t w = s == 0 ? q.x : s == 1 ? q.y : s == 2 ? q.z : q.w;
      return dequant_word<4>(w, s24, s20, bi);
    } else {
      const uint4 q = r.q[cb][s >> 1];
      const uint32_t w0 = (s & 1) ? q.z : q.x, w1 = (s & 1) ? q.w : q.y;
      const uint4 lo = dequant_word<8>(w0, s24, s20, bi), hi = dequant_word<8>(w1, s24, s20, bi);
      return make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  };
  // the lane's packed weights and (scale, bias) words of group kg, from LDS
  auto read_b = [&](int kg) __attribute__((always_inline)) -> R {
    R r;
    const int c = kg / C::GPC;
    const uint8_t* bs = smem + C::kBOff + (c & 1) * C::kBSlot + wave * 4096 + l32 * 64;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int i = 0; i < C::NQ; ++i) {
        const int piece = BITS == 4 ? ((kg & 1) << 1) | kh : 2 * kh + i;
        r.q[cb][i] = *reinterpret_cast<const uint4*>(bs + cb * 2048 + ((piece ^ bh) << 4));
      }
    uint32_t sb[2];
    if (SB4) {
      const uint8_t* ss = smem + C::kSbOff + ((kg >> 2) & 1) * 4096 + wave * 1024 + (kg & 3) * 4;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        sb[cb] = *reinterpret_cast<const uint32_t*>(ss + (cb * 32 + l32) * 16);
    } else {
      const uint8_t* ss = smem + C::kSbOff + (kg % 3) * 1024 + wave * 256;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        sb[cb] = *reinterpret_cast<const uint32_t*>(ss + (cb * 32 + l32) * 4);
    }
    // the group's scale and bias, once for its four MFMA steps
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float sc = bf16_lo(sb[cb]);
      r.s24[cb] = sc * 16777216.0f;
      r.s20[cb] = sc * 1048576.0f;
      r.bi[cb] = bf16_hi(sb[cb]);
    }
    return r;
  };

  f32x16_t acc[BM / 32][2];
#pragma unroll
  for (int i = 0; i < BM / 32; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  // The K pipeline.  Barrier point j opens group j: past it the A rows of
  // group j are in LDS for every wave, and no wave reads group j - 1's A slot
  // any more.  At point j each wave refills the ring slots whose last reader
  // is done:
  //   A rows of group j + 2, into group j - 1's slot;
  //   int4, odd j: the weight slice of groups j + 3 and j + 4, into the
  //   slice of groups j - 1 and j (both already read into registers);
  //   int8: the weights of group j + 2, into group j's slot (already read);
  //   (scale, bias) words, four groups per load: at j = 3 mod 4 the block
  //   from group j + 5, into the block of groups j - 3 .. j; one word per
  //   group: group j + 3.
  // Point 0 sits in the prologue and point j + 1 in step 3 of group j, after
  // that step's first MFMAs, so the matrix core works through the barrier.
  // Group j + 1's packed weights are read into registers during step 2 of
  // group j, after the wave waits for every load it issued up to point
  // j - 1 (which also covers group j + 1's A rows); group j + 1's first A
  // fragments are read right after point j + 1.  Every load is waited for
  // before the wave exits.
  const int nslice = (NK + C::GPC - 1) / C::GPC;
  const int nsb = SB4 ? NK / 4 : NK;
  auto issue_at = [&](int j) __attribute__((always_inline)) -> int {
    int n = 0;
    if (j + 2 < NK) {
      issue_a(j + 2);
      n += C::kAOps;
    }
    if (C::GPC == 2) {
      if ((j & 1) && (j + 3) / 2 < nslice) {
        issue_b((j + 3) / 2);
        n += C::kBOps;
      }
    } else if (j + 2 < nslice) {
      issue_b(j + 2);
      n += C::kBOps;
    }
    if (SB4) {
      if ((j & 3) == 3 && (j + 5) / 4 < nsb) {
        issue_sb((j + 5) / 4);
        n += 1;
      }
    } else if (j + 3 < NK) {
      issue_sb(j + 3);
      n += 1;
    }
    return n;
  };

  auto run = [&](auto nrb_c) __attribute__((always_inline)) {
    constexpr int NRB = decltype(nrb_c)::value;
    issue_a(0);
    if (NK > 1) issue_a(1);
    issue_b(0);
    if (nslice > 1) issue_b(1);
    issue_sb(0);
    if (SB4) {
      if (nsb > 1) issue_sb(1);
    } else {
      if (NK > 1) issue_sb(1);
      if (NK > 2) issue_sb(2);
    }
    wait_vm_n<0>();
    R r = read_b(0);
    wait_lgkm_n<0>();  // point 0 may refill the slots just read
    barrier();
    int n_cur = issue_at(0);  // loads issued at the point that opened the current group
    uint4 af[2][NRB], bo[2][2];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) af[0][rb] = a_frag(smem, rb, 0);
    bo[0][0] = b_operand(r, 0, 0);
    bo[0][1] = b_operand(r, 1, 0);

    // One K group.  MFMA step s runs on operands prepared during step s - 1
    // (A fragments read from LDS, B dequantised in registers); the scheduler
    // is told to interleave each MFMA with a share of the next step's
    // dequantisation.  P = kg mod 4 fixes how many loads the point that
    // opened the group issued away from the ends of K, so every wait below
    // is a constant (near the ends: a full wait).
    auto group = [&](auto p_c, int kg) __attribute__((always_inline)) {
      constexpr int P = decltype(p_c)::value;
      constexpr int NS = C::kAOps + ((C::GPC == 1 || (P & 1)) ? C::kBOps : 0) +
                         (SB4 ? (P == 3 ? 1 : 0) : 1);
      const uint8_t* st = smem + (kg % 3) * kAStage;
      const uint8_t* st1 = smem + ((kg + 1) % 3) * kAStage;
      const bool more = kg + 1 < NK;
      R rn;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int cur = s4 & 1, nxt = cur ^ 1;
        __builtin_amdgcn_sched_barrier(0);
        if (s4 < 3) {
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) af[nxt][rb] = a_frag(st, rb, s4 + 1);
        }
        if (s4 == 2 && more) {
          if (n_cur == NS)
            wait_vm_n<NS>();
          else
            wait_vm_n<0>();
          rn = read_b(kg + 1);
        }
        if (s4 < 3) {
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
            acc[rb][0] = mfma(af[cur][rb], bo[cur][0], acc[rb][0]);
            acc[rb][1] = mfma(af[cur][rb], bo[cur][1], acc[rb][1]);
          }
          bo[nxt][0] = b_operand(r, 0, s4 + 1);
          bo[nxt][1] = b_operand(r, 1, s4 + 1);
          // LDS reads first, then one MFMA per share of the dequant VALU ops
          if (s4 == 2)
            __builtin_amdgcn_sched_group_barrier(0x100, NRB + 2 * C::NQ + 2, 0);
          else
            __builtin_amdgcn_sched_group_barrier(0x100, NRB, 0);
#pragma unroll
          for (int i = 0; i < 2 * NRB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, BITS == 4 ? 48 / (2 * NRB) : 40 / (2 * NRB), 0);
          }
        } else {
          acc[0][0] = mfma(af[cur][0], bo[cur][0], acc[0][0]);
          acc[0][1] = mfma(af[cur][0], bo[cur][1], acc[0][1]);
          __builtin_amdgcn_sched_barrier(0);
          if (more) {
            wait_lgkm_n<0>();  // this wave's reads of group kg's A slot are done
            barrier();
            n_cur = issue_at(kg + 1);
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) af[nxt][rb] = a_frag(st1, rb, 0);
          }
#pragma unroll
          for (int rb = 1; rb < NRB; ++rb) {
            acc[rb][0] = mfma(af[cur][rb], bo[cur][0], acc[rb][0]);
            acc[rb][1] = mfma(af[cur][rb], bo[cur][1], acc[rb][1]);
          }
          if (more) {
            bo[nxt][0] = b_operand(rn, 0, 0);
            bo[nxt][1] = b_operand(rn, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, NRB, 0);
#pragma unroll
            for (int i = 0; i < 2 * NRB - 2; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 48 / 4, 0);
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (more) r = rn;
    };
    for (int k0 = 0; k0 < NK; k0 += 4) {
      group(std::integral_constant<int, 0>{}, k0);
      if (k0 + 1 < NK) group(std::integral_constant<int, 1>{}, k0 + 1);
      if (k0 + 2 < NK) group(std::integral_constant<int, 2>{}, k0 + 2);
      if (k0 + 3 < NK) group(std::integral_constant<int, 3>{}, k0 + 3);
    }
    wait_vm_n<0>();
  };
  static_assert(BM == 96, "row-block dispatch below");
  switch (nrb) {
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    default: run(std::integral_constant<int, 3>{}); break;
  }

  if (!wave_live) return;
  if (GU) {
    // acc[rb][0] = gate, acc[rb][1] = up for the same rows and columns
    const int col = c0 + 32 * wave + l32;
#pragma unroll
    for (int rb = 0; rb < BM / 32; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rl = rb * 32 + (v >> 2) * 8 + kh * 4 + (v & 3);
        if (rl < mrows && col < inner) {
          const float gv = acc[rb][0][v], uv = acc[rb][1][v];
          const float hv = gv / (1.0f + __expf(-gv)) * uv;
          a.h[(size_t)(r0 + rl) * a.hI + col] = (uint16_t)f32_to_bf16(hv);
        }
      }
  } else {
#pragma unroll
    for (int rb = 0; rb < BM / 32; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rl = rb * 32 + (v >> 2) * 8 + kh * 4 + (v & 3);
          if (rl < mrows)
            a.yd[(size_t)(r0 + rl) * a.H + c0 + 64 * wave + 32 * cb + l32] = acc[rb][cb][v];
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
    // every row's load in flight first, then the sum in j order
    float4 vr[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      vr[j] = j < k ? *reinterpret_cast<const float4*>(a.yd + (size_t)rows[j] * H + c)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 v = *reinterpret_cast<const float4*>(a.yd + (size_t)shared_row * H + c);
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k) {
        y.x = fmaf(wj[j], vr[j].x, y.x);
        y.y = fmaf(wj[j], vr[j].y, y.y);
        y.z = fmaf(wj[j], vr[j].z, y.z);
        y.w = fmaf(wj[j], vr[j].w, y.w);
      }
    }
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

int router_splits(int T, int E, int H) {
  const int tiles = (T + RT - 1) / RT * ((E + RT - 1) / RT);
  int ks = 1;
  while (2 * ks <= kRouterMaxSplits && 2 * ks <= H / KG && tiles * ks < 512) ks *= 2;
  return ks;
}

hipError_t launch_split_router(const float* Wr, int E, int H, uint16_t* wr3, hipStream_t s) {
  const int64_t n = (int64_t)E * H;
  hipLaunchKernelGGL(split_router_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, Wr, E, H, wr3);
  return hipGetLastError();
}

hipError_t launch_router_gemm(const uint16_t* x, int T, int H, const uint16_t* wr3, int E,
                              float* part, hipStream_t s) {
  if ((int64_t)T * H >= (1ll << 31) || (int64_t)E * H >= (1ll << 31) || H % KG != 0)
    return hipErrorInvalidValue;
  const int ks = router_splits(T, E, H);
  const int n_et = (E + RT - 1) / RT;
  const size_t lds = kRouterStage;
  hipError_t e = allow_lds(router_gemm_kernel, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(router_gemm_kernel, dim3(pad8((T + RT - 1) / RT) * n_et * ks), dim3(kThreads),
                     lds, s, x, T, H, wr3, E, n_et, ks, part);
  return hipGetLastError();
}

hipError_t launch_prefill_perm(const PrefillArgs& a, int32_t* perm, hipStream_t s) {
  const int P = a.T * a.k;
  if (P == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min((P + kThreads - 1) / kThreads, 1024);
  hipLaunchKernelGGL(prefill_perm_kernel, dim3(blocks), dim3(kThreads), 0, s, a, perm);
  return hipGetLastError();
}

hipError_t launch_prefill_sort(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(prefill_hist_kernel, dim3(kSortChunks), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_scatter_kernel, dim3(kSortChunks), dim3(kThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_segsort_kernel, dim3(a.E + 1), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int BITS, bool GU, bool SB4>
hipError_t launch_grouped_sb(const PrefillArgs& a, hipStream_t s) {
  const int nt = GU ? (std::max(a.I, a.Is) + 127) / 128 : a.H / 256;
  const int tiles8 = pad8(a.max_tiles);  // every XCD gets tiles8 / 8 tiles x nt blocks
  const size_t lds = GemmCfg<BITS>::kLds;
  hipError_t e = allow_lds(grouped_gemm_kernel<BITS, GU, SB4>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((grouped_gemm_kernel<BITS, GU, SB4>), dim3(tiles8 * nt), dim3(kGemmThreads),
                     lds, s, a, nt);
  return hipGetLastError();
}

// (scale, bias) words four groups at a time when every K of the launch is a
// multiple of 256
template <int BITS, bool GU>
hipError_t launch_grouped(const PrefillArgs& a, hipStream_t s) {
  const bool sb4 = GU ? a.H % 256 == 0 : a.I % 256 == 0 && a.Is % 256 == 0;
  return sb4 ? launch_grouped_sb<BITS, GU, true>(a, s) : launch_grouped_sb<BITS, GU, false>(a, s);
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
