// Decode-path expert kernels (1 <= T <= 8 tokens): dequant-GEMV straight
// from packed int4/int8 group-quantised weights.
//
// The pages run each chosen expert's matrices as GEMVs on the GPU and keep
// the shared experts resident ([xix] how-it-works and lineage paragraphs;
// [lens] "TurboFieldfareとの関係": MLX-style int4/int8 group quantisation,
// byte-addressable kernels with 64-bit offsets, a cooperative GEMV fast
// path).  Their Apple simdgroup GEMV is prior art only; this is a wave64
// design for gfx950 that is bound by HBM bandwidth:
//
// * Work unit = one 16-byte chunk of a weight row (32 int4 or 16 int8
//   values) per lane, read with one global_load_dwordx4; a row of the 2048-
//   wide gate/up matrices is exactly one chunk per lane of a wave.  The
//   lane's slice of x (or of h) is fixed for all rows it visits, so it is
//   loaded once, pre-paired into bf16x2 registers, and reused.
// * int4 -> bf16 without a convert: (word >> 4j) & 0x000F000F | 0x43004300
//   is the bf16 pair (128 + q_j, 128 + q_{j+4}); v_dot2_f32_bf16 multiplies
//   it with the matching x pair and accumulates in f32.  The 128 offset is
//   folded into the bias: sum (s q + b) x = s D + (b - 128 s) X, with
//   D = sum (128 + q) x and X = sum x over the chunk.  int8 fields are
//   converted exactly with v_cvt_f32_ubyte (integers <= 255 are exact bf16).
// * Dequantised weights are therefore used exactly (s q + b is a float32
//   value for these ranges); products and sums are f32.
// * gate/up: one workgroup = one expert slot x a block of rows of gate AND
//   up, so h = bf16(silu(g) * u) is finished in registers and written once.
// * down + combine: one workgroup = a block of output rows for all chosen
//   experts and the shared expert; per-(token, slot) partial sums meet in
//   LDS and are combined in the fixed order j = 0..k-1, then the shared
//   term, so the arithmetic never depends on where a blob lives (pool slot
//   or resident) -- hit and miss give bit-identical outputs.
#include <algorithm>

#include "device.h"
#include "gemv.h"
#include "kernels.h"

namespace moe {
namespace {

using namespace dev;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

__device__ __forceinline__ const uint8_t* slot_blob(const DecodeArgs& a, const SlotArgs& sa,
                                                    int s) {
  if (a.routed_base) return a.routed_base + (int64_t)a.slot_expert[s] * a.stride;
  if (a.slot_ptrs) return a.slot_ptrs[s];
  // select rather than index, so the argument block stays in registers
  const uint8_t* p = sa.p[0];
#pragma unroll
  for (int i = 1; i < kSlotArgs; ++i) p = s == i ? sa.p[i] : p;
  return p;
}

// ---------------------------------------------------------------- gate/up

template <int BITS, int NT, int CPL, int PASSES>
__global__ __launch_bounds__(kThreads) void gate_up_kernel(DecodeArgs a, SlotArgs sa) {
  if (a.go && *a.go == 0) return;  // pool mode: an expert is not resident
  using F = Fmt<BITS>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H = a.H;
  const int C = H / F::kEpc;     // chunks per row
  const int LPR = C / CPL;       // lanes per row (power of two <= 64)
  const int RPP = kWave / LPR;   // rows per wave per pass
  const int rows_per_wg = kWaves * PASSES * RPP;

  // which expert slot / row block: the shared expert's blocks come first
  // (they do not wait for routing), then the routed slots'
  const int rb_shared = a.shared_blob ? (a.Is + rows_per_wg - 1) / rows_per_wg : 0;
  const int rb_routed = (a.I + rows_per_wg - 1) / rows_per_wg;
  int slot, rblock, nrows;
  const uint8_t* blob = nullptr;
  QLayout L;
  bool shared;
  if ((int)blockIdx.x < rb_shared) {
    slot = -1;
    rblock = blockIdx.x;
    blob = a.shared_blob;
    L = a.ls;
    nrows = a.Is;
    shared = true;
  } else {
    const int b = blockIdx.x - rb_shared;
    slot = b / rb_routed;
    rblock = b % rb_routed;
    if (NT > 1 && slot >= *a.n_slots) return;
    L = a.lr;
    nrows = a.I;
    shared = false;
  }
  int jt[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (NT == 1)  // one token: its k experts are distinct, slot s is choice j = s
      jt[t] = shared ? a.k : slot;
    else
      jt[t] = (t < a.T) ? (shared ? a.k : (int)a.jmap[slot * kJmapStride + t]) : -1;
  }

  const int sub = lane % LPR, rsub = lane / LPR;
  const int64_t row_bytes = (int64_t)H * BITS / 8;
  const int G = H / 64;

  // the lane's x slices (independent of routing: issued first), paired
  uint32_t xp[NT][CPL][F::kPairs];
  float xs[NT][CPL];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (jt[t] < 0) continue;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ci = sub + c * LPR;
      const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)t * H + ci * F::kEpc);
      pair_natural<BITS>(src, xp[t][c], xs[t][c]);
    }
  }

  if (!shared) blob = slot_blob(a, sa, slot);
  // weights for all passes: PASSES x 2 x CPL 16-byte loads in flight per lane
  uint4 q[2][PASSES][CPL];
  uint32_t sb[2][PASSES][CPL];
  int rows[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = rblock * rows_per_wg + (p * kWaves + wave) * RPP + rsub;
    rows[p] = r;
    const bool ok = r < nrows;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint8_t* qb = blob + L.q_off[m] + (int64_t)r * row_bytes;
      const uint8_t* sbb = blob + L.sb_off[m] + (int64_t)r * G * 4;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int ci = sub + c * LPR;
        q[m][p][c] = ok ? ld16(qb + ci * 16) : make_uint4(0, 0, 0, 0);
        sb[m][p][c] = ok ? ldu32(sbb + (ci * F::kEpc / 64) * 4) : 0u;
      }
    }
  }

  const int kp1 = a.k + 1;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (jt[t] < 0) continue;
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        g = chunk_term<BITS>(g, sb[0][p][c], chunk_dot<BITS>(q[0][p][c], xp[t][c]), xs[t][c]);
        u = chunk_term<BITS>(u, sb[1][p][c], chunk_dot<BITS>(q[1][p][c], xp[t][c]), xs[t][c]);
      }
      g = group_sum(g, LPR);
      u = group_sum(u, LPR);
      if (sub == 0 && rows[p] < nrows) {
        const float hv = g / (1.0f + __expf(-g)) * u;
        a.h[((size_t)t * kp1 + jt[t]) * a.hI + h_pos<BITS>(rows[p])] = (uint16_t)f32_to_bf16(hv);
      }
    }
  }
}

// ------------------------------------------------------------ down+combine

constexpr int kDownThreads = 1024;
constexpr int kDownWaves = kDownThreads / kWave;

template <int BITS, int NT, int BATCH>
__global__ __launch_bounds__(kDownThreads) void down_kernel(DecodeArgs a, SlotArgs sa, int R) {
  if (a.go && *a.go == 0) return;  // pool mode: an expert is not resident
  using F = Fmt<BITS>;
  extern __shared__ __align__(16) uint8_t smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int T = a.T, k = a.k, kp1 = k + 1, hI = a.hI;
  const int nchunk_h = hI / F::kEpc;
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(smem);                     // [T][k+1][hI]
  float* hsum = reinterpret_cast<float*>(smem + (size_t)T * kp1 * hI * 2);  // [T][k+1][hI/EPC]
  float* part = hsum + (size_t)T * kp1 * nchunk_h;                         // [T][k+1][R]
  int8_t* jm = reinterpret_cast<int8_t*>(part + (size_t)T * kp1 * R);       // [n_routed][NT]

  const int n_routed = a.n_slot_max ? *a.n_slots : 0;
  const bool has_shared = a.shared_blob != nullptr;

  // stage h (written by the gate/up kernel) and its per-chunk sums; each
  // thread requests 8 pieces before storing any (one round trip per 8)
  {
    const int n16 = T * kp1 * hI * 2 / 16;
    const uint4* src = reinterpret_cast<const uint4*>(a.h);
    uint4* dst = reinterpret_cast<uint4*>(hbuf);
    for (int base = 0; base < n16; base += kDownThreads * 8) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + threadIdx.x + u * kDownThreads;
        v[u] = i < n16 ? ld16(src + i) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + threadIdx.x + u * kDownThreads;
        if (i < n16) dst[i] = v[u];
      }
    }
  }
  for (int i = threadIdx.x; i < n_routed * NT; i += kDownThreads)
    jm[i] = a.jmap[(i / NT) * kJmapStride + i % NT];
  __syncthreads();
  for (int i = threadIdx.x; i < T * kp1 * nchunk_h; i += kDownThreads) {
    const uint32_t* c = reinterpret_cast<const uint32_t*>(hbuf + (size_t)i * F::kEpc);
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < F::kPairs; ++v) s += bf16_lo(c[v]) + bf16_hi(c[v]);
    hsum[i] = s;
  }
  __syncthreads();

  const int row0 = blockIdx.x * R;
  const int Cr = a.I / F::kEpc, Cs = a.Is / F::kEpc;
  const int RPPr = kWave / Cr, RPPs = kWave / Cs;
  const int NRPr = (R + RPPr - 1) / RPPr, NRPs = (R + RPPs - 1) / RPPs;
  const int n_items = n_routed * NRPr + (has_shared ? NRPs : 0);

  for (int it0 = wave; it0 < n_items; it0 += kDownWaves * BATCH) {
    uint4 q[BATCH];
    uint32_t sbw[BATCH];
    int rloc[BATCH], slot[BATCH], ci[BATCH], lpr[BATCH];
#pragma unroll
    for (int bi = 0; bi < BATCH; ++bi) {
      const int it = it0 + bi * kDownWaves;
      slot[bi] = -2;
      q[bi] = make_uint4(0, 0, 0, 0);
      sbw[bi] = 0;
      rloc[bi] = 0;
      ci[bi] = 0;
      lpr[bi] = 1;
      if (it >= n_items) continue;
      const uint8_t* blob;
      QLayout L;
      int C, rp, RPP, inner;
      if (it < n_routed * NRPr) {
        slot[bi] = it / NRPr;
        rp = it % NRPr;
        blob = slot_blob(a, sa, slot[bi]);
        L = a.lr;
        C = Cr;
        RPP = RPPr;
        inner = a.I;
      } else {
        slot[bi] = -1;
        rp = it - n_routed * NRPr;
        blob = a.shared_blob;
        L = a.ls;
        C = Cs;
        RPP = RPPs;
        inner = a.Is;
      }
      lpr[bi] = C;
      ci[bi] = lane % C;
      rloc[bi] = rp * RPP + lane / C;
      const int row = row0 + rloc[bi];
      if (rloc[bi] < R && row < a.H) {
        const int64_t row_bytes = (int64_t)inner * BITS / 8;
        q[bi] = ld16(blob + L.q_off[2] + (int64_t)row * row_bytes + ci[bi] * 16);
        sbw[bi] = ldu32(blob + L.sb_off[2] + ((int64_t)row * (inner / 64) + ci[bi] * F::kEpc / 64) * 4);
      }
    }
#pragma unroll
    for (int bi = 0; bi < BATCH; ++bi) {
      if (slot[bi] == -2) continue;
      const bool row_ok = rloc[bi] < R && row0 + rloc[bi] < a.H;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t >= T) continue;
        const int j = slot[bi] < 0 ? k : (int)jm[slot[bi] * NT + t];
        if (j < 0) continue;
        const int hb = (t * kp1 + j);
        const uint4* hsrc = reinterpret_cast<const uint4*>(hbuf + (size_t)hb * hI + ci[bi] * F::kEpc);
        uint32_t hp[F::kPairs];
#pragma unroll
        for (int v = 0; v < F::kPairs / 4; ++v) {
          const uint4 d = hsrc[v];
          hp[4 * v] = d.x;
          hp[4 * v + 1] = d.y;
          hp[4 * v + 2] = d.z;
          hp[4 * v + 3] = d.w;
        }
        float acc = chunk_term<BITS>(0.f, sbw[bi], chunk_dot<BITS>(q[bi], hp),
                                     hsum[hb * nchunk_h + ci[bi]]);
        acc = group_sum(acc, lpr[bi]);
        if (ci[bi] == 0 && row_ok) part[hb * R + rloc[bi]] = acc;
      }
    }
  }
  __syncthreads();

  for (int i = threadIdx.x; i < T * R; i += kDownThreads) {
    const int t = i / R, r = i % R, row = row0 + r;
    if (row >= a.H) continue;
    float y = a.accumulate ? a.y_f32[(size_t)t * a.H + row] : 0.f;
    for (int j = 0; j < k; ++j) y = fmaf(a.w[t * k + j], part[(t * kp1 + j) * R + r], y);
    if (has_shared) y = fmaf(a.gate[t], part[(t * kp1 + k) * R + r], y);
    if (a.y_f32) a.y_f32[(size_t)t * a.H + row] = y;
    if (a.y_bf16) a.y_bf16[(size_t)t * a.H + row] = (uint16_t)f32_to_bf16(y);
  }
}

// ------------------------------------------------- down+combine, one token
//
// Wave w owns slots w, w+4, ... (slot s < k is the token's choice j = s;
// slot k is the shared expert).  It loads its slots' h slices once into
// registers (no LDS staging), then the down-projection chunks of the
// workgroup's R output rows for each of its slots; partial row sums meet in
// LDS and one thread per row combines them in j order, then the shared term.
template <int BITS, int SPW, int NPMAX>
__global__ __launch_bounds__(kThreads) void down1_kernel(DecodeArgs a, SlotArgs sa) {
  if (a.go && *a.go == 0) return;  // pool mode: an expert is not resident
  using F = Fmt<BITS>;
  constexpr int R = 8;
  __shared__ float part[(kWaves * SPW) * R];
  __shared__ float s_w[MOE_MAX_TOPK + 1];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int k = a.k, nsl = k + (a.shared_blob ? 1 : 0);
  const int row0 = blockIdx.x * R;

  if ((int)threadIdx.x < k) s_w[threadIdx.x] = a.w[threadIdx.x];
  if ((int)threadIdx.x == k) s_w[k] = a.gate[0];

  uint32_t hp[SPW][F::kPairs];
  float hs[SPW];
  uint4 q[SPW][NPMAX];
  uint32_t sbw[SPW][NPMAX];
  int C[SPW];
#pragma unroll
  for (int si = 0; si < SPW; ++si) {
    const int s = wave + kWaves * si;
    C[si] = 1;
    if (s >= nsl) continue;
    const bool sh = s == k;
    const int inner = sh ? a.Is : a.I;
    C[si] = inner / F::kEpc;
    const int ci = lane % C[si];
    const uint4* hsrc = reinterpret_cast<const uint4*>(a.h + (size_t)s * a.hI + ci * F::kEpc);
#pragma unroll
    for (int v = 0; v < F::kPairs / 4; ++v) {
      const uint4 d = hsrc[v];
      hp[si][4 * v] = d.x;
      hp[si][4 * v + 1] = d.y;
      hp[si][4 * v + 2] = d.z;
      hp[si][4 * v + 3] = d.w;
    }
  }
#pragma unroll
  for (int si = 0; si < SPW; ++si) {
    const int s = wave + kWaves * si;
    if (s >= nsl) continue;
    const bool sh = s == k;
    const uint8_t* blob = sh ? a.shared_blob : slot_blob(a, sa, s);
    const QLayout L = sh ? a.ls : a.lr;
    const int inner = sh ? a.Is : a.I;
    const int ci = lane % C[si], RPP = kWave / C[si];
    const int64_t row_bytes = (int64_t)inner * BITS / 8;
#pragma unroll
    for (int p = 0; p < NPMAX; ++p) {
      const int rloc = p * RPP + lane / C[si];
      const int row = row0 + rloc;
      q[si][p] = make_uint4(0, 0, 0, 0);
      sbw[si][p] = 0;
      if (rloc < R && row < a.H) {
        q[si][p] = ld16(blob + L.q_off[2] + (int64_t)row * row_bytes + ci * 16);
        sbw[si][p] = ldu32(blob + L.sb_off[2] + ((int64_t)row * (inner / 64) + ci * F::kEpc / 64) * 4);
      }
    }
  }
#pragma unroll
  for (int si = 0; si < SPW; ++si) {
    float s_ = 0.f;
#pragma unroll
    for (int v = 0; v < F::kPairs; ++v) s_ += bf16_lo(hp[si][v]) + bf16_hi(hp[si][v]);
    hs[si] = s_;
  }
#pragma unroll
  for (int si = 0; si < SPW; ++si) {
    const int s = wave + kWaves * si;
    if (s >= nsl) continue;
    const int ci = lane % C[si], RPP = kWave / C[si];
#pragma unroll
    for (int p = 0; p < NPMAX; ++p) {
      const int rloc = p * RPP + lane / C[si];
      if (p * RPP >= R) break;
      float acc = chunk_term<BITS>(0.f, sbw[si][p], chunk_dot<BITS>(q[si][p], hp[si]), hs[si]);
      acc = group_sum(acc, C[si]);
      if (ci == 0 && rloc < R) part[s * R + rloc] = acc;
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < R) {
    const int r = threadIdx.x, row = row0 + r;
    if (row < a.H) {
      float y = a.accumulate ? a.y_f32[row] : 0.f;
      for (int j = 0; j < k; ++j) y = fmaf(s_w[j], part[j * R + r], y);
      if (a.shared_blob) y = fmaf(s_w[k], part[k * R + r], y);
      if (a.y_f32) a.y_f32[row] = y;
      if (a.y_bf16) a.y_bf16[row] = (uint16_t)f32_to_bf16(y);
    }
  }
}

// ------------------------------------------------------------ dequant hook

template <int BITS>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* blob, QLayout L,
                                                           int rows, int cols, int which,
                                                           float* out_f32, uint16_t* out_bf16) {
  using F = Fmt<BITS>;
  const int64_t words = (int64_t)rows * cols / F::kPerWord;
  const int64_t wi = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (wi >= words) return;
  const uint32_t w = reinterpret_cast<const uint32_t*>(blob + L.q_off[which])[wi];
  const int64_t e0 = wi * F::kPerWord;
  const int64_t r = e0 / cols, c0 = e0 % cols;
  const uint32_t sbw = reinterpret_cast<const uint32_t*>(blob + L.sb_off[which])
      [r * (cols / 64) + c0 / 64];
  const float s = bf16_lo(sbw), b = bf16_hi(sbw);
  // the same f16-subnormal fma_mix arithmetic as the many-token GEMMs, so
  // this entry point pins it bit for bit against s * q + b
  float v[F::kPerWord];
  if constexpr (BITS == 4)
    dequant8_int4(w, s, b, v);
  else
    dequant4_int8(w, s, b, v);
#pragma unroll
  for (int i = 0; i < F::kPerWord; ++i) {
    out_f32[e0 + i] = v[i];
    if (out_bf16) out_bf16[e0 + i] = (uint16_t)f32_to_bf16(v[i]);
  }
}

// ----------------------------------------------------------------- launch

constexpr int kGuPasses = 2;
constexpr int kDownRows = 8;
constexpr int kDownBatch = 4;

int chunks_per_lane(int H, int bits) {
  const int C = H / (128 / bits);
  if (C <= 64) return (64 % C == 0) ? 1 : 0;
  if (C % 64) return 0;
  return C / 64;  // 2 supported below
}

template <int BITS, int NT>
hipError_t gate_up_bits_nt(const DecodeArgs& a, hipStream_t s, const SlotArgs& sa) {
  const int cpl = chunks_per_lane(a.H, BITS);
  const int C = a.H / Fmt<BITS>::kEpc;
  const int rpp = kWave / (C / cpl);
  const int rows_per_wg = kWaves * kGuPasses * rpp;
  const int blocks = a.n_slot_max * ((a.I + rows_per_wg - 1) / rows_per_wg) +
                     (a.shared_blob ? (a.Is + rows_per_wg - 1) / rows_per_wg : 0);
  if (blocks == 0) return hipSuccess;
#define MOE_GU_CASE(CP)                                                                 \
  if (cpl == CP) {                                                                      \
    hipLaunchKernelGGL((gate_up_kernel<BITS, NT, CP, kGuPasses>), dim3(blocks),         \
                       dim3(kThreads), 0, s, a, sa);                                        \
    return hipGetLastError();                                                           \
  }
  MOE_GU_CASE(1)
  MOE_GU_CASE(2)
#undef MOE_GU_CASE
  return hipErrorInvalidValue;
}

template <int BITS, int SPW, int NPMAX>
hipError_t down1_launch(const DecodeArgs& a, hipStream_t s, const SlotArgs& sa) {
  const int blocks = (a.H + 7) / 8;
  hipLaunchKernelGGL((down1_kernel<BITS, SPW, NPMAX>), dim3(blocks), dim3(kThreads), 0, s, a, sa);
  return hipGetLastError();
}

template <int BITS, int SPW>
hipError_t down1_spw(const DecodeArgs& a, hipStream_t s, const SlotArgs& sa) {
  // row passes needed for 8 rows: 8 / (64 / chunks per row)
  const int cmax = std::max(a.I, a.shared_blob ? a.Is : 0) / Fmt<BITS>::kEpc;
  const int np = (8 * cmax + kWave - 1) / kWave;
  if (np <= 2) return down1_launch<BITS, SPW, 2>(a, s, sa);
  if (np <= 4) return down1_launch<BITS, SPW, 4>(a, s, sa);
  return down1_launch<BITS, SPW, 8>(a, s, sa);
}

template <int BITS>
hipError_t down1_bits(const DecodeArgs& a, hipStream_t s, const SlotArgs& sa) {
  const int nsl = a.k + (a.shared_blob ? 1 : 0);
  if (nsl <= 4) return down1_spw<BITS, 1>(a, s, sa);
  if (nsl <= 8) return down1_spw<BITS, 2>(a, s, sa);
  if (nsl <= 12) return down1_spw<BITS, 3>(a, s, sa);
  return down1_spw<BITS, 5>(a, s, sa);
}

template <int BITS, int NT>
hipError_t down_bits_nt(const DecodeArgs& a, hipStream_t s, const SlotArgs& sa) {
  const int kp1 = a.k + 1;
  const size_t lds = (size_t)a.T * kp1 * a.hI * 2 +
                     (size_t)a.T * kp1 * (a.hI / Fmt<BITS>::kEpc) * 4 +
                     (size_t)a.T * kp1 * kDownRows * 4 + (size_t)a.n_slot_max * NT;
  const int blocks = (a.H + kDownRows - 1) / kDownRows;
  hipError_t e = allow_lds(down_kernel<BITS, NT, kDownBatch>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((down_kernel<BITS, NT, kDownBatch>), dim3(blocks), dim3(kDownThreads), lds,
                     s, a, sa, kDownRows);
  return hipGetLastError();
}

}  // namespace

bool decode_shape_supported(int H, int I, int Is, int bits) {
  if (H % 256 || I % 64 || Is % 64 || H > 2048) return false;
  const int cpl = chunks_per_lane(H, bits);
  if (cpl != 1 && cpl != 2) return false;
  const int epc = 128 / bits;
  for (int inner : {I, Is}) {
    const int C = inner / epc;
    if (C < 1 || C > 64 || 64 % C) return false;
  }
  return true;
}

hipError_t launch_gate_up(const DecodeArgs& a, hipStream_t s, const SlotArgs& sa) {
  if (a.bits == 4) return a.T <= 1 ? gate_up_bits_nt<4, 1>(a, s, sa) : gate_up_bits_nt<4, 8>(a, s, sa);
  return a.T <= 1 ? gate_up_bits_nt<8, 1>(a, s, sa) : gate_up_bits_nt<8, 8>(a, s, sa);
}

hipError_t launch_down(const DecodeArgs& a, hipStream_t s, const SlotArgs& sa) {
  if (a.T <= 1) return a.bits == 4 ? down1_bits<4>(a, s, sa) : down1_bits<8>(a, s, sa);
  return a.bits == 4 ? down_bits_nt<4, 8>(a, s, sa) : down_bits_nt<8, 8>(a, s, sa);
}

hipError_t launch_dequant(const uint8_t* blob, const QLayout& lay, int rows, int cols, int bits,
                          int which, float* out_f32, uint16_t* out_bf16, hipStream_t s) {
  const int64_t words = (int64_t)rows * cols / (32 / bits);
  const dim3 grid((unsigned)((words + kThreads - 1) / kThreads));
  if (bits == 4)
    hipLaunchKernelGGL((dequant_kernel<4>), grid, dim3(kThreads), 0, s, blob, lay, rows, cols,
                       which, out_f32, out_bf16);
  else
    hipLaunchKernelGGL((dequant_kernel<8>), grid, dim3(kThreads), 0, s, blob, lay, rows, cols,
                       which, out_f32, out_bf16);
  return hipGetLastError();
}

}  // namespace moe
