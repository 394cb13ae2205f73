// Persistent batch-1 decode through a whole stack of MoE layers.
//
// Per token and layer the MoE layer is: router logits, softmax, top-k,
// renormalised weights, the chosen SwiGLU experts straight from the packed
// group-quantised weights, the sigmoid-gated shared expert and the weighted
// combine ([xix] how-it-works paragraph; [lens] "エキスパートストリーミングの仕組み").
// The pages find their decode loop bound by dispatch rather than by IO
// ([ttj] "실무자가 따져볼 지점").  On MI355X one layer-token of the 35B-shaped
// model moves ~18 MB of weights, 2.3 us at 8 TB/s, less than the launch gaps
// and dependency stalls of three kernels, so this kernel runs every layer of
// the stack in one launch:
//
// * 256 workgroups, no more than the device has compute units, so on an
//   otherwise idle device all are resident at once.  The launch is an
//   ordinary one: the kernel uses no grid-wide primitive, and the
//   cooperative launch path costs ~16 us more per call.  If work on another
//   stream keeps some workgroups from starting, the bounded waits (below)
//   turn that into a reported error, not a hang.  The shape (bits, H, I, Is,
//   k, top-k width) is compile-time, so all index arithmetic folds to
//   constants;
// * a layer has three all-to-all hand-offs: its output y (every workgroup
//   needs all of it for the next router and gate/up), the router logits
//   (every workgroup runs the top-k itself) and the SwiGLU activations h
//   (every output row of the down projection needs all of h).  Each hand-off
//   word holds its value and a call tag in ONE atomic store that writes
//   through to the device coherence point (64-bit: f32 | 32-bit tag; h:
//   bf16 << 16 | 16-bit tag).  A consumer polls with coherent loads until
//   every word it needs carries this call's tag -- no counters, fences or
//   grid barriers.  Each layer has its own hand-off buffers, so nothing is
//   overwritten while a slower workgroup may still read it.  Every word is
//   written in 8 copies and a workgroup polls the copy of its XCD (blocks
//   are dealt to the 8 XCDs round-robin): 32 readers per line instead of 256
//   spreads the polling over more memory channels.
// * the call tag comes from a per-workgroup counter in device memory that
//   each workgroup bumps when it leaves, so replaying the same launch (a
//   captured graph) still gives every call a fresh tag.
// * weights that do not depend on routing (router rows, shared expert) are
//   requested before the wait for the data they multiply.
// * every value is computed with the same arithmetic, in the same order, as
//   the per-layer kernels (router GEMV, top-k, gate/up, down, fixed-order
//   combine), so the two paths give bit-identical outputs.
// * every wait is bounded by a wall-clock deadline; a workgroup that runs
//   out of time sets a host-visible error word and leaves, and so do the
//   workgroups waiting on it, so the grid always drains.
#include <algorithm>

#include "device.h"
#include "gemv.h"
#include "kernels.h"

namespace moe {
namespace {

using namespace dev;

// Phase timestamps (profiling builds only, -DMOE_STACK_PHASES): thread 0 of
// every workgroup records the wall clock (100 MHz) at the phase boundaries
// of each layer into a.phases[(l * grid + block) * kStackPhases + p].
// STACK_PHASE_AT records the same clock from thread T (lane 0 of another
// wave) at points of that wave's own work.
#ifdef MOE_STACK_PHASES
#define STACK_PHASE_AT(P, T)                                                    \
  do {                                                                          \
    if (threadIdx.x == (T) && a.phases)                                         \
      a.phases[((size_t)l * kG + blk) * kStackPhases + (P)] = wall_clock64();   \
  } while (0)
#else
#define STACK_PHASE_AT(P, T) \
  do {                       \
  } while (0)
#endif
#define STACK_PHASE(P) STACK_PHASE_AT(P, 0)

// A pointer every lane holds the same value of, kept in scalar registers.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

constexpr int kNT = kStackThreads;
constexpr int kNW = kNT / kWave;
constexpr int kG = kStackGrid;
constexpr int kRep = kStackReplicas;

__device__ __forceinline__ uint32_t tag32_of(uint32_t epoch) { return 2u * epoch + 1u; }
__device__ __forceinline__ uint32_t tag16_of(uint32_t epoch) { return (epoch & 0x7FFFu) | 0x8000u; }

__device__ __forceinline__ uint64_t pack64(float v, uint32_t tag) {
  return (uint64_t)__float_as_uint(v) | ((uint64_t)tag << 32);
}

// Polls run per wave: each polling wave loops on its own until all of its
// lanes' words carry the call's tag (no workgroup barrier per round, so a
// wave whose words are in stops polling and the round trip of one wave
// does not wait for the slowest), then one barrier joins the workgroup and
// makes the result uniform.  One round of a wave: true when all its lanes
// are done; *timed_out (wave-uniform) once the deadline has passed.
__device__ __forceinline__ bool wave_round(bool ok, int64_t deadline, bool* timed_out) {
  if (__ballot(!ok) == 0ull) return true;
  if (wall_clock64() > deadline) {
    *timed_out = true;
    return true;
  }
  __builtin_amdgcn_s_sleep(1);
  return false;
}

// Wait for the previous layer's output y: the threads of waves 4..7 (t =
// threadIdx - 256 in 0..255) take y[t + 256 m] (the per-layer router's
// order for the sum of squares) into registers.  Waves 0..3, which own the
// router rows and so have those rows' loads in flight, do not poll.
constexpr int kYT0 = 256;  // first thread of the y pollers
template <int H>
__device__ bool poll_y(const uint64_t* buf, uint32_t tag, float* yv, int64_t deadline) {
  constexpr int M = H / 256;
  const int t = (int)threadIdx.x - kYT0;
  bool to = false;
  if (t >= 0) {  // waves 4..7
    uint32_t done = 0;
    for (;;) {
      uint64_t e[M];
#pragma unroll
      for (int m = 0; m < M; ++m) e[m] = !((done >> m) & 1u) ? ld_dev(buf + t + m * 256) : 0ull;
      bool ok = true;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if (!((done >> m) & 1u)) {
          if ((uint32_t)(e[m] >> 32) == tag) {
            yv[m] = __uint_as_float((uint32_t)e[m]);
            done |= 1u << m;
          } else {
            ok = false;
          }
        }
      }
      if (wave_round(ok, deadline, &to)) break;
    }
  }
  return !__syncthreads_or(to);
}

// Pairs [FIRST, FIRST + COUNT) of this layer's h words (dense: slot j < k
// at j * I, shared at k * I), PER per polling thread.  Pollers are the
// threads [T0, T0 + N): every thread, or (see Roles) waves 0..3 alone.
template <int N, int COUNT>
constexpr int h_per() {
  return (COUNT + N - 1) / N;
}

// Request this thread's pairs; `done` marks pairs already staged.
template <int T0, int N, int FIRST, int COUNT>
__device__ __forceinline__ void h_request(const uint64_t* src, uint32_t done,
                                          uint64_t (&e)[h_per<N, COUNT>()]) {
  const int t = (int)threadIdx.x - T0;
#pragma unroll
  for (int m = 0; m < h_per<N, COUNT>(); ++m) {
    const int i = t + m * N;
    e[m] = (t >= 0 && t < N && i < COUNT && !((done >> m) & 1u)) ? ld_dev(src + FIRST + i) : 0ull;
  }
}

// Wait for the pairs, starting from the already requested round `e`, and
// stage them in LDS as bf16 pairs: hl[i] = (h[2i], h[2i+1]).
template <int T0, int N, int FIRST, int COUNT>
__device__ bool poll_h(const uint64_t* src, uint32_t tag16, uint32_t* hl, int64_t deadline,
                       uint64_t (&e)[h_per<N, COUNT>()]) {
  constexpr int PER = h_per<N, COUNT>();
  static_assert(PER <= 32, "h pairs per thread");
  static_assert(T0 % 64 == 0 && N % 64 == 0, "h pollers are whole waves");
  const int t = (int)threadIdx.x - T0;
  bool to = false;
  if (t >= 0 && t < N) {  // whole waves (T0 and N are multiples of 64)
    uint32_t done = 0;
    for (;;) {
      bool ok = true;
#pragma unroll
      for (int m = 0; m < PER; ++m) {
        const int i = t + m * N;
        if (i < COUNT && !((done >> m) & 1u)) {
          const uint32_t w0 = (uint32_t)e[m], w1 = (uint32_t)(e[m] >> 32);
          if ((w0 & 0xFFFFu) == tag16 && (w1 & 0xFFFFu) == tag16) {
            hl[FIRST + i] = perm(w1, w0, 0x07060302u);  // (bf16 of w0, bf16 of w1)
            done |= 1u << m;
          } else {
            ok = false;
          }
        }
      }
      if (wave_round(ok, deadline, &to)) break;
      h_request<T0, N, FIRST, COUNT>(src, done, e);
    }
  }
  return !__syncthreads_or(to);
}

// Division of the down-phase work between the waves of a workgroup.  A
// wave's loads complete in order, so a poll issued behind a wave's own
// down-weight loads waits for them.  SPLIT: waves 4..7 (which have the
// fewest routed gate/up rows) load every down item's weights and waves
// 0..3 poll h -- fewer address registers per wave, which the 8-bit shapes
// need to stay within 256 VGPRs; otherwise every wave loads the items it
// computes and every thread polls.
template <int BITS>
struct Roles {
  static constexpr bool SPLIT = BITS == 8;
  static constexpr int HT0 = 0, HN = SPLIT ? 256 : kNT;
};

// Compile-time geometry of one model shape.
template <int BITS_, int H_, int I_, int IS_, int K_>
struct Shape {
  static constexpr int BITS = BITS_, H = H_, I = I_, IS = IS_, K = K_;
  using F = Fmt<BITS>;
  static constexpr int EPC = F::kEpc;
  // gate/up: a row group = RPP rows of a matrix, one wave pass; CPL chunks per lane
  static constexpr int CG = H / EPC;
  static constexpr int CPL = CG > kWave ? CG / kWave : 1;
  static constexpr int LPR = CG / CPL, RPP = kWave / LPR;
  static constexpr int PS = IS / RPP, PR = I / RPP;
  // shared row groups go to waves 1..7 (wave 0 runs the selection meanwhile),
  // routed row groups to all waves
  static constexpr int NPS = (PS + (kNW - 1) * kG - 1) / ((kNW - 1) * kG);
  static constexpr int NPR = (K * PR + kNW * kG - 1) / (kNW * kG);
  // down: R output rows per workgroup; a row of a matrix with C chunks takes C lanes
  static constexpr int R = H / kG;
  static constexpr int CR = I / EPC, CS = IS / EPC;
  static constexpr int RPPR = kWave / CR, RPPS = kWave / CS;
  static constexpr int NIR = R > RPPR ? R / RPPR : 1, NIS = R > RPPS ? R / RPPS : 1;
  static constexpr int NITEMS = K * NIR + NIS;
  static constexpr int DN = (NITEMS + kNW - 1) / kNW;               // down items per wave
  static constexpr int HW = K * I + IS;                             // h words per layer
  static_assert(H % kG == 0 && (R & (R - 1)) == 0, "rows per workgroup");
  static_assert(LPR * CPL == CG && LPR <= kWave && kWave % LPR == 0, "gate/up lanes");
  static_assert(CR <= kWave && CS <= kWave && kWave % CR == 0 && kWave % CS == 0, "down lanes");
  static_assert(R * kRep <= kNT, "combine threads");
  static_assert(H <= 2048 && H % 256 == 0, "router row in one wave");
};

// LDS of one workgroup (bytes; every region 16-byte aligned): the layer
// input (f32 and bf16), the h pairs, the router row of each wave that may
// own one, and one slot per down item of the workgroup (NITEMS): its
// weights (16 bytes per lane) and (scale, bias) words (4 bytes per lane),
// filled by direct-to-LDS loads.
template <class S, int VPL>
struct StackLds {
  static constexpr int kRwRaw = (64 * VPL + 1 + kG - 1) / kG;
  static constexpr int RW = kRwRaw < kNW ? kRwRaw : kNW;
  static constexpr size_t XB = (size_t)S::H * 4;
  static constexpr size_t HL = (size_t)S::H * 6;
  static constexpr size_t WR = HL + (size_t)S::HW * 2;
  static constexpr size_t DW = WR + (size_t)RW * S::H * 4;
  static constexpr size_t DSB = DW + (size_t)S::NITEMS * 1024;
  static constexpr size_t BYTES = DSB + (size_t)S::NITEMS * 256;
  static_assert(XB % 16 == 0 && HL % 16 == 0 && WR % 16 == 0 && DW % 16 == 0, "LDS alignment");
};

// POOL: routed blobs come from each layer's row of the pool's device table
// (StackLayerDesc::res_row) and the call may start at a.l0 > 0; the resident
// instance reads routed_base and always starts at layer 0.
template <class S, int VPL, bool POOL>
__global__ __launch_bounds__(kNT, 1) void stack_decode_kernel(StackArgs a) {
  using F = typename S::F;
  using RO = Roles<S::BITS>;
  constexpr int BITS = S::BITS, H = S::H, I = S::I, IS = S::IS, K = S::K, R = S::R;
  constexpr int CPL = S::CPL, LPR = S::LPR, RPP = S::RPP;
  constexpr int kWrN = H / 256;  // float4 router loads per lane (a whole row per wave)
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float red[4];
  __shared__ int s_sel[MOE_MAX_TOPK];
  __shared__ float s_val[MOE_MAX_TOPK];
  __shared__ float s_w[MOE_MAX_TOPK + 1];
  __shared__ float s_gate_in;  // the shared gate's logit, for its sigmoid
  __shared__ int tmp_e[kWave];
  __shared__ float tmp_v[kWave];
  __shared__ uint32_t tmp_k[kWave];
  __shared__ const uint8_t* s_addr[POOL ? MOE_MAX_TOPK : 1];  // pool mode: blob of choice j
  __shared__ int s_stop;
  __shared__ StackLayerDesc s_layers[kStackMaxLayers];
  __shared__ float part[(K + 1) * R];
  __shared__ float hsum[S::HW / S::EPC];

  const int E = a.E;
  const int blk = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int e_rows = E + (a.has_wsg ? 1 : 0);

  // LDS carve-up (StackLds)
  using LD = StackLds<S, VPL>;
  float* xf = reinterpret_cast<float*>(smem);                       // [H] f32 input
  uint16_t* xb = reinterpret_cast<uint16_t*>(smem + LD::XB);        // [H] bf16 input
  uint32_t* hl = reinterpret_cast<uint32_t*>(smem + LD::HL);        // [HW / 2] h pairs
  // router row of each wave that has one (waves 0 .. (E + 1) / G), f32 [H]
  float* wrl = reinterpret_cast<float*>(smem + LD::WR) + (size_t)wave * H;
  // down items' slots: weights (item it at dwl + 1024 it, lane i's 16 bytes
  // at + 16 i) and (scale, bias) words (at dsbl + 256 it + 4 i)
  const uint8_t* dwl = smem + LD::DW;
  const uint8_t* dsbl = smem + LD::DSB;
  const uint32_t dq_m0 = lds_addr(dwl), dsb_m0 = lds_addr(dsbl);

  const int rep = blk % kRep;  // the XCD of this workgroup
  const uint32_t epoch = ld_dev(a.epochs + blk);
  const uint32_t tag = tag32_of(epoch), tag16 = tag16_of(epoch);
  const int64_t deadline = wall_clock64() + a.timeout_ticks;
  bool failed = false;

  // layer descriptors stay in LDS: a scalar load per layer would miss the
  // caches, which the weight stream keeps flushing
  for (int i = tid; i < a.L * (int)(sizeof(StackLayerDesc) / 8); i += kNT)
    reinterpret_cast<uint64_t*>(s_layers)[i] = reinterpret_cast<const uint64_t*>(a.layers)[i];
  __syncthreads();

  // this lane's place in a gate/up row group, and in the down row groups
  const int sub = lane % LPR, rsub = lane / LPR;
  const int gw = wave * kG + blk;  // global wave index: gate/up row group gw + n * 8G
  const int row0 = blk * R;        // down rows [row0, row0 + R)
  // one down item's weights into its slot: lane i loads what lane i of the
  // wave that computes the item will read (lanes of rows past R load
  // nothing; their sums are never used).  Each wave loads the items it
  // computes.
  auto down_request = [&](int it, const uint8_t* blob, bool shared) {
    const int C = shared ? S::CS : S::CR, RP = shared ? S::RPPS : S::RPPR;
    const int II = shared ? IS : I;
    const int pp = shared ? it - K * S::NIR : it % S::NIR;
    const int ci = lane % C, rloc = pp * RP + lane / C;
    const uint32_t* qo = shared ? a.sq : a.lq;
    const uint32_t* so = shared ? a.ssb : a.lsb;
    if (rloc < R) {
      const int row = row0 + rloc;
      dma16(blob + qo[2] + (size_t)row * (II * BITS / 8) + ci * 16, dq_m0 + it * 1024);
      dma4(blob + so[2] + ((size_t)row * (II / 64) + ci * F::kEpc / 64) * 4, dsb_m0 + it * 256);
    }
  };

  // router row of each wave (E = the shared gate), requested one layer
  // ahead straight into LDS (lane i's float4 m at wrl + 256 m + 4 i)
  const int rrow = blk + kG * wave;
  const int l0 = POOL ? a.l0 : 0;
  const uint32_t wrl_m0 = lds_addr(wrl);
  auto router_request = [&](const StackLayerDesc& Dx) {
    const float* wr = rrow < E ? Dx.Wr + (size_t)rrow * H : Dx.wsg;
#pragma unroll
    for (int m = 0; m < kWrN; ++m) dma16(wr + m * 256 + lane * 4, wrl_m0 + m * 1024);
  };
  float rbv = 0.f;
  if (rrow < e_rows) {
    const StackLayerDesc& D0 = s_layers[l0];
    router_request(D0);
    if (rrow < E && D0.rb) rbv = ldf(D0.rb + rrow);
  }

  int l_fail = a.L;  // the layer a wait ran out of time in
  for (int l = l0; l < a.L && !failed; ++l) {
    const StackLayerDesc D = s_layers[l];
    STACK_PHASE(0);  // layer start

    // ---- layer input: x0, or bf16(y / rms(y)) of the previous layer
    if (l == 0) {  // (a call starting later than layer 0 begins from y_start)
      for (int i = tid; i < H; i += kNT) {
        const uint16_t v = a.x0[i];
        xb[i] = v;
        xf[i] = bf16_to_f32(v);
        if (blk == 0 && a.x_layers) a.x_layers[i] = v;
      }
      __syncthreads();
    } else {
      float yv[H / 256];
      if (POOL && l == l0) {
        if (tid >= kYT0) {
#pragma unroll
          for (int m = 0; m < H / 256; ++m) yv[m] = a.y_start[tid - kYT0 + m * 256];
        }
      } else if (!poll_y<H>(a.ybuf + ((size_t)(l - 1) * kRep + rep) * H, tag, yv, deadline)) {
        failed = true;
        l_fail = l;
        break;
      }
      STACK_PHASE(1);  // previous layer's y received
      // sum of squares in the per-layer router's order (256 threads)
      if (tid >= kYT0) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < H / 256; ++m) s = fmaf(yv[m], yv[m], s);
        s = group_sum(s, kWave);
        if (lane == 0) red[(tid - kYT0) >> 6] = s;
      }
      __syncthreads();
      const float tot = ((red[0] + red[1]) + red[2]) + red[3];
      const float r = 1.0f / sqrtf(tot / (float)H + 1e-6f);
      if (tid >= kYT0) {
#pragma unroll
        for (int m = 0; m < H / 256; ++m) {
          const int i = tid - kYT0 + m * 256;
          const uint32_t bb = f32_to_bf16(yv[m] * r);
          xb[i] = (uint16_t)bb;
          xf[i] = bf16_to_f32(bb);
          if (blk == 0 && a.x_layers) a.x_layers[(size_t)l * H + i] = (uint16_t)bb;
        }
      }
      __syncthreads();
    }

    STACK_PHASE(2);  // input x staged
    // ---- router row: halves summed separately, as the per-layer router
    if (rrow < e_rows) {
      constexpr int half = (H % 512 == 0) ? kWrN / 2 : kWrN;
      float acc0 = 0.f, acc1 = 0.f;
      wait_vm_n<0>();  // this wave's router row has landed in LDS
#pragma unroll
      for (int m = 0; m < kWrN; ++m) {
        const float4 xv = *reinterpret_cast<const float4*>(xf + m * 256 + lane * 4);
        const float4 wm = *reinterpret_cast<const float4*>(wrl + m * 256 + lane * 4);
        float s = m < half ? acc0 : acc1;
        s = fmaf(wm.x, xv.x, s);
        s = fmaf(wm.y, xv.y, s);
        s = fmaf(wm.z, xv.z, s);
        s = fmaf(wm.w, xv.w, s);
        if (m < half) acc0 = s; else acc1 = s;
      }
      acc0 = group_sum(acc0, kWave);
      float out = acc0;
      if (half < kWrN) out = acc0 + group_sum(acc1, kWave);
      if (lane < kRep) {
        const float v = rrow < E ? out + (D.rb ? rbv : 0.f) : out;
        st_dev(a.lbuf + ((size_t)l * kRep + lane) * (E + 1) + rrow, pack64(v, tag));
      }
    }

    STACK_PHASE(3);  // router row published
    // ---- shared expert, independent of routing: its down rows are
    // requested and its gate/up rows computed (h published) while the
    // logits round trip is in flight
    uint32_t* hb = a.hbuf + (size_t)l * kRep * S::HW;
    // this lane's x chunks as bf16 pairs, and their sums.  8-bit weights
    // pair with x in natural order, so those pairs are read from LDS where
    // they are used rather than held in registers across the layer
    constexpr bool kXpLds = BITS == 8;
    uint32_t xp[kXpLds ? 1 : CPL][F::kPairs];
    float xs[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ci = sub + c * LPR;
      uint32_t tmp[F::kPairs];
      pair_natural<BITS>(reinterpret_cast<const uint4*>(xb + ci * F::kEpc),
                         kXpLds ? tmp : xp[kXpLds ? 0 : c], xs[c]);
    }
    auto x_pairs = [&](int c, uint32_t (&out)[F::kPairs]) {
      if constexpr (kXpLds) {
        const uint4* src = reinterpret_cast<const uint4*>(xb + (sub + c * LPR) * F::kEpc);
#pragma unroll
        for (int v = 0; v < F::kPairs / 4; ++v) {
          const uint4 d = src[v];
          out[4 * v] = d.x;
          out[4 * v + 1] = d.y;
          out[4 * v + 2] = d.z;
          out[4 * v + 3] = d.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < F::kPairs; ++i) out[i] = xp[kXpLds ? 0 : c][i];
      }
    };
    // one row group of gate/up: h = bf16(silu(g) * u), kRep copies
    auto gu_rows = [&](const uint4 (&q)[2][CPL], const uint32_t (&sbw)[2][CPL], int base, int row) {
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        uint32_t xc[F::kPairs];
        x_pairs(c, xc);
        g = chunk_term<BITS>(g, sbw[0][c], chunk_dot<BITS>(q[0][c], xc), xs[c]);
        u = chunk_term<BITS>(u, sbw[1][c], chunk_dot<BITS>(q[1][c], xc), xs[c]);
      }
      g = group_sum(g, LPR);
      u = group_sum(u, LPR);
      if (sub < kRep) {  // every lane of the row group holds g and u
        const float hv = g / (1.0f + __expf(-g)) * u;
        st_dev(hb + (size_t)sub * S::HW + base + h_pos<BITS>(row), (f32_to_bf16(hv) << 16) | tag16);
      }
    };
    auto gu_load = [&](const uint8_t* blob, const uint32_t* q_off, const uint32_t* sb_off, int row,
                       uint4 (&q)[2][CPL], uint32_t (&sbw)[2][CPL]) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint8_t* qb = blob + q_off[m] + (size_t)row * (H * BITS / 8);
        const uint8_t* sbb = blob + sb_off[m] + (size_t)row * (H / 64) * 4;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int ci = sub + c * LPR;
          q[m][c] = ld16(qb + ci * 16);
          sbw[m][c] = ldu32(sbb + (ci * F::kEpc / 64) * 4);
        }
      }
    };

    // Wave 0 waits for the logits (in the registers the top-k reads) and
    // selects; waves 1..7 compute the shared expert's gate/up meanwhile.
    __shared__ int s_abort;
    if (wave == 0) {
      const uint64_t* lb = a.lbuf + ((size_t)l * kRep + rep) * (E + 1);
      float v[VPL], vs = 0.f;
      uint32_t key[VPL];
      uint32_t done = 0;
      bool timed_out = false;
      for (;;) {
        uint64_t e[VPL + 1];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
          const int idx = lane + kWave * i;
          e[i] = (idx < E && !((done >> i) & 1u)) ? ld_dev(lb + idx) : 0ull;
        }
        e[VPL] = (lane == 0 && a.has_wsg && !((done >> VPL) & 1u)) ? ld_dev(lb + E) : 0ull;
        bool ok = true;
#pragma unroll
        for (int i = 0; i <= VPL; ++i) {
          const bool need = i < VPL ? lane + kWave * i < E : (lane == 0 && a.has_wsg);
          if (need && !((done >> i) & 1u)) {
            if ((uint32_t)(e[i] >> 32) == tag) {
              if (i < VPL) v[i] = __uint_as_float((uint32_t)e[i]); else vs = __uint_as_float((uint32_t)e[i]);
              done |= 1u << i;
            } else {
              ok = false;
            }
          }
        }
        if (__ballot(!ok) == 0) break;
        if (wall_clock64() > deadline) {
          timed_out = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      STACK_PHASE(10);  // wave 0: every logit received
      if (!timed_out) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
          if (lane + kWave * i >= E) v[i] = 0.f;
          key[i] = lane + kWave * i < E ? order_key(v[i]) : 0u;
        }
        wave_topk<VPL>(v, key, K, tmp_e, tmp_v, tmp_k, s_sel, s_val);
        STACK_PHASE(11);  // wave 0: top-k selected
        // the choices go out now (the host acquires a stopped layer's);
        // their weights are formed once the routed loads are in flight
        if (blk == 0 && a.idx && lane < K) a.idx[(size_t)l * K + lane] = s_sel[lane];
        if (lane == 0) s_gate_in = vs;
        if (POOL) {  // pool mode: the chosen blobs, if all resident
          const uint8_t* addr = lane < K ? D.res_row[s_sel[lane]] : nullptr;
          if (lane < K) s_addr[lane] = addr;
          const bool miss = __ballot(lane < K && addr == nullptr) != 0ull;
          if (lane == 0) s_stop = miss ? 1 : 0;
        }
      }
      if (lane == 0) s_abort = timed_out ? 1 : 0;
      STACK_PHASE(14);  // wave 0: choices written, at the barrier
    } else {
      uint4 gq[S::NPS][2][CPL];
      uint32_t gsb[S::NPS][2][CPL];
      const int q0 = (wave - 1) * kG + blk;
#pragma unroll
      for (int n = 0; n < S::NPS; ++n) {
        const int p = q0 + n * (kNW - 1) * kG;
        if (p < S::PS) gu_load(D.shared_blob, a.sq, a.ssb, p * RPP + rsub, gq[n], gsb[n]);
      }
#pragma unroll
      for (int n = 0; n < S::NPS; ++n) {
        const int p = q0 + n * (kNW - 1) * kG;
        if (p < S::PS) gu_rows(gq[n], gsb[n], K * I, p * RPP + rsub);
      }
      // shared down items -> LDS, after the loads above have been used
      if constexpr (RO::SPLIT) {
        if (wave >= 4) {
#pragma unroll
          for (int n = 0; n < (S::NIS + 3) / 4; ++n) {
            const int it = K * S::NIR + (wave - 4) + 4 * n;
            if (it < S::NITEMS) down_request(it, D.shared_blob, true);
          }
        }
      } else {
        // waves 1..7 in turn (wave 0 is selecting); whoever computes an item
        // reads it after the workgroup barrier that follows every wave's
        // wait for its own loads
#pragma unroll
        for (int n = 0; n < (S::NIS + kNW - 2) / (kNW - 1); ++n) {
          const int it = K * S::NIR + (wave - 1) + (kNW - 1) * n;
          if (it < S::NITEMS) down_request(it, D.shared_blob, true);
        }
      }
      STACK_PHASE_AT(12, 4 * kWave);  // wave 4: shared work issued, at the barrier
      STACK_PHASE_AT(13, kWave);      // wave 1: the same
    }
    __syncthreads();
    STACK_PHASE(4);  // top-k done (and the shared gate/up)
    if (s_abort) {
      failed = true;
        l_fail = l;
      break;
    }
    if (POOL && s_stop) {  // the same decision in every workgroup
      if (blk == 0 && tid == 0) *a.stop = l;
      break;
    }
    // the shared h (published while the logits were in flight) is requested
    // after the first routed gate/up pass and looked at after the last
    const uint64_t* hrep = reinterpret_cast<const uint64_t*>(hb + (size_t)rep * S::HW);
    uint64_t hsh[h_per<RO::HN, IS / 2>()];

    // ---- routed gate/up: row group gw + n * 8G of K * PR; at most DEPTH
    // passes of weights are in flight per lane
    {
      constexpr int DEPTH = CPL == 1 ? S::NPR : 2;
      uint4 gq[DEPTH][2][CPL];
      uint32_t gsb[DEPTH][2][CPL];
      auto routed_load = [&](int n) {
        const int pr = gw + n * kNW * kG;
        if (pr < K * S::PR) {
          const int j = pr / S::PR;
          const uint8_t* blob =
              POOL ? uniform_ptr(s_addr[j])
                        : D.routed_base + (int64_t)__builtin_amdgcn_readfirstlane(s_sel[j]) * a.stride;
          gu_load(blob, a.lq, a.lsb, (pr % S::PR) * RPP + rsub, gq[n % DEPTH], gsb[n % DEPTH]);
        }
      };
#pragma unroll
      for (int n = 0; n < DEPTH; ++n) routed_load(n);
      if (wave == 0) {
        // renormalised weights = softmax over the chosen logits, summed in j
        // order, and the shared gate (used by wave 0's combine at the end)
        const float ex = lane < K ? expf(s_val[lane] - s_val[0]) : 0.f;
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < K; ++j) sum += readlane_f32(ex, j);
        if (lane < K) {
          const float wj = ex / sum;
          s_w[lane] = wj;
          if (blk == 0 && a.w) a.w[(size_t)l * K + lane] = wj;
        }
        if (lane == 0) s_w[K] = a.has_wsg ? 1.0f / (1.0f + expf(-s_gate_in)) : 0.f;
      }
#pragma unroll
      for (int n = 0; n < S::NPR; ++n) {
        const int pr = gw + n * kNW * kG;
        if (pr < K * S::PR) {
          const int j = pr / S::PR;
          gu_rows(gq[n % DEPTH], gsb[n % DEPTH], j * I, (pr % S::PR) * RPP + rsub);
        }
        if (n + DEPTH < S::NPR) routed_load(n + DEPTH);
        if (n == 0) h_request<RO::HT0, RO::HN, K * I / 2, IS / 2>(hrep, 0u, hsh);
      }
    }

    STACK_PHASE(5);  // routed gate/up done
    // ---- routed down items -> LDS (needed after the h wait)
    auto routed_item = [&](int it) {
      const int j = it / S::NIR;
      const uint8_t* blob =
          POOL ? uniform_ptr(s_addr[j])
               : D.routed_base + (int64_t)__builtin_amdgcn_readfirstlane(s_sel[j]) * a.stride;
      down_request(it, blob, false);
    };
    if constexpr (RO::SPLIT) {
      static_assert(S::NIR % 4 == 0, "split down phase: items of an expert in fours");
      if (wave >= 4) {
        // wave 4 + w takes the items it = j * NIR + w + 4 m of every choice
        // j; the chosen blobs are read once (LDS, then scalar registers)
        const uint8_t* blobs[K];
#pragma unroll
        for (int j = 0; j < K; ++j)
          blobs[j] = POOL ? uniform_ptr(s_addr[j])
                          : D.routed_base + (int64_t)__builtin_amdgcn_readfirstlane(s_sel[j]) * a.stride;
#pragma unroll
        for (int j = 0; j < K; ++j)
#pragma unroll
          for (int m = 0; m < S::NIR / 4; ++m) down_request(j * S::NIR + (wave - 4) + 4 * m, blobs[j], false);
        STACK_PHASE_AT(15, 4 * kWave);  // wave 4: routed down items requested
        wait_vm_n<0>();
        STACK_PHASE_AT(16, 4 * kWave);  // wave 4: its down items landed
      }
    } else {
#pragma unroll
      for (int n = 0; n < S::DN; ++n) {
        const int it = wave + n * kNW;
        if (it < K * S::NIR) routed_item(it);
      }
    }


    // ---- down + combine for rows [row0, row0 + R): shared rows first (its h
    // was published during the logits round trip), then the routed rows
    // per-chunk sums of h (the bias term's X), each once per workgroup
    auto chunk_sums = [&](int c0, int c1) {
      for (int i = c0 + tid; i < c1; i += kNT) {
        const uint4* c4 = reinterpret_cast<const uint4*>(hl + (size_t)i * F::kPairs);
        float hs = 0.f;
#pragma unroll
        for (int v = 0; v < F::kPairs / 4; ++v) {
          const uint4 d = c4[v];
          hs += bf16_lo(d.x) + bf16_hi(d.x);
          hs += bf16_lo(d.y) + bf16_hi(d.y);
          hs += bf16_lo(d.z) + bf16_hi(d.z);
          hs += bf16_lo(d.w) + bf16_hi(d.w);
        }
        hsum[i] = hs;
      }
    };
    auto down_items = [&](bool shared_part) {
#pragma unroll
      for (int n = 0; n < S::DN; ++n) {
        const int it = wave + n * kNW;
        const bool is_shared = it >= K * S::NIR;
        if (it < S::NITEMS && is_shared == shared_part) {
          const int s = is_shared ? K : it / S::NIR;
          const int pp = is_shared ? it - K * S::NIR : it % S::NIR;
          const int C = is_shared ? S::CS : S::CR, RP = is_shared ? S::RPPS : S::RPPR;
          int ci = lane % C, rloc = pp * RP + lane / C;
          // recomputed per layer, not held across the layer loop: the
          // registers are scarcer than the two integer operations
          asm volatile("" : "+v"(ci), "+v"(rloc));
          const int chunk = s * (I / F::kEpc) + ci;  // chunk index in the dense h
          const uint4* hsrc = reinterpret_cast<const uint4*>(hl + (size_t)chunk * F::kPairs);
          uint32_t hp[F::kPairs];
#pragma unroll
          for (int v = 0; v < F::kPairs / 4; ++v) {
            const uint4 d = hsrc[v];
            hp[4 * v] = d.x;
            hp[4 * v + 1] = d.y;
            hp[4 * v + 2] = d.z;
            hp[4 * v + 3] = d.w;
          }
          const uint4 dq = *reinterpret_cast<const uint4*>(dwl + (size_t)it * 1024 + lane * 16);
          const uint32_t dsb = *reinterpret_cast<const uint32_t*>(dsbl + (size_t)it * 256 + lane * 4);
          float acc = chunk_term<BITS>(0.f, dsb, chunk_dot<BITS>(dq, hp), hsum[chunk]);
          acc = group_sum(acc, C);
          if (ci == 0 && rloc < R) part[s * R + rloc] = acc;
        }
      }
    };
    if (!poll_h<RO::HT0, RO::HN, K * I / 2, IS / 2>(hrep, tag16, hl, deadline, hsh)) {
      failed = true;
        l_fail = l;
      break;
    }
    STACK_PHASE(17);  // wave 0: shared h polled, at the barrier
    __syncthreads();
    STACK_PHASE(6);  // shared h received
    wait_vm_n<0>();  // this wave's down-item loads have landed
    // 8-bit split: the routed h's first poll round (waves 0..3) is in
    // flight while the shared rows are computed (measured faster there;
    // with every wave polling, the 4-bit shapes were slower with it)
    uint64_t hrt[h_per<RO::HN, K * I / 2>()];
    if constexpr (RO::SPLIT) h_request<RO::HT0, RO::HN, 0, K * I / 2>(hrep, 0u, hrt);
    chunk_sums(K * I / F::kEpc, S::HW / F::kEpc);
    __syncthreads();
    down_items(true);
    if constexpr (!RO::SPLIT) h_request<RO::HT0, RO::HN, 0, K * I / 2>(hrep, 0u, hrt);
    if (!poll_h<RO::HT0, RO::HN, 0, K * I / 2>(hrep, tag16, hl, deadline, hrt)) {
      failed = true;
        l_fail = l;
      break;
    }
    STACK_PHASE(18);  // wave 0: routed h polled, at the barrier
    __syncthreads();
    STACK_PHASE(7);  // routed h received
    chunk_sums(0, K * I / F::kEpc);
    __syncthreads();
    STACK_PHASE(19);  // routed chunk sums done
    down_items(false);
    __syncthreads();
    STACK_PHASE(8);  // down rows done
    if (tid < R * kRep) {  // kRep threads per row, one per copy
      const int r = tid % R, cp = tid / R, row = row0 + r;
      float y = 0.f;
#pragma unroll
      for (int j = 0; j < K; ++j) y = fmaf(s_w[j], part[j * R + r], y);
      y = fmaf(s_w[K], part[K * R + r], y);
      st_dev(a.ybuf + ((size_t)l * kRep + cp) * H + row, pack64(y, tag));
      if (cp == 0) {
        if (a.y_layers) a.y_layers[(size_t)l * H + row] = y;
        if (l == a.L - 1) a.y_last[row] = (uint16_t)f32_to_bf16(y);
      }
    }
    STACK_PHASE(9);  // y rows published
    // the next layer's router row goes out once this layer's loads are all
    // done (a wave's loads complete in order, so any later wait in this
    // layer would wait for it too); waves 0..3, which own the router rows,
    // do not poll the next y
    if (l + 1 < a.L && rrow < e_rows) {
      const StackLayerDesc& Dn = s_layers[l + 1];
      router_request(Dn);
      if (rrow < E && Dn.rb) rbv = ldf(Dn.rb + rrow);
    }
    // No barrier here: the next LDS writes that could meet this layer's
    // reads (s_w, part, hl) come after the next layer's y wait, itself a
    // workgroup barrier.
  }

  if (failed) {
    // the rows this workgroup owns become NaN in the call's outputs (the
    // final bf16 output and the f32 output of every layer from the one that
    // failed on), so a call that ran out of time never leaves valid-looking
    // data; the host reports the error
    for (int r = tid; r < R; r += kNT) {
      a.y_last[row0 + r] = (uint16_t)0x7FC0u;
      if (a.y_layers)
        for (int lf = l_fail; lf < a.L; ++lf)
          a.y_layers[(size_t)lf * H + row0 + r] = __uint_as_float(0x7FC00000u);
    }
  }
  if (tid == 0) {
    if (failed) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    st_dev(a.epochs + blk, epoch + 1u);
  }
  wait_vm_n<0>();  // no direct-to-LDS load outlives the workgroup's LDS
}

// Zero-fill of n 32-bit words (hand-off buffers whose tags could alias).
__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = 0u;
}

template <class S, int VPL, bool POOL>
hipError_t launch_mode(const StackArgs& a, hipStream_t s) {
  const size_t lds = StackLds<S, VPL>::BYTES;
  hipError_t e = allow_lds(stack_decode_kernel<S, VPL, POOL>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((stack_decode_kernel<S, VPL, POOL>), dim3(kG), dim3(kNT), lds, s, a);
  return hipGetLastError();
}

template <class S, int VPL>
hipError_t launch_shape(const StackArgs& a, hipStream_t s) {
  return a.pool ? launch_mode<S, VPL, true>(a, s) : launch_mode<S, VPL, false>(a, s);
}

// The instances: (bits, H, I, Is, k) x top-k width (64 * VPL >= E).
#define MOE_STACK_SHAPES(X)             \
  X(4, 2048, 512, 512, 8, 4)  /* 256 experts, top-8 */  \
  X(4, 2048, 512, 512, 10, 8) /* 512 experts, top-10 */ \
  X(8, 2048, 512, 512, 10, 8) /* int8, 512 experts, top-10 */ \
  X(4, 256, 64, 64, 2, 1)     /* small test shape */

}  // namespace

bool stack_decode_supported(int H, int E, int k, int I, int Is, int bits, int cus) {
  if (cus < kG || E + 1 > kNW * kG || E < k) return false;
  const int vpl = (E + 63) / 64;
#define MOE_STACK_MATCH(B, HH, II, SS, KK, V) \
  if (bits == B && H == HH && I == II && Is == SS && k == KK && vpl <= V && vpl > V / 2) return true;
  MOE_STACK_SHAPES(MOE_STACK_MATCH)
#undef MOE_STACK_MATCH
  return false;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, s, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_stack_decode(const StackArgs& a, int H, int k, int I, int Is, int bits,
                               hipStream_t s) {
  const int vpl = (a.E + 63) / 64;
#define MOE_STACK_LAUNCH(B, HH, II, SS, KK, V)                                       \
  if (bits == B && H == HH && I == II && Is == SS && k == KK && vpl <= V && vpl > V / 2) \
    return launch_shape<Shape<B, HH, II, SS, KK>, V>(a, s);
  MOE_STACK_SHAPES(MOE_STACK_LAUNCH)
#undef MOE_STACK_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace moe
