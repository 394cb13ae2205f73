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
// * one workgroup per compute unit, all resident (cooperative launch);
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

constexpr int kNT = kStackThreads;
constexpr int kNW = kNT / kWave;
constexpr int kGuMax = kStackGuPasses;
constexpr int kDnMax = kStackDownItems;
constexpr int kHBatch = 8;
constexpr int kHBatches = kStackHPairs / kHBatch;
constexpr int kMaxH = 2048;
constexpr int kRep = kStackReplicas;
constexpr int kWrIt = kMaxH / 256;  // float4 router loads per lane (full row per wave)

__device__ __forceinline__ uint32_t tag32_of(uint32_t epoch) { return 2u * epoch + 1u; }
__device__ __forceinline__ uint32_t tag16_of(uint32_t epoch) { return (epoch & 0x7FFFu) | 0x8000u; }

__device__ __forceinline__ uint64_t pack64(float v, uint32_t tag) {
  return (uint64_t)__float_as_uint(v) | ((uint64_t)tag << 32);
}

// WG-uniform end of one poll round: true when every thread saw all its
// words, false to poll again; *timed_out when the deadline has passed.
__device__ __forceinline__ bool poll_round(bool ok, int64_t deadline, bool* timed_out) {
  if (__syncthreads_and(ok)) return true;
  *timed_out = __syncthreads_or(threadIdx.x == 0 && wall_clock64() > deadline) != 0;
  __builtin_amdgcn_s_sleep(1);
  return false;
}

// Wait for n 64-bit tagged words (n <= PER * kNT) and put their f32 values
// into dst (LDS).  Returns false on timeout.
template <int PER>
__device__ bool poll_f32(const uint64_t* buf, int n, uint32_t tag, float* dst, int64_t deadline) {
  uint32_t done = 0;
  for (;;) {
    uint64_t e[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int i = threadIdx.x + m * kNT;
      e[m] = (i < n && !((done >> m) & 1u)) ? ld_dev(buf + i) : 0ull;
    }
    bool ok = true;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int i = threadIdx.x + m * kNT;
      if (i < n && !((done >> m) & 1u)) {
        if ((uint32_t)(e[m] >> 32) == tag) {
          dst[i] = __uint_as_float((uint32_t)e[m]);
          done |= 1u << m;
        } else {
          ok = false;
        }
      }
    }
    bool to = false;
    if (poll_round(ok, deadline, &to)) return true;
    if (to) return false;
  }
}

// Wait for the previous layer's output y: thread t < 256 takes y[t + 256 m]
// (the per-layer router's order for the sum of squares) into registers.
__device__ bool poll_y(const uint64_t* buf, int H, uint32_t tag, float* yv, int64_t deadline) {
  const int t = threadIdx.x;
  uint32_t done = 0;
  for (;;) {
    uint64_t e[kMaxH / 256];
#pragma unroll
    for (int m = 0; m < kMaxH / 256; ++m) {
      const int i = t + m * 256;
      e[m] = (t < 256 && i < H && !((done >> m) & 1u)) ? ld_dev(buf + i) : 0ull;
    }
    bool ok = true;
#pragma unroll
    for (int m = 0; m < kMaxH / 256; ++m) {
      const int i = t + m * 256;
      if (t < 256 && i < H && !((done >> m) & 1u)) {
        if ((uint32_t)(e[m] >> 32) == tag) {
          yv[m] = __uint_as_float((uint32_t)e[m]);
          done |= 1u << m;
        } else {
          ok = false;
        }
      }
    }
    bool to = false;
    if (poll_round(ok, deadline, &to)) return true;
    if (to) return false;
  }
}

// Wait for this layer's h words (dense: slot j < k at j * I, shared at k * I)
// and stage them in LDS as bf16 pairs: hl[i] = (h[2i], h[2i+1]).
__device__ bool poll_h(const uint32_t* hb, int hwords, uint32_t tag16, uint32_t* hl,
                       int64_t deadline) {
  const int npairs = hwords / 2;
  const uint64_t* src = reinterpret_cast<const uint64_t*>(hb);
  uint32_t done = 0;
  for (;;) {
    bool ok = true;
    for (int bt = 0; bt < kHBatches; ++bt) {
      const int base = threadIdx.x + bt * kHBatch * kNT;
      if (base >= npairs) break;
      uint64_t e[kHBatch];
#pragma unroll
      for (int m = 0; m < kHBatch; ++m) {
        const int i = base + m * kNT;
        e[m] = (i < npairs && !((done >> (bt * kHBatch + m)) & 1u)) ? ld_dev(src + i) : 0ull;
      }
#pragma unroll
      for (int m = 0; m < kHBatch; ++m) {
        const int i = base + m * kNT;
        const int bit = bt * kHBatch + m;
        if (i < npairs && !((done >> bit) & 1u)) {
          const uint32_t w0 = (uint32_t)e[m], w1 = (uint32_t)(e[m] >> 32);
          if ((w0 & 0xFFFFu) == tag16 && (w1 & 0xFFFFu) == tag16) {
            hl[i] = perm(w1, w0, 0x07060302u);  // (bf16 of w0, bf16 of w1)
            done |= 1u << bit;
          } else {
            ok = false;
          }
        }
      }
    }
    bool to = false;
    if (poll_round(ok, deadline, &to)) return true;
    if (to) return false;
  }
}

template <int BITS, int VPL, int CPL>
__global__ __launch_bounds__(kNT, 1) void stack_decode_kernel(StackArgs a) {
  using F = Fmt<BITS>;
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float red[4];
  __shared__ int s_sel[MOE_MAX_TOPK];
  __shared__ float s_val[MOE_MAX_TOPK];
  __shared__ float s_w[MOE_MAX_TOPK + 1];
  __shared__ int tmp_e[MOE_MAX_TOPK];
  __shared__ float tmp_v[MOE_MAX_TOPK];

  const int H = a.H, E = a.E, k = a.k, I = a.I, Is = a.Is;
  const int R = a.rows_per_wg;
  const int blk = blockIdx.x, G = gridDim.x;
  const int wv0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln0 = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int e_rows = E + (a.has_wsg ? 1 : 0);

  // LDS carve-up (sizes as in stack_lds_bytes)
  float* xf = reinterpret_cast<float*>(smem);                       // [H] f32 input
  uint16_t* xb = reinterpret_cast<uint16_t*>(smem + (size_t)H * 4);  // [H] bf16 input
  float* lg = reinterpret_cast<float*>(smem + (size_t)H * 6);        // [E + 1] logits
  uint32_t* hl = reinterpret_cast<uint32_t*>(smem + (size_t)H * 6 + ((size_t)(E + 1) * 4 + 15) / 16 * 16);
  float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(hl) + ((size_t)a.hwords * 2 + 15) / 16 * 16);

  const int rep = blk % kRep;  // the XCD of this workgroup
  const uint32_t epoch = ld_dev(a.epochs + blk);
  const uint32_t tag = tag32_of(epoch), tag16 = tag16_of(epoch);
  const int64_t deadline = wall_clock64() + a.timeout_ticks;
  bool failed = false;

  for (int l = 0; l < a.L && !failed; ++l) {
    // The per-row-group index arithmetic below is cheap; hoisted out of the
    // layer loop it would hold hundreds of registers for the whole loop.
    // An empty asm makes the ids opaque per layer so it is redone each time.
    int b = blk, wave = wv0, lane = ln0;
    asm volatile("" : "+s"(b), "+s"(wave), "+v"(lane));
    // gate/up geometry: a row group is RPP rows, one wave pass
    const int Cg = H / F::kEpc, LPR = Cg / CPL, RPP = kWave / LPR;
    const int sub = lane % LPR, rsub = lane / LPR;
    const int64_t row_bytes_g = (int64_t)H * BITS / 8;
    const int Gg = H / 64;
    const int Ps = a.has_shared ? Is / RPP : 0, Pr = I / RPP;
    const int P = Ps + k * Pr;
    const int gw = wave * G + b;  // global wave index

    // down geometry: this workgroup's rows [row0, row0 + R)
    const int row0 = b * R;
    const int Cr = I / F::kEpc, Cs = a.has_shared ? Is / F::kEpc : 1;
    const int RPPr = kWave / Cr, RPPs = kWave / Cs;
    const int NIr = (R + RPPr - 1) / RPPr, NIs = a.has_shared ? (R + RPPs - 1) / RPPs : 0;
    const int n_items = k * NIr + NIs;
    const StackLayerDesc D = a.layers[l];

    // ---- requests that do not depend on routing: router row, shared expert
    const int rrow = b + G * wave;  // router row of this wave (E = the shared gate)
    float4 wv[kWrIt];
    if (rrow < e_rows) {
      const float* wr = rrow < E ? D.Wr + (size_t)rrow * H : D.wsg;
#pragma unroll
      for (int m = 0; m < kWrIt; ++m)
        if (m * 256 < H) wv[m] = *reinterpret_cast<const float4*>(wr + m * 256 + lane * 4);
    }

    uint4 gq[kGuMax][2][CPL];
    uint32_t gsb[kGuMax][2][CPL];
#pragma unroll
    for (int n = 0; n < kGuMax; ++n) {
      const int p = gw + n * kNW * G;
      if (p < Ps) {
        const int row = p * RPP + rsub;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint8_t* qb = D.shared_blob + a.ls.q_off[m] + (int64_t)row * row_bytes_g;
          const uint32_t* sbb = reinterpret_cast<const uint32_t*>(D.shared_blob + a.ls.sb_off[m]) +
                                (int64_t)row * Gg;
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const int ci = sub + c * LPR;
            gq[n][m][c] = ld16(qb + ci * 16);
            gsb[n][m][c] = sbb[ci * F::kEpc / 64];
          }
        }
      }
    }

    uint4 dq[kDnMax];
    uint32_t dsb[kDnMax];
#pragma unroll
    for (int n = 0; n < kDnMax; ++n) {
      const int it = wave + n * kNW;
      if (it >= k * NIr && it < n_items) {
        const int pp = it - k * NIr;
        const int ci = lane % Cs, rloc = pp * RPPs + lane / Cs, row = row0 + rloc;
        dq[n] = make_uint4(0, 0, 0, 0);
        dsb[n] = 0;
        if (rloc < R && row < H) {
          dq[n] = ld16(D.shared_blob + a.ls.q_off[2] + (int64_t)row * (Is * BITS / 8) + ci * 16);
          dsb[n] = reinterpret_cast<const uint32_t*>(D.shared_blob + a.ls.sb_off[2])
              [(int64_t)row * (Is / 64) + ci * F::kEpc / 64];
        }
      }
    }

    // ---- layer input: x0, or bf16(y / rms(y)) of the previous layer
    if (l == 0) {
      for (int i = tid; i < H; i += kNT) {
        const uint16_t v = a.x0[i];
        xb[i] = v;
        xf[i] = bf16_to_f32(v);
        if (b == 0 && a.x_layers) a.x_layers[i] = v;
      }
      __syncthreads();
    } else {
      float yv[kMaxH / 256];
      if (!poll_y(a.ybuf + ((size_t)(l - 1) * kRep + rep) * H, H, tag, yv, deadline)) {
        failed = true;
        break;
      }
      // sum of squares in the per-layer router's order (256 threads)
      if (tid < 256) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < kMaxH / 256; ++m)
          if (tid + m * 256 < H) s = fmaf(yv[m], yv[m], s);
        s = group_sum(s, kWave);
        if (lane == 0) red[tid >> 6] = s;
      }
      __syncthreads();
      const float tot = ((red[0] + red[1]) + red[2]) + red[3];
      const float r = 1.0f / sqrtf(tot / (float)H + 1e-6f);
      if (tid < 256) {
#pragma unroll
        for (int m = 0; m < kMaxH / 256; ++m) {
          const int i = tid + m * 256;
          if (i < H) {
            const uint32_t bb = f32_to_bf16(yv[m] * r);
            xb[i] = (uint16_t)bb;
            xf[i] = bf16_to_f32(bb);
            if (b == 0 && a.x_layers) a.x_layers[(size_t)l * H + i] = (uint16_t)bb;
          }
        }
      }
      __syncthreads();
    }

    // ---- router row: halves summed separately, as the per-layer router
    if (rrow < e_rows) {
      const int nit = H / 256;
      const int half = (H % 512 == 0) ? nit / 2 : nit;
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
      for (int m = 0; m < kWrIt; ++m) {
        if (m < nit) {
          const float4 xv = *reinterpret_cast<const float4*>(xf + m * 256 + lane * 4);
          float s = m < half ? acc0 : acc1;
          s = fmaf(wv[m].x, xv.x, s);
          s = fmaf(wv[m].y, xv.y, s);
          s = fmaf(wv[m].z, xv.z, s);
          s = fmaf(wv[m].w, xv.w, s);
          if (m < half) acc0 = s; else acc1 = s;
        }
      }
      acc0 = group_sum(acc0, kWave);
      float out = acc0;
      if (half < nit) out = acc0 + group_sum(acc1, kWave);
      if (lane < kRep) {
        const float v = rrow < E ? out + (D.rb ? D.rb[rrow] : 0.f) : out;
        st_dev(a.lbuf + ((size_t)l * kRep + lane) * (E + 1) + rrow, pack64(v, tag));
      }
    }

    // ---- selection: every workgroup runs the top-k on all logits
    if (!poll_f32<(1024 + 1 + kNT - 1) / kNT>(a.lbuf + ((size_t)l * kRep + rep) * (E + 1), e_rows,
                                             tag, lg, deadline)) {
      failed = true;
      break;
    }
    if (wave == 0) {
      float v[VPL];
      uint32_t key[VPL];
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = lane + kWave * i;
        v[i] = e < E ? lg[e] : 0.f;
        key[i] = e < E ? order_key(v[i]) : 0u;
      }
      wave_topk<VPL>(v, key, k, tmp_e, tmp_v, s_sel, s_val);
      // renormalised weights = softmax over the chosen logits, summed in j order
      const float ex = lane < k ? expf(s_val[lane] - s_val[0]) : 0.f;
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOPK; ++j)
        if (j < k) sum += readlane_f32(ex, j);
      if (lane < k) {
        const float wj = ex / sum;
        s_w[lane] = wj;
        if (b == 0 && a.w) a.w[(size_t)l * k + lane] = wj;
        if (b == 0 && a.idx) a.idx[(size_t)l * k + lane] = s_sel[lane];
      }
      if (lane == 0) s_w[k] = a.has_wsg ? 1.0f / (1.0f + expf(-lg[E])) : 0.f;
    }
    __syncthreads();

    // ---- routed gate/up requests
#pragma unroll
    for (int n = 0; n < kGuMax; ++n) {
      const int p = gw + n * kNW * G;
      if (p >= Ps && p < P) {
        const int pr = p - Ps, j = pr / Pr;
        const int row = (pr - j * Pr) * RPP + rsub;
        const uint8_t* blob = D.routed_base + (int64_t)__builtin_amdgcn_readfirstlane(s_sel[j]) * a.stride;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint8_t* qb = blob + a.lr.q_off[m] + (int64_t)row * row_bytes_g;
          const uint32_t* sbb = reinterpret_cast<const uint32_t*>(blob + a.lr.sb_off[m]) +
                                (int64_t)row * Gg;
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const int ci = sub + c * LPR;
            gq[n][m][c] = ld16(qb + ci * 16);
            gsb[n][m][c] = sbb[ci * F::kEpc / 64];
          }
        }
      }
    }

    // ---- gate/up: h = bf16(silu(g) * u) for this wave's row groups
    uint32_t* hb = a.hbuf + (size_t)l * kRep * a.hwords;
    {
      uint32_t xp[CPL][F::kPairs];
      float xs[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int ci = sub + c * LPR;
        pair_natural<BITS>(reinterpret_cast<const uint4*>(xb + ci * F::kEpc), xp[c], xs[c]);
      }
#pragma unroll
      for (int n = 0; n < kGuMax; ++n) {
        const int p = gw + n * kNW * G;
        if (p < P) {
          int base, row;
          if (p < Ps) {
            base = k * I;
            row = p * RPP + rsub;
          } else {
            const int pr = p - Ps, j = pr / Pr;
            base = j * I;
            row = (pr - j * Pr) * RPP + rsub;
          }
          float g = 0.f, u = 0.f;
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            g = chunk_term<BITS>(g, gsb[n][0][c], chunk_dot<BITS>(gq[n][0][c], xp[c]), xs[c]);
            u = chunk_term<BITS>(u, gsb[n][1][c], chunk_dot<BITS>(gq[n][1][c], xp[c]), xs[c]);
          }
          g = group_sum(g, LPR);
          u = group_sum(u, LPR);
          if (sub < kRep) {  // every lane of the row group holds g and u
            const float hv = g / (1.0f + __expf(-g)) * u;
            st_dev(hb + (size_t)sub * a.hwords + base + h_pos<BITS>(row),
                   (f32_to_bf16(hv) << 16) | tag16);
          }
        }
      }
    }

    // ---- routed down requests for this workgroup's rows (needed after the h wait)
#pragma unroll
    for (int n = 0; n < kDnMax; ++n) {
      const int it = wave + n * kNW;
      if (it < k * NIr) {
        const int j = it / NIr, pp = it - j * NIr;
        const int ci = lane % Cr, rloc = pp * RPPr + lane / Cr, row = row0 + rloc;
        const uint8_t* blob = D.routed_base + (int64_t)__builtin_amdgcn_readfirstlane(s_sel[j]) * a.stride;
        dq[n] = make_uint4(0, 0, 0, 0);
        dsb[n] = 0;
        if (rloc < R && row < H) {
          dq[n] = ld16(blob + a.lr.q_off[2] + (int64_t)row * (I * BITS / 8) + ci * 16);
          dsb[n] = reinterpret_cast<const uint32_t*>(blob + a.lr.sb_off[2])
              [(int64_t)row * (I / 64) + ci * F::kEpc / 64];
        }
      }
    }

    // ---- down + combine for rows [row0, row0 + R)
    if (!poll_h(hb + (size_t)rep * a.hwords, a.hwords, tag16, hl, deadline)) {
      failed = true;
      break;
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < kDnMax; ++n) {
      const int it = wave + n * kNW;
      if (it < n_items) {
        int s, C, pp, RPPx;
        if (it < k * NIr) {
          s = it / NIr;
          pp = it - s * NIr;
          C = Cr;
          RPPx = RPPr;
        } else {
          s = k;
          pp = it - k * NIr;
          C = Cs;
          RPPx = RPPs;
        }
        const int ci = lane % C, rloc = pp * RPPx + lane / C;
        const uint4* hsrc = reinterpret_cast<const uint4*>(hl + (size_t)s * (I / 2) + ci * (F::kEpc / 2));
        uint32_t hp[F::kPairs];
#pragma unroll
        for (int v = 0; v < F::kPairs / 4; ++v) {
          const uint4 d = hsrc[v];
          hp[4 * v] = d.x;
          hp[4 * v + 1] = d.y;
          hp[4 * v + 2] = d.z;
          hp[4 * v + 3] = d.w;
        }
        float hs = 0.f;
#pragma unroll
        for (int v = 0; v < F::kPairs; ++v) hs += bf16_lo(hp[v]) + bf16_hi(hp[v]);
        float acc = chunk_term<BITS>(0.f, dsb[n], chunk_dot<BITS>(dq[n], hp), hs);
        acc = group_sum(acc, C);
        if (ci == 0 && rloc < R) part[s * R + rloc] = acc;
      }
    }
    __syncthreads();
    if (tid < R * kRep) {  // kRep threads per row, one per copy
      const int r = tid % R, cp = tid / R, row = row0 + r;
      if (row < H) {
        float y = 0.f;
#pragma unroll
        for (int j = 0; j < MOE_MAX_TOPK; ++j)
          if (j < k) y = fmaf(s_w[j], part[j * R + r], y);
        if (a.has_shared) y = fmaf(s_w[k], part[k * R + r], y);
        st_dev(a.ybuf + ((size_t)l * kRep + cp) * H + row, pack64(y, tag));
        if (cp == 0) {
          if (a.y_layers) a.y_layers[(size_t)l * H + row] = y;
          if (l == a.L - 1) a.y_last[row] = (uint16_t)f32_to_bf16(y);
        }
      }
    }
    __syncthreads();
  }

  if (tid == 0) {
    if (failed) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    st_dev(a.epochs + blk, epoch + 1u);
  }
}

template <int BITS, int CPL>
hipError_t launch_bits(const StackArgs& a, int grid, hipStream_t s) {
  const int vpl = (a.E + 63) / 64;
  void* args[] = {const_cast<StackArgs*>(&a)};
#define MOE_STACK_CASE(V)                                                                    \
  if (vpl <= V) {                                                                            \
    const void* fn = reinterpret_cast<const void*>(&stack_decode_kernel<BITS, V, CPL>);      \
    hipError_t e = allow_lds(stack_decode_kernel<BITS, V, CPL>, a.lds_bytes);                \
    if (e != hipSuccess) return e;                                                           \
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kNT), args, (unsigned)a.lds_bytes, s); \
  }
  MOE_STACK_CASE(1)
  MOE_STACK_CASE(2)
  MOE_STACK_CASE(4)
  MOE_STACK_CASE(8)
  MOE_STACK_CASE(16)
#undef MOE_STACK_CASE
  return hipErrorInvalidValue;
}

}  // namespace

size_t stack_lds_bytes(int H, int E, int k, int hwords, int rows_per_wg) {
  return (size_t)H * 6 + ((size_t)(E + 1) * 4 + 15) / 16 * 16 + ((size_t)hwords * 2 + 15) / 16 * 16 +
         (size_t)(k + 1) * rows_per_wg * 4;
}

bool stack_decode_supported(int H, int E, int k, int I, int Is, int bits, int grid) {
  if (!decode_shape_supported(H, I, Is, bits) || grid < 1) return false;
  if (E + 1 > kNW * grid || E > 1024) return false;  // one router row per wave
  const int epc = 128 / bits;
  const int C = H / epc, cpl = C <= 64 ? 1 : C / 64;
  const int rpp = kWave / (C / cpl);
  if (Is + k * I > (int64_t)kGuMax * kNW * grid * rpp) return false;
  const int R = (H + grid - 1) / grid;
  const int ni = k * ((R + kWave / (I / epc) - 1) / (kWave / (I / epc))) +
                 (R + kWave / (Is / epc) - 1) / (kWave / (Is / epc));
  if (ni > kDnMax * kNW) return false;
  if ((k * I + Is) / 2 > kStackHPairs * kNT) return false;
  if (R * kRep > kNT) return false;
  return stack_lds_bytes(H, E, k, k * I + Is, R) + 1024 <= 160 * 1024;
}

hipError_t launch_stack_decode(const StackArgs& a, int grid, hipStream_t s) {
  const int C = a.H / (128 / a.bits);
  if (a.bits == 4) return launch_bits<4, 1>(a, grid, s);
  if (C <= 64) return launch_bits<8, 1>(a, grid, s);
  return launch_bits<8, 2>(a, grid, s);
}

}  // namespace moe
