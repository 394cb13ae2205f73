// Router: logits GEMV, then softmax / top-k / renormalise.
//
// Each layer sends a token to k of E routed experts (10 of 512 in the 80B
// model, 8 of 256 in the 35B model) -- [xix] how-it-works paragraph; [lens]
// "エキスパートストリーミングの仕組み".  The router stays resident and
// unquantised in f32 (the pages list routers among the dense weights kept in
// memory).
//
// Kernel shape (decode, T <= 8 tokens; 256 threads for one token, 512 for
// up to 8):
//   * the layer input is staged once per workgroup in LDS as f32; for layer
//     l > 0 of a stack it is bf16(y_{l-1} / rms(y_{l-1})), computed here;
//   * one 64-lane wave streams half a row of Wr (or all of it for H < 512)
//     with 16-byte loads and keeps all T token sums in registers, so Wr is
//     read exactly once per call;
//   * the last workgroup to finish (device-scope ticket) reads the E logits
//     back and runs the top-k on one wave per token (a bitwise search for
//     the k-th largest key with ballot counts, see wave_topk).  Selection
//     compares logits (softmax is monotone); ties go to the lower expert
//     index.
//   * the same workgroup builds the list of distinct experts of the call
//     (first appearance order) and, per distinct expert, which slot j each
//     token gave it -- the expert kernels read every chosen expert once.
#include "device.h"
#include "kernels.h"

namespace moe {
namespace {

using namespace dev;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxIt = 8;  // 16-byte Wr loads per lane: H / (256 * waves per row) <= 8

// The layer input of up to NT tokens in LDS as f32: x, or bf16(y / rms(y))
// of the previous layer.  Every thread requests all of its values before it
// uses any (one memory round trip, not one per value).  The sums of squares
// have a fixed order whatever the workgroup size: thread t of a group of 256
// adds y[t + 256 m] over m, then a 64-lane sum per wave, then
// ((w0 + w1) + w2) + w3 over the group's four waves; with THR = 512 the two
// groups take tokens [0, NT/2) and [NT/2, NT).
template <int NT, int THR>
__device__ void stage_input(const RouteArgs& a, float* xs, float (*red)[4], int T) {
  constexpr int MM = 8;            // values per thread and token: H <= 2048 on the stacked path
  constexpr int NG = THR / 256;    // token groups
  constexpr int NTG = (NT + NG - 1) / NG;
  const int tid = threadIdx.x & 255, grp = threadIdx.x >> 8;
  const int H = a.H;
  if (a.y_prev) {
    float v[NTG][MM];
#pragma unroll
    for (int tt = 0; tt < NTG; ++tt)
#pragma unroll
      for (int m = 0; m < MM; ++m) {
        const int t = grp * NTG + tt, i = tid + m * 256;
        v[tt][m] = (t < T && i < H) ? a.y_prev[(size_t)t * H + i] : 0.f;
      }
#pragma unroll
    for (int tt = 0; tt < NTG; ++tt) {
      const int t = grp * NTG + tt;
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < MM; ++m)
        if (tid + m * 256 < H) s = fmaf(v[tt][m], v[tt][m], s);
      s = group_sum(s, kWave);
      if ((tid & 63) == 0 && t < NT) red[t][tid >> 6] = s;
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < NTG; ++tt) {
      const int t = grp * NTG + tt;
      if (t < T) {
        const float tot = ((red[t][0] + red[t][1]) + red[t][2]) + red[t][3];
        const float r = 1.0f / sqrtf(tot / (float)H + 1e-6f);
#pragma unroll
        for (int m = 0; m < MM; ++m) {
          const int i = tid + m * 256;
          if (i < H) {
            const uint32_t b = f32_to_bf16(v[tt][m] * r);
            xs[t * H + i] = bf16_to_f32(b);
            if (blockIdx.x == 0 && a.x_out) a.x_out[(size_t)t * H + i] = (uint16_t)b;
          }
        }
      }
    }
  } else {
    const int n = T * H;
    const int th = threadIdx.x;
    for (int base = 0; base < n; base += THR * MM) {
      uint16_t v[MM];
#pragma unroll
      for (int u = 0; u < MM; ++u) {
        const int i = base + th + u * THR;
        v[u] = i < n ? a.x[i] : (uint16_t)0;
      }
#pragma unroll
      for (int u = 0; u < MM; ++u) {
        const int i = base + th + u * THR;
        if (i < n) {
          xs[i] = bf16_to_f32(v[u]);
          if (blockIdx.x == 0 && a.x_out) a.x_out[i] = v[u];
        }
      }
    }
  }
}

// Top-k of tokens [t0, t1), one wave per token (ballot radix-select, see
// wave_topk); selections go to LDS.  Logits are read from the device
// coherence point: they may have been written by workgroups on other XCDs.
// With MFMA partial sums (a.part) the logits are formed here, and with
// s_sraw the shared gate's input x . wsg of each token goes to s_sraw.
template <int VPL, int NW>
__device__ void topk_tokens(const RouteArgs& a, int t0, int t1, int* s_sel, float* s_val,
                            float* s_sraw) {
  __shared__ int tmp_e[NW][kWave];
  __shared__ float tmp_v[NW][kWave];
  __shared__ uint32_t tmp_k[NW][kWave];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int E = a.E, k = a.k;
  for (int t = t0 + wave; t < t1; t += NW) {
    const float* lg = a.logits + (size_t)t * E;
    float v[VPL];
    uint32_t key[VPL];
    if (a.part) {
      // partial sums of the MFMA router (earlier launch): every load in
      // flight at once, then the slices added in order, then rb
      float pv[VPL][kRouterMaxSplits], bv[VPL];
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = lane + kWave * i;
#pragma unroll
        for (int sp = 0; sp < kRouterMaxSplits; ++sp)
          pv[i][sp] = e < E && sp < a.ksplit ? a.part[((size_t)sp * a.T + t) * E + e] : 0.f;
        bv[i] = e < E && a.rb ? a.rb[e] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = lane + kWave * i;
        float s = 0.f;
        if (e < E) {
          s = pv[i][0];
#pragma unroll
          for (int sp = 1; sp < kRouterMaxSplits; ++sp)
            if (sp < a.ksplit) s += pv[i][sp];
          s += bv[i];
          if (a.logits) a.logits[(size_t)t * E + e] = s;
        }
        v[i] = s;
        key[i] = e < E ? order_key(s) : 0u;
      }
      if (s_sraw) {
        // shared gate input wsg . x[t], f32, lane-strided then one wave sum
        float g = 0.f;
        for (int h = lane * 8; h < a.H; h += kWave * 8) {
          const uint4 q = ld16(a.x + (size_t)t * a.H + h);
          const float4 w0 = ldf4(a.wsg + h), w1 = ldf4(a.wsg + h + 4);
          g = fmaf(bf16_lo(q.x), w0.x, g);
          g = fmaf(bf16_hi(q.x), w0.y, g);
          g = fmaf(bf16_lo(q.y), w0.z, g);
          g = fmaf(bf16_hi(q.y), w0.w, g);
          g = fmaf(bf16_lo(q.z), w1.x, g);
          g = fmaf(bf16_hi(q.z), w1.y, g);
          g = fmaf(bf16_lo(q.w), w1.z, g);
          g = fmaf(bf16_hi(q.w), w1.w, g);
        }
        g = group_sum(g, kWave);
        if (lane == 0) s_sraw[t - t0] = g;
      }
    } else {
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = lane + kWave * i;
        v[i] = e < E ? ld_dev(lg + e) : 0.f;
        key[i] = e < E ? order_key(v[i]) : 0u;
      }
    }
    wave_topk<VPL>(v, key, k, tmp_e[wave], tmp_v[wave], tmp_k[wave], s_sel + (t - t0) * k,
                   s_val + (t - t0) * k);
  }
}

// Renormalised weights over the chosen k (= softmax over the chosen
// logits: the full-softmax denominator cancels) and the shared gate.
template <int THR>
__device__ void write_weights(const RouteArgs& a, int t0, int t1, const int* s_sel,
                              const float* s_val, const float* s_sraw) {
  const int k = a.k;
  for (int t = t0 + (int)threadIdx.x; t < t1; t += THR) {
    const int r = t - t0;
    const float m = s_val[r * k];
    float ex[MOE_MAX_TOPK];
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k) {
        ex[j] = expf(s_val[r * k + j] - m);
        sum += ex[j];
      }
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k) {
        a.w[(size_t)t * k + j] = ex[j] / sum;
        a.idx[(size_t)t * k + j] = s_sel[r * k + j];
      }
    }
    if (a.sigma && a.wsg)
      a.sigma[t] = 1.0f / (1.0f + expf(-(s_sraw ? s_sraw[r] : ld_dev(a.sigma + t))));
    if (a.counts) {
      for (int j = 0; j < k; ++j) atomicAdd(a.counts + s_sel[r * k + j], 1);
    }
  }
}

// Distinct experts of the call in first-appearance order (token-major).
template <int THR>
__device__ void build_slots(const RouteArgs& a, const int* s_sel, int* s_first, int* s_slot) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = a.T * a.k, k = a.k;
  for (int e = threadIdx.x; e < a.E; e += THR) s_first[e] = 0x7fffffff;
  for (int i = threadIdx.x; i < n * kJmapStride; i += THR) a.jmap[i] = -1;
  __syncthreads();
  for (int p = threadIdx.x; p < n; p += THR) atomicMin(&s_first[s_sel[p]], p);
  __syncthreads();
  if (wave == 0) {
    int base = 0;
    for (int p0 = 0; p0 < n; p0 += kWave) {
      const int p = p0 + lane;
      const bool first = p < n && s_first[s_sel[p]] == p;
      const unsigned long long b = __ballot(first);
      if (p < n) s_slot[p] = first ? base + __popcll(b & ((1ull << lane) - 1ull)) : -1;
      base += __popcll(b);
    }
    if (lane == 0) {
      *a.n_slots = base;
      if (a.host_list) a.host_list[1] = base;
    }
  }
  __syncthreads();
  __shared__ int s_miss;
  if (threadIdx.x == 0) s_miss = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < n; p += THR) {
    const int e = s_sel[p];
    const int slot = s_slot[s_first[e]];
    a.jmap[slot * kJmapStride + p / k] = (int8_t)(p % k);
    if (s_first[e] == p) {
      a.slot_expert[slot] = e;
      if (a.host_list) a.host_list[2 + slot] = e;
      if (a.res_tab) {
        const uint8_t* addr = a.res_tab[e];
        a.slot_addr[slot] = addr;
        if (!addr) s_miss = 1;
      }
    }
  }
  if (a.res_tab) {
    __syncthreads();
    if (threadIdx.x == 0) {
      const int go = s_miss ? 0 : 1;
      *a.go = go;
      if (a.host_list) a.host_list[2 + n] = go;
    }
  }
  if (a.host_list) {
    // the host polls word 0: everything above is visible before it changes
    __syncthreads();
    if (threadIdx.x == 0) {
      __threadfence_system();
      __hip_atomic_store(a.host_list, a.host_epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

// GEMV over Wr (and wsg as row E) for up to NT tokens: blockIdx.y selects a
// tile of NT tokens.  With a ticket counter the last block runs the top-k
// (one wave per token: THR = 512 takes 8 tokens in one round).
template <int NT, int VPL, int THR>
__global__ __launch_bounds__(THR) void route_kernel(RouteArgs a) {
  constexpr int NW = THR / kWave;
  extern __shared__ __align__(16) float xs[];  // [NT][H]
  __shared__ float red_t[NT][4];
  __shared__ float halves[NW][NT];
  __shared__ int s_last;

  const int t0 = blockIdx.y * NT;
  const int T = min(NT, a.T - t0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H = a.H, E = a.E;
  const int rows = E + (a.wsg && a.sigma ? 1 : 0);
  const int wpr = (H % 512 == 0) ? 2 : 1;
  const int item = blockIdx.x * NW + wave;
  const int row = item / wpr, part = item % wpr;
  const int span = H / wpr, c0 = part * span, nit = span / (4 * kWave);

  // Wr does not depend on the input: start its loads before staging x.
  float4 wv[kMaxIt];
  if (row < rows) {
    const float* wr = row < E ? a.Wr + (size_t)row * H : a.wsg;
#pragma unroll
    for (int i = 0; i < kMaxIt; ++i)
      if (i < nit) wv[i] = ldf4(wr + c0 + lane * 4 + i * 4 * kWave);
  }

  RouteArgs b = a;
  if (a.x) b.x = a.x + (size_t)t0 * a.H;
  if (a.y_prev) b.y_prev = a.y_prev + (size_t)t0 * a.H;
  if (a.x_out) b.x_out = a.x_out + (size_t)t0 * a.H;
  stage_input<NT, THR>(b, xs, red_t, T);
  __syncthreads();

  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.f;
  if (row < rows) {
#pragma unroll
    for (int i = 0; i < kMaxIt; ++i) {
      if (i < nit) {
        const int c = c0 + lane * 4 + i * 4 * kWave;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t < T) {
            const float4 xv = *reinterpret_cast<const float4*>(xs + t * H + c);
            float s = acc[t];
            s = fmaf(wv[i].x, xv.x, s);
            s = fmaf(wv[i].y, xv.y, s);
            s = fmaf(wv[i].z, xv.z, s);
            s = fmaf(wv[i].w, xv.w, s);
            acc[t] = s;
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = group_sum(acc[t], kWave);
  }
  float out[NT];
  if (wpr == 2) {
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t) halves[wave][t] = acc[t];
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) out[t] = halves[wave & ~1][t] + halves[wave | 1][t];
  } else {
#pragma unroll
    for (int t = 0; t < NT; ++t) out[t] = acc[t];
  }
  if (row < rows && part == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < T && lane == t) {
        if (row < E)
          st_dev(a.logits + (size_t)(t0 + t) * E + row, out[t] + (a.rb ? a.rb[row] : 0.f));
        else
          st_dev(a.sigma + t0 + t, out[t]);
      }
    }
  }

  if (!a.counter) return;
  // Last block: the logits stores of every block are complete at the
  // device coherence point before that block takes its ticket.
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (ticket(a.counter) == gridDim.x - 1) ? 1 : 0;
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0) st_dev(a.counter, 0u);

  __shared__ int s_sel[NT * MOE_MAX_TOPK];
  __shared__ float s_val[NT * MOE_MAX_TOPK];
  __shared__ int s_slot[NT * MOE_MAX_TOPK];
  __shared__ int s_first[1024];
  __shared__ float s_sraw[NT];
  // the shared gate's inputs x . wsg are requested together with the
  // logits (one round trip to the coherence point, not two)
  const bool gate = a.sigma && a.wsg && (int)threadIdx.x < a.T;
  const float sraw = gate ? ld_dev(a.sigma + threadIdx.x) : 0.f;
  topk_tokens<VPL, NW>(a, 0, a.T, s_sel, s_val, nullptr);
  if (gate) s_sraw[threadIdx.x] = sraw;
  __syncthreads();
  write_weights<THR>(a, 0, a.T, s_sel, s_val, a.sigma && a.wsg ? s_sraw : nullptr);
  if (a.n_slots) build_slots<THR>(a, s_sel, s_first, s_slot);
}

// Top-k over logits written by an earlier launch (or formed here from the
// MFMA router's partial sums), 4 tokens per block.
template <int VPL>
__global__ __launch_bounds__(kThreads) void topk_kernel(RouteArgs a) {
  __shared__ int s_sel[kWaves * MOE_MAX_TOPK];
  __shared__ float s_val[kWaves * MOE_MAX_TOPK];
  __shared__ float s_sraw[kWaves];
  const int t0 = blockIdx.x * kWaves;
  const int t1 = min(a.T, t0 + kWaves);
  float* sr = a.part && a.sigma && a.wsg ? s_sraw : nullptr;
  topk_tokens<VPL, kWaves>(a, t0, t1, s_sel, s_val, sr);
  __syncthreads();
  write_weights<kThreads>(a, t0, t1, s_sel, s_val, sr);
}

template <int NT>
hipError_t launch_route_nt(const RouteArgs& a, hipStream_t s, bool fused) {
  constexpr int THR = NT == 1 ? 256 : 512;
  constexpr int NW = THR / kWave;
  const int rows = a.E + (a.wsg && a.sigma ? 1 : 0);
  const int wpr = (a.H % 512 == 0) ? 2 : 1;
  dim3 grid((rows * wpr + NW - 1) / NW, fused ? 1 : (a.T + NT - 1) / NT);
  const size_t lds = (size_t)NT * a.H * sizeof(float);
  RouteArgs b = a;
  if (!fused) {
    b.counter = nullptr;
  }
  const int vpl = (a.E + 63) / 64;
#define MOE_ROUTE_CASE(V)                                                           \
  if (vpl <= V) {                                                                   \
    hipError_t e = allow_lds(route_kernel<NT, V, THR>, lds);                        \
    if (e != hipSuccess) return e;                                                  \
    hipLaunchKernelGGL((route_kernel<NT, V, THR>), grid, dim3(THR), lds, s, b);     \
    return hipGetLastError();                                                       \
  }
  MOE_ROUTE_CASE(1)
  MOE_ROUTE_CASE(2)
  MOE_ROUTE_CASE(4)
  MOE_ROUTE_CASE(8)
  MOE_ROUTE_CASE(16)
#undef MOE_ROUTE_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T <= 1) return launch_route_nt<1>(a, s, a.counter != nullptr);
  if (a.T <= MOE_MAX_DECODE_T) return launch_route_nt<MOE_MAX_DECODE_T>(a, s, a.counter != nullptr);
  // Many tokens: GEMV over token tiles only; the top-k runs as its own launch.
  return launch_route_nt<MOE_MAX_DECODE_T>(a, s, false);
}

hipError_t launch_topk_only(const RouteArgs& a, hipStream_t s) {
  dim3 grid((a.T + kWaves - 1) / kWaves);
  const int vpl = (a.E + 63) / 64;
#define MOE_TOPK_CASE(V)                                                         \
  if (vpl <= V) {                                                                \
    hipLaunchKernelGGL((topk_kernel<V>), grid, dim3(kThreads), 0, s, a);         \
    return hipGetLastError();                                                    \
  }
  MOE_TOPK_CASE(1)
  MOE_TOPK_CASE(2)
  MOE_TOPK_CASE(4)
  MOE_TOPK_CASE(8)
  MOE_TOPK_CASE(16)
#undef MOE_TOPK_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
