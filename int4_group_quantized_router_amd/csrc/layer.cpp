// MoE layer and stack objects, and the standalone router / expert / dequant
// entry points.  Host code only: argument checks, workspace, launches.
//
// The layer follows the pages' statement of the model's MoE layer ([xix]
// how-it-works paragraph; [lens] "エキスパートストリーミングの仕組み"): the
// router, the shared experts and the dense core stay resident; routed experts
// are read from wherever they live -- all resident in HBM, or a bounded slot
// pool filled from a host store.
#include <algorithm>
#include <cstring>
#include <atomic>
#include <chrono>
#include <vector>

#include "common.h"
#include "kernels.h"

struct moe_layer {
  moe_layer_cfg cfg;
  const float* Wr;
  const float* rb;
  const float* wsg;
  const uint8_t* shared_blob;
  const uint8_t* resident_base;
  slotpool* pool;
  moe_blob_layout lay_r, lay_s;
  int device;
  // device workspace, one allocation
  void* ws;
  float* logits;
  int32_t* idx;
  float* w;
  float* sigma;
  unsigned* counter;
  int32_t* slots;       // [0] = n_slots, [1..] = slot_expert
  int8_t* jmap;
  uint16_t* x_cur;
  uint16_t* h;
  float* y;
  int hI;
  // pool path: pinned host copy of the distinct-expert list written by the
  // router kernel ([0] call epoch, [1] count, [2..] experts), the call
  // epoch, and the slot-pointer table
  int32_t* host_slots;
  int32_t list_epoch;
  const uint8_t** host_ptrs;   // pinned [kMaxSlots]
  const uint8_t** dev_ptrs;    // device [kMaxSlots]
  // many-token path: workspace allocated on first use, grown with T
  void* pf;
  int pf_T;
  uint16_t* wr3;               // router as three bf16 planes [3][E+1][H]
  bool wr3_ready;
  float* pf_logits;
  int32_t* pf_idx;
  float* pf_w;
  float* pf_sigma;
  int32_t* pf_hist;
  int32_t* pf_row_off;
  int32_t* pf_ntiles;
  int32_t* pf_tg;
  int32_t* pf_tm;
  int32_t* pf_perm;
  int32_t* pf_inv;
  uint16_t* pf_h;
  float* pf_yd;
  int pf_max_tiles;
  const uint8_t** pf_dev_tab;  // device [E]: blob per expert (pool mode)
  const uint8_t** pf_host_tab; // pinned [E]
  int32_t* pf_host_rowoff;     // pinned [E+2]
};

struct moe_stack {
  std::vector<moe_layer*> layers;
  // persistent one-token path (set up at create when the stack qualifies)
  bool persistent_enabled;
  bool persistent_ok;
  int grid;
  void* ps_mem;                 // device: layer table, hand-off buffers, epochs
  int32_t* err_host;            // pinned, written by the kernel on a timeout
  moe::StackArgs ps;            // constant part of the kernel arguments
  // pool mode of the persistent path (every layer on one pool)
  slotpool* pool = nullptr;
  int32_t* stop_host = nullptr;  // pinned: the layer the kernel stopped at
  int32_t* idx_host = nullptr;   // pinned [L][k]: every layer's choices
  uint16_t* xl_dev = nullptr;    // device [L][H]: layer inputs (export)
  float* yl_dev = nullptr;       // device [L][H]: layer outputs, to resume from
  std::vector<int32_t> layer_ids;
  // launches so far (the device's per-workgroup call counters hold the
  // same value), and per layer a lower bound on the launch that wrote any
  // word still in that layer's hand-off buffers
  uint32_t epoch = 0;
  std::vector<uint32_t> fresh;
  int64_t clk_khz = 0;
};

struct moe_timer {
  int32_t kernel;
  int32_t capacity;
  int32_t count;
  std::vector<hipEvent_t> start, stop;
};

static moe_timer* g_timer = nullptr;

namespace moe {
namespace {

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

int max_lds_per_block(int device) {
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, device) != hipSuccess)
    return 65536;
  return v;
}

size_t down_lds_bytes(int T, int k, int hI, int bits) {
  const int epc = 128 / bits;
  return (size_t)T * (k + 1) * hI * 2 + (size_t)T * (k + 1) * (hI / epc) * 4 +
         (size_t)T * (k + 1) * 8 * 4 + (size_t)T * k * kJmapStride;
}

int32_t check_layer_cfg(const moe_layer_cfg& c) {
  MOE_REQUIRE(c.group == 64, "group must be 64 (got %d)", c.group);
  MOE_REQUIRE(c.bits == 4 || c.bits == 8, "bits must be 4 or 8 (got %d)", c.bits);
  MOE_REQUIRE(c.hidden > 0 && c.hidden % 256 == 0 && c.hidden <= 2048,
              "hidden must be a multiple of 256 in [256, 2048] (got %d)", c.hidden);
  MOE_REQUIRE(c.experts >= 1 && c.experts <= 1024, "experts must be in [1, 1024] (got %d)",
              c.experts);
  MOE_REQUIRE(c.top_k >= 1 && c.top_k <= MOE_MAX_TOPK && c.top_k <= c.experts,
              "top_k must be in [1, min(E, %d)] (got %d)", MOE_MAX_TOPK, c.top_k);
  MOE_REQUIRE(decode_shape_supported(c.hidden, c.inter, c.shared_inter, c.bits),
              "unsupported expert shape H=%d I=%d Is=%d bits=%d", c.hidden, c.inter,
              c.shared_inter, c.bits);
  MOE_REQUIRE(c.layer_index >= 0, "layer_index must be >= 0");
  return MOE_OK;
}

void timer_mark(int kernel, bool begin, hipStream_t stream) {
  moe_timer* t = g_timer;
  if (!t || t->kernel != kernel || t->count >= t->capacity) return;
  if (begin) {
    (void)hipEventRecord(t->start[t->count], stream);
  } else {
    (void)hipEventRecord(t->stop[t->count], stream);
    t->count += 1;
  }
}

// One forward of a layer on T <= 8 tokens.  Input is either x (bf16) or
// y_prev (f32 output of the previous layer, rescaled in the router).
int32_t forward_decode(moe_layer* L, const uint16_t* x, const float* y_prev, uint16_t* x_export,
                       int T, uint16_t* y_bf16, float* y_f32, int32_t* idx_out, float* w_out,
                       hipStream_t stream) {
  const moe_layer_cfg& c = L->cfg;
  RouteArgs r{};
  r.x = y_prev ? nullptr : x;
  r.y_prev = y_prev;
  r.x_out = y_prev ? (x_export ? x_export : L->x_cur) : x_export;
  r.Wr = L->Wr;
  r.rb = L->rb;
  r.wsg = L->wsg;
  r.T = T;
  r.H = c.hidden;
  r.E = c.experts;
  r.k = c.top_k;
  r.logits = L->logits;
  r.counter = L->counter;
  r.idx = idx_out ? idx_out : L->idx;
  r.w = w_out ? w_out : L->w;
  r.sigma = L->sigma;
  r.n_slots = L->slots;
  r.slot_expert = L->slots + 1;
  r.jmap = L->jmap;
  int32_t* go = L->slots + 1 + MOE_MAX_DECODE_T * c.top_k;  // device flag
  if (L->pool) {
    r.host_list = L->host_slots;
    r.host_epoch = L->list_epoch = L->list_epoch == 0x7fffffff ? 1 : L->list_epoch + 1;
    // the router looks the chosen experts up in the pool's device table
    int32_t st = pool_before_lookup(L->pool, stream);
    if (st != MOE_OK) return st;
    r.res_tab = pool_device_table(L->pool, c.layer_index);
    r.slot_addr = L->dev_ptrs;
    r.go = go;
  }
  timer_mark(MOE_KERNEL_ROUTE, true, stream);
  MOE_HIP_TRY(launch_route(r, stream));
  timer_mark(MOE_KERNEL_ROUTE, false, stream);

  DecodeArgs d{};
  d.x = y_prev ? r.x_out : x;
  d.T = T;
  d.H = c.hidden;
  d.I = c.inter;
  d.Is = c.shared_inter;
  d.k = c.top_k;
  d.bits = c.bits;
  d.n_slot_max = T * c.top_k;
  d.stride = L->lay_r.stride;
  d.lr = to_qlayout(L->lay_r);
  d.ls = to_qlayout(L->lay_s);
  d.shared_blob = L->shared_blob;
  d.n_slots = L->slots;
  d.slot_expert = L->slots + 1;
  d.jmap = L->jmap;
  d.h = L->h;
  d.hI = L->hI;
  d.w = r.w;
  d.gate = L->sigma;
  d.y_f32 = y_f32;
  d.y_bf16 = y_bf16;
  d.accumulate = 0;

  if (!L->pool) {
    d.routed_base = L->resident_base + (int64_t)c.layer_index * c.experts * L->lay_r.stride;
    timer_mark(MOE_KERNEL_GATE_UP, true, stream);
    hipError_t e1 = launch_gate_up(d, stream);
    timer_mark(MOE_KERNEL_GATE_UP, false, stream);
    timer_mark(MOE_KERNEL_DOWN, true, stream);
    hipError_t e2 = e1 == hipSuccess ? launch_down(d, stream) : e1;
    timer_mark(MOE_KERNEL_DOWN, false, stream);
    MOE_HIP_TRY(e2);
    return MOE_OK;
  }

  // Pool: the expert kernels are enqueued right behind the router, reading
  // the slot addresses the router found in the pool's device table; they
  // run only if every chosen expert was resident (*go).  Meanwhile the host
  // waits for the router's expert list and runs the pool policy on it; if
  // an expert was missing, the kernels above did nothing, and after the
  // misses are filled they are enqueued again with the acquired addresses.
  d.routed_base = nullptr;
  {
    DecodeArgs ds = d;
    ds.slot_ptrs = L->dev_ptrs;
    ds.go = go;
    timer_mark(MOE_KERNEL_GATE_UP, true, stream);
    hipError_t e1 = launch_gate_up(ds, stream);
    timer_mark(MOE_KERNEL_GATE_UP, false, stream);
    timer_mark(MOE_KERNEL_DOWN, true, stream);
    hipError_t e2 = e1 == hipSuccess ? launch_down(ds, stream) : e1;
    timer_mark(MOE_KERNEL_DOWN, false, stream);
    MOE_HIP_TRY(e2);
  }
  // The chosen experts are needed on the host to run the pool policy: the
  // router kernel writes them to pinned memory and then the call's epoch;
  // the host waits for the epoch (no stream synchronisation: the router
  // has not finished when the list is complete).
  const int32_t want = L->list_epoch;
  const auto t_start = std::chrono::steady_clock::now();
  volatile int32_t* flag = L->host_slots;
  int spins = 0;
  while (*flag != want) {
    // the stream is queried only once the wait is long (a query costs
    // microseconds and would delay noticing the list)
    if (++spins % 1024 == 0 &&
        std::chrono::steady_clock::now() - t_start > std::chrono::microseconds(500)) {
      const hipError_t q = hipStreamQuery(stream);
      if (q != hipSuccess && q != hipErrorNotReady)
        return fail(MOE_E_HIP, "router failed: %s", hipGetErrorString(q));
      if (q == hipSuccess && *flag != want)
        return fail(MOE_E_HIP, "router finished without publishing its expert list");
      if (std::chrono::steady_clock::now() - t_start > std::chrono::seconds(10))
        return fail(MOE_E_HIP, "timed out waiting for the router's expert list");
    }
  }
  std::atomic_thread_fence(std::memory_order_acquire);
  const int n = L->host_slots[1];
  if (n < 0 || n > T * c.top_k) return fail(MOE_E_HIP, "router produced %d slots", n);
  const bool dev_all_resident = L->host_slots[2 + T * c.top_k] != 0;
  std::vector<int32_t> experts(L->host_slots + 2, L->host_slots + 2 + n);
  const void* ptrs[kMaxSlots];
  uint8_t was_miss[kMaxSlots];
  int32_t st = slotpool_acquire(L->pool, c.layer_index, experts.data(), n, stream, ptrs, was_miss);
  if (st != MOE_OK) return st;
  bool any_miss = false;
  for (int i = 0; i < n; ++i) any_miss = any_miss || was_miss[i];
  if (dev_all_resident && any_miss) {
    // cannot happen: the table changes only inside calls on the pool, in
    // stream order with the kernels that read it
    (void)slotpool_release(L->pool, c.layer_index, experts.data(), n, stream);
    return fail(MOE_E_HIP, "pool table found an expert resident that the pool had not");
  }
  hipError_t e2 = hipSuccess;
  if (!dev_all_resident) {
    SlotArgs sa{};
    if (n <= kSlotArgs) {
      // few slots: their addresses go in the kernel arguments (no upload)
      for (int i = 0; i < n; ++i) sa.p[i] = static_cast<const uint8_t*>(ptrs[i]);
      d.slot_ptrs = nullptr;
    } else {
      for (int i = 0; i < n; ++i) L->host_ptrs[i] = static_cast<const uint8_t*>(ptrs[i]);
      // host_ptrs is rewritten only after the next call's router has run,
      // i.e. after this upload
      e2 = hipMemcpyAsync(L->dev_ptrs, L->host_ptrs, sizeof(void*) * n, hipMemcpyHostToDevice,
                          stream);
      d.slot_ptrs = L->dev_ptrs;
    }
    if (e2 == hipSuccess) e2 = launch_gate_up(d, stream, sa);
    if (e2 == hipSuccess) e2 = launch_down(d, stream, sa);
  }
  st = slotpool_release(L->pool, c.layer_index, experts.data(), n, stream);
  if (st != MOE_OK) return st;
  MOE_HIP_TRY(e2);
  return MOE_OK;
}

// Sets up the persistent one-token path if every layer is resident, all
// layers share one shape and the device has at least as many compute units
// as the kernel has workgroups (so all of them can be resident at once).  A
// stack that does not qualify keeps persistent_ok = false (not an error).
int32_t setup_persistent(moe_stack* st) {
  st->persistent_ok = false;
  const moe_layer* L0 = st->layers[0];
  const moe_layer_cfg& c = L0->cfg;
  const int n = (int)st->layers.size();
  // every layer resident, or every layer on the same pool
  slotpool* pool = L0->pool;
  for (const moe_layer* L : st->layers) {
    const moe_layer_cfg& d = L->cfg;
    if (L->pool != pool || (!pool && !L->resident_base) || L->device != L0->device) return MOE_OK;
    if (d.hidden != c.hidden || d.experts != c.experts || d.top_k != c.top_k ||
        d.inter != c.inter || d.shared_inter != c.shared_inter || d.bits != c.bits)
      return MOE_OK;
    if ((L->wsg != nullptr) != (L0->wsg != nullptr) || !L->shared_blob) return MOE_OK;
  }
  int cus = 0, clk_khz = 0;
  MOE_HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, L0->device));
  MOE_HIP_TRY(hipDeviceGetAttribute(&clk_khz, hipDeviceAttributeWallClockRate, L0->device));
  if (cus < 1 || clk_khz < 1 || n > kStackMaxLayers) return MOE_OK;
  const int H = c.hidden, E = c.experts, k = c.top_k;
  if (!stack_decode_supported(H, E, k, c.inter, c.shared_inter, c.bits, cus)) return MOE_OK;
  const int grid = kStackGrid;
  const int hwords = k * c.inter + c.shared_inter;
  const size_t sizes[] = {
      (size_t)n * sizeof(StackLayerDesc),
      (size_t)n * kStackReplicas * H * 8,         // ybuf
      (size_t)n * kStackReplicas * (E + 1) * 8,   // lbuf
      (size_t)n * kStackReplicas * hwords * 4,    // hbuf
      (size_t)grid * 4,              // epochs
  };
  size_t total = 0;
  for (size_t sz : sizes) total += align256(sz);
  hipError_t e = hipMalloc(&st->ps_mem, total);
  if (e != hipSuccess) return fail(MOE_E_NOMEM, "stack hand-off buffers hipMalloc(%zu): %s", total,
                                   hipGetErrorString(e));
  uint8_t* p = static_cast<uint8_t*>(st->ps_mem);
  void* parts[5];
  for (int i = 0; i < 5; ++i) {
    parts[i] = p;
    p += align256(sizes[i]);
  }
  std::vector<StackLayerDesc> descs(n);
  for (int l = 0; l < n; ++l) {
    const moe_layer* L = st->layers[l];
    descs[l].Wr = L->Wr;
    descs[l].rb = L->rb;
    descs[l].wsg = L->wsg;
    descs[l].shared_blob = L->shared_blob;
    descs[l].routed_base =
        pool ? nullptr : L->resident_base + (int64_t)L->cfg.layer_index * E * L->lay_r.stride;
    descs[l].res_row = pool ? pool_device_table(pool, L->cfg.layer_index) : nullptr;
  }
  // zeroed hand-off words carry tag 0, which no call uses
  e = hipMemset(st->ps_mem, 0, total);
  if (e == hipSuccess)
    e = hipMemcpy(parts[0], descs.data(), sizes[0], hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipHostMalloc(reinterpret_cast<void**>(&st->err_host), sizeof(int32_t),
                      hipHostMallocDefault);
  if (e == hipSuccess && pool) {
    e = hipHostMalloc(reinterpret_cast<void**>(&st->stop_host), sizeof(int32_t),
                      hipHostMallocDefault);
    if (e == hipSuccess)
      e = hipHostMalloc(reinterpret_cast<void**>(&st->idx_host), (size_t)n * k * sizeof(int32_t),
                        hipHostMallocDefault);
    if (e == hipSuccess)
      e = hipMalloc(reinterpret_cast<void**>(&st->xl_dev), (size_t)n * H * sizeof(uint16_t));
    if (e == hipSuccess)
      e = hipMalloc(reinterpret_cast<void**>(&st->yl_dev), (size_t)n * H * sizeof(float));
    for (const moe_layer* L : st->layers) st->layer_ids.push_back(L->cfg.layer_index);
  }
  if (e != hipSuccess) {
    (void)hipFree(st->ps_mem);
    st->ps_mem = nullptr;
    if (st->stop_host) (void)hipHostFree(st->stop_host);
    if (st->idx_host) (void)hipHostFree(st->idx_host);
    if (st->xl_dev) (void)hipFree(st->xl_dev);
    if (st->yl_dev) (void)hipFree(st->yl_dev);
    st->stop_host = st->idx_host = nullptr;
    st->xl_dev = nullptr;
    st->yl_dev = nullptr;
    return fail(MOE_E_HIP, "stack setup: %s", hipGetErrorString(e));
  }
  *st->err_host = 0;
  StackArgs& a = st->ps;
  a = StackArgs{};
  a.layers = static_cast<const StackLayerDesc*>(parts[0]);
  a.L = n;
  a.E = E;
  a.has_wsg = L0->wsg != nullptr;
  a.stride = L0->lay_r.stride;
  for (int i = 0; i < 3; ++i) {
    a.lq[i] = (uint32_t)L0->lay_r.q_off[i];
    a.lsb[i] = (uint32_t)L0->lay_r.sb_off[i];
    a.sq[i] = (uint32_t)L0->lay_s.q_off[i];
    a.ssb[i] = (uint32_t)L0->lay_s.sb_off[i];
  }
  a.ybuf = static_cast<uint64_t*>(parts[1]);
  a.lbuf = static_cast<uint64_t*>(parts[2]);
  a.hbuf = static_cast<uint32_t*>(parts[3]);
  a.epochs = static_cast<uint32_t*>(parts[4]);
  a.err = st->err_host;
  a.timeout_ticks = (int64_t)clk_khz * 1000 * 2;  // 2 s
  st->pool = pool;
  if (pool) {
    a.pool = 1;
    a.stop = st->stop_host;
  }
  st->clk_khz = clk_khz;
  st->epoch = 0;
  st->fresh.assign(n, 0u);
  st->grid = grid;
  st->persistent_ok = true;
  return MOE_OK;
}

// A hand-off word carries the tag of the launch that wrote it: 32 bits for
// y and the logits, 15 bits for h (a bf16 shares its 32-bit word), so an h
// word left behind kTagSpan launches earlier carries the tag of the next
// launch.  A layer's words are rewritten by every launch that runs the
// layer to its end; a pooled launch that stops at a layer, or starts after
// it, leaves the layer's words as they were.  Before a launch, every layer
// it may run whose oldest word could be that old is zeroed (tag 0 matches
// no launch).
constexpr uint32_t kTagSpan = 32768;

int32_t stack_clear_stale(moe_stack* st, int l0, hipStream_t stream) {
  const moe_layer_cfg& c = st->layers[0]->cfg;
  const int n = (int)st->layers.size();
  const size_t yb = (size_t)kStackReplicas * c.hidden * 8;
  const size_t lb = (size_t)kStackReplicas * (c.experts + 1) * 8;
  const size_t hb = (size_t)kStackReplicas * (c.top_k * c.inter + c.shared_inter) * 4;
  for (int l = l0; l < n; ++l) {
    if (st->epoch - st->fresh[l] < kTagSpan) continue;
    MOE_HIP_TRY(launch_fill_zero(st->ps.ybuf + (size_t)l * yb / 8, yb, stream));
    MOE_HIP_TRY(launch_fill_zero(st->ps.lbuf + (size_t)l * lb / 8, lb, stream));
    MOE_HIP_TRY(launch_fill_zero(st->ps.hbuf + (size_t)l * hb / 4, hb, stream));
    st->fresh[l] = st->epoch;
  }
  return MOE_OK;
}

// After a launch (epoch st->epoch) that ran layers [l0, l1) to their end.
void stack_launched(moe_stack* st, int l0, int l1) {
  for (int l = l0; l < l1; ++l) st->fresh[l] = st->epoch;
  st->epoch += 1;
}

// A launch failed part-way: any layer may hold words of any earlier launch.
void stack_forget(moe_stack* st) {
  for (uint32_t& f : st->fresh) f = st->epoch - kTagSpan;
}

int max_tiles_for(int T, int k, int E) {
  return (T * k + kPrefillBM - 1) / kPrefillBM + E + (T + kPrefillBM - 1) / kPrefillBM + 1;
}

int32_t ensure_prefill_ws(moe_layer* L, int T) {
  if (L->pf && L->pf_T >= T) return MOE_OK;
  const moe_layer_cfg& c = L->cfg;
  const int E = c.experts, k = c.top_k, H = c.hidden;
  const int64_t P = (int64_t)T * k, R = P + T;
  const int mt = max_tiles_for(T, k, E);
  const size_t sizes[] = {
      (size_t)3 * E * H * 2,        // wr3
      (size_t)kRouterMaxSplits * T * E * 4,  // router partial sums (any T' <= T)
      (size_t)T * k * 4,            // idx
      (size_t)T * k * 4,            // w
      (size_t)T * 4,                // sigma
      (size_t)kSortChunks * E * 4,  // hist
      (size_t)(E + 2) * 4,          // row_off
      4,                            // n_tiles
      (size_t)mt * 4,               // tile_group
      (size_t)mt * 4,               // tile_m0
      (size_t)R * 4,                // perm
      (size_t)P * 4,                // inv
      (size_t)R * L->hI * 2,        // h
      (size_t)R * H * 4,            // yd
      (size_t)E * sizeof(void*),    // dev_tab
  };
  size_t total = 0;
  for (size_t sz : sizes) total += align256(sz);
  if (L->pf) {
    MOE_HIP_TRY(hipDeviceSynchronize());
    (void)hipFree(L->pf);
    L->pf = nullptr;
  }
  hipError_t e = hipMalloc(&L->pf, total);
  if (e != hipSuccess) return fail(MOE_E_NOMEM, "prefill workspace hipMalloc(%zu): %s", total,
                                   hipGetErrorString(e));
  MOE_HIP_TRY(hipMemset(L->pf, 0, total));
  uint8_t* p = static_cast<uint8_t*>(L->pf);
  void* parts[15];
  for (int i = 0; i < 15; ++i) {
    parts[i] = p;
    p += align256(sizes[i]);
  }
  L->wr3 = static_cast<uint16_t*>(parts[0]);
  L->pf_logits = static_cast<float*>(parts[1]);
  L->pf_idx = static_cast<int32_t*>(parts[2]);
  L->pf_w = static_cast<float*>(parts[3]);
  L->pf_sigma = static_cast<float*>(parts[4]);
  L->pf_hist = static_cast<int32_t*>(parts[5]);
  L->pf_row_off = static_cast<int32_t*>(parts[6]);
  L->pf_ntiles = static_cast<int32_t*>(parts[7]);
  L->pf_tg = static_cast<int32_t*>(parts[8]);
  L->pf_tm = static_cast<int32_t*>(parts[9]);
  L->pf_perm = static_cast<int32_t*>(parts[10]);
  L->pf_inv = static_cast<int32_t*>(parts[11]);
  L->pf_h = static_cast<uint16_t*>(parts[12]);
  L->pf_yd = static_cast<float*>(parts[13]);
  L->pf_dev_tab = static_cast<const uint8_t**>(parts[14]);
  L->pf_max_tiles = mt;
  L->pf_T = T;
  L->wr3_ready = false;
  if (L->pool && !L->pf_host_tab) {
    MOE_HIP_TRY(hipHostMalloc(reinterpret_cast<void**>(&L->pf_host_tab), E * sizeof(void*),
                              hipHostMallocDefault));
    MOE_HIP_TRY(hipHostMalloc(reinterpret_cast<void**>(&L->pf_host_rowoff), (E + 2) * 4,
                              hipHostMallocDefault));
  }
  return MOE_OK;
}

// Many tokens: MFMA router, sort by expert, grouped GEMMs, combine.
int32_t forward_prefill(moe_layer* L, const uint16_t* x, int T, uint16_t* y_bf16, float* y_f32,
                        int32_t* idx_out, float* w_out, hipStream_t stream) {
  int32_t st = ensure_prefill_ws(L, T);
  if (st != MOE_OK) return st;
  const moe_layer_cfg& c = L->cfg;
  const int E = c.experts, k = c.top_k, H = c.hidden;
  if (!L->wr3_ready) {
    MOE_HIP_TRY(launch_split_router(L->Wr, E, H, L->wr3, stream));
    L->wr3_ready = true;
  }
  timer_mark(MOE_KERNEL_ROUTE, true, stream);
  MOE_HIP_TRY(launch_router_gemm(x, T, H, L->wr3, E, L->pf_logits, stream));
  timer_mark(MOE_KERNEL_ROUTE, false, stream);
  RouteArgs r{};
  r.x = x;
  r.T = T;
  r.H = H;
  r.E = E;
  r.k = k;
  r.rb = L->rb;
  r.wsg = L->wsg;
  r.part = L->pf_logits;
  r.ksplit = router_splits(T, E, H);
  r.idx = idx_out ? idx_out : L->pf_idx;
  r.w = w_out ? w_out : L->pf_w;
  r.sigma = L->pf_sigma;
  MOE_HIP_TRY(launch_topk_only(r, stream));

  PrefillArgs p{};
  p.T = T;
  p.H = H;
  p.I = c.inter;
  p.Is = c.shared_inter;
  p.E = E;
  p.k = k;
  p.bits = c.bits;
  p.hI = L->hI;
  p.x = x;
  p.idx = r.idx;
  p.w = r.w;
  p.sigma = L->pf_sigma;
  p.hist = L->pf_hist;
  p.row_off = L->pf_row_off;
  p.n_tiles = L->pf_ntiles;
  p.tile_group = L->pf_tg;
  p.tile_m0 = L->pf_tm;
  p.max_tiles = L->pf_max_tiles;
  p.perm_tok = L->pf_perm;
  p.inv = L->pf_inv;
  p.stride = L->lay_r.stride;
  p.lr = to_qlayout(L->lay_r);
  p.ls = to_qlayout(L->lay_s);
  p.shared_blob = L->shared_blob;
  p.h = L->pf_h;
  p.yd = L->pf_yd;
  p.y_f32 = y_f32;
  p.y_bf16 = y_bf16;
  MOE_HIP_TRY(launch_prefill_sort(p, stream));

  std::vector<int32_t> used;
  if (L->pool) {
    MOE_HIP_TRY(hipMemcpyAsync(L->pf_host_rowoff, L->pf_row_off, (E + 2) * 4,
                               hipMemcpyDeviceToHost, stream));
    MOE_HIP_TRY(hipStreamSynchronize(stream));
    for (int e = 0; e < E; ++e)
      if (L->pf_host_rowoff[e + 1] > L->pf_host_rowoff[e]) used.push_back(e);
    std::vector<const void*> ptrs(used.size());
    st = slotpool_acquire(L->pool, c.layer_index, used.data(), (int)used.size(), stream,
                          ptrs.data(), nullptr);
    if (st != MOE_OK) return st;
    for (int e = 0; e < E; ++e) L->pf_host_tab[e] = nullptr;
    for (size_t i = 0; i < used.size(); ++i)
      L->pf_host_tab[used[i]] = static_cast<const uint8_t*>(ptrs[i]);
    MOE_HIP_TRY(hipMemcpyAsync(L->pf_dev_tab, L->pf_host_tab, E * sizeof(void*),
                               hipMemcpyHostToDevice, stream));
    p.routed_base = nullptr;
    p.slot_ptrs = L->pf_dev_tab;
  } else {
    p.routed_base = L->resident_base + (int64_t)c.layer_index * E * L->lay_r.stride;
  }
  timer_mark(MOE_KERNEL_GATE_UP, true, stream);
  hipError_t e = launch_prefill_gu(p, stream);
  timer_mark(MOE_KERNEL_GATE_UP, false, stream);
  timer_mark(MOE_KERNEL_DOWN, true, stream);
  if (e == hipSuccess) e = launch_prefill_down(p, stream);
  timer_mark(MOE_KERNEL_DOWN, false, stream);
  if (e == hipSuccess) e = launch_prefill_combine(p, stream);
  if (L->pool) {
    st = slotpool_release(L->pool, c.layer_index, used.data(), (int)used.size(), stream);
    if (st != MOE_OK) return st;
  }
  MOE_HIP_TRY(e);
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int32_t moe_route_topk(const uint16_t* x, int32_t T, int32_t H, const float* Wr, const float* rb,
                       int32_t E, int32_t k, const float* wsg, int32_t* idx, float* w,
                       float* sigma, float* logits, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(T >= 0, "T must be >= 0");
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(x && Wr && idx && w, "null argument");
  MOE_REQUIRE(H > 0 && H % 256 == 0 && H <= 4096, "H must be a multiple of 256 in [256, 4096]");
  MOE_REQUIRE(E >= 1 && E <= 1024, "E must be in [1, 1024]");
  MOE_REQUIRE(k >= 1 && k <= E && k <= MOE_MAX_TOPK, "k must be in [1, min(E, %d)]",
              MOE_MAX_TOPK);
  RouteArgs r{};
  r.x = x;
  r.Wr = Wr;
  r.rb = rb;
  r.wsg = sigma ? wsg : nullptr;
  r.T = T;
  r.H = H;
  r.E = E;
  r.k = k;
  r.logits = logits;
  r.idx = idx;
  r.w = w;
  r.sigma = sigma;
  if (T <= MOE_MAX_DECODE_T) {
    // the GEMV writes the logits and the top-k reads them: without a caller
    // buffer they go to stream-ordered scratch
    float* scratch = nullptr;
    if (!logits) {
      MOE_HIP_TRY(hipMallocAsync(reinterpret_cast<void**>(&scratch), (size_t)T * E * 4, stream));
      r.logits = scratch;
    }
    hipError_t e = launch_route(r, stream);
    if (e == hipSuccess) e = launch_topk_only(r, stream);
    const hipError_t e2 = scratch ? hipFreeAsync(scratch, stream) : hipSuccess;
    MOE_HIP_TRY(e);
    MOE_HIP_TRY(e2);
    return MOE_OK;
  }
  {
    // many tokens: router on bf16 MFMA with Wr split into three exact planes;
    // the top-k sums the K slices' partials and computes the shared gate
    const int ks = router_splits(T, E, H);
    uint16_t* wr3 = nullptr;
    float* part = nullptr;
    MOE_HIP_TRY(hipMallocAsync(reinterpret_cast<void**>(&wr3), (size_t)3 * E * H * 2, stream));
    hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&part), (size_t)ks * T * E * 4, stream);
    if (e == hipSuccess) e = launch_split_router(Wr, E, H, wr3, stream);
    if (e == hipSuccess) e = launch_router_gemm(x, T, H, wr3, E, part, stream);
    r.part = part;
    r.ksplit = ks;
    if (e == hipSuccess) e = launch_topk_only(r, stream);
    hipError_t e2 = hipFreeAsync(wr3, stream);
    hipError_t e3 = part ? hipFreeAsync(part, stream) : hipSuccess;
    MOE_HIP_TRY(e);
    MOE_HIP_TRY(e2);
    MOE_HIP_TRY(e3);
    return MOE_OK;
  }
}

int32_t moe_expert_sort(const int32_t* idx, int32_t T, int32_t k, int32_t E, int32_t* perm,
                        int32_t* offsets, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(T >= 0, "T must be >= 0");
  MOE_REQUIRE(k >= 1 && k <= MOE_MAX_TOPK, "k must be in [1, %d]", MOE_MAX_TOPK);
  MOE_REQUIRE(E >= 1 && E <= 1024, "E must be in [1, 1024]");
  MOE_REQUIRE((int64_t)T * (k + 1) < (1ll << 30), "T * (k + 1) must be below 2^30");
  MOE_REQUIRE(offsets, "null argument");
  if (T == 0) {
    MOE_HIP_TRY(launch_fill_zero(offsets, (size_t)(E + 1) * 4, stream));
    return MOE_OK;
  }
  MOE_REQUIRE(idx && perm, "null argument");
  const int64_t P = (int64_t)T * k;
  const int mt = max_tiles_for(T, k, E);
  const size_t sizes[] = {
      (size_t)kSortChunks * E * 4,  // per-chunk histograms
      (size_t)(E + 2) * 4,          // row offsets (group E: the shared rows)
      4,                            // tile count
      (size_t)mt * 4,               // tile groups
      (size_t)mt * 4,               // tile first rows
      (size_t)(P + T) * 4,          // sorted row -> token
      (size_t)P * 4,                // pair -> sorted row
  };
  size_t total = 0;
  for (size_t sz : sizes) total += align256(sz);
  void* ws = nullptr;
  MOE_HIP_TRY(hipMallocAsync(&ws, total, stream));
  uint8_t* q = static_cast<uint8_t*>(ws);
  void* parts[7];
  for (int i = 0; i < 7; ++i) {
    parts[i] = q;
    q += align256(sizes[i]);
  }
  PrefillArgs a{};
  a.T = T;
  a.k = k;
  a.E = E;
  a.idx = idx;
  a.hist = static_cast<int32_t*>(parts[0]);
  a.row_off = static_cast<int32_t*>(parts[1]);
  a.n_tiles = static_cast<int32_t*>(parts[2]);
  a.tile_group = static_cast<int32_t*>(parts[3]);
  a.tile_m0 = static_cast<int32_t*>(parts[4]);
  a.max_tiles = mt;
  a.perm_tok = static_cast<int32_t*>(parts[5]);
  a.inv = static_cast<int32_t*>(parts[6]);
  hipError_t e = launch_prefill_sort(a, stream);
  if (e == hipSuccess) e = launch_prefill_perm(a, perm, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(offsets, a.row_off, (size_t)(E + 1) * 4, hipMemcpyDeviceToDevice, stream);
  const hipError_t e2 = hipFreeAsync(ws, stream);
  MOE_HIP_TRY(e);
  MOE_HIP_TRY(e2);
  return MOE_OK;
}

int32_t moe_dequant(const void* blob, const moe_qshape* shape, int32_t which, float* out_f32,
                    uint16_t* out_bf16, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(blob && shape && out_f32, "null argument");
  MOE_REQUIRE(which >= 0 && which <= 2, "which must be 0, 1 or 2");
  moe_blob_layout lay;
  if (!blob_layout(*shape, &lay)) return MOE_E_INVAL;
  const int rows = which == 2 ? shape->hidden : shape->inter;
  const int cols = which == 2 ? shape->inter : shape->hidden;
  MOE_HIP_TRY(launch_dequant(static_cast<const uint8_t*>(blob), to_qlayout(lay), rows, cols,
                             shape->bits, which, out_f32, out_bf16, stream));
  return MOE_OK;
}

int32_t moe_expert_forward(const uint16_t* x, int32_t T, const moe_qshape* shape, const void* blob,
                           const float* coef, float* y_accum, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(x && shape && blob && coef && y_accum, "null argument");
  MOE_REQUIRE(T >= 1 && T <= MOE_MAX_DECODE_T, "T must be in [1, %d]", MOE_MAX_DECODE_T);
  moe_blob_layout lay;
  if (!blob_layout(*shape, &lay)) return MOE_E_INVAL;
  MOE_REQUIRE(shape->hidden % 256 == 0 && shape->hidden <= 2048 &&
                  decode_shape_supported(shape->hidden, shape->inter, shape->inter, shape->bits),
              "unsupported expert shape H=%d I=%d bits=%d", shape->hidden, shape->inter,
              shape->bits);
  int dev = 0;
  MOE_HIP_TRY(hipGetDevice(&dev));
  MOE_REQUIRE(down_lds_bytes(T, 0, shape->inter, shape->bits) <= (size_t)max_lds_per_block(dev),
              "intermediate size too large for LDS");
  uint16_t* h = nullptr;
  const size_t hbytes = align256((size_t)T * shape->inter * 2);
  MOE_HIP_TRY(hipMallocAsync(reinterpret_cast<void**>(&h), hbytes, stream));
  DecodeArgs d{};
  d.x = x;
  d.T = T;
  d.H = shape->hidden;
  d.I = shape->inter;
  d.Is = shape->inter;
  d.k = 0;
  d.bits = shape->bits;
  d.n_slot_max = 0;
  d.ls = to_qlayout(lay);
  d.lr = d.ls;
  d.shared_blob = static_cast<const uint8_t*>(blob);
  d.h = h;
  d.hI = shape->inter;
  d.gate = coef;
  d.y_f32 = y_accum;
  d.accumulate = 1;
  hipError_t e1 = launch_gate_up(d, stream);
  hipError_t e2 = e1 == hipSuccess ? launch_down(d, stream) : e1;
  hipError_t e3 = hipFreeAsync(h, stream);
  MOE_HIP_TRY(e2);
  MOE_HIP_TRY(e3);
  return MOE_OK;
}

int32_t moe_layer_create(const moe_layer_cfg* cfg, const float* Wr, const float* rb,
                         const void* shared_blob, const float* wsg, const void* resident_base,
                         slotpool* pool, moe_layer** out) {
  clear_error();
  MOE_REQUIRE(cfg && Wr && shared_blob && wsg && out, "null argument");
  MOE_REQUIRE((resident_base != nullptr) != (pool != nullptr),
              "exactly one of resident_base and pool must be given");
  int32_t st = check_layer_cfg(*cfg);
  if (st != MOE_OK) return st;
  moe_qshape sr{cfg->hidden, cfg->inter, cfg->group, cfg->bits};
  moe_qshape ss{cfg->hidden, cfg->shared_inter, cfg->group, cfg->bits};
  if (pool) {
    // the layer reads blob (layer_index, e) of the pool's store, in its own
    // blob layout: the store must hold that layer and this many experts at
    // this layout's stride
    moe_blob_layout lr;
    blob_layout(sr, &lr);
    st = pool_check_layer(pool, cfg->layer_index, cfg->experts, lr.stride);
    if (st != MOE_OK) return st;
  }
  moe_layer* L = new (std::nothrow) moe_layer{};
  if (!L) return fail(MOE_E_NOMEM, "host allocation failed");
  L->cfg = *cfg;
  blob_layout(sr, &L->lay_r);
  blob_layout(ss, &L->lay_s);
  L->Wr = Wr;
  L->rb = rb;
  L->wsg = wsg;
  L->shared_blob = static_cast<const uint8_t*>(shared_blob);
  L->resident_base = static_cast<const uint8_t*>(resident_base);
  L->pool = pool;
  L->hI = std::max(cfg->inter, cfg->shared_inter);
  hipError_t he = hipGetDevice(&L->device);
  if (he != hipSuccess) {
    delete L;
    return fail(MOE_E_HIP, "hipGetDevice: %s", hipGetErrorString(he));
  }
  if (down_lds_bytes(MOE_MAX_DECODE_T, cfg->top_k, L->hI, cfg->bits) >
      (size_t)max_lds_per_block(L->device)) {
    delete L;
    return fail(MOE_E_INVAL, "top_k x intermediate too large for the down kernel's LDS");
  }
  const int T = MOE_MAX_DECODE_T, E = cfg->experts, k = cfg->top_k, H = cfg->hidden;
  const size_t sizes[] = {
      (size_t)T * E * 4,                 // logits
      (size_t)T * k * 4,                 // idx
      (size_t)T * k * 4,                 // w
      (size_t)T * 4,                     // sigma
      4,                                 // counter
      (size_t)(2 + T * k) * 4,           // slots: count, experts, go flag
      (size_t)T * k * kJmapStride,       // jmap
      (size_t)T * H * 2,                 // x_cur
      (size_t)T * (k + 1) * L->hI * 2,   // h
      (size_t)T * H * 4,                 // y
      (size_t)kMaxSlots * sizeof(void*), // dev_ptrs
  };
  size_t total = 0;
  for (size_t s : sizes) total += align256(s);
  he = hipMalloc(&L->ws, total);
  if (he != hipSuccess) {
    delete L;
    return fail(MOE_E_NOMEM, "workspace hipMalloc(%zu): %s", total, hipGetErrorString(he));
  }
  uint8_t* p = static_cast<uint8_t*>(L->ws);
  void* parts[11];
  for (int i = 0; i < 11; ++i) {
    parts[i] = p;
    p += align256(sizes[i]);
  }
  L->logits = static_cast<float*>(parts[0]);
  L->idx = static_cast<int32_t*>(parts[1]);
  L->w = static_cast<float*>(parts[2]);
  L->sigma = static_cast<float*>(parts[3]);
  L->counter = static_cast<unsigned*>(parts[4]);
  L->slots = static_cast<int32_t*>(parts[5]);
  L->jmap = static_cast<int8_t*>(parts[6]);
  L->x_cur = static_cast<uint16_t*>(parts[7]);
  L->h = static_cast<uint16_t*>(parts[8]);
  L->y = static_cast<float*>(parts[9]);
  L->dev_ptrs = static_cast<const uint8_t**>(parts[10]);
  he = hipMemset(L->ws, 0, total);
  if (he == hipSuccess && pool) {
    he = hipHostMalloc(reinterpret_cast<void**>(&L->host_slots), (3 + T * k) * sizeof(int32_t),
                       hipHostMallocDefault);
    if (he == hipSuccess) std::memset(L->host_slots, 0, (3 + T * k) * sizeof(int32_t));
    L->list_epoch = 0;  // the first call publishes epoch 1
  }
  if (he == hipSuccess && pool)
    he = hipHostMalloc(reinterpret_cast<void**>(&L->host_ptrs), kMaxSlots * sizeof(void*),
                       hipHostMallocDefault);
  if (he == hipSuccess) he = hipDeviceSynchronize();
  if (he != hipSuccess) {
    (void)hipFree(L->ws);
    delete L;
    return fail(MOE_E_HIP, "layer setup: %s", hipGetErrorString(he));
  }
  *out = L;
  return MOE_OK;
}

int32_t moe_layer_forward(moe_layer* layer, const uint16_t* x, int32_t T, uint16_t* y_bf16,
                          float* y_f32, int32_t* idx_out, float* w_out, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(layer, "null argument");
  MOE_REQUIRE(T >= 0, "T must be >= 0");
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(x && y_bf16, "null argument");
  if (T > MOE_MAX_DECODE_T)
    return forward_prefill(layer, x, T, y_bf16, y_f32, idx_out, w_out, stream);
  return forward_decode(layer, x, nullptr, nullptr, T, y_bf16, y_f32 ? y_f32 : layer->y, idx_out,
                        w_out, stream);
}

int32_t moe_layer_destroy(moe_layer* layer) {
  clear_error();
  if (!layer) return MOE_OK;
  hipError_t e = hipDeviceSynchronize();
  if (layer->ws) (void)hipFree(layer->ws);
  if (layer->host_slots) (void)hipHostFree(layer->host_slots);
  if (layer->host_ptrs) (void)hipHostFree(layer->host_ptrs);
  if (layer->pf) (void)hipFree(layer->pf);
  if (layer->pf_host_tab) (void)hipHostFree(layer->pf_host_tab);
  if (layer->pf_host_rowoff) (void)hipHostFree(layer->pf_host_rowoff);
  delete layer;
  if (e != hipSuccess) return fail(MOE_E_HIP, "hipDeviceSynchronize: %s", hipGetErrorString(e));
  return MOE_OK;
}

int32_t moe_stack_create(moe_layer* const* layers, int32_t n_layers, moe_stack** out) {
  clear_error();
  MOE_REQUIRE(layers && out && n_layers >= 1, "bad argument");
  for (int i = 0; i < n_layers; ++i) {
    MOE_REQUIRE(layers[i], "layer %d is NULL", i);
    MOE_REQUIRE(layers[i]->cfg.hidden == layers[0]->cfg.hidden &&
                    layers[i]->cfg.top_k == layers[0]->cfg.top_k,
                "all layers of a stack must share hidden size and top_k");
  }
  moe_stack* s = new (std::nothrow) moe_stack{};
  if (!s) return fail(MOE_E_NOMEM, "host allocation failed");
  s->layers.assign(layers, layers + n_layers);
  s->persistent_enabled = true;
  int32_t st = setup_persistent(s);
  if (st != MOE_OK) {
    delete s;
    return st;
  }
  *out = s;
  return MOE_OK;
}

int32_t moe_stack_forward(moe_stack* stack, const uint16_t* x0, int32_t T, uint16_t* x_layers,
                          float* y_layers, int32_t* idx, float* w, uint16_t* y_last,
                          hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(stack && x0 && y_last, "null argument");
  MOE_REQUIRE(T >= 1 && T <= MOE_MAX_DECODE_T, "T must be in [1, %d]", MOE_MAX_DECODE_T);
  if (stack->err_host && *stack->err_host) {
    *stack->err_host = 0;
    stack_forget(stack);
    return fail(MOE_E_HIP, "an earlier persistent decode call on this stack timed out");
  }
  if (T == 1 && stack->persistent_ok && stack->persistent_enabled) {
    StackArgs a = stack->ps;
    a.x0 = x0;
    a.x_layers = x_layers;
    a.y_layers = y_layers;
    a.idx = idx;
    a.w = w;
    a.y_last = y_last;
    const moe_layer_cfg& c = stack->layers[0]->cfg;
    const int nl = (int)stack->layers.size(), H = c.hidden, k = c.top_k;
    if (stack->pool) {
      // the kernel reads the pool's table; it exports every layer's output
      // (to resume from) and choices (for the pool policy)
      a.x_layers = x_layers ? x_layers : stack->xl_dev;
      a.y_layers = y_layers ? y_layers : stack->yl_dev;
      a.idx = stack->idx_host;
      *stack->stop_host = nl;
      const int32_t st = pool_before_lookup(stack->pool, stream);
      if (st != MOE_OK) return st;
    }
    int32_t cst = stack_clear_stale(stack, 0, stream);
    if (cst != MOE_OK) return cst;
    timer_mark(MOE_KERNEL_STACK, true, stream);
    hipError_t e = launch_stack_decode(a, H, k, c.inter, c.shared_inter, c.bits, stream);
    timer_mark(MOE_KERNEL_STACK, false, stream);
    MOE_HIP_TRY(e);
    if (!stack->pool) {
      stack_launched(stack, 0, nl);
      return MOE_OK;
    }
    // the previous call's hits enter the policy while this kernel runs
    int32_t pst = pool_apply_pending(stack->pool);
    if (pst != MOE_OK) return pst;

    // Pool mode: the host needs the layer the kernel stopped at (the first
    // with a non-resident choice, or nl) before it can go on.  The policy
    // then sees the layers the kernel ran as the per-layer path would have
    // (each a call whose experts all hit, in order; held in the pool and
    // applied before its next use).  The stopped layer's choices, which the
    // kernel exported before it stopped, are acquired (its misses filled),
    // and the kernel is launched again at that layer, from the previous
    // layer's output; the layer is released right behind that launch, as
    // the per-layer path releases it behind its kernels.
    int l0 = 0;       // first layer of the launch in flight
    int replay0 = 0;  // first layer of it whose accesses the pool has not seen
    for (;;) {
      const hipError_t se = hipStreamSynchronize(stream);
      if (se != hipSuccess) {
        stack_forget(stack);
        stack->epoch += 1;
        return fail(MOE_E_HIP, "persistent decode: %s", hipGetErrorString(se));
      }
      if (*stack->err_host) {
        *stack->err_host = 0;
        stack->epoch += 1;
        stack_forget(stack);
        return fail(MOE_E_HIP, "a persistent decode call on this stack timed out");
      }
      const int stop = *stack->stop_host;
      if (stop < replay0 || stop > nl) {
        stack->epoch += 1;
        stack_forget(stack);
        return fail(MOE_E_HIP, "persistent decode stopped at layer %d (launched at %d)", stop, l0);
      }
      stack_launched(stack, l0, stop);
      int32_t st = pool_defer_hits(stack->pool, stack->layer_ids.data() + replay0,
                                   stack->idx_host + (size_t)replay0 * k, stop - replay0, k,
                                   stream);
      if (st != MOE_OK) return st;
      if (idx && stop > l0)
        MOE_HIP_TRY(hipMemcpyAsync(idx + (size_t)l0 * k, stack->idx_host + (size_t)l0 * k,
                                   (size_t)(stop - l0) * k * sizeof(int32_t),
                                   hipMemcpyHostToDevice, stream));
      if (stop == nl) return MOE_OK;
      // the stopped layer's choices (distinct, in selection order, as the
      // per-layer router lists them) -> resident and pinned
      int32_t experts[MOE_MAX_TOPK];
      const void* ptrs[MOE_MAX_TOPK];
      for (int j = 0; j < k; ++j) experts[j] = stack->idx_host[(size_t)stop * k + j];
      const int32_t lid = stack->layer_ids[stop];
      st = slotpool_acquire(stack->pool, lid, experts, k, stream, ptrs, nullptr);
      if (st != MOE_OK) return st;
      // the kernel that wrote the pinned words has finished (the sync
      // above); the relaunch writes them again only after what was enqueued
      // since, the copy of the choices included
      l0 = stop;
      replay0 = stop + 1;
      a.l0 = l0;
      a.y_start = stop > 0 ? a.y_layers + (size_t)(stop - 1) * H : nullptr;
      *stack->stop_host = nl;
      st = pool_before_lookup(stack->pool, stream);
      if (st == MOE_OK) st = stack_clear_stale(stack, l0, stream);
      const hipError_t le =
          st == MOE_OK ? launch_stack_decode(a, H, k, c.inter, c.shared_inter, c.bits, stream)
                       : hipSuccess;
      const int32_t rst = slotpool_release(stack->pool, lid, experts, k, stream);
      if (st != MOE_OK) return st;
      MOE_HIP_TRY(le);
      if (rst != MOE_OK) return rst;
    }
  }
  const int n = (int)stack->layers.size();
  const int H = stack->layers[0]->cfg.hidden, k = stack->layers[0]->cfg.top_k;
  const float* prev = nullptr;
  for (int l = 0; l < n; ++l) {
    moe_layer* L = stack->layers[l];
    float* yout = y_layers ? y_layers + (size_t)l * T * H : L->y;
    int32_t st = forward_decode(L, l == 0 ? x0 : nullptr, prev,
                                x_layers ? x_layers + (size_t)l * T * H : nullptr, T,
                                l == n - 1 ? y_last : nullptr, yout,
                                idx ? idx + (size_t)l * T * k : nullptr,
                                w ? w + (size_t)l * T * k : nullptr, stream);
    if (st != MOE_OK) return st;
    prev = yout;
  }
  return MOE_OK;
}

int32_t moe_stack_set_persistent(moe_stack* stack, int32_t enable) {
  clear_error();
  MOE_REQUIRE(stack, "null argument");
  stack->persistent_enabled = enable != 0;
  return MOE_OK;
}

int32_t moe_stack_persistent_active(const moe_stack* stack, int32_t* active) {
  clear_error();
  MOE_REQUIRE(stack && active, "null argument");
  *active = (stack->persistent_ok && stack->persistent_enabled) ? 1 : 0;
  return MOE_OK;
}

int32_t moe_stack_epoch(const moe_stack* stack, uint32_t* epoch) {
  clear_error();
  MOE_REQUIRE(stack && epoch, "null argument");
  *epoch = stack->epoch;
  return MOE_OK;
}

int32_t moe_stack_advance_epoch(moe_stack* stack, uint32_t n) {
  clear_error();
  MOE_REQUIRE(stack, "null argument");
  MOE_REQUIRE(stack->ps_mem, "the stack has no persistent path");
  MOE_HIP_TRY(hipDeviceSynchronize());
  std::vector<uint32_t> ep(stack->grid);
  MOE_HIP_TRY(hipMemcpy(ep.data(), stack->ps.epochs, ep.size() * 4, hipMemcpyDeviceToHost));
  for (uint32_t& v : ep) {
    if (v != stack->epoch) return fail(MOE_E_HIP, "device call counter %u, host %u", v, stack->epoch);
    v += n;
  }
  MOE_HIP_TRY(hipMemcpy(stack->ps.epochs, ep.data(), ep.size() * 4, hipMemcpyHostToDevice));
  stack->epoch += n;
  return MOE_OK;
}

int32_t moe_stack_set_phase_log(moe_stack* stack, uint64_t* phases) {
  clear_error();
  MOE_REQUIRE(stack, "null argument");
  MOE_REQUIRE(stack->ps_mem, "the stack has no persistent path");
#ifdef MOE_STACK_PHASES
  stack->ps.phases = phases;
  return MOE_OK;
#else
  (void)phases;
  return fail(MOE_E_INVAL, "this library was built without phase timestamps (MOE_STACK_PHASES)");
#endif
}

int32_t moe_stack_set_timeout(moe_stack* stack, int64_t microseconds) {
  clear_error();
  MOE_REQUIRE(stack && microseconds >= 0, "bad argument");
  MOE_REQUIRE(stack->ps_mem, "the stack has no persistent path");
  stack->ps.timeout_ticks = stack->clk_khz * microseconds / 1000;
  return MOE_OK;
}

int32_t moe_stack_destroy(moe_stack* stack) {
  clear_error();
  if (!stack) return MOE_OK;
  hipError_t e = hipSuccess;
  if (stack->ps_mem) {
    e = hipDeviceSynchronize();
    (void)hipFree(stack->ps_mem);
  }
  if (stack->err_host) (void)hipHostFree(stack->err_host);
  if (stack->stop_host) (void)hipHostFree(stack->stop_host);
  if (stack->idx_host) (void)hipHostFree(stack->idx_host);
  if (stack->xl_dev) (void)hipFree(stack->xl_dev);
  if (stack->yl_dev) (void)hipFree(stack->yl_dev);
  delete stack;
  if (e != hipSuccess) return fail(MOE_E_HIP, "hipDeviceSynchronize: %s", hipGetErrorString(e));
  return MOE_OK;
}

int32_t moe_calibrate_stream(const void* buf, int64_t bytes, int32_t phases, int32_t handoffs,
                             int32_t reps, float* ms, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(buf && ms, "null argument");
  MOE_REQUIRE(bytes > 0 && bytes % 16 == 0, "bytes must be a positive multiple of 16");
  MOE_REQUIRE(phases >= 1 && handoffs >= 0 && handoffs <= 8 && reps >= 1, "bad argument");
  int dev = 0, cus = 0, clk_khz = 0;
  MOE_HIP_TRY(hipGetDevice(&dev));
  MOE_HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  MOE_HIP_TRY(hipDeviceGetAttribute(&clk_khz, hipDeviceAttributeWallClockRate, dev));
  MOE_REQUIRE(cus >= kStackGrid, "needs %d compute units (the device has %d)", kStackGrid, cus);
  const size_t wbytes = (size_t)phases * (handoffs > 0 ? handoffs : 1) * kStackReplicas *
                        kStackGrid * 8;
  const size_t sizes[] = {wbytes, (size_t)kStackGrid * 4, (size_t)kStackGrid * kStackThreads * 4};
  size_t total = 0;
  for (size_t sz : sizes) total += align256(sz);
  void* mem = nullptr;
  int32_t* err = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  MOE_HIP_TRY(hipMalloc(&mem, total));
  hipError_t e = hipMemset(mem, 0, total);
  if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&err), 4, hipHostMallocDefault);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  uint8_t* p = static_cast<uint8_t*>(mem);
  uint64_t* words = reinterpret_cast<uint64_t*>(p);
  uint32_t* epochs = reinterpret_cast<uint32_t*>(p + align256(sizes[0]));
  float* sink = reinterpret_cast<float*>(p + align256(sizes[0]) + align256(sizes[1]));
  const int64_t ticks = (int64_t)clk_khz * 1000 * 2;
  if (e == hipSuccess) {
    *err = 0;
    // one launch to warm up, then `reps` timed ones (fresh tags each time)
    e = launch_stream_phases(buf, bytes, phases, handoffs, words, epochs, sink, err, ticks, stream);
    if (e == hipSuccess) e = hipEventRecord(e0, stream);
    for (int r = 0; r < reps && e == hipSuccess; ++r)
      e = launch_stream_phases(buf, bytes, phases, handoffs, words, epochs, sink, err, ticks,
                               stream);
    if (e == hipSuccess) e = hipEventRecord(e1, stream);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(ms, e0, e1);
    if (e == hipSuccess) *ms /= (float)reps;
  }
  const bool timed_out = err && *err;
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (err) (void)hipHostFree(err);
  (void)hipFree(mem);
  MOE_HIP_TRY(e);
  if (timed_out) return fail(MOE_E_HIP, "calibration kernel ran out of time");
  return MOE_OK;
}

int32_t moe_timer_create(int32_t kernel, int32_t capacity, moe_timer** out) {
  clear_error();
  MOE_REQUIRE(out && capacity >= 1 && kernel >= MOE_KERNEL_ROUTE && kernel <= MOE_KERNEL_STACK,
              "bad argument");
  moe_timer* t = new (std::nothrow) moe_timer{};
  if (!t) return fail(MOE_E_NOMEM, "host allocation failed");
  t->kernel = kernel;
  t->capacity = capacity;
  t->start.assign(capacity, nullptr);
  t->stop.assign(capacity, nullptr);
  for (int i = 0; i < capacity; ++i) {
    hipError_t e = hipEventCreate(&t->start[i]);
    if (e == hipSuccess) e = hipEventCreate(&t->stop[i]);
    if (e != hipSuccess) {
      moe_timer_destroy(t);
      return fail(MOE_E_HIP, "hipEventCreate: %s", hipGetErrorString(e));
    }
  }
  *out = t;
  return MOE_OK;
}

int32_t moe_timer_attach(moe_timer* timer) {
  clear_error();
  g_timer = timer;
  return MOE_OK;
}

int32_t moe_timer_read(moe_timer* timer, float* ms, int32_t* n) {
  clear_error();
  MOE_REQUIRE(timer && ms && n, "null argument");
  for (int i = 0; i < timer->count; ++i) {
    MOE_HIP_TRY(hipEventSynchronize(timer->stop[i]));
    MOE_HIP_TRY(hipEventElapsedTime(&ms[i], timer->start[i], timer->stop[i]));
  }
  *n = timer->count;
  timer->count = 0;
  return MOE_OK;
}

int32_t moe_timer_destroy(moe_timer* timer) {
  clear_error();
  if (!timer) return MOE_OK;
  if (g_timer == timer) g_timer = nullptr;
  for (hipEvent_t e : timer->start)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : timer->stop)
    if (e) (void)hipEventDestroy(e);
  delete timer;
  return MOE_OK;
}

}  // extern "C"
