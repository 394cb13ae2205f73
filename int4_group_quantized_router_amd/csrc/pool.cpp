// Fixed-stride pinned-host expert store and the bounded HBM slot pool.
//
// The pages keep only the dense core resident and stream routed experts on
// demand: each expert is one fixed-stride blob fetched with a single read
// into a bounded slot pool, popular experts stay cached, eviction is LFU
// plus recency, and the hit rate they report is 43-70% ([xix] how-it-works
// and lineage paragraphs; [digest] "Core Mechanics"; [lens]
// "エキスパートストリーミングの仕組み").  Here the backing store is pinned
// host memory and one miss is exactly one hipMemcpyAsync of `stride` bytes
// on the pool's own copy stream, overlapped with compute on the caller's
// stream.  Hazards are ordered with events ([lens] "TurboFieldfareとの関係"
// mentions explicit hazard management):
//   * refilling a slot waits for the event recorded when its previous
//     contents were last released on a compute stream (write after read);
//   * the compute stream waits for the copy's event before any kernel reads
//     the slot (read after write).
#include <cstring>
#include <set>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "common.h"

struct expert_store {
  int32_t layers;
  int32_t experts;
  int64_t stride;
  uint8_t* base;  // pinned host
};

namespace {

struct Slot {
  int32_t layer = -1;
  int32_t expert = -1;
  int64_t count = 0;
  int64_t last = 0;
  int32_t pins = 0;
  hipEvent_t ready = nullptr;      // recorded on the copy stream after the fill
  bool fill_pending = false;       // ready not yet observed complete
  hipEvent_t last_use = nullptr;   // ring event recorded at the last release
};

using VictimKey = std::tuple<int64_t, int64_t, int32_t, int32_t, int32_t>;  // count, tick, l, e, slot

constexpr int kEventRing = 4096;

}  // namespace

struct slotpool {
  const expert_store* store;
  int64_t capacity;
  int device;
  uint8_t* dev;
  hipStream_t copy;
  std::vector<Slot> slots;
  std::unordered_map<int64_t, int32_t> where;  // l*E + e -> slot
  std::set<VictimKey> victims;                 // resident and unpinned
  std::set<int32_t> free_slots;
  std::vector<hipEvent_t> ring;                // release events, reused round-robin
  size_t ring_next = 0;
  int64_t tick = 0;
  slotpool_stats stats{};

  int64_t key(int32_t l, int32_t e) const { return (int64_t)l * store->experts + e; }
  VictimKey vkey(int32_t s) const {
    const Slot& x = slots[s];
    return VictimKey(x.count, x.last, x.layer, x.expert, s);
  }
};

using namespace moe;

namespace {

int32_t check_le(const expert_store* st, int32_t l, int32_t e) {
  if (l < 0 || l >= st->layers || e < 0 || e >= st->experts)
    return fail(MOE_E_RANGE, "(layer %d, expert %d) outside [0,%d) x [0,%d)", l, e, st->layers,
                st->experts);
  return MOE_OK;
}

void unpin(slotpool* p, int32_t s) {
  Slot& x = p->slots[s];
  if (x.pins > 0 && --x.pins == 0) p->victims.insert(p->vkey(s));
}

void drop(slotpool* p, int32_t s) {
  Slot& x = p->slots[s];
  p->victims.erase(p->vkey(s));
  p->where.erase(p->key(x.layer, x.expert));
  x.layer = x.expert = -1;
  x.count = x.last = 0;
  p->free_slots.insert(s);
}

}  // namespace

extern "C" {

int32_t expert_store_create(int32_t layers, int32_t experts, int64_t stride, expert_store** out) {
  clear_error();
  MOE_REQUIRE(out && layers >= 1 && experts >= 1, "bad argument");
  MOE_REQUIRE(stride > 0 && stride % 4096 == 0, "stride must be a positive multiple of 4096");
  const int64_t bytes = (int64_t)layers * experts * stride;
  void* base = nullptr;
  hipError_t e = hipHostMalloc(&base, (size_t)bytes, hipHostMallocDefault);
  if (e != hipSuccess || !base)
    return fail(MOE_E_NOMEM, "hipHostMalloc(%lld bytes): %s", (long long)bytes,
                hipGetErrorString(e));
  expert_store* s = new (std::nothrow) expert_store{layers, experts, stride,
                                                    static_cast<uint8_t*>(base)};
  if (!s) {
    (void)hipHostFree(base);
    return fail(MOE_E_NOMEM, "host allocation failed");
  }
  *out = s;
  return MOE_OK;
}

int32_t expert_store_write(expert_store* store, int32_t layer, int32_t expert, const void* blob,
                           int64_t n) {
  clear_error();
  MOE_REQUIRE(store && blob, "null argument");
  int32_t st = check_le(store, layer, expert);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(n >= 0 && n <= store->stride, "n = %lld exceeds stride %lld", (long long)n,
              (long long)store->stride);
  std::memcpy(store->base + ((int64_t)layer * store->experts + expert) * store->stride, blob,
              (size_t)n);
  return MOE_OK;
}

int32_t expert_store_host_ptr(const expert_store* store, int32_t layer, int32_t expert,
                              void** ptr) {
  clear_error();
  MOE_REQUIRE(store && ptr, "null argument");
  int32_t st = check_le(store, layer, expert);
  if (st != MOE_OK) return st;
  *ptr = store->base + ((int64_t)layer * store->experts + expert) * store->stride;
  return MOE_OK;
}

int32_t expert_store_destroy(expert_store* store) {
  clear_error();
  if (!store) return MOE_OK;
  hipError_t e = hipHostFree(store->base);
  delete store;
  if (e != hipSuccess) return fail(MOE_E_HIP, "hipHostFree: %s", hipGetErrorString(e));
  return MOE_OK;
}

int32_t slotpool_create(const expert_store* store, int64_t capacity, int32_t device,
                        slotpool** out) {
  clear_error();
  MOE_REQUIRE(store && out, "null argument");
  MOE_REQUIRE(capacity >= 1 && capacity <= (1ll << 31) - 1, "capacity must be >= 1");
  MOE_HIP_TRY(hipSetDevice(device));
  slotpool* p = new (std::nothrow) slotpool{};
  if (!p) return fail(MOE_E_NOMEM, "host allocation failed");
  p->store = store;
  p->capacity = capacity;
  p->device = device;
  hipError_t e = hipMalloc(reinterpret_cast<void**>(&p->dev), (size_t)(capacity * store->stride));
  if (e != hipSuccess) {
    delete p;
    return fail(MOE_E_NOMEM, "slot pool hipMalloc(%lld x %lld): %s", (long long)capacity,
                (long long)store->stride, hipGetErrorString(e));
  }
  e = hipStreamCreateWithFlags(&p->copy, hipStreamNonBlocking);
  p->slots.resize((size_t)capacity);
  for (int64_t s = 0; s < capacity && e == hipSuccess; ++s) {
    e = hipEventCreateWithFlags(&p->slots[s].ready, hipEventDisableTiming);
    p->free_slots.insert((int32_t)s);
  }
  p->ring.resize(kEventRing, nullptr);
  for (int i = 0; i < kEventRing && e == hipSuccess; ++i)
    e = hipEventCreateWithFlags(&p->ring[i], hipEventDisableTiming);
  if (e != hipSuccess) {
    slotpool_destroy(p);
    return fail(MOE_E_HIP, "slot pool setup: %s", hipGetErrorString(e));
  }
  *out = p;
  return MOE_OK;
}

int32_t slotpool_acquire(slotpool* pool, int32_t layer, const int32_t* experts, int32_t n,
                         hipStream_t compute, const void** slot_ptrs, uint8_t* was_miss) {
  clear_error();
  MOE_REQUIRE(pool && (n == 0 || (experts && slot_ptrs)) && n >= 0, "bad argument");
  for (int i = 0; i < n; ++i) {
    int32_t st = check_le(pool->store, layer, experts[i]);
    if (st != MOE_OK) return st;
  }
  std::vector<int32_t> pinned;
  pinned.reserve(n);
  const int64_t stride = pool->store->stride;
  for (int i = 0; i < n; ++i) {
    const int32_t e = experts[i];
    const int64_t k = pool->key(layer, e);
    ++pool->tick;
    auto it = pool->where.find(k);
    int32_t s;
    bool miss = false;
    if (it != pool->where.end()) {
      s = it->second;
      Slot& x = pool->slots[s];
      if (x.pins == 0) pool->victims.erase(pool->vkey(s));
      x.count += 1;
      x.last = pool->tick;
      x.pins += 1;
      pool->stats.hits += 1;
      if (x.fill_pending) {
        hipError_t q = hipEventQuery(x.ready);
        if (q == hipSuccess) {
          x.fill_pending = false;
        } else if (q == hipErrorNotReady) {
          MOE_HIP_TRY(hipStreamWaitEvent(compute, x.ready, 0));
        } else {
          MOE_HIP_TRY(q);
        }
      }
    } else {
      if (pool->free_slots.empty()) {
        if (pool->victims.empty()) {
          for (int32_t ps : pinned) unpin(pool, ps);
          return fail(MOE_E_POOL_EXHAUSTED,
                      "all %lld slots pinned; cannot admit (layer %d, expert %d)",
                      (long long)pool->capacity, layer, e);
        }
        const int32_t v = std::get<4>(*pool->victims.begin());
        drop(pool, v);
        pool->stats.evictions += 1;
      }
      s = *pool->free_slots.begin();
      pool->free_slots.erase(pool->free_slots.begin());
      Slot& x = pool->slots[s];
      if (x.last_use) MOE_HIP_TRY(hipStreamWaitEvent(pool->copy, x.last_use, 0));
      const uint8_t* src = pool->store->base + k * stride;
      MOE_HIP_TRY(hipMemcpyAsync(pool->dev + (int64_t)s * stride, src, (size_t)stride,
                                 hipMemcpyHostToDevice, pool->copy));
      MOE_HIP_TRY(hipEventRecord(x.ready, pool->copy));
      MOE_HIP_TRY(hipStreamWaitEvent(compute, x.ready, 0));
      x.fill_pending = true;
      x.layer = layer;
      x.expert = e;
      x.count = 1;
      x.last = pool->tick;
      x.pins = 1;
      pool->where[k] = s;
      pool->stats.misses += 1;
      pool->stats.bytes_h2d += stride;
      miss = true;
    }
    pinned.push_back(s);
    slot_ptrs[i] = pool->dev + (int64_t)s * stride;
    if (was_miss) was_miss[i] = miss ? 1 : 0;
  }
  return MOE_OK;
}

int32_t slotpool_release(slotpool* pool, int32_t layer, const int32_t* experts, int32_t n,
                         hipStream_t compute) {
  clear_error();
  MOE_REQUIRE(pool && (n == 0 || experts) && n >= 0, "bad argument");
  if (n == 0) return MOE_OK;
  hipEvent_t ev = pool->ring[pool->ring_next];
  pool->ring_next = (pool->ring_next + 1) % pool->ring.size();
  // A re-recorded ring event marks a later point of the same stream, so a
  // slot still holding it only waits longer: ordering stays safe.
  MOE_HIP_TRY(hipEventRecord(ev, compute));
  for (int i = 0; i < n; ++i) {
    auto it = pool->where.find(pool->key(layer, experts[i]));
    if (it == pool->where.end()) continue;
    pool->slots[it->second].last_use = ev;
    unpin(pool, it->second);
  }
  return MOE_OK;
}

int32_t slotpool_evict(slotpool* pool, int32_t layer, int32_t expert) {
  clear_error();
  MOE_REQUIRE(pool, "null argument");
  int32_t st = check_le(pool->store, layer, expert);
  if (st != MOE_OK) return st;
  auto it = pool->where.find(pool->key(layer, expert));
  if (it == pool->where.end()) return MOE_OK;
  if (pool->slots[it->second].pins)
    return fail(MOE_E_BUSY, "(layer %d, expert %d) is pinned", layer, expert);
  drop(pool, it->second);
  pool->stats.evictions += 1;
  return MOE_OK;
}

int32_t slotpool_flush(slotpool* pool) {
  clear_error();
  MOE_REQUIRE(pool, "null argument");
  for (const auto& kv : pool->where)
    if (pool->slots[kv.second].pins) return fail(MOE_E_BUSY, "flush with pinned slots");
  std::vector<int32_t> res;
  for (const auto& kv : pool->where) res.push_back(kv.second);
  for (int32_t s : res) drop(pool, s);
  return MOE_OK;
}

int32_t slotpool_get_stats(const slotpool* pool, slotpool_stats* out) {
  clear_error();
  MOE_REQUIRE(pool && out, "null argument");
  *out = pool->stats;
  return MOE_OK;
}

int32_t slotpool_slot_of(const slotpool* pool, int32_t layer, int32_t expert, int32_t* slot) {
  clear_error();
  MOE_REQUIRE(pool && slot, "null argument");
  auto it = pool->where.find(pool->key(layer, expert));
  *slot = it == pool->where.end() ? -1 : it->second;
  return MOE_OK;
}

int32_t slotpool_destroy(slotpool* pool) {
  clear_error();
  if (!pool) return MOE_OK;
  hipError_t e = hipSuccess;
  if (pool->copy) e = hipStreamSynchronize(pool->copy);
  for (Slot& x : pool->slots)
    if (x.ready) (void)hipEventDestroy(x.ready);
  for (hipEvent_t ev : pool->ring)
    if (ev) (void)hipEventDestroy(ev);
  if (pool->copy) (void)hipStreamDestroy(pool->copy);
  if (pool->dev) (void)hipFree(pool->dev);
  delete pool;
  if (e != hipSuccess) return fail(MOE_E_HIP, "copy stream sync: %s", hipGetErrorString(e));
  return MOE_OK;
}

}  // extern "C"
