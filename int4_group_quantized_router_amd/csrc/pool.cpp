// Fixed-stride expert stores (pinned host memory, or a file read with one
// pread per expert) and the bounded HBM slot pool.
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
// A file-backed store is the pages' container itself: blob (l, e) at byte
// offset (l*E + e)*stride of one file, fetched by ONE pread of `stride`
// bytes ([xix] how-it-works paragraph).  Reads use O_DIRECT where the file
// system allows it (the OS page cache is bypassed, as the pages' reads of
// the SSD are).  The kernel cannot DMA a direct read into HIP's pinned
// memory (the read fails with EFAULT), so a direct read lands in an
// ordinary page-aligned buffer and is copied into one of a ring of pinned
// staging buffers; a buffered read goes straight into the staging buffer.
// Each staging buffer is reused only after the host-to-device copy from it
// has finished.
// The pool also keeps a device table (layer, expert) -> slot address (NULL
// when not resident) so that kernels can find resident experts without the
// host.  The host changes a pinned mirror of it and, at the end of each call
// that changed entries, copies those entries on the copy stream after the
// fills; the compute stream waits for that, so a kernel enqueued after the
// call never sees an address before its blob has landed, nor an evicted one.
#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <atomic>
#include <cerrno>
#include <chrono>
#include <cstdlib>
#include <cstring>
#include <set>
#include <thread>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "common.h"

struct expert_store {
  int32_t layers;
  int32_t experts;
  int64_t stride;
  uint8_t* base;      // pinned host memory (kind 0), else NULL
  int32_t kind;       // 0 memory, 1 file read with O_DIRECT, 2 file read through the OS cache
  int fd = -1;        // file: buffered descriptor (writes, cache control, kind-2 reads)
  int fd_direct = -1; // file, kind 1: O_DIRECT read descriptor
  bool writable = false;
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
constexpr int kStaging = 8;  // pinned staging buffers of a pool over a file store

// pread until n bytes arrived; 0 or an errno value (EIO for a short file)
int read_full(int fd, uint8_t* dst, int64_t n, int64_t off) {
  while (n > 0) {
    const ssize_t r = pread(fd, dst, (size_t)n, (off_t)off);
    if (r < 0) {
      if (errno == EINTR) continue;
      return errno;
    }
    if (r == 0) return EIO;
    dst += r;
    off += r;
    n -= r;
  }
  return 0;
}

int write_full(int fd, const uint8_t* src, int64_t n, int64_t off) {
  while (n > 0) {
    const ssize_t r = pwrite(fd, src, (size_t)n, (off_t)off);
    if (r < 0) {
      if (errno == EINTR) continue;
      return errno;
    }
    src += r;
    off += r;
    n -= r;
  }
  return 0;
}

// One blob of a file store into dst (4096-aligned when the store reads
// with O_DIRECT).
int read_blob(const expert_store* st, int64_t key, uint8_t* dst) {
  const int fd = st->kind == 1 ? st->fd_direct : st->fd;
  return read_full(fd, dst, st->stride, key * st->stride);
}

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
  hipStream_t release_stream = nullptr;        // stream of the most recent release
  hipEvent_t release_event = nullptr;          // and the event it recorded
  const uint8_t** tab_dev = nullptr;           // device [L*E]: slot address or NULL
  const uint8_t** tab_host = nullptr;          // pinned mirror of tab_dev
  std::vector<int64_t> tab_changed;            // keys changed since the last push
  hipEvent_t tab_ready = nullptr;              // recorded after the last push
  bool tab_pushed = false;                     // tab_ready has been recorded
  hipStream_t tab_stream = nullptr;            // last stream made to wait on tab_ready
  // hits a stack call found through the device table, not yet applied to
  // the policy: (layer, expert) pairs in access order, and per batch the
  // end offset and the release event recorded for it
  std::vector<int32_t> pend;
  std::vector<std::pair<size_t, hipEvent_t>> pend_marks;
  std::vector<uint8_t*> stage;                 // file store: pinned staging buffers
  std::vector<hipEvent_t> stage_done;          // copy out of stage[i] finished
  std::vector<bool> stage_used;
  int stage_next = 0;
  std::vector<uint8_t*> bounce;                // file store: page-aligned ordinary memory
  bool read_via_bounce = false;
  int64_t tick = 0;
  slotpool_counters stats{};

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
  const int64_t key = p->key(x.layer, x.expert);
  p->where.erase(key);
  if (p->tab_host) {
    p->tab_host[key] = nullptr;
    p->tab_changed.push_back(key);
  }
  x.layer = x.expert = -1;
  x.count = x.last = 0;
  p->free_slots.insert(s);
#ifdef MOE_POOL_POISON
  // Debug builds: a dropped slot is overwritten with 0xFF bytes (f32 and
  // bf16 NaN, all-ones scales and fields) once its last reader is done, so
  // a kernel that reads a slot it no longer owns produces NaN instead of a
  // plausible stale expert.  The next fill of the slot replaces them.
  if (x.last_use) (void)hipStreamWaitEvent(p->copy, x.last_use, 0);
  (void)hipMemsetAsync(p->dev + (int64_t)s * p->store->stride, 0xFF, (size_t)p->store->stride,
                       p->copy);
#endif
}

// Copy the table entries changed since the last push (after everything
// already on the copy stream, i.e. after the fills they describe) and make
// `compute` wait for them; with compute NULL the host waits instead.
int32_t push_table(slotpool* p, hipStream_t compute) {
  if (p->tab_changed.empty()) return MOE_OK;
  // one copy per changed entry when few changed, else one per touched layer
  // row (the mirror row as it is now: later values only move it forward)
  const int64_t E = p->store->experts;
  std::set<int64_t> rows;
  for (int64_t key : p->tab_changed) rows.insert(key / E);
  if ((int64_t)p->tab_changed.size() <= (int64_t)rows.size() * 2) {
    for (int64_t key : p->tab_changed)
      MOE_HIP_TRY(hipMemcpyAsync(p->tab_dev + key, p->tab_host + key, sizeof(void*),
                                 hipMemcpyHostToDevice, p->copy));
  } else {
    for (int64_t row : rows)
      MOE_HIP_TRY(hipMemcpyAsync(p->tab_dev + row * E, p->tab_host + row * E,
                                 (size_t)E * sizeof(void*), hipMemcpyHostToDevice, p->copy));
  }
  p->tab_changed.clear();
  MOE_HIP_TRY(hipEventRecord(p->tab_ready, p->copy));
  p->tab_pushed = true;
  if (compute) {
    MOE_HIP_TRY(hipStreamWaitEvent(compute, p->tab_ready, 0));
    p->tab_stream = compute;
  } else {
    MOE_HIP_TRY(hipEventSynchronize(p->tab_ready));
  }
  return MOE_OK;
}

}  // namespace

namespace moe {

const uint8_t* const* pool_device_table(const slotpool* p, int32_t layer) {
  return p->tab_dev + (int64_t)layer * p->store->experts;
}

int32_t pool_defer_hits(slotpool* p, const int32_t* layers, const int32_t* experts, int32_t nl,
                        int32_t k, hipStream_t stream) {
  if (nl <= 0) return MOE_OK;
  // one release point for every slot the calls read, as release() records
  if (p->release_event && stream != p->release_stream)
    MOE_HIP_TRY(hipStreamWaitEvent(stream, p->release_event, 0));
  hipEvent_t ev = p->ring[p->ring_next];
  p->ring_next = (p->ring_next + 1) % p->ring.size();
  MOE_HIP_TRY(hipEventRecord(ev, stream));
  p->release_stream = stream;
  p->release_event = ev;
  for (int32_t l = 0; l < nl; ++l)
    for (int32_t i = 0; i < k; ++i) {
      p->pend.push_back(layers[l]);
      p->pend.push_back(experts[(size_t)l * k + i]);
    }
  p->pend_marks.emplace_back(p->pend.size(), ev);
  return MOE_OK;
}

int32_t pool_apply_pending(slotpool* p) {
  size_t i = 0;
  int32_t st = MOE_OK;
  for (const auto& mk : p->pend_marks) {
    for (; i < mk.first && st == MOE_OK; i += 2) {
      const int32_t layer = p->pend[i], e = p->pend[i + 1];
      auto it = p->where.find(p->key(layer, e));
      if (it == p->where.end()) {
        st = fail(MOE_E_HIP, "replayed access (layer %d, expert %d) is not resident", layer, e);
        break;
      }
      const int32_t sl = it->second;
      Slot& x = p->slots[sl];
      ++p->tick;
      if (x.pins == 0) p->victims.erase(p->vkey(sl));
      x.count += 1;
      x.last = p->tick;
      x.last_use = mk.second;
      p->stats.hits += 1;
      if (x.pins == 0) p->victims.insert(p->vkey(sl));
    }
  }
  p->pend.clear();
  p->pend_marks.clear();
  return st;
}

int32_t pool_check_layer(const slotpool* p, int32_t layer_index, int32_t experts,
                         int64_t stride) {
  const expert_store* st = p->store;
  if (layer_index < 0 || layer_index >= st->layers)
    return fail(MOE_E_INVAL, "layer_index %d outside the pool's store of %d layers", layer_index,
                st->layers);
  if (experts != st->experts)
    return fail(MOE_E_INVAL, "layer has %d experts, the pool's store %d", experts, st->experts);
  if (stride != st->stride)
    return fail(MOE_E_INVAL, "layer's blob stride %lld differs from the pool's store stride %lld",
                (long long)stride, (long long)st->stride);
  return MOE_OK;
}

int32_t pool_before_lookup(slotpool* p, hipStream_t stream) {
  // a stream that has not waited for the latest table push does so now
  if (p->tab_pushed && stream != p->tab_stream) {
    MOE_HIP_TRY(hipStreamWaitEvent(stream, p->tab_ready, 0));
    p->tab_stream = stream;
  }
  return MOE_OK;
}

}  // namespace moe

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
                                                    static_cast<uint8_t*>(base), 0};
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
  if (!store->base) {
    MOE_REQUIRE(store->writable, "file store was opened read-only");
    const int err = write_full(store->fd, static_cast<const uint8_t*>(blob), n,
                               ((int64_t)layer * store->experts + expert) * store->stride);
    if (err) return fail(MOE_E_IO, "pwrite of blob (%d, %d): %s", layer, expert, strerror(err));
    return MOE_OK;
  }
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
  MOE_REQUIRE(store->base, "a file-backed store has no host address");
  *ptr = store->base + ((int64_t)layer * store->experts + expert) * store->stride;
  return MOE_OK;
}

int32_t expert_store_open_file(const char* path, int32_t layers, int32_t experts, int64_t stride,
                               int32_t create, expert_store** out) {
  clear_error();
  MOE_REQUIRE(path && out && layers >= 1 && experts >= 1, "bad argument");
  MOE_REQUIRE(stride > 0 && stride % 4096 == 0, "stride must be a positive multiple of 4096");
  const int64_t bytes = (int64_t)layers * experts * stride;
  const int fd = open(path, create ? (O_RDWR | O_CREAT | O_TRUNC) : O_RDONLY, 0644);
  if (fd < 0) return fail(MOE_E_IO, "open(%s): %s", path, strerror(errno));
  if (create) {
    if (ftruncate(fd, (off_t)bytes) != 0) {
      const int err = errno;
      close(fd);
      return fail(MOE_E_IO, "ftruncate(%s, %lld): %s", path, (long long)bytes, strerror(err));
    }
  } else {
    struct stat sb;
    if (fstat(fd, &sb) != 0 || (int64_t)sb.st_size < bytes) {
      close(fd);
      return fail(MOE_E_INVAL, "%s holds fewer than %d x %d x %lld bytes", path, layers, experts,
                  (long long)stride);
    }
  }
  // O_DIRECT if the file system takes it for an aligned read of one page
  int fdd = open(path, O_RDONLY | O_DIRECT);
  if (fdd >= 0) {
    void* probe = nullptr;
    bool ok = posix_memalign(&probe, 4096, 4096) == 0;
    if (ok) ok = pread(fdd, probe, 4096, 0) == 4096;
    free(probe);
    if (!ok) {
      close(fdd);
      fdd = -1;
    }
  }
  expert_store* s = new (std::nothrow) expert_store{layers, experts, stride, nullptr,
                                                    fdd >= 0 ? 1 : 2};
  if (!s) {
    if (fdd >= 0) close(fdd);
    close(fd);
    return fail(MOE_E_NOMEM, "host allocation failed");
  }
  s->fd = fd;
  s->fd_direct = fdd;
  s->writable = create != 0;
  *out = s;
  return MOE_OK;
}

int32_t expert_store_kind(const expert_store* store, int32_t* kind) {
  clear_error();
  MOE_REQUIRE(store && kind, "null argument");
  *kind = store->kind;
  return MOE_OK;
}

int32_t expert_store_read(const expert_store* store, int32_t layer, int32_t expert, void* dst) {
  clear_error();
  MOE_REQUIRE(store && dst, "null argument");
  int32_t st = check_le(store, layer, expert);
  if (st != MOE_OK) return st;
  const int64_t key = (int64_t)layer * store->experts + expert;
  if (store->base) {
    std::memcpy(dst, store->base + key * store->stride, (size_t)store->stride);
    return MOE_OK;
  }
  uint8_t* out = static_cast<uint8_t*>(dst);
  void* bounce = nullptr;
  if (store->kind == 1 && reinterpret_cast<uintptr_t>(dst) % 4096) {
    if (posix_memalign(&bounce, 4096, (size_t)store->stride) != 0)
      return fail(MOE_E_NOMEM, "bounce buffer of %lld bytes", (long long)store->stride);
    out = static_cast<uint8_t*>(bounce);
  }
  const int err = read_blob(store, key, out);
  if (!err && bounce) std::memcpy(dst, bounce, (size_t)store->stride);
  free(bounce);
  if (err) return fail(MOE_E_IO, "pread of blob (%d, %d): %s", layer, expert, strerror(err));
  return MOE_OK;
}

int32_t expert_store_drop_cache(expert_store* store) {
  clear_error();
  MOE_REQUIRE(store, "null argument");
  if (store->base) return MOE_OK;
  if (store->writable && fdatasync(store->fd) != 0)
    return fail(MOE_E_IO, "fdatasync: %s", strerror(errno));
  const int err = posix_fadvise(store->fd, 0, 0, POSIX_FADV_DONTNEED);
  if (err) return fail(MOE_E_IO, "posix_fadvise: %s", strerror(err));
  return MOE_OK;
}

int32_t expert_store_destroy(expert_store* store) {
  clear_error();
  if (!store) return MOE_OK;
  if (!store->base) {
    if (store->fd_direct >= 0) close(store->fd_direct);
    const int rc = close(store->fd);
    delete store;
    if (rc != 0) return fail(MOE_E_IO, "close: %s", strerror(errno));
    return MOE_OK;
  }
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
  const size_t tab_bytes = (size_t)store->layers * store->experts * sizeof(void*);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&p->tab_ready, hipEventDisableTiming);
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&p->tab_dev), tab_bytes);
  if (e == hipSuccess) e = hipMemset(p->tab_dev, 0, tab_bytes);
  if (e == hipSuccess)
    e = hipHostMalloc(reinterpret_cast<void**>(&p->tab_host), tab_bytes, hipHostMallocDefault);
  if (e == hipSuccess) std::memset(p->tab_host, 0, tab_bytes);
  if (!store->base) {
    p->bounce.resize(kStaging, nullptr);
    for (int i = 0; i < kStaging && e == hipSuccess; ++i) {
      void* b = nullptr;
      if (posix_memalign(&b, 4096, (size_t)store->stride) != 0) e = hipErrorOutOfMemory;
      p->bounce[i] = static_cast<uint8_t*>(b);
    }
    p->read_via_bounce = store->kind == 1;
    p->stage.resize(kStaging, nullptr);
    p->stage_done.resize(kStaging, nullptr);
    p->stage_used.resize(kStaging, false);
    for (int i = 0; i < kStaging && e == hipSuccess; ++i) {
      e = hipHostMalloc(reinterpret_cast<void**>(&p->stage[i]), (size_t)store->stride,
                        hipHostMallocDefault);
      if (e == hipSuccess && reinterpret_cast<uintptr_t>(p->stage[i]) % 4096)
        e = hipErrorInvalidValue;  // O_DIRECT needs page-aligned buffers
      if (e == hipSuccess) e = hipEventCreateWithFlags(&p->stage_done[i], hipEventDisableTiming);
    }
  }
  if (e != hipSuccess) {
    slotpool_destroy(p);
    return fail(MOE_E_HIP, "slot pool setup: %s", hipGetErrorString(e));
  }
  *out = p;
  return MOE_OK;
}

}  // extern "C"

namespace {

// prefetch: load only the experts not resident, into free slots, unpinned,
// count 0, without advancing the tick; stop at the first that finds no free
// slot (slot_ptrs and was_miss unused; *loaded counts the loads)
int32_t acquire_impl(slotpool* pool, int32_t layer, const int32_t* experts, int32_t n,
                     hipStream_t compute, const void** slot_ptrs, uint8_t* was_miss,
                     bool prefetch = false, int32_t* loaded = nullptr) {
  for (int i = 0; i < n; ++i) {
    int32_t st = check_le(pool->store, layer, experts[i]);
    if (st != MOE_OK) return st;
  }
  std::vector<int32_t> pinned;
  pinned.reserve(n);
  const int64_t stride = pool->store->stride;
  // misses of a file store whose reads have not run yet: (slot, key, staging buffer)
  std::vector<std::tuple<int32_t, int64_t, int>> pend;

  // Enqueue the fill of slot s from host bytes src: the copy waits for the
  // slot's last reader, the compute stream waits for the copy.
  auto fill = [&](int32_t s, const uint8_t* src, int si) -> int32_t {
    Slot& x = pool->slots[s];
    if (x.last_use) MOE_HIP_TRY(hipStreamWaitEvent(pool->copy, x.last_use, 0));
    MOE_HIP_TRY(hipMemcpyAsync(pool->dev + (int64_t)s * stride, src, (size_t)stride,
                               hipMemcpyHostToDevice, pool->copy));
    if (si >= 0) MOE_HIP_TRY(hipEventRecord(pool->stage_done[si], pool->copy));
    MOE_HIP_TRY(hipEventRecord(x.ready, pool->copy));
    MOE_HIP_TRY(hipStreamWaitEvent(compute, x.ready, 0));
    x.fill_pending = true;
    pool->stats.bytes_h2d += stride;
    return MOE_OK;
  };

  // Run the pending reads (one thread each when there are several), then
  // enqueue their copies in order.  A failed read drops every pending slot
  // and unpins the rest of the call.
  auto flush = [&]() -> int32_t {
    if (pend.empty()) return MOE_OK;
    std::vector<int> errs(pend.size(), 0);
    std::atomic<bool> efault{false};
    const bool via_bounce = pool->read_via_bounce;
    auto read_one = [&](size_t i) {
      const int64_t k = std::get<1>(pend[i]);
      const int si = std::get<2>(pend[i]);
      int err = via_bounce ? EFAULT : read_blob(pool->store, k, pool->stage[si]);
      if (err == EFAULT) {
        if (!via_bounce) efault = true;
        err = read_blob(pool->store, k, pool->bounce[si]);
        if (!err) std::memcpy(pool->stage[si], pool->bounce[si], (size_t)stride);
      }
      errs[i] = err;
    };
    const auto t0 = std::chrono::steady_clock::now();
    if (pend.size() == 1) {
      read_one(0);
    } else {
      std::vector<std::thread> th;
      th.reserve(pend.size());
      for (size_t i = 0; i < pend.size(); ++i) th.emplace_back(read_one, i);
      for (std::thread& t : th) t.join();
    }
    pool->stats.read_ns += std::chrono::duration_cast<std::chrono::nanoseconds>(
                               std::chrono::steady_clock::now() - t0)
                               .count();
    if (efault) pool->read_via_bounce = true;
    for (size_t i = 0; i < pend.size(); ++i) {
      if (!errs[i]) continue;
      const int64_t k_bad = std::get<1>(pend[i]);
      std::set<int32_t> dropped;
      for (const auto& q : pend) {
        pool->slots[std::get<0>(q)].pins = 0;
        drop(pool, std::get<0>(q));
        dropped.insert(std::get<0>(q));
      }
      for (int32_t ps : pinned)
        if (!dropped.count(ps)) unpin(pool, ps);
      pend.clear();
      return fail(MOE_E_IO, "pread of blob (layer %lld, expert %lld): %s",
                  (long long)(k_bad / pool->store->experts),
                  (long long)(k_bad % pool->store->experts), strerror(errs[i]));
    }
    for (const auto& [s, k, si] : pend) {
      (void)k;
      const int32_t st = fill(s, pool->stage[si], si);
      if (st != MOE_OK) return st;
      pool->stats.bytes_read += stride;
    }
    pend.clear();
    return MOE_OK;
  };

  for (int i = 0; i < n; ++i) {
    const int32_t e = experts[i];
    const int64_t k = pool->key(layer, e);
    auto it = pool->where.find(k);
    if (prefetch) {
      if (it != pool->where.end()) continue;
      if (pool->free_slots.empty()) break;
    } else {
      ++pool->tick;
    }
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
          // experts admitted earlier in the call are filled, then unpinned
          const int32_t st = flush();
          if (st != MOE_OK) return st;
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
      x.layer = layer;
      x.expert = e;
      x.count = prefetch ? 0 : 1;
      x.last = pool->tick;
      x.pins = prefetch ? 0 : 1;
      pool->where[k] = s;
      pool->tab_host[k] = pool->dev + (int64_t)s * stride;
      pool->tab_changed.push_back(k);
      if (prefetch) {
        pool->victims.insert(pool->vkey(s));
        pool->stats.prefetched += 1;
        if (loaded) *loaded += 1;
      } else {
        pool->stats.misses += 1;
      }
      miss = true;
      if (pool->store->base) {
        const int32_t st = fill(s, pool->store->base + k * stride, -1);
        if (st != MOE_OK) return st;
      } else {
        // file store: the read waits in `pend` (at most one per staging
        // buffer) until the call's misses are known
        if ((int)pend.size() == kStaging) {
          const int32_t st = flush();
          if (st != MOE_OK) return st;
        }
        const int si = pool->stage_next;
        pool->stage_next = (si + 1) % kStaging;
        if (pool->stage_used[si]) MOE_HIP_TRY(hipEventSynchronize(pool->stage_done[si]));
        pool->stage_used[si] = true;
        pend.emplace_back(s, k, si);
      }
    }
    if (prefetch) continue;
    pinned.push_back(s);
    slot_ptrs[i] = pool->dev + (int64_t)s * stride;
    if (was_miss) was_miss[i] = miss ? 1 : 0;
  }
  return flush();
}

}  // namespace

// every public call that reads or changes the policy first applies the hits
// a stack call held back (pool_defer_hits), so all see one access order
#define MOE_POOL_APPLY(p)                                 \
  do {                                                    \
    const int32_t pst_ = moe::pool_apply_pending(p);      \
    if (pst_ != MOE_OK) return pst_;                      \
  } while (0)

extern "C" {

int32_t slotpool_acquire(slotpool* pool, int32_t layer, const int32_t* experts, int32_t n,
                         hipStream_t compute, const void** slot_ptrs, uint8_t* was_miss) {
  clear_error();
  MOE_REQUIRE(pool && (n == 0 || (experts && slot_ptrs)) && n >= 0, "bad argument");
  MOE_POOL_APPLY(pool);
  const int32_t st = acquire_impl(pool, layer, experts, n, compute, slot_ptrs, was_miss);
  // the table follows every admission and eviction of the call, also on
  // the error paths (entries dropped there are cleared)
  const int32_t pt = push_table(pool, compute);
  return st != MOE_OK ? st : pt;
}

int32_t slotpool_prefetch(slotpool* pool, int32_t layer, const int32_t* experts, int32_t n,
                          hipStream_t compute, int32_t* loaded) {
  clear_error();
  MOE_REQUIRE(pool && (n == 0 || experts) && n >= 0, "bad argument");
  if (loaded) *loaded = 0;
  MOE_POOL_APPLY(pool);
  for (int i = 0; i < n; ++i) {
    const int32_t st = check_le(pool->store, layer, experts[i]);
    if (st != MOE_OK) return st;
  }
  const int32_t st = acquire_impl(pool, layer, experts, n, compute, nullptr, nullptr, true, loaded);
  const int32_t pt = push_table(pool, compute);
  return st != MOE_OK ? st : pt;
}

int32_t slotpool_release(slotpool* pool, int32_t layer, const int32_t* experts, int32_t n,
                         hipStream_t compute) {
  clear_error();
  MOE_REQUIRE(pool && (n == 0 || experts) && n >= 0, "bad argument");
  if (n == 0) return MOE_OK;
  MOE_POOL_APPLY(pool);
  hipEvent_t ev = pool->ring[pool->ring_next];
  pool->ring_next = (pool->ring_next + 1) % pool->ring.size();
  // A slot may still hold a ring event that is re-recorded here.  That is
  // safe while every release comes from one stream: the event then marks a
  // later point of the same stream and a refill only waits longer.  When
  // the caller switches streams, the new stream first waits for the old
  // stream's last release, so every later release point is also after
  // every read released before it, whichever stream made it.
  if (pool->release_event && compute != pool->release_stream)
    MOE_HIP_TRY(hipStreamWaitEvent(compute, pool->release_event, 0));
  MOE_HIP_TRY(hipEventRecord(ev, compute));
  pool->release_stream = compute;
  pool->release_event = ev;
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
  MOE_POOL_APPLY(pool);
  auto it = pool->where.find(pool->key(layer, expert));
  if (it == pool->where.end()) return MOE_OK;
  if (pool->slots[it->second].pins)
    return fail(MOE_E_BUSY, "(layer %d, expert %d) is pinned", layer, expert);
  drop(pool, it->second);
  pool->stats.evictions += 1;
  return push_table(pool, nullptr);
}

int32_t slotpool_flush(slotpool* pool) {
  clear_error();
  MOE_REQUIRE(pool, "null argument");
  MOE_POOL_APPLY(pool);
  for (const auto& kv : pool->where)
    if (pool->slots[kv.second].pins) return fail(MOE_E_BUSY, "flush with pinned slots");
  std::vector<int32_t> res;
  for (const auto& kv : pool->where) res.push_back(kv.second);
  for (int32_t s : res) drop(pool, s);
  return push_table(pool, nullptr);
}

int32_t slotpool_stats(const slotpool* pool, slotpool_counters* out) {
  clear_error();
  MOE_REQUIRE(pool && out, "null argument");
  // hits held back by a stack call are part of the pool's logical state
  MOE_POOL_APPLY(const_cast<slotpool*>(pool));
  *out = pool->stats;
  return MOE_OK;
}

int32_t slotpool_get_stats(const slotpool* pool, slotpool_counters* out) {
  return slotpool_stats(pool, out);
}

int32_t slotpool_slot_of(const slotpool* pool, int32_t layer, int32_t expert, int32_t* slot) {
  clear_error();
  MOE_REQUIRE(pool && slot, "null argument");
  MOE_POOL_APPLY(const_cast<slotpool*>(pool));
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
  if (pool->tab_ready) (void)hipEventDestroy(pool->tab_ready);
  if (pool->tab_dev) (void)hipFree(pool->tab_dev);
  if (pool->tab_host) (void)hipHostFree(pool->tab_host);
  for (hipEvent_t ev : pool->stage_done)
    if (ev) (void)hipEventDestroy(ev);
  for (uint8_t* b : pool->stage)
    if (b) (void)hipHostFree(b);
  for (uint8_t* b : pool->bounce) free(b);
  if (pool->copy) (void)hipStreamDestroy(pool->copy);
  if (pool->dev) (void)hipFree(pool->dev);
  delete pool;
  if (e != hipSuccess) return fail(MOE_E_HIP, "copy stream sync: %s", hipGetErrorString(e));
  return MOE_OK;
}

}  // extern "C"
