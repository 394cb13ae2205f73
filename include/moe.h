/*
 * moe.h -- C ABI of libmoe: a routed-expert MoE layer whose experts run
 * straight from affine group-quantised int4/int8 weights on AMD gfx950.
 *
 * Page abbreviations in the citations:
 *   [xix]    xix.ai, "Swiftlet Packs 80B Qwen Into Mac With 4.3GB Memory;
 *            iPhone 17 to Run 35B Natively" (Korean; xix.ai/ru has the same
 *            text in Russian).
 *   [ttj]    ttj.kr article on Swiftlet, the MoE streaming runtime for Apple
 *            devices.
 *   [digest] paper-digest.app, "Swiftlet: Mac에서 80B Qwen을 4.3GB RAM으로,
 *            iPhone에서 35B를 돌리는 런타임".
 *   [lens]   agentlenshq.com, "Swiftletは低RAM使用量でMacとiPhone上で35Bおよび
 *            80B Qwenモデルを可能にする".
 *
 * Conventions for every call:
 *   - Returns int32_t status: MOE_OK (0) or a negative MOE_E_* code; the
 *     message of the last failure on the calling thread is moe_last_error().
 *     No C++ exception crosses this boundary.
 *   - Device work is enqueued on the caller's stream and the call returns
 *     without synchronising, except where a call says otherwise.  A kernel
 *     fault surfaces at the next synchronising HIP call as MOE_E_HIP.
 *   - bf16 values travel as uint16_t bit patterns.  Matrices are row-major.
 *   - Pointers named "device" are caller-owned device memory; the library
 *     keeps non-owning views of weights until the object that uses them is
 *     destroyed.  Stores, pools, layers and stacks own their own memory.
 *   - Objects are single-host-thread: calls on one object must not overlap.
 */
#ifndef MOE_H
#define MOE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_E_INVAL = -1,          /* bad argument (shape, null pointer, k > E ...) */
  MOE_E_NOMEM = -2,          /* host or device allocation failed */
  MOE_E_HIP = -3,            /* a HIP runtime call failed */
  MOE_E_RANGE = -4,          /* layer or expert index out of range */
  MOE_E_POOL_EXHAUSTED = -5, /* every slot is pinned; nothing can be evicted */
  MOE_E_BUSY = -6,           /* the slot is pinned by an in-flight acquire */
  MOE_E_IO = -7              /* a file operation of a file-backed store failed */
};

#define MOE_MAX_TOPK 16      /* largest k the router supports */
#define MOE_MAX_DECODE_T 8   /* tokens per call on the per-token (GEMV) path */

/* Last failure message on this thread ("" if none). */
const char* moe_last_error(void);

/* ------------------------------------------------------------------------
 * Quantised expert format.
 *
 * One expert is three matrices W[out, in]: gate [inter, hidden], up [inter,
 * hidden] and down [hidden, inter] (SwiGLU).  Each is affine group-quantised
 * in the MLX convention the pages name ([xix] lineage paragraph: MLX-style
 * int4/int8 group quantisation; [lens] "TurboFieldfareとの関係"):
 *   W[r, c] = s[r, c/group] * q[r, c] + b[r, c/group],
 * q unsigned in [0, 2^bits), packed 32/bits fields per uint32 word with
 * field c of a row at bit bits*(c mod 32/bits) of word c/(32/bits); s and b
 * bf16.  group is 64; bits is 4 or 8.
 *
 * Blob: one expert in one contiguous fixed-size record, so fetching an
 * expert is one copy ([xix] how-it-works paragraph: experts repacked into
 * fixed-stride blobs so one read is one fetch).  Sections, each 256-byte
 * aligned, in this order: gate.q, up.q, down.q, gate.sb, up.sb, down.sb.
 * An "sb" section holds one uint32 per (row, group): scale bits in the low
 * half, bias bits in the high half.  stride = bytes rounded up to 4096;
 * blob (l, e) of a layered store sits at byte (l*E + e) * stride (64-bit).
 * ---------------------------------------------------------------------- */
typedef struct moe_qshape {
  int32_t hidden;   /* H: input of gate/up, output of down; multiple of group */
  int32_t inter;    /* I: expert intermediate size; multiple of group */
  int32_t group;    /* must be 64 */
  int32_t bits;     /* 4 or 8 */
} moe_qshape;

typedef struct moe_blob_layout {
  int64_t q_off[3];     /* byte offsets of gate/up/down packed words */
  int64_t sb_off[3];    /* byte offsets of gate/up/down (scale, bias) words */
  int64_t q_bytes[3];
  int64_t sb_bytes[3];
  int64_t bytes;        /* end of the last section */
  int64_t stride;       /* bytes rounded up to 4096 */
} moe_blob_layout;

/* One matrix in canonical host form: q words [out, in*bits/32], s and b
 * bf16 bits [out, in/group]. */
typedef struct moe_qmatrix_host {
  const uint32_t* q;
  const uint16_t* s;
  const uint16_t* b;
} moe_qmatrix_host;

/* Section offsets and stride of one expert blob.  MOE_E_INVAL on a shape
 * the kernels do not support. */
int32_t moe_blob_layout_get(const moe_qshape* shape, moe_blob_layout* out);

/* Write one expert (gate, up, down in canonical form) into a host blob of
 * layout.stride bytes; padding bytes are zeroed.  Host only, synchronous. */
int32_t moe_blob_pack(const moe_qshape* shape, const moe_qmatrix_host* gate,
                      const moe_qmatrix_host* up, const moe_qmatrix_host* down,
                      void* blob_host);

/* ------------------------------------------------------------------------
 * Router: logits, softmax, top-k, renormalise ([xix] how-it-works
 * paragraph: each layer sends a token to 10 of 512 experts (80B) or 8 of
 * 256 (35B); [lens] "エキスパートストリーミングの仕組み").
 *
 *   logits[t, e] = sum_h x[t, h] * Wr[e, h] + rb[e]      (f32 accumulation)
 *   idx[t, :]    = the k largest logits, ordered by (logit desc, index asc)
 *   w[t, j]      = softmax over all E, renormalised over the chosen k
 *                = exp(l_j - l_0) / sum_i exp(l_i - l_0)
 *   sigma[t]     = 1 / (1 + exp(-(wsg . x_t)))           (shared-expert gate)
 *
 * x: device bf16 [T, H]; Wr: device f32 [E, H]; rb: device f32 [E] or
 * NULL (zero bias); wsg: device f32 [H] or NULL (then sigma is not written).
 * idx: device int32 [T, k]; w: device f32 [T, k]; sigma: device f32 [T] or
 * NULL; logits: device f32 [T, E] or NULL (then not exported; the
 * per-token path keeps them in stream-ordered scratch, hipMallocAsync /
 * hipFreeAsync on `stream`).  MOE_E_INVAL if k < 1, k > E,
 * k > MOE_MAX_TOPK, E > 1024, H not a positive multiple of 256 up to 4096,
 * or T < 0 (T = 0 is a no-op).
 *
 * T <= 8: an f32 GEMV launch, then the top-k launch (a layer's own router
 * fuses the two: its last workgroup runs the top-k).
 * T > 8: the logits come from bf16 MFMA on Wr split exactly into three bf16
 * planes (hi + mid + lo == Wr, so every product is exact in f32), with K cut
 * into up to 4 slices whose partial sums the top-k adds in slice order, then
 * rb; sigma is then x . wsg in f32 per token.  The planes and partial sums
 * live in stream-ordered scratch (hipMallocAsync / hipFreeAsync on `stream`).
 * ---------------------------------------------------------------------- */
int32_t moe_route_topk(const uint16_t* x, int32_t T, int32_t H, const float* Wr,
                       const float* rb, int32_t E, int32_t k, const float* wsg,
                       int32_t* idx, float* w, float* sigma, float* logits,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * Group the (token, choice) pairs of a routed batch by expert: each token
 * goes to k of E experts ([xix] how-it-works paragraph; [lens]
 * "エキスパートストリーミングの仕組み"), and the many-token path runs each
 * expert once on all of its rows, so rows are sorted by expert, keeping
 * (token, choice) order inside an expert.  This is the sort the layer's
 * many-token path runs before its grouped GEMMs.
 *
 * idx: device int32 [T, k] (a router's output); pair p = t*k + j.
 * perm: device int32 [T*k] (out): perm[r] = the pair in sorted row r.
 * offsets: device int32 [E + 1] (out): first row of expert e; offsets[E] =
 * number of pairs sorted.  Pairs whose expert lies outside [0, E) are left
 * out (perm rows from offsets[E] on are not written).  T = 0 zeroes
 * offsets.  Scratch is stream-ordered (hipMallocAsync / hipFreeAsync on
 * `stream`).  MOE_E_INVAL if k is not in [1, MOE_MAX_TOPK], E not in
 * [1, 1024], T < 0, T * (k + 1) >= 2^30, or a needed pointer is NULL.
 * ---------------------------------------------------------------------- */
int32_t moe_expert_sort(const int32_t* idx, int32_t T, int32_t k, int32_t E, int32_t* perm,
                        int32_t* offsets, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Dequantise one matrix of a device blob (test hook for the bit-exact
 * dequant check): the MLX-style affine group dequantisation the pages name
 * for the expert weights ([xix] lineage paragraph: MLX-style int4/int8
 * group quantisation; [lens] "TurboFieldfareとの関係"), W = s*q + b per
 * group of 64 inputs.  which: 0 gate, 1 up, 2 down.  out_f32: device f32
 * [out, in] with s*q + b computed in f32 (exact for the supported value
 * ranges); out_bf16: device bf16 [out, in] (round to nearest even of the
 * f32 value) or NULL.  blob: device expert blob of `shape` (read only).
 * MOE_E_INVAL on a null pointer, a bad `which` or an unsupported shape.
 * ---------------------------------------------------------------------- */
int32_t moe_dequant(const void* blob, const moe_qshape* shape, int32_t which,
                    float* out_f32, uint16_t* out_bf16, hipStream_t stream);

/* ------------------------------------------------------------------------
 * One SwiGLU expert on T tokens, accumulated -- the unit the pages' layer
 * runs for each chosen routed expert and for the shared expert, straight
 * from the quantised weights ([xix] how-it-works paragraph; [lens]
 * "エキスパートストリーミングの仕組み"):
 *   h = bf16(silu(Wg x) * (Wu x)),   y_accum[t] += coef[t] * (Wd h)
 * x: device bf16 [T, H]; blob: device expert blob (read only); coef: device
 * f32 [T]; y_accum: device f32 [T, H] (read and written).
 * 1 <= T <= MOE_MAX_DECODE_T, else MOE_E_INVAL (also for an unsupported
 * shape or a null pointer).  Uses stream-ordered scratch (hipMallocAsync /
 * hipFreeAsync on `stream`) for h, T * inter bf16 values.
 * ---------------------------------------------------------------------- */
int32_t moe_expert_forward(const uint16_t* x, int32_t T, const moe_qshape* shape,
                           const void* blob, const float* coef, float* y_accum,
                           hipStream_t stream);

/* moe_expert_forward without any allocation, for callers that cannot
 * allocate device memory: code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, kernels and results
 * (bit for bit) as moe_expert_forward; h goes to a fixed array of the
 * library of MOE_NOALLOC_MAX_H bf16 values per device (32 KiB, held until
 * the process ends) instead of stream-ordered scratch.  MOE_E_INVAL if
 * T * shape->inter > MOE_NOALLOC_MAX_H (and as moe_expert_forward
 * otherwise).  Every call on a device uses the same array: calls that
 * overlap on one device (other streams, other threads) race. */
#define MOE_NOALLOC_MAX_H (MOE_MAX_DECODE_T * 2048)
int32_t moe_expert_forward_noalloc(const uint16_t* x, int32_t T, const moe_qshape* shape,
                                   const void* blob, const float* coef, float* y_accum,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * Fixed-stride expert store in pinned host memory: L*E blobs of `stride`
 * bytes ([xix] how-it-works paragraph: fixed-stride blobs in a .qpack
 * container, one read per expert; [xix] lineage paragraph: 64-bit offsets
 * for multi-gigabyte shards).  Allocated with hipHostMalloc; MOE_E_NOMEM if
 * pinning fails.  stride must be a positive multiple of 4096.
 * ---------------------------------------------------------------------- */
typedef struct expert_store expert_store;

int32_t expert_store_create(int32_t layers, int32_t experts, int64_t stride,
                            expert_store** out);
/* Copy n <= stride bytes into blob (l, e) (host memcpy). */
int32_t expert_store_write(expert_store* store, int32_t layer, int32_t expert,
                           const void* blob, int64_t n);
/* Host address of blob (l, e). */
int32_t expert_store_host_ptr(const expert_store* store, int32_t layer,
                              int32_t expert, void** ptr);
int32_t expert_store_destroy(expert_store* store);

/* File-backed store: the container itself.  Blob (l, e) sits at byte offset
 * (int64)(l*E + e)*stride of the file at `path` (no header), and a pool miss
 * fetches it with ONE pread of `stride` bytes ([xix] how-it-works
 * paragraph: one pread per expert from a fixed-stride container).  create
 * != 0: create or truncate the file to L*E*stride bytes, writable through
 * expert_store_write (pwrite); create == 0: open an existing file of at
 * least that size, read-only.  Reads bypass the OS page cache (O_DIRECT)
 * when the file system allows it, else go through it; expert_store_kind
 * tells which.  MOE_E_IO (with the errno text in moe_last_error) if a file
 * operation fails.  The store owns its descriptors until
 * expert_store_destroy. */
int32_t expert_store_open_file(const char* path, int32_t layers, int32_t experts,
                               int64_t stride, int32_t create, expert_store** out);
/* kind (out): 0 pinned memory, 1 file read with O_DIRECT, 2 file read
 * through the OS page cache. */
int32_t expert_store_kind(const expert_store* store, int32_t* kind);
/* Copy blob (l, e) into dst (host, stride bytes) -- for a file store one
 * pread (test hook). */
int32_t expert_store_read(const expert_store* store, int32_t layer, int32_t expert,
                          void* dst);
/* File store: write back and drop the file's pages from the OS page cache,
 * so that later reads come from the device.  No-op for a memory store. */
int32_t expert_store_drop_cache(expert_store* store);

/* ------------------------------------------------------------------------
 * Bounded HBM slot pool over a store ([xix] how-it-works paragraph:
 * popular experts cached in a bounded pool with LFU plus recency eviction;
 * [lens] "エキスパートストリーミングの仕組み").
 *
 * Policy: each access advances a tick; a hit adds one to the slot's use
 * count and stamps the tick.  A miss takes the lowest-numbered free slot,
 * else evicts the unpinned resident slot with the smallest (use count, last
 * tick, layer, expert), and is filled by exactly one hipMemcpyAsync of
 * `stride` bytes from the store on the pool's own copy stream (for a file
 * store, after one pread of the blob -- with O_DIRECT into an ordinary
 * page-aligned buffer, then copied to one of 8 pinned staging buffers;
 * otherwise into the staging buffer itself; acquire blocks the calling
 * thread for that read).  That copy
 * waits for the evicted slot's last reader (write-after-read) and the
 * compute stream waits for the copy (read-after-write) -- [lens]
 * "TurboFieldfareとの関係": explicit hazard management.  The policy decides
 * hits only; results never depend on it.
 *
 * The pool also keeps a device table (layer, expert) -> slot address, NULL
 * when not resident, that the layer's router kernel reads; it is updated on
 * the copy stream after the fills of each acquire that changes it, and the
 * compute stream waits for the update, so kernels enqueued after a call see
 * the table as that call left it.  Evict and flush update it before they
 * return.
 * ---------------------------------------------------------------------- */
typedef struct slotpool slotpool;

typedef struct slotpool_counters {
  int64_t hits;
  int64_t misses;
  int64_t evictions;
  int64_t bytes_h2d;
  int64_t bytes_read;  /* file store: bytes read from the file */
  int64_t read_ns;     /* file store: host time spent in those reads */
  int64_t prefetched;  /* experts loaded by slotpool_prefetch (their copies
                          count in bytes_h2d) */
} slotpool_counters;

/* capacity: number of slots (>= 1); device: HIP device ordinal.  Allocates
 * capacity * stride bytes of device memory and a copy stream (and, over a
 * file store, 8 x stride bytes of pinned staging and one stride-sized
 * page-aligned buffer).  The store must outlive the pool. */
int32_t slotpool_create(const expert_store* store, int64_t capacity,
                        int32_t device, slotpool** out);
/* Make experts[0..n) of `layer` resident and pin them.  slot_ptrs (out, n
 * entries): device addresses of the blobs.  was_miss (out, nullable).
 * `compute` is made to wait for every copy this call enqueued.  The experts
 * must be distinct.  MOE_E_POOL_EXHAUSTED if a miss finds every slot
 * pinned (experts admitted earlier in the call stay resident, unpinned). */
int32_t slotpool_acquire(slotpool* pool, int32_t layer, const int32_t* experts,
                         int32_t n, hipStream_t compute, const void** slot_ptrs,
                         uint8_t* was_miss);
/* Unpin; records on `compute` the event a later refill of these slots
 * waits for.  Calls may use different compute streams: a release on a
 * stream other than the previous release's first makes that stream wait
 * for the previous release. */
int32_t slotpool_release(slotpool* pool, int32_t layer, const int32_t* experts,
                         int32_t n, hipStream_t compute);
/* Speculative load of experts[0..n) of `layer` ([lens] "結論" names expert
 * prefetching as open room; the rule is this library's): in list order,
 * each expert not resident is loaded into a free slot; a prefetch never
 * evicts and stops at the first expert that finds no free slot.  It is not
 * an access: no tick, hit or miss is counted; a loaded expert is unpinned,
 * with use count 0 and the current tick, so one never used afterwards is
 * the first eviction victim.  Outputs of later calls do not change, only
 * which of their accesses hit.  `compute` is made to wait for the copies
 * (as for slotpool_acquire).  loaded (out, nullable): experts loaded.
 * MOE_E_RANGE for an expert or layer outside the store. */
int32_t slotpool_prefetch(slotpool* pool, int32_t layer, const int32_t* experts,
                          int32_t n, hipStream_t compute, int32_t* loaded);
/* Drop (layer, expert) if resident.  MOE_E_BUSY if pinned. */
int32_t slotpool_evict(slotpool* pool, int32_t layer, int32_t expert);
/* Drop every resident expert (next accesses all miss); MOE_E_BUSY if any
 * slot is pinned.  Counters are kept. */
int32_t slotpool_flush(slotpool* pool);
/* The pool's counters (hits, misses, evictions, prefetched experts, bytes
 * copied and read). */
int32_t slotpool_stats(const slotpool* pool, slotpool_counters* out);
/* The same as slotpool_stats (earlier name). */
int32_t slotpool_get_stats(const slotpool* pool, slotpool_counters* out);
/* Slot index of (layer, expert), or -1 if not resident (test hook). */
int32_t slotpool_slot_of(const slotpool* pool, int32_t layer, int32_t expert,
                         int32_t* slot);
/* Synchronises the copy stream, then frees. */
int32_t slotpool_destroy(slotpool* pool);

/* ------------------------------------------------------------------------
 * MoE layer ([xix] how-it-works paragraph; [lens]
 * "エキスパートストリーミングの仕組み"): route, run the k chosen SwiGLU
 * experts from quantised weights, add the sigmoid-gated shared expert,
 * combine:  y[t] = sum_j w[t,j] * E_idx[t,j](x_t) + sigma_t * S(x_t),
 * summed in j order then the shared term, f32.  y_bf16 = RNE(y_f32).
 * ---------------------------------------------------------------------- */
typedef struct moe_layer_cfg {
  int32_t hidden;        /* H, multiple of 256, <= 2048 */
  int32_t experts;       /* E <= 1024 */
  int32_t top_k;         /* k <= MOE_MAX_TOPK */
  int32_t inter;         /* I of routed experts */
  int32_t shared_inter;  /* I of the shared expert */
  int32_t group;         /* 64 */
  int32_t bits;          /* 4 or 8 */
  int32_t layer_index;   /* l: routed blob (l, e) of resident_base / pool */
} moe_layer_cfg;

typedef struct moe_layer moe_layer;

/* Wr f32 [E,H], rb f32 [E] (nullable), wsg f32 [H], shared_blob: device
 * blob of shape (H, shared_inter).  Exactly one of resident_base (device
 * base of the L*E routed blobs, blob (l,e) at (l*E+e)*stride) and pool is
 * non-NULL.  With a pool, the pool's store must hold layer_index (< its
 * layers), exactly `experts` experts per layer and blobs of this layer's
 * stride, else MOE_E_INVAL.  Allocates the layer's device workspace. */
int32_t moe_layer_create(const moe_layer_cfg* cfg, const float* Wr,
                         const float* rb, const void* shared_blob,
                         const float* wsg, const void* resident_base,
                         slotpool* pool, moe_layer** out);

/* x: device bf16 [T, H].  y_bf16: device bf16 [T, H] (required); y_f32:
 * device f32 [T, H] or NULL; idx_out: device int32 [T, k] or NULL; w_out:
 * device f32 [T, k] or NULL.  T == 0 returns MOE_OK and touches nothing
 * (x and y_bf16 may then be NULL); 1 <= T <= MOE_MAX_DECODE_T takes the
 * per-token GEMV path; larger T takes the sorted grouped-GEMM path.  With a
 * pool (GEMV path), the router kernel looks the chosen experts up in the
 * pool's device table and the expert kernels, enqueued right behind it, run
 * only if all of them are resident; the router also publishes its expert
 * list to pinned host memory, and the calling thread waits for it, runs the
 * pool policy (slotpool_acquire / _release on the call's stream) and, after
 * a miss, enqueues the expert kernels again once the misses are filled.
 * One host round trip per call; the outputs never depend on hit or miss. */
int32_t moe_layer_forward(moe_layer* layer, const uint16_t* x, int32_t T,
                          uint16_t* y_bf16, float* y_f32, int32_t* idx_out,
                          float* w_out, hipStream_t stream);
int32_t moe_layer_destroy(moe_layer* layer);

/* ------------------------------------------------------------------------
 * Stack of MoE layers run one after another on the same tokens.  Layer
 * l > 0 takes x_l = bf16(y_{l-1} / sqrt(mean(y_{l-1}^2) + 1e-6)) (f32), a
 * weightless stand-in for the residual and norm layers between the pages'
 * MoE layers, fused into layer l's router.  All layers share H and top_k.
 *
 * One-token calls (T == 1) on a stack whose layers share one shape and are
 * either all resident or all on the same slot pool run as ONE persistent
 * kernel for the whole stack (256
 * workgroups, needing a device with at least 256 compute units; all of them
 * must be resident at once, so other work on the device during the call can
 * make it time out): the pages find their
 * decode loop bound by dispatch, not IO ([ttj] "실무자가 따져볼 지점"), and
 * this removes the launches and dependency stalls between layers.  Its
 * outputs are bit-identical to the per-layer kernels'.  Workgroups hand
 * data to each other through per-layer buffers owned by the stack, so calls
 * on one stack must not overlap (use one stream).  Every wait inside the
 * kernel is bounded (2 s); a call that ran out of time is reported as
 * MOE_E_HIP by the next moe_stack_forward on the same stack.
 *
 * On a pool the kernel reads each chosen expert's address from the pool's
 * device table and stops at the first layer with a non-resident choice
 * (all workgroups see the same top-k, so all stop there), after exporting
 * that layer's choices.  The calling thread waits for the kernel, records
 * the hits of the layers that ran (they enter the pool policy in access
 * order before any later use of the pool: every slotpool_* call, and the
 * next pooled stack call right after its launch, applies them first),
 * acquires the stopped layer's choices (filling its misses: one copy each),
 * launches the kernel again at that layer from the previous layer's output,
 * and releases the layer behind that launch.  The calling thread thus waits
 * for every persistent launch of the call (work after the last one may
 * still be queued on `stream` when it returns); the pool sees the same
 * accesses, in the same order, as per-layer calls would give, and the
 * outputs equal the resident stack's bit for bit.
 * ---------------------------------------------------------------------- */
typedef struct moe_stack moe_stack;

int32_t moe_stack_create(moe_layer* const* layers, int32_t n_layers,
                         moe_stack** out);
/* x0: device bf16 [T, H].  Optional exports (NULL to skip): x_layers bf16
 * [L, T, H] (each layer's input), y_layers f32 [L, T, H], idx [L, T, k],
 * w [L, T, k].  y_last: device bf16 [T, H] (required).  1 <= T <=
 * MOE_MAX_DECODE_T. */
int32_t moe_stack_forward(moe_stack* stack, const uint16_t* x0, int32_t T,
                          uint16_t* x_layers, float* y_layers, int32_t* idx,
                          float* w, uint16_t* y_last, hipStream_t stream);
/* enable != 0 (the default): T == 1 calls take the persistent kernel when
 * the stack qualifies; 0: always the per-layer kernels (for comparisons).
 *
 * A call that runs out of time writes NaN to the rows of y_last (and of
 * y_layers from the layer that failed on) that the stalled workgroups own,
 * so its outputs never look valid; the error is returned by that call
 * (pooled stacks, which wait for the kernel) or by the next call on the
 * stack (resident stacks, which do not). */
int32_t moe_stack_set_persistent(moe_stack* stack, int32_t enable);
/* *active = 1 if the next T == 1 call runs the persistent kernel. */
int32_t moe_stack_persistent_active(const moe_stack* stack, int32_t* active);
/* Test hooks of the persistent path.  moe_stack_epoch: launches of the
 * persistent kernel so far (each tags its hand-off words with it).
 * moe_stack_advance_epoch: synchronises the device and advances the
 * launch count by n, as n launches that wrote nothing would; the host keeps
 * every hand-off word that could carry a later launch's tag out of reach,
 * whatever the count.  moe_stack_set_timeout: the bound on a workgroup's
 * waits (default 2 s); 0 makes every wait that is not already satisfied
 * time out at once.  MOE_E_INVAL if the stack has no persistent path. */
int32_t moe_stack_epoch(const moe_stack* stack, uint32_t* epoch);
int32_t moe_stack_advance_epoch(moe_stack* stack, uint32_t n);
int32_t moe_stack_set_timeout(moe_stack* stack, int64_t microseconds);
/* Profiling hook of a library built with -DMOE_STACK_PHASES (the
 * libmoe_phases.so variant; MOE_E_INVAL otherwise): phases, device uint64
 * [L][256][20] or NULL, receives per layer and workgroup the wall-clock
 * ticks (100 MHz) at twenty points of every persistent launch: 0-9 layer
 * start, previous output received, input staged, router row published,
 * top-k done (all waves), routed gate/up done, shared h received, routed h
 * received, down rows done, output published; then single waves at points
 * of their own work: 10-11 wave 0 every logit received, top-k selected;
 * 12-14 waves 4, 1 and 0 at the barrier that ends the top-k; 15-16 wave 4
 * routed down items requested, its down items landed (8-bit shapes only);
 * 17-18 wave 0 shared h polled, routed h polled; 19 routed chunk sums done.
 * Each launch overwrites it. */
int32_t moe_stack_set_phase_log(moe_stack* stack, uint64_t* phases);
int32_t moe_stack_destroy(moe_stack* stack);

/* ------------------------------------------------------------------------
 * Profiling hook: per-launch kernel durations from HIP events.  While a
 * timer is attached (one per process), every launch of its kernel by a layer
 * or stack forward is bracketed by two events recorded on the launch's
 * stream, up to `capacity` launches.  Not thread-safe; for benchmarks.
 * ---------------------------------------------------------------------- */
enum {
  MOE_KERNEL_ROUTE = 0,
  MOE_KERNEL_GATE_UP = 1,
  MOE_KERNEL_DOWN = 2,
  MOE_KERNEL_STACK = 3 /* the persistent one-token stack kernel */
};

typedef struct moe_timer moe_timer;

int32_t moe_timer_create(int32_t kernel, int32_t capacity, moe_timer** out);
/* Attach (timer) or detach (NULL). */
int32_t moe_timer_attach(moe_timer* timer);
/* Waits for the recorded events; ms (out, capacity entries): duration of
 * each recorded launch in milliseconds; n (out): how many.  Resets the
 * count. */
int32_t moe_timer_read(moe_timer* timer, float* ms, int32_t* n);
int32_t moe_timer_destroy(moe_timer* timer);

/* ------------------------------------------------------------------------
 * Gated DeltaNet recurrent decode step.  Three of every four layers of the
 * hybrid stack are Gated DeltaNet linear attention with a fixed-size
 * recurrent state ([xix] paragraph on Metal and DeltaNet; [lens]
 * "エキスパートストリーミングの仕組み"); the pages print no recurrence, and
 * this is the published gated delta rule.  For every sequence b < B and
 * value head h < Hv, with key / query head g = h / (Hv / Hk):
 *   k^ = k / sqrt(|k|^2 + eps), q^ = q / sqrt(|q|^2 + eps),
 *   S  <- alpha (S - beta (S k^) k^T) + beta v k^T,   o = scale S q^,
 * in f32 (the new state is used for o).
 *   q, k   bf16 bits [B][Hk][dk]        v      bf16 bits [B][Hv][dv]
 *   alpha, beta  f32 [B][Hv] (decay in (0, 1], write strength in [0, 1];
 *                the model's gate activations, computed by the caller)
 *   state  f32 [B][Hv][dv][dk], read and overwritten in place
 *   out    f32 [B][Hv][dv]
 * All device pointers, caller-owned, q, k and state 16-byte aligned; work
 * is enqueued on `stream`.  (dk, dv) = (128, 128) or (64, 64).  B = 0 is a
 * no-op.  MOE_E_INVAL: bad sizes, Hv not a multiple of Hk, eps < 0, null
 * or misaligned pointers.
 * ---------------------------------------------------------------------- */
int32_t moe_gdn_step(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     const float* alpha, const float* beta, float* state, float* out,
                     int32_t B, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, float scale,
                     float eps, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Calibration hook: the ceiling of a batch-1 decode layer on this device.
 * On the persistent stack kernel's grid (256 workgroups, all resident),
 * `phases` times: read `bytes` of fresh memory (phase p reads buf + p*bytes,
 * 16-byte loads), then `handoffs` all-to-all exchanges of tagged words (the
 * stack kernel's hand-off).  buf: device memory of at least phases * bytes
 * (read only); bytes a positive multiple of 16; 0 <= handoffs <= 8.  One
 * warm-up launch, then `reps` timed ones; ms (out): mean milliseconds per
 * launch.  Synchronises `stream`.  MOE_E_INVAL on a device with fewer than
 * 256 compute units; MOE_E_HIP if a wait runs out of time (2 s).
 * ---------------------------------------------------------------------- */
int32_t moe_calibrate_stream(const void* buf, int64_t bytes, int32_t phases, int32_t handoffs,
                             int32_t reps, float* ms, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
