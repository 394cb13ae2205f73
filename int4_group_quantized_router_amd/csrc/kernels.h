// Internal launch interface between the host objects and the HIP kernels.
#pragma once

#include "common.h"

namespace moe {

constexpr int kMaxSlots = MOE_MAX_DECODE_T * MOE_MAX_TOPK;  // distinct routed experts per call
constexpr int kJmapStride = MOE_MAX_DECODE_T;              // jmap row length

// Router (GEMV + fused softmax/top-k) arguments.
struct RouteArgs {
  const uint16_t* x;      // bf16 [T,H] input, or NULL when y_prev is given
  const float* y_prev;    // f32 [T,H]: input is bf16(y_prev / rms(y_prev)), or NULL
  uint16_t* x_out;        // bf16 [T,H] copy of the input actually used (block 0), or NULL
  const float* Wr;        // f32 [E,H]
  const float* rb;        // f32 [E] or NULL
  const float* wsg;       // f32 [H] or NULL
  int T, H, E, k;
  float* logits;          // f32 [T,E]
  unsigned* counter;      // ticket for the fused top-k (0 at launch), or NULL
  int32_t* idx;           // [T,k]
  float* w;               // [T,k]
  float* sigma;           // [T]: wsg . x from the GEMV, then sigmoid of it; NULL
                          // (with wsg NULL) to skip the shared gate
  // distinct-expert list for the expert kernels (NULL to skip)
  int32_t* n_slots;       // [1]
  int32_t* slot_expert;   // [T*k]
  int8_t* jmap;           // [T*k][kJmapStride]: j of token t in slot s, or -1
  int32_t* counts;        // [E] per-expert selection counts (atomic adds), or NULL
  // host-visible copy of the distinct-expert list (pinned memory, or NULL):
  // [1] = count, [2 + s] = expert of slot s, then [0] = host_epoch, stored
  // last with system-scope release so the host may read [1..] once it sees it
  int32_t* host_list;
  int32_t host_epoch;
  // pool mode: the layer's row of the pool's device table (expert -> slot
  // address or NULL); the router then writes slot_addr[s] for every slot and
  // *go = 1 when all are resident, else 0 (also to host_list[2 + T*k]), or
  // NULL to skip
  const uint8_t* const* res_tab;
  const uint8_t** slot_addr;  // [T*k]
  int32_t* go;                // [1]
  // top-k over MFMA partial sums (launch_topk_only): logits = sum of
  // part[0..ksplit) in order + rb, written to `logits` when that is not
  // NULL; the shared gate is then sigmoid(x . wsg) computed per token here
  const float* part;      // f32 [ksplit][T][E], or NULL
  int ksplit;
};

// Kernels whose LDS (dynamic `bytes` plus up to 16 KiB static) may exceed
// 64 KiB opt in to more dynamic LDS (gfx950 has 160 KiB per workgroup).
template <typename Kernel>
inline hipError_t allow_lds(Kernel kernel, size_t bytes) {
  if (bytes + 16384 <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s);
hipError_t launch_topk_only(const RouteArgs& a, hipStream_t s);  // logits already written

// Decode (T <= 8) expert kernels.
// Pool-mode blob addresses travel in the kernel arguments when a call has
// at most this many distinct experts (one token with k <= 16), else in a
// device table.  A separate argument block, so that DecodeArgs stays small
// enough to live in registers.
constexpr int kSlotArgs = 16;
struct SlotArgs {
  const uint8_t* p[kSlotArgs];
};

struct DecodeArgs {
  const uint16_t* x;          // bf16 [T,H] layer input
  int T, H, I, Is, k, bits;
  int n_slot_max;             // routed slots in the grid (T*k, or 0)
  const uint8_t* routed_base; // device address of blob (l, 0), or NULL (pool mode)
  int64_t stride;             // routed blob stride
  QLayout lr, ls;             // routed / shared section offsets
  const uint8_t* shared_blob; // or NULL
  const int32_t* n_slots;     // device [1]
  const int32_t* slot_expert; // device [n_slot_max]
  const int8_t* jmap;         // device [n_slot_max][kJmapStride]
  const uint8_t* const* slot_ptrs;  // device [n_slot_max]: blob address per slot
                                    // when routed_base is NULL (pool mode), or
                                    // NULL: then the SlotArgs hold them
  uint16_t* h;                // bf16 [T][k+1][hI], down-kernel order
  int hI;                     // max(I, Is)
  const float* w;             // [T,k] routing weights
  const float* gate;          // [T] shared-expert scale (sigma, or coef)
  float* y_f32;               // [T,H] or NULL
  uint16_t* y_bf16;           // [T,H] or NULL
  int accumulate;             // y = y_f32_in + ... (y_f32 required)
  const int32_t* go;          // device [1]: run only if *go != 0; NULL: always run
};

hipError_t launch_gate_up(const DecodeArgs& a, hipStream_t s, const SlotArgs& sa = SlotArgs{});
hipError_t launch_down(const DecodeArgs& a, hipStream_t s, const SlotArgs& sa = SlotArgs{});
bool decode_shape_supported(int H, int I, int Is, int bits);

// Many-token (prefill) path: sort (token, choice) pairs by expert, grouped
// MFMA GEMMs with dequant-to-bf16 weight tiles, fixed-order combine.
constexpr int kPrefillBM = 96;   // rows per grouped-GEMM tile (routed experts average ~80 rows)

constexpr int kSortChunks = 64;  // chunks of (token, choice) pairs in the prefill sort

struct PrefillArgs {
  int T, H, I, Is, E, k, bits, hI;
  const uint16_t* x;            // bf16 [T, H]
  const int32_t* idx;           // [T, k]
  const float* w;               // [T, k]
  const float* sigma;           // [T]
  int32_t* hist;                // [kSortChunks][E]: per-chunk expert counts, then offsets
  int32_t* row_off;             // [E + 2]: first sorted row of each group (group E = shared)
  int32_t* n_tiles;             // [1]
  int32_t* tile_group;          // [max_tiles]
  int32_t* tile_m0;             // [max_tiles]
  int max_tiles;
  int32_t* perm_tok;            // [T*k + T]: sorted row -> token
  int32_t* inv;                 // [T*k]: (t, j) -> sorted row
  const uint8_t* routed_base;   // blob (l, 0), or NULL: then slot_ptrs[e]
  const uint8_t* const* slot_ptrs;
  int64_t stride;
  QLayout lr, ls;
  const uint8_t* shared_blob;
  uint16_t* h;                  // bf16 [rows][hI]
  float* yd;                    // f32 [rows][H]: every expert's down output
  float* y_f32;                 // [T, H] or NULL
  uint16_t* y_bf16;             // [T, H] or NULL
};

// Router for many tokens on bf16 MFMA with f32 accumulation: Wr is held as
// three bf16 planes (hi + mid + lo == Wr exactly), wr3: bf16 [3][E][H].  The
// GEMM splits K into router_splits(T, E, H) slices and writes partial sums
// part: f32 [splits][T][E]; the top-k adds them in slice order, then rb.
constexpr int kRouterMaxSplits = 4;
int router_splits(int T, int E, int H);  // 1, 2 or 4
hipError_t launch_split_router(const float* Wr, int E, int H, uint16_t* wr3, hipStream_t s);
hipError_t launch_router_gemm(const uint16_t* x, int T, int H, const uint16_t* wr3, int E,
                              float* part, hipStream_t s);
hipError_t launch_prefill_sort(const PrefillArgs& a, hipStream_t s);
// perm[row] = pair index t * k + j, for every pair whose expert is in [0, E)
// (after launch_prefill_sort, from its inverse map).
hipError_t launch_prefill_perm(const PrefillArgs& a, int32_t* perm, hipStream_t s);
hipError_t launch_prefill_gu(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_down(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_combine(const PrefillArgs& a, hipStream_t s);

// Persistent decode of a stack of layers for one token: one workgroup per
// compute unit runs every layer; workgroups hand data to each other through
// tagged words (value and call tag in one atomic store), so no grid barrier
// and no kernel boundary sits between the steps of a layer or between layers.
// Shapes are compile-time (one instance per supported model shape).
constexpr int kStackThreads = 512;
constexpr int kStackGrid = 256;       // workgroups: one per compute unit of MI355X
constexpr int kStackReplicas = 8;     // copies of every hand-off word (one per XCD)
constexpr int kStackMaxLayers = 64;   // layer descriptors kept in LDS
constexpr int kStackPhases = 20;      // phase timestamps per layer and workgroup (profiling)

struct StackLayerDesc {
  const float* Wr;              // f32 [E, H]
  const float* rb;              // f32 [E] or NULL
  const float* wsg;             // f32 [H] or NULL
  const uint8_t* shared_blob;   // shared expert
  const uint8_t* routed_base;   // device address of blob (l, 0) (resident), or NULL
  const uint8_t* const* res_row;  // pool mode: the pool's device-table row of this
                                  // layer's index (expert -> slot address or NULL)
};

struct StackArgs {
  const StackLayerDesc* layers; // device [L]
  int L, E, has_wsg;
  int64_t stride;               // routed blob stride
  uint32_t lq[3], lsb[3];       // routed blob: q / (s,b) section offsets (gate, up, down)
  uint32_t sq[3], ssb[3];       // shared blob
  const uint16_t* x0;           // bf16 [H]
  uint16_t* x_layers;           // bf16 [L][H] or NULL
  float* y_layers;              // f32 [L][H] or NULL
  int32_t* idx;                 // [L][k] or NULL
  float* w;                     // [L][k] or NULL
  uint16_t* y_last;             // bf16 [H]
  // hand-off words, per layer and replica (value | tag)
  uint64_t* ybuf;               // [L][replica][H]: f32 bits | tag << 32
  uint64_t* lbuf;               // [L][replica][E + 1]
  uint32_t* hbuf;               // [L][replica][k * I + Is]: slot j < k at j * I, shared at
                                // k * I; bf16 << 16 | 16-bit tag
  uint32_t* epochs;             // [grid]: calls completed, one counter per workgroup
  int32_t* err;                 // host-visible word set on a wait timeout
  int64_t timeout_ticks;        // wall-clock ticks a workgroup may wait in total
  // pool mode (pool != 0): each layer's row of the pool's device table
  // (StackLayerDesc::res_row, expert -> slot address, NULL: not resident)
  // replaces routed_base; every workgroup runs the same top-k, so all stop
  // together at the first layer with a non-resident choice, and workgroup 0
  // writes that layer to *stop (left alone when all ran)
  int pool;
  int32_t* stop;
  // first layer to run (0: input x0), and for l0 > 0 the previous layer's
  // f32 output, from which layer l0's input is formed as usual
  int l0;
  const float* y_start;
  // profiling builds (MOE_STACK_PHASES): [L][grid][kStackPhases] wall-clock
  // timestamps, or NULL
  uint64_t* phases;
};

// True if the persistent kernel has an instance for this shape on a device
// with `cus` compute units (else the per-layer kernels run).
bool stack_decode_supported(int H, int E, int k, int I, int Is, int bits, int cus);
hipError_t launch_stack_decode(const StackArgs& a, int H, int k, int I, int Is, int bits,
                               hipStream_t s);
// Calibration: phases x (stream `bytes` of buf, then `handoffs` all-to-all
// tagged exchanges) on the stack kernel's grid.  words: [phases][handoffs]
// [replicas][grid] u64; epochs: [grid] call counters; sink: [grid][threads].
hipError_t launch_stream_phases(const void* buf, int64_t bytes, int phases, int handoffs,
                                uint64_t* words, uint32_t* epochs, float* sink, int32_t* err,
                                int64_t timeout_ticks, hipStream_t s);

// Zero `bytes` (a multiple of 4) of device memory with a kernel (usable
// where a memset node would not be, e.g. under stream capture).
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

hipError_t launch_dequant(const uint8_t* blob, const QLayout& lay, int rows, int cols,
                          int bits, int which, float* out_f32, uint16_t* out_bf16,
                          hipStream_t s);

}  // namespace moe
