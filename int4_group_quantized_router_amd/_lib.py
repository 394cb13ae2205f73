"""ctypes declarations of libmoe's C ABI (include/moe.h).

Loading fails loudly when ``libmoe.so`` has not been built: there is no
other implementation to fall back to.
"""

from __future__ import annotations

import ctypes as C
import os

# MOE_LIBRARY may name a profiling build of the same library (libmoe_phases.so)
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoe.so")
PHASES_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_phases.so")

MOE_OK = 0
MOE_E_INVAL = -1
MOE_E_NOMEM = -2
MOE_E_HIP = -3
MOE_E_RANGE = -4
MOE_E_POOL_EXHAUSTED = -5
MOE_E_BUSY = -6
MOE_E_IO = -7
MOE_MAX_TOPK = 16
MOE_KERNEL_ROUTE, MOE_KERNEL_GATE_UP, MOE_KERNEL_DOWN, MOE_KERNEL_STACK = 0, 1, 2, 3
MOE_MAX_DECODE_T = 8
MOE_NOALLOC_MAX_H = MOE_MAX_DECODE_T * 2048

STATUS_NAMES = {0: "MOE_OK", -1: "MOE_E_INVAL", -2: "MOE_E_NOMEM", -3: "MOE_E_HIP",
                -4: "MOE_E_RANGE", -5: "MOE_E_POOL_EXHAUSTED", -6: "MOE_E_BUSY",
                -7: "MOE_E_IO"}


class QShape(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("inter", C.c_int32),
                ("group", C.c_int32), ("bits", C.c_int32)]


class BlobLayout(C.Structure):
    _fields_ = [("q_off", C.c_int64 * 3), ("sb_off", C.c_int64 * 3),
                ("q_bytes", C.c_int64 * 3), ("sb_bytes", C.c_int64 * 3),
                ("bytes", C.c_int64), ("stride", C.c_int64)]


class QMatrixHost(C.Structure):
    _fields_ = [("q", C.c_void_p), ("s", C.c_void_p), ("b", C.c_void_p)]


class PoolStats(C.Structure):
    _fields_ = [("hits", C.c_int64), ("misses", C.c_int64),
                ("evictions", C.c_int64), ("bytes_h2d", C.c_int64),
                ("bytes_read", C.c_int64), ("read_ns", C.c_int64),
                ("prefetched", C.c_int64)]


class LayerCfg(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("hidden", "experts", "top_k", "inter",
                                         "shared_inter", "group", "bits", "layer_index")]


_P = C.c_void_p
_I32 = C.c_int32
_I64 = C.c_int64

# name -> argtypes (every function returns int32 status unless listed in _RESTYPE)
SIGNATURES = {
    "moe_last_error": [],
    "moe_blob_layout_get": [C.POINTER(QShape), C.POINTER(BlobLayout)],
    "moe_blob_pack": [C.POINTER(QShape), C.POINTER(QMatrixHost), C.POINTER(QMatrixHost),
                      C.POINTER(QMatrixHost), _P],
    "moe_route_topk": [_P, _I32, _I32, _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _P],
    "moe_expert_sort": [_P, _I32, _I32, _I32, _P, _P, _P],
    "moe_dequant": [_P, C.POINTER(QShape), _I32, _P, _P, _P],
    "moe_expert_forward": [_P, _I32, C.POINTER(QShape), _P, _P, _P, _P],
    "moe_expert_forward_noalloc": [_P, _I32, C.POINTER(QShape), _P, _P, _P, _P],
    "expert_store_create": [_I32, _I32, _I64, C.POINTER(_P)],
    "expert_store_write": [_P, _I32, _I32, _P, _I64],
    "expert_store_host_ptr": [_P, _I32, _I32, C.POINTER(_P)],
    "expert_store_destroy": [_P],
    "expert_store_open_file": [C.c_char_p, _I32, _I32, _I64, _I32, C.POINTER(_P)],
    "expert_store_kind": [_P, C.POINTER(_I32)],
    "expert_store_read": [_P, _I32, _I32, _P],
    "expert_store_drop_cache": [_P],
    "slotpool_create": [_P, _I64, _I32, C.POINTER(_P)],
    "slotpool_acquire": [_P, _I32, _P, _I32, _P, _P, _P],
    "slotpool_release": [_P, _I32, _P, _I32, _P],
    "slotpool_prefetch": [_P, _I32, _P, _I32, _P, C.POINTER(_I32)],
    "slotpool_evict": [_P, _I32, _I32],
    "slotpool_flush": [_P],
    "slotpool_stats": [_P, C.POINTER(PoolStats)],
    "slotpool_get_stats": [_P, C.POINTER(PoolStats)],
    "slotpool_slot_of": [_P, _I32, _I32, C.POINTER(_I32)],
    "slotpool_destroy": [_P],
    "moe_layer_create": [C.POINTER(LayerCfg), _P, _P, _P, _P, _P, _P, C.POINTER(_P)],
    "moe_layer_forward": [_P, _P, _I32, _P, _P, _P, _P, _P],
    "moe_layer_destroy": [_P],
    "moe_stack_create": [_P, _I32, C.POINTER(_P)],
    "moe_stack_forward": [_P, _P, _I32, _P, _P, _P, _P, _P, _P],
    "moe_stack_set_persistent": [_P, _I32],
    "moe_stack_persistent_active": [_P, C.POINTER(_I32)],
    "moe_stack_epoch": [_P, C.POINTER(C.c_uint32)],
    "moe_stack_advance_epoch": [_P, C.c_uint32],
    "moe_stack_set_timeout": [_P, _I64],
    "moe_stack_set_phase_log": [_P, _P],
    "moe_stack_destroy": [_P],
    "moe_calibrate_stream": [_P, _I64, _I32, _I32, _I32, C.POINTER(C.c_float), _P],
    "moe_gdn_step": [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, C.c_float,
                     C.c_float, _P],
    "moe_timer_create": [_I32, _I32, C.POINTER(_P)],
    "moe_timer_attach": [_P],
    "moe_timer_read": [_P, _P, C.POINTER(_I32)],
    "moe_timer_destroy": [_P],
}
_RESTYPE = {"moe_last_error": C.c_char_p}

_lib = None


def load() -> C.CDLL:
    """Load libmoe.so and declare its functions (once)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
            "(hipcc --offload-arch=gfx950); there is no fallback implementation")
    lib = C.CDLL(LIB_PATH)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = _RESTYPE.get(name, C.c_int32)
    _lib = lib
    return lib
