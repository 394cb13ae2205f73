"""Python binding of libmoe: the routed-expert MoE layer on AMD gfx950, with
experts run straight from affine group-quantised int4/int8 weights.

Every function here has the name of the C entry point it calls (see
``include/moe.h``) and only marshals arguments: tensors become device
pointers, the current torch stream becomes the ``hipStream_t``, output
tensors are allocated with torch when the caller passes none.  All compute
happens in the HIP kernels of ``libmoe.so``; importing this package does not
need a GPU, calling it does.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import _lib
from ._lib import (LayerCfg, PoolStats, QMatrixHost, QShape, BlobLayout,  # noqa: F401
                   MOE_MAX_DECODE_T, MOE_MAX_TOPK, STATUS_NAMES)


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {message}")


class Handle:
    """Opaque C object plus the Python objects it must keep alive."""

    def __init__(self, ptr: int, keep=()):
        self.ptr = int(ptr)
        self.keep = list(keep)

    def __int__(self):
        return self.ptr


def _lib_():
    return _lib.load()


def _check(status: int, where: str) -> None:
    if status != 0:
        msg = _lib_().moe_last_error()
        raise MoEError(status, where, msg.decode() if msg else "")


def _h(obj) -> int:
    return 0 if obj is None else int(obj)


def _dptr(t, dtypes=None, name="tensor"):
    """Device pointer of a contiguous torch tensor (None -> NULL)."""
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        return int(t)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _bf16_types():
    import torch
    return (torch.bfloat16, torch.int16, torch.uint16)


def _shape(hidden, inter, bits, group=64) -> QShape:
    return QShape(int(hidden), int(inter), int(group), int(bits))


# ------------------------------------------------------------------ format

def moe_blob_layout_get(hidden: int, inter: int, bits: int, group: int = 64) -> dict:
    lay = BlobLayout()
    _check(_lib_().moe_blob_layout_get(C.byref(_shape(hidden, inter, bits, group)), C.byref(lay)),
           "moe_blob_layout_get")
    return {"q_off": list(lay.q_off), "sb_off": list(lay.sb_off),
            "q_bytes": list(lay.q_bytes), "sb_bytes": list(lay.sb_bytes),
            "bytes": lay.bytes, "stride": lay.stride}


def moe_blob_pack(hidden: int, inter: int, bits: int, arrays: dict, out=None,
                  group: int = 64) -> np.ndarray:
    """Pack {'gate','up','down'} -> (q uint32, s uint16, b uint16) into one blob.

    ``out``: optional writable uint8 buffer of at least ``stride`` bytes (a
    numpy array, or an int host address); a new array is returned otherwise.
    """
    lay = moe_blob_layout_get(hidden, inter, bits, group)
    keep = []
    mats = []
    for name in ("gate", "up", "down"):
        q, s, b = (np.ascontiguousarray(arrays[name][0], dtype=np.uint32),
                   np.ascontiguousarray(arrays[name][1], dtype=np.uint16),
                   np.ascontiguousarray(arrays[name][2], dtype=np.uint16))
        keep += [q, s, b]
        mats.append(QMatrixHost(q.ctypes.data, s.ctypes.data, b.ctypes.data))
    if out is None:
        out = np.empty(lay["stride"], dtype=np.uint8)
    addr = out if isinstance(out, int) else out.ctypes.data
    if not isinstance(out, int) and out.nbytes < lay["stride"]:
        raise ValueError("out is smaller than the blob stride")
    _check(_lib_().moe_blob_pack(C.byref(_shape(hidden, inter, bits, group)), C.byref(mats[0]),
                                 C.byref(mats[1]), C.byref(mats[2]), C.c_void_p(addr)),
           "moe_blob_pack")
    return out


# ------------------------------------------------------------------ compute

def moe_route_topk(x, Wr, rb, k: int, wsg=None, with_sigma: bool = True, idx=None, w=None,
                   sigma=None, logits=None, stream=None, with_logits: bool = True) -> dict:
    """Router on x (bf16 [T,H]); returns {'idx','w','sigma','logits'} device tensors
    (``logits`` None when ``with_logits`` is false and none is given: not exported)."""
    import torch
    T, H = x.shape
    E = Wr.shape[0]
    dev = x.device
    idx = idx if idx is not None else torch.empty((T, k), dtype=torch.int32, device=dev)
    w = w if w is not None else torch.empty((T, k), dtype=torch.float32, device=dev)
    if with_sigma and wsg is not None and sigma is None:
        sigma = torch.empty((T,), dtype=torch.float32, device=dev)
    if logits is None and with_logits:
        logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    _check(_lib_().moe_route_topk(
        _dptr(x, _bf16_types(), "x"), T, H, _dptr(Wr, (torch.float32,), "Wr"),
        _dptr(rb, (torch.float32,), "rb"), E, int(k), _dptr(wsg, (torch.float32,), "wsg"),
        _dptr(idx, (torch.int32,), "idx"), _dptr(w, (torch.float32,), "w"),
        _dptr(sigma, (torch.float32,), "sigma"), _dptr(logits, (torch.float32,), "logits"),
        _stream(stream)), "moe_route_topk")
    return {"idx": idx, "w": w, "sigma": sigma, "logits": logits}


def moe_expert_sort(idx, E: int, perm=None, offsets=None, stream=None):
    """Group the (token, choice) pairs of idx (device int32 [T, k]) by expert;
    returns (perm [T*k], offsets [E+1]) device int32 tensors."""
    import torch
    T, k = idx.shape
    perm = perm if perm is not None else torch.empty(T * k, dtype=torch.int32, device=idx.device)
    offsets = offsets if offsets is not None else torch.empty(E + 1, dtype=torch.int32,
                                                               device=idx.device)
    _check(_lib_().moe_expert_sort(_dptr(idx, (torch.int32,), "idx"), T, k, int(E),
                                   _dptr(perm, (torch.int32,), "perm"),
                                   _dptr(offsets, (torch.int32,), "offsets"), _stream(stream)),
           "moe_expert_sort")
    return perm, offsets


def moe_dequant(blob, hidden: int, inter: int, bits: int, which: int, want_bf16: bool = True,
                stream=None, group: int = 64):
    """Dequantise matrix `which` (0 gate, 1 up, 2 down) of a device blob."""
    import torch
    rows, cols = (hidden, inter) if which == 2 else (inter, hidden)
    dev = blob.device if isinstance(blob, torch.Tensor) else torch.device("cuda")
    f32 = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    b16 = torch.empty((rows, cols), dtype=torch.int16, device=dev) if want_bf16 else None
    _check(_lib_().moe_dequant(_dptr(blob), C.byref(_shape(hidden, inter, bits, group)),
                               int(which), _dptr(f32), _dptr(b16), _stream(stream)),
           "moe_dequant")
    return f32, b16


def moe_expert_forward(x, hidden: int, inter: int, bits: int, blob, coef, y_accum,
                       stream=None, group: int = 64):
    """y_accum[t] += coef[t] * SwiGLU expert(x[t]); returns y_accum."""
    import torch
    _check(_lib_().moe_expert_forward(
        _dptr(x, _bf16_types(), "x"), x.shape[0], C.byref(_shape(hidden, inter, bits, group)),
        _dptr(blob), _dptr(coef, (torch.float32,), "coef"),
        _dptr(y_accum, (torch.float32,), "y_accum"), _stream(stream)), "moe_expert_forward")
    return y_accum


def moe_expert_forward_noalloc(x, hidden: int, inter: int, bits: int, blob, coef, y_accum,
                               stream=None, group: int = 64):
    """moe_expert_forward with h in the library's fixed per-device array (no
    allocation); returns y_accum."""
    import torch
    _check(_lib_().moe_expert_forward_noalloc(
        _dptr(x, _bf16_types(), "x"), x.shape[0], C.byref(_shape(hidden, inter, bits, group)),
        _dptr(blob), _dptr(coef, (torch.float32,), "coef"),
        _dptr(y_accum, (torch.float32,), "y_accum"), _stream(stream)),
        "moe_expert_forward_noalloc")
    return y_accum


# ------------------------------------------------------------ store / pool

def expert_store_create(layers: int, experts: int, stride: int) -> Handle:
    out = C.c_void_p()
    _check(_lib_().expert_store_create(layers, experts, stride, C.byref(out)),
           "expert_store_create")
    return Handle(out.value)


def expert_store_write(store, layer: int, expert: int, blob) -> None:
    blob = np.ascontiguousarray(blob)
    _check(_lib_().expert_store_write(_h(store), layer, expert, blob.ctypes.data, blob.nbytes),
           "expert_store_write")


def expert_store_host_ptr(store, layer: int, expert: int) -> int:
    out = C.c_void_p()
    _check(_lib_().expert_store_host_ptr(_h(store), layer, expert, C.byref(out)),
           "expert_store_host_ptr")
    return out.value


def expert_store_destroy(store) -> None:
    _check(_lib_().expert_store_destroy(_h(store)), "expert_store_destroy")


def expert_store_open_file(path: str, layers: int, experts: int, stride: int,
                           create: bool = False) -> Handle:
    out = C.c_void_p()
    _check(_lib_().expert_store_open_file(os.fsencode(path), layers, experts, stride,
                                          1 if create else 0, C.byref(out)),
           "expert_store_open_file")
    return Handle(out.value)


STORE_KINDS = {0: "pinned memory", 1: "file, O_DIRECT reads", 2: "file, reads through the OS cache"}


def expert_store_kind(store) -> int:
    out = C.c_int32()
    _check(_lib_().expert_store_kind(_h(store), C.byref(out)), "expert_store_kind")
    return out.value


def expert_store_read(store, layer: int, expert: int, stride: int) -> np.ndarray:
    out = np.empty(stride, dtype=np.uint8)
    _check(_lib_().expert_store_read(_h(store), layer, expert, out.ctypes.data),
           "expert_store_read")
    return out


def expert_store_drop_cache(store) -> None:
    _check(_lib_().expert_store_drop_cache(_h(store)), "expert_store_drop_cache")


def slotpool_create(store, capacity: int, device: int = 0) -> Handle:
    out = C.c_void_p()
    _check(_lib_().slotpool_create(_h(store), capacity, device, C.byref(out)), "slotpool_create")
    return Handle(out.value, keep=[store])


def slotpool_acquire(pool, layer: int, experts, stream=None):
    """Returns (device addresses, was_miss flags) for the given experts."""
    ex = np.ascontiguousarray(experts, dtype=np.int32)
    n = ex.size
    ptrs = (C.c_void_p * max(n, 1))()
    miss = np.zeros(max(n, 1), dtype=np.uint8)
    _check(_lib_().slotpool_acquire(_h(pool), layer, ex.ctypes.data, n, _stream(stream), ptrs,
                                    miss.ctypes.data), "slotpool_acquire")
    return [ptrs[i] for i in range(n)], [bool(m) for m in miss[:n]]


def slotpool_prefetch(pool, layer: int, experts, stream=None) -> int:
    """Loads the listed experts not resident into free slots (no eviction,
    not an access); returns how many were loaded."""
    ex = np.ascontiguousarray(experts, dtype=np.int32)
    loaded = C.c_int32(0)
    _check(_lib_().slotpool_prefetch(_h(pool), layer, ex.ctypes.data, ex.size, _stream(stream),
                                      C.byref(loaded)), "slotpool_prefetch")
    return loaded.value


def slotpool_release(pool, layer: int, experts, stream=None) -> None:
    ex = np.ascontiguousarray(experts, dtype=np.int32)
    _check(_lib_().slotpool_release(_h(pool), layer, ex.ctypes.data, ex.size, _stream(stream)),
           "slotpool_release")


def slotpool_evict(pool, layer: int, expert: int) -> None:
    _check(_lib_().slotpool_evict(_h(pool), layer, expert), "slotpool_evict")


def slotpool_flush(pool) -> None:
    _check(_lib_().slotpool_flush(_h(pool)), "slotpool_flush")


def slotpool_stats(pool) -> dict:
    st = PoolStats()
    _check(_lib_().slotpool_stats(_h(pool), C.byref(st)), "slotpool_stats")
    return {"hits": st.hits, "misses": st.misses, "evictions": st.evictions,
            "bytes_h2d": st.bytes_h2d, "bytes_read": st.bytes_read, "read_ns": st.read_ns,
            "prefetched": st.prefetched}


def slotpool_get_stats(pool) -> dict:
    st = PoolStats()
    _check(_lib_().slotpool_get_stats(_h(pool), C.byref(st)), "slotpool_get_stats")
    return {"hits": st.hits, "misses": st.misses, "evictions": st.evictions,
            "bytes_h2d": st.bytes_h2d, "bytes_read": st.bytes_read, "read_ns": st.read_ns,
            "prefetched": st.prefetched}


def slotpool_slot_of(pool, layer: int, expert: int) -> int:
    out = C.c_int32()
    _check(_lib_().slotpool_slot_of(_h(pool), layer, expert, C.byref(out)), "slotpool_slot_of")
    return out.value


def slotpool_destroy(pool) -> None:
    _check(_lib_().slotpool_destroy(_h(pool)), "slotpool_destroy")


# ------------------------------------------------------------- layer/stack

def moe_layer_create(cfg: dict, Wr, rb, shared_blob, wsg, resident_base=None,
                     pool=None) -> Handle:
    """cfg keys: hidden, experts, top_k, inter, shared_inter, bits, layer_index (group=64)."""
    c = LayerCfg(cfg["hidden"], cfg["experts"], cfg["top_k"], cfg["inter"],
                 cfg["shared_inter"], cfg.get("group", 64), cfg["bits"], cfg.get("layer_index", 0))
    out = C.c_void_p()
    _check(_lib_().moe_layer_create(C.byref(c), _dptr(Wr), _dptr(rb), _dptr(shared_blob),
                                    _dptr(wsg), _dptr(resident_base), _h(pool) or None,
                                    C.byref(out)), "moe_layer_create")
    return Handle(out.value, keep=[Wr, rb, shared_blob, wsg, resident_base, pool])


def moe_layer_forward(layer, x, y_bf16=None, y_f32=None, idx_out=None, w_out=None,
                      stream=None):
    import torch
    if y_bf16 is None:
        y_bf16 = torch.empty(x.shape, dtype=torch.int16, device=x.device)
    _check(_lib_().moe_layer_forward(_h(layer), _dptr(x, _bf16_types(), "x"), x.shape[0],
                                     _dptr(y_bf16, _bf16_types(), "y_bf16"),
                                     _dptr(y_f32, (torch.float32,), "y_f32"),
                                     _dptr(idx_out, (torch.int32,), "idx_out"),
                                     _dptr(w_out, (torch.float32,), "w_out"), _stream(stream)),
           "moe_layer_forward")
    return y_bf16


def moe_layer_destroy(layer) -> None:
    _check(_lib_().moe_layer_destroy(_h(layer)), "moe_layer_destroy")


def moe_stack_create(layers) -> Handle:
    arr = (C.c_void_p * len(layers))(*[_h(l) for l in layers])
    out = C.c_void_p()
    _check(_lib_().moe_stack_create(arr, len(layers), C.byref(out)), "moe_stack_create")
    return Handle(out.value, keep=list(layers))


def moe_stack_forward(stack, x0, y_last=None, x_layers=None, y_layers=None, idx=None, w=None,
                      stream=None):
    import torch
    if y_last is None:
        y_last = torch.empty(x0.shape, dtype=torch.int16, device=x0.device)
    _check(_lib_().moe_stack_forward(_h(stack), _dptr(x0, _bf16_types(), "x0"), x0.shape[0],
                                     _dptr(x_layers, _bf16_types(), "x_layers"),
                                     _dptr(y_layers, (torch.float32,), "y_layers"),
                                     _dptr(idx, (torch.int32,), "idx"),
                                     _dptr(w, (torch.float32,), "w"),
                                     _dptr(y_last, _bf16_types(), "y_last"), _stream(stream)),
           "moe_stack_forward")
    return y_last


def moe_stack_set_persistent(stack, enable: bool) -> None:
    _check(_lib_().moe_stack_set_persistent(_h(stack), 1 if enable else 0),
           "moe_stack_set_persistent")


def moe_stack_persistent_active(stack) -> bool:
    out = C.c_int32()
    _check(_lib_().moe_stack_persistent_active(_h(stack), C.byref(out)),
           "moe_stack_persistent_active")
    return bool(out.value)


def moe_stack_epoch(stack) -> int:
    out = C.c_uint32()
    _check(_lib_().moe_stack_epoch(_h(stack), C.byref(out)), "moe_stack_epoch")
    return out.value


def moe_stack_advance_epoch(stack, n: int) -> None:
    _check(_lib_().moe_stack_advance_epoch(_h(stack), int(n)), "moe_stack_advance_epoch")


def moe_stack_set_timeout(stack, microseconds: int) -> None:
    _check(_lib_().moe_stack_set_timeout(_h(stack), int(microseconds)), "moe_stack_set_timeout")


def moe_stack_set_phase_log(stack, phases) -> None:
    """Profiling builds only: phases = device int64 tensor [L, 256, 20] or None."""
    _check(_lib_().moe_stack_set_phase_log(_h(stack), _dptr(phases)), "moe_stack_set_phase_log")


def moe_stack_destroy(stack) -> None:
    _check(_lib_().moe_stack_destroy(_h(stack)), "moe_stack_destroy")


# ------------------------------------------------------------- calibration

def moe_gdn_step(q, k, v, alpha, beta, state, out=None, scale=None, eps=1e-6, stream=None):
    """One Gated DeltaNet decode step (see include/moe.h): q, k bf16 [B, Hk, dk],
    v bf16 [B, Hv, dv], alpha / beta f32 [B, Hv], state f32 [B, Hv, dv, dk]
    (updated in place); returns out f32 [B, Hv, dv].  scale defaults to
    dk ** -0.5."""
    import torch
    B, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if out is None:
        out = torch.empty((B, Hv, dv), dtype=torch.float32, device=state.device)
    scale = dk ** -0.5 if scale is None else scale
    _check(_lib_().moe_gdn_step(_dptr(q, _bf16_types(), "q"), _dptr(k, _bf16_types(), "k"),
                                _dptr(v, _bf16_types(), "v"), _dptr(alpha, (torch.float32,), "alpha"),
                                _dptr(beta, (torch.float32,), "beta"),
                                _dptr(state, (torch.float32,), "state"),
                                _dptr(out, (torch.float32,), "out"), B, Hk, Hv, dk, dv,
                                float(scale), float(eps), _stream(stream)), "moe_gdn_step")
    return out


def moe_calibrate_stream(buf, bytes_per_phase: int, phases: int, handoffs: int, reps: int = 5,
                         stream=None) -> float:
    """Mean ms per launch of the streaming calibration kernel (see moe.h)."""
    ms = C.c_float()
    _check(_lib_().moe_calibrate_stream(_dptr(buf), int(bytes_per_phase), int(phases),
                                        int(handoffs), int(reps), C.byref(ms), _stream(stream)),
           "moe_calibrate_stream")
    return ms.value


# ------------------------------------------------------------------ timing

def moe_timer_create(kernel: int, capacity: int) -> Handle:
    out = C.c_void_p()
    _check(_lib_().moe_timer_create(kernel, capacity, C.byref(out)), "moe_timer_create")
    return Handle(out.value, keep=[capacity])


def moe_timer_attach(timer) -> None:
    _check(_lib_().moe_timer_attach(_h(timer) or None), "moe_timer_attach")


def moe_timer_read(timer) -> np.ndarray:
    cap = timer.keep[0]
    ms = np.zeros(cap, dtype=np.float32)
    n = C.c_int32()
    _check(_lib_().moe_timer_read(_h(timer), ms.ctypes.data, C.byref(n)), "moe_timer_read")
    return ms[:n.value].copy()


def moe_timer_destroy(timer) -> None:
    _check(_lib_().moe_timer_destroy(_h(timer)), "moe_timer_destroy")
