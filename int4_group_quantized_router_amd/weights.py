"""Placing quantised experts where the layer reads them.

* ``pack_experts``: canonical arrays -> fixed-stride host blobs (C packer).
* ``upload_resident``: every routed expert of every layer in one HBM buffer,
  blob (l, e) at byte (l*E + e)*stride.
* ``fill_store``: the same blobs in the library's pinned-host expert store,
  for the slot-pool path.
* ``fill_file_store``: the same blobs in a fixed-stride container file (blob
  (l, e) at byte (l*E + e)*stride), read back with one pread per expert.

The arrays come from caller-supplied functions, so this module knows nothing
about where weights come from.  Packing runs on a thread pool (the C packer
and NumPy release the GIL).
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import (expert_store_create, expert_store_drop_cache, expert_store_host_ptr,
               expert_store_open_file, expert_store_write, moe_blob_layout_get, moe_blob_pack)


def _threads(n):
    import os
    return max(1, min(n or 16, os.cpu_count() or 4, 16))


def pack_experts(hidden, inter, bits, expert_fn, experts, out: np.ndarray, threads=None):
    """Pack expert_fn(e) for e in ``experts`` into rows of out [len(experts), stride]."""
    def one(i_e):
        i, e = i_e
        moe_blob_pack(hidden, inter, bits, expert_fn(e), out=out[i])
    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(one, enumerate(experts)))
    return out


def upload_resident(dims: dict, layers: int, expert_fn, device="cuda", threads=None):
    """Device uint8 tensor holding all L*E routed blobs; expert_fn(l, e) -> arrays."""
    import torch
    H, E, I, bits = dims["hidden"], dims["experts"], dims["inter"], dims["bits"]
    stride = moe_blob_layout_get(H, I, bits)["stride"]
    dev = torch.empty(layers * E * stride, dtype=torch.uint8, device=device)
    host = torch.empty((E, stride), dtype=torch.uint8, pin_memory=True)
    hnp = host.numpy()
    for l in range(layers):
        pack_experts(H, I, bits, lambda e, l=l: expert_fn(l, e), range(E), hnp, threads)
        dev[l * E * stride:(l + 1) * E * stride].copy_(host.view(-1), non_blocking=False)
    return dev, stride


def upload_blob(hidden, inter, bits, arrays, device="cuda"):
    """One expert blob as a device uint8 tensor."""
    import torch
    blob = moe_blob_pack(hidden, inter, bits, arrays)
    return torch.from_numpy(blob).to(device)


def fill_store(dims: dict, layers: int, expert_fn, threads=None):
    """Pinned-host store of all L*E routed blobs; expert_fn(l, e) -> arrays."""
    H, E, I, bits = dims["hidden"], dims["experts"], dims["inter"], dims["bits"]
    stride = moe_blob_layout_get(H, I, bits)["stride"]
    store = expert_store_create(layers, E, stride)
    for l in range(layers):
        base = expert_store_host_ptr(store, l, 0)
        view = np.ctypeslib.as_array((np.ctypeslib.ctypes.c_uint8 * (E * stride)).from_address(base))
        pack_experts(H, I, bits, lambda e, l=l: expert_fn(l, e), range(E),
                     view.reshape(E, stride), threads)
    return store, stride


def fill_file_store(path, dims: dict, layers: int, expert_fn, threads=None):
    """Container file of all L*E routed blobs (created or truncated), opened as
    a file-backed store; its pages are dropped from the OS cache afterwards so
    that pool misses read the device.  expert_fn(l, e) -> arrays."""
    H, E, I, bits = dims["hidden"], dims["experts"], dims["inter"], dims["bits"]
    stride = moe_blob_layout_get(H, I, bits)["stride"]
    store = expert_store_open_file(path, layers, E, stride, create=True)
    host = np.empty((E, stride), dtype=np.uint8)
    for l in range(layers):
        pack_experts(H, I, bits, lambda e, l=l: expert_fn(l, e), range(E), host, threads)
        for e in range(E):
            expert_store_write(store, l, e, host[e])
    expert_store_drop_cache(store)
    return store, stride
