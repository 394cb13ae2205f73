"""CPU tests of the C ABI: the library loads and exports every declared
symbol, the blob format matches the canonical arrays byte for byte, and
argument errors are reported without touching a GPU."""

import os
import re

import numpy as np
import pytest

from moe_inputs import CONFIGS, expert_arrays
from oracle import moe_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _lib_or_skip():
    from int4_group_quantized_router_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmoe.so is not built: run __graft_entry__.build()")
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("moe_route_topk", "moe_expert_forward", "slotpool_acquire", "slotpool_evict",
                 "moe_layer_forward", "moe_dequant", "expert_store_create", "moe_last_error"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = _lib_or_skip()
    from int4_group_quantized_router_amd import _lib
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"{name} has no ctypes declaration"


def test_blob_layout_numbers():
    import int4_group_quantized_router_amd as m
    lay = m.moe_blob_layout_get(2048, 512, 4)
    assert lay["q_bytes"] == [524288, 524288, 524288]
    assert lay["sb_bytes"] == [65536, 65536, 65536]
    assert lay["stride"] == 1769472 and lay["stride"] % 4096 == 0
    assert m.moe_blob_layout_get(2048, 512, 8)["stride"] == 3342336
    for off in lay["q_off"] + lay["sb_off"]:
        assert off % 256 == 0


@pytest.mark.parametrize("name", ["tiny", "decode80b_int8"])
def test_blob_bytes_match_canonical_arrays(name):
    """Byte-level container check: every section of a packed blob holds the
    canonical arrays (words as-is; scale/bias interleaved per group), the
    oracle's dequantisation read from the blob equals the one from the arrays,
    and the padding is zero."""
    import int4_group_quantized_router_amd as m
    cfg = CONFIGS[name].replace(hidden=512, inter=128)
    arr = expert_arrays(cfg, 0, 3)
    blob = m.moe_blob_pack(cfg.hidden, cfg.inter, cfg.bits, arr)
    lay = m.moe_blob_layout_get(cfg.hidden, cfg.inter, cfg.bits)
    assert blob.nbytes == lay["stride"]
    used = np.zeros(lay["stride"], bool)
    for i, mat in enumerate(("gate", "up", "down")):
        q, s, b = arr[mat]
        qo, qn = lay["q_off"][i], lay["q_bytes"][i]
        so, sn = lay["sb_off"][i], lay["sb_bytes"][i]
        qb = blob[qo:qo + qn].view(np.uint32).reshape(q.shape)
        sb = blob[so:so + sn].view(np.uint32).reshape(s.shape)
        assert np.array_equal(qb, q)
        assert np.array_equal((sb & 0xFFFF).astype(np.uint16), s)
        assert np.array_equal((sb >> 16).astype(np.uint16), b)
        W_blob = O.dequantize(qb, (sb & 0xFFFF).astype(np.uint16), (sb >> 16).astype(np.uint16),
                              cfg.bits, 64)
        assert np.array_equal(W_blob, O.dequantize(q, s, b, cfg.bits, 64))
        used[qo:qo + qn] = True
        used[so:so + sn] = True
    assert not blob[~used].any()


def test_argument_errors_without_gpu():
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import _lib
    lib = _lib_or_skip()
    # k > E, bad H, bad bits: rejected before any HIP call
    st = lib.moe_route_topk(1, 1, 256, 1, None, 4, 5, None, 1, 1, None, 1, None)
    assert st == _lib.MOE_E_INVAL and b"k must be" in lib.moe_last_error()
    st = lib.moe_route_topk(1, 1, 100, 1, None, 16, 2, None, 1, 1, None, 1, None)
    assert st == _lib.MOE_E_INVAL
    assert lib.moe_route_topk(None, 0, 256, None, None, 16, 2, None, None, None, None, None,
                              None) == _lib.MOE_OK
    with pytest.raises(m.MoEError):
        m.moe_blob_layout_get(2048, 512, 3)
    with pytest.raises(m.MoEError):
        m.moe_blob_layout_get(2048, 500, 4)
    cfg = _lib.LayerCfg(2048, 512, 17, 512, 512, 64, 4, 0)
    import ctypes as C
    out = C.c_void_p()
    st = lib.moe_layer_create(C.byref(cfg), 1, None, 1, 1, 1, None, C.byref(out))
    assert st == _lib.MOE_E_INVAL
    cfg = _lib.LayerCfg(2048, 512, 10, 512, 512, 64, 4, 0)
    st = lib.moe_layer_create(C.byref(cfg), 1, None, 1, 1, 1, 1, C.byref(out))  # both base and pool
    assert st == _lib.MOE_E_INVAL
    st = lib.expert_store_create(1, 1, 1000, C.byref(out))
    assert st == _lib.MOE_E_INVAL
    # a layer call needs a layer, even for an empty batch
    st = lib.moe_layer_forward(None, None, 0, None, None, None, None, None)
    assert st == _lib.MOE_E_INVAL and b"null" in lib.moe_last_error()
    # Gated DeltaNet step: head dims, head grouping, eps; an empty batch is a no-op
    gdn = lib.moe_gdn_step
    assert gdn(1, 1, 1, 1, 1, 1, 1, 2, 2, 4, 96, 96, 1.0, 1e-6, None) == _lib.MOE_E_INVAL
    assert gdn(1, 1, 1, 1, 1, 1, 1, 2, 3, 4, 128, 128, 1.0, 1e-6, None) == _lib.MOE_E_INVAL
    assert b"multiple" in lib.moe_last_error()
    assert gdn(1, 1, 1, 1, 1, 1, 1, 2, 2, 4, 128, 128, 1.0, -1.0, None) == _lib.MOE_E_INVAL
    assert gdn(None, 1, 1, 1, 1, 1, 1, 2, 2, 4, 64, 64, 1.0, 1e-6, None) == _lib.MOE_E_INVAL
    assert gdn(None, None, None, None, None, None, None, 0, 2, 4, 64, 64, 1.0, 1e-6,
               None) == _lib.MOE_OK
    if not os.path.exists("/dev/kfd"):
        # misaligned q / state (only where no GPU could run the launch if
        # the check were missing)
        assert gdn(8, 16, 16, 16, 16, 32, 16, 2, 2, 4, 64, 64, 1.0, 1e-6, None) == _lib.MOE_E_INVAL
        assert b"aligned" in lib.moe_last_error()
        assert gdn(16, 16, 16, 16, 16, 40, 16, 2, 2, 4, 64, 64, 1.0, 1e-6, None) == _lib.MOE_E_INVAL


def test_file_store_round_trip_without_gpu(tmp_path):
    """A file-backed store puts blob (l, e) at byte (l*E + e)*stride of the
    file and reads it back with one pread, through O_DIRECT or the OS cache;
    reopened read-only it refuses writes; a short file is refused."""
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import _lib
    _lib_or_skip()
    L, E, stride = 2, 5, 8192
    path = str(tmp_path / "experts.qpack")
    rng = np.random.default_rng(11)
    blobs = rng.integers(0, 256, size=(L, E, stride), dtype=np.uint8)
    st = m.expert_store_open_file(path, L, E, stride, create=True)
    try:
        assert m.expert_store_kind(st) in (1, 2)
        for l in range(L):
            for e in range(E):
                n = stride if (l + e) % 2 == 0 else stride - 100  # partial blobs: rest stays 0
                m.expert_store_write(st, l, e, blobs[l, e, :n])
        m.expert_store_drop_cache(st)
        for l in range(L):
            for e in range(E):
                want = blobs[l, e].copy()
                if (l + e) % 2:
                    want[stride - 100:] = 0
                assert np.array_equal(m.expert_store_read(st, l, e, stride), want)
        with pytest.raises(m.MoEError) as ei:
            m.expert_store_read(st, L, 0, stride)
        assert ei.value.status == _lib.MOE_E_RANGE
        with pytest.raises(m.MoEError):
            m.expert_store_host_ptr(st, 0, 0)
    finally:
        m.expert_store_destroy(st)
    raw = np.fromfile(path, dtype=np.uint8).reshape(L, E, stride)
    assert np.array_equal(raw[1, 3], blobs[1, 3])  # offset (1*E + 3)*stride
    ro = m.expert_store_open_file(path, L, E, stride)
    try:
        assert np.array_equal(m.expert_store_read(ro, 0, 2, stride), blobs[0, 2])
        with pytest.raises(m.MoEError) as ei:
            m.expert_store_write(ro, 0, 0, blobs[0, 0])
        assert ei.value.status == _lib.MOE_E_INVAL
    finally:
        m.expert_store_destroy(ro)
    with pytest.raises(m.MoEError) as ei:
        m.expert_store_open_file(path, L + 1, E, stride)
    assert ei.value.status == _lib.MOE_E_INVAL
    with pytest.raises(m.MoEError) as ei:
        m.expert_store_open_file(str(tmp_path / "missing" / "x.qpack"), L, E, stride)
    assert ei.value.status == _lib.MOE_E_IO
