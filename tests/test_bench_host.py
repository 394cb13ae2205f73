"""Host-side checks of bench.py's bookkeeping (CPU, no GPU).

The counter traffic in a bench line is only meaningful for the launch the
counters were read on: the same kernel sources and the same workload shape.
"""

import bench
from moe_inputs import CONFIGS


def test_recorded_traffic_matches_current_sources():
    for workload, (kind, fetch, write, digest) in bench.TRAFFIC.items():
        assert kind in bench.KERNEL_SOURCES
        assert fetch > 0 and write > 0
        got = bench.counter_traffic(workload, kind)
        if digest == bench.kernel_digest(kind):
            assert got == (fetch * bench.COPY_FETCH_SCALE + write * bench.COPY_WRITE_SCALE) * 1024
        else:
            assert got is None


def test_traffic_withheld_for_other_shapes_and_kernels():
    stock = CONFIGS["decode80b_int8"]
    cut = stock.replace(layers=8)
    assert bench.counter_traffic(cut.name, "stack", stock=cut == stock) is None
    assert bench.counter_traffic("decode80b_int8", "prefill_gu") is None
    assert bench.counter_traffic("no_such_workload", "stack") is None


def test_bench_refuses_several_gpus():
    """The bench runs on one GPU; asked for more it says so and exits 2
    before touching a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_match_the_blob_layout():
    """The roofline's per-layer byte counts: the quantised expert bytes are
    (k + 1) whole expert blobs as the library lays them out, and the layer
    adds the f32 router rows (E x H, plus bias, the shared gate row and the
    input) and the activations; pinned to the figures the profiles quote."""
    import int4_group_quantized_router_amd as m
    want_layer = {"decode80b_int8": 41_017_344, "decode80b": 23_715_840, "decode35b": 18_074_624}
    for name, layer_bytes in want_layer.items():
        cfg = CONFIGS[name]
        ab = bench.algorithmic_bytes(cfg)
        blob = m.moe_blob_layout_get(cfg.hidden, cfg.inter, cfg.bits)["bytes"]
        assert cfg.shared_inter == cfg.inter
        assert ab["expert_quantized"] == (cfg.top_k + 1) * blob
        router = cfg.experts * cfg.hidden * 4 + cfg.experts * 4 + 2 * cfg.hidden * 4
        assert ab["route"] == router
        assert ab["layer"] - ab["expert_quantized"] - router < 64 * 1024  # activations
        assert ab["layer"] == layer_bytes


def test_prefetch_by_bias_takes_each_layers_highest_router_bias(monkeypatch):
    """The streaming bench's prefetch asks the pool, layer by layer, for the
    n experts of highest router bias, highest first, and adds up what the
    pool reports loaded."""
    import numpy as np
    import torch
    from moe_inputs import router_arrays
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    calls = []

    class Pool:
        @staticmethod
        def slotpool_prefetch(pool, layer, experts, stream=None):
            calls.append((layer, [int(e) for e in experts]))
            return len(experts) - 1

    cfg = CONFIGS["stream80b"].replace(layers=3)
    loaded, _ = bench.prefetch_by_bias(Pool, None, cfg, 5)
    assert loaded == 3 * 4
    assert [layer for layer, _ in calls] == [0, 1, 2]
    for layer, ex in calls:
        _, rb, _ = router_arrays(cfg, layer)
        assert len(set(ex)) == 5
        assert rb[ex].min() >= np.delete(rb, ex).max()
        assert list(rb[ex]) == sorted(rb[ex], reverse=True)
    assert bench.prefetch_by_bias(Pool, None, cfg, 0) == (0, 0.0)
