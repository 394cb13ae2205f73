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
