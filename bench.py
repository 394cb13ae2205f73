#!/usr/bin/env python3
"""Batch-1 decode benchmark of the group-quantised MoE layer stack on one GPU.

Workload (default ``decode80b_int8``): 48 stacked MoE layers shaped like the
80B-A3B model (hidden 2048, 512 experts, top-10, expert and shared
intermediate 512, affine int8 group 64, Zipf(1.1) routing bias), all experts
resident in HBM, tokens processed one at a time -- the largest batch-1 decode
configuration of the workload set.  One step = one token through all 48
layers (router + gate/up + down/combine per layer, RMS rescale between
layers).  After the timed batch-1 steps the same stack also runs 64 steps of
8 tokens (reported under ``config.batch8``, not part of ``value``).
``--workload decode35b`` runs the 35B-shaped int4 stack (40 layers, 256
experts, top-8) instead; ``stream80b`` and ``prefill80b`` have their own
modes.

One-token calls run as ONE persistent kernel per token (all layers in one
launch; ``--per-layer`` runs the three kernels per layer instead).

Prints one JSON line: tokens/s, plus
* ``roofline``: the dominant kernel -- the persistent stack kernel (or, with
  ``--per-layer``, the gate/up dequant-GEMV kernel, the largest share of the
  bytes): algorithmic bytes per launch / its mean launch time, measured with
  HIP events around every launch of it in the timed steps, against 8 TB/s;
  the same for the quantised expert bytes alone (``expert_quantized_*``);
* ``cpu_baseline``: the float64 CPU oracle on a bounded sample (one token
  through as many layers as fit the budget), converted to tokens/s.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# Measured on one MI355X with `bench.py --calibrate-peaks`: a 1 GiB device
# copy (read + write) and an 8192^3 bf16 torch.mm through the vendor BLAS.
MEASURED_COPY_GBS = 5105.0
MEASURED_BF16_MM_TFLOPS = 1213.0

# HBM counters (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) of the dominant
# kernel of a workload, from two rocprofv3 --pmc runs of this benchmark, with
# the factors that map a plain copy's counter readings onto its byte count
# (bench.py --calibrate-copy).  Each entry names the digest of the kernel
# sources it was taken on; once those sources change the reading no longer
# describes the kernel and ``traffic`` is reported as null.
COPY_FETCH_SCALE = 262144 / 131084
COPY_WRITE_SCALE = 262144 / 262144
KERNEL_SOURCES = {
    "stack": ("stack.hip", "gemv.h", "device.h", "kernels.h"),
    "prefill_gu": ("prefill.hip", "device.h", "kernels.h"),
    "gdn": ("gdn.hip", "device.h", "kernels.h", "common.h"),
}
TRAFFIC = {
    # workload: (kernel, fetch KiB, write KiB, source digest)
    # profiles/decode80b_int8_stack_decode_kernel.md
    "decode80b_int8": ("stack", 974333, 79900, "5c31e0b40da3ec54"),
    # profiles/decode80b_stack_decode_kernel.md
    "decode80b": ("stack", 568405, 79900, "5c31e0b40da3ec54"),
    # profiles/decode35b_stack_decode_kernel.md
    "decode35b": ("stack", 361725, 53786, "5c31e0b40da3ec54"),
    # profiles/prefill80b_grouped_gemm.md
    "prefill80b": ("prefill_gu", 582346, 45056, "9b1c1bde315c56d6"),
    # profiles/gdn80b_step.md
    "gdn80b": ("gdn", 66969, 132116, "51877f82619402ae"),
}
# bench.py --calibrate-stream on one MI355X: GB/s when a workload's per-layer
# algorithmic bytes are streamed once per phase with 3 dependent all-to-all
# hand-offs per phase (the stack kernel's count per layer) -- the ceiling a
# batch-1 decode layer of that size reaches on this device
# (profiles/decode_layer_ceiling.md).
CEILING_3HANDOFFS_GBPS = {"decode80b_int8": 3141.0, "decode80b": 2306.0, "decode35b": 1993.0}


def kernel_digest(kind):
    """sha256 (16 hex digits) over the sources of a kernel."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "int4_group_quantized_router_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(workload, kind, stock=True):
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per launch, or None when no
    reading was taken on the current sources, or when the workload was
    changed from its stock shape (``stock`` false: e.g. fewer layers)."""
    t = TRAFFIC.get(workload)
    if not stock or not t or t[0] != kind or t[3] != kernel_digest(kind):
        return None
    return (t[1] * COPY_FETCH_SCALE + t[2] * COPY_WRITE_SCALE) * 1024


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(cfg):
    """Bytes each kernel must move per layer for one token (T=1)."""
    H, I, Is, E, k, bits = cfg.hidden, cfg.inter, cfg.shared_inter, cfg.experts, cfg.top_k, cfg.bits
    mat = lambda out, inn: out * inn * bits // 8 + out * (inn // 64) * 4  # words + (s,b) words
    gate_up = k * 2 * mat(I, H) + 2 * mat(Is, H) + H * 2 + (k * I + Is) * 2
    down = k * mat(H, I) + mat(H, Is) + (k * I + Is) * 2 + H * 4 + H * 2
    route = E * H * 4 + E * 4 + H * 4 + H * 4
    quant = k * 3 * mat(I, H) + 3 * mat(Is, H)
    return {"route": route, "gate_up": gate_up, "down": down,
            "layer": route + gate_up + down, "expert_quantized": quant,
            "gate_up_quantized": k * 2 * mat(I, H) + 2 * mat(Is, H)}


def prefill_flops(cfg, T):
    """MFMA FLOPs of the grouped GEMMs for one T-token call (routed + shared)."""
    rows = T * cfg.top_k
    gu = 2 * (rows * 2 * cfg.inter + T * 2 * cfg.shared_inter) * cfg.hidden
    down = 2 * (rows * cfg.inter + T * cfg.shared_inter) * cfg.hidden
    return gu, down


def cpu_baseline_prefill(cfg, budget_s=20.0):
    """Oracle (per token, bf16-weight mode) on the first tokens that fit the budget."""
    import numpy as np
    from moe_inputs import expert_arrays, router_arrays, shared_arrays, token_x
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    Wr, rb, wsg = router_arrays(cfg, 0)
    sh = shared_arrays(cfg, 0)
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < budget_s and n < cfg.tokens:
        O.moe_layer(token_x(cfg, n), Wr, rb, wsg, sh, lambda e: expert_arrays(cfg, 0, e),
                    cfg.top_k, cfg.bits, bf16_weights=True)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
            "sample": f"{n} of {cfg.tokens} tokens, one at a time, in {dt:.1f} s (NumPy float64, "
                      f"bf16-weight mode; BLAS {blas} threads)"}


def _oracle_layers(cfg, budget_s):
    """Run the oracle on token 0 through the stack until the budget is spent:
    (layers done, seconds)."""
    import numpy as np
    from moe_inputs import expert_arrays, router_arrays, shared_arrays, token_x
    from oracle import moe_oracle as O
    x = token_x(cfg, 0)
    t0 = time.perf_counter()
    done = 0
    for l in range(cfg.layers):
        Wr, rb, wsg = router_arrays(cfg, l)
        out = O.moe_layer(x, Wr, rb, wsg, shared_arrays(cfg, l),
                          lambda e: expert_arrays(cfg, l, e), cfg.top_k, cfg.bits)
        x = O.rms_rescale(out["y"].astype(np.float32))
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    return done, time.perf_counter() - t0


def cpu_baseline(cfg, budget_s=20.0, one_thread_budget_s=8.0):
    """Time the oracle on token 0 through as many layers as fit the budget,
    with the host's BLAS threads, then again on one thread."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas, threadpool_limits = 1, None
    done, dt = _oracle_layers(cfg, budget_s)
    per_layer = dt / done
    res = {"value": 1.0 / (per_layer * cfg.layers), "unit": "tokens/s", "cores": int(blas),
           "kind": "oracle",
           "sample": f"token 0 through {done} of {cfg.layers} layers in {dt:.1f} s "
                     f"(NumPy float64; dequantisation single-threaded, BLAS {blas} threads); "
                     f"tokens/s = 1 / (s per layer x {cfg.layers})"}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            d1, t1 = _oracle_layers(cfg, one_thread_budget_s)
        res["one_thread"] = {"value": 1.0 / (t1 / d1 * cfg.layers), "unit": "tokens/s",
                             "sample": f"token 0 through {d1} layers in {t1:.1f} s, BLAS 1 thread"}
    return res


def calibrate_copy(nbytes):
    """A plain device copy of known size: what the HBM counters (FETCH_SIZE,
    WRITE_SIZE) read for it scales their readings of the MoE kernels."""
    import torch
    torch.cuda.set_device(0)
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 10
    print(json.dumps({"calibrate_copy_bytes": nbytes, "copies": 10,
                      "GBps_read_plus_write": 2 * nbytes / dt / 1e9}), flush=True)


def calibrate_peaks():
    """Measured ceilings on this GPU: a plain device copy (read + write GB/s)
    and a large bf16 matrix product from the vendor BLAS (TFLOP/s), the
    references the roofline fractions can also be read against."""
    import torch
    torch.cuda.set_device(0)
    n = 1 << 30
    a = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(20):
        b.copy_(a)
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 20 / (time.perf_counter() - t0) / 1e9
    del a, b
    m = 8192
    x = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    y = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        torch.mm(x, y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 20
    for _ in range(reps):
        torch.mm(x, y)
    torch.cuda.synchronize()
    tflops = 2 * m ** 3 * reps / (time.perf_counter() - t0) / 1e12
    print(json.dumps({"copy_GBps_read_plus_write": copy_gbs, "copy_bytes": n,
                      "bf16_mm_TFLOPs": tflops, "mm_shape": [m, m, m],
                      "vendor_peaks": {"hbm_GBps": HBM_PEAK_GBS, "bf16_TFLOPs": 2500.0}}),
          flush=True)


def calibrate_stream():
    """The ceiling of a batch-1 decode layer: the calibration kernel streams
    each workload's per-layer algorithmic bytes once per phase, on the stack
    kernel's grid, with 0, 1 or 3 dependent all-to-all hand-offs per phase
    (the stack kernel has 3 per layer), over as many phases as the stack has
    layers; microseconds per phase and the GB/s they give."""
    import torch
    import int4_group_quantized_router_amd as m
    from moe_inputs import CONFIGS
    torch.cuda.set_device(0)
    rows = []
    for name in ("decode80b_int8", "decode80b", "decode35b"):
        cfg = CONFIGS[name]
        nbytes = (algorithmic_bytes(cfg)["layer"] + 15) // 16 * 16
        buf = torch.empty(cfg.layers * nbytes, dtype=torch.uint8, device="cuda")
        for handoffs in (0, 1, 3):
            ms = m.moe_calibrate_stream(buf, nbytes, cfg.layers, handoffs, reps=10)
            us = ms * 1e3 / cfg.layers
            rows.append({"workload": name, "bytes_per_phase": nbytes, "phases": cfg.layers,
                         "handoffs_per_phase": handoffs, "us_per_phase": us,
                         "GBps": nbytes / us / 1e3, "frac_of_hbm_peak": nbytes / us / 1e3 / HBM_PEAK_GBS})
            log(f"[calibrate] {name}: {nbytes / 1e6:.2f} MB + {handoffs} hand-offs per phase: "
                f"{us:.2f} us ({nbytes / us / 1e3:.0f} GB/s)")
        del buf
    print(json.dumps({"calibrate_stream": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode80b_int8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--per-layer", action="store_true",
                    help="decode: three kernels per layer instead of one persistent kernel")
    ap.add_argument("--store", choices=("memory", "file"), default="memory",
                    help="stream80b: pinned-memory store, or a container file read with one "
                         "pread per miss (written to --store-path first, then dropped from the "
                         "OS cache)")
    ap.add_argument("--store-path", default=None,
                    help="file for --store file (default: $TMPDIR or /tmp, removed afterwards)")
    ap.add_argument("--pool-sweep", default=None, metavar="FRACS",
                    help="stream80b: run the same tokens at each pool size in FRACS (comma-"
                         "separated shares of the L x E experts) over one pinned store and "
                         "print tokens/s, hit rate, misses and evictions per size")
    ap.add_argument("--prefetch-bias", type=int, default=0, metavar="N",
                    help="stream80b: before the first token, prefetch each layer's N experts "
                         "of highest router bias into the empty pool (slotpool_prefetch: free "
                         "slots only, not an access)")
    ap.add_argument("--layers", type=int, default=None,
                    help="stream80b / decode80b_int8: build only this many layers")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run 10 device-to-device copies of BYTES (reference for HBM counters)")
    ap.add_argument("--calibrate-peaks", action="store_true",
                    help="only measure a 1 GiB device copy and an 8192^3 bf16 matmul")
    ap.add_argument("--calibrate-stream", action="store_true",
                    help="only measure the decode-layer ceiling: each workload's per-layer "
                         "bytes streamed per phase with 0, 1 or 3 all-to-all hand-offs")
    ap.add_argument("--phases", type=int, default=0, metavar="TOKENS",
                    help="decode: run TOKENS tokens through the profiling build "
                         "(libmoe_phases.so, built by `python -m "
                         "int4_group_quantized_router_amd._build --phases`) and print the "
                         "persistent kernel's per-phase times")
    args = ap.parse_args()
    if args.phases:  # before the package is imported: it loads the library named there
        os.environ["MOE_LIBRARY"] = os.path.join(ROOT, "int4_group_quantized_router_amd",
                                                 "libmoe_phases.so")
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy)
    if args.calibrate_peaks:
        return calibrate_peaks()
    if args.calibrate_stream:
        return calibrate_stream()
    from moe_inputs import CONFIGS, GDN_CONFIGS

    if args.workload in GDN_CONFIGS:
        return bench_gdn(args, args.workload, GDN_CONFIGS[args.workload])
    cfg = CONFIGS[args.workload]
    if args.layers:
        cfg = cfg.replace(layers=args.layers)
    if cfg.batch > 8:
        return bench_prefill(args, cfg)
    if not cfg.resident:
        if args.pool_sweep:
            return bench_pool_sweep(args, cfg, [float(f) for f in args.pool_sweep.split(",")])
        return bench_stream(args, cfg)
    if args.phases:
        return bench_phases(args, cfg)
    return bench_decode(args, cfg)


PHASE_NAMES = ["previous output received", "input staged (RMS rescale)", "router row published",
               "logits received + top-k (shared gate/up alongside)", "routed gate/up",
               "shared h received", "routed h received", "down rows", "output published"]


def bench_phases(args, cfg):
    """Per-phase times of the persistent stack kernel (profiling build): for
    every layer but the first, workgroup and token, the wall-clock time from
    one phase boundary to the next; medians and 90th percentiles."""
    import numpy as np
    import torch
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import _lib
    from moe_inputs import tokens_x
    assert _lib.LIB_PATH.endswith("libmoe_phases.so"), _lib.LIB_PATH
    torch.cuda.set_device(0)
    log(f"[phases] building {cfg.name}: {cfg.layers} layers")
    layers, stack, keep = _build_stack(cfg)
    assert m.moe_stack_persistent_active(stack)
    L, G, P = cfg.layers, 256, 20
    n = args.phases
    warm = 8
    X = torch.from_numpy(tokens_x(cfg, 0, warm + n).view(np.int16)).cuda()
    Y = torch.empty((warm + n, cfg.hidden), dtype=torch.int16, device="cuda")
    buf = torch.zeros((L, G, P), dtype=torch.int64, device="cuda")
    for i in range(warm):
        m.moe_stack_forward(stack, X[i:i + 1], y_last=Y[i:i + 1])
    m.moe_stack_set_phase_log(stack, buf)
    runs = []
    for i in range(warm, warm + n):
        buf.zero_()
        m.moe_stack_forward(stack, X[i:i + 1], y_last=Y[i:i + 1])
        torch.cuda.synchronize()
        runs.append(buf.cpu().numpy().astype(np.int64))
    m.moe_stack_set_phase_log(stack, None)
    t = np.stack(runs)[:, 1:]              # tokens, layers 1.., workgroups, phases
    split = cfg.bits == 8                  # 8-bit shapes: waves 4..7 load the down items
    need = [p for p in range(P) if split or p not in (15, 16)]
    assert np.all(t[..., need] > 0), "missing timestamps"
    us = 0.01                              # 100 MHz wall clock
    d = np.diff(t[..., :10], axis=-1) * us  # phase p-1 -> p, p = 1..9

    def since(p, q):
        return (t[..., p] - t[..., q]) * us
    # inside a phase: when single waves reach points of their own work,
    # counted from the start of that phase
    sub = {3: {"logits wait (wave 0)": since(10, 3),
               "top-k selection (wave 0)": since(11, 10),
               "wave 0 at the barrier (choices written)": since(14, 3),
               "wave 1 at the barrier (shared gate/up published)": since(13, 3),
               "wave 4 at the barrier (shared down requested)": since(12, 3)},
           5: {"wave 0 has polled the shared h": since(17, 5)},
           6: {"wave 0 has polled the routed h": since(18, 6)},
           7: {"routed chunk sums": since(19, 7), "down items": since(8, 19)}}
    if split:
        sub[5].update({"wave 4 routed down items requested": since(15, 5),
                       "wave 4 down items landed": since(16, 5)})
    period = (t[:, 1:, :, 0] - t[:, :-1, :, 0]) * us
    spread = (t[:, :, :, 9].max(axis=2) - t[:, :, :, 9].min(axis=2)) * us
    rows = []
    for p in range(9):
        v = d[..., p].ravel()
        rows.append({"phase": PHASE_NAMES[p], "median_us": float(np.median(v)),
                     "p90_us": float(np.percentile(v, 90))})
        for name, sv in sub.get(p, {}).items():
            rows.append({"phase": "  " + name, "median_us": float(np.median(sv)),
                         "p90_us": float(np.percentile(sv, 90))})
    out = {"phases": rows, "workload": cfg.name, "tokens": n,
           "layer_period_median_us": float(np.median(period)),
           "layer_period_p90_us": float(np.percentile(period, 90)),
           "output_publish_spread_median_us": float(np.median(spread))}
    for r in rows:
        log(f"[phases] {r['phase']:52s} {r['median_us']:7.2f} us (p90 {r['p90_us']:.2f})")
    log(f"[phases] layer period {out['layer_period_median_us']:.2f} us; output spread "
        f"{out['output_publish_spread_median_us']:.2f} us")
    print(json.dumps(out), flush=True)
    m.moe_stack_destroy(stack)
    for Lh in layers:
        m.moe_layer_destroy(Lh)


def bench_decode(args, cfg):
    """Resident batch-1 decode of a stack (one persistent launch per token),
    then, for the 80B-shaped int8 stack, 64 steps of 8 tokens."""
    import numpy as np
    import torch
    import int4_group_quantized_router_amd as m
    from moe_inputs import CONFIGS, tokens_x
    args.steps = 256 if args.steps is None else args.steps
    args.warmup = 16 if args.warmup is None else args.warmup
    assert cfg.batch == 1 and cfg.resident, "decode bench workload must be resident batch-1"
    torch.cuda.set_device(0)
    log(f"[bench] building {cfg.name}: {cfg.layers} layers x {cfg.experts} experts, int{cfg.bits}")
    t_build = time.perf_counter()
    layers, stack, keep = _build_stack(cfg)
    if args.per_layer:
        m.moe_stack_set_persistent(stack, False)
    persistent = m.moe_stack_persistent_active(stack)
    log(f"[bench] built in {time.perf_counter() - t_build:.1f} s; "
        f"{'persistent stack kernel' if persistent else 'per-layer kernels'}")

    n_tok = args.warmup + args.steps
    X = torch.from_numpy(tokens_x(cfg, 0, n_tok).view(np.int16)).cuda()
    Y = torch.empty((n_tok, cfg.hidden), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        m.moe_stack_forward(stack, X[i:i + 1], y_last=Y[i:i + 1], stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    kind = m._lib.MOE_KERNEL_STACK if persistent else m._lib.MOE_KERNEL_GATE_UP
    timer = m.moe_timer_create(kind, args.steps * cfg.layers)
    m.moe_timer_attach(timer)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, n_tok):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    m.moe_timer_attach(None)
    gu_ms = m.moe_timer_read(timer)
    m.moe_timer_destroy(timer)
    dn_ms = None
    if not persistent:
        # the same tokens again with the down kernel timed (the expert-kernel reading)
        timer = m.moe_timer_create(m._lib.MOE_KERNEL_DOWN, args.steps * cfg.layers)
        m.moe_timer_attach(timer)
        for i in range(args.warmup, n_tok):
            step(i)
        torch.cuda.synchronize()
        m.moe_timer_attach(None)
        dn_ms = m.moe_timer_read(timer)
        m.moe_timer_destroy(timer)

    tok_s = args.steps / elapsed
    ab = algorithmic_bytes(cfg)
    per_token_bytes = ab["layer"] * cfg.layers
    k_mean_s = float(np.mean(gu_ms)) / 1e3
    if persistent:
        k_name = (f"stack_decode_kernel (one token through all {cfg.layers} layers: router, "
                  f"top-k, dequant-GEMV gate/up + down, combine)")
        k_bytes = per_token_bytes
        k_quant = ab["expert_quantized"] * cfg.layers
        traffic = counter_traffic(cfg.name, "stack", stock=cfg == CONFIGS[cfg.name])
    else:
        k_name = "gate_up_kernel (dequant-GEMV gate+up, fused SiLU*up)"
        k_bytes = ab["gate_up"]
        k_quant = ab["gate_up_quantized"]
        traffic = None
    achieved = k_bytes / k_mean_s / 1e9
    log(f"[bench] {tok_s:.1f} tok/s, {elapsed / args.steps * 1e3:.3f} ms/token, "
        f"kernel mean {k_mean_s * 1e6:.2f} us over {len(gu_ms)} launches, "
        f"{achieved:.0f} GB/s all bytes, {k_quant / k_mean_s / 1e9:.0f} GB/s quantised expert bytes")

    batch8 = None
    if cfg.name == "decode80b_int8" and not args.per_layer:
        # the configuration's second decode shape: 8 tokens per step (the
        # per-layer kernels; each distinct expert of a layer read once)
        steps8, warm8 = 64, 4
        n8 = (warm8 + steps8) * 8
        X8 = torch.from_numpy(tokens_x(cfg, 0, n8).view(np.int16)).cuda()
        Y8 = torch.empty((n8, cfg.hidden), dtype=torch.int16, device="cuda")
        dt8 = _run_tokens(m, stack, X8, Y8, 8, warm8, steps8)
        batch8 = {"tokens_per_s": steps8 * 8 / dt8, "ms_per_step": dt8 / steps8 * 1e3,
                  "steps": steps8, "warmup": warm8, "path": "per-layer kernels (T = 8)"}
        log(f"[bench] batch 8: {batch8['tokens_per_s']:.1f} tok/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        cpu = cpu_baseline(cfg)

    out = {
        "metric": "MoE layer tokens/sec + achieved HBM GB/s (% of peak) at batch-1 decode, 1 GPU",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"int{cfg.bits} weights (affine group 64), f32 accumulate, bf16 I/O",
        "data": "synthetic (seeded; random-init weights of the stated shape)",
        "config": {
            "workload": f"{cfg.name}: {cfg.layers} stacked MoE layers, hidden {cfg.hidden}, "
                        f"{cfg.experts} experts top-{cfg.top_k}, intermediate {cfg.inter} + "
                        f"shared {cfg.shared_inter}, int{cfg.bits} group 64, Zipf(1.1) bias, "
                        f"batch 1, all experts resident",
            "launch": "one persistent kernel per token" if persistent else "3 kernels per layer",
            "batch": 1, "layers": cfg.layers, "tokens_timed": args.steps,
            "bytes_per_token": per_token_bytes,
            "quantized_expert_bytes_per_token": ab["expert_quantized"] * cfg.layers,
            "stack_GBps": per_token_bytes * tok_s / 1e9,
            "stack_frac_of_hbm_peak": per_token_bytes * tok_s / 1e9 / HBM_PEAK_GBS,
            "stack_frac_of_measured_copy": per_token_bytes * tok_s / 1e9 / MEASURED_COPY_GBS,
            "layer_tokens_per_s": tok_s * cfg.layers,
        },
        "roofline": {
            "kernel": k_name,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "bytes_per_launch": k_bytes,
            "expert_quantized_bytes_per_launch": k_quant,
            "expert_quantized_GBps": k_quant / k_mean_s / 1e9,
            "expert_quantized_frac": k_quant / k_mean_s / 1e9 / HBM_PEAK_GBS,
            "frac_of_measured_copy": achieved / MEASURED_COPY_GBS,
            "frac_of_layer_ceiling": (achieved / CEILING_3HANDOFFS_GBPS[cfg.name]
                                      if persistent and cfg.name in CEILING_3HANDOFFS_GBPS
                                      else None),
            "mean_launch_us": k_mean_s * 1e6,
            "launches": int(len(gu_ms)),
        },
        "cpu_baseline": cpu,
    }
    if batch8 is not None:
        out["config"]["batch8"] = batch8
    if dn_ms is not None:
        # quantised expert bytes over the two expert kernels' mean durations
        t_exp = (float(np.mean(gu_ms)) + float(np.mean(dn_ms))) / 1e3
        out["config"]["expert_kernels"] = {
            "gate_up_mean_us": float(np.mean(gu_ms)) * 1e3, "down_mean_us": float(np.mean(dn_ms)) * 1e3,
            "quantized_bytes_per_layer": ab["expert_quantized"],
            "GBps": ab["expert_quantized"] / t_exp / 1e9,
            "frac_of_hbm_peak": ab["expert_quantized"] / t_exp / 1e9 / HBM_PEAK_GBS}
    print(json.dumps(out), flush=True)
    m.moe_stack_destroy(stack)
    for L in layers:
        m.moe_layer_destroy(L)


def _build_stack(cfg, pool=None):
    """Layers (resident, or served by `pool`) and their stack for cfg."""
    import torch
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import weights as W
    from moe_inputs import expert_arrays, router_arrays, shared_arrays
    dims = {"hidden": cfg.hidden, "experts": cfg.experts, "top_k": cfg.top_k,
            "inter": cfg.inter, "shared_inter": cfg.shared_inter, "bits": cfg.bits}
    routed = None
    if pool is None:
        routed, _ = W.upload_resident(dims, cfg.layers, lambda l, e: expert_arrays(cfg, l, e))
    layers, keep = [], [routed]
    for l in range(cfg.layers):
        Wr, rb, wsg = (torch.from_numpy(a).cuda() for a in router_arrays(cfg, l))
        sh = W.upload_blob(cfg.hidden, cfg.shared_inter, cfg.bits, shared_arrays(cfg, l))
        keep += [Wr, rb, wsg, sh]
        layers.append(m.moe_layer_create(dict(dims, layer_index=l), Wr, rb, sh, wsg,
                                         resident_base=routed, pool=pool))
    return layers, m.moe_stack_create(layers), keep


def _run_tokens(m, stack, X, Y, T, warmup, steps, after_warmup=None):
    import torch
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        m.moe_stack_forward(stack, X[i * T:(i + 1) * T], y_last=Y[i * T:(i + 1) * T], stream=stream)
    torch.cuda.synchronize()
    if after_warmup is not None:
        after_warmup()
    t0 = time.perf_counter()
    for i in range(warmup, warmup + steps):
        m.moe_stack_forward(stack, X[i * T:(i + 1) * T], y_last=Y[i * T:(i + 1) * T], stream=stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def prefetch_by_bias(m, pool, cfg, n):
    """slotpool_prefetch of each layer's n experts of highest router bias
    (the Zipf skew of the routing lives in the bias); returns (experts
    loaded, seconds including the copies)."""
    import numpy as np
    import torch
    from moe_inputs import router_arrays
    if n <= 0:
        return 0, 0.0
    t0 = time.perf_counter()
    loaded = 0
    for l in range(cfg.layers):
        _, rb, _ = router_arrays(cfg, l)
        order = np.argsort(-rb, kind="stable")[:n]
        loaded += m.slotpool_prefetch(pool, l, order)
    torch.cuda.synchronize()
    return loaded, time.perf_counter() - t0


def bench_pool_sweep(args, cfg, fracs):
    """Batch-1 streaming decode at several pool sizes over one pinned store:
    per size a fresh (empty) pool of floor(frac * L * E) slots, the same
    warm-up and timed tokens, and its tokens/s, warm hit rate, misses,
    evictions and host-to-HBM rate.  The pages report that on their machine
    the cache size barely moves the speed (the SSD absorbs the misses); here
    a miss is a copy over the host link."""
    import numpy as np
    import torch
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import weights as W
    from moe_inputs import expert_arrays, tokens_x
    warmup = min(64, cfg.tokens) if args.warmup is None else args.warmup
    steps = cfg.tokens - warmup if args.steps is None else args.steps
    torch.cuda.set_device(0)
    dims = {"hidden": cfg.hidden, "experts": cfg.experts, "inter": cfg.inter, "bits": cfg.bits}
    log(f"[bench] filling the pinned store: {cfg.layers} layers x {cfg.experts} experts")
    store, stride = W.fill_store(dims, cfg.layers, lambda l, e: expert_arrays(cfg, l, e))
    n = warmup + steps
    X = torch.from_numpy(tokens_x(cfg, 0, n).view(np.int16)).cuda()
    Y_ref, rows = None, []
    for f in fracs:
        cap = int(f * cfg.layers * cfg.experts)
        if cap < cfg.top_k:
            raise SystemExit(f"pool share {f} gives {cap} slots, fewer than top-k {cfg.top_k}")
        pool = m.slotpool_create(store, cap, 0)
        layers, stack, keep = _build_stack(cfg, pool=pool)
        pre, _ = prefetch_by_bias(m, pool, cfg, args.prefetch_bias)
        Y = torch.empty((n, cfg.hidden), dtype=torch.int16, device="cuda")
        snap = {}
        dt = _run_tokens(m, stack, X, Y, 1, warmup, steps,
                         after_warmup=lambda: snap.update(m.slotpool_get_stats(pool)))
        s1 = m.slotpool_get_stats(pool)
        d = {k: s1[k] - snap[k] for k in s1}
        acc = d["hits"] + d["misses"]
        # every pool size must give the same outputs, bit for bit
        same = True if Y_ref is None else bool(torch.equal(Y, Y_ref))
        Y_ref = Y if Y_ref is None else Y_ref
        row = {"pool_frac": f, "slots": cap, "tokens_per_s": steps / dt,
               "ms_per_token": dt / steps * 1e3, "hit_rate": d["hits"] / max(acc, 1),
               "misses": d["misses"], "evictions": d["evictions"],
               "misses_per_token": d["misses"] / steps,
               "h2d_GBps": d["bytes_h2d"] / dt / 1e9, "prefetched": pre,
               "outputs_equal_first_size": same}
        rows.append(row)
        log(f"[bench] pool {f:.3f} ({cap} slots): {row['tokens_per_s']:.1f} tok/s, hit rate "
            f"{row['hit_rate']:.4f}, {d['misses']} misses, {d['evictions']} evictions over "
            f"{steps} tokens, {row['h2d_GBps']:.2f} GB/s host->HBM, outputs equal: {same}")
        m.moe_stack_destroy(stack)
        for L in layers:
            m.moe_layer_destroy(L)
        m.slotpool_destroy(pool)
        del keep
    m.expert_store_destroy(store)
    out = {"metric": "MoE stack tokens/sec against HBM pool size, batch-1 decode with expert "
                     "streaming, 1 GPU",
           "value": rows[-1]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": steps,
           "warmup": warmup, "ms_per_step": rows[-1]["ms_per_token"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None,
           "dtype": f"int{cfg.bits} weights, f32 accumulate, bf16 I/O",
           "data": "synthetic (seeded; random-init weights of the stated shape)",
           "config": {"workload": f"{cfg.name}: {cfg.layers} stacked MoE layers, hidden "
                                  f"{cfg.hidden}, {cfg.experts} experts top-{cfg.top_k}, "
                                  f"int{cfg.bits}; value = the last pool size"
                                  + (f"; each pool first given its {args.prefetch_bias} experts "
                                     f"per layer of highest router bias"
                                     if args.prefetch_bias else ""),
                      "sweep": rows}}
    print(json.dumps(out), flush=True)


def bench_stream(args, cfg):
    """Batch-1 decode with routed experts served from the HBM slot pool
    (floor(pool_frac * L * E) slots) filled from the pinned host store."""
    import numpy as np
    import torch
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import weights as W
    from moe_inputs import expert_arrays, tokens_x
    # default: all of the workload's tokens, the first 64 as warm-up (the pool
    # starts empty), so the timed tokens give the warm hit rate
    warmup = min(64, cfg.tokens) if args.warmup is None else args.warmup
    steps = cfg.tokens - warmup if args.steps is None else args.steps
    torch.cuda.set_device(0)
    dims = {"hidden": cfg.hidden, "experts": cfg.experts, "inter": cfg.inter, "bits": cfg.bits}
    t_b = time.perf_counter()
    path = None
    if args.store == "file":
        path = args.store_path or os.path.join(os.environ.get("TMPDIR", "/tmp"),
                                               f"moe_store_{os.getpid()}.qpack")
        log(f"[bench] writing the container file {path}: {cfg.layers} layers x {cfg.experts} experts")
        store, stride = W.fill_file_store(path, dims, cfg.layers, lambda l, e: expert_arrays(cfg, l, e))
        log(f"[bench] store: {m.STORE_KINDS[m.expert_store_kind(store)]}")
    else:
        log(f"[bench] filling the pinned store: {cfg.layers} layers x {cfg.experts} experts")
        store, stride = W.fill_store(dims, cfg.layers, lambda l, e: expert_arrays(cfg, l, e))
    cap = int(cfg.pool_frac * cfg.layers * cfg.experts)
    pool = m.slotpool_create(store, cap, 0)
    layers, stack, keep = _build_stack(cfg, pool=pool)
    log(f"[bench] built in {time.perf_counter() - t_b:.1f} s; pool {cap} slots x {stride} B")
    pre, pre_s = prefetch_by_bias(m, pool, cfg, args.prefetch_bias)
    if args.prefetch_bias:
        log(f"[bench] prefetched {pre} experts ({args.prefetch_bias} per layer of highest router "
            f"bias) in {pre_s:.2f} s")
    n = warmup + steps
    X = torch.from_numpy(tokens_x(cfg, 0, n).view(np.int16)).cuda()
    Y = torch.empty((n, cfg.hidden), dtype=torch.int16, device="cuda")
    s0 = m.slotpool_get_stats(pool)
    snap = {}
    dt = _run_tokens(m, stack, X, Y, 1, warmup, steps,
                     after_warmup=lambda: snap.update(m.slotpool_get_stats(pool)))
    s1 = m.slotpool_get_stats(pool)
    d = {k: s1[k] - snap[k] for k in s1}          # timed tokens
    d_all = {k: s1[k] - s0[k] for k in s1}        # warm-up and timed tokens
    acc, acc_all = d["hits"] + d["misses"], d_all["hits"] + d_all["misses"]
    tok_s = steps / dt
    log(f"[bench] {tok_s:.1f} tok/s; timed tokens: hits {d['hits']} misses {d['misses']} "
        f"({d['hits'] / max(acc, 1):.4f} hit rate); all {warmup + steps} tokens: "
        f"{d_all['hits'] / max(acc_all, 1):.4f} hit rate, {d_all['misses']} misses; "
        f"{d['bytes_h2d'] / dt / 1e9:.2f} GB/s host->HBM")
    if path:
        log(f"[bench] file reads: {d['bytes_read'] / 1e9:.2f} GB in {d['read_ns'] / 1e9:.3f} s "
            f"({d['read_ns'] / 1e3 / max(d['misses'], 1):.0f} us per miss)")
    # the same tokens again after a flush (every expert a miss on first use):
    # outputs must equal those of the timed run, mostly served by hits, bit for bit
    nchk = min(8, steps)
    m.slotpool_flush(pool)
    sf = m.slotpool_get_stats(pool)
    Y2 = torch.empty((nchk, cfg.hidden), dtype=torch.int16, device="cuda")
    for i in range(nchk):
        m.moe_stack_forward(stack, X[warmup + i:warmup + i + 1], y_last=Y2[i:i + 1],
                            stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    s2 = m.slotpool_get_stats(pool)
    same = bool(torch.equal(Y2, Y[warmup:warmup + nchk]))
    log(f"[bench] tokens {warmup}..{warmup + nchk - 1} rerun from a flushed pool "
        f"({s2['misses'] - sf['misses']} misses): outputs bitwise equal: {same}")
    out = {"metric": "MoE stack tokens/sec, batch-1 decode with expert streaming (30% HBM pool), 1 GPU",
           "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
           "ms_per_step": dt / steps * 1e3, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": f"int{cfg.bits} weights, f32 accumulate, bf16 I/O",
           "data": "synthetic (seeded; random-init weights of the stated shape)",
           "config": {"workload": f"{cfg.name}: {cfg.layers} stacked MoE layers, hidden {cfg.hidden}, "
                                  f"{cfg.experts} experts top-{cfg.top_k}, int{cfg.bits}, slot pool "
                                  f"{cap} = floor({cfg.pool_frac} x L x E), pool starts empty",
                      "tokens": warmup + steps, "warmup_tokens": warmup,
                      "pool_hits": d["hits"], "pool_misses": d["misses"],
                      "pool_evictions": d["evictions"], "hit_rate": d["hits"] / max(acc, 1),
                      "hit_rate_all_tokens": d_all["hits"] / max(acc_all, 1),
                      "misses_all_tokens": d_all["misses"],
                      "evictions_all_tokens": d_all["evictions"],
                      "bytes_h2d": d["bytes_h2d"], "h2d_GBps": d["bytes_h2d"] / dt / 1e9,
                      "flushed_rerun_tokens": nchk,
                      "flushed_rerun_misses": s2["misses"] - sf["misses"],
                      "flushed_rerun_bitwise_equal": same}}
    if args.prefetch_bias:
        out["metric"] = out["metric"].replace("(30% HBM pool)",
                                              "(30% HBM pool, prefetched by router bias)")
        out["config"]["workload"] = out["config"]["workload"].replace(
            "pool starts empty", f"pool starts with each layer's {args.prefetch_bias} experts "
                                 "of highest router bias, prefetched")
        out["config"]["prefetched"] = pre
        out["config"]["prefetch_s"] = pre_s
    if path:
        out["metric"] = out["metric"].replace("expert streaming", "expert streaming from a file")
        out["config"]["store"] = m.STORE_KINDS[m.expert_store_kind(store)]
        out["config"]["file_read_s"] = d["read_ns"] / 1e9
        out["config"]["file_read_us_per_miss"] = d["read_ns"] / 1e3 / max(d["misses"], 1)
        out["config"]["file_read_GBps"] = d["bytes_read"] / max(d["read_ns"], 1)
    print(json.dumps(out), flush=True)
    m.moe_stack_destroy(stack)
    for L in layers:
        m.moe_layer_destroy(L)
    m.slotpool_destroy(pool)
    m.expert_store_destroy(store)
    if path and not args.store_path:
        os.remove(path)


def bench_prefill(args, cfg):
    """One step = one MoE layer call on all cfg.tokens tokens (the prefill path)."""
    import numpy as np
    import torch
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import weights as W
    from moe_inputs import CONFIGS, expert_arrays, router_arrays, shared_arrays, tokens_x

    steps = 20 if args.steps is None else args.steps
    warmup = 3 if args.warmup is None else args.warmup
    torch.cuda.set_device(0)
    dims = {"hidden": cfg.hidden, "experts": cfg.experts, "top_k": cfg.top_k,
            "inter": cfg.inter, "shared_inter": cfg.shared_inter, "bits": cfg.bits}
    log(f"[bench] building {cfg.name}")
    routed, _ = W.upload_resident(dims, 1, lambda l, e: expert_arrays(cfg, l, e))
    Wr, rb, wsg = (torch.from_numpy(a).cuda() for a in router_arrays(cfg, 0))
    sh = W.upload_blob(cfg.hidden, cfg.shared_inter, cfg.bits, shared_arrays(cfg, 0))
    layer = m.moe_layer_create(dict(dims, layer_index=0), Wr, rb, sh, wsg, resident_base=routed)
    T = cfg.tokens
    X = torch.from_numpy(tokens_x(cfg, 0, T).view(np.int16)).cuda()
    Y = torch.empty((T, cfg.hidden), dtype=torch.int16, device="cuda")
    for _ in range(warmup):
        m.moe_layer_forward(layer, X, Y)
    torch.cuda.synchronize()
    timers = {k: m.moe_timer_create(k, steps) for k in (0, 1, 2)}
    ms = {}
    t_all = 0.0
    # one timer can be attached at a time: three passes over the same steps
    for kind, name in ((1, "gate_up"), (2, "down"), (0, "route")):
        m.moe_timer_attach(timers[kind])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            m.moe_layer_forward(layer, X, Y)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        m.moe_timer_attach(None)
        ms[name] = float(np.mean(m.moe_timer_read(timers[kind])))
        if kind == 1:
            t_all = dt
    for t in timers.values():
        m.moe_timer_destroy(t)
    gu_flops, dn_flops = prefill_flops(cfg, T)
    traffic = (counter_traffic(cfg.name, "prefill_gu", stock=cfg == CONFIGS[cfg.name])
               if T == cfg.tokens else None)
    achieved = gu_flops / (ms["gate_up"] / 1e3) / 1e12
    both = (gu_flops + dn_flops) / ((ms["gate_up"] + ms["down"]) / 1e3) / 1e12
    tok_s = T * steps / t_all
    log(f"[bench] prefill {tok_s:.0f} tok/s, {t_all / steps * 1e3:.3f} ms/call; gate_up "
        f"{ms['gate_up'] * 1e3:.1f} us, down {ms['down'] * 1e3:.1f} us, router {ms['route'] * 1e3:.1f} us")
    cpu = None if args.no_cpu_baseline else cpu_baseline_prefill(cfg)
    out = {
        "metric": "MoE layer tokens/sec, prefill (4096 tokens), 1 GPU",
        "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": t_all / steps * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"int{cfg.bits} weights dequantised to bf16, bf16 MFMA, f32 accumulate",
        "data": "synthetic (seeded; random-init weights of the stated shape)",
        "config": {"workload": f"{cfg.name}: one MoE layer, {T} tokens, hidden {cfg.hidden}, "
                               f"{cfg.experts} experts top-{cfg.top_k}, intermediate "
                               f"{cfg.inter} + shared {cfg.shared_inter}, int{cfg.bits}",
                   "gemm_flops_per_call": gu_flops + dn_flops,
                   "gate_up_plus_down_TFLOPs": both,
                   "gate_up_plus_down_frac_of_bf16_peak": both / 2500.0,
                   "gate_up_plus_down_frac_of_measured_bf16_mm": both / MEASURED_BF16_MM_TFLOPS,
                   "down_mean_us": ms["down"] * 1e3, "router_mean_us": ms["route"] * 1e3},
        "roofline": {"kernel": "grouped_gemm_kernel<4, true, true> (grouped gate/up GEMM, "
                               "dequant-to-bf16, MFMA)",
                     "bound": "mfma", "achieved": achieved, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": achieved / 2500.0, "traffic": traffic,
                     "flops_per_launch": gu_flops, "mean_launch_us": ms["gate_up"] * 1e3},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    m.moe_layer_destroy(layer)




def gdn_bytes(c):
    """Algorithmic bytes of one Gated DeltaNet step: the f32 state read and
    written, the bf16 q, k, v, f32 alpha and beta read, the f32 output."""
    B, Hk, Hv, dk, dv = c["B"], c["Hk"], c["Hv"], c["dk"], c["dv"]
    return B * (Hv * dv * dk * 4 * 2 + 2 * Hk * dk * 2 + Hv * dv * 2 + Hv * 8 + Hv * dv * 4)


def bench_gdn(args, name, c):
    """One step = one Gated DeltaNet recurrent decode step of one layer for
    c["B"] sequences (every value head's state read and written once);
    value = sequence-tokens per second through the layer."""
    import numpy as np
    import torch
    import int4_group_quantized_router_amd as m
    from moe_inputs import gdn_inputs

    steps = 200 if args.steps is None else args.steps
    warmup = 10 if args.warmup is None else args.warmup
    torch.cuda.set_device(0)
    B, Hk, Hv, dk, dv = c["B"], c["Hk"], c["Hv"], c["dk"], c["dv"]
    n_in = 8  # distinct token inputs, cycled
    d = gdn_inputs(0, B, Hk, Hv, dk, dv, n_in)
    dev = {x: torch.from_numpy(d[x].view(np.int16) if d[x].dtype == np.uint16 else d[x]).cuda()
           for x in ("q", "k", "v", "alpha", "beta")}
    S = torch.from_numpy(d["S0"]).cuda()
    out = torch.empty((B, Hv, dv), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        j = i % n_in
        m.moe_gdn_step(dev["q"][j], dev["k"][j], dev["v"][j], dev["alpha"][j], dev["beta"][j], S,
                       out=out, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    launch_us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    nbytes = gdn_bytes(c)
    state_bytes = B * Hv * dv * dk * 8
    achieved = nbytes / (launch_us * 1e-6) / 1e9
    log(f"[bench] {name}: {steps} steps of B={B}, {launch_us:.2f} us per step "
        f"({achieved:.0f} GB/s)")
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import gdn_oracle as G
        t1 = time.perf_counter()
        n = 0
        Sc = d["S0"].astype(np.float64)
        while n == 0 or time.perf_counter() - t1 < 10.0:
            j = n % n_in
            Sc, _ = G.gdn_step_bf16(Sc, d["q"][j], d["k"][j], d["v"][j], d["alpha"][j],
                                    d["beta"][j], dk ** -0.5, 1e-6)
            n += 1
        sec = (time.perf_counter() - t1) / n
        cpu = {"value": B / sec, "unit": "sequence-tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} steps of B={B} in {sec * n:.1f} s (NumPy float64, per-head loop)"}
    line = {
        "metric": "Gated DeltaNet decode step: sequence-tokens/s through one layer + state GB/s "
                  "(% of HBM peak), 1 GPU",
        "value": B * steps / dt, "unit": "sequence-tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": dt / steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32 state, bf16 q/k/v",
        "data": "synthetic (seeded)",
        "config": {"workload": f"{name}: one Gated DeltaNet layer's recurrent step, {B} sequences, "
                               f"{Hv} value heads over {Hk} key heads, dk = dv = {dk}",
                   "state_bytes_per_step": state_bytes},
        "roofline": {"kernel": f"gdn_step_kernel<{dk}, {dv}>", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": counter_traffic(name, "gdn"),
                     "bytes_per_launch": nbytes, "mean_launch_us": launch_us},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
