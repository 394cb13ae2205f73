"""Shared helpers for the GPU parity tests: put a synthetic config on the
device through the C ABI, and compare GPU results with the CPU oracle."""

from __future__ import annotations

import numpy as np

from moe_inputs import expert_arrays, router_arrays, shared_arrays
from oracle import moe_oracle as O

# Relative error bar on the layer's f32 output: max-norm error over the
# max-norm of the oracle's output, per token.
REL_TOL = 2e-3
U32 = 2.0 ** -24


def dims_of(cfg) -> dict:
    return {"hidden": cfg.hidden, "experts": cfg.experts, "top_k": cfg.top_k,
            "inter": cfg.inter, "shared_inter": cfg.shared_inter, "bits": cfg.bits,
            "group": cfg.group}


class DeviceModel:
    """Routers, shared experts and (resident) routed experts of a config on the GPU."""

    def __init__(self, cfg, layers=None, resident=True, device="cuda", threads=None):
        import torch
        import int4_group_quantized_router_amd as m
        from int4_group_quantized_router_amd import weights as W
        self.cfg = cfg
        self.L = cfg.layers if layers is None else layers
        self.device = device
        self.Wr, self.rb, self.wsg, self.shared = [], [], [], []
        for l in range(self.L):
            Wr, rb, wsg = router_arrays(cfg, l)
            self.Wr.append(torch.from_numpy(Wr).to(device))
            self.rb.append(torch.from_numpy(rb).to(device))
            self.wsg.append(torch.from_numpy(wsg).to(device))
            self.shared.append(W.upload_blob(cfg.hidden, cfg.shared_inter, cfg.bits,
                                             shared_arrays(cfg, l), device))
        self.routed = None
        self.stride = m.moe_blob_layout_get(cfg.hidden, cfg.inter, cfg.bits)["stride"]
        if resident:
            self.routed, _ = W.upload_resident(dims_of(cfg), self.L,
                                               lambda l, e: expert_arrays(cfg, l, e),
                                               device, threads)
        self.layers = []

    def make_layers(self, pool=None):
        import int4_group_quantized_router_amd as m
        out = []
        for l in range(self.L):
            d = dims_of(self.cfg)
            d["layer_index"] = l
            out.append(m.moe_layer_create(d, self.Wr[l], self.rb[l], self.shared[l], self.wsg[l],
                                          resident_base=None if pool else self.routed,
                                          pool=pool))
        self.layers.append(out)
        return out

    def destroy(self):
        import int4_group_quantized_router_amd as m
        for group in self.layers:
            for h in group:
                m.moe_layer_destroy(h)
        self.layers = []


# ----------------------------------------------------------------- oracle

def oracle_layer(cfg, layer: int, x_bits, bf16_weights=False):
    Wr, rb, wsg = router_arrays(cfg, layer)
    return O.moe_layer(x_bits, Wr, rb, wsg, shared_arrays(cfg, layer),
                       lambda e: expert_arrays(cfg, layer, e), cfg.top_k, cfg.bits,
                       cfg.group, bf16_weights)


def oracle_tokens(cfg, layer: int, X_bits, bf16_weights=False):
    import os
    Wr, rb, wsg = router_arrays(cfg, layer)
    return O.moe_layer_tokens(X_bits, Wr, rb, wsg, shared_arrays(cfg, layer),
                              lambda e: expert_arrays(cfg, layer, e), cfg.top_k, cfg.bits,
                              cfg.group, bf16_weights, workers=min(16, os.cpu_count() or 1))


# ------------------------------------------------------------- comparisons

def rel_err(y_gpu, y_ref) -> float:
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    den = np.max(np.abs(y_ref))
    return float(np.max(np.abs(y_gpu - y_ref)) / (den if den > 0 else 1.0))


def gemv_depth(H):
    """Summation depth of the per-token router: 4 products per lane per
    256-column step (H/256 steps at most), a 6-level butterfly, the two
    half-rows and the bias."""
    return 4 * (H // 256) + 10


def mfma_depth(H):
    """Summation depth of the many-token router: per 64-wide K group, 3 bf16
    planes x 4 MFMA steps of 16 products each (192 additions, counted as if
    sequential), then one addition per group into the total, then the bias."""
    return 3 * 64 + H // 64 + 2


def logit_bounds(x, Wr, rb, depth=None):
    """Per-expert bound on |f32 logit - exact logit|: gamma_D * (sum_h |x_h
    Wr[e,h]| + |rb_e|), the classic bound for a sum evaluated by a tree of
    depth D (see gemv_depth / mfma_depth)."""
    x = np.asarray(x, np.float64)
    n = depth if depth is not None else gemv_depth(x.shape[-1])
    gamma = n * U32 / (1 - n * U32)
    return gamma * (np.abs(np.asarray(Wr, np.float64)) @ np.abs(x) + np.abs(np.asarray(rb, np.float64)))


def check_routing(idx_gpu, logits_gpu, x, Wr, rb, k, w_gpu=None, depth=None):
    """Routing parity for one token.

    (i) the GPU's selection equals the oracle's selection rule applied to the
        GPU's own f32 logits -- always (when the logits are exported);
    (ii) where the exact logits' ordering of the top k+1 is decided beyond
        the f32 error bound, the GPU's indices equal the oracle's exactly.
    Returns True if (ii) applied (the token was decidable)."""
    idx_gpu = np.asarray(idx_gpu, np.int64)
    exact = O.router_logits(x, Wr, rb)
    B = logit_bounds(x, Wr, rb, depth)
    if logits_gpu is not None:
        lg = np.asarray(logits_gpu, np.float64)
        assert np.array_equal(idx_gpu, O.select_topk(lg, k)), "GPU top-k differs from its logits"
        assert np.all(np.abs(lg - exact) <= B + 1e-30), "GPU logits outside the f32 error bound"
    order = O.select_topk(exact, min(k + 1, len(exact)))
    decidable = all(exact[a] - exact[b] > B[a] + B[b] for a, b in zip(order[:-1], order[1:]))
    if decidable:
        assert np.array_equal(idx_gpu, order[:k]), (idx_gpu, order[:k])
    if w_gpu is not None and logits_gpu is not None:
        p = O.softmax(lg)
        w_ref = p[idx_gpu] / p[idx_gpu].sum()
        assert np.allclose(np.asarray(w_gpu, np.float64), w_ref, rtol=2e-6, atol=1e-9)
        assert abs(float(np.sum(w_gpu)) - 1.0) <= k * 2 ** -23 + 1e-7
    return decidable


def check_bf16_of_f32(y_bf16_bits, y_f32):
    """The bf16 output is the round-to-nearest-even of the f32 output."""
    ref = O.bf16_bits(O.round_bf16(np.asarray(y_f32, np.float32).astype(np.float64)))
    assert np.array_equal(np.asarray(y_bf16_bits).view(np.uint16), ref)
