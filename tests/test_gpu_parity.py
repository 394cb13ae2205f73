"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.  Dequantisation and routing decisions exact; layer
outputs within 2e-3 max-norm relative error on the f32 result; bf16 output
= round-to-nearest-even of the f32 output."""

import ctypes

import numpy as np
import pytest

from moe_inputs import (CONFIGS, GDN_CONFIGS, expert_arrays, gdn_inputs, router_arrays,
                        shared_arrays, token_x, tokens_x)
from oracle import gdn_oracle as G
from oracle import moe_oracle as O

from harness import (REL_TOL, DeviceModel, check_bf16_of_f32, check_routing, mfma_depth,
                     oracle_layer, oracle_tokens, rel_err)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _x(torch, cfg, t0, n):
    return torch.from_numpy(tokens_x(cfg, t0, n).view(np.int16)).cuda()


def _print(*a):
    print(*a, flush=True)


def _device_bytes(addr, n):
    """Copy n bytes at a raw device address to the host (HIP runtime call)."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    out = np.empty(n, np.uint8)
    assert hip.hipMemcpy(out.ctypes.data, addr, n, 2) == 0  # hipMemcpyDeviceToHost
    return out


# ------------------------------------------------------------------ dequant

@pytest.mark.parametrize("name,H,I", [("tiny", 256, 64), ("decode35b", 2048, 512),
                                      ("decode80b_int8", 2048, 512), ("decode80b_int8", 256, 128)])
def test_dequant_bit_exact(torch, name, H, I):
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd.weights import upload_blob
    cfg = CONFIGS[name].replace(hidden=H, inter=I)
    _print("dequant", name, H, I)
    arr = expert_arrays(cfg, 0, 11)
    blob = upload_blob(H, I, cfg.bits, arr)
    for which, mat in enumerate(("gate", "up", "down")):
        f32, b16 = m.moe_dequant(blob, H, I, cfg.bits, which)
        torch.cuda.synchronize()
        W = O.dequantize(*arr[mat], bits=cfg.bits, group=64)
        assert np.array_equal(f32.cpu().numpy().astype(np.float64), W)
        assert np.array_equal(b16.cpu().numpy().view(np.uint16), O.bf16_bits(O.round_bf16(W)))


@pytest.mark.parametrize("bits", [4, 8])
def test_dequant_rounding_wide_ranges(torch, bits):
    """s * q + b over scales and biases whose exponents differ by up to 30
    binades (either sign, some zero biases): the f32 result must be the exact
    value rounded once to float32 (the exact value is a float64 here: at
    most 16 + 8 significant bits over a span of under 53), the bf16 result
    that f32 value rounded to nearest even."""
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd.weights import upload_blob
    H, I = 256, 128
    _print("dequant wide ranges", bits)
    rng = np.random.default_rng(77)

    def bf16_of(x):
        return O.bf16_bits(O.round_bf16(np.asarray(x, np.float64)))

    arr = {}
    for mat, (rows, cols) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        words = rng.integers(0, 2**32, size=(rows, cols * bits // 32), dtype=np.uint64).astype(np.uint32)
        g = cols // 64
        s = np.ldexp(rng.uniform(1, 2, (rows, g)), rng.integers(-20, 11, (rows, g)))
        s *= rng.choice([-1.0, 1.0], (rows, g))
        b = s * np.ldexp(rng.uniform(1, 2, (rows, g)), rng.integers(-30, 31, (rows, g)))
        b *= rng.choice([-1.0, 1.0], (rows, g))
        b[rng.random((rows, g)) < 0.05] = 0.0
        arr[mat] = (words, bf16_of(s), bf16_of(b))
    blob = upload_blob(H, I, bits, arr)
    for which, mat in enumerate(("gate", "up", "down")):
        f32, b16 = m.moe_dequant(blob, H, I, bits, which)
        torch.cuda.synchronize()
        W = O.dequantize(*arr[mat], bits=bits, group=64)
        want32 = W.astype(np.float32)
        got32 = f32.cpu().numpy()
        assert np.array_equal(got32.view(np.uint32), want32.view(np.uint32))
        assert np.array_equal(b16.cpu().numpy().view(np.uint16),
                              O.bf16_bits(O.round_bf16(want32.astype(np.float64))))


# ------------------------------------------------------------------ router

@pytest.mark.parametrize("name,T", [("tiny", 1), ("tiny", 8), ("decode35b", 1), ("decode35b", 8),
                                    ("stream80b", 1), ("stream80b", 5), ("stream80b", 37),
                                    ("prefill80b", 300)])
def test_route_topk(torch, name, T):
    import int4_group_quantized_router_amd as m
    cfg = CONFIGS[name]
    _print("route", name, T)
    decided = 0
    for layer in (0, 1):
        Wr, rb, wsg = router_arrays(cfg, layer)
        xb = tokens_x(cfg, 100 * layer, T)
        out = m.moe_route_topk(torch.from_numpy(xb.view(np.int16)).cuda(),
                               torch.from_numpy(Wr).cuda(), torch.from_numpy(rb).cuda(),
                               cfg.top_k, wsg=torch.from_numpy(wsg).cuda())
        torch.cuda.synchronize()
        idx, w = out["idx"].cpu().numpy(), out["w"].cpu().numpy()
        lg, sg = out["logits"].cpu().numpy(), out["sigma"].cpu().numpy()
        depth = mfma_depth(cfg.hidden) if T > 8 else None
        for t in range(T):
            x = O.bf16_to_f64(xb[t])
            decided += check_routing(idx[t], lg[t], x, Wr, rb, cfg.top_k, w[t], depth=depth)
            s_ref = O.sigmoid(np.dot(wsg.astype(np.float64), x))
            assert abs(sg[t] - s_ref) <= 1e-6
    assert decided >= 0.9 * 2 * T


@pytest.mark.parametrize("T", [1, 8, 300])
def test_route_max_sizes(torch, T):
    """The router at its largest supported shape: E = 1024, k = 16, H = 4096
    (GEMV path for T <= 8; MFMA path with split K above)."""
    import int4_group_quantized_router_amd as m
    cfg = CONFIGS["stream80b"].replace(hidden=4096, experts=1024, top_k=16)
    _print("route max", T)
    Wr, rb, wsg = router_arrays(cfg, 0)
    xb = tokens_x(cfg, 0, T)
    out = m.moe_route_topk(torch.from_numpy(xb.view(np.int16)).cuda(),
                           torch.from_numpy(Wr).cuda(), torch.from_numpy(rb).cuda(),
                           cfg.top_k, wsg=torch.from_numpy(wsg).cuda())
    torch.cuda.synchronize()
    idx, w = out["idx"].cpu().numpy(), out["w"].cpu().numpy()
    lg, sg = out["logits"].cpu().numpy(), out["sigma"].cpu().numpy()
    depth = mfma_depth(cfg.hidden) if T > 8 else None
    decided = 0
    for t in range(T):
        x = O.bf16_to_f64(xb[t])
        decided += check_routing(idx[t], lg[t], x, Wr, rb, cfg.top_k, w[t], depth=depth)
        assert abs(sg[t] - O.sigmoid(np.dot(wsg.astype(np.float64), x))) <= 1e-6
    # with 1024 logits and k = 16 the k-th / (k+1)-th gap falls inside the f32
    # bound more often; at least 3 tokens in 4 must still be decided exactly
    assert decided >= 0.75 * T


def test_route_edge_cases(torch):
    import int4_group_quantized_router_amd as m
    cfg = CONFIGS["tiny"]
    Wr, rb, wsg = router_arrays(cfg, 0)
    dWr, dwsg = torch.from_numpy(Wr).cuda(), torch.from_numpy(wsg).cuda()
    # x = 0 and no bias: all logits tie -> experts 0..k-1, equal weights, sigma 1/2
    x0 = torch.zeros((3, cfg.hidden), dtype=torch.int16, device="cuda")
    for k in (1, 2, 16):
        out = m.moe_route_topk(x0, dWr, None, k, wsg=dwsg)
        torch.cuda.synchronize()
        assert (out["idx"].cpu().numpy() == np.arange(k)).all()
        assert np.allclose(out["w"].cpu().numpy(), 1.0 / k, rtol=0, atol=1e-7)
        assert np.all(out["sigma"].cpu().numpy() == 0.5)
    # k = E: weights equal the full softmax of the GPU logits
    xb = tokens_x(cfg, 0, 4)
    out = m.moe_route_topk(torch.from_numpy(xb.view(np.int16)).cuda(), dWr,
                           torch.from_numpy(rb).cuda(), cfg.experts)
    torch.cuda.synchronize()
    lg = out["logits"].cpu().numpy()
    for t in range(4):
        p = O.softmax(lg[t].astype(np.float64))
        idx = out["idx"].cpu().numpy()[t]
        assert sorted(idx.tolist()) == list(range(cfg.experts))
        assert np.allclose(out["w"].cpu().numpy()[t], p[idx], rtol=2e-6)
    # T = 0 is a no-op
    m.moe_route_topk(x0[:0], dWr, None, 2)


@pytest.mark.parametrize("E,k,group", [(256, 8, 2), (512, 10, 2), (512, 10, 3), (1024, 16, 4)])
@pytest.mark.parametrize("T", [1, 8, 300])
def test_route_exact_ties(torch, E, k, group, T):
    """Router rows repeated in groups of `group` (equal rows, equal bias):
    every logit occurs `group` times exactly, so the best logits tie with
    each other and the k-th place falls inside a tie.  The GPU's choice must
    be the oracle's selection rule on the GPU's own logits -- (logit desc,
    index asc) -- on every token."""
    import int4_group_quantized_router_amd as m
    cfg = CONFIGS["stream80b"].replace(experts=E, top_k=k)
    _print("route ties", E, k, group, T)
    Wr, rb, _ = router_arrays(cfg, 0)
    Wr = np.repeat(Wr[: (E + group - 1) // group], group, axis=0)[:E].copy()
    rb = np.repeat(rb[: (E + group - 1) // group], group)[:E].copy()
    xb = tokens_x(cfg, 0, T)
    out = m.moe_route_topk(torch.from_numpy(xb.view(np.int16)).cuda(), torch.from_numpy(Wr).cuda(),
                           torch.from_numpy(rb).cuda(), k)
    torch.cuda.synchronize()
    idx, lg = out["idx"].cpu().numpy(), out["logits"].cpu().numpy()
    ties = 0
    for t in range(T):
        want = O.select_topk(lg[t].astype(np.float64), k)
        assert np.array_equal(idx[t], want), (t, idx[t], want)
        ties += int(np.sum(lg[t] == lg[t][want[-1]]) > 1)
    assert ties == T  # the k-th logit is tied on every token


# ------------------------------------------------------------ single expert

@pytest.mark.parametrize("name,H,I,T", [("tiny", 256, 64, 3), ("decode35b", 2048, 512, 1),
                                        ("decode35b", 2048, 512, 8),
                                        ("decode80b_int8", 2048, 512, 2),
                                        ("decode80b_int8", 512, 256, 5)])
def test_expert_forward(torch, name, H, I, T):
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd.weights import upload_blob
    cfg = CONFIGS[name].replace(hidden=H, inter=I)
    _print("expert", name, H, I, T)
    arr = expert_arrays(cfg, 0, 5)
    blob = upload_blob(H, I, cfg.bits, arr)
    xb = tokens_x(cfg, 0, T)
    rng = np.random.default_rng(0)
    y0 = rng.standard_normal((T, H)).astype(np.float32)
    coef = rng.uniform(0.1, 1.0, T).astype(np.float32)
    y = torch.from_numpy(y0.copy()).cuda()
    m.moe_expert_forward(torch.from_numpy(xb.view(np.int16)).cuda(), H, I, cfg.bits, blob,
                         torch.from_numpy(coef).cuda(), y)
    torch.cuda.synchronize()
    Wg, Wu, Wd = O.dequant_expert(arr, cfg.bits, 64)
    for t in range(T):
        e = O.swiglu(O.bf16_to_f64(xb[t]), Wg, Wu, Wd)[0] * float(coef[t])
        err = np.max(np.abs(y.cpu().numpy()[t] - (y0[t] + e))) / np.max(np.abs(e))
        assert err <= REL_TOL, err


# -------------------------------------------------------------------- layer

def _layer_case(torch, cfg, calls, layer=0, max_undecided=1):
    """Run the layer on calls = [token-id lists] and compare every token whose
    routing equals the oracle's; at most `max_undecided` tokens may differ
    in routing (each only where the f32 error bound leaves the choice open)."""
    import int4_group_quantized_router_amd as m
    dm = DeviceModel(cfg, layers=layer + 1)
    L = dm.make_layers()[layer]
    worst = 0.0
    total = compared = 0
    try:
        for toks in calls:
            T = len(toks)
            xb = np.stack([token_x(cfg, t) for t in toks])
            y16 = torch.empty((T, cfg.hidden), dtype=torch.int16, device="cuda")
            y32 = torch.empty((T, cfg.hidden), dtype=torch.float32, device="cuda")
            idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
            w = torch.empty((T, cfg.top_k), dtype=torch.float32, device="cuda")
            m.moe_layer_forward(L, torch.from_numpy(xb.view(np.int16)).cuda(), y16, y32, idx, w)
            torch.cuda.synchronize()
            Wr, rb, _ = router_arrays(cfg, layer)
            for i in range(T):
                ref = oracle_layer(cfg, layer, xb[i])
                x = O.bf16_to_f64(xb[i])
                check_routing(idx.cpu().numpy()[i], None, x, Wr, rb, cfg.top_k)
                total += 1
                if np.array_equal(idx.cpu().numpy()[i], ref["idx"]):
                    compared += 1
                    err = rel_err(y32.cpu().numpy()[i], ref["y"])
                    worst = max(worst, err)
                    assert err <= REL_TOL, (toks, i, err)
            check_bf16_of_f32(y16.cpu().numpy(), y32.cpu().numpy())
    finally:
        dm.destroy()
    _print("worst rel err", worst, "tokens compared", compared, "/", total)
    assert compared >= total - max_undecided, (compared, total)
    return worst


def test_layer_tiny(torch):
    cfg = CONFIGS["tiny"]
    _print("layer tiny")
    _layer_case(torch, cfg, [list(range(8)), [8], [9, 10, 11], [12]])


@pytest.mark.parametrize("name", ["stream80b", "decode80b_int8", "decode35b"])
def test_layer_full_shape(torch, name):
    cfg = CONFIGS[name].replace(layers=1)
    _print("layer", name)
    _layer_case(torch, cfg, [[0], [1], list(range(2, 10)), [10, 11, 12], [13]])


@pytest.mark.parametrize("name", ["decode80b_int8", "decode35b"])
def test_layer_batch_repeated_tokens(torch, name):
    """Batches of 8 in which tokens repeat (all 8 equal: every distinct
    expert is shared by all tokens): each distinct expert is read once and
    applied to every token that chose it, so equal tokens give bitwise equal
    rows, and every row matches the oracle."""
    import int4_group_quantized_router_amd as m
    cfg = CONFIGS[name].replace(layers=1)
    _print("layer repeated tokens", name)
    _layer_case(torch, cfg, [[3, 3, 5, 3, 7, 7, 3, 5], [4] * 8])
    dm = DeviceModel(cfg, layers=1)
    L = dm.make_layers()[0]
    try:
        for toks in ([3, 3, 5, 3, 7, 7, 3, 5], [4] * 8):
            xb = np.stack([token_x(cfg, t) for t in toks])
            y32 = torch.empty((8, cfg.hidden), dtype=torch.float32, device="cuda")
            y16 = torch.empty((8, cfg.hidden), dtype=torch.int16, device="cuda")
            idx = torch.empty((8, cfg.top_k), dtype=torch.int32, device="cuda")
            w = torch.empty((8, cfg.top_k), dtype=torch.float32, device="cuda")
            m.moe_layer_forward(L, torch.from_numpy(xb.view(np.int16)).cuda(), y16, y32, idx, w)
            torch.cuda.synchronize()
            y, ix, wv = y32.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
            for i in range(8):
                j = toks.index(toks[i])
                assert np.array_equal(ix[i], ix[j])
                assert np.array_equal(wv[i].view(np.uint32), wv[j].view(np.uint32))
                assert np.array_equal(y[i].view(np.uint32), y[j].view(np.uint32))
    finally:
        dm.destroy()


@pytest.mark.parametrize("name", ["tiny", "decode35b"])
def test_layer_empty_and_zero_input(torch, name):
    """Degenerate inputs on every layer path (1 token, a batch of 8, the
    many-token path at 24): an empty batch is a no-op on a resident and on a
    pooled layer (the pool sees no access); x = 0 makes every gate and up
    product zero, so h = silu(0) * 0 = 0 and y = 0 exactly, while routing
    ranks the router bias alone (ties to the lowest index, so experts
    0..k-1 with weights 1/k when there is no bias)."""
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import weights as Wt
    from harness import dims_of
    cfg = CONFIGS[name].replace(layers=1)
    _print("layer empty / zero input", name)
    dm = DeviceModel(cfg, layers=1)
    store, _ = Wt.fill_store(dims_of(cfg), 1, lambda l, e: expert_arrays(cfg, l, e))
    pool = m.slotpool_create(store, cfg.experts, 0)
    L, Lp = dm.make_layers()[0], dm.make_layers(pool=pool)[0]
    H, k = cfg.hidden, cfg.top_k
    try:
        for layer in (L, Lp):
            x = torch.zeros((0, H), dtype=torch.int16, device="cuda")
            y16 = torch.empty((0, H), dtype=torch.int16, device="cuda")
            m.moe_layer_forward(layer, x, y16)
            torch.cuda.synchronize()
        st = m.slotpool_get_stats(pool)
        assert st["hits"] == 0 and st["misses"] == 0, st
        _, rb, _ = router_arrays(cfg, 0)
        want_idx = np.argsort(-rb.astype(np.float64), kind="stable")[:k]
        lw = rb.astype(np.float64)[want_idx]
        want_w = np.exp(lw - lw.max()) / np.exp(lw - lw.max()).sum()
        for T in (1, 8, 24):
            x = torch.zeros((T, H), dtype=torch.int16, device="cuda")
            y16 = torch.full((T, H), 7, dtype=torch.int16, device="cuda")
            y32 = torch.full((T, H), 7.0, dtype=torch.float32, device="cuda")
            idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
            w = torch.empty((T, k), dtype=torch.float32, device="cuda")
            m.moe_layer_forward(L, x, y16, y32, idx, w)
            torch.cuda.synchronize()
            assert np.all(y32.cpu().numpy() == 0.0), T
            assert np.all(y16.cpu().numpy() == 0), T
            assert (idx.cpu().numpy() == want_idx).all(), (T, idx.cpu().numpy()[0], want_idx)
            assert np.allclose(w.cpu().numpy(), want_w, rtol=4e-6, atol=0), T
    finally:
        dm.destroy()
        m.slotpool_destroy(pool)
        m.expert_store_destroy(store)


def test_layer_shared_inter_differs(torch):
    cfg = CONFIGS["tiny"].replace(inter=128, shared_inter=64, experts=32, top_k=4)
    _print("layer I != Is")
    _layer_case(torch, cfg, [[0], list(range(1, 8))])


# -------------------------------------------------------------------- stack

def test_stack_teacher_forced(torch):
    """Per-layer parity in a stack: each layer's GPU output against the oracle
    run on the GPU's own bf16 input to that layer; the RMS rescale between
    layers against the oracle's, to one bf16 ulp."""
    import int4_group_quantized_router_amd as m
    cfg = CONFIGS["decode35b"].replace(layers=4)
    _print("stack", cfg.name)
    dm = DeviceModel(cfg)
    layers = dm.make_layers()
    st = m.moe_stack_create(layers)
    H, k, L = cfg.hidden, cfg.top_k, cfg.layers
    assert m.moe_stack_persistent_active(st)  # one-token calls: one launch per stack
    try:
        for tok in range(3):
            T = 1
            x0 = torch.from_numpy(token_x(cfg, tok).view(np.int16)).cuda().view(1, H)
            xl = torch.empty((L, T, H), dtype=torch.int16, device="cuda")
            yl = torch.empty((L, T, H), dtype=torch.float32, device="cuda")
            idx = torch.empty((L, T, k), dtype=torch.int32, device="cuda")
            w = torch.empty((L, T, k), dtype=torch.float32, device="cuda")
            ylast = m.moe_stack_forward(st, x0, x_layers=xl, y_layers=yl, idx=idx, w=w)
            torch.cuda.synchronize()
            _check_stack_layers(cfg, tok, ylast.cpu().numpy(), xl.cpu().numpy(),
                                yl.cpu().numpy(), idx.cpu().numpy())
    finally:
        m.moe_stack_destroy(st)
        dm.destroy()


def _check_stack_layers(cfg, tok, ylast, xl_, yl_, ix, max_undecided=1):
    """Every layer of one token's stack exports against the oracle on the
    GPU's own input to that layer (teacher forcing), the RMS rescale chain
    to one bf16 ulp, the final bf16 output the rounding of the last f32
    output.  Layers whose routing differs from the oracle's (allowed only
    inside the f32 error bound) are counted; at most `max_undecided`."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    H, k, L = cfg.hidden, cfg.top_k, xl_.shape[0]
    xl_ = xl_.view(np.uint16)
    assert np.array_equal(xl_[0, 0], token_x(cfg, tok))
    # each layer's oracle run is independent (teacher forcing): one per worker
    with threadpool_limits(limits=1, user_api="blas"), \
            ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        refs = list(ex.map(lambda l: oracle_layer(cfg, l, xl_[l, 0]), range(L)))
    compared, worst = 0, 0.0
    for l in range(L):
        ref = refs[l]
        Wr, rb, _ = router_arrays(cfg, l)
        check_routing(ix[l, 0], None, O.bf16_to_f64(xl_[l, 0]), Wr, rb, k)
        if np.array_equal(ix[l, 0], ref["idx"]):
            compared += 1
            err = rel_err(yl_[l, 0], ref["y"])
            worst = max(worst, err)
            assert err <= REL_TOL, (tok, l, err)
        if l + 1 < L:
            nxt = O.rms_rescale(yl_[l, 0])
            diff = np.abs(nxt.astype(np.int64) - xl_[l + 1, 0].astype(np.int64))
            assert diff.max() <= 1, (tok, l)
    check_bf16_of_f32(ylast, yl_[L - 1])
    _print("token", tok, "layers compared", compared, "/", L, "worst rel err", worst)
    assert compared >= L - max_undecided, (tok, compared, L)


@pytest.mark.parametrize("name,tokens", [("decode35b", (0, 131)), ("decode80b_int8", (7,))])
def test_stack_full_depth_sampled(torch, name, tokens):
    """A resident stack at its full depth (35B-shaped int4: 40 layers;
    80B-shaped int8: 48), in the launch the bench times (one persistent
    kernel per token): for sampled tokens, every layer's output against the
    oracle on the GPU's own input to that layer, the rescale chain to one
    bf16 ulp, and the per-layer kernels giving the same bits."""
    import int4_group_quantized_router_amd as m
    cfg = CONFIGS[name]
    _print("stack full depth", cfg.name, cfg.layers)
    dm = DeviceModel(cfg)
    layers = dm.make_layers()
    st = m.moe_stack_create(layers)
    H, k, L = cfg.hidden, cfg.top_k, cfg.layers
    try:
        for tok in tokens:
            x0 = torch.from_numpy(token_x(cfg, tok).view(np.int16)).cuda().view(1, H)
            outs = []
            for persistent in (True, False):
                m.moe_stack_set_persistent(st, persistent)
                assert m.moe_stack_persistent_active(st) == persistent
                xl = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
                yl = torch.empty((L, 1, H), dtype=torch.float32, device="cuda")
                idx = torch.empty((L, 1, k), dtype=torch.int32, device="cuda")
                ylast = m.moe_stack_forward(st, x0, x_layers=xl, y_layers=yl, idx=idx)
                torch.cuda.synchronize()
                outs.append((ylast.cpu().numpy(), xl.cpu().numpy(), yl.cpu().numpy(),
                             idx.cpu().numpy()))
            for a, b in zip(outs[0], outs[1]):
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), tok
            _check_stack_layers(cfg, tok, *outs[0])
    finally:
        m.moe_stack_set_persistent(st, True)
        m.moe_stack_destroy(st)
        dm.destroy()


def test_stack_80b_int4_full_depth_resident_and_pooled(torch):
    """The 80B-shaped int4 stack at full depth (48 layers, 512 experts,
    top-10): resident, and through a slot pool of 30% of the experts over the
    pinned store (cold: every choice misses; warm: all hit, one launch; after
    a flush: misses again), in the persistent kernel.  All runs give the same
    bits, and every layer of the resident run matches the oracle on its own
    input.  The pool's counters and slots equal the oracle's replay."""
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import weights as Wt
    from oracle.pool_replay import PoolReplay
    from harness import dims_of
    cfg = CONFIGS["stream80b"]
    L, k = cfg.layers, cfg.top_k
    _print("80B int4 stack, full depth", L)
    dm = DeviceModel(cfg)
    store, stride = Wt.fill_store(dims_of(cfg), L, lambda l, e: expert_arrays(cfg, l, e))
    cap = int(cfg.pool_frac * L * cfg.experts)
    pool = m.slotpool_create(store, cap, 0)
    s_res = m.moe_stack_create(dm.make_layers())
    s_pool = m.moe_stack_create(dm.make_layers(pool=pool))
    assert m.moe_stack_persistent_active(s_res) and m.moe_stack_persistent_active(s_pool)
    replay = PoolReplay(cap, stride)
    try:
        for rnd, toks in enumerate(((0, 1), (0,))):
            for tok in toks:
                want = _stack_outputs(torch, m, s_res, cfg, tok)
                for run in ("first", "again"):
                    e0 = m.moe_stack_epoch(s_pool)
                    got = _stack_outputs(torch, m, s_pool, cfg, tok)
                    for u, v in zip(got, want):
                        assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), (rnd, tok, run)
                    for l in range(L):
                        replay.acquire(l, got[3][l, 0].tolist())
                        replay.release(l, got[3][l, 0].tolist())
                    if run == "again":  # every choice resident: one launch, no stop
                        assert m.moe_stack_epoch(s_pool) == e0 + 1
                if rnd == 0:
                    _check_stack_layers(cfg, tok, *want[:4])
            st = m.slotpool_stats(pool)
            assert {x: st[x] for x in replay.stats()} == replay.stats(), (st, replay.stats())
            for l in (0, L // 2, L - 1):
                for e in range(cfg.experts):
                    want_slot = replay.slot_of[(l, e)] if replay.resident(l, e) else -1
                    assert m.slotpool_slot_of(pool, l, e) == want_slot
            m.slotpool_flush(pool)
            replay.flush()
    finally:
        m.moe_stack_destroy(s_res)
        m.moe_stack_destroy(s_pool)
        dm.destroy()
        m.slotpool_destroy(pool)
        m.expert_store_destroy(store)


@pytest.mark.parametrize("name,L", [("tiny", 3), ("decode35b", 6), ("stream80b", 2),
                                    ("decode80b_int8", 2)])
def test_stack_persistent_matches_per_layer(torch, name, L):
    """The one-launch stack kernel computes every value with the per-layer
    kernels' arithmetic in the same order: all exports equal bit for bit, over
    consecutive calls whose hand-off buffers still hold the previous call's
    words."""
    import int4_group_quantized_router_amd as m
    cfg = CONFIGS[name].replace(layers=L)
    _print("stack persistent vs per-layer", name, L)
    dm = DeviceModel(cfg)
    st = m.moe_stack_create(dm.make_layers())
    H, k = cfg.hidden, cfg.top_k
    try:
        assert m.moe_stack_persistent_active(st)
        for tok in range(4):
            x0 = torch.from_numpy(token_x(cfg, tok).view(np.int16)).cuda().view(1, H)
            outs = []
            for persistent in (True, False):
                m.moe_stack_set_persistent(st, persistent)
                xl = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
                yl = torch.empty((L, 1, H), dtype=torch.float32, device="cuda")
                idx = torch.empty((L, 1, k), dtype=torch.int32, device="cuda")
                w = torch.empty((L, 1, k), dtype=torch.float32, device="cuda")
                y = m.moe_stack_forward(st, x0, x_layers=xl, y_layers=yl, idx=idx, w=w)
                torch.cuda.synchronize()
                outs.append([t.cpu().numpy().view(np.uint32 if t.element_size() == 4 else np.uint16)
                             for t in (y, xl, yl, idx, w)])
            for got, want, what in zip(outs[0], outs[1], ("y", "x_layers", "y_layers", "idx", "w")):
                assert np.array_equal(got, want), (name, tok, what)
            # no exports: only the stack's own hand-off buffers
            m.moe_stack_set_persistent(st, True)
            y = m.moe_stack_forward(st, x0)
            torch.cuda.synchronize()
            assert np.array_equal(y.cpu().numpy().view(np.uint16), outs[1][0])
    finally:
        m.moe_stack_destroy(st)
        dm.destroy()


@pytest.mark.parametrize("name", ["decode80b_int8", "decode35b"])
def test_stack_exact_ties_persistent_matches_per_layer(torch, name):
    """Routers whose rows come in equal triples (every logit occurs three
    times, and with k = 8 or 10 the k-th place splits a triple, so the tie
    rule decides which of equal experts are chosen): the persistent
    kernel's top-k instance picks exactly what the per-layer router picks
    (whose ties are checked against the oracle's rule elsewhere), and every
    export agrees bit for bit."""
    import int4_group_quantized_router_amd as m
    cfg = CONFIGS[name].replace(layers=3)
    _print("stack ties persistent vs per-layer", name)
    dm = DeviceModel(cfg)
    E = cfg.experts
    for l in range(cfg.layers):
        Wr, rb, _ = router_arrays(cfg, l)
        dm.Wr[l] = torch.from_numpy(np.repeat(Wr[: (E + 2) // 3], 3, axis=0)[:E].copy()).cuda()
        dm.rb[l] = torch.from_numpy(np.repeat(rb[: (E + 2) // 3], 3)[:E].copy()).cuda()
    st = m.moe_stack_create(dm.make_layers())
    try:
        assert m.moe_stack_persistent_active(st)
        for tok in range(4):
            outs = []
            for persistent in (True, False):
                m.moe_stack_set_persistent(st, persistent)
                outs.append(_stack_outputs(torch, m, st, cfg, tok))
            for got, want in zip(*outs):
                assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), (name, tok)
            idx = outs[0][3].reshape(cfg.layers, cfg.top_k)
            for r in idx:
                # whole triples, then the lowest indices of the triple the
                # k-th place splits
                groups = {}
                for e in r.tolist():
                    groups.setdefault(e // 3, []).append(e)
                partial = [g for g in groups.values() if len(g) < min(3, E - 3 * (g[0] // 3))]
                assert len(partial) <= 1
                for g in partial:
                    assert sorted(g) == list(range(3 * (g[0] // 3), 3 * (g[0] // 3) + len(g)))
    finally:
        m.moe_stack_destroy(st)
        dm.destroy()


# --------------------------------------------------------------------- pool

def test_pool_matches_resident_bitwise_and_replay(torch):
    """An expert served from the slot pool (hit or miss) gives exactly the
    resident result; the pool's decisions equal the oracle's replay."""
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import weights as Wt
    from oracle.pool_replay import PoolReplay
    from harness import dims_of
    cfg = CONFIGS["stream80b"].replace(layers=3)
    _print("pool", cfg.name)
    dm = DeviceModel(cfg)
    store, stride = Wt.fill_store(dims_of(cfg), cfg.layers, lambda l, e: expert_arrays(cfg, l, e))
    cap = 24
    pool = m.slotpool_create(store, cap, 0)
    res_layers = dm.make_layers()
    pool_layers = dm.make_layers(pool=pool)
    s_res, s_pool = m.moe_stack_create(res_layers), m.moe_stack_create(pool_layers)
    H, k, L = cfg.hidden, cfg.top_k, cfg.layers
    replay = PoolReplay(cap, stride)
    try:
        for rnd in range(2):
            for tok in range(6):
                x0 = torch.from_numpy(token_x(cfg, tok).view(np.int16)).cuda().view(1, H)
                outs = []
                for st in (s_res, s_pool):
                    yl = torch.empty((L, 1, H), dtype=torch.float32, device="cuda")
                    idx = torch.empty((L, 1, k), dtype=torch.int32, device="cuda")
                    y = m.moe_stack_forward(st, x0, y_layers=yl, idx=idx)
                    torch.cuda.synchronize()
                    outs.append((y.cpu().numpy(), yl.cpu().numpy(), idx.cpu().numpy()))
                assert np.array_equal(outs[0][0], outs[1][0])
                assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
                for l in range(L):
                    ex = outs[1][2][l, 0].tolist()
                    replay.acquire(l, ex)
                    replay.release(l, ex)
            stats = m.slotpool_get_stats(pool)
            assert {k: stats[k] for k in replay.stats()} == replay.stats(), (stats, replay.stats())
            assert stats["bytes_read"] == 0  # a memory store reads no file
            for l in range(L):
                for e in range(cfg.experts):
                    want = replay.slot_of[(l, e)] if replay.resident(l, e) else -1
                    assert m.slotpool_slot_of(pool, l, e) == want
            # slot bytes equal store bytes (a hit: no copy in flight)
            l, e = next(iter(replay.slot_of))
            ptrs, miss = m.slotpool_acquire(pool, l, [e])
            replay.acquire(l, [e])
            assert not miss[0]
            torch.cuda.synchronize()
            got = _device_bytes(ptrs[0], stride)
            src = m.expert_store_host_ptr(store, l, e)
            want = np.ctypeslib.as_array((ctypes.c_uint8 * stride).from_address(src))
            assert np.array_equal(got, want)
            m.slotpool_release(pool, l, [e])
            replay.release(l, [e])
            # second round starts from an empty pool: every access misses at first
            m.slotpool_flush(pool)
            replay.flush()
        with pytest.raises(m.MoEError) as ei:
            m.slotpool_acquire(pool, 0, list(range(cap + 1)))
        assert "POOL_EXHAUSTED" in str(ei.value)
        torch.cuda.synchronize()
    finally:
        m.moe_stack_destroy(s_res)
        m.moe_stack_destroy(s_pool)
        dm.destroy()
        m.slotpool_destroy(pool)
        m.expert_store_destroy(store)


def test_pool_prefetch_is_output_neutral(torch):
    """Experts prefetched by router-bias rank (12 per layer) into an empty
    pool before the first token: the pooled stack's outputs and exports stay
    bitwise the resident stack's, the pool's hits, misses, evictions, loads
    and the slot of every expert equal the oracle's replay of the prefetch
    and the accesses, and accesses hit prefetched experts."""
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import weights as Wt
    from oracle.pool_replay import PoolReplay
    from harness import dims_of
    cfg = CONFIGS["stream80b"].replace(layers=3)
    _print("pool prefetch", cfg.name)
    dm = DeviceModel(cfg)
    store, stride = Wt.fill_store(dims_of(cfg), cfg.layers, lambda l, e: expert_arrays(cfg, l, e))
    cap = 40
    pool = m.slotpool_create(store, cap, 0)
    res_layers = dm.make_layers()
    pool_layers = dm.make_layers(pool=pool)
    s_res, s_pool = m.moe_stack_create(res_layers), m.moe_stack_create(pool_layers)
    H, k, L = cfg.hidden, cfg.top_k, cfg.layers
    replay = PoolReplay(cap, stride)
    try:
        fresh = set()  # prefetched and not accessed yet
        for l in range(L):
            _, rb, _ = router_arrays(cfg, l)
            order = np.argsort(-rb, kind="stable")[:12].tolist()
            n = m.slotpool_prefetch(pool, l, order)
            assert n == replay.prefetch(l, order) == 12
            fresh |= {(l, e) for e in order}
        # a full pool loads nothing and evicts nothing
        spare = [e for e in range(cfg.experts) if not replay.resident(0, e)][:cap]
        n = m.slotpool_prefetch(pool, 0, spare)
        assert n == replay.prefetch(0, spare) == cap - 3 * 12
        assert m.slotpool_prefetch(pool, 1, spare) == replay.prefetch(1, spare) == 0
        fresh |= {(0, e) for e in spare[:cap - 36]}
        hits_on_prefetched = 0
        for tok in range(8):
            x0 = torch.from_numpy(token_x(cfg, tok).view(np.int16)).cuda().view(1, H)
            outs = []
            for st in (s_res, s_pool):
                yl = torch.empty((L, 1, H), dtype=torch.float32, device="cuda")
                idx = torch.empty((L, 1, k), dtype=torch.int32, device="cuda")
                y = m.moe_stack_forward(st, x0, y_layers=yl, idx=idx)
                torch.cuda.synchronize()
                outs.append((y.cpu().numpy(), yl.cpu().numpy(), idx.cpu().numpy()))
            assert np.array_equal(outs[0][0], outs[1][0]), tok
            assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32)), tok
            assert np.array_equal(outs[0][2], outs[1][2]), tok
            for l in range(L):
                ex = outs[1][2][l, 0].tolist()
                for e in ex:
                    if (l, e) in fresh and replay.resident(l, e):
                        hits_on_prefetched += 1
                    fresh.discard((l, e))
                replay.acquire(l, ex)
                replay.release(l, ex)
        stats = m.slotpool_get_stats(pool)
        assert {k_: stats[k_] for k_ in replay.stats()} == replay.stats(), (stats, replay.stats())
        assert stats["prefetched"] == cap and stats["evictions"] > 0, stats
        assert hits_on_prefetched > 0
        for l in range(L):
            for e in range(cfg.experts):
                want = replay.slot_of[(l, e)] if replay.resident(l, e) else -1
                assert m.slotpool_slot_of(pool, l, e) == want
        _print("prefetch hits", hits_on_prefetched, "stats", stats)
    finally:
        m.moe_stack_destroy(s_res)
        m.moe_stack_destroy(s_pool)
        dm.destroy()
        m.slotpool_destroy(pool)
        m.expert_store_destroy(store)


@pytest.mark.parametrize("cap", [24, 44])
def test_pool_stack_persistent_equals_per_layer(torch, cap):
    """A pooled stack run through the persistent kernel (stopping at the first
    layer with a miss, the host filling it and resuming) gives the per-layer
    pooled stack's outputs and exports bit for bit and leaves its pool in the
    same state: the same hits, misses, evictions and slot of every expert, so
    the replay of the hits keeps the policy's access order."""
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import weights as Wt
    from harness import dims_of
    cfg = CONFIGS["stream80b"].replace(layers=4)
    _print("pooled stack persistent vs per-layer", cfg.name)
    dm = DeviceModel(cfg)
    store, _ = Wt.fill_store(dims_of(cfg), cfg.layers, lambda l, e: expert_arrays(cfg, l, e))
    # 24 < 4 layers x top-10: every token stops somewhere; 44 holds a whole
    # token, so a repeated token runs all layers in one launch
    pools = [m.slotpool_create(store, cap, 0), m.slotpool_create(store, cap, 0)]
    stacks = [m.moe_stack_create(dm.make_layers(pool=p)) for p in pools]
    m.moe_stack_set_persistent(stacks[1], False)
    assert m.moe_stack_persistent_active(stacks[0])
    assert not m.moe_stack_persistent_active(stacks[1])
    H, k, L = cfg.hidden, cfg.top_k, cfg.layers
    try:
        for tok in [0, 0, 1, 2, 0, 0, 3, 1, 4, 4, 2]:
            x0 = torch.from_numpy(token_x(cfg, tok).view(np.int16)).cuda().view(1, H)
            outs = []
            for st in stacks:
                xl = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
                yl = torch.empty((L, 1, H), dtype=torch.float32, device="cuda")
                idx = torch.empty((L, 1, k), dtype=torch.int32, device="cuda")
                w = torch.empty((L, 1, k), dtype=torch.float32, device="cuda")
                y = m.moe_stack_forward(st, x0, x_layers=xl, y_layers=yl, idx=idx, w=w)
                torch.cuda.synchronize()
                outs.append([t.cpu().numpy() for t in (y, xl, yl, idx, w)])
            for a, b in zip(*outs):
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), tok
            st0, st1 = ({k: v for k, v in m.slotpool_get_stats(p).items() if k != "read_ns"}
                        for p in pools)
            assert st0 == st1, (tok, st0, st1)
        # at 24 slots the 40 accesses per token cycle through the pool and all
        # miss (the kernel stops at every layer); at 44 repeats hit
        assert st0["evictions"] > 0 and (cap < 40 or st0["hits"] > 0), st0
        for l in range(L):
            for e in range(cfg.experts):
                assert m.slotpool_slot_of(pools[0], l, e) == m.slotpool_slot_of(pools[1], l, e)
    finally:
        for st in stacks:
            m.moe_stack_destroy(st)
        dm.destroy()
        for p in pools:
            m.slotpool_destroy(p)
        m.expert_store_destroy(store)


def _stack_outputs(torch, m, st, cfg, tok):
    """One token through a stack: (y_last, x_layers, y_layers, idx, w) on the host."""
    H, k, L = cfg.hidden, cfg.top_k, len(st.keep)
    x0 = torch.from_numpy(token_x(cfg, tok).view(np.int16)).cuda().view(1, H)
    xl = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    yl = torch.empty((L, 1, H), dtype=torch.float32, device="cuda")
    idx = torch.empty((L, 1, k), dtype=torch.int32, device="cuda")
    w = torch.empty((L, 1, k), dtype=torch.float32, device="cuda")
    y = m.moe_stack_forward(st, x0, x_layers=xl, y_layers=yl, idx=idx, w=w)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (y, xl, yl, idx, w)]


def test_pool_stack_layer_indices_offset_and_permuted(torch):
    """Pooled stacks whose layers draw on store layers other than 0..n-1 (a
    permutation of the store's layers, and an offset run of two of them):
    the persistent kernel looks each layer's choices up in that layer's own
    row of the pool's table, so it equals the per-layer pooled path bit for
    bit and leaves the pool in the same state."""
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import weights as Wt
    from harness import dims_of
    cfg = CONFIGS["stream80b"].replace(layers=4)
    _print("pooled stack, layer indices permuted / offset")
    dm = DeviceModel(cfg, resident=False)
    store, _ = Wt.fill_store(dims_of(cfg), cfg.layers, lambda l, e: expert_arrays(cfg, l, e))
    try:
        for order in ([2, 0, 3, 1], [1, 2]):
            pools = [m.slotpool_create(store, 30, 0), m.slotpool_create(store, 30, 0)]
            stacks = []
            for p in pools:
                layers = []
                for l in order:
                    d = dims_of(cfg)
                    d["layer_index"] = l
                    layers.append(m.moe_layer_create(d, dm.Wr[l], dm.rb[l], dm.shared[l], dm.wsg[l],
                                                     pool=p))
                stacks.append(m.moe_stack_create(layers))
            m.moe_stack_set_persistent(stacks[1], False)
            assert m.moe_stack_persistent_active(stacks[0])
            try:
                for tok in [0, 0, 1, 2, 1, 0]:
                    a = _stack_outputs(torch, m, stacks[0], cfg, tok)
                    b = _stack_outputs(torch, m, stacks[1], cfg, tok)
                    for u, v in zip(a, b):
                        assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), (order, tok)
                    st0, st1 = ({k: v for k, v in m.slotpool_stats(p).items() if k != "read_ns"}
                                for p in pools)
                    assert st0 == st1, (order, tok, st0, st1)
                for l in range(cfg.layers):
                    for e in range(cfg.experts):
                        assert m.slotpool_slot_of(pools[0], l, e) == m.slotpool_slot_of(pools[1], l, e)
                # a store layer the stack does not use is never touched
                unused = [l for l in range(cfg.layers) if l not in order]
                for l in unused:
                    assert all(m.slotpool_slot_of(pools[0], l, e) == -1 for e in range(cfg.experts))
            finally:
                for st in stacks:
                    for L in st.keep:
                        m.moe_layer_destroy(L)
                    m.moe_stack_destroy(st)
                for p in pools:
                    m.slotpool_destroy(p)
    finally:
        m.expert_store_destroy(store)


def test_pool_layer_must_match_store(torch):
    """A pooled layer is checked against its pool's store before any launch:
    its layer index must exist there, its expert count and blob stride must
    equal the store's."""
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import _lib
    cfg = CONFIGS["tiny"].replace(layers=2)
    stride = m.moe_blob_layout_get(cfg.hidden, cfg.inter, cfg.bits)["stride"]
    store = m.expert_store_create(cfg.layers, cfg.experts, stride)
    pool = m.slotpool_create(store, 4, 0)
    dm = DeviceModel(cfg, resident=False)
    try:
        from harness import dims_of
        for bad in ({"layer_index": 2}, {"experts": 32}, {"inter": 128}):
            d = dict(dims_of(cfg), layer_index=0)
            d.update(bad)
            with pytest.raises(m.MoEError) as ei:
                m.moe_layer_create(d, dm.Wr[0], dm.rb[0], dm.shared[0], dm.wsg[0], pool=pool)
            assert ei.value.status == _lib.MOE_E_INVAL, bad
        ok = m.moe_layer_create(dict(dims_of(cfg), layer_index=1), dm.Wr[1], dm.rb[1],
                                dm.shared[1], dm.wsg[1], pool=pool)
        m.moe_layer_destroy(ok)
    finally:
        m.slotpool_destroy(pool)
        m.expert_store_destroy(store)


def test_stack_stale_handoff_words_never_match(torch):
    """The persistent kernel's h hand-off words carry a 15-bit launch tag.  A
    pooled call that stops at a layer leaves that layer's routed h words from
    an earlier launch; here the launch count is advanced so that a later
    launch's tag equals theirs, and that launch must still equal the
    resident stack bit for bit (the host clears words that old)."""
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import weights as Wt
    from harness import dims_of
    cfg = CONFIGS["tiny"].replace(layers=2)
    _print("stale hand-off words", cfg.name)
    dm = DeviceModel(cfg)
    store, _ = Wt.fill_store(dims_of(cfg), cfg.layers, lambda l, e: expert_arrays(cfg, l, e))
    pool = m.slotpool_create(store, cfg.layers * cfg.experts, 0)
    s_res = m.moe_stack_create(dm.make_layers())
    s_pool = m.moe_stack_create(dm.make_layers(pool=pool))
    assert m.moe_stack_persistent_active(s_pool) and m.moe_stack_persistent_active(s_res)
    try:
        tok_a = 0
        _stack_outputs(torch, m, s_pool, cfg, tok_a)           # fills A's experts
        e_a = m.moe_stack_epoch(s_pool)
        _stack_outputs(torch, m, s_pool, cfg, tok_a)           # one launch through both layers
        assert m.moe_stack_epoch(s_pool) == e_a + 1
        # a token whose experts are not all resident: the kernel stops at a layer
        tok_b = next(t for t in range(1, 64)
                     if any(set(r) - set(q) for r, q in zip(
                         _stack_outputs(torch, m, s_res, cfg, t)[3][:, 0].tolist(),
                         _stack_outputs(torch, m, s_res, cfg, tok_a)[3][:, 0].tolist())))
        want = _stack_outputs(torch, m, s_res, cfg, tok_b)
        miss0 = m.slotpool_stats(pool)["misses"]
        got = _stack_outputs(torch, m, s_pool, cfg, tok_b)
        assert m.slotpool_stats(pool)["misses"] > miss0
        for u, v in zip(got, want):
            assert np.array_equal(u.view(np.uint8), v.view(np.uint8))
        # next launch gets the tag of the launch that last wrote the stopped
        # layer's routed h words
        m.moe_stack_advance_epoch(s_pool, e_a + 32768 - m.moe_stack_epoch(s_pool))
        for rep in range(3):
            e0 = m.moe_stack_epoch(s_pool)
            got = _stack_outputs(torch, m, s_pool, cfg, tok_b)
            assert m.moe_stack_epoch(s_pool) == e0 + 1  # all resident: one launch
            for u, v in zip(got, want):
                assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), rep
            m.moe_stack_advance_epoch(s_pool, 32767)
        # the resident stack, advanced a whole tag period, is unaffected too
        m.moe_stack_advance_epoch(s_res, 32767)
        got = _stack_outputs(torch, m, s_res, cfg, tok_b)
        for u, v in zip(got, want):
            assert np.array_equal(u.view(np.uint8), v.view(np.uint8))
    finally:
        m.moe_stack_destroy(s_res)
        m.moe_stack_destroy(s_pool)
        dm.destroy()
        m.slotpool_destroy(pool)
        m.expert_store_destroy(store)


def test_stack_timeout_poisons_outputs(torch):
    """Failure handling of the persistent kernel, forced from the host with
    a zero bound on every wait (each wait returns at its first unmet poll,
    so every workgroup still leaves): the call's outputs hold NaN, the error
    comes back on the next call, and after the bound is restored the stack
    gives the per-layer result again."""
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import _lib
    cfg = CONFIGS["tiny"].replace(layers=3)
    _print("stack timeout", cfg.name)
    dm = DeviceModel(cfg)
    st = m.moe_stack_create(dm.make_layers())
    try:
        m.moe_stack_set_persistent(st, False)
        want = _stack_outputs(torch, m, st, cfg, 5)
        m.moe_stack_set_persistent(st, True)
        m.moe_stack_set_timeout(st, 0)
        got = _stack_outputs(torch, m, st, cfg, 5)
        y16 = got[0].view(np.uint16)
        assert np.any(y16 == 0x7FC0) or np.any(np.isnan(got[2])), "no output marked"
        with pytest.raises(m.MoEError) as ei:
            _stack_outputs(torch, m, st, cfg, 5)
        assert ei.value.status == _lib.MOE_E_HIP and "timed out" in str(ei.value)
        m.moe_stack_set_timeout(st, 2_000_000)
        for _ in range(2):
            got = _stack_outputs(torch, m, st, cfg, 5)
            for u, v in zip(got, want):
                assert np.array_equal(u.view(np.uint8), v.view(np.uint8))
    finally:
        m.moe_stack_destroy(st)
        dm.destroy()


def test_pool_shared_by_two_streams_bitwise(torch):
    """Two pooled layers on two compute streams share one small pool (every
    few calls evict a slot the other stream read last): results equal the
    resident layers bit for bit, with no synchronisation between calls."""
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import weights as Wt
    from harness import dims_of
    cfg = CONFIGS["tiny"].replace(layers=2)
    _print("pool shared by two streams", cfg.name)
    dm = DeviceModel(cfg)
    store, _ = Wt.fill_store(dims_of(cfg), cfg.layers, lambda l, e: expert_arrays(cfg, l, e))
    pool = m.slotpool_create(store, 3, 0)
    res_layers = dm.make_layers()
    pool_layers = dm.make_layers(pool=pool)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    H, n_tok = cfg.hidden, 12
    try:
        xs = [torch.from_numpy(token_x(cfg, t).view(np.int16)).cuda().view(1, H) for t in range(n_tok)]
        torch.cuda.synchronize()
        outs = {}
        for t in range(n_tok):
            for l in range(cfg.layers):
                st = streams[l]
                with torch.cuda.stream(st):
                    y = torch.empty((1, H), dtype=torch.float32, device="cuda")
                    m.moe_layer_forward(pool_layers[l], xs[t], None, y, stream=st)
                outs[(t, l)] = y
        torch.cuda.synchronize()
        for t in range(n_tok):
            for l in range(cfg.layers):
                want = torch.empty((1, H), dtype=torch.float32, device="cuda")
                m.moe_layer_forward(res_layers[l], xs[t], None, want)
                torch.cuda.synchronize()
                assert torch.equal(outs[(t, l)], want), (t, l)
        st = m.slotpool_get_stats(pool)
        assert st["evictions"] > 0, st
    finally:
        dm.destroy()
        m.slotpool_destroy(pool)
        m.expert_store_destroy(store)


def test_file_store_pool_matches_resident_bitwise(torch, tmp_path):
    """Experts fetched from the container file (one pread per miss into
    pinned staging, then the copy to the slot) give exactly the resident
    result, per token and layer, with hits and misses mixed."""
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import weights as Wt
    from oracle.pool_replay import PoolReplay
    from harness import dims_of
    cfg = CONFIGS["stream80b"].replace(layers=2, experts=64)
    _print("file store pool", cfg.name)
    dm = DeviceModel(cfg)
    store, stride = Wt.fill_file_store(str(tmp_path / "experts.qpack"), dims_of(cfg), cfg.layers,
                                       lambda l, e: expert_arrays(cfg, l, e))
    _print("store kind", m.STORE_KINDS[m.expert_store_kind(store)])
    cap = 24
    pool = m.slotpool_create(store, cap, 0)
    res_layers = dm.make_layers()
    pool_layers = dm.make_layers(pool=pool)
    s_res, s_pool = m.moe_stack_create(res_layers), m.moe_stack_create(pool_layers)
    H, k, L = cfg.hidden, cfg.top_k, cfg.layers
    replay = PoolReplay(cap, stride)
    try:
        for tok in range(12):
            x0 = torch.from_numpy(token_x(cfg, tok).view(np.int16)).cuda().view(1, H)
            outs = []
            for st in (s_res, s_pool):
                yl = torch.empty((L, 1, H), dtype=torch.float32, device="cuda")
                idx = torch.empty((L, 1, k), dtype=torch.int32, device="cuda")
                y = m.moe_stack_forward(st, x0, y_layers=yl, idx=idx)
                torch.cuda.synchronize()
                outs.append((y.cpu().numpy(), yl.cpu().numpy(), idx.cpu().numpy()))
            assert np.array_equal(outs[0][0], outs[1][0])
            assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
            for l in range(L):
                ex = outs[1][2][l, 0].tolist()
                replay.acquire(l, ex)
                replay.release(l, ex)
        stats = m.slotpool_get_stats(pool)
        assert {k_: stats[k_] for k_ in replay.stats()} == replay.stats()
        assert stats["misses"] > cap and stats["hits"] > 0 and stats["evictions"] > 0, stats
        assert stats["bytes_read"] == stats["misses"] * stride and stats["read_ns"] > 0
        # slot bytes equal the file's bytes (a hit: no copy in flight)
        l, e = next(iter(replay.slot_of))
        ptrs, miss = m.slotpool_acquire(pool, l, [e])
        assert not miss[0]
        torch.cuda.synchronize()
        assert np.array_equal(_device_bytes(ptrs[0], stride), m.expert_store_read(store, l, e, stride))
        m.slotpool_release(pool, l, [e])
        torch.cuda.synchronize()
    finally:
        m.moe_stack_destroy(s_res)
        m.moe_stack_destroy(s_pool)
        dm.destroy()
        m.slotpool_destroy(pool)
        m.expert_store_destroy(store)


# ------------------------------------------------------------------ prefill

def _prefill_run(torch, m, L, cfg, xb):
    T = xb.shape[0]
    y16 = torch.empty((T, cfg.hidden), dtype=torch.int16, device="cuda")
    y32 = torch.empty((T, cfg.hidden), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.top_k), dtype=torch.float32, device="cuda")
    m.moe_layer_forward(L, torch.from_numpy(xb.view(np.int16)).cuda(), y16, y32, idx, w)
    torch.cuda.synchronize()
    return y16.cpu().numpy(), y32.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def _prefill_case(torch, cfg, T, t0=0):
    """Many-token call against the oracle's bf16-weight mode on every token."""
    import int4_group_quantized_router_amd as m
    dm = DeviceModel(cfg, layers=1)
    L = dm.make_layers()[0]
    try:
        xb = tokens_x(cfg, t0, T)
        y16, y32, idx, w = _prefill_run(torch, m, L, cfg, xb)
        ref = oracle_tokens(cfg, 0, xb, bf16_weights=True)
        Wr, rb, _ = router_arrays(cfg, 0)
        same, worst = 0, 0.0
        for t in range(T):
            check_routing(idx[t], None, O.bf16_to_f64(xb[t]), Wr, rb, cfg.top_k,
                          depth=mfma_depth(cfg.hidden))
            if np.array_equal(idx[t], ref["idx"][t]):
                same += 1
                err = rel_err(y32[t], ref["y"][t])
                worst = max(worst, err)
                assert err <= REL_TOL, (t, err)
        assert same >= 0.95 * T
        check_bf16_of_f32(y16, y32)
        assert np.allclose(w.sum(axis=1), 1.0, atol=cfg.top_k * 2 ** -23 + 1e-7)
        _print("prefill", cfg.name, T, "worst rel err", worst, "routing equal", same, "/", T)
        return dm, L, xb, y32
    except Exception:
        dm.destroy()
        raise


@pytest.mark.parametrize("T", [9, 64, 200])
def test_prefill_tiny(torch, T):
    dm, *_ = _prefill_case(torch, CONFIGS["tiny"], T)
    dm.destroy()


@pytest.mark.parametrize("name,T", [("prefill80b", 300), ("decode80b_int8", 200)])
def test_prefill_reduced_experts(torch, name, T):
    cfg = CONFIGS[name].replace(layers=1, experts=64, top_k=4, zipf=None)
    dm, *_ = _prefill_case(torch, cfg, T)
    dm.destroy()


def test_prefill_shared_inter_differs(torch):
    """Shared intermediate 64 != routed 128 (the shared group's down has one
    K group and loads its (scale, bias) words one group at a time)."""
    cfg = CONFIGS["tiny"].replace(inter=128, shared_inter=64, experts=32, top_k=4)
    dm, *_ = _prefill_case(torch, cfg, 40)
    dm.destroy()


@pytest.mark.parametrize("name", ["prefill80b", "decode80b_int8"])
def test_prefill_down_per_group_scales_deep_k(torch, name):
    """Routed intermediate 512 (eight K groups in the down GEMM) with a
    shared intermediate of 128, which is not a multiple of 256: the down
    launch loads one (scale, bias) word per group, so its K pipeline runs
    that layout's steady state (int4 and int8) as well as its ends."""
    cfg = CONFIGS[name].replace(layers=1, experts=64, top_k=4, shared_inter=128, zipf=None)
    dm, *_ = _prefill_case(torch, cfg, 150)
    dm.destroy()


def test_prefill_int8_small_inter(torch):
    """int8 weights with K = 128 for down (not a multiple of 256)."""
    cfg = CONFIGS["decode80b_int8"].replace(layers=1, hidden=256, experts=32, top_k=4,
                                            inter=128, shared_inter=128)
    dm, *_ = _prefill_case(torch, cfg, 50)
    dm.destroy()


def test_prefill_pool_matches_resident_bitwise(torch):
    """Many tokens with experts served from the slot pool (all misses, then
    all hits) give exactly the resident result."""
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import weights as Wt
    from harness import dims_of
    cfg = CONFIGS["stream80b"].replace(layers=1, experts=64, top_k=4)
    _print("prefill pool", cfg.name)
    dm = DeviceModel(cfg, layers=1)
    store, _ = Wt.fill_store(dims_of(cfg), 1, lambda l, e: expert_arrays(cfg, l, e))
    pool = m.slotpool_create(store, cfg.experts, 0)
    try:
        L_res = dm.make_layers()[0]
        L_pool = dm.make_layers(pool=pool)[0]
        xb = tokens_x(cfg, 0, 96)
        want = _prefill_run(torch, m, L_res, cfg, xb)
        for rnd in range(2):  # first call misses, second hits
            got = _prefill_run(torch, m, L_pool, cfg, xb)
            assert np.array_equal(got[0], want[0])
            assert np.array_equal(got[1].view(np.uint32), want[1].view(np.uint32))
            assert np.array_equal(got[2], want[2])
            assert np.array_equal(got[3].view(np.uint32), want[3].view(np.uint32))
        stats = m.slotpool_get_stats(pool)
        assert stats["misses"] > 0 and stats["hits"] > 0, stats
    finally:
        dm.destroy()
        m.slotpool_destroy(pool)
        m.expert_store_destroy(store)


def test_prefill_token_permutation_is_bitwise(torch):
    import int4_group_quantized_router_amd as m
    cfg = CONFIGS["prefill80b"].replace(layers=1, experts=64, top_k=4)
    dm = DeviceModel(cfg, layers=1)
    L = dm.make_layers()[0]
    try:
        xb = tokens_x(cfg, 0, 300)
        perm = np.random.default_rng(3).permutation(300)
        _, y_a, idx_a, _ = _prefill_run(torch, m, L, cfg, xb)
        _, y_b, idx_b, _ = _prefill_run(torch, m, L, cfg, xb[perm])
        assert np.array_equal(idx_a[perm], idx_b)
        assert np.array_equal(y_a[perm].view(np.uint32), y_b.view(np.uint32))
    finally:
        dm.destroy()


def _sort_case(torch, idx_host, E):
    import int4_group_quantized_router_amd as m
    idx = torch.from_numpy(np.ascontiguousarray(idx_host, dtype=np.int32)).cuda()
    perm, off = m.moe_expert_sort(idx, E)
    torch.cuda.synchronize()
    want_perm, want_off = O.sort_by_expert(idx_host, E)
    got_off = off.cpu().numpy()
    assert np.array_equal(got_off, want_off), (got_off[:8], want_off[:8])
    n = int(want_off[E])
    assert np.array_equal(perm.cpu().numpy()[:n], want_perm)


def test_expert_sort_matches_oracle(torch):
    """The many-token path's grouping of (token, choice) pairs by expert,
    exported through moe_expert_sort, equals the oracle's stable counting
    sort exactly: on the router's own choices for the 4096-token 80B-shaped
    batch, on random choices, on one expert taking more rows than the
    in-LDS sort holds (9000), with a single expert, with choices outside
    [0, E) (left out), and with no tokens."""
    import int4_group_quantized_router_amd as m
    cfg = CONFIGS["prefill80b"]
    Wr, rb, _ = router_arrays(cfg, 0)
    xb = tokens_x(cfg, 0, cfg.tokens)
    out = m.moe_route_topk(torch.from_numpy(xb.view(np.int16)).cuda(), torch.from_numpy(Wr).cuda(),
                           torch.from_numpy(rb).cuda(), cfg.top_k, with_logits=False)
    torch.cuda.synchronize()
    assert out["logits"] is None
    _print("sort: router choices", cfg.tokens, cfg.top_k)
    _sort_case(torch, out["idx"].cpu().numpy(), cfg.experts)
    rng = np.random.default_rng(9)
    _print("sort: random")
    _sort_case(torch, rng.integers(0, 50, size=(777, 3)), 50)
    _print("sort: long segment")
    crowd = np.full((9000, 1), 7)
    crowd[::97, 0] = rng.integers(0, 16, size=crowd[::97, 0].shape)
    _sort_case(torch, crowd, 16)
    _print("sort: one expert")
    _sort_case(torch, np.zeros((10, 2), np.int64), 1)
    _print("sort: out-of-range choices")
    bad = rng.integers(0, 64, size=(300, 4))
    bad[::7, 1] = -1
    bad[::5, 2] = 64
    _sort_case(torch, bad, 64)
    _print("sort: max experts, top-16")
    _sort_case(torch, rng.integers(0, 1024, size=(2000, 16)), 1024)
    off = torch.full((9,), 5, dtype=torch.int32, device="cuda")
    m.moe_expert_sort(torch.zeros((0, 2), dtype=torch.int32, device="cuda"), 8, offsets=off)
    torch.cuda.synchronize()
    assert off.cpu().numpy().tolist() == [0] * 9


def test_prefill_full_size_every_token(torch):
    """4096 tokens, 512 experts, top-10 -- the only shape whose experts span
    several 96-row tiles and whose shared group has 43 tiles -- against the
    oracle's bf16-weight mode on every token: at least 95% of the tokens
    route exactly as the oracle does (the rest only within the f32 error
    bound), and every one of those is within 2e-3."""
    dm, *_ = _prefill_case(torch, CONFIGS["prefill80b"], CONFIGS["prefill80b"].tokens)
    dm.destroy()


def test_prefill_full_size_sampled(torch):
    """4096 tokens, 512 experts, top-10: every invariant on all tokens, the
    oracle on a sample of tokens (per token, bf16-weight mode)."""
    import int4_group_quantized_router_amd as m
    cfg = CONFIGS["prefill80b"]
    dm = DeviceModel(cfg, layers=1)
    L = dm.make_layers()[0]
    try:
        xb = tokens_x(cfg, 0, cfg.tokens)
        y16, y32, idx, w = _prefill_run(torch, m, L, cfg, xb)
        assert np.all(np.isfinite(y32))
        check_bf16_of_f32(y16, y32)
        assert np.allclose(w.sum(axis=1), 1.0, atol=cfg.top_k * 2 ** -23 + 1e-7)
        assert all(len(set(r)) == cfg.top_k for r in idx.tolist())
        Wr, rb, _ = router_arrays(cfg, 0)
        for t in [0, 1, 127, 128, 2047, 4000, 4094, 4095]:
            ref = oracle_layer(cfg, 0, xb[t], bf16_weights=True)
            check_routing(idx[t], None, O.bf16_to_f64(xb[t]), Wr, rb, cfg.top_k,
                          depth=mfma_depth(cfg.hidden))
            if np.array_equal(idx[t], ref["idx"]):
                assert rel_err(y32[t], ref["y"]) <= REL_TOL
    finally:
        dm.destroy()


def test_decode_and_prefill_agree(torch):
    """The same tokens through the per-token path (T <= 8) and the many-token
    path: each against its own oracle mode elsewhere; here, against each
    other (they differ by the bf16 rounding of the weights)."""
    import int4_group_quantized_router_amd as m
    cfg = CONFIGS["prefill80b"].replace(layers=1, experts=64, top_k=4)
    dm = DeviceModel(cfg, layers=1)
    L = dm.make_layers()[0]
    try:
        xb = tokens_x(cfg, 0, 64)
        _, y_p, idx_p, _ = _prefill_run(torch, m, L, cfg, xb)
        for t0 in range(0, 64, 8):
            _, y_d, idx_d, _ = _prefill_run(torch, m, L, cfg, xb[t0:t0 + 8])
            for i in range(8):
                if np.array_equal(idx_d[i], idx_p[t0 + i]):
                    assert rel_err(y_d[i], y_p[t0 + i]) <= 1e-2
    finally:
        dm.destroy()


# ---------------------------------------------------------- Gated DeltaNet

# Each step's f32 arithmetic: dot products of dk terms (|k|^2, |q|^2, S k^,
# S q^) and two roundings per state element.  Relative to the max-norm of
# the oracle's value, gamma_(dk + 4) ~ 8e-6 for dk = 128 bounds one step;
# the free-running state adds one such bound per step (alpha <= 1 keeps
# older errors from growing).
GDN_STEP_TOL = 2e-5


def _gdn_run(torch, m, name, B, T, seed=0):
    c = dict(GDN_CONFIGS[name], B=B)
    d = gdn_inputs(seed, c["B"], c["Hk"], c["Hv"], c["dk"], c["dv"], T)
    return c, d


@pytest.mark.parametrize("name,B,T", [("gdn_tiny", 3, 24), ("gdn80b", 2, 16), ("gdn80b", 64, 4)])
def test_gdn_step_matches_oracle(torch, name, B, T):
    """T consecutive decode steps on the GPU against the float64 oracle:
    each step from the GPU's own previous state (teacher-forced, within one
    step's f32 bound) and the whole run from the initial state (within T
    bounds)."""
    import int4_group_quantized_router_amd as m
    c, d = _gdn_run(torch, m, name, B, T)
    _print("gdn", name, B, T)
    scale = c["dk"] ** -0.5
    S = torch.from_numpy(d["S0"].copy()).cuda()
    S_free = d["S0"].astype(np.float64)
    for t in range(T):
        S_prev = S.cpu().numpy().astype(np.float64)
        q, k, v = (torch.from_numpy(d[x][t].view(np.int16)).cuda() for x in ("q", "k", "v"))
        al, be = (torch.from_numpy(d[x][t]).cuda() for x in ("alpha", "beta"))
        o = m.moe_gdn_step(q, k, v, al, be, S, scale=scale, eps=1e-6)
        torch.cuda.synchronize()
        S_ref, o_ref = G.gdn_step_bf16(S_prev, d["q"][t], d["k"][t], d["v"][t], d["alpha"][t],
                                       d["beta"][t], scale, 1e-6)
        assert rel_err(S.cpu().numpy(), S_ref) <= GDN_STEP_TOL, t
        assert rel_err(o.cpu().numpy(), o_ref) <= GDN_STEP_TOL, t
        S_free, _ = G.gdn_step_bf16(S_free, d["q"][t], d["k"][t], d["v"][t], d["alpha"][t],
                                    d["beta"][t], scale, 1e-6)
    assert rel_err(S.cpu().numpy(), S_free) <= T * GDN_STEP_TOL


@pytest.mark.parametrize("Hk,Hv,dk", [(8, 8, 128), (1, 8, 128), (3, 12, 64)])
def test_gdn_step_head_grouping(torch, Hk, Hv, dk):
    """Value heads over key heads at other ratios than the workloads' 2:
    one key head per value head, one key head for all, and 3 key heads for
    12 value heads (64x64 heads); 3 steps from the GPU's own state, each
    within one step's bound of the oracle."""
    import int4_group_quantized_router_amd as m
    B, T = 5, 3
    d = gdn_inputs(11, B, Hk, Hv, dk, dk, T)
    _print("gdn grouping", Hk, Hv, dk)
    scale = dk ** -0.5
    S = torch.from_numpy(d["S0"].copy()).cuda()
    for t in range(T):
        S_prev = S.cpu().numpy().astype(np.float64)
        q, k, v = (torch.from_numpy(d[x][t].view(np.int16)).cuda() for x in ("q", "k", "v"))
        al, be = (torch.from_numpy(d[x][t]).cuda() for x in ("alpha", "beta"))
        o = m.moe_gdn_step(q, k, v, al, be, S, scale=scale, eps=1e-6)
        torch.cuda.synchronize()
        S_ref, o_ref = G.gdn_step_bf16(S_prev, d["q"][t], d["k"][t], d["v"][t], d["alpha"][t],
                                       d["beta"][t], scale, 1e-6)
        assert rel_err(S.cpu().numpy(), S_ref) <= GDN_STEP_TOL, t
        assert rel_err(o.cpu().numpy(), o_ref) <= GDN_STEP_TOL, t


def test_gdn_step_exact_cases(torch):
    """beta = 0, and a zero key with eps > 0, write nothing: the new state is
    exactly f32(alpha * S) (one rounding, as the kernel forms it), and the
    output reads it; rejected shapes leave the state untouched."""
    import int4_group_quantized_router_amd as m
    c, d = _gdn_run(torch, m, "gdn80b", 2, 1, seed=3)
    S0 = d["S0"]
    q, k, v = (torch.from_numpy(d[x][0].view(np.int16)).cuda() for x in ("q", "k", "v"))
    al = torch.from_numpy(d["alpha"][0]).cuda()
    for case in ("beta0", "zero_key"):
        S = torch.from_numpy(S0.copy()).cuda()
        be = torch.from_numpy(np.zeros_like(d["beta"][0]) if case == "beta0" else d["beta"][0]).cuda()
        kk = torch.zeros_like(k) if case == "zero_key" else k
        o = m.moe_gdn_step(q, kk, v, al, be, S, scale=1.0, eps=1e-6)
        torch.cuda.synchronize()
        want = (d["alpha"][0][:, :, None, None] * S0).astype(np.float32)
        assert np.array_equal(S.cpu().numpy(), want), case
        _, o_ref = G.gdn_step_bf16(want.astype(np.float64), d["q"][0], np.zeros_like(d["k"][0]),
                                   d["v"][0], np.ones_like(d["alpha"][0]),
                                   np.zeros_like(d["beta"][0]), 1.0, 1e-6)
        assert rel_err(o.cpu().numpy(), o_ref) <= GDN_STEP_TOL
    S = torch.from_numpy(S0.copy()).cuda()
    v3, a3 = v[:, :3].contiguous(), al[:, :3].contiguous()
    with pytest.raises(m.MoEError):
        m.moe_gdn_step(q, k, v3, a3, a3, S)  # 3 value heads over 16 key heads
    torch.cuda.synchronize()
    assert np.array_equal(S.cpu().numpy(), S0)
