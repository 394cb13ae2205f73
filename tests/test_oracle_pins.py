"""Pins for the CPU oracle: each test ties an oracle function to something
other than itself (a library routine, a brute-force definition, a closed
form or an invariant), so a dropped term, a wrong index or sign, or a
transposed operand fails one of them."""

import itertools

import numpy as np
import pytest
import scipy.special
import torch

from moe_inputs import CONFIGS, expert_arrays, router_arrays, shared_arrays, token_x
from moe_inputs.generate import bf16_bits_from_f32
from oracle import moe_oracle as O

TINY = CONFIGS["tiny"]


# ------------------------------------------------------------------ bf16

def test_round_bf16_matches_torch_rne():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # exact ties: bf16 value + half an ulp (bit 15 set, lower bits zero)
    tie_bits = (rng.integers(0, 1 << 16, 5000, dtype=np.uint32) << 16) | 0x8000
    tie_bits &= 0x7EFFFFFF          # keep the rounded value finite
    x = np.concatenate([x, tie_bits.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_is_nearest_from_f64():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(20_000) * 10.0 ** rng.integers(-30, 30, 20_000)
    r = O.round_bf16(x)
    # representable in bf16: widening the bits reproduces the value
    assert np.array_equal(O.bf16_to_f64(O.bf16_bits(r)), r)
    bits = O.bf16_bits(r).astype(np.int64)
    up = O.bf16_to_f64(((bits + 1) & 0xFFFF).astype(np.uint16))
    dn = O.bf16_to_f64(((bits - 1) & 0xFFFF).astype(np.uint16))
    for nb in (up, dn):
        ok = np.isfinite(nb) & (np.sign(nb) == np.sign(r))
        d_r, d_n = np.abs(x - r), np.abs(x - nb)
        assert np.all(d_r[ok] <= d_n[ok])
        tie = ok & (d_r == d_n)
        assert np.all((bits[tie] & 1) == 0)


def test_generator_bf16_agrees_with_oracle_rounding():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(10_000).astype(np.float32)
    assert np.array_equal(O.bf16_to_f64(bf16_bits_from_f32(x)),
                          O.round_bf16(x.astype(np.float64)))


# ------------------------------------------------------- packed fields

def _fields_by_bits(words, bits, n_cols):
    """Bit-by-bit extraction, written independently of the oracle's shifts."""
    out = np.zeros((words.shape[0], n_cols), dtype=np.int64)
    for r in range(words.shape[0]):
        for c in range(n_cols):
            v = 0
            for i in range(bits):
                bit_index = c * bits + i            # position in the row's bit string
                word = int(words[r, bit_index // 32])
                v |= ((word >> (bit_index % 32)) & 1) << i
            out[r, c] = v
    return out


@pytest.mark.parametrize("bits", [4, 8])
def test_unpack_against_bit_loop(bits):
    rng = np.random.default_rng(bits)
    words = rng.integers(0, 1 << 32, size=(3, 8), dtype=np.uint32)
    n_cols = 8 * 32 // bits
    assert np.array_equal(O.unpack_fields(words, bits, n_cols),
                          _fields_by_bits(words, bits, n_cols))


@pytest.mark.parametrize("bits", [4, 8])
def test_pack_then_unpack_is_identity(bits):
    rng = np.random.default_rng(10 + bits)
    n_cols = 64
    q = rng.integers(0, 1 << bits, size=(5, n_cols))
    words = np.zeros((5, n_cols * bits // 32), dtype=np.uint32)
    for r in range(5):
        for c in range(n_cols):       # least-significant field first
            words[r, c * bits // 32] |= np.uint32(q[r, c] << ((c * bits) % 32))
    assert np.array_equal(O.unpack_fields(words, bits, n_cols), q)


# ------------------------------------------------------------ dequant

@pytest.mark.parametrize("cfg_name", ["tiny", "decode80b_int8"])
def test_dequant_exact_in_f32_and_requantises(cfg_name):
    cfg = CONFIGS[cfg_name].replace(hidden=256, inter=128)
    arr = expert_arrays(cfg, 0, 3)
    for name in ("gate", "up", "down"):
        words, s, b = arr[name]
        W = O.dequantize(words, s, b, cfg.bits, cfg.group)
        assert np.array_equal(W.astype(np.float32).astype(np.float64), W)
        n_cols = s.shape[1] * cfg.group
        q = _fields_by_bits(words[:2], cfg.bits, n_cols)
        sv = np.repeat(O.bf16_to_f64(s[:2]), cfg.group, axis=1)
        bv = np.repeat(O.bf16_to_f64(b[:2]), cfg.group, axis=1)
        assert np.array_equal((W[:2] - bv) / sv, q.astype(np.float64))
        # every weight in f32: s*q + b with one rounding equals the exact value
        s32, q32, b32 = sv.astype(np.float32), q.astype(np.float32), bv.astype(np.float32)
        assert np.array_equal((s32 * q32 + b32).astype(np.float64), W[:2])


def test_dequant_group_and_row_indexing():
    # s differs per (row, group) so a transposed or shifted group index shows up
    out, inn, g = 3, 256, 64
    words = np.full((out, inn // 8), 0x76543210, dtype=np.uint32)  # q = c mod 8
    s_val = np.array([[1, 2, 4, 8], [16, 32, 64, 128], [0.5, 0.25, 0.125, 0.0625]])
    b_val = -np.arange(12, dtype=np.float64).reshape(3, 4)
    s = bf16_bits_from_f32(s_val.astype(np.float32))
    b = bf16_bits_from_f32(b_val.astype(np.float32))
    W = O.dequantize(words, s, b, 4, g)
    for r in range(out):
        for c in range(inn):
            assert W[r, c] == s_val[r, c // g] * (c % 8) + b_val[r, c // g]


def _zero_point_matrix(out, inn, bits, scale):
    per = 32 // bits
    mid = 1 << (bits - 1)
    word = 0
    for i in range(per):
        word |= mid << (bits * i)
    words = np.full((out, inn // per), word, dtype=np.uint32)
    s = bf16_bits_from_f32(np.full((out, inn // 64), scale, np.float32))
    b = bf16_bits_from_f32(np.full((out, inn // 64), -mid * scale, np.float32))
    return words, s, b


@pytest.mark.parametrize("bits", [4, 8])
def test_zero_point_expert_outputs_zero(bits):
    H, I = 128, 64
    arr = {"gate": _zero_point_matrix(I, H, bits, 0.0078125),
           "up": _zero_point_matrix(I, H, bits, 0.015625),
           "down": _zero_point_matrix(H, I, bits, 0.03125)}
    Wg, Wu, Wd = O.dequant_expert(arr, bits, 64)
    assert not Wg.any() and not Wu.any() and not Wd.any()
    x = O.bf16_to_f64(token_x(TINY.replace(hidden=H), 0))
    y, h = O.swiglu(x, Wg, Wu, Wd)
    assert not y.any() and not h.any()


def test_constant_group_dot():
    rng = np.random.default_rng(7)
    x = O.round_bf16(rng.standard_normal(64))
    for c in (0, 5, 15):
        words = np.full((1, 8), sum(c << (4 * i) for i in range(8)), dtype=np.uint32)
        s_v, b_v = 0.01171875, -0.09375
        s = bf16_bits_from_f32(np.array([[s_v]], np.float32))
        b = bf16_bits_from_f32(np.array([[b_v]], np.float32))
        W = O.dequantize(words, s, b, 4, 64)
        assert np.isclose((W @ x)[0], (s_v * c + b_v) * x.sum(), rtol=1e-13, atol=1e-13)


def test_gemv_against_loops():
    cfg = TINY
    arr = expert_arrays(cfg, 0, 5)
    x = O.bf16_to_f64(token_x(cfg, 0))
    words, s, b = arr["gate"]
    W = O.dequantize(words, s, b, 4, 64)
    q = _fields_by_bits(words[:4], 4, cfg.hidden)
    sv, bv = O.bf16_to_f64(s[:4]), O.bf16_to_f64(b[:4])
    for r in range(4):
        acc = 0.0
        for c in range(cfg.hidden):
            acc += (sv[r, c // 64] * q[r, c] + bv[r, c // 64]) * x[c]
        assert np.isclose((W @ x)[r], acc, rtol=1e-12, atol=1e-12)
    assert np.allclose(W @ x, np.dot(W, x), rtol=1e-14, atol=1e-14)


# ----------------------------------------------------------- routing

def test_topk_bruteforce_with_ties():
    rng = np.random.default_rng(11)
    for trial in range(300):
        E = 16
        logits = rng.integers(-3, 4, size=E).astype(np.float64)  # many exact ties
        if trial % 2:
            logits = logits + rng.standard_normal(E) * 0.1
        for k in range(1, E + 1):
            S = O.select_topk(logits, k)
            # brute force: e is chosen iff fewer than k experts beat it, where
            # e' beats e when its logit is larger, or equal with a lower index
            beats = lambda a, b: logits[a] > logits[b] or (logits[a] == logits[b] and a < b)
            chosen = [e for e in range(E) if sum(beats(o, e) for o in range(E)) < k]
            assert sorted(S.tolist()) == chosen
            for a, b in zip(S[:-1], S[1:]):
                assert beats(a, b)


def test_topk_all_pairs():
    E = 16
    for a, b in itertools.combinations(range(E), 2):
        logits = np.linspace(-1, 0, E) * 0.0 - 5.0
        logits[a], logits[b] = 2.0, 3.0
        assert O.select_topk(logits, 2).tolist() == [b, a]
        logits[a] = logits[b] = 1.0
        assert O.select_topk(logits, 2).tolist() == [a, b]


def test_route_zero_input_no_bias():
    cfg = CONFIGS["decode35b"].replace(hidden=128)
    Wr, _, _ = router_arrays(cfg, 0)
    for k in (2, 8, 10):
        logits, p, idx, w = O.route(np.zeros(cfg.hidden), Wr, np.zeros(cfg.experts), k)
        assert idx.tolist() == list(range(k))
        assert np.allclose(w, 1.0 / k, rtol=0, atol=1e-16)


def test_route_zero_input_zipf_closed_form():
    cfg = CONFIGS["stream80b"].replace(hidden=64)
    Wr, rb, _ = router_arrays(cfg, 2)
    k = cfg.top_k
    logits, p, idx, w = O.route(np.zeros(cfg.hidden), Wr, rb, k)
    perm = np.random.default_rng((cfg.seed, 4, 2)).permutation(cfg.experts)
    assert idx.tolist() == perm[:k].tolist()          # ranks 1..k in order
    ranks = np.arange(1, k + 1, dtype=np.float64)
    expect = ranks ** -1.1 / np.sum(ranks ** -1.1)
    # rb is float32, so compare at float32 resolution of the bias
    assert np.allclose(w, expect, rtol=1e-6, atol=0)


def test_k_equals_E_gives_full_softmax():
    rng = np.random.default_rng(12)
    E, H = 16, 64
    Wr = rng.standard_normal((E, H)) * 0.1
    rb = rng.standard_normal(E)
    x = rng.standard_normal(H)
    logits, p, idx, w = O.route(x, Wr, rb, E)
    ref = scipy.special.softmax(Wr @ x + rb)
    assert np.allclose(w, ref[idx], rtol=1e-13, atol=0)
    assert np.allclose(p, ref, rtol=1e-13, atol=0)


def test_routing_weight_invariants():
    cfg = CONFIGS["stream80b"]
    Wr, rb, _ = router_arrays(cfg, 0)
    for t in range(8):
        x = O.bf16_to_f64(token_x(cfg, t))
        logits, p, idx, w = O.route(x, Wr, rb, cfg.top_k)
        assert abs(w.sum() - 1.0) < 1e-15
        assert np.all(w >= 0) and np.all(np.diff(w) <= 0)
        assert len(set(idx.tolist())) == cfg.top_k
        # the renormalised weights equal a softmax over the chosen logits
        assert np.allclose(w, scipy.special.softmax(logits[idx]), rtol=1e-13)


# ------------------------------------------------------- activations

def test_silu_and_sigmoid_against_scipy():
    z = np.concatenate([np.linspace(-50, 50, 2001), [-800.0, 800.0, 0.0]])
    with np.errstate(over="raise"):
        s = O.sigmoid(z)
        f = O.silu(z)
    assert np.allclose(s, scipy.special.expit(z), rtol=1e-15, atol=0)
    assert np.allclose(f, z * scipy.special.expit(z), rtol=1e-15, atol=0)
    assert np.all(np.isfinite(f))


# ------------------------------------------------------------- expert

def test_expert_closed_form_constant_weights():
    H = I = 64
    cg, cu, cd = 11, 3, 9
    sg, bg, su, bu, sd, bd = 0.0078125, -0.0625, 0.015625, -0.125, 0.03125, -0.25

    def const(out, inn, c, s_v, b_v):
        words = np.full((out, inn // 8), sum(c << (4 * i) for i in range(8)), np.uint32)
        s = bf16_bits_from_f32(np.full((out, 1), s_v, np.float32))
        b = bf16_bits_from_f32(np.full((out, 1), b_v, np.float32))
        return words, s, b

    arr = {"gate": const(I, H, cg, sg, bg), "up": const(I, H, cu, su, bu),
           "down": const(H, I, cd, sd, bd)}
    x = O.round_bf16(np.random.default_rng(4).standard_normal(H))
    Sx = x.sum()
    g = (sg * cg + bg) * Sx
    u = (su * cu + bu) * Sx
    h = O.round_bf16(np.array([g / (1 + np.exp(-g)) * u]))[0]
    y_expect = (sd * cd + bd) * I * h
    y, hh = O.swiglu(x, *O.dequant_expert(arr, 4, 64))
    assert np.allclose(hh, h, rtol=0, atol=0)
    assert np.allclose(y, y_expect, rtol=1e-13, atol=1e-15)


def test_bf16_weight_mode_rounds_each_weight():
    arr = expert_arrays(TINY, 0, 1)
    exact = O.dequant_expert(arr, 4, 64, bf16_weights=False)
    rounded = O.dequant_expert(arr, 4, 64, bf16_weights=True)
    for W, Wb in zip(exact, rounded):
        assert np.array_equal(Wb, torch.from_numpy(W.astype(np.float32))
                              .to(torch.bfloat16).double().numpy())


# -------------------------------------------------------------- layer

def _tiny_layer(cfg=TINY, layer=0):
    Wr, rb, wsg = router_arrays(cfg, layer)
    sh = shared_arrays(cfg, layer)
    return Wr, rb, wsg, sh


def test_layer_with_identical_experts_is_expert_plus_gated_shared():
    cfg = TINY
    Wr, rb, wsg, sh = _tiny_layer()
    same = expert_arrays(cfg, 0, 0)
    x_bits = token_x(cfg, 0)
    x = O.bf16_to_f64(x_bits)
    out = O.moe_layer(x_bits, Wr, rb, wsg, sh, lambda e: same, cfg.top_k, 4)
    y_e = O.swiglu(x, *O.dequant_expert(same, 4, 64))[0]
    y_s = O.swiglu(x, *O.dequant_expert(sh, 4, 64))[0]
    sigma = scipy.special.expit(np.dot(wsg.astype(np.float64), x))
    assert np.allclose(out["y"], y_e + sigma * y_s, rtol=1e-12, atol=1e-12)


def test_layer_weights_attach_to_the_right_expert():
    cfg = TINY.replace(top_k=4)
    Wr, rb, wsg, _ = _tiny_layer(cfg)
    H, I = cfg.hidden, cfg.inter
    zero = {"gate": _zero_point_matrix(I, H, 4, 0.0078125),
            "up": _zero_point_matrix(I, H, 4, 0.0078125),
            "down": _zero_point_matrix(H, I, 4, 0.0078125)}
    x_bits = token_x(cfg, 3)
    x = O.bf16_to_f64(x_bits)
    _, _, idx, w = O.route(x, Wr, rb, cfg.top_k)
    live = expert_arrays(cfg, 0, 9)
    y_live = O.swiglu(x, *O.dequant_expert(live, 4, 64))[0]
    for j, e in enumerate(idx):
        fn = lambda ee, e=e: live if ee == e else zero
        out = O.moe_layer(x_bits, Wr, rb, wsg, zero, fn, cfg.top_k, 4)
        assert np.allclose(out["y"], w[j] * y_live, rtol=1e-12, atol=1e-14)


def test_layer_zero_input():
    cfg = TINY
    Wr, rb, wsg, sh = _tiny_layer()
    x_bits = np.zeros(cfg.hidden, np.uint16)
    out = O.moe_layer(x_bits, Wr, rb, wsg, sh, lambda e: expert_arrays(cfg, 0, e),
                      cfg.top_k, 4)
    assert out["idx"].tolist() == [0, 1]
    assert np.all(out["w"] == 0.5) and out["sigma"] == 0.5
    assert not out["y"].any()


def test_layer_tokens_matches_per_token():
    cfg = TINY
    Wr, rb, wsg, sh = _tiny_layer()
    X = np.stack([token_x(cfg, t) for t in range(cfg.tokens)])
    fn = lambda e: expert_arrays(cfg, 0, e)
    for bf in (False, True):
        many = O.moe_layer_tokens(X, Wr, rb, wsg, sh, fn, cfg.top_k, 4, bf16_weights=bf)
        for t in range(cfg.tokens):
            one = O.moe_layer(X[t], Wr, rb, wsg, sh, fn, cfg.top_k, 4, bf16_weights=bf)
            assert np.array_equal(one["idx"], many["idx"][t])
            assert np.allclose(one["y"], many["y"][t], rtol=1e-12, atol=1e-12)


def test_rms_rescale_unit_rms_and_rounding():
    rng = np.random.default_rng(5)
    y = (rng.standard_normal(2048) * 37.0).astype(np.float32)
    xb = O.rms_rescale(y)
    x = O.bf16_to_f64(xb)
    assert abs(np.sqrt(np.mean(x ** 2)) - 1.0) < 4e-3
    ref = y.astype(np.float64) / np.sqrt(np.mean(y.astype(np.float64) ** 2) + 1e-6)
    ulp = np.ldexp(1.0, np.frexp(ref)[1] - 8)
    assert np.all(np.abs(x - ref) <= ulp * 0.5 + np.abs(ref) * 1e-6)


# ------------------------------------------------------- grouping by expert

def test_sort_by_expert_hand_worked():
    """3 tokens, k = 2, E = 3: pairs p = t*k + j choose experts 2,0 | 0,1 |
    2,1; grouped by expert with (token, choice) order kept inside each
    expert: expert 0 <- pairs 1, 2; expert 1 <- 3, 5; expert 2 <- 0, 4."""
    perm, off = O.sort_by_expert(np.array([[2, 0], [0, 1], [2, 1]]), 3)
    assert perm.tolist() == [1, 2, 3, 5, 0, 4]
    assert off.tolist() == [0, 2, 4, 6]


@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (7, 2, 16, 1), (50, 4, 8, 2),
                                        (33, 10, 512, 3), (200, 3, 5, 4)])
def test_sort_by_expert_against_comparison_sort(T, k, E, seed):
    """Brute force: Python's comparison sort of the pairs by (expert, pair
    index); offsets from counting each expert's rows in that order; every
    row's pair chose the expert of its segment; perm is a permutation."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, size=(T, k))
    if T > 3:
        idx[: T // 2, 0] = idx[0, 0]  # a crowded expert
    perm, off = O.sort_by_expert(idx, E)
    flat = idx.reshape(-1).tolist()
    want = sorted(range(T * k), key=lambda p: (flat[p], p))
    assert perm.tolist() == want
    assert sorted(perm.tolist()) == list(range(T * k))
    assert off[0] == 0 and off[E] == T * k and np.all(np.diff(off) >= 0)
    for e in range(E):
        rows = perm[off[e]:off[e + 1]]
        assert all(flat[p] == e for p in rows)
        assert np.all(np.diff(rows) > 0)
        assert off[e + 1] - off[e] == flat.count(e)


def test_sort_by_expert_edge_cases():
    """No pairs; a single expert taking every pair; experts outside [0, E)
    are left out and offsets count only the rest."""
    perm, off = O.sort_by_expert(np.zeros((0, 4), np.int64), 6)
    assert perm.size == 0 and off.tolist() == [0] * 7
    perm, off = O.sort_by_expert(np.full((5, 2), 3), 4)
    assert perm.tolist() == list(range(10)) and off.tolist() == [0, 0, 0, 0, 10]
    perm, off = O.sort_by_expert(np.array([[1, -1], [4, 0], [1, 2]]), 3)
    assert perm.tolist() == [3, 0, 4, 5] and off.tolist() == [0, 1, 3, 4]
