"""CPU oracle for the group-quantized routed-expert MoE layer (NumPy, float64).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library
never calls it and shares no code with it; the two meet only in the seeded
inputs of ``moe_inputs``.

Page abbreviations used in the citations below:

* [xix]    xix.ai (Korean), "Swiftlet Packs 80B Qwen Into Mac With 4.3GB
           Memory; iPhone 17 to Run 35B Natively"; [xix-ru] is its Russian
           translation on xix.ai/ru.
* [ttj]    ttj.kr article on Swiftlet ("80B 큐원을 4.3GB로 ... 애플 기기용 MoE
           스트리밍 런타임 스위프트렛").
* [digest] paper-digest.app, "Swiftlet: Mac에서 80B Qwen을 4.3GB RAM으로,
           iPhone에서 35B를 돌리는 런타임".
* [lens]   agentlenshq.com, "Swiftletは低RAM使用量でMacとiPhone上で35Bおよび
           80B Qwenモデルを可能にする".

What the pages fix: per layer each token goes to k of E routed experts (10 of
512 for 80B, 8 of 256 for 35B) plus always-resident shared experts, and the
experts are MLX-style affine int4/int8 group-quantised ([xix] paragraphs on
how it works and on lineage; [lens] "エキスパートストリーミングの仕組み" and
"TurboFieldfareとの関係").  The pages print no equations and no worked
example, so every formula here is the plainest reading of those words, and
each reading is stated where it is used:

* affine group quantisation (MLX convention): w = s*q + b per group of
  ``group`` consecutive inputs, q an unsigned ``bits``-bit field, fields packed
  into 32-bit words least-significant first, s and b in bf16;
* router: logits = Wr x + rb, softmax, top-k, weights renormalised over the
  k chosen; shared expert scaled by sigmoid(wsg . x);
* SwiGLU expert: h = silu(Wg x) * (Wu x), y = Wd h; the activation h is held
  in bf16 (the activation dtype, as MLX runs activations);
* combine: y = sum_j w_j y_j + sigma * y_shared.

All arithmetic is float64 unless a step is defined to round to bf16.
Every function is pinned by a CPU test (``tests/test_oracle_*.py``).
"""

from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------- bf16 helpers

def bf16_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    Done directly from float64 (no intermediate float32 rounding): a value
    with exponent e is snapped to the grid 2**(e-7) (8 significant bits),
    with the grid floored at bf16's subnormal spacing 2**-133.  Finite
    inputs within bf16's range only.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    q = np.maximum(e.astype(np.int64) - 8, -133)
    scale = np.ldexp(1.0, q)
    return np.rint(x / scale) * scale       # np.rint: round half to even


def bf16_bits(x) -> np.ndarray:
    """Bit patterns of float64 values that are already exact bf16 values."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------- quantised weights

def unpack_fields(words, bits: int, n_cols: int) -> np.ndarray:
    """Unpack a [out, n_cols*bits/32] uint32 matrix into [out, n_cols] fields.

    Field c of a row sits in word c // (32/bits) at bit offset
    bits * (c mod 32/bits): least-significant field first ([xix] lineage
    paragraph: MLX-style int4/int8 group quantisation).
    """
    per = 32 // bits
    w = np.asarray(words, dtype=np.uint32)
    assert w.shape[-1] * per == n_cols
    shifts = (np.arange(per, dtype=np.uint32) * np.uint32(bits))
    fields = (w[..., :, None] >> shifts) & np.uint32((1 << bits) - 1)
    return fields.reshape(*w.shape[:-1], n_cols).astype(np.int64)


def dequantize(words, s_bits, b_bits, bits: int, group: int) -> np.ndarray:
    """Affine group dequantisation W[r, c] = s[r, c//group] * q[r, c] + b[r, c//group].

    Reading of "MLX-style affine int4/int8 group quantisation" ([xix] lineage
    paragraph; [lens] "TurboFieldfareとの関係"): unsigned q, one bf16 scale
    and one bf16 bias per group of ``group`` consecutive input columns.
    float64; for the workload's value ranges the result is exactly a float32
    value (s*q needs at most 16 significant bits).
    """
    s = bf16_to_f64(s_bits)
    b = bf16_to_f64(b_bits)
    n_cols = s.shape[-1] * group
    q = unpack_fields(words, bits, n_cols).astype(np.float64)
    return q * np.repeat(s, group, axis=-1) + np.repeat(b, group, axis=-1)


# --------------------------------------------------------------------- routing

def softmax(z) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def select_topk(logits, k: int) -> np.ndarray:
    """Indices of the k largest logits, ordered by (logit desc, index asc).

    The pages say only "top-k" ([xix] how-it-works paragraph); equal logits
    go to the lower expert index, which makes the choice unique.
    """
    logits = np.asarray(logits, dtype=np.float64)
    order = np.lexsort((np.arange(logits.shape[-1]), -logits))
    return order[:k].astype(np.int64)


def router_logits(x, Wr, rb) -> np.ndarray:
    """logits[e] = sum_h x[h] * Wr[e, h] + rb[e] (router kept resident, unquantised:
    [xix] how-it-works paragraph lists the routers among the resident dense weights)."""
    return np.asarray(Wr, np.float64) @ np.asarray(x, np.float64) + np.asarray(rb, np.float64)


def route(x, Wr, rb, k: int):
    """Softmax over all E logits, top-k, renormalise over the chosen k.

    Returns (logits, p, idx, w) with w_j = p[idx_j] / sum_i p[idx_i].
    """
    logits = router_logits(x, Wr, rb)
    p = softmax(logits)
    idx = select_topk(logits, k)
    w = p[idx] / p[idx].sum()
    return logits, p, idx, w


# ------------------------------------------------------------------ activations

def sigmoid(z) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def silu(z) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


# ---------------------------------------------------------------------- experts

def dequant_expert(arrays: dict, bits: int, group: int, bf16_weights: bool = False):
    """Dequantise one expert's gate, up and down matrices.

    ``bf16_weights`` rounds each dequantised weight to bf16 (round to nearest
    even), the operand precision of the dequant-to-bf16 matrix-core path used
    for many tokens at once.
    """
    mats = []
    for name in ("gate", "up", "down"):
        W = dequantize(*arrays[name], bits=bits, group=group)
        mats.append(round_bf16(W) if bf16_weights else W)
    return tuple(mats)


def swiglu(x, Wg, Wu, Wd):
    """SwiGLU expert on rows of x: h = bf16(silu(x Wg^T) * (x Wu^T)), y = h Wd^T.

    x: [..., H] float64; returns (y [..., H], h [..., I]).  The activation h
    is rounded to bf16 (reading: activations are held in the bf16 activation
    dtype between the two quantised products).
    """
    x = np.asarray(x, dtype=np.float64)
    g = x @ Wg.T
    u = x @ Wu.T
    h = round_bf16(silu(g) * u)
    return h @ Wd.T, h


# ------------------------------------------------------------------- MoE layer

def moe_layer(x_bits, Wr, rb, wsg, shared: dict, expert_fn, k: int, bits: int,
              group: int = 64, bf16_weights: bool = False) -> dict:
    """One MoE layer for one token.

    x_bits: bf16 bits [H]; shared: the shared expert's arrays; expert_fn(e)
    returns routed expert e's arrays.  Steps (pages: [xix] how-it-works
    paragraph; [lens] "エキスパートストリーミングの仕組み"):

    1. route: logits, softmax, top-k, renormalised weights w;
    2. each chosen expert's SwiGLU output y_j;
    3. shared expert output y_sh scaled by sigma = sigmoid(wsg . x);
    4. y = sum_j w_j y_j + sigma y_sh, summed in j order.
    """
    x = bf16_to_f64(x_bits)
    logits, p, idx, w = route(x, Wr, rb, k)
    y = np.zeros_like(x)
    for j, e in enumerate(idx):
        Wg, Wu, Wd = dequant_expert(expert_fn(int(e)), bits, group, bf16_weights)
        y = y + w[j] * swiglu(x, Wg, Wu, Wd)[0]
    sigma = float(sigmoid(np.dot(np.asarray(wsg, np.float64), x)))
    Wg, Wu, Wd = dequant_expert(shared, bits, group, bf16_weights)
    y = y + sigma * swiglu(x, Wg, Wu, Wd)[0]
    return {"y": y, "idx": idx, "w": w, "logits": logits, "p": p, "sigma": sigma}


def moe_layer_tokens(X_bits, Wr, rb, wsg, shared: dict, expert_fn, k: int,
                     bits: int, group: int = 64, bf16_weights: bool = False,
                     workers: int = 1) -> dict:
    """The same layer for many tokens at once.

    Identical per token to ``moe_layer``; each expert is dequantised once and
    applied (one matrix product) to the rows of the tokens that chose it.
    The combine is still summed per token in j order, then the shared term.
    ``workers`` > 1 runs different experts on a thread pool; each expert's
    arithmetic, and so the result, is unchanged.
    """
    X = bf16_to_f64(X_bits)
    T, H = X.shape
    logits = X @ np.asarray(Wr, np.float64).T + np.asarray(rb, np.float64)
    idx = np.zeros((T, k), dtype=np.int64)
    w = np.zeros((T, k))
    for t in range(T):
        p = softmax(logits[t])
        idx[t] = select_topk(logits[t], k)
        w[t] = p[idx[t]] / p[idx[t]].sum()
    Yj = np.zeros((T, k, H))

    def one_expert(e):
        rows, slots = np.nonzero(idx == e)
        Wg, Wu, Wd = dequant_expert(expert_fn(int(e)), bits, group, bf16_weights)
        Yj[rows, slots] = swiglu(X[rows], Wg, Wu, Wd)[0]

    if workers > 1:
        # one BLAS thread per worker: concurrent multi-threaded BLAS calls
        # would queue on each other
        from concurrent.futures import ThreadPoolExecutor
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(workers) as ex:
            list(ex.map(one_expert, np.unique(idx)))
    else:
        for e in np.unique(idx):
            one_expert(e)
    sigma = sigmoid(X @ np.asarray(wsg, np.float64))
    Wg, Wu, Wd = dequant_expert(shared, bits, group, bf16_weights)
    ysh = swiglu(X, Wg, Wu, Wd)[0]
    y = np.zeros((T, H))
    for j in range(k):
        y = y + w[:, j:j + 1] * Yj[:, j]
    y = y + sigma[:, None] * ysh
    return {"y": y, "idx": idx, "w": w, "logits": logits, "sigma": sigma}


# ------------------------------------------------- grouping rows by expert

def sort_by_expert(idx, E: int):
    """Group the (token, choice) pairs of a routed batch by expert.

    Routing sends each token to k experts ([xix] how-it-works paragraph;
    [lens] "エキスパートストリーミングの仕組み"); to run each expert once on
    all its tokens, the pairs are grouped by expert.  Pair p = t*k + j is the
    j-th choice of token t.  Counting sort: count the pairs per expert, turn
    the counts into first rows (exclusive prefix sums), then walk the pairs
    in order p = 0, 1, ... and put each at its expert's next free row, so
    an expert's rows keep (token, choice) order (reading: the pages give no
    order; this one makes the grouping unique).

    Returns (perm, offsets): perm[r] = the pair in row r, int64 [T*k];
    offsets[e] = first row of expert e, offsets[E] = T*k, int64 [E+1].
    Pairs whose expert lies outside [0, E) are left out (and offsets[E]
    counts only the others).
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = [0] * E
    for e in flat.tolist():
        if 0 <= e < E:
            counts[e] += 1
    offsets = [0] * (E + 1)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:E]
    perm = [0] * offsets[E]
    for p, e in enumerate(flat.tolist()):
        if 0 <= e < E:
            perm[cursor[e]] = p
            cursor[e] += 1
    return np.asarray(perm, dtype=np.int64), np.asarray(offsets, dtype=np.int64)


# ------------------------------------------------------ stacked-layer rescale

def rms_rescale(y_f32) -> np.ndarray:
    """Next layer's input in a stack of MoE layers: bf16(y / sqrt(mean(y^2) + 1e-6)).

    The pages stack MoE layers inside a full model whose residual and norm
    layers are out of scope; this weightless RMS rescale stands in for them
    and keeps activations at unit scale.  Computed in float32 from the
    float32 layer output, as the stated precision of the chained activation.
    """
    y = np.asarray(y_f32, dtype=np.float32)
    ms = np.float32(np.mean(y.astype(np.float64) ** 2))
    r = np.float32(1.0) / np.sqrt(ms + np.float32(1e-6))
    return bf16_bits(round_bf16((y * r).astype(np.float64)))
