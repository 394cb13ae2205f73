"""CPU oracle for one Gated DeltaNet recurrent decode step (NumPy, float64).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library
never calls it and shares no code with it; the two meet only in the seeded
inputs of ``moe_inputs.gdn_inputs``.

What the pages fix: three of every four layers of the hybrid stack use
Gated DeltaNet linear attention, whose recurrent state has a fixed size, so
no KV cache grows with the context ([xix] paragraph on Metal and DeltaNet;
[lens] "エキスパートストリーミングの仕組み"; the DeltaNet projections are
among the resident dense weights, [xix] how-it-works paragraph).  The pages
print no recurrence.  This module takes the gated delta rule as published
for Gated DeltaNet (a decaying, delta-rule-updated associative memory) and
states every reading where it is used:

* per value head, a state S of shape [dv, dk] (maps a key to a value);
* the key and query of a token are L2-normalised:
  k^ = k / sqrt(|k|^2 + eps), q^ = q / sqrt(|q|^2 + eps);
* update with decay alpha in (0, 1] and write strength beta in [0, 1]:
  S <- alpha * (S - beta * (S k^) k^T) + beta * v k^T,
  i.e. S <- S * alpha (I - beta k^ k^T) + beta v k^T;
* output o = scale * S q^ with the updated state;
* grouped heads: value head h reads key / query head h // (Hv / Hk).

alpha and beta are inputs (the model derives them from its own gate
projections, which are not part of this step).  Pinned by
``tests/test_oracle_gdn.py`` against the delta rule's defining properties
(decay only at beta = 0; with alpha = beta = 1 and a unit key the new state
maps the key to its value; writes along orthonormal keys form an
associative memory), an explicit matrix form and the head grouping.
"""

from __future__ import annotations

import numpy as np

from .moe_oracle import bf16_to_f64


def l2_normalise(x, eps: float) -> np.ndarray:
    """x / sqrt(|x|^2 + eps) along the last axis (float64)."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def gdn_step(S, q, k, v, alpha, beta, scale: float, eps: float):
    """One token for every sequence and value head.

    S: [B, Hv, dv, dk] float64 (not modified); q, k: [B, Hk, dk]; v: [B, Hv,
    dv]; alpha, beta: [B, Hv].  Returns (S_new, o) with o: [B, Hv, dv]."""
    S = np.asarray(S, np.float64)
    B, Hv, dv, dk = S.shape
    Hk = np.asarray(k).shape[1]
    assert Hv % Hk == 0
    g = Hv // Hk
    kn = l2_normalise(k, eps)
    qn = l2_normalise(q, eps)
    v = np.asarray(v, np.float64)
    S_new = np.empty_like(S)
    o = np.empty((B, Hv, dv))
    for b in range(B):
        for h in range(Hv):
            kh, qh = kn[b, h // g], qn[b, h // g]
            a, be = float(alpha[b, h]), float(beta[b, h])
            sk = S[b, h] @ kh                                   # S k^      [dv]
            Sn = a * (S[b, h] - be * np.outer(sk, kh)) + be * np.outer(v[b, h], kh)
            S_new[b, h] = Sn
            o[b, h] = scale * (Sn @ qh)
    return S_new, o


def gdn_step_bf16(S, q_bits, k_bits, v_bits, alpha, beta, scale: float, eps: float):
    """gdn_step on bf16 activations given as their bit patterns (widened
    exactly); alpha, beta and the state are f32 values widened to f64."""
    return gdn_step(S, bf16_to_f64(q_bits), bf16_to_f64(k_bits), bf16_to_f64(v_bits),
                    np.asarray(alpha, np.float64), np.asarray(beta, np.float64), scale, eps)
