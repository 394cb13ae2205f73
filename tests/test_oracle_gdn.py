"""Pins of the Gated DeltaNet decode-step oracle (CPU).

The pages name the layer type but print no recurrence, so the oracle is
pinned to what the published gated delta rule itself fixes, each test
written from the property, not from the oracle's formula:

* beta = 0 writes nothing: the state only decays by alpha;
* alpha = beta = 1 with a unit key: the new state maps that key to exactly
  its value (the delta rule replaces the value stored under the key);
* writes along orthonormal keys build an associative memory S = sum v_i k_i^T
  that returns every stored value;
* the update equals the matrix form S alpha (I - beta k k^T) + beta v k^T;
* grouped heads, batch independence, and the normalisation of q and k.
"""

import numpy as np
import pytest

from oracle.gdn_oracle import gdn_step, l2_normalise

RNG = np.random.default_rng(1234)


def _rand(B=2, Hk=2, Hv=4, dk=8, dv=6):
    S = RNG.standard_normal((B, Hv, dv, dk))
    q = RNG.standard_normal((B, Hk, dk))
    k = RNG.standard_normal((B, Hk, dk))
    v = RNG.standard_normal((B, Hv, dv))
    alpha = RNG.uniform(0.5, 1.0, (B, Hv))
    beta = RNG.uniform(0.0, 1.0, (B, Hv))
    return S, q, k, v, alpha, beta


def test_beta_zero_only_decays():
    S, q, k, v, alpha, _ = _rand()
    beta = np.zeros_like(alpha)
    S1, o = gdn_step(S, q, k, v, alpha, beta, 0.5, 1e-6)
    assert np.allclose(S1, alpha[:, :, None, None] * S, rtol=0, atol=1e-14)
    # o = scale * (alpha S) q^, with q^ computed here by hand
    for b in range(S.shape[0]):
        for h in range(S.shape[1]):
            qh = q[b, h // 2] / np.sqrt(np.dot(q[b, h // 2], q[b, h // 2]) + 1e-6)
            assert np.allclose(o[b, h], 0.5 * alpha[b, h] * S[b, h].dot(qh), atol=1e-13)


def test_unit_key_full_write_stores_value_exactly():
    S, q, k, v, alpha, beta = _rand(B=3, Hk=1, Hv=3, dk=16, dv=5)
    k = k / np.linalg.norm(k, axis=-1, keepdims=True)   # unit keys, eps = 0
    S1, _ = gdn_step(S, q, k, v, np.ones_like(alpha), np.ones_like(beta), 1.0, 0.0)
    for b in range(3):
        for h in range(3):
            assert np.allclose(S1[b, h] @ k[b, 0], v[b, h], rtol=0, atol=1e-12)
            # and the state is unchanged on keys orthogonal to k
            z = RNG.standard_normal(16)
            z -= z.dot(k[b, 0]) * k[b, 0]
            assert np.allclose(S1[b, h] @ z, S[b, h] @ z, atol=1e-12)


def test_orthonormal_writes_form_an_associative_memory():
    dk, dv, n = 8, 4, 5
    basis = np.linalg.qr(RNG.standard_normal((dk, dk)))[0][:, :n].T  # n orthonormal keys
    vals = RNG.standard_normal((n, dv))
    S = np.zeros((1, 1, dv, dk))
    for i in range(n):
        S, _ = gdn_step(S, basis[None, i:i + 1], basis[None, i:i + 1], vals[None, i:i + 1],
                        np.ones((1, 1)), np.ones((1, 1)), 1.0, 0.0)
    want = sum(np.outer(vals[i], basis[i]) for i in range(n))
    assert np.allclose(S[0, 0], want, atol=1e-12)
    for i in range(n):
        _, o = gdn_step(S, basis[None, i:i + 1], basis[None, i:i + 1], np.zeros((1, 1, dv)),
                        np.ones((1, 1)), np.zeros((1, 1)), 1.0, 0.0)
        assert np.allclose(o[0, 0], vals[i], atol=1e-12)   # reading with beta = 0


def test_matches_matrix_form():
    S, q, k, v, alpha, beta = _rand(B=2, Hk=2, Hv=2, dk=7, dv=3)
    eps = 1e-3
    S1, o = gdn_step(S, q, k, v, alpha, beta, 0.25, eps)
    for b in range(2):
        for h in range(2):
            kn = k[b, h] / np.sqrt(np.sum(k[b, h] ** 2) + eps)
            qn = q[b, h] / np.sqrt(np.sum(q[b, h] ** 2) + eps)
            M = alpha[b, h] * (np.eye(7) - beta[b, h] * np.outer(kn, kn))
            want = S[b, h].dot(M) + beta[b, h] * np.outer(v[b, h], kn)
            assert np.allclose(S1[b, h], want, atol=1e-12)
            assert np.allclose(o[b, h], 0.25 * want.dot(qn), atol=1e-12)


def test_grouped_heads_and_batch_independence():
    S, q, k, v, alpha, beta = _rand(B=2, Hk=2, Hv=6, dk=4, dv=3)
    S1, o = gdn_step(S, q, k, v, alpha, beta, 1.0, 1e-6)
    for b in range(2):
        for h in range(6):
            # value head h reads key head h // 3; alone in a batch of one
            s1, o1 = gdn_step(S[b:b + 1, h:h + 1], q[b:b + 1, h // 3:h // 3 + 1],
                              k[b:b + 1, h // 3:h // 3 + 1], v[b:b + 1, h:h + 1],
                              alpha[b:b + 1, h:h + 1], beta[b:b + 1, h:h + 1], 1.0, 1e-6)
            assert np.array_equal(s1[0, 0], S1[b, h]) and np.array_equal(o1[0, 0], o[b, h])


def test_normalisation():
    x = np.array([[3.0, 4.0], [0.0, 0.0]])
    n = l2_normalise(x, 0.0 + 1e-300)
    assert np.allclose(n[0], [0.6, 0.8], atol=1e-15)
    assert np.all(n[1] == 0.0)                       # a zero key stays zero
    # a zero key with eps > 0 writes nothing: S <- alpha S
    S, q, k, v, alpha, beta = _rand(B=1, Hk=1, Hv=1, dk=4, dv=2)
    S1, _ = gdn_step(S, q, np.zeros_like(k), v, alpha, beta, 1.0, 1e-6)
    assert np.allclose(S1, alpha[0, 0] * S, atol=1e-15)


@pytest.mark.parametrize("scale", [1.0, 0.125])
def test_output_is_linear_in_scale_and_uses_updated_state(scale):
    S, q, k, v, alpha, beta = _rand(B=1, Hk=1, Hv=1, dk=5, dv=5)
    S1, o = gdn_step(S, q, k, v, alpha, beta, scale, 1e-6)
    _, o_read = gdn_step(S1, q, k, np.zeros_like(v), np.ones_like(alpha), np.zeros_like(beta),
                         scale, 1e-6)
    assert np.allclose(o, o_read, atol=1e-13)
