"""Seeded draws for every input of the MoE layer (see ``configs`` for the key scheme).

Arrays are returned in the canonical, layout-free form both sides consume:

* a quantised matrix [out, in] is ``(words, s, b)``: ``words`` uint32
  [out, in*bits/32] holding the packed unsigned fields, ``s`` and ``b`` bf16
  bit patterns (uint16) [out, in/group] for the per-group scale and bias;
* router weights ``Wr`` float32 [E, H], bias ``rb`` float32 [E], shared-gate
  vector ``wsg`` float32 [H];
* tokens as bf16 bit patterns (uint16) [H].

The only arithmetic here turns random draws into stored values (bf16
rounding of the drawn scales and biases).  Nothing of the layer is computed.
"""

from __future__ import annotations

import numpy as np

from .configs import MoEConfig


def bf16_bits_from_f32(a) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def _bf16_bits_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _quant_matrix(rng: np.random.Generator, cfg: MoEConfig, out: int, inn: int):
    per = 32 // cfg.bits
    ng = inn // cfg.group
    words = rng.integers(0, 1 << 32, size=(out, inn // per), dtype=np.uint32)
    s = bf16_bits_from_f32(rng.uniform(cfg.scale_lo, cfg.scale_hi, size=(out, ng)))
    b_val = cfg.bias_offset * _bf16_bits_to_f64(s)
    if cfg.bias_noise > 0.0:
        b_val = b_val + rng.normal(0.0, cfg.bias_noise, size=(out, ng))
    b = bf16_bits_from_f32(b_val.astype(np.float32))
    return words, s, b


def _expert(rng: np.random.Generator, cfg: MoEConfig, inter: int) -> dict:
    H = cfg.hidden
    return {
        "gate": _quant_matrix(rng, cfg, inter, H),
        "up": _quant_matrix(rng, cfg, inter, H),
        "down": _quant_matrix(rng, cfg, H, inter),
    }


def expert_arrays(cfg: MoEConfig, layer: int, expert: int) -> dict:
    """Routed expert (layer, expert): {'gate','up','down'} -> (words, s, b)."""
    rng = np.random.default_rng((cfg.seed, 1, layer, expert))
    return _expert(rng, cfg, cfg.inter)


def shared_arrays(cfg: MoEConfig, layer: int) -> dict:
    """Shared expert of a layer, same format and bit width as the routed ones."""
    rng = np.random.default_rng((cfg.seed, 2, layer))
    return _expert(rng, cfg, cfg.shared_inter)


def router_arrays(cfg: MoEConfig, layer: int):
    """Return (Wr f32 [E,H], rb f32 [E], wsg f32 [H]) for one layer.

    With a Zipf exponent z, expert e gets the bias -z*ln(rank_e), where the
    ranks 1..E follow a seeded permutation; otherwise the bias is zero.
    """
    E, H = cfg.experts, cfg.hidden
    rng = np.random.default_rng((cfg.seed, 3, layer))
    Wr = rng.normal(0.0, cfg.router_std, size=(E, H)).astype(np.float32)
    wsg = rng.normal(0.0, cfg.router_std, size=H).astype(np.float32)
    if cfg.zipf:
        perm = np.random.default_rng((cfg.seed, 4, layer)).permutation(E)
        rank = np.empty(E, dtype=np.float64)
        rank[perm] = np.arange(1, E + 1, dtype=np.float64)
        rb = (-cfg.zipf * np.log(rank)).astype(np.float32)
    else:
        rb = np.zeros(E, dtype=np.float32)
    return Wr, rb, wsg


def token_x(cfg: MoEConfig, t: int) -> np.ndarray:
    """Token t's layer-0 input: H draws of N(0,1) rounded to bf16 (uint16 bits)."""
    rng = np.random.default_rng((cfg.seed, 5, t))
    return bf16_bits_from_f32(rng.standard_normal(cfg.hidden).astype(np.float32))


def tokens_x(cfg: MoEConfig, t0: int, n: int) -> np.ndarray:
    return np.stack([token_x(cfg, t) for t in range(t0, t0 + n)]) if n else \
        np.zeros((0, cfg.hidden), dtype=np.uint16)


def gdn_inputs(seed: int, B: int, Hk: int, Hv: int, dk: int, dv: int, T: int) -> dict:
    """Seeded inputs of T consecutive Gated DeltaNet decode steps for B
    sequences: q, k [T][B][Hk][dk] and v [T][B][Hv][dv] as bf16 bits of
    N(0, 1) draws; decay alpha [T][B][Hv] ~ U(0.9, 1) and write strength
    beta ~ U(0, 1) as f32; an initial state S0 [B][Hv][dv][dk] ~ N(0, 0.1^2)
    as f32."""
    rng = np.random.default_rng((seed, 6, B, Hk, Hv, dk, dv, T))
    f32 = np.float32
    return {
        "q": bf16_bits_from_f32(rng.standard_normal((T, B, Hk, dk)).astype(f32)),
        "k": bf16_bits_from_f32(rng.standard_normal((T, B, Hk, dk)).astype(f32)),
        "v": bf16_bits_from_f32(rng.standard_normal((T, B, Hv, dv)).astype(f32)),
        "alpha": rng.uniform(0.9, 1.0, (T, B, Hv)).astype(f32),
        "beta": rng.uniform(0.0, 1.0, (T, B, Hv)).astype(f32),
        "S0": (0.1 * rng.standard_normal((B, Hv, dv, dk))).astype(f32),
    }
