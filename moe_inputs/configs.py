"""Workload shapes for the synthetic Qwen-shaped MoE layers.

Expert counts and top-k follow the routing facts stated on the pages:
each layer routes a token to 10 of 512 experts in the 80B-A3B model and to
8 of 256 in the 35B-A3B model (xix.ai, "Swiftlet Packs 80B Qwen Into Mac With
4.3GB Memory; iPhone 17 to Run 35B Natively", paragraph on how it works;
agentlenshq, "エキスパートストリーミングの仕組み").  Hidden size 2048, expert
intermediate 512, group 64 and the value distributions are the synthetic
workload definitions; the pages give none of them.

Draw order (every draw uses ``numpy.random.default_rng`` keyed by a tuple so
any expert, router or token can be regenerated on its own):

* routed expert (layer l, expert e): key ``(seed, 1, l, e)``; for gate, up,
  down in that order: packed words, then scale uniforms, then (int4 only)
  bias noise.
* shared expert of layer l: key ``(seed, 2, l)``, same order.
* router of layer l: key ``(seed, 3, l)``: ``Wr`` [E, H] then ``wsg`` [H].
* Zipf routing bias of layer l: key ``(seed, 4, l)``: one permutation of E.
* token t: key ``(seed, 5, t)``: H standard normals.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class MoEConfig:
    name: str
    layers: int
    hidden: int            # H
    experts: int           # E
    top_k: int             # k
    inter: int             # I, routed-expert intermediate size
    shared_inter: int      # Is, shared-expert intermediate size
    bits: int              # 4 or 8
    tokens: int            # tokens in the workload
    batch: int             # tokens per decode step (T)
    zipf: Optional[float]  # exponent of the per-expert routing bias, or None
    scale_lo: float
    scale_hi: float
    bias_noise: float      # std of the N(0, .) added to the int4 bias; 0 for int8
    pool_frac: Optional[float] = None  # HBM slot pool size as a fraction of L*E
    resident: bool = True
    group: int = 64
    router_std: float = 0.02
    seed: int = 0

    @property
    def bias_offset(self) -> float:
        """Zero point folded into the bias: -8*scale (int4), -128*scale (int8)."""
        return -float(1 << (self.bits - 1))

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


_INT4 = dict(bits=4, scale_lo=0.005, scale_hi=0.02, bias_noise=1e-3)
_INT8 = dict(bits=8, scale_lo=0.0003, scale_hi=0.0012, bias_noise=0.0)

CONFIGS = {
    # Tiny layer: 16 experts, top-2, 8 tokens, all resident.
    "tiny": MoEConfig(name="tiny", layers=1, hidden=256, experts=16, top_k=2,
                      inter=64, shared_inter=64, tokens=8, batch=8, zipf=None,
                      **_INT4),
    # 35B-A3B-shaped decode: 40 stacked layers, 256 of 8, batch 1, resident.
    "decode35b": MoEConfig(name="decode35b", layers=40, hidden=2048, experts=256,
                           top_k=8, inter=512, shared_inter=512, tokens=256,
                           batch=1, zipf=1.1, **_INT4),
    # 80B-A3B-shaped decode with a 30% HBM slot pool over a pinned-host store.
    "stream80b": MoEConfig(name="stream80b", layers=48, hidden=2048, experts=512,
                           top_k=10, inter=512, shared_inter=512, tokens=512,
                           batch=1, zipf=1.1, pool_frac=0.3, resident=False,
                           **_INT4),
    # The same 80B-A3B-shaped int4 stack with every expert resident in HBM
    # (same seeded weights as stream80b).
    "decode80b": MoEConfig(name="decode80b", layers=48, hidden=2048, experts=512,
                           top_k=10, inter=512, shared_inter=512, tokens=512,
                           batch=1, zipf=1.1, **_INT4),
    # 80B-A3B-shaped decode, int8 experts, all resident; batch 1 and batch 8.
    "decode80b_int8": MoEConfig(name="decode80b_int8", layers=48, hidden=2048,
                                experts=512, top_k=10, inter=512,
                                shared_inter=512, tokens=512, batch=1,
                                zipf=1.1, **_INT8),
    # 80B-A3B-shaped prefill: one layer, 4096 tokens, no routing bias.
    "prefill80b": MoEConfig(name="prefill80b", layers=1, hidden=2048,
                            experts=512, top_k=10, inter=512, shared_inter=512,
                            tokens=4096, batch=4096, zipf=None, **_INT4),
}


def get_config(name: str) -> MoEConfig:
    return CONFIGS[name]


# Gated DeltaNet recurrent decode step shapes (value heads Hv, key heads Hk,
# head dims dk = dv): the 80B-A3B model's linear-attention layers, and a
# small one for tests.  B = sequences decoded together.
GDN_CONFIGS = {
    "gdn_tiny": {"B": 3, "Hk": 2, "Hv": 4, "dk": 64, "dv": 64},
    "gdn80b": {"B": 64, "Hk": 16, "Hv": 32, "dk": 128, "dv": 128},
}
