"""The MoE-layer workloads (shapes of the layers the source pages describe).

Sizes follow the pages' running examples: 64 experts with top-2 ([mlqm] §2.2, [wmrh]
§2.2), hidden width 4096 ([mlqm] §3.1), 16 routed experts plus one shared expert
([200B-5] "共享专家…"), capacity (T*k)/E ([rkmt] §2.3), a tiny GeLU layer like the
pages' teaching code ([rkmt] §3.3, [wmrh] §5.1).
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    seed: int
    T: int              # tokens
    d: int              # model width
    E: int              # routed experts
    k: int              # experts per token
    F: int              # expert hidden width
    act: str            # "gelu" | "swiglu"
    dtype: str          # "f32" | "bf16": activations and weights
    shared: bool = False    # one always-on shared expert
    capacity: int = 0       # per-expert capacity, 0 = unlimited
    bias_var: float = 0.0   # variance of the per-expert router offsets, 0 = no offsets
    weights: str = "renormalized"   # "renormalized" | "softmax": routing-weight formulation
    priority: str = "token"         # "token" | "slot": order in which slots claim capacity
    overflow: str = "drop"          # "drop" | "reroute": fate of a slot beyond capacity

    def scaled(self, **kw) -> "MoEConfig":
        return replace(self, **kw)

    @property
    def label(self) -> str:
        return (f"{self.name}(T={self.T},d={self.d},E={self.E}{'+1' if self.shared else ''},"
                f"k={self.k},F={self.F},{self.act},{self.dtype}"
                f"{',C=%d' % self.capacity if self.capacity else ''}"
                f"{',w=' + self.weights if self.weights != 'renormalized' else ''}"
                f"{',' + self.priority + '-major' if self.priority != 'token' else ''}"
                f"{',' + self.overflow if self.overflow != 'drop' else ''})")


CONFIGS = {
    1: MoEConfig("tiny-gelu-f32", 1, T=64, d=64, E=4, k=2, F=128, act="gelu", dtype="f32"),
    2: MoEConfig("prefill-e64", 2, T=4096, d=4096, E=64, k=2, F=14336, act="swiglu", dtype="bf16"),
    3: MoEConfig("shared-routed-e16", 3, T=8192, d=4096, E=16, k=2, F=14336, act="swiglu",
                 dtype="bf16", shared=True, bias_var=0.5),
    4: MoEConfig("capacity-e16", 4, T=1024, d=4096, E=16, k=2, F=14336, act="swiglu",
                 dtype="bf16", capacity=128, bias_var=1.0),
    5: MoEConfig("decode-e64", 5, T=16, d=4096, E=64, k=2, F=14336, act="swiglu", dtype="bf16"),
    # wider routing shapes: 384 routed experts, 6 per token, one shared expert ([200B-5]
    # closing section's recent-model example) and 128 experts top-2 (the MoE-128 option of
    # the expert-count comparison on the first page); the pages give no widths for them,
    # so d and F stay those of the other workloads
    6: MoEConfig("wide-e384-top6-shared", 6, T=4096, d=4096, E=384, k=6, F=14336, act="swiglu", dtype="bf16",
                 shared=True),
    7: MoEConfig("wide-e128-top2", 7, T=4096, d=4096, E=128, k=2, F=14336, act="swiglu", dtype="bf16"),
    # the capacity-limited layer in the drop regime its description aims at (5-20% of the
    # slots dropped): offsets drawn literally from N(0, 1) drop about 41% of the slots at
    # C = 128 ([rkmt] §2.3 sets its alarm at a 5% drop rate), so this variant draws them
    # with standard deviation 0.15 (variance 0.0225), which drops 13.8% of the slots with
    # its seed and the inputs drawn on the GPU (std 0.1 / 0.2 / 0.25: 10.4% / 17.7% / 21.7%)
    8: MoEConfig("capacity-e16-calibrated", 8, T=1024, d=4096, E=16, k=2, F=14336, act="swiglu",
                 dtype="bf16", capacity=128, bias_var=0.0225),
}

# the workloads by name
BY_NAME = {c.name: c for c in CONFIGS.values()}
