"""Seeded synthetic inputs for the MoE layer (no arithmetic of the method lives here).

Recipe: hidden states ~ N(0, 1); router weights W_r ~ N(0, 1/d); expert gate/up
weights ~ N(0, 1/d) and down weights ~ N(0, 1/F) (fan-in variance); router offsets
~ N(0, bias_var) in fp32.  The shared expert uses the same recipe.  Every tensor (and
every expert of a stacked tensor) has its own seed derived from (config seed, tensor
tag, expert), so any expert can be regenerated alone.  Values are drawn in fp32 with
``torch.randn`` on the requested device and, for bf16 layers, rounded to nearest-even.

The same tensors are handed to the GPU library and (copied to the host) to the CPU
oracle, so both sides consume identical bits.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
import torch

from .configs import MoEConfig

_TAGS = {"x": 1, "w_r": 2, "bias": 3, "w_gate": 4, "w_up": 5, "w_down": 6,
         "s_gate": 7, "s_up": 8, "s_down": 9}


def seed_of(cfg_seed: int, tag: str, expert: int = 0) -> int:
    return int(np.random.SeedSequence([cfg_seed, _TAGS[tag], expert]).generate_state(1, np.uint64)[0]
               & 0x7FFF_FFFF_FFFF_FFFF)


def _dtype(cfg: MoEConfig):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def normal(shape, std: float, seed: int, device, dtype) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    return v.to(dtype)


def expert_weights(cfg: MoEConfig, e: int, device="cpu", shared: bool = False):
    """(w_gate [F,d], w_up [F,d] or None, w_down [d,F]) of routed expert e or the shared one."""
    dt = _dtype(cfg)
    pre = "s_" if shared else "w_"
    wg = normal((cfg.F, cfg.d), 1 / math.sqrt(cfg.d), seed_of(cfg.seed, pre + "gate", e), device, dt)
    wu = (normal((cfg.F, cfg.d), 1 / math.sqrt(cfg.d), seed_of(cfg.seed, pre + "up", e), device, dt)
          if cfg.act == "swiglu" else None)
    wd = normal((cfg.d, cfg.F), 1 / math.sqrt(cfg.F), seed_of(cfg.seed, pre + "down", e), device, dt)
    return wg, wu, wd


def make_inputs(cfg: MoEConfig, device="cpu") -> Dict[str, Optional[torch.Tensor]]:
    """All inputs of one layer, on ``device``: x [T,d], w_r [d,E], bias [E] f32 or None,
    w_gate/w_up [E,F,d], w_down [E,d,F], and s_gate/s_up/s_down for a shared expert."""
    dt = _dtype(cfg)
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = normal((cfg.T, cfg.d), 1.0, seed_of(cfg.seed, "x"), device, dt)
    out["w_r"] = normal((cfg.d, cfg.E), 1 / math.sqrt(cfg.d), seed_of(cfg.seed, "w_r"), device, dt)
    out["bias"] = (normal((cfg.E,), math.sqrt(cfg.bias_var), seed_of(cfg.seed, "bias"), device, torch.float32)
                   if cfg.bias_var > 0 else None)
    wg = torch.empty((cfg.E, cfg.F, cfg.d), device=device, dtype=dt)
    wu = torch.empty((cfg.E, cfg.F, cfg.d), device=device, dtype=dt) if cfg.act == "swiglu" else None
    wd = torch.empty((cfg.E, cfg.d, cfg.F), device=device, dtype=dt)
    for e in range(cfg.E):
        g, u, dn = expert_weights(cfg, e, device)
        wg[e].copy_(g)
        if wu is not None:
            wu[e].copy_(u)
        wd[e].copy_(dn)
        del g, u, dn
    out["w_gate"], out["w_up"], out["w_down"] = wg, wu, wd
    if cfg.shared:
        out["s_gate"], out["s_up"], out["s_down"] = expert_weights(cfg, 0, device, shared=True)
    else:
        out["s_gate"] = out["s_up"] = out["s_down"] = None
    return out


def to_numpy(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Host float64 copy (exact for bf16 and fp32 values)."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()


def tie_router_inputs(T: int, d: int, E: int, seed: int, dtype=torch.bfloat16, offsets: bool = True):
    """Router inputs whose logits tie exactly, on any summation order.

    Every hidden state is one-hot (a single 1.0 in a random column r_t), so token t's
    logit for expert e is the single product W_r[r_t, e] (plus the offset b[e]); all other
    terms are exact zeros.  W_r entries are multiples of 1/4 drawn from 3 to 9 levels per
    row, the offsets multiples of 1/4 in [-1/2, 1/2]: sums are exact in fp32, and with so
    few levels many experts share the largest logits, so ties fall inside the top-k and
    across the k-th / (k+1)-th boundary.  Some zero entries are negative zeros.
    Returns (x [T, d], w_r [d, E], bias [E] fp32 or None) as CPU tensors of `dtype`."""
    rng = np.random.default_rng(seed)
    x = np.zeros((T, d), np.float32)
    x[np.arange(T), rng.integers(0, d, size=T)] = 1.0
    lev = rng.integers(1, 5, size=(d, 1))
    w = (rng.integers(-4, 5, size=(d, E)) % (2 * lev + 1) - lev).astype(np.float32) / 4.0
    w[(w == 0) & (rng.random((d, E)) < 0.5)] = -0.0
    b = None
    if offsets:
        b = rng.integers(-2, 3, size=E).astype(np.float32) / 4.0
        b[(b == 0) & (rng.random(E) < 0.5)] = -0.0
        b = torch.from_numpy(b)
    return torch.from_numpy(x).to(dtype), torch.from_numpy(w).to(dtype), b


def tie_logits(T: int, E: int, seed: int, skew: float = 0.0) -> torch.Tensor:
    """fp32 logits [T, E] with exact ties: integers in [-2, 2] (a quarter of the zeros
    negative zeros), plus an optional per-expert integer skew rounded from
    skew * (E - 1 - e) / E so that a few experts overflow their capacity."""
    rng = np.random.default_rng(seed)
    z = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    if skew:
        z += np.round(skew * (E - 1 - np.arange(E)) / E).astype(np.float32)[None, :]
    z[(z == 0) & (rng.random((T, E)) < 0.25)] = -0.0
    return torch.from_numpy(z)
