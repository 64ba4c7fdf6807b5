"""Shared helpers of the GPU parity tests: run the HIP layer, compare with the oracle.

Comparison rules (stage-wise and teacher-forced, so one near-tie flip cannot cascade):
  * route: logits within 1e-4 relative (bf16 inputs; 1e-5 for fp32).  The top-k stage
    on the GPU's own fp32 logits is bit-exact on EVERY token, slot order included: the
    GPU's selection equals the oracle's selection rule applied to the GPU's logits, so
    an exact tie must go to the lowest index with no margin excuse; its weights match
    the oracle's weights of those logits within 1e-5.  Against the oracle's own logits:
    on every token whose fp32 logit row equals the oracle's bit for bit (-0 == +0) the
    selection must be the oracle's, whatever its margin; elsewhere the selected set must
    equal the oracle's where the k-th vs (k+1)-th oracle logit margin exceeds 1e-4 (flips
    below it, which come from a different fp32 summation order, are counted and
    reported); slot order must match wherever every gap inside the top-k exceeds 1e-4;
    weights within 1e-5 absolute of the oracle's weights of the GPU's selection.
  * dispatch: the oracle's dispatch of the GPU's own selection, bit-exact.
  * expert FFN + combine: the oracle's FFN and combine on the GPU's selection and the
    oracle's weights for it; max |out - ref| <= tol * RMS(ref) with tol = 1e-4 (fp32
    layers) or 2e-2 (bf16 layers).  RMS is taken over the tokens that received any
    expert output (kept slot or shared expert); fully dropped tokens must be exactly 0.
    The layer output is fp32 (the accumulator, rounded once).  With a bf16 output the
    reference's own rounding to bf16 is added: |out - ref| <= tol*RMS + half a bf16
    ulp of ref, elementwise.
"""
from __future__ import annotations

import math
import sys
from typing import Dict, Optional

import numpy as np
import torch

from oracle import moe_oracle as O
from sparse_mixture_experts_27_amd import binding as B
from sparse_mixture_experts_27_amd import synth

MARGIN = 1e-4
TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def layer_for(cfg, inp, out_dtype=torch.float32, packed=False, tile=None):
    return B.Layer(inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.k, act=cfg.act,
                   bias=inp["bias"], capacity=cfg.capacity, s_gate=inp["s_gate"], s_up=inp["s_up"],
                   s_down=inp["s_down"], out_dtype=out_dtype, weights=cfg.weights, priority=cfg.priority,
                   overflow=cfg.overflow, packed=packed, tile=tile)


def half_ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |v| (8 significant bits): 2^(e-8) for |v| in [2^e, 2^(e+1))."""
    _, ex = np.frexp(np.abs(v))
    return np.where(v == 0, 0.0, np.ldexp(1.0, ex - 9))


def run_layer(cfg, inp, out_dtype=torch.float32, packed=False, tile=None) -> Dict[str, np.ndarray]:
    L = layer_for(cfg, inp, out_dtype, packed, tile)
    out = L(inp["x"])
    torch.cuda.synchronize()
    res = dict(out=out.float().cpu().numpy().astype(np.float64),
               idx=L.topk_idx.cpu().numpy().astype(np.int64),
               w=L.topk_w.cpu().numpy().astype(np.float64),
               logits=L.logits.cpu().numpy(),
               counts=L.counts.cpu().numpy().astype(np.int64),
               offsets=L.offsets.cpu().numpy().astype(np.int64),
               perm=L.perm.cpu().numpy().astype(np.int64),
               inv=L.inv.cpu().numpy().astype(np.int64),
               n_dropped=int(L.n_dropped.cpu().item()))
    return res


def expert_fetcher(cfg, inp):
    """expert e -> float64 host copies of its weights (fetched on demand, cached)."""
    cache = {}

    def get(e):
        if e not in cache:
            cache.clear()
            wu = inp["w_up"]
            cache[e] = (synth.to_numpy(inp["w_gate"][e]), None if wu is None else synth.to_numpy(wu[e]),
                        synth.to_numpy(inp["w_down"][e]))
        return cache[e]
    return get


def shared_weights(inp):
    if inp["s_gate"] is None:
        return None
    return (synth.to_numpy(inp["s_gate"]), synth.to_numpy(inp["s_up"]), synth.to_numpy(inp["s_down"]))


def check_route(cfg, x64, w_r64, bias64, res, report: dict):
    z_o = O.router_logits(x64, w_r64, bias64)
    z_g = res["logits"]
    rel = np.abs(z_g.astype(np.float64) - z_o) / (1.0 + np.abs(z_o))
    ztol = 1e-5 if cfg.dtype == "f32" else 1e-4
    assert rel.max() <= ztol, f"logits differ: max rel {rel.max():.3g}"
    # the top-k stage, teacher-forced on the GPU's own logits: bit-exact on every token
    idx_gz = O.select_topk(z_g.astype(np.float64), cfg.k)
    bad = np.any(res["idx"] != idx_gz, axis=1)
    assert not bad.any(), (f"top-k of the GPU's own logits differs on {int(bad.sum())} tokens "
                           f"(first {int(np.argmax(bad))}: {res['idx'][bad][0].tolist()} vs {idx_gz[bad][0].tolist()})")
    w_gz = O.topk_weights(z_g.astype(np.float64), res["idx"], cfg.weights)
    assert np.abs(res["w"] - w_gz).max(initial=0.0) <= 1e-5, "weights of the GPU's own logits differ"
    idx_o = O.select_topk(z_o, cfg.k)
    margin = O.topk_margin(z_o, cfg.k)
    set_g = np.sort(res["idx"], axis=1)
    set_o = np.sort(idx_o, axis=1)
    flip = np.any(set_g != set_o, axis=1)
    same_row = np.all(z_g == z_o, axis=1)
    assert not np.any(flip & same_row), \
        f"selection differs on {int(np.sum(flip & same_row))} tokens whose logits equal the oracle's"
    assert np.array_equal(res["idx"][same_row], idx_o[same_row]), "slot order differs on exact-logit tokens"
    assert not np.any(flip & (margin > MARGIN)), \
        f"selection differs on {int(np.sum(flip & (margin > MARGIN)))} tokens with margin > {MARGIN}"
    # slot order where the top-k gaps are all clear
    zs = -np.sort(-z_o.astype(np.float64), axis=1)[:, :cfg.k]
    clear = np.all(-np.diff(zs, axis=1) > MARGIN, axis=1) & ~flip
    assert np.array_equal(res["idx"][clear], idx_o[clear]), "slot order differs on clear tokens"
    # weights keyed by expert
    w_o = O.topk_weights(z_o, res["idx"], cfg.weights)
    assert np.abs(res["w"] - w_o)[~flip].max(initial=0.0) <= 1e-5, "routing weights differ"
    report.update(route_flips=int(flip.sum()), min_margin=float(margin.min()),
                  max_logit_rel=float(rel.max()), exact_logit_tokens=int(same_row.sum()),
                  exact_ties=int(np.sum(margin == 0)))
    return z_o, flip


def check_dispatch(cfg, res):
    """The oracle's dispatch on the GPU's own routing (selection and logits), bit-exact."""
    dp = O.dispatch(res["idx"], cfg.E, cfg.capacity, cfg.priority, cfg.overflow,
                    res["logits"].astype(np.float64))
    assert np.array_equal(res["counts"], dp["counts"]), "counts differ"
    assert np.array_equal(res["offsets"], dp["offsets"]), "offsets differ"
    R = int(dp["offsets"][-1])
    assert np.array_equal(res["perm"][:R], dp["perm"]), "perm differs"
    assert np.array_equal(res["inv"], dp["inv"]), "inv differs"
    assert res["n_dropped"] == dp["n_dropped"], "n_dropped differs"
    return dp


def check_output(cfg, x64, z_o, res, fetch, shared, tokens: Optional[np.ndarray], report: dict,
                 out_bf16: bool = False):
    """FFN + combine on the GPU's routing, for `tokens` (None = all)."""
    idx = res["idx"]
    keep = res["inv"] >= 0
    w_o = O.topk_weights(z_o, idx, cfg.weights)
    # the expert that computed each kept slot: the segment its row lies in (re-routing
    # can move a slot off the router's choice; it keeps its weight)
    seg = np.searchsorted(res["offsets"], np.maximum(res["inv"], 0), side="right") - 1
    if cfg.overflow == "drop":
        assert np.array_equal(seg[keep], idx[keep]), "a kept slot left its expert"
    idx = np.where(keep, seg, idx)
    sel = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    ref = O.routed_output(x64[sel], idx[sel], w_o[sel], keep[sel], cfg.act, fetch, shared)
    got = res["out"][sel]
    alive = np.any(keep[sel], axis=1) | (shared is not None)
    assert np.all(got[~alive] == 0.0), "a fully dropped token has a non-zero output"
    live = ref[alive]
    rms = math.sqrt(float(np.mean(live ** 2))) if live.size else 1.0
    tol = TOL[cfg.dtype]
    excess = np.abs(got - ref) - (half_ulp_bf16(ref) if out_bf16 else 0.0)
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    worst = float(excess.max()) if ref.size else 0.0
    report.update(max_abs_err=err, rms=rms, err_over_rms=err / rms if rms else err)
    assert worst <= tol * rms, f"output error {err:.4g} (beyond rounding {worst:.4g}) > {tol} x RMS {rms:.4g}"
    return ref
