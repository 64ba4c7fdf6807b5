"""Pins of the CPU oracle against what the source pages and the mathematics fix.

Each ``check_*`` function is one pin; the ``test_*`` functions run them against the
oracle as it stands, and ``test_mutation_*`` plant a plausible mistake in the oracle
(on the CPU, through monkeypatch) and require that some pin catches it.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------------
# torch (CPU, float64) textbook forms used as independent references
# ---------------------------------------------------------------------------------
def _torch_ffn(x, act, wg, wu, wd):
    x = torch.as_tensor(np.asarray(x, np.float64))
    wg = torch.as_tensor(np.asarray(wg, np.float64))
    wd = torch.as_tensor(np.asarray(wd, np.float64))
    if act == "gelu":
        h = Fnn.gelu(Fnn.linear(x, wg))
    else:
        wu = torch.as_tensor(np.asarray(wu, np.float64))
        h = Fnn.silu(Fnn.linear(x, wg)) * Fnn.linear(x, wu)
    return Fnn.linear(h, wd).numpy()


def _rand_experts(rng, E, d, F, act):
    wg = rng.standard_normal((E, F, d)) / math.sqrt(d)
    wu = rng.standard_normal((E, F, d)) / math.sqrt(d) if act == "swiglu" else None
    wd = rng.standard_normal((E, d, F)) / math.sqrt(F)
    return wg, wu, wd


# ---------------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------------
def check_worked_combine():
    g = _golden("worked_combine.json")
    y = np.array([g["expert_outputs"]])            # [1, k=2, d=3]
    w = np.array([g["weights"]])
    out = O.combine(y, w)[0]
    np.testing.assert_allclose(out, g["mixture"], rtol=0, atol=1e-15)
    assert abs(out[0] - (0.75 * 0.8 + 0.25 * 0.4)) < 1e-15


def _worked_layer(act):
    """E=4, d=3: token x = e_0; the router puts logit ln 3 on E1 and 0 on E3 (others far
    below), so the renormalised weights are 3/4 and 1/4.  Each expert has F=1 and is
    built so that it returns a prescribed vector for this token."""
    g = _golden("worked_combine.json")
    targets = np.array([g["expert_outputs"][0], [9.0, 9.0, 9.0],
                        g["expert_outputs"][1], [-9.0, 9.0, -9.0]])
    d, E, F = 3, 4, 1
    x = np.array([[1.0, 0.0, 0.0]])
    w_r = np.zeros((d, E))
    w_r[0] = [math.log(3.0), -10.0, 0.0, -10.0]
    a = 1.0
    wg = np.zeros((E, F, d))
    wg[:, 0, 0] = a
    if act == "swiglu":
        wu = np.zeros((E, F, d))
        wu[:, 0, 0] = 1.0
        hval = O.silu(np.array(a))
    else:
        wu = None
        hval = O.gelu(np.array(a))
    wd = targets[:, :, None] / hval                  # [E, d, F]
    return O.moe_layer(x, w_r, 2, act, wg, wu, wd), g


def _worked_layer_args():
    """(w_r, k, act, wg, wu, wd) of the SwiGLU worked layer, for variants."""
    g = _golden("worked_combine.json")
    targets = np.array([g["expert_outputs"][0], [9.0, 9.0, 9.0], g["expert_outputs"][1], [-9.0, 9.0, -9.0]])
    w_r = np.zeros((3, 4))
    w_r[0] = [math.log(3.0), -10.0, 0.0, -10.0]
    wg = np.zeros((4, 1, 3))
    wg[:, 0, 0] = 1.0
    wu = wg.copy()
    wd = targets[:, :, None] / O.silu(np.array(1.0))
    return w_r, 2, "swiglu", wg, wu, wd


def check_worked_layer():
    for act in ("swiglu", "gelu"):
        res, g = _worked_layer(act)
        assert list(res["idx"][0]) == g["chosen"]
        np.testing.assert_allclose(res["w"][0], g["weights"], rtol=0, atol=1e-7)
        np.testing.assert_allclose(res["out"][0], g["mixture"], rtol=0, atol=1e-6)


def check_printed_gate():
    g = _golden("printed_gate.json")
    p = np.array([g["gate_probabilities"]])
    z = np.log(p).astype(np.float32)
    idx = O.select_topk(z, 2)
    assert list(idx[0]) == g["top2_experts"]
    probs = np.take_along_axis(O.softmax(z), idx, axis=1)[0]
    np.testing.assert_allclose(probs, g["top2_probabilities"], rtol=1e-6)
    w = O.topk_weights(z, idx)[0]
    np.testing.assert_allclose(w, np.array([0.85, 0.08]) / 0.93, rtol=1e-6)


def check_softmax_weights():
    """Un-renormalised weights ([cnnet] §3.2 output = p1 e1 + p2 e2; [wmrh] §5.1): the
    printed probabilities are the weights; with k = E they equal the renormalised ones."""
    g = _golden("printed_gate.json")
    z = np.log(np.array([g["gate_probabilities"]])).astype(np.float32)
    idx = O.select_topk(z, 2)
    np.testing.assert_allclose(O.topk_weights(z, idx, "softmax")[0], g["top2_probabilities"], rtol=1e-6)
    rng = _rng(13)
    z = rng.standard_normal((20, 5)).astype(np.float32)
    idx = O.select_topk(z, 5)
    np.testing.assert_allclose(O.topk_weights(z, idx, "softmax"), O.topk_weights(z, idx), rtol=1e-13)
    idx = O.select_topk(z, 2)
    assert np.all(O.topk_weights(z, idx, "softmax").sum(axis=1) < 1.0)
    res, gold = _worked_layer("swiglu")
    x = np.array([[1.0, 0.0, 0.0]])
    r2 = O.moe_layer(x, *_worked_layer_args(), weights="softmax")
    p = O.softmax(O.router_logits(x, _worked_layer_args()[0]))[0]
    want = p[0] * np.array(gold["expert_outputs"][0]) + p[2] * np.array(gold["expert_outputs"][1])
    np.testing.assert_allclose(r2["out"][0], want, rtol=1e-6)


def check_ln3_weights():
    z = np.array([[0.0, math.log(3.0), -1.0]])
    idx = O.select_topk(z, 2)
    assert list(idx[0]) == [1, 0]
    np.testing.assert_allclose(O.topk_weights(z, idx)[0], [0.75, 0.25], rtol=0, atol=1e-15)


def check_weight_formulations():
    """Renormalised top-k probabilities == softmax of the selected logits ([rkmt] §3.3
    TinyMoE) == softmax with the unselected logits masked to -inf ([mlqm] §3.3)."""
    rng = _rng(7)
    for E, k in [(4, 2), (16, 2), (64, 2), (64, 6), (8, 8), (5, 1)]:
        z = (rng.standard_normal((50, E)) * 3).astype(np.float32)
        idx = O.select_topk(z, k)
        w = O.topk_weights(z, idx)
        zs = np.take_along_axis(z.astype(np.float64), idx, axis=1)
        w2 = torch.softmax(torch.as_tensor(zs), dim=1).numpy()
        masked = np.full(z.shape, -np.inf)
        np.put_along_axis(masked, idx, zs, axis=1)
        w3 = np.take_along_axis(torch.softmax(torch.as_tensor(masked), dim=1).numpy(), idx, axis=1)
        np.testing.assert_allclose(w, w2, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(w, w3, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-13)
        assert np.all(w > 0) and np.all(w <= 1)
        assert np.all(np.diff(w, axis=1) <= 1e-15)          # best slot first


def _topk_brute(zrow, k):
    """Enumerate all k-subsets; keep the largest sum of logits, ties to the
    lexicographically smallest index tuple; return it best-first."""
    best = min(itertools.combinations(range(len(zrow)), k),
               key=lambda s: (-sum(float(zrow[e]) for e in s), s))
    return sorted(best, key=lambda e: (-float(zrow[e]), e))


def check_topk_bruteforce():
    rng = _rng(11)
    for E in range(1, 8):
        for k in range(1, min(E, 3) + 1):
            for _ in range(40):
                z = rng.integers(-2, 3, size=(1, E)).astype(np.float32)  # many exact ties
                assert list(O.select_topk(z, k)[0]) == _topk_brute(z[0], k)
    assert sum(1 for _ in itertools.combinations(range(64), 2)) == \
        _golden("ledgers.json")["pairs_of_64"]["combinations"]


def check_topk_margin():
    z = np.array([[1.0, 4.0, 2.5, 2.0]], np.float32)
    np.testing.assert_allclose(O.topk_margin(z, 2), [0.5])
    np.testing.assert_allclose(O.topk_margin(z, 1), [1.5])
    assert np.isinf(O.topk_margin(z, 4)[0])


def check_router_logits():
    """One-hot tokens read out a row of W_r plus the bias; general inputs match a
    float64 linear layer rounded to fp32."""
    rng = _rng(3)
    d, E = 16, 5
    w_r = rng.standard_normal((d, E)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    x = np.eye(d, dtype=np.float32)[[3, 0, 15]]
    z = O.router_logits(x, w_r, b)
    np.testing.assert_array_equal(z, (w_r[[3, 0, 15]].astype(np.float64) + b).astype(np.float32))
    x = rng.standard_normal((9, d))
    ref = Fnn.linear(torch.as_tensor(x), torch.as_tensor(w_r.astype(np.float64)).T,
                     torch.as_tensor(b.astype(np.float64))).numpy().astype(np.float32)
    np.testing.assert_array_equal(O.router_logits(x, w_r, b), ref)
    assert O.router_logits(x, w_r).shape == (9, E)


def check_capacity_rule():
    c = _golden("ledgers.json")["capacity"]
    assert O.capacity_rule(c["T"], c["k"], c["E"]) == c["capacity"]
    assert O.capacity_rule(10, 2, 4) == 5
    assert O.capacity_rule(10, 1, 4) == 3          # ceil(2.5)
    assert O.capacity_rule(1000, 2, 16, 1.25) == 157   # ceil(156.25)
    # DeepSpeed knobs of [cnnet] §4.2: capacity_factor 1.2, eval 2.0, min_capacity 4
    assert O.capacity_rule(1024, 2, 16, 1.2, 4) == 154   # ceil(153.6)
    assert O.capacity_rule(1024, 2, 16, 2.0, 4) == 256
    assert O.capacity_rule(1, 2, 16, 1.2, 4) == 4        # tiny batch: the floor applies


def _keep_bruteforce(idx, capacity):
    """Slot (t, j) of expert e survives iff fewer than C earlier tokens chose e."""
    T, k = idx.shape
    keep = np.ones((T, k), bool)
    for t in range(T):
        for j in range(k):
            earlier = sum(1 for t2 in range(t) if idx[t, j] in idx[t2])
            keep[t, j] = capacity <= 0 or earlier < capacity
    return keep


def _random_idx(rng, T, E, k, skew=0.0):
    z = rng.standard_normal((T, E)) + skew * np.arange(E)[None, ::-1]
    return O.select_topk(z.astype(np.float32), k)


def check_dispatch():
    c = _golden("ledgers.json")["calls"]
    T, E, k = c["T"], c["E"], c["k"]
    idx = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)])   # balanced
    dp = O.dispatch(idx, E)
    assert dp["counts"].sum() == c["calls"]
    assert list(dp["counts"]) == [c["per_expert_balanced"]] * E
    rng = _rng(5)
    for (T, E, k, C, skew) in [(37, 5, 2, 0, 0), (64, 8, 3, 0, 1.0), (40, 4, 2, 6, 0.5),
                               (25, 6, 1, 3, 2.0), (30, 3, 3, 100, 0), (20, 4, 2, 1, 0)]:
        idx = _random_idx(rng, T, E, k, skew)
        dp = O.dispatch(idx, E, C)
        assert dp["counts"].sum() == T * k
        np.testing.assert_array_equal(dp["counts"], np.bincount(idx.ravel(), minlength=E))
        keep = _keep_bruteforce(idx, C)
        np.testing.assert_array_equal(dp["inv"] >= 0, keep)
        cap = C if C > 0 else T * k
        np.testing.assert_array_equal(dp["kept"], np.minimum(dp["counts"], cap))
        assert dp["n_dropped"] == int(np.maximum(dp["counts"] - cap, 0).sum())
        # permutation = stable argsort of the expert of each kept slot
        flat_e = idx.ravel()
        kept_slots = np.nonzero(keep.ravel())[0]
        order = kept_slots[np.argsort(flat_e[kept_slots], kind="stable")]
        np.testing.assert_array_equal(dp["perm"], order)
        np.testing.assert_array_equal(dp["offsets"], np.concatenate([[0], np.cumsum(dp["kept"])]))
        inv = dp["inv"].ravel()
        assert np.all(inv[dp["perm"]] == np.arange(len(dp["perm"])))    # bijection
        if C >= T:
            np.testing.assert_array_equal(dp["perm"], O.dispatch(idx, E, 0)["perm"])


def check_capacity_policies():
    """Slot-major priority and re-routing of overflow to the next-best expert ([rkmt] §2.3:
    tokens beyond an expert's capacity are dropped or sent to the next-best expert)."""
    # worked by hand: 3 tokens choosing both of 2 experts, capacity 1
    idx = np.array([[0, 1], [1, 0], [1, 0]])
    tok = O.dispatch(idx, 2, 1, "token")
    np.testing.assert_array_equal(tok["inv"], [[0, 1], [-1, -1], [-1, -1]])     # token 0 takes both
    slot = O.dispatch(idx, 2, 1, "slot")
    np.testing.assert_array_equal(slot["inv"], [[0, -1], [1, -1], [-1, -1]])    # first choices first
    np.testing.assert_array_equal(slot["perm"], [0, 2])
    assert tok["n_dropped"] == slot["n_dropped"] == 4
    # slot-major against library routines: keep the C smallest (slot, token) per expert
    rng = _rng(11)
    for (T, E, k, C) in [(30, 5, 2, 4), (40, 4, 3, 7), (17, 6, 2, 0), (25, 3, 2, 100)]:
        idx = _random_idx(rng, T, E, k, 1.0)
        dp = O.dispatch(idx, E, C, "slot")
        tt, jj = np.meshgrid(np.arange(T), np.arange(k), indexing="ij")
        order = np.lexsort((tt.ravel(), jj.ravel()))          # slot-major positions
        flat_e = idx.ravel()[order]
        by_expert = order[np.argsort(flat_e, kind="stable")]   # stable: slot-major within an expert
        e_sorted = np.sort(flat_e, kind="stable")
        rank = np.arange(T * k) - np.searchsorted(e_sorted, e_sorted)
        keep = rank < (C if C > 0 else T * k)
        np.testing.assert_array_equal(dp["perm"], by_expert[keep])
        assert dp["n_dropped"] == int((~keep).sum())
        if C <= 0 or C >= T * k:                               # no drops: only the row order differs
            np.testing.assert_array_equal(np.sort(dp["perm"]), np.arange(T * k))
    # re-route worked by hand: 4 tokens all choosing expert 0, capacity 1
    z = np.array([[3.0, 2, 1], [3, 1, 2], [3, 2, 1], [3, 2, 1]])
    rr = O.dispatch(np.zeros((4, 1), int), 3, 1, "token", "reroute", z)
    np.testing.assert_array_equal(rr["expert"], [[0], [2], [1], [-1]])
    np.testing.assert_array_equal(rr["perm"], [0, 2, 1])
    np.testing.assert_array_equal(rr["inv"], [[0], [2], [1], [-1]])
    np.testing.assert_array_equal(rr["kept"], [1, 1, 1])
    np.testing.assert_array_equal(rr["counts"], [4, 0, 0])
    assert rr["n_dropped"] == 1
    # top-k experts and earlier re-routes of the same token are not candidates
    z = np.array([[4.0, 3, 2, 1], [4, 3, 1, 2]])
    for pr in ("token", "slot"):
        rr = O.dispatch(np.array([[0, 1], [0, 1]]), 4, 1, pr, "reroute", z)
        np.testing.assert_array_equal(rr["expert"], [[0, 1], [3, 2]])
    # invariants on random cases
    for (T, E, k, C) in [(40, 6, 2, 5), (60, 8, 3, 9), (33, 5, 2, 3), (50, 4, 1, 10)]:
        zz = rng.standard_normal((T, E)) + np.linspace(2, 0, E)     # skewed preferences
        idx = O.select_topk(zz, k)
        for pr in ("token", "slot"):
            dr = O.dispatch(idx, E, C, pr, "drop")
            rr = O.dispatch(idx, E, C, pr, "reroute", zz)
            np.testing.assert_array_equal(rr["counts"], dr["counts"])
            assert np.all(rr["kept"] <= C) and rr["n_dropped"] <= dr["n_dropped"]
            first = dr["inv"] >= 0                                # the router's kept choices stay
            np.testing.assert_array_equal(rr["expert"][first], idx[first])
            for t in range(T):
                ex = [int(e) for e in rr["expert"][t] if e >= 0]
                assert len(ex) == len(set(ex))                    # distinct experts per token
                for j in range(k):
                    e = rr["expert"][t, j]
                    if not first[t, j] and e >= 0:
                        assert e not in idx[t]                    # moved off the top-k
                    if e < 0:                                     # nothing left for it
                        free = [f for f in range(E) if f not in idx[t] and f not in ex]
                        assert all(rr["kept"][f] == C for f in free)
            inv = rr["inv"].ravel()
            assert np.all(inv[rr["perm"]] == np.arange(len(rr["perm"])))
        # capacity that never overflows: re-route changes nothing
        big = O.dispatch(idx, E, T * k, "token", "reroute", zz)
        np.testing.assert_array_equal(big["perm"], O.dispatch(idx, E, 0)["perm"])


def check_activations():
    assert O.gelu(np.array(0.0)) == 0.0 and O.silu(np.array(0.0)) == 0.0
    np.testing.assert_allclose(O.gelu(np.array([1.0, -1.0])),
                               [0.8413447460685429, -0.15865525393145707], rtol=1e-15)
    np.testing.assert_allclose(O.silu(np.array([1.0, -2.0])),
                               [1 / (1 + math.exp(-1)), -2 / (1 + math.exp(2))], rtol=1e-15)
    v = np.linspace(-8, 8, 101)
    np.testing.assert_allclose(O.gelu(v), Fnn.gelu(torch.as_tensor(v)).numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(O.silu(v), Fnn.silu(torch.as_tensor(v)).numpy(), rtol=1e-13, atol=1e-15)


def check_expert_ffn():
    rng = _rng(9)
    for act in ("gelu", "swiglu"):
        wg, wu, wd = _rand_experts(rng, 1, 24, 40, act)
        x = rng.standard_normal((7, 24))
        got = O.expert_ffn(x, act, wg[0], None if wu is None else wu[0], wd[0])
        ref = _torch_ffn(x, act, wg[0], None if wu is None else wu[0], wd[0])
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def check_layer_special_cases():
    rng = _rng(21)
    T, d, F = 33, 16, 24
    for act in ("gelu", "swiglu"):
        # E=1, k=1: a dense FFN
        wg, wu, wd = _rand_experts(rng, 1, d, F, act)
        x = rng.standard_normal((T, d))
        w_r = rng.standard_normal((d, 1))
        res = O.moe_layer(x, w_r, 1, act, wg, wu, wd)
        np.testing.assert_allclose(res["out"], _torch_ffn(x, act, wg[0], None if wu is None else wu[0], wd[0]),
                                   rtol=1e-12, atol=1e-13)
        # identical experts: any routing gives FFN(x); a shared expert adds its own FFN
        E, k = 6, 2
        wg1, wu1, wd1 = _rand_experts(rng, 1, d, F, act)
        rep = lambda a: None if a is None else np.repeat(a, E, axis=0)  # noqa: E731
        w_r = rng.standard_normal((d, E))
        bias = rng.standard_normal(E)
        ffn = _torch_ffn(x, act, wg1[0], None if wu1 is None else wu1[0], wd1[0])
        res = O.moe_layer(x, w_r, k, act, rep(wg1), rep(wu1), rep(wd1), bias=bias)
        np.testing.assert_allclose(res["out"], ffn, rtol=1e-11, atol=1e-12)
        sg, su, sd = _rand_experts(rng, 1, d, F, act)
        shared = (sg[0], None if su is None else su[0], sd[0])
        res = O.moe_layer(x, w_r, k, act, rep(wg1), rep(wu1), rep(wd1), bias=bias, shared=shared)
        np.testing.assert_allclose(res["out"], ffn + _torch_ffn(x, act, *shared), rtol=1e-11, atol=1e-12)
        # k = E without capacity: the dense soft mixture over all experts
        E = 4
        wg, wu, wd = _rand_experts(rng, E, d, F, act)
        w_r = rng.standard_normal((d, E))
        res = O.moe_layer(x, w_r, E, act, wg, wu, wd)
        p = torch.softmax(torch.as_tensor(res["logits"].astype(np.float64)), dim=1).numpy()
        dense = sum(p[:, e:e + 1] * _torch_ffn(x, act, wg[e], None if wu is None else wu[e], wd[e])
                    for e in range(E))
        np.testing.assert_allclose(res["out"], dense, rtol=1e-11, atol=1e-12)
        # token permutation equivariance (no capacity)
        res = O.moe_layer(x, w_r, 2, act, wg, wu, wd)
        pi = rng.permutation(T)
        res_p = O.moe_layer(x[pi], w_r, 2, act, wg, wu, wd)
        np.testing.assert_allclose(res_p["out"], res["out"][pi], rtol=1e-12, atol=1e-14)
        # a token whose every slot is dropped outputs zero (no shared expert)
        res = O.moe_layer(x, w_r, 2, act, wg, wu, wd, capacity=1)
        dead = np.all(res["inv"] < 0, axis=1)
        assert dead.any()
        assert np.all(res["out"][dead] == 0.0)
        # a partly dropped token keeps its other weighted term, not renormalised
        part = (res["inv"] >= 0).sum(axis=1) == 1
        for t in np.nonzero(part)[0][:3]:
            j = int(np.nonzero(res["inv"][t] >= 0)[0][0])
            e = int(res["idx"][t, j])
            y = _torch_ffn(x[t:t + 1], act, wg[e], None if wu is None else wu[e], wd[e])[0]
            np.testing.assert_allclose(res["out"][t], res["w"][t, j] * y, rtol=1e-12, atol=1e-14)


def check_ledgers():
    a = _golden("ledgers.json")["active_params"]
    assert O.active_params(0, a["routed_total"], a["E"], a["k"]) == a["routed_active"]
    assert O.active_params(a["common"], a["routed_total"], a["E"], a["k"]) == a["active"]
    assert abs(a["active"] / a["total"] - 0.3) < 1e-12
    assert O.expert_weight_bytes(64, 4096, 14336, "swiglu", 2) == 64 * 3 * 4096 * 14336 * 2
    assert abs(O.expert_weight_bytes(64, 4096, 14336, "swiglu", 2) / 1e9 - 22.55) < 0.01
    assert O.expert_weight_bytes(4, 64, 128, "gelu", 4) == 4 * 2 * 64 * 128 * 4


# ---------------------------------------------------------------------------------
# Routing statistics
# ---------------------------------------------------------------------------------
def check_routing_stats():
    """Balance ratio against the page's own formulation in torch (one-hot mask summed
    over slots, mean over tokens, torch.std); entropy against scipy; closed forms for
    uniform and collapsed routing."""
    from scipy.stats import entropy as sp_entropy
    rng = _rng(31)
    T, E, k = 200, 8, 2
    z = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    idx = O.select_topk(z, k)
    counts = np.bincount(idx.ravel(), minlength=E)
    st = O.routing_stats(z, counts, 7, k)
    mask = Fnn.one_hot(torch.as_tensor(idx), num_classes=E).sum(dim=1).double()
    freq = mask.mean(dim=0)
    ratio = (torch.std(freq) / (torch.mean(freq) + 1e-8)).item()
    assert abs(st["balance_ratio"] - ratio) < 1e-12
    assert abs(st["l_balance"] - 0.01 * ratio) < 1e-14
    assert abs(st["l_aux"] - 0.01 * (torch.std(freq).item() + 100 * freq.max().item())) < 1e-12
    p = O.softmax(z)
    ent = np.mean([sp_entropy(p[t]) for t in range(T)])
    assert abs(st["entropy"] - ent) < 1e-12
    np.testing.assert_allclose(st["utilization"].sum(), 1.0)
    assert st["drop_rate"] == 7 / (T * k)
    # uniform: ratio 0, l_aux = lambda*gamma*k/E; equal logits: entropy ln E
    uni = O.routing_stats(np.zeros((16, 16), np.float32), np.full(16, 2), 0, 2)
    assert uni["balance_ratio"] == 0.0
    assert abs(uni["l_aux"] - 0.01 * 100 * 2 / 16) < 1e-15
    assert abs(uni["entropy"] - math.log(16)) < 1e-12
    np.testing.assert_allclose(uni["utilization"], 1 / 16)
    # collapsed: one expert takes every token's first slot -> near-zero entropy when the
    # logit gap is huge
    zc = np.full((4, 4), -60.0, np.float32)
    zc[:, 0] = 60.0
    assert O.routing_stats(zc, np.array([4, 4, 0, 0]), 0, 2)["entropy"] < 1e-40




PINS = [check_worked_combine, check_worked_layer, check_printed_gate, check_softmax_weights, check_ln3_weights,
        check_weight_formulations, check_topk_bruteforce, check_topk_margin,
        check_router_logits, check_capacity_rule, check_dispatch, check_capacity_policies, check_activations,
        check_expert_ffn, check_layer_special_cases, check_ledgers, check_routing_stats]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ---------------------------------------------------------------------------------
# Planted mistakes: each must be caught by at least one pin
# ---------------------------------------------------------------------------------
def _fails(monkeypatch, name, bad):
    monkeypatch.setattr(O, name, bad)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure of a pin counts as caught
            caught.append(pin.__name__)
    return caught


_orig = {n: getattr(O, n) for n in ("expert_order", "topk_weights", "dispatch", "expert_ffn",
                                    "combine", "router_logits", "gelu", "silu", "capacity_rule",
                                    "active_params")}


def _mut_highest_index_ties(z):
    E = np.asarray(z).shape[1]
    return (E - 1 - np.argsort(-np.asarray(z, np.float64)[:, ::-1], axis=1, kind="stable"))


def _mut_inverted_weights(z, idx, mode="renormalized"):
    zs = np.take_along_axis(np.asarray(z, np.float64), idx, axis=1)
    e = np.exp(zs[:, :1] - zs)
    return e / e.sum(axis=1, keepdims=True)


def _mut_keep_latest(idx, E, capacity=0, priority="token", overflow="drop", z=None):
    res = _orig["dispatch"](idx, E, 0)
    if capacity <= 0:
        return res
    keep = (_orig["dispatch"](idx[::-1], E, capacity)["inv"] >= 0)[::-1]
    return dict(res, inv=np.where(keep, res["inv"], -1),
                kept=np.minimum(res["counts"], capacity), n_dropped=int((~keep).sum()))


def _mut_transposed_down(xr, act, wg, wu, wd):
    return _orig["expert_ffn"](xr, act, wg, wu, np.ascontiguousarray(wd.T).reshape(wd.shape))


def _mut_slot_as_token(idx, E, capacity=0, priority="token", overflow="drop", z=None):
    return _orig["dispatch"](idx, E, capacity, "token", overflow, z)


def _mut_reroute_worst(idx, E, capacity=0, priority="token", overflow="drop", z=None):
    return _orig["dispatch"](idx, E, capacity, priority, overflow, None if z is None else -np.asarray(z))


def _mut_reroute_keeps_topk(idx, E, capacity=0, priority="token", overflow="drop", z=None):
    res = _orig["dispatch"](idx, E, capacity, priority, overflow, z)
    if overflow != "reroute":
        return res
    return _reroute_any(np.asarray(idx), E, capacity, priority, z)


def _reroute_any(idx, E, capacity, priority, z):
    """Planted mistake: overflow may move to the token's own other top-k experts."""
    T, k = idx.shape
    expert = np.full((T, k), -1)
    load = np.zeros(E, int)
    over = []
    for t, j in O.priority_order(T, k, priority):
        e = idx[t, j]
        if load[e] < capacity:
            expert[t, j] = e
            load[e] += 1
        else:
            over.append((t, j))
    pref = O.expert_order(z)
    for t, j in over:
        for e in pref[t]:
            if e not in expert[t] and load[e] < capacity:
                expert[t, j] = e
                load[e] += 1
                break
    return dict(expert=expert, kept=load, n_dropped=int((expert < 0).sum()), counts=np.bincount(idx.ravel(), minlength=E),
                perm=np.zeros(0, int), inv=np.full((T, k), -1), offsets=np.zeros(E + 1, int))


def _mut_unweighted(y, w, keep=None, shared=None):
    return _orig["combine"](y, np.ones_like(np.asarray(w, np.float64)), keep, shared)


def _mut_no_shared(y, w, keep=None, shared=None):
    return _orig["combine"](y, w, keep, None)


def _mut_bias_dropped(x, w_r, bias=None):
    return _orig["router_logits"](x, w_r, None)


def _mut_tanh_gelu(v):
    v = np.asarray(v, np.float64)
    return 0.5 * v * (1 + np.tanh(math.sqrt(2 / math.pi) * (v + 0.044715 * v ** 3)))


def _mut_sigmoid_only(v):
    return 1.0 / (1.0 + np.exp(-np.asarray(v, np.float64)))


def _mut_capacity_floor_no_k(T, k, E, factor=1.0, min_capacity=0):
    return max(min_capacity, int(factor * T / E))


def _mut_ledger_no_k(common, routed_total, E, k):
    return common + routed_total / E


MUTATIONS = [("expert_order", _mut_highest_index_ties), ("topk_weights", _mut_inverted_weights),
             ("dispatch", _mut_keep_latest), ("expert_ffn", _mut_transposed_down),
             ("combine", _mut_unweighted), ("combine", _mut_no_shared),
             ("router_logits", _mut_bias_dropped), ("gelu", _mut_tanh_gelu),
             ("silu", _mut_sigmoid_only), ("capacity_rule", _mut_capacity_floor_no_k),
             ("active_params", _mut_ledger_no_k), ("dispatch", _mut_slot_as_token),
             ("dispatch", _mut_reroute_worst), ("dispatch", _mut_reroute_keeps_topk)]


@pytest.mark.parametrize("name,bad", MUTATIONS, ids=[m[1].__name__ for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, bad):
    caught = _fails(monkeypatch, name, bad)
    assert caught, f"planted mistake in {name} ({bad.__name__}) passed every pin"


def _mut_population_std(z, counts, n_dropped, k, lambda_balance=0.01, lambda_aux=0.01, gamma_aux=100.0):
    r = _orig_stats(z, counts, n_dropped, k, lambda_balance, lambda_aux, gamma_aux)
    u = np.asarray(counts, np.float64) / np.asarray(z).shape[0]
    r["balance_ratio"] = float(np.std(u)) / float(np.mean(u))
    return r


_orig_stats = O.routing_stats


def test_routing_stats_mutation_is_caught(monkeypatch):
    monkeypatch.setattr(O, "routing_stats", _mut_population_std)
    with pytest.raises(AssertionError):
        check_routing_stats()
