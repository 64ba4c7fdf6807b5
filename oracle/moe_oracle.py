"""Plain CPU oracle for the forward pass of one sparse Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library imports, links or calls this
module, and this module imports nothing from the GPU library.  It may be used by
``tests/``, by ``__graft_entry__.smoke()`` and by the CPU-baseline leg of ``bench.py``.

Every step is written out as its plain definition in float64 (numpy), with library
primitives (matmul, a stable sort, erf) as the only building blocks.  No blocking,
fusion or reordering is applied beyond what the definition states.

Sources (web pages, cited by title/site and section):
  [mlqm]   www.mlqm.cn/news/130088 (MoE explainer, no title in the extract):
           §3.1 "Router", §3.3 "Gate", §4.2 "模型定义" (the PyTorch MoE layer code).
  [rkmt]   "大模型MoE架构揭秘：为什么总参数≠激活参数" (www.rkmt.cn/news/1609753):
           §2.3 "路由器的设计哲学" (load balance, expert capacity), §3.3 TinyMoE code.
  [wmrh]   www.wmrh.cn/news/107921 (MoE explainer, no title in the extract):
           §2.1 gating network, §5.1 toy MoE layer and its printed gate probabilities.
  [cnnet]  "MoE混合专家架构原理与工程实践：解密大模型稀疏计算真相" (cnnetsun.cn/a/2502649):
           §3.2 router cost, the DeepSpeed-MoE block.
  [200B-5] "[从零训练一个200B大语言模型] 5/25：MoE怎样用一部分参数，完成一次计算？"
           (shanhuang.net): sections "谁来决定请哪几个专家？" (router, top-k, worked
           combine), "共享专家，给每个token都走的一条路" (shared expert),
           "200B还在，为什么每次可以少算？" (active-parameter ledger),
           "四个专家同时算，选两个会更快吗？" (calls per expert).

Readings taken where the pages are silent or disagree (each is pinned by a test in
tests/test_oracle_pins.py):
  * selection is made on the fp32 router logits; softmax is monotone, so the top-k of
    the probabilities equals the top-k of the logits.  Equal logits: lowest expert
    index first.  Slot j is the j-th best expert.
  * weights are the softmax probabilities of the selected experts renormalised to sum
    to 1 ([mlqm] §3.3 and §4.2); temperature is 1.  Variant: the raw probabilities.
  * capacity keeps, per expert, the earliest tokens (ascending token index); an
    overflowing slot contributes zero and the other weights are not renormalised.
    Variants: first choices before second choices (slot-major priority), and overflow
    re-routed to the token's next-best expert with room (router choices first, then the
    overflow in priority order; a re-routed slot keeps its weight).
  * GeLU is the exact erf form; SwiGLU is down(silu(gate x) * (up x)); experts carry no
    biases; the shared expert is added with weight 1.

Every function here is pinned (see the test module); no function is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Callable, Dict, List, Optional, Tuple

import numpy as np
from scipy.special import erf as _erf

F64 = np.float64


# ----------------------------------------------------------------------------------
# Router: logits, top-k selection, weights
# ----------------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_r: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Router logits z = x W_r (+ b), one score per expert.

    [mlqm] §3.1: the router is one linear layer W_r mapping the hidden state h to an
    E-vector of logits, followed by a softmax.  [rkmt] §3.3 and [wmrh] §5.1 use a linear
    layer with a bias; the bias here is an optional per-expert offset.
    The dot products are taken in float64 and the logit is rounded once to fp32, the
    precision in which the selection is defined.
    x: [T, d], w_r: [d, E], bias: [E] or None  ->  z: float32 [T, E]
    """
    z = np.asarray(x, F64) @ np.asarray(w_r, F64)
    if bias is not None:
        z = z + np.asarray(bias, F64)[None, :]
    return z.astype(np.float32)


def expert_order(z: np.ndarray) -> np.ndarray:
    """Experts of each token ordered by descending logit; equal logits keep ascending
    expert index (a stable sort of -z).  [200B-5] "谁来决定请哪几个专家？": top-k takes
    the k highest-scoring candidates."""
    return np.argsort(-np.asarray(z, F64), axis=1, kind="stable")


def select_topk(z: np.ndarray, k: int) -> np.ndarray:
    """Indices [T, k] of the k best experts per token, best first (int64)."""
    return expert_order(z)[:, :k].astype(np.int64)


def softmax(z: np.ndarray) -> np.ndarray:
    """Row softmax p_e = exp(z_e) / sum_e' exp(z_e') in float64 ([mlqm] §3.1)."""
    z64 = np.asarray(z, F64)
    ez = np.exp(z64 - z64.max(axis=1, keepdims=True))
    return ez / ez.sum(axis=1, keepdims=True)


def topk_weights(z: np.ndarray, idx: np.ndarray, mode: str = "renormalized") -> np.ndarray:
    """Routing weights of the selected experts s, float64 [T, k].

    mode "renormalized" (default): w_j = p_{s_j} / sum_i p_{s_i}.  [mlqm] §3.3: for top-2,
        w_i = p_i / (p_i + p_j); [mlqm] §4.2 divides the top-k probabilities by their sum.
    mode "softmax": w_j = p_{s_j}, the softmax probabilities themselves.  [cnnet] §3.2:
        output = p1 x e1 + p2 x e2; [wmrh] §5.1 weights by the top-k probabilities.
    """
    p = softmax(z)
    sel = np.take_along_axis(p, np.asarray(idx, np.int64), axis=1)
    if mode == "softmax":
        return sel
    if mode != "renormalized":
        raise ValueError(mode)
    return sel / sel.sum(axis=1, keepdims=True)


def topk_margin(z: np.ndarray, k: int) -> np.ndarray:
    """z_(k) - z_(k+1): gap between the k-th and (k+1)-th largest logit per token (fp64).
    Where it is tiny, a different summation order may legitimately flip the selection.
    +inf when k equals the number of experts."""
    z64 = np.asarray(z, F64)
    E = z64.shape[1]
    if k >= E:
        return np.full(z64.shape[0], np.inf)
    s = -np.sort(-z64, axis=1)
    return s[:, k - 1] - s[:, k]


# ----------------------------------------------------------------------------------
# Capacity and dispatch
# ----------------------------------------------------------------------------------
def capacity_rule(T: int, k: int, E: int, factor: float = 1.0, min_capacity: int = 0) -> int:
    """Per-expert capacity C = max(min_capacity, ceil(factor * T * k / E)).

    [rkmt] §2.3: with 1024 tokens, K=2 and 16 experts the capacity is (1024x2)/16 = 128.
    The page's example divides exactly; for a non-integral quotient the ceiling is taken
    so that a perfectly balanced load never drops a token.  [cnnet] §4.2 (DeepSpeed-MoE
    block): capacity_factor 1.2 in training, eval_capacity_factor 2.0 at inference, and
    min_capacity 4 as a floor for tiny batches.
    """
    return max(int(min_capacity), int(math.ceil(factor * T * k / E)))


def priority_order(T: int, k: int, priority: str = "token") -> List[Tuple[int, int]]:
    """Order in which slots (t, j) claim capacity.

    "token": ascending token, then slot - the earliest tokens are kept ([rkmt] §2.3 drops
    the tokens beyond an expert's capacity; arrival order is the plainest reading).
    "slot": every token's first choice before any second choice, tokens ascending within a
    slot position (first choices are protected from being displaced by second choices).
    """
    if priority == "token":
        return [(t, j) for t in range(T) for j in range(k)]
    if priority == "slot":
        return [(t, j) for j in range(k) for t in range(T)]
    raise ValueError(priority)


def dispatch(idx: np.ndarray, E: int, capacity: int = 0, priority: str = "token",
             overflow: str = "drop", z: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Group token slots by expert, apply the capacity, build the permutation.

    [rkmt] §2.3: each expert takes at most C tokens; the ones beyond it are dropped, or
    sent to the next-best expert.  [200B-5] "四个专家同时算…": every selection is one
    call of one expert, so sum(counts) = T*k.

    idx: [T, k] expert per slot.  capacity <= 0 means no limit.
    Slots claim capacity in priority_order(priority).
    overflow "drop": a slot beyond its expert's capacity is dropped.
    overflow "reroute" (needs the logits z [T, E]): first the router's choices claim
    capacity as with "drop"; then the overflowed slots, in the same priority order, each
    go to the token's best expert (descending logit, lowest index on ties) that is not
    among its top-k or its earlier re-routes and still has capacity, else are dropped.
    A re-routed slot keeps its routing weight.
    Returns
      counts  [E]    number of slots that selected each expert (demand)
      kept    [E]    rows each expert computes
      offsets [E+1]  exclusive prefix sum of kept
      perm    [R]    row r of the expert-sorted order holds slot t*k+j; the rows of one
                     expert are its router-chosen slots in priority order, then the
                     slots re-routed to it in re-route order
      inv     [T,k]  row of slot (t, j), or -1 if the slot was dropped
      expert  [T,k]  expert that computes slot (t, j), or -1 if dropped
      n_dropped      number of dropped slots
    """
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    order = priority_order(T, k, priority)
    if overflow not in ("drop", "reroute"):
        raise ValueError(overflow)
    counts = np.zeros(E, np.int64)
    for t in range(T):
        for j in range(k):
            counts[idx[t, j]] += 1
    expert = np.full((T, k), -1, np.int64)
    load = np.zeros(E, np.int64)
    placed = {e: [] for e in range(E)}
    overflowed = []
    for t, j in order:                              # the router's choices
        e = int(idx[t, j])
        if capacity <= 0 or load[e] < capacity:
            expert[t, j] = e
            load[e] += 1
            placed[e].append((t, j))
        else:
            overflowed.append((t, j))
    if overflow == "reroute" and overflowed:
        if z is None:
            raise ValueError("reroute needs the logits")
        pref = expert_order(z)
        used = [set(int(e) for e in idx[t]) for t in range(T)]
        for t, j in overflowed:                     # the next-best experts
            for e in pref[t]:
                e = int(e)
                if e in used[t]:
                    continue
                if load[e] < capacity:
                    expert[t, j] = e
                    load[e] += 1
                    placed[e].append((t, j))
                    used[t].add(e)
                    break
    kept = load.copy()
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(kept)
    perm = np.empty(int(offsets[-1]), np.int64)
    inv = np.full((T, k), -1, np.int64)
    for e in range(E):
        for r, (t, j) in enumerate(placed[e]):
            row = int(offsets[e]) + r
            perm[row] = t * k + j
            inv[t, j] = row
    return dict(counts=counts, kept=kept, offsets=offsets, perm=perm, inv=inv, expert=expert,
                n_dropped=int((expert < 0).sum()))


# ----------------------------------------------------------------------------------
# Expert FFN and combine
# ----------------------------------------------------------------------------------
def gelu(v: np.ndarray) -> np.ndarray:
    """Exact GeLU v * Phi(v) = 0.5 v (1 + erf(v / sqrt 2)) ([cnnet] and [rkmt] §3.3 use nn.GELU)."""
    v = np.asarray(v, F64)
    return 0.5 * v * (1.0 + _erf(v / math.sqrt(2.0)))


def silu(v: np.ndarray) -> np.ndarray:
    """SiLU v * sigmoid(v) = v / (1 + exp(-v))."""
    v = np.asarray(v, F64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def expert_ffn(xr: np.ndarray, act: str, w_gate: np.ndarray, w_up: Optional[np.ndarray],
               w_down: np.ndarray) -> np.ndarray:
    """One expert applied to the rows xr [n, d] (weights in nn.Linear layout, [out, in]).

    GeLU expert ([cnnet] DeepSpeed block, [rkmt] §3.3): y = W2 gelu(W1 x),
        w_gate = W1 [F, d], w_down = W2 [d, F], w_up unused.
    SwiGLU expert ([mlqm] §3.2 names SwiGLU): y = Wd (silu(Wg x) * (Wu x)),
        w_gate = Wg [F, d], w_up = Wu [F, d], w_down = Wd [d, F].
    """
    xr = np.asarray(xr, F64)
    g = xr @ np.asarray(w_gate, F64).T
    if act == "gelu":
        h = gelu(g)
    elif act == "swiglu":
        h = silu(g) * (xr @ np.asarray(w_up, F64).T)
    else:
        raise ValueError(act)
    return h @ np.asarray(w_down, F64).T


def combine(y_slots: np.ndarray, w: np.ndarray, keep: Optional[np.ndarray] = None,
            shared: Optional[np.ndarray] = None) -> np.ndarray:
    """out[t] = sum_j keep[t,j] * w[t,j] * y_slots[t,j] (+ shared[t]).

    [200B-5] "谁来决定请哪几个专家？": the selected experts' output vectors are mixed in
    proportion to the routing weights (0.75 x E1 + 0.25 x E3 in the worked example).
    [200B-5] "共享专家…": the shared expert's result is added to the routed result.
    y_slots: [T, k, d], w: [T, k], keep: [T, k] bool or None, shared: [T, d] or None.
    """
    y_slots = np.asarray(y_slots, F64)
    w = np.asarray(w, F64)
    if keep is not None:
        w = np.where(np.asarray(keep, bool), w, 0.0)
    out = np.einsum("tk,tkd->td", w, y_slots)
    if shared is not None:
        out = out + np.asarray(shared, F64)
    return out


ExpertWeights = Tuple[np.ndarray, Optional[np.ndarray], np.ndarray]


def routed_output(x_rows: np.ndarray, idx_rows: np.ndarray, w_rows: np.ndarray,
                  keep_rows: np.ndarray, act: str,
                  expert_weights: Callable[[int], ExpertWeights],
                  shared_weights: Optional[ExpertWeights] = None) -> np.ndarray:
    """Layer output for some tokens, given their routing (teacher-forced FFN + combine).

    x_rows [n, d]; idx_rows, w_rows, keep_rows [n, k].  expert_weights(e) returns
    (w_gate, w_up, w_down) of routed expert e; shared_weights those of the shared expert.
    Each expert is evaluated on the rows that selected it and kept the slot.
    """
    x_rows = np.asarray(x_rows, F64)
    n, k = idx_rows.shape
    y_slots = np.zeros((n, k, x_rows.shape[1]), F64)
    for e in np.unique(idx_rows[keep_rows]):
        sel = (idx_rows == e) & keep_rows
        tok, slot = np.nonzero(sel)
        y_slots[tok, slot] = expert_ffn(x_rows[tok], act, *expert_weights(int(e)))
    shared = None
    if shared_weights is not None:
        shared = expert_ffn(x_rows, act, *shared_weights)
    return combine(y_slots, w_rows, keep_rows, shared)


def moe_layer(x: np.ndarray, w_r: np.ndarray, k: int, act: str,
              w_gate: np.ndarray, w_up: Optional[np.ndarray], w_down: np.ndarray,
              bias: Optional[np.ndarray] = None, capacity: int = 0,
              shared: Optional[ExpertWeights] = None, weights: str = "renormalized",
              priority: str = "token", overflow: str = "drop") -> Dict[str, np.ndarray]:
    """Whole layer: router -> top-k -> weights -> capacity/dispatch -> experts -> combine.

    Follows [mlqm] §3.1-§3.3 and §4.2, [rkmt] §2.3 and [200B-5].  Stacked expert weights:
    w_gate [E, F, d], w_up [E, F, d] or None, w_down [E, d, F].
    Returns the float64 output [T, d] (unrounded) and every intermediate.
    """
    E = np.asarray(w_r).shape[1]
    z = router_logits(x, w_r, bias)
    idx = select_topk(z, k)
    w = topk_weights(z, idx, weights)
    disp = dispatch(idx, E, capacity, priority, overflow, z)
    keep = disp["inv"] >= 0
    out = routed_output(
        x, np.where(keep, disp["expert"], idx), w, keep, act,
        lambda e: (w_gate[e], None if w_up is None else w_up[e], w_down[e]),
        shared)
    res = dict(out=out, logits=z, idx=idx, w=w, margin=topk_margin(z, k))
    res.update(disp)
    return res


# ----------------------------------------------------------------------------------
# Ledgers
# ----------------------------------------------------------------------------------
def active_params(common: float, routed_total: float, E: int, k: int) -> float:
    """Parameters one token passes through: common + routed_total * k / E.

    [200B-5] "200B还在，为什么每次可以少算？": 40B common + 160B routed over 16 experts,
    2 selected -> 160B x 2 / 16 + 40B = 60B.
    """
    return common + routed_total * k / E


def expert_weight_bytes(E: int, d: int, F: int, act: str, bytes_per_elem: int) -> int:
    """Bytes of E stacked experts: 3 d F weights each for SwiGLU, 2 d F for GeLU."""
    mats = 3 if act == "swiglu" else 2
    return E * mats * d * F * bytes_per_elem


# ----------------------------------------------------------------------------------
# Routing statistics (monitoring and load-balance terms of one forward pass)
# ----------------------------------------------------------------------------------
def routing_stats(z: np.ndarray, counts: np.ndarray, n_dropped: int, k: int,
                  lambda_balance: float = 0.01, lambda_aux: float = 0.01, gamma_aux: float = 100.0
                  ) -> Dict[str, np.ndarray]:
    """Load-balance and monitoring statistics of one batch.

    u_e = counts_e / T, the fraction of tokens that selected expert e ([mlqm] §4.2: the
    mean over tokens of the summed one-hot selection mask; sum_e u_e = k).
      balance_ratio = std(u) / (mean(u) + 1e-8), std with Bessel's correction ([mlqm]
                      §4.2 code); L_balance = lambda_balance * balance_ratio ([mlqm] §3.1,
                      lambda = 0.01)
      l_aux         = lambda_aux * (std(u) + gamma_aux * max(u)) ([cnnet] §3.2, lambda = 0.01,
                      gamma = 100)
      utilization   = counts_e / (T k), each expert's share of all selections ([rkmt] §6.1;
                      16 balanced experts take 6.25% each, [rkmt] §2.3)
      drop_rate     = dropped slots / (T k) ([rkmt] §6.1 token_drop_rate)
      entropy       = mean over tokens of -sum_e p_e ln p_e, p = softmax(z) ([rkmt] §6.1
                      router_entropy; natural logarithm)
    """
    z64 = np.asarray(z, F64)
    T, E = z64.shape
    counts = np.asarray(counts, F64)
    u = counts / T
    std = float(np.std(u, ddof=1)) if E > 1 else 0.0
    ratio = std / (float(np.mean(u)) + 1e-8)
    p = softmax(z64)
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(p), 0.0)
    entropy = float(np.mean(-plogp.sum(axis=1)))
    return dict(balance_ratio=ratio, l_balance=lambda_balance * ratio,
                l_aux=lambda_aux * (std + gamma_aux * float(np.max(u))),
                utilization=counts / (T * k), drop_rate=n_dropped / (T * k), entropy=entropy)
