"""moe_layer_forward_noalloc: the layer on the library's fixed device scratch.

Checked against moe_layer_forward (the same kernels on a caller workspace): outputs and
routing results bit-identical, on two calls in a row with the second on fewer tokens,
and the first call also against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from sparse_mixture_experts_27_amd import binding as B
from sparse_mixture_experts_27_amd import synth
from sparse_mixture_experts_27_amd.configs import MoEConfig
from tests.gpu_helpers import check_dispatch, check_output, check_route, expert_fetcher, say, shared_weights

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = {
    "bf16-shared-capacity-reroute": MoEConfig("noalloc-bf16", 91, T=300, d=512, E=16, k=2, F=1024, act="swiglu",
                                              dtype="bf16", shared=True, capacity=50, bias_var=0.5,
                                              overflow="reroute"),
    "bf16-decode": MoEConfig("noalloc-decode", 92, T=16, d=1024, E=64, k=2, F=2048, act="swiglu", dtype="bf16"),
    "f32-gelu": MoEConfig("noalloc-f32", 93, T=64, d=64, E=4, k=2, F=128, act="gelu", dtype="f32"),
}


def _layer(cfg, inp, noalloc):
    packed = cfg.dtype == "bf16"
    return B.Layer(inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.k, act=cfg.act, bias=inp["bias"],
                   capacity=cfg.capacity, s_gate=inp["s_gate"], s_up=inp["s_up"], s_down=inp["s_down"],
                   overflow=cfg.overflow, prepacked=packed, noalloc=noalloc)


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_workspace_entry_point(name):
    cfg = CASES[name]
    inp = synth.make_inputs(cfg, DEV)
    x_all = inp["x"]
    if cfg.dtype == "bf16":
        for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
            if inp[n] is not None:
                inp[n] = B.pack_weights(inp[n])
    Lw, Ln = _layer(cfg, inp, False), _layer(cfg, inp, True)
    assert Ln.ws is None if hasattr(Ln, "ws") else True
    for i, T in enumerate((cfg.T, cfg.T // 2 + 1)):
        x = x_all[:T].contiguous()
        say(f"[case] no-alloc {cfg.label} call {i + 1}: T={T}")
        got = Ln(x).clone()
        ref = Lw(x).clone()
        torch.cuda.synchronize()
        assert Ln.ws is None
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), f"call {i + 1}: output differs"
        for f in ("topk_idx", "topk_w", "logits", "counts", "offsets", "inv", "n_dropped"):
            assert torch.equal(getattr(Ln, f), getattr(Lw, f)), f"call {i + 1}: {f} differs"
        R = int(Lw.offsets[-1].item())
        assert torch.equal(Ln.perm[:R], Lw.perm[:R])
        if i == 0:                                   # and the first call against the oracle
            sub = cfg.scaled(T=T)
            res = dict(out=got.float().cpu().numpy().astype(np.float64),
                       idx=Ln.topk_idx.cpu().numpy().astype(np.int64), w=Ln.topk_w.cpu().numpy().astype(np.float64),
                       logits=Ln.logits.cpu().numpy(), counts=Ln.counts.cpu().numpy().astype(np.int64),
                       offsets=Ln.offsets.cpu().numpy().astype(np.int64), perm=Ln.perm.cpu().numpy().astype(np.int64),
                       inv=Ln.inv.cpu().numpy().astype(np.int64), n_dropped=int(Ln.n_dropped.item()))
            x64, wr64, b64 = synth.to_numpy(x), synth.to_numpy(inp["w_r"]), synth.to_numpy(inp["bias"])
            rep = {}
            z_o, _ = check_route(sub, x64, wr64, b64, res, rep)
            check_dispatch(sub, res)
            lin = synth.make_inputs(cfg, DEV)             # the oracle reads the nn.Linear layout
            check_output(sub, x64, z_o, res, expert_fetcher(cfg, lin), shared_weights(lin), None, rep)
            say(f"[ok] no-alloc vs oracle: {rep}")


def _packed(cfg):
    inp = synth.make_inputs(cfg, DEV)
    for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
        if inp[n] is not None:
            inp[n] = B.pack_weights(inp[n])
    return inp


def test_noalloc_graph_replay():
    """The fixed-scratch entry point captured in a HIP graph (the callers it is for): every
    replay, with a new input copied into the captured buffer and another layer's
    fixed-scratch calls in between (they overwrite the shared scratch), gives the bits of
    the workspace entry point on the same input."""
    cfg = CASES["bf16-decode"]
    inp = _packed(cfg)
    Lw, Ln = _layer(cfg, inp, False), _layer(cfg, inp, True)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(cfg.seed + 1)
    xs = [inp["x"], torch.randn(inp["x"].shape, generator=gen, device=DEV).to(inp["x"].dtype)]
    ref = [Lw(x).clone() for x in xs]
    _ = Ln(xs[0])                                    # first call on the device, outside the capture
    x_static = xs[0].clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = Ln(x_static)
    ocfg = CASES["bf16-shared-capacity-reroute"]
    oinp = _packed(ocfg)
    Lo = _layer(ocfg, oinp, True)
    for i in (1, 0, 1, 1, 0):
        x_static.copy_(xs[i])
        g.replay()
        torch.cuda.synchronize()
        say(f"[case] no-alloc graph replay {cfg.label} input {i}")
        assert torch.equal(out.view(torch.int32), ref[i].view(torch.int32)), i
        _ = Lo(oinp["x"]).sum().item()
