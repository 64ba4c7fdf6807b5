"""Host-side checks that need no GPU: the seeded input recipe and the benchmark's command
line contract."""
import json
import os
import subprocess
import sys

import numpy as np
import torch

from sparse_mixture_experts_27_amd import synth
from sparse_mixture_experts_27_amd.configs import BY_NAME, CONFIGS, MoEConfig

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _small(**kw):
    base = dict(name="host", seed=41, T=33, d=64, E=5, k=2, F=128, act="swiglu", dtype="bf16", shared=True,
                bias_var=0.5)
    base.update(kw)
    return MoEConfig(**base)


def test_inputs_are_reproducible_and_per_expert():
    """Same config -> same bits; every expert (and the shared one) can be regenerated alone
    with the bits the stacked tensors hold (the benchmark's CPU baseline relies on it)."""
    cfg = _small()
    a, b = synth.make_inputs(cfg), synth.make_inputs(cfg)
    for name, t in a.items():
        if t is None:
            assert b[name] is None
            continue
        assert torch.equal(t.view(torch.int16) if t.dtype == torch.bfloat16 else t,
                           b[name].view(torch.int16) if t.dtype == torch.bfloat16 else b[name]), name
    for e in range(cfg.E):
        g, u, dn = synth.expert_weights(cfg, e)
        assert torch.equal(g, a["w_gate"][e]) and torch.equal(u, a["w_up"][e]) and torch.equal(dn, a["w_down"][e])
    sg, su, sd = synth.expert_weights(cfg, 0, shared=True)
    assert torch.equal(sg, a["s_gate"]) and torch.equal(su, a["s_up"]) and torch.equal(sd, a["s_down"])
    # a different config seed gives different values
    c = synth.make_inputs(_small(seed=42))
    assert not torch.equal(a["x"], c["x"])


def test_input_recipe_statistics():
    """x ~ N(0,1), gate/up ~ N(0,1/d), down ~ N(0,1/F), offsets ~ N(0, bias_var), bf16 values
    rounded to nearest even (exactly representable in bf16)."""
    cfg = _small(T=4096, d=256, E=4, F=512, shared=False, bias_var=0.5)
    inp = synth.make_inputs(cfg)
    x = inp["x"].float().numpy()
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    assert abs(inp["w_gate"].float().numpy().std() * np.sqrt(cfg.d) - 1.0) < 0.02
    assert abs(inp["w_down"].float().numpy().std() * np.sqrt(cfg.F) - 1.0) < 0.02
    assert inp["bias"].dtype == torch.float32 and inp["bias"].shape == (cfg.E,)
    assert inp["x"].dtype == torch.bfloat16
    f32 = _small(dtype="f32", shared=False)
    assert synth.make_inputs(f32)["x"].dtype == torch.float32


def test_workload_table():
    """The eight workloads and their shapes (the benchmark measures number 2, and number 5
    beside it)."""
    assert len(CONFIGS) == 8
    p = BY_NAME["prefill-e64"]
    assert (p.T, p.d, p.E, p.k, p.F, p.act, p.dtype) == (4096, 4096, 64, 2, 14336, "swiglu", "bf16")
    assert CONFIGS[2] is p
    assert BY_NAME["capacity-e16"].capacity == 128           # (1024 x 2) / 16
    assert BY_NAME["shared-routed-e16"].shared and BY_NAME["wide-e384-top6-shared"].shared
    assert BY_NAME["decode-e64"].T == 16
    cal = BY_NAME["capacity-e16-calibrated"]
    assert (cal.T, cal.E, cal.k, cal.capacity) == (1024, 16, 2, 128) and cal.bias_var == 0.0225


def test_bench_rejects_several_gpus():
    """One GPU only: --gpus N > 1 exits with a message before touching a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_bench_traffic_record_matches_the_sources():
    """The committed HBM-traffic record names the bench workload and layout, and its GEMM
    source hash matches the current source (else bench.py reports traffic as null)."""
    sys.path.insert(0, ROOT)
    import bench
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert t["workload"] == "prefill-e64" and t["weight_layout"] == "packed"
    fresh = t["ffn_source_sha256_16"] == bench.source_digest(bench.FFN_SOURCE)
    assert bench.measured_traffic("prefill-e64", "packed") == (t["hbm_bytes_per_launch"] if fresh else None)
    assert bench.measured_traffic("prefill-e64", "linear") is None
    alg = t["algorithmic_bytes_per_launch"]
    assert 1.0 <= t["hbm_bytes_per_launch"] / alg < 1.05
