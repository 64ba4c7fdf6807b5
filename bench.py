#!/usr/bin/env python3
"""Benchmark of the MoE-layer forward on one MI355X.

Workload (default): the prefill-shaped layer with E=64 experts, top-2, T=4096 tokens,
d=4096, SwiGLU experts of width 14336, bf16 weights/activations, fp32 router logits and
accumulation; seeded synthetic inputs and random-init weights resident in HBM.
A step is one moe_layer_forward (route, dispatch, grouped expert FFN, combine).

Prints ONE JSON line: tokens/s, the roofline of the dominant kernel (the gate/up grouped
GEMM) measured with HIP events recorded by the library on its stream, and the CPU
oracle timed on a bounded sample of the same workload.  The default run also measures
the decode-shaped layer (T=16, same E, k, d, F) and reports it as the `decode` object:
its tokens/s and the fraction of the HBM bandwidth its touched experts' weights reach.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2,
                    help="workload number 1-8 (default 2: prefill, E=64; the decode workload, 5, is then "
                         "measured in the same run and reported as the `decode` object)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode workload of the default run")
    ap.add_argument("--tile", default=None, metavar="ROWS,WAVES",
                    help="explicit tile of the expert FFN (moe_tile_t), e.g. 256,4; default: the library's choice")
    ap.add_argument("--priority", choices=("token", "slot"), default=None,
                    help="capacity priority (default: the workload's, token-major)")
    ap.add_argument("--overflow", choices=("drop", "reroute"), default=None,
                    help="fate of a slot beyond capacity (default: the workload's, drop)")
    ap.add_argument("--layout", choices=("packed", "linear"), default="packed",
                    help="storage order of the expert weights in HBM (default packed: reordered once "
                         "at load time by moe_pack_weights; linear: the nn.Linear layout as given)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one layer forward captured in a HIP graph (no per-launch host "
                         "overhead); the stage times then come from an extra eager pass of the same kernels")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-experts", type=int, default=1024,
                    help="experts whose rows the CPU oracle computes for its timed sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times): the reference "
                         "kernel whose FETCH_SIZE / WRITE_SIZE counters calibrate the HBM byte counts")
    return ap.parse_args()


FFN_SOURCE = os.path.join(ROOT, "sparse_mixture_experts_27_amd", "csrc", "moe_ffn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_up_prefill_e64_traffic.json")


def source_digest(path: str) -> str:
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(cfg_name: str, layout: str):
    """HBM bytes per launch of the gate/up GEMM from the committed counter summary, or None
    when there is none for this workload and weight layout or the GEMM source changed
    since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("workload") != cfg_name or t.get("weight_layout") != layout
            or t.get("ffn_source_sha256_16") != source_digest(FFN_SOURCE)):
        return None
    return t.get("hbm_bytes_per_launch")


def copy_calibration(mib: int):
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_launch": n * 4, "bytes_written_per_launch": n * 4,
                      "launches": 3}), flush=True)


def layer_counts(cfg, L):
    offsets = L.offsets.cpu().numpy().astype(np.int64)
    kept = np.diff(offsets)
    touched = int((kept > 0).sum())
    rows = int(kept.sum())
    return kept, touched, rows


def algorithmic(cfg, touched, rows):
    """What the method must touch, per stage and for the whole layer: the weights of the
    touched experts once, the hidden states x once, the output once (and W_r), and the
    flops of the kept rows.  The hidden activation H (written by gate/up, read by down) and
    the per-row expert outputs are implementation traffic: reported, not counted."""
    b = 2 if cfg.dtype == "bf16" else 4
    mats_up = 2 if cfg.act == "swiglu" else 1
    T, d, F, E = cfg.T, cfg.d, cfg.F, cfg.E
    sh_rows = T if cfg.shared else 0
    n_exp = touched + (1 if cfg.shared else 0)
    up_bytes = n_exp * mats_up * F * d * b + T * d * b
    up_flops = 2.0 * (rows + sh_rows) * F * d * mats_up
    down_bytes = n_exp * d * F * b
    down_flops = 2.0 * (rows + sh_rows) * d * F
    layer_bytes = n_exp * (mats_up + 1) * F * d * b + T * d * b + d * E * b + T * d * b
    layer_flops = 2.0 * T * d * E + up_flops + down_flops
    impl = dict(h_write=(rows + sh_rows) * F * b, h_read=(rows + sh_rows) * F * b, y_write=(rows + sh_rows) * d * 4)
    return dict(up_bytes=up_bytes, up_flops=up_flops, down_bytes=down_bytes, down_flops=down_flops,
                layer_bytes=layer_bytes, layer_flops=layer_flops, impl=impl)


def roofline(bytes_, flops, seconds, dtype):
    ai = flops / bytes_
    peak_t = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_F32_TFLOPS
    ridge = peak_t * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ai < ridge:
        a = bytes_ / seconds / 1e9
        return dict(bound="hbm", achieved=round(a, 1), peak=PEAK_HBM_GBS, unit="GB/s", frac=round(a / PEAK_HBM_GBS, 4))
    a = flops / seconds / 1e12
    return dict(bound="mfma" if dtype == "bf16" else "alu", achieved=round(a, 1), peak=peak_t, unit="TFLOP/s",
                frac=round(a / peak_t, 4))


def cpu_baseline(cfg, inp, L, n_exp):
    """The oracle, as it stands, timed on the host cores: routing and dispatch of all T
    tokens, then, for the first n_exp touched experts (all of them by default), the FFN
    of every row routed there and its weighted contribution to the output.  Each expert's
    weights are regenerated from their seed on the GPU (the bits the layer was given, in
    the nn.Linear layout) and converted to float64 outside the timed region.
    Tokens-equivalent = rows computed / k."""
    from oracle import moe_oracle as O
    from sparse_mixture_experts_27_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    x64 = synth.to_numpy(inp["x"])
    wr64 = synth.to_numpy(inp["w_r"])
    b64 = synth.to_numpy(inp["bias"])
    t0 = time.perf_counter()
    z = O.router_logits(x64, wr64, b64)
    idx = O.select_topk(z, cfg.k)
    w = O.topk_weights(z, idx, cfg.weights)
    dp = O.dispatch(idx, cfg.E, cfg.capacity, cfg.priority, cfg.overflow, z)
    out = np.zeros((cfg.T, cfg.d))
    t_oracle = time.perf_counter() - t0
    kept = np.diff(dp["offsets"])
    experts = [int(e) for e in np.nonzero(kept)[0][:n_exp]]
    rows = 0
    for e in experts:
        wts = tuple(synth.to_numpy(t) for t in synth.expert_weights(cfg, e, inp["x"].device))
        r = np.arange(dp["offsets"][e], dp["offsets"][e + 1])
        slots = dp["perm"][r]
        tok, j = slots // cfg.k, slots % cfg.k
        t1 = time.perf_counter()
        y = O.expert_ffn(x64[tok], cfg.act, *wts)
        np.add.at(out, tok, w[tok, j][:, None] * y)          # this expert's share of the combine
        t_oracle += time.perf_counter() - t1
        rows += len(r)
        del wts, y
    tokens_equiv = rows / cfg.k
    whole = len(experts) == int((kept > 0).sum())
    what = "the whole layer" if whole else f"{rows} of {int(kept.sum())} routed rows ({len(experts)} experts)"
    if cfg.shared:
        what += " (routed experts only: the shared expert is not timed)"
    return dict(value=round(tokens_equiv / t_oracle, 2), unit="tokens/s", cores=int(threads), kind="oracle",
                sample=(f"{cfg.name}: routing + dispatch of all {cfg.T} tokens and FFN + combine of {what} "
                        f"(= {tokens_equiv:.0f} token-equivalents), float64 numpy, {t_oracle:.1f} s of oracle time"),
                seconds=round(t_oracle, 2))


def load_layer(cfg, packed, tile=None):
    """Seeded inputs of the workload on cuda:0 and its layer (expert weights packed once at
    load time, one tensor at a time, each linear copy freed once its packed copy exists)."""
    import torch
    from sparse_mixture_experts_27_amd import binding as B
    from sparse_mixture_experts_27_amd import synth
    dev = torch.device("cuda", 0)
    inp = synth.make_inputs(cfg, dev)
    if packed:
        for name in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
            if inp[name] is not None:
                inp[name] = B.pack_weights(inp[name])
                torch.cuda.synchronize()
                torch.cuda.empty_cache()
    L = B.Layer(inp["w_r"], inp["w_gate"], inp["w_up"], inp["w_down"], cfg.k, act=cfg.act, bias=inp["bias"],
                capacity=cfg.capacity, s_gate=inp["s_gate"], s_up=inp["s_up"], s_down=inp["s_down"],
                weights=cfg.weights, priority=cfg.priority, overflow=cfg.overflow, prepacked=packed, tile=tile)
    return inp, L


def time_layer(cfg, L, x, steps, warmup, graph):
    """Warm-up, then `steps` forwards between two synchronisations -> (seconds, stage ms).
    The library records its stage events on its stream in every timed eager step."""
    import torch
    from sparse_mixture_experts_27_amd import binding as B
    for _ in range(warmup):
        L(x)
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        row = [torch.cuda.Event(enable_timing=True) for _ in range(B.STAGE_EVENTS)]
        for e in row:
            e.record()                           # create the underlying HIP events
        evs.append(row)
    torch.cuda.synchronize()
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            L(x)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        for i in range(steps):                   # stage times: the same kernels, eager
            L(x, stage_events=evs[i])
        torch.cuda.synchronize()
    else:
        t0 = time.perf_counter()
        for i in range(steps):
            L(x, stage_events=evs[i])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    stage_ms = {name: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)]))
                for j, name in enumerate(B.STAGES)}
    return elapsed, stage_ms


def measure(cfg, args, packed, graph):
    """One workload: tokens/s, the rooflines of its GEMMs and of the whole step, routing
    facts, and (unless disabled) the oracle baseline."""
    import torch
    tile = tuple(int(v) for v in args.tile.split(",")) if args.tile else None
    inp, L = load_layer(cfg, packed, tile)
    elapsed, stage_ms = time_layer(cfg, L, inp["x"], args.steps, args.warmup, graph)
    ms_step = elapsed / args.steps * 1e3
    kept, touched, rows = layer_counts(cfg, L)
    alg = algorithmic(cfg, touched, rows)
    up_s = stage_ms["ffn_up"] / 1e3
    roof = roofline(alg["up_bytes"], alg["up_flops"], up_s, cfg.dtype)
    roof["algorithmic_bytes"] = int(alg["up_bytes"])
    roof["kernel"] = "ffn_gemm_bf16_kernel<SwiGLU up>" if cfg.dtype == "bf16" else "ffn_gemm_f32_kernel<up>"
    peak_t = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    mfma_t = alg["up_flops"] / up_s / 1e12
    out = dict(
        value=round(cfg.T * args.steps / elapsed, 1),
        ms_per_step=round(ms_step, 4),
        roofline=roof,
        mfma_utilization=dict(kernel=roof["kernel"], achieved=round(mfma_t, 1), peak=peak_t, unit="TFLOP/s",
                              frac=round(mfma_t / peak_t, 4)),
        layer_roofline=roofline(alg["layer_bytes"], alg["layer_flops"], ms_step / 1e3, cfg.dtype),
        down_roofline=roofline(alg["down_bytes"], alg["down_flops"], stage_ms["ffn_down"] / 1e3, cfg.dtype),
        implementation_bytes=alg["impl"],
        stage_ms={k: round(v, 4) for k, v in stage_ms.items()},
        plan=L.plan(cfg.T),
        routing={"touched_experts": touched, "rows": rows, "load_min": int(kept.min()),
                 "load_max": int(kept.max()), "n_dropped": int(L.n_dropped.item()),
                 "drop_rate": round(int(L.n_dropped.item()) / (cfg.T * cfg.k), 4)},
    )
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, L, args.cpu_experts)
    del L, inp
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the layer runs on a "
              "single MI355X (expert-parallel sharding over several GPUs is designed, not built).", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_mixture_experts_27_amd import binding as B
    from sparse_mixture_experts_27_amd.configs import CONFIGS

    cfg = CONFIGS[args.config]
    if args.priority or args.overflow:
        cfg = cfg.scaled(priority=args.priority or cfg.priority, overflow=args.overflow or cfg.overflow)
    B.lib()                                  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    packed = args.layout == "packed" and cfg.dtype == "bf16"
    m = measure(cfg, args, packed, args.graph)
    m["roofline"]["traffic"] = measured_traffic(cfg.name, "packed" if packed else "linear")

    line = {
        "metric": "MoE-layer tokens/s at E=64,k=2; % bf16 MFMA peak (prefill), % HBM BW (decode)",
        "value": m["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) hidden states, N(0,1/fan_in) random-init weights)",
        "config": {"workload": cfg.label, "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k, "F": cfg.F,
                   "act": cfg.act, "shared": cfg.shared, "capacity": cfg.capacity, "priority": cfg.priority,
                   "overflow": cfg.overflow, "weight_layout": "packed" if packed else "linear",
                   "launch": "hip graph replay" if args.graph else "eager",
                   "parallelism": "single-gpu"},
    }
    line.update({k: v for k, v in m.items() if k not in ("value", "ms_per_step")})
    # the metric's other half: the decode-shaped layer (E=64, k=2, T=16), measured in the
    # same process on its own seeded weights, against the HBM roofline of the weights of
    # the experts it touches
    if args.config == 2 and not args.no_decode:
        dcfg = CONFIGS[5]
        dm = measure(dcfg, args, packed, args.graph)
        line["decode"] = {"workload": dcfg.label, "value": dm["value"], "unit": "tokens/s",
                          "ms_per_step": dm["ms_per_step"], "roofline": dm["layer_roofline"],
                          "gate_up_roofline": dm["roofline"], "down_roofline": dm["down_roofline"],
                          "stage_ms": dm["stage_ms"], "plan": dm["plan"], "routing": dm["routing"]}
        if "cpu_baseline" in dm:
            line["decode"]["cpu_baseline"] = dm["cpu_baseline"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
