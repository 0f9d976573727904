#!/usr/bin/env python3
"""Benchmark of the OLMoE MoE-layer forward on one MI355X.

    python bench.py [--workload decode-256] [--steps K] [--warmup W] [--gpus 1]

One step = one full layer forward through the C ABI (router, dispatch, gate/up,
down, combine) over one batch of synthetic tokens already resident in HBM; for
the 16-layer stack a step is the whole stack including RMSNorm and residual
updates.  Prints ONE JSON line with tokens/s, the roofline of the dominant
kernel (timed with HIP events on the launch stream, per stage) and the CPU
oracle's throughput on a bounded sample of the same workload.

The default workload is the decode-like batch T=256; the prefill batch T=4096
(the other token count the metric names) is measured the same way and reported
under "secondary" (skip it with --no-secondary).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + TFLOP/s and % HBM/MFMA roofline at T=256 and T=4096"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
D, F, E, K = 2048, 1024, 64, 8
RIDGE = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # FLOP per byte

# Algorithmic work (counts only what the layer needs: every touched expert's
# weights read once, activations read and written once, 8 experts x 3 GEMMs
# per token plus the router; unselected experts and tile padding excluded).
FLOP_PER_TOKEN = 2 * D * E + K * 3 * 2 * D * F            # 100,925,440
EXPERT_BYTES = 3 * F * D * 2                                # 12,582,912
GATEUP_EXPERT_BYTES = 2 * F * D * 2                         # 8,388,608
DOWN_EXPERT_BYTES = F * D * 2                               # 4,194,304


def layer_bytes(T, touched):
    return EXPERT_BYTES * touched + E * D * 4 + 2 * D * 2 * T


def stage_model(stage, T, touched):
    """(algorithmic FLOP, algorithmic bytes) of one launch of a stage."""
    rows = K * T
    if stage == "gateup":
        return 2 * rows * D * (2 * F), GATEUP_EXPERT_BYTES * touched + T * D * 2 + rows * F * 2
    if stage == "down":
        return 2 * rows * F * D, DOWN_EXPERT_BYTES * touched + rows * F * 2 + rows * D * 2
    if stage == "router":
        return 2 * T * D * E, T * D * 2 + E * D * 4 + rows * 9
    if stage == "combine":
        return 2 * rows * D, rows * D * 2 + T * D * 2 + rows * 8
    return 0, 0


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_mixture_experts_expert_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload, stage):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def time_steps(step, steps, warmup, sync):
    for _ in range(warmup):
        step()
    sync()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    sync()
    return (time.perf_counter() - t0) / steps


def measure(workload, steps, warmup, seed=0):
    import torch
    from sparse_mixture_experts_expert_amd import binding, inputs

    wl = inputs.WORKLOADS[workload]
    T = wl.tokens
    d = inputs.device_workload(workload, seed=seed)
    ws = binding.make_workspace(T)
    dev = "cuda"
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    aux = torch.empty(1, dtype=torch.float32, device=dev)
    z = torch.empty(1, dtype=torch.float32, device=dev)
    sync = torch.cuda.synchronize

    if wl.layers == 1:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
        ids = torch.empty((T, K), dtype=torch.int32, device=dev)
        probs = torch.empty((T, K), dtype=torch.float32, device=dev)

        def step():
            binding.moe_forward(d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"], out=out,
                                route_ids=ids, route_probs=probs, expert_counts=counts, aux_loss=aux,
                                z_loss=z, workspace=ws)
        step()
        sync()
        touched_per_layer = [int((counts > 0).sum().item())]
    else:
        h = d["h0"].clone()
        stack_ws = ws

        def step():
            binding.moe_stack_forward(h, d["layers"], workspace=stack_ws)
        r = binding.moe_stack_forward(d["h0"].clone(), d["layers"], workspace=stack_ws)
        sync()
        touched_per_layer = [int(v) for v in (r["expert_counts"] > 0).sum(1).tolist()]

    sec = time_steps(step, steps, warmup, sync)

    # per-stage durations with HIP events on the launch stream (separate pass)
    binding.timing_enable(True)
    for _ in range(steps):
        step()
    sync()
    stage_sum, calls = binding.timing_read()
    binding.timing_enable(False)
    stage_ms = {k: v / calls for k, v in stage_sum.items()}     # per launch

    L = wl.layers
    touched = sum(touched_per_layer) / L
    flop = FLOP_PER_TOKEN * T * L
    byts = sum(layer_bytes(T, t) for t in touched_per_layer)
    dom = max(("gateup", "down"), key=lambda s: stage_ms[s])
    f_k, b_k = stage_model(dom, T, touched)
    dur = stage_ms[dom] * 1e-3
    intensity = f_k / b_k
    if intensity < RIDGE:
        achieved = b_k / dur / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = f_k / dur / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof["kernel"] = dom
    roof["kernel_ms"] = round(stage_ms[dom], 5)
    roof["algorithmic_flop"] = f_k
    roof["algorithmic_bytes"] = b_k
    roof["traffic"] = traffic_from_profiles(workload, dom)
    res = {
        "workload": workload, "tokens": T, "layers": L, "sec": sec,
        "tokens_per_s": T / sec, "tflops": flop / sec / 1e12, "hbm_gbs": byts / sec / 1e9,
        "layer_hbm_frac": byts / sec / 1e9 / HBM_PEAK_GBS,
        "layer_mfma_frac": flop / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "experts_touched": touched, "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "roofline": roof, "host_inputs": None,
    }
    if wl.layers == 1:
        res["host_inputs"] = d
    return res


def cpu_baseline(d, workload, budget_s=20.0):
    """The float64 oracle, as it stands, on a bounded sample of the workload."""
    import numpy as np
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    x = bits(d["x"])
    wr = d["w_router"].cpu().numpy()
    wg, wu, wd = bits(d["w_gate"]), bits(d["w_up"]), bits(d["w_down"])
    T = x.shape[0]
    n = min(T, 256)
    t0 = time.perf_counter()
    done = 0
    runs = 0
    while True:
        oracle.moe_layer_ref(x[done % T:done % T + n], wr, wg, wu, wd, 8)
        done += n
        runs += 1
        if time.perf_counter() - t0 > budget_s or runs >= 8:
            break
    el = time.perf_counter() - t0
    return {"value": round(done / el, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{runs} oracle call(s) of {n} tokens of {workload} (first {n} rows), "
                      f"{el:.1f} s, float64 NumPy"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode-256")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share: this build runs on a single MI355X "
              "(the data-parallel shard needs no communication); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)
    from sparse_mixture_experts_expert_amd import binding
    binding.lib()

    main_res = measure(args.workload, args.steps, args.warmup, args.seed)
    line = {
        "metric": METRIC,
        "value": round(main_res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["sec"] * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; N(0,1) tokens, N(0,0.02) weights, random init)",
        "config": {"workload": args.workload, "tokens": main_res["tokens"], "layers": main_res["layers"],
                   "hidden": D, "expert_width": F, "experts": E, "top_k": K},
        "tflops": round(main_res["tflops"], 2),
        "hbm_gbs": round(main_res["hbm_gbs"], 1),
        "layer_hbm_frac": round(main_res["layer_hbm_frac"], 4),
        "layer_mfma_frac": round(main_res["layer_mfma_frac"], 4),
        "experts_touched": main_res["experts_touched"],
        "stage_ms": main_res["stage_ms"],
        "roofline": main_res["roofline"],
    }
    d = main_res.pop("host_inputs")
    if not args.no_secondary and args.workload != "prefill-4096":
        del d
        torch.cuda.empty_cache()
        s = measure("prefill-4096", args.steps, args.warmup, args.seed)
        s.pop("host_inputs")
        line["secondary"] = {"workload": "prefill-4096", "value": round(s["tokens_per_s"], 1),
                             "unit": "tokens/s", "ms_per_step": round(s["sec"] * 1e3, 5),
                             "tflops": round(s["tflops"], 2), "layer_mfma_frac": round(s["layer_mfma_frac"], 4),
                             "stage_ms": s["stage_ms"], "roofline": s["roofline"]}
        d = None
    if not args.no_cpu:
        if d is None:
            from sparse_mixture_experts_expert_amd import inputs
            d = inputs.device_workload(args.workload, seed=args.seed)
        if "x" in d:
            line["cpu_baseline"] = cpu_baseline(d, args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
