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


# sources that define each forward stage's kernels (besides the shared common.hpp / kernels.hpp)
STAGE_SOURCES = {"router": ("router.hip", "routing.hpp"), "dispatch": ("dispatch.hip", "routing.hpp"),
                 "gateup": ("grouped_gemm.hip",), "down": ("grouped_gemm.hip",), "combine": ("combine.hip",)}


def kernel_source_hash(stage=None):
    """Hash of the kernel sources: of every source, or of those that define one stage's kernels."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_mixture_experts_expert_amd", "csrc")
    names = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".hpp")))
    if stage is not None:
        names = sorted(set(STAGE_SOURCES[stage]) | {"common.hpp", "kernels.hpp"})
    for f in names:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload, stage):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != kernel_source_hash(stage):
        return None
    return rec.get("hbm_bytes_per_launch")


N_WEIGHT_SETS = 4   # single-layer steps cycle through distinct weight sets (3.2 GB, far above the 256 MB MALL)
EVENT_EVERY = 8     # the dominant kernel's events are recorded on one timed step in this many


def wl_layers_of(workload):
    from sparse_mixture_experts_expert_amd import inputs
    return inputs.WORKLOADS[workload].layers


def measure(workload, steps, warmup, seed=0, tokens=None):
    import torch
    from sparse_mixture_experts_expert_amd import binding, inputs

    wl = inputs.WORKLOADS[workload]
    T = wl.tokens if tokens is None else tokens
    d = inputs.device_workload(workload, seed=seed, tokens=T)
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
        # set 0 is the workload's own layer; the others are further layers of the same recipe, so
        # consecutive steps never find the previous step's weights in a cache
        sets = [d] + [inputs.device_weights(seed, workload, layer=r, skew=wl.skew)
                      for r in range(1, N_WEIGHT_SETS)]
        it = [0]

        def step():
            w = sets[it[0] % N_WEIGHT_SETS]
            it[0] += 1
            binding.moe_forward(d["x"], w["w_router"], w["w_gate"], w["w_up"], w["w_down"], out=out,
                                route_ids=ids, route_probs=probs, expert_counts=counts, aux_loss=aux,
                                z_loss=z, workspace=ws)
        touched_per_layer = []
        for _ in range(N_WEIGHT_SETS):
            step()
            touched_per_layer.append(int((counts > 0).sum().item()))
    else:
        h = d["h0"].clone()

        def step():
            binding.moe_stack_forward(h, d["layers"], workspace=ws)
        r = binding.moe_stack_forward(d["h0"].clone(), d["layers"], workspace=ws)
        sync()
        touched_per_layer = [int(v) for v in (r["expert_counts"] > 0).sum(1).tolist()]

    for _ in range(warmup):
        step()
    sync()
    # short pass with every stage bracketed: the per-stage split, and which expert GEMM dominates
    binding.timing_enable(True)
    for _ in range(max(3, steps // 5)):
        step()
    sync()
    stage_sum, calls = binding.timing_read()
    stage_ms = {k: v / calls for k, v in stage_sum.items()}     # per launch
    dom = max(("gateup", "down"), key=lambda s: stage_ms[s])
    # event-free pass: the plain wall clock of K steps
    binding.timing_enable(False)
    sync()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    sync()
    sec_plain = (time.perf_counter() - t0) / steps
    # timed region: K steps with the dominant kernel bracketed by HIP events on its launch stream,
    # on every EVENT_EVERY-th step (events on every call cost the step a few microseconds)
    binding.timing_enable([dom])
    binding.timing_every(EVENT_EVERY)
    sync()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    sync()
    sec = (time.perf_counter() - t0) / steps
    dom_sum, dom_calls = binding.timing_read()
    binding.timing_enable(False)
    dom_ms = dom_sum[dom] / dom_calls
    # per-call distribution: events around each call on the stream the layer runs on
    n_dist = min(steps, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_dist)]
    for a, b in evs:
        a.record()
        step()
        b.record()
    sync()
    per_call = sorted(a.elapsed_time(b) for a, b in evs)
    pick = lambda q: per_call[min(len(per_call) - 1, int(q * len(per_call)))]

    L = wl.layers
    touched = sum(touched_per_layer) / len(touched_per_layer)      # per layer call
    flop = FLOP_PER_TOKEN * T * L
    byts = layer_bytes(T, touched) * L
    f_k, b_k = stage_model(dom, T, touched)
    dur = dom_ms * 1e-3
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
    roof["kernel_ms"] = round(dom_ms, 5)
    roof["algorithmic_flop"] = f_k
    roof["algorithmic_bytes"] = b_k
    roof["traffic"] = traffic_from_profiles(workload, dom)
    res = {
        "workload": workload, "tokens": T, "layers": L, "sec": sec, "sec_plain": sec_plain,
        "tokens_per_s": T / sec, "tflops": flop / sec / 1e12, "hbm_gbs": byts / sec / 1e9,
        "layer_hbm_frac": byts / sec / 1e9 / HBM_PEAK_GBS,
        "layer_mfma_frac": flop / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "experts_touched": touched, "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "roofline": roof, "host_inputs": None,
        "per_call_ms": {"calls": n_dist, "p10": round(pick(0.1), 5), "median": round(pick(0.5), 5),
                        "p90": round(pick(0.9), 5)},
    }
    if wl.layers == 1:
        res["host_inputs"] = d
    return res


# backward: the gradient GEMMs are twice the forward's expert GEMMs (dgrad + wgrad), plus the
# router's two small products; the forward recomputed inside is not counted
BWD_FLOP_PER_TOKEN = 2 * K * 3 * 2 * D * F + 2 * 2 * D * E


def measure_backward(workload, steps, warmup, seed=0, routing="token"):
    """Wall-clock time per call of the backward pass (forward recompute + gradients), and of a
    training step of the layer: one forward call and one backward call.  routing "token" uses
    olmoe_moe_forward / olmoe_moe_backward, "expert" the expert-choice entry points."""
    import torch
    from sparse_mixture_experts_expert_amd import binding, inputs

    wl = inputs.WORKLOADS[workload]
    T = wl.tokens
    d = inputs.device_workload(workload, seed=seed)
    sets = [d] + [inputs.device_weights(seed, workload, layer=r, skew=wl.skew) for r in range(1, N_WEIGHT_SETS)]
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 7)
    dout = torch.randn((T, D), generator=g, device="cuda").to(torch.bfloat16)
    f32 = torch.float32
    dev = "cuda"
    outs = dict(dx=torch.empty((T, D), dtype=f32, device=dev),
                dw_router=torch.empty((E, D), dtype=f32, device=dev),
                dw_gate=torch.empty((E, F, D), dtype=f32, device=dev),
                dw_up=torch.empty((E, F, D), dtype=f32, device=dev),
                dw_down=torch.empty((E, D, F), dtype=f32, device=dev))
    y = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    aux = torch.empty(1, dtype=f32, device=dev)
    z = torch.empty(1, dtype=f32, device=dev)
    if routing == "expert":
        bws = torch.empty(binding.ec_backward_workspace_bytes(T), dtype=torch.uint8, device=dev)
        fws = torch.empty(binding.ec_workspace_bytes(T), dtype=torch.uint8, device=dev)
        C = binding.ec_capacity(T)
        ct = torch.empty((E, C), dtype=torch.int32, device=dev)
        tc = torch.empty(T, dtype=torch.int32, device=dev)

        def fwd(w):
            binding.moe_forward_expert_choice(d["x"], w["w_router"], w["w_gate"], w["w_up"], w["w_down"], out=y,
                                              choice_tokens=ct, token_counts=tc, choice_probs=None, aux_loss=aux,
                                              z_loss=z, workspace=fws, want_routing=False)

        def bwd(w):
            binding.moe_backward_expert_choice(d["x"], w["w_router"], w["w_gate"], w["w_up"], w["w_down"], dout,
                                               g_aux=1.0, g_z=1.0, workspace=bws, **outs)
    else:
        bws = torch.empty(binding.backward_workspace_bytes(T), dtype=torch.uint8, device=dev)
        fws = binding.make_workspace(T)
        ids = torch.empty((T, K), dtype=torch.int32, device=dev)
        cnt = torch.empty(E, dtype=torch.int32, device=dev)

        def fwd(w):
            binding.moe_forward(d["x"], w["w_router"], w["w_gate"], w["w_up"], w["w_down"], out=y, route_ids=ids,
                                expert_counts=cnt, aux_loss=aux, z_loss=z, workspace=fws, want_routing=False)

        def bwd(w):
            binding.moe_backward(d["x"], w["w_router"], w["w_gate"], w["w_up"], w["w_down"], dout, g_aux=1.0,
                                 g_z=1.0, workspace=bws, **outs)
    it = [0]

    def timed(fn_list):
        for _ in range(warmup):
            w = sets[it[0] % N_WEIGHT_SETS]
            it[0] += 1
            for fn in fn_list:
                fn(w)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            w = sets[it[0] % N_WEIGHT_SETS]
            it[0] += 1
            for fn in fn_list:
                fn(w)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps
    sec = timed([bwd])
    sec_train = timed([fwd, bwd])
    extra = {}
    if routing == "expert":   # the training pair: the forward keeps its state, the backward starts from it
        def fwd_train(w):
            binding.moe_forward_expert_choice_train(d["x"], w["w_router"], w["w_gate"], w["w_up"], w["w_down"],
                                                    saved=bws, out=y, choice_tokens=ct, token_counts=tc,
                                                    aux_loss=aux, z_loss=z)

        def bwd_saved(w):
            binding.moe_backward_expert_choice_saved(d["x"], w["w_router"], w["w_gate"], w["w_up"], w["w_down"],
                                                     dout, bws, g_aux=1.0, g_z=1.0, **outs)
        sec_pair = timed([fwd_train, bwd_saved])
        extra = {"train_step_saved_ms": round(sec_pair * 1e3, 5), "train_saved_tokens_per_s": round(T / sec_pair, 1)}
    if routing == "token":   # the training pair: the forward keeps its state, the backward starts from it
        def fwd_train(w):
            binding.moe_forward_train(d["x"], w["w_router"], w["w_gate"], w["w_up"], w["w_down"], saved=bws, out=y,
                                      expert_counts=cnt, aux_loss=aux, z_loss=z)

        def bwd_saved(w):
            binding.moe_backward_saved(d["x"], w["w_router"], w["w_gate"], w["w_up"], w["w_down"], dout, bws,
                                       g_aux=1.0, g_z=1.0, **outs)
        sec_pair = timed([fwd_train, bwd_saved])
        extra = {"train_step_saved_ms": round(sec_pair * 1e3, 5), "train_saved_tokens_per_s": round(T / sec_pair, 1)}
    # the same backward with the expert weight gradients returned in bf16 (OLMOE_BWD_GRAD_BF16)
    bf = torch.bfloat16
    outs16 = dict(outs, dw_gate=torch.empty((E, F, D), dtype=bf, device=dev),
                  dw_up=torch.empty((E, F, D), dtype=bf, device=dev), dw_down=torch.empty((E, D, F), dtype=bf, device=dev))
    flags16 = binding.BWD_GRAD_BF16 | (binding.BWD_EXPERT_CHOICE if routing == "expert" else 0)

    def bwd16(w):
        binding.moe_backward_ex(d["x"], w["w_router"], w["w_gate"], w["w_up"], w["w_down"], dout, flags=flags16,
                                g_aux=1.0, g_z=1.0, workspace=bws, **outs16)
    sec16 = timed([bwd16])
    extra.update({"grad_bf16_ms": round(sec16 * 1e3, 5), "grad_bf16_tokens_per_s": round(T / sec16, 1)})
    return {"routing": routing, "workload": workload, "tokens": T, "ms_per_step": round(sec * 1e3, 5), **extra,
            "tokens_per_s": round(T / sec, 1),
            "tflops": round(BWD_FLOP_PER_TOKEN * T / sec / 1e12, 2),
            "mfma_frac": round(BWD_FLOP_PER_TOKEN * T / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "train_step_ms": round(sec_train * 1e3, 5), "train_tokens_per_s": round(T / sec_train, 1),
            "note": "backward: gradients of x and all weights, the forward recompute inside timed, not counted "
                    "in tflops; train step: one forward call + one backward call; train step saved: the "
                    "training pair (forward keeping its state + backward from it, no recompute); grad bf16: "
                    "the backward with the expert weight gradients written in bf16"}


def measure_expert_choice(workload, steps, warmup, seed=0):
    """Wall-clock time of one expert-choice layer forward (olmoe_moe_forward_expert_choice) per
    call, with the per-stage split from a separate event-bracketed pass."""
    import torch
    from sparse_mixture_experts_expert_amd import binding, inputs

    wl = inputs.WORKLOADS[workload]
    T = wl.tokens
    d = inputs.device_workload(workload, seed=seed)
    sets = [d] + [inputs.device_weights(seed, workload, layer=r, skew=wl.skew) for r in range(1, N_WEIGHT_SETS)]
    C = binding.ec_capacity(T)
    dev = "cuda"
    outs = dict(out=torch.empty((T, D), dtype=torch.bfloat16, device=dev),
                choice_tokens=torch.empty((E, C), dtype=torch.int32, device=dev),
                choice_probs=torch.empty((E, C), dtype=torch.float32, device=dev),
                token_counts=torch.empty(T, dtype=torch.int32, device=dev),
                aux_loss=torch.empty(1, dtype=torch.float32, device=dev),
                z_loss=torch.empty(1, dtype=torch.float32, device=dev),
                workspace=torch.empty(binding.ec_workspace_bytes(T), dtype=torch.uint8, device=dev))
    it = [0]

    def step():
        w = sets[it[0] % N_WEIGHT_SETS]
        it[0] += 1
        binding.moe_forward_expert_choice(d["x"], w["w_router"], w["w_gate"], w["w_up"], w["w_down"], **outs)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    binding.timing_enable(True)
    for _ in range(max(3, steps // 5)):
        step()
    torch.cuda.synchronize()
    stage_sum, calls = binding.timing_read()
    binding.timing_enable(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    rows = E * C
    flop = 2 * T * D * E + rows * 3 * 2 * D * F
    return {"workload": workload, "tokens": T, "capacity": C, "ms_per_step": round(sec * 1e3, 5),
            "tokens_per_s": round(T / sec, 1), "tflops": round(flop / sec / 1e12, 2),
            "stage_ms": {k: round(v / calls, 5) for k, v in stage_sum.items()},
            "untouched_tokens": int((outs["token_counts"] == 0).sum().item()),
            "max_experts_per_token": int(outs["token_counts"].max().item())}


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
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{runs} oracle call(s) of {n} tokens of {workload} (first {n} rows), "
                      f"{el:.1f} s, float64 NumPy"}


def _cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


# ---------------------------------------------------------------------------
# rocprofv3 summaries: kernel-trace statistics and HBM traffic from counters
# ---------------------------------------------------------------------------
COPY_PROBE_BYTES = 1 << 30


def copy_probe():
    """A plain elementwise copy of known size (reads and writes 1 GiB), the calibration
    kernel for the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES}), flush=True)


def _stage_of(kernel_name):
    n = kernel_name
    if "ec_softmax" in n or "ec_choose" in n or "ec_combine" in n:
        return "expert_choice"
    for key in ("dgrad_kernel", "wgrad_kernel", "bwd_"):
        if key in n:
            return "backward"
    if "grouped_gemm_kernel" in n:
        cfg = n[n.index("Cfg<") + 4:n.index(">")].split(",")
        return "gateup" if cfg[4].strip() == "true" else "down"
    for key, stage in (("router", "router"), ("scan", "dispatch"), ("permute", "dispatch"),
                       ("combine_kernel", "combine"), ("rmsnorm", "rmsnorm"), ("residual", "residual")):
        if key in n:
            return stage
    return None


def _counter_rows(d):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        rows += list(csv.DictReader(open(f)))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


def _per_dispatch(rows, counter, select):
    """Median over dispatches of the counter's per-dispatch total, for kernels `select` accepts."""
    per = {}
    for r in rows:
        if r["Counter_Name"] == counter and select(r["Kernel_Name"]):
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    v = sorted(per.values())
    return (v[len(v) // 2], len(v)) if v else (None, 0)


def traffic_summary(args):
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE over the workload and over
    the copy probe) into per-launch HBM bytes per stage, scaled so that the copy probe reads
    and writes exactly its known size."""
    wl = args.workload
    fetch, write = _counter_rows(args.fetch_dir), _counter_rows(args.write_dir)
    cf, cw = _counter_rows(args.copy_fetch_dir), _counter_rows(args.copy_write_dir)
    is_copy = lambda n: "elementwise" in n
    copy_f, _ = _per_dispatch(cf, "FETCH_SIZE", is_copy)
    copy_w, _ = _per_dispatch(cw, "WRITE_SIZE", is_copy)
    kf = COPY_PROBE_BYTES / copy_f      # bytes per counted unit (nominally KiB)
    kw = COPY_PROBE_BYTES / copy_w
    lines = [f"# HBM traffic per launch, {wl}", "",
             "Counters FETCH_SIZE and WRITE_SIZE (rocprofv3, one counter per run), median over",
             "dispatches, scaled by the same counters for a plain 1 GiB elementwise copy",
             f"(torch.neg over float32: reads and writes {COPY_PROBE_BYTES} B).", "",
             f"- copy probe: FETCH_SIZE {copy_f:.1f}, WRITE_SIZE {copy_w:.1f} per dispatch",
             f"- scale: fetch {kf:.2f} B/unit, write {kw:.2f} B/unit",
             "- source hash per stage: of the files defining that stage's kernels (plus common.hpp",
             "  and kernels.hpp); bench.py reports traffic only while it matches", "",
             "| stage | dispatches | fetch bytes | write bytes | HBM bytes / launch | algorithmic bytes | ratio | source hash |",
             "|---|---|---|---|---|---|---|---|"]
    T = None
    from sparse_mixture_experts_expert_amd import inputs
    T = inputs.WORKLOADS[wl].tokens
    touched = args.touched
    for stage in ("router", "dispatch", "gateup", "down", "combine"):
        f, nf = _per_dispatch(fetch, "FETCH_SIZE", lambda n, st=stage: _stage_of(n) == st)
        w, nw = _per_dispatch(write, "WRITE_SIZE", lambda n, st=stage: _stage_of(n) == st)
        if f is None or w is None:
            continue
        fb, wb = f * kf, w * kw
        _, alg = stage_model(stage, T, touched)
        ratio = f"{(fb + wb) / alg:.3f}" if alg else "-"
        src_hash = kernel_source_hash(stage)
        lines.append(f"| {stage} | {nf} | {fb:.4g} | {wb:.4g} | {fb + wb:.4g} | {alg:.4g} | {ratio} | {src_hash} |")
        rec = {"workload": wl, "stage": stage, "hbm_bytes_per_launch": round(fb + wb),
               "fetch_bytes": round(fb), "write_bytes": round(wb), "algorithmic_bytes": alg,
               "source_hash": src_hash, "copy_scale_fetch": kf, "copy_scale_write": kw}
        with open(os.path.join(ROOT, "profiles", f"traffic_{stage}_{wl}.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
    lines += ["", "Commands (from the repository root, TMPDIR=/tmp):", "", "```"] + args.commands + ["```", ""]
    with open(os.path.join(ROOT, "profiles", f"traffic_{wl}.md"), "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


MFMA_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_BUSY_CU_CYCLES")
N_XCD, N_SIMD = 8, 1024          # MI355X: 8 XCDs, 256 CUs x 4 SIMDs
PEAK_CLOCK_GHZ = 2.4             # the clock the published MFMA peak assumes
FLOP_PER_MOP = 512               # SQ_INSTS_VALU_MFMA_MOPS_* count matrix work in units of 512 FLOP


def _durations_us(d, select):
    import csv
    import glob
    out = {}
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if select(r["Kernel_Name"]):
                out[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    return out


def mfma_summary(args):
    """Turn one rocprofv3 --kernel-trace --pmc run over MFMA_COUNTERS into the matrix-core
    utilisation of the grouped GEMMs: per dispatch, the average shader clock (GRBM_GUI_ACTIVE
    summed over the XCDs / duration), the fraction of SIMD cycles the MFMA unit was busy, the
    matrix work counted by the hardware against the algorithmic FLOP, and the duration-based
    fraction of the 2.5 PFLOP/s bf16 peak (medians over dispatches).  At full MFMA rate a busy
    cycle does peak/(SIMDs x 2.4 GHz) of work, so busy fraction x clock / 2.4 GHz should match the
    duration-based fraction."""
    from sparse_mixture_experts_expert_amd import inputs
    import statistics
    wl = args.workload
    T = inputs.WORKLOADS[wl].tokens
    rows = _counter_rows(args.mfma_dir)
    lines = [f"# Matrix-core utilisation of the grouped GEMMs, {wl}", "",
             "rocprofv3 --kernel-trace --pmc " + " ".join(MFMA_COUNTERS) + "; medians over dispatches.",
             f"clock = GRBM_GUI_ACTIVE / {N_XCD} XCDs / duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /"
             f" ({N_SIMD} SIMDs x clock cycles); counted FLOP = MOPS x {FLOP_PER_MOP};",
             "roofline = algorithmic FLOP / duration / 2.5 PFLOP/s; busy x clock/2.4 GHz is the same",
             "fraction seen from the counters.", "",
             "| stage | dispatches | duration us | clock GHz | MFMA busy | busy x clock/2.4 | roofline (duration) | "
             "counted / algorithmic FLOP | source hash |", "|---|---|---|---|---|---|---|---|---|"]
    for stage in ("gateup", "down"):
        sel = lambda n, st=stage: _stage_of(n) == st
        dur = _durations_us(args.mfma_dir, sel)
        per = {}
        for r in rows:
            if sel(r["Kernel_Name"]):
                per.setdefault(r["Counter_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
                per[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        ids = [i for i in dur if all(i in per.get(c, {}) for c in MFMA_COUNTERS[:2])]
        if not ids:
            continue
        clk, busy, frac, mops = [], [], [], []
        flop_alg, _ = stage_model(stage, T, args.touched)
        for i in ids:
            cycles = per["GRBM_GUI_ACTIVE"][i] / N_XCD
            clk.append(cycles / dur[i] / 1e3)
            busy.append(per["SQ_VALU_MFMA_BUSY_CYCLES"][i] / (N_SIMD * cycles))
            frac.append(flop_alg / (dur[i] * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12))
            mops.append(per.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", {}).get(i, 0.0) +
                        per.get("SQ_INSTS_VALU_MFMA_MOPS_F16", {}).get(i, 0.0))
        med = statistics.median
        rec = {"workload": wl, "stage": stage, "dispatches": len(ids), "duration_us": round(med(dur[i] for i in ids), 2),
               "clock_ghz": round(med(clk), 3), "mfma_busy": round(med(busy), 4),
               "busy_x_clock_over_peak_clock": round(med(busy) * med(clk) / PEAK_CLOCK_GHZ, 4),
               "roofline_frac_duration": round(med(frac), 4),
               "counted_flop": med(mops) * FLOP_PER_MOP, "algorithmic_flop": flop_alg,
               "source_hash": kernel_source_hash(stage)}
        lines.append(f"| {stage} | {len(ids)} | {rec['duration_us']:.1f} | {rec['clock_ghz']:.2f} | "
                     f"{rec['mfma_busy']:.3f} | {rec['busy_x_clock_over_peak_clock']:.3f} | "
                     f"{rec['roofline_frac_duration']:.3f} | {rec['counted_flop'] / flop_alg:.3f} | {rec['source_hash']} |")
        with open(os.path.join(ROOT, "profiles", f"mfma_{stage}_{wl}.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
    lines += ["", "Commands (from the repository root, TMPDIR=/tmp):", "", "```"] + args.commands + ["```", ""]
    with open(os.path.join(ROOT, "profiles", f"mfma_{wl}.md"), "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def stats_summary(args):
    """Short text summary of a rocprofv3 --kernel-trace --stats run."""
    import csv
    import glob
    fs = glob.glob(os.path.join(args.stats_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not fs:
        raise SystemExit(f"no kernel_stats.csv under {args.stats_dir}")
    rows = list(csv.DictReader(open(fs[0])))
    lines = [f"# Kernel durations, {args.workload}{' (' + args.profile_label + ')' if args.profile_label else ''}", "",
             "rocprofv3 --kernel-trace --stats; durations in microseconds per dispatch.", "",
             "| kernel | stage | calls | average | min | max |", "|---|---|---|---|---|---|"]
    for r in rows:
        n = r["Name"]
        st = _stage_of(n)
        if st is None:
            continue    # input generation and copies made by the harness around the layer
        short = n.replace("olmoe::(anonymous namespace)::", "").replace("void ", "")
        if "Cfg" in short:
            short = short[:short.index(">") + 1]
            for k in ("grouped_gemm_kernel", "dgrad_kernel", "wgrad_kernel"):
                short = short.replace(k + "<", k + " ")
        else:
            short = short.split("(")[0]
        lines.append(f"| {short} | {st} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", f"kernel sources hash: {kernel_source_hash()}", "",
              "Command (from the repository root, TMPDIR=/tmp):", "", "```"] + args.commands + ["```", ""]
    name = f"kernels_{args.profile_label + '_' if args.profile_label else ''}{args.workload}.md"
    with open(os.path.join(ROOT, "profiles", name), "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode-256")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--tokens", type=int, default=None, help="override the workload's token count")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass timing")
    ap.add_argument("--no-expert-choice", action="store_true", help="skip the expert-choice forward timing")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the 32-token, skewed 16384-token and 16-layer stack measurements")
    ap.add_argument("--copy-probe", action="store_true", help="run the counter-calibration copy and exit")
    ap.add_argument("--traffic-summary", action="store_true", help="summarise --pmc runs into profiles/")
    ap.add_argument("--mfma-summary", metavar="DIR", dest="mfma_dir",
                    help="summarise a --kernel-trace --pmc run over the MFMA counters into profiles/")
    ap.add_argument("--stats-summary", metavar="DIR", dest="stats_dir", help="summarise a --stats run")
    ap.add_argument("--profile-label", default="", help="extra word in the kernel summary's file name")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--copy-fetch-dir")
    ap.add_argument("--copy-write-dir")
    ap.add_argument("--touched", type=float, default=64.0, help="experts touched per layer (traffic model)")
    ap.add_argument("--command", dest="commands", action="append", default=[],
                    help="command line recorded in a summary (repeatable)")
    args = ap.parse_args()
    if args.mfma_dir:
        mfma_summary(args)
        return
    if args.traffic_summary:
        traffic_summary(args)
        return
    if args.stats_dir:
        stats_summary(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share: the library runs on a single MI355X "
              "(the data-parallel shard needs no communication); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe()
        return
    from sparse_mixture_experts_expert_amd import binding
    binding.lib()

    main_res = measure(args.workload, args.steps, args.warmup, args.seed, args.tokens)
    line = {
        "metric": METRIC,
        "value": round(main_res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["sec"] * 1e3, 5),
        "ms_per_step_without_events": round(main_res["sec_plain"] * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+fp16",
        "dtype_detail": "bf16 inputs, weights and output; gate/up GEMM on bf16 MFMA, down GEMM on f16 MFMA "
                        "(fp16 SwiGLU activations, W_down converted to fp16); fp32 accumulation, router "
                        "and softmax; fp16 expert outputs",
        "data": f"synthetic (seeded; N(0,1) tokens, N(0,0.02) weights, random init; "
                f"{N_WEIGHT_SETS if main_res['layers'] == 1 else main_res['layers']} distinct weight sets cycled)",
        "config": {"workload": args.workload, "tokens": main_res["tokens"], "layers": main_res["layers"],
                   "hidden": D, "expert_width": F, "experts": E, "top_k": K},
        "tflops": round(main_res["tflops"], 2),
        "hbm_gbs": round(main_res["hbm_gbs"], 1),
        "layer_hbm_frac": round(main_res["layer_hbm_frac"], 4),
        "layer_mfma_frac": round(main_res["layer_mfma_frac"], 4),
        "experts_touched": main_res["experts_touched"],
        "stage_ms": main_res["stage_ms"],
        "per_call_ms": main_res["per_call_ms"],
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
                             "ms_per_step_without_events": round(s["sec_plain"] * 1e3, 5),
                             "tflops": round(s["tflops"], 2), "layer_mfma_frac": round(s["layer_mfma_frac"], 4),
                             "stage_ms": s["stage_ms"], "per_call_ms": s["per_call_ms"],
                             "layer_hbm_frac": round(s["layer_hbm_frac"], 4), "roofline": s["roofline"]}
        d = None
    if not args.no_backward and wl_layers_of(args.workload) == 1:
        wls = [args.workload] + ([] if args.no_secondary or args.workload == "prefill-4096" else ["prefill-4096"])
        torch.cuda.empty_cache()
        line["backward"] = [measure_backward(w, max(5, args.steps // 5), 2, args.seed, routing=r)
                            for w in wls for r in ("token", "expert")]
    if not args.no_expert_choice and wl_layers_of(args.workload) == 1:
        wls = [args.workload] + ([] if args.no_secondary or args.workload == "prefill-4096" else ["prefill-4096"])
        torch.cuda.empty_cache()
        line["expert_choice"] = [measure_expert_choice(w, args.steps, min(args.warmup, 5), args.seed) for w in wls]
    if not args.no_other_configs and args.workload == "decode-256":
        torch.cuda.empty_cache()
        others = []
        for w in ("tiny-32", "skew-16384", "stack-16x8192"):
            r = measure(w, min(args.steps, 20), min(args.warmup, 3), args.seed)
            r.pop("host_inputs")
            others.append({"workload": w, "tokens": r["tokens"], "layers": r["layers"],
                           "ms_per_step": round(r["sec"] * 1e3, 5), "tokens_per_s": round(r["tokens_per_s"], 1),
                           "tflops": round(r["tflops"], 2), "layer_hbm_frac": round(r["layer_hbm_frac"], 4),
                           "layer_mfma_frac": round(r["layer_mfma_frac"], 4), "experts_touched": r["experts_touched"],
                           "per_call_ms": r["per_call_ms"], "roofline": r["roofline"]})
            torch.cuda.empty_cache()
        line["other_configs"] = others
    if not args.no_cpu:
        if d is None:
            from sparse_mixture_experts_expert_amd import inputs
            d = inputs.device_workload(args.workload, seed=args.seed)
        if "x" in d:
            line["cpu_baseline"] = cpu_baseline(d, args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
