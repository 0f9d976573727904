"""Seeded synthetic inputs for the OLMoE MoE layer.

This module only draws random numbers and rounds them to the storage types the
layer takes (bf16 activations and expert weights, fp32 router weights). It
holds none of the layer's arithmetic, so both the GPU path and the CPU oracle
can be fed from it.

Workloads (all sizes from the OLMoE architecture: hidden 2048, expert width
1024, 64 experts, top-8; see "OLMoE Guide: 64-Expert Fine-Grained Open MoE
Architecture", table "1. Model Specifications & Dimensionality"):

  tiny-32      T=32      x ~ N(0,1), router fp32 ~ N(0,0.02), experts bf16 ~ N(0,0.02)
  decode-256   T=256     same recipe
  prefill-4096 T=4096    same, then 1% of the rows (round(0.01*T), drawn without
                         replacement) multiplied by 8 after bf16 rounding (exact)
  skew-16384   T=16384   same, plus a per-expert router bias b_e = -2.4*ln(rank_e)
                         over a random ranking rank = 1 + permutation(64),
                         folded into the fixed interface as x[:,2047] = 1 and
                         W_router[e,2047] = b_e
  stack-16x8192 T=8192   16 layers with their own weights; the residual stream
                         h0 ~ N(0,1) is kept in fp32

The weight scale 0.02 is the initialisation standard deviation quoted for
OLMoE's pretraining ("OLMoE: Open Mixture-of-Experts Language Models",
"Pretraining" under B Training Configuration); plain normals are drawn instead
of truncated ones.

Two generators exist: NumPy PCG64 on the host (small tests) and torch's
generator on the device (full-size runs, where drawing 6.4e9 normals on the
host would be slow). Parity never depends on which one made the bytes: the
oracle always receives the bytes the GPU used.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

D_MODEL = 2048
D_EXPERT = 1024
N_EXPERTS = 64
TOP_K = 8
WEIGHT_STD = 0.02

# tensor ids for sub-seeds
_X, _WR, _WG, _WU, _WD, _ROWS, _RANK = range(7)


@dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    layers: int = 1
    scaled_rows_frac: float = 0.0   # share of x rows multiplied by 8
    skew: bool = False              # fold a Zipf-like router bias into x / W_router


WORKLOADS = {
    "tiny-32": Workload("tiny-32", 32),
    "decode-256": Workload("decode-256", 256),
    "prefill-4096": Workload("prefill-4096", 4096, scaled_rows_frac=0.01),
    "skew-16384": Workload("skew-16384", 16384, skew=True),
    "stack-16x8192": Workload("stack-16x8192", 8192, layers=16),
}
WORKLOAD_IDS = {name: i for i, name in enumerate(WORKLOADS)}


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest even); return the bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def skew_bias(rank: np.ndarray) -> np.ndarray:
    """Router bias of the skewed workload: 2.0 * ln(1 / rank**1.2), natural log."""
    return (2.0 * np.log(1.0 / np.power(rank.astype(np.float64), 1.2))).astype(np.float32)


def _rng(seed: int, workload: str, layer: int, tensor: int) -> np.random.Generator:
    ss = np.random.SeedSequence([seed, WORKLOAD_IDS.get(workload, 99), layer, tensor])
    return np.random.Generator(np.random.PCG64(ss))


def _sub_seed(seed: int, workload: str, layer: int, tensor: int) -> int:
    ss = np.random.SeedSequence([seed, WORKLOAD_IDS.get(workload, 99), layer, tensor])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _scaled_rows(seed, workload, T, frac):
    n = int(round(frac * T))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(seed, workload, 0, _ROWS).choice(T, size=n, replace=False))


def _expert_ranking(seed, workload, layer):
    return 1 + _rng(seed, workload, layer, _RANK).permutation(N_EXPERTS)


# --------------------------------------------------------------------------- host


def host_layer(T: int, seed: int = 0, workload: str = "custom", layer: int = 0,
               dims=(D_MODEL, D_EXPERT, N_EXPERTS), scaled_rows_frac: float = 0.0,
               skew: bool = False, x_std: float = 1.0, w_std: float = WEIGHT_STD):
    """One layer's inputs drawn on the host with NumPy.

    Returns a dict of bf16 bit arrays (uint16) for x / w_gate / w_up / w_down
    and float32 for w_router.  dims = (D, F, E) allows reduced test shapes.
    """
    D, F, E = dims
    x = _rng(seed, workload, layer, _X).standard_normal((T, D), dtype=np.float32) * np.float32(x_std)
    xb = f32_to_bf16_bits(x)
    if scaled_rows_frac > 0 and T > 0:
        rows = _scaled_rows(seed, workload, T, scaled_rows_frac)
        xb[rows] = f32_to_bf16_bits(bf16_bits_to_f32(xb[rows]) * np.float32(8.0))
    wr = _rng(seed, workload, layer, _WR).standard_normal((E, D), dtype=np.float32) * np.float32(w_std)
    if skew:
        rank = _expert_ranking(seed, workload, layer)
        wr[:, D - 1] = skew_bias(rank)
        xb[:, D - 1] = f32_to_bf16_bits(np.ones(1, np.float32))[0]
    wg = f32_to_bf16_bits(_rng(seed, workload, layer, _WG).standard_normal((E, F, D), dtype=np.float32) * np.float32(w_std))
    wu = f32_to_bf16_bits(_rng(seed, workload, layer, _WU).standard_normal((E, F, D), dtype=np.float32) * np.float32(w_std))
    wd = f32_to_bf16_bits(_rng(seed, workload, layer, _WD).standard_normal((E, D, F), dtype=np.float32) * np.float32(w_std))
    return {"x": xb, "w_router": wr.astype(np.float32), "w_gate": wg, "w_up": wu, "w_down": wd}


def host_workload(name: str, seed: int = 0, tokens: int | None = None):
    """Host inputs for a named workload (optionally with fewer tokens)."""
    w = WORKLOADS[name]
    T = w.tokens if tokens is None else tokens
    layers = [host_layer(T, seed, name, l, scaled_rows_frac=w.scaled_rows_frac, skew=w.skew)
              for l in range(w.layers)]
    if w.layers > 1:
        h0 = _rng(seed, name, 99, _X).standard_normal((T, D_MODEL), dtype=np.float32)
        return {"h0": h0, "layers": layers}
    return layers[0]


# ------------------------------------------------------------------------- device


def _device_normal(shape, seed, workload, layer, tensor_id, std, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_sub_seed(seed, workload, layer, tensor_id))
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, 1.0, generator=g)
    return t.mul_(std)


def device_x(T: int, seed: int = 0, workload: str = "custom", layer: int = 0,
             scaled_rows_frac: float = 0.0, skew: bool = False, device="cuda"):
    """Token rows x bf16 [T,2048] drawn on the device (see the module docstring)."""
    import torch
    x = _device_normal((T, D_MODEL), seed, workload, layer, _X, 1.0, device).to(torch.bfloat16)
    if scaled_rows_frac > 0 and T > 0:
        rows = torch.from_numpy(_scaled_rows(seed, workload, T, scaled_rows_frac)).to(device)
        x[rows] = x[rows] * 8
    if skew:
        x[:, D_MODEL - 1] = 1.0
    return x.contiguous()


def device_weights(seed: int = 0, workload: str = "custom", layer: int = 0, skew: bool = False,
                   device="cuda"):
    """One layer's router (fp32) and expert (bf16) weights drawn on the device."""
    import torch
    out = {}
    wr = _device_normal((N_EXPERTS, D_MODEL), seed, workload, layer, _WR, WEIGHT_STD, device)
    if skew:
        rank = _expert_ranking(seed, workload, layer)
        wr[:, D_MODEL - 1] = torch.from_numpy(skew_bias(rank)).to(device)
    out["w_router"] = wr.contiguous()
    # draw and round expert weights one expert at a time to bound the fp32 scratch
    for key, tid, shape in (("w_gate", _WG, (D_EXPERT, D_MODEL)),
                            ("w_up", _WU, (D_EXPERT, D_MODEL)),
                            ("w_down", _WD, (D_MODEL, D_EXPERT))):
        g = torch.Generator(device=device)
        g.manual_seed(_sub_seed(seed, workload, layer, tid))
        buf = torch.empty((N_EXPERTS,) + shape, dtype=torch.bfloat16, device=device)
        tmp = torch.empty(shape, dtype=torch.float32, device=device)
        for e in range(N_EXPERTS):
            tmp.normal_(0.0, 1.0, generator=g)
            buf[e].copy_(tmp.mul_(WEIGHT_STD))
        out[key] = buf
    return out


def device_layer(T: int, seed: int = 0, workload: str = "custom", layer: int = 0,
                 scaled_rows_frac: float = 0.0, skew: bool = False, device="cuda"):
    """One layer's inputs drawn on the device with torch's generator (fast at full size)."""
    out = device_weights(seed, workload, layer, skew, device)
    out["x"] = device_x(T, seed, workload, layer, scaled_rows_frac, skew, device)
    return out


def device_workload(name: str, seed: int = 0, device="cuda", tokens: int | None = None):
    """Device inputs for a named workload; the stack returns h0 (fp32) and per-layer weights."""
    import torch

    w = WORKLOADS[name]
    T = w.tokens if tokens is None else tokens
    if w.layers == 1:
        return device_layer(T, seed, name, 0, w.scaled_rows_frac, w.skew, device)
    g = torch.Generator(device=device)
    g.manual_seed(_sub_seed(seed, name, 99, _X))
    h0 = torch.empty((T, D_MODEL), dtype=torch.float32, device=device).normal_(generator=g)
    layers = [device_weights(seed, name, l, device=device) for l in range(w.layers)]
    return {"h0": h0, "layers": layers}


def logits_2n01(n_tokens: int, n_experts: int = N_EXPERTS, seed: int = 0) -> np.ndarray:
    """Router scores 2*N(0,1), the distribution of the router comparison in
    "Mixture-of-experts LLMs from scratch with OLMoE", section 2."""
    return 2.0 * _rng(seed, "scores", 0, 0).standard_normal((n_tokens, n_experts))

