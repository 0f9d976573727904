"""Comparison of one GPU layer call with the float64 oracle, to the bar the
layer is held to:
  * route_ids, expert counts, perm / inv / offsets bit-exact, except tokens
    whose 8th/9th logit gap (oracle, fp64) is below 1e-5: there either
    routing is correct, so the GPU's choice is checked for validity and the
    oracle is re-run with the GPU's ids for everything downstream;
  * route_probs relative error <= 1e-5 + 4 ulp_fp32(largest |logit| of the token)
    (the probabilities come from fp32 logits);
  * out: relative L2 error <= 1e-2 and max abs error <= 2e-2 * RMS(out_oracle)
    beyond half a bf16 unit of the exact value (the bf16 output's own rounding);
  * aux / z losses relative error <= 1e-4.
"""
from __future__ import annotations

import numpy as np

import oracle

GAP_TOL = 1e-5
PROB_RTOL = 1e-5
OUT_REL_L2 = 1e-2
OUT_MAX_ABS_RMS = 2e-2
LOSS_RTOL = 1e-4


def bf16_tensor_to_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ulp_f32(a):
    """Spacing of float32 values at magnitude a (a >= 0)."""
    _, e = np.frexp(np.maximum(a, 2.0 ** -126))
    return np.ldexp(1.0, e - 24)


def check_routing(ids_gpu, probs_gpu, ref, label="", renormalize=False):
    """ids / probs against the oracle's full-router result `ref` (no forcing).
    Pruned experts carry logit -inf in `ref`.  With renormalize the GPU's weights
    are compared with its experts' probabilities divided by their sum.
    Returns the number of near-tie tokens."""
    ids_gpu = np.asarray(ids_gpu, dtype=np.int64)
    T, k = ids_gpu.shape
    logits = ref["logits"]
    gap = ref["gap"]
    tie = gap < GAP_TOL
    # every token: 8 distinct experts in range
    assert ((ids_gpu >= 0) & (ids_gpu < logits.shape[1])).all(), label
    assert (np.sort(ids_gpu, 1)[:, 1:] != np.sort(ids_gpu, 1)[:, :-1]).all(), label
    # exact sets (and order where the top-9 logits are separated) away from near ties
    clear = ~tie
    set_gpu = np.sort(ids_gpu[clear], 1)
    set_ref = np.sort(ref["ids"][clear], 1)
    bad = np.nonzero((set_gpu != set_ref).any(1))[0]
    assert bad.size == 0, f"{label}: {bad.size} tokens route differently, first {np.nonzero(clear)[0][bad[:5]]}"
    srt = -np.sort(-logits, 1)
    sep = (srt[:, :k] - srt[:, 1:k + 1]).min(1) >= GAP_TOL
    np.testing.assert_array_equal(ids_gpu[sep], ref["ids"][sep], err_msg=f"{label}: slot order")
    # near ties: the GPU's set must be a valid top-k within the tolerance
    for t in np.nonzero(tie)[0]:
        chosen = logits[t, ids_gpu[t]]
        others = np.delete(logits[t], ids_gpu[t])
        assert chosen.min() >= others.max() - GAP_TOL, f"{label}: token {t} invalid near-tie routing"
    # probabilities of the GPU's experts
    p_ref = np.take_along_axis(ref["p_all"], ids_gpu, 1)
    if renormalize:
        p_ref = p_ref / p_ref.sum(1, keepdims=True)
    rel = np.abs(np.asarray(probs_gpu, np.float64) - p_ref) / p_ref
    # fp32 logits of magnitude L carry ~ulp(L) of error, which enters p relatively
    finite = np.where(np.isfinite(logits), np.abs(logits), 0.0)
    tol = PROB_RTOL + 4 * ulp_f32(finite.max(1, keepdims=True))
    worst = (rel / tol).max() if rel.size else 0.0
    assert worst <= 1.0, f"{label}: route_probs rel err {rel.max():.3e} (bar {tol.min():.2e}..{tol.max():.2e})"
    return int(tie.sum())


def check_dispatch(ids_gpu, counts_gpu, perm_gpu, inv_gpu, offsets_gpu, E=64, label=""):
    counts, offsets, perm, inv = oracle.dispatch(np.asarray(ids_gpu, np.int64), E)
    np.testing.assert_array_equal(np.asarray(counts_gpu), counts, err_msg=f"{label}: counts")
    np.testing.assert_array_equal(np.asarray(offsets_gpu), offsets, err_msg=f"{label}: offsets")
    np.testing.assert_array_equal(np.asarray(perm_gpu), perm, err_msg=f"{label}: perm")
    np.testing.assert_array_equal(np.asarray(inv_gpu).reshape(inv.shape), inv, err_msg=f"{label}: inv")


def half_ulp_bf16(r):
    """Half the spacing of bf16 values around |r|: the rounding error of the
    best possible bf16 output (ties included)."""
    a = np.abs(np.asarray(r, np.float64))
    _, e = np.frexp(a)
    return np.where(a > 0, np.ldexp(0.5, np.maximum(e, -125) - 8), 0.0)


def out_errors(out_gpu, out_ref):
    o = np.asarray(out_gpu, np.float64)
    r = np.asarray(out_ref, np.float64)
    rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
    rel_l2 = np.linalg.norm(o - r) / max(np.linalg.norm(r), 1e-300)
    err = np.abs(o - r)
    max_abs = err.max() if r.size else 0.0
    # error beyond the output's own unavoidable bf16 rounding
    beyond = np.maximum(err - half_ulp_bf16(r), 0.0).max() if r.size else 0.0
    return rel_l2, max_abs, beyond, rms


def check_out(out_gpu, out_ref, label=""):
    """rel L2 <= 1e-2 and max abs <= 2e-2 * RMS(out), the max-abs bar applied to
    the error beyond half a bf16 unit of the exact value (the output is bf16:
    for |out| >= 0.25 its rounding alone can reach 2e-2 * RMS)."""
    rel_l2, max_abs, beyond, rms = out_errors(out_gpu, out_ref)
    assert rel_l2 <= OUT_REL_L2, f"{label}: rel L2 {rel_l2:.3e}"
    assert beyond <= OUT_MAX_ABS_RMS * rms, \
        f"{label}: max abs beyond bf16 rounding {beyond:.3e} > {OUT_MAX_ABS_RMS} * rms {rms:.3e} (raw {max_abs:.3e})"
    return rel_l2, max_abs / max(rms, 1e-300)


def check_losses(aux_gpu, z_gpu, aux_ref, z_ref, label=""):
    assert abs(aux_gpu - aux_ref) <= LOSS_RTOL * abs(aux_ref) + 1e-12, f"{label}: aux {aux_gpu} vs {aux_ref}"
    assert abs(z_gpu - z_ref) <= LOSS_RTOL * abs(z_ref) + 1e-12, f"{label}: z {z_gpu} vs {z_ref}"


def ec_tie_tol(p_c, logits):
    """Near-tie width for an expert's C-th probability p_c: twice the bar on one
    probability's relative error (fp32 logits of magnitude L enter p relatively)."""
    finite = np.where(np.isfinite(logits), np.abs(logits), 0.0)
    return 2.0 * (PROB_RTOL + 4 * ulp_f32(finite.max())) * p_c


def check_expert_choice(tokens_gpu, probs_gpu, counts_gpu, p_all, logits, label=""):
    """Expert-choice selection against the oracle's probabilities p_all [T,64]
    (fp64).  Every expert's row must hold C distinct ascending token ids;
    where the oracle's C-th and (C+1)-th probabilities of the expert are further
    apart than the tie width the set must equal the oracle's exactly, otherwise
    it must be a valid top-C within that width.  choice_probs within the
    probability bar, token_counts exactly the GPU selection's multiplicities.
    Returns the number of near-tie experts."""
    tok = np.asarray(tokens_gpu, np.int64)
    E_, C = tok.shape
    T = p_all.shape[0]
    assert C == oracle.expert_capacity(T, 8, E_), label
    if C == 0:
        return 0
    assert ((tok >= 0) & (tok < T)).all(), label
    assert (np.diff(tok, axis=1) > 0).all(), f"{label}: tokens not strictly ascending per expert"
    ref_chosen, gap = oracle.expert_choice_select(p_all, C)
    n_tie = 0
    for e in range(E_):
        col = p_all[:, e]
        p_c = np.sort(col)[::-1][C - 1]
        tol = ec_tie_tol(p_c, logits)
        if gap[e] >= tol:
            np.testing.assert_array_equal(tok[e], ref_chosen[e], err_msg=f"{label}: expert {e} chosen set")
        else:
            n_tie += 1
            mask = np.zeros(T, bool)
            mask[tok[e]] = True
            if (~mask).any():
                assert col[mask].min() >= col[~mask].max() - tol, f"{label}: expert {e} invalid near-tie choice"
    p_ref = np.take_along_axis(p_all.T, tok, axis=1)
    rel = np.abs(np.asarray(probs_gpu, np.float64) - p_ref) / p_ref
    finite = np.where(np.isfinite(logits), np.abs(logits), 0.0)
    bar = PROB_RTOL + 4 * ulp_f32(finite.max(1))[tok]
    assert (rel <= bar).all(), f"{label}: choice_probs rel err {rel.max():.3e}"
    np.testing.assert_array_equal(np.asarray(counts_gpu), np.bincount(tok.ravel(), minlength=T),
                                  err_msg=f"{label}: token_counts")
    return n_tie
