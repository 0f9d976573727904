"""Plain CPU oracle of the OLMoE mixture-of-experts feed-forward layer, in float64.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the CPU-baseline
leg of bench.py may import or run this module; the GPU library never does, and
this module imports nothing from it. Inputs arrive as bf16 bit patterns
(uint16) or float32 arrays and are widened to float64 exactly; no intermediate
value is rounded except where a step of the layer says so (the bf16 input of
each layer of the residual stack).

Sources (page title, then section / equation):
  [G]  "OLMoE Guide: 64-Expert Fine-Grained Open MoE Architecture":
       "Router Mechanics & Loss Formulations", items 1 (top-8 softmax routing),
       2 (auxiliary load balancing loss), 3 (router z-loss); and the PyTorch
       module under "Hands-On Implementation".
  [P]  "OLMoE: Open Mixture-of-Experts Language Models": "Pretraining
       architecture" (router = linear layer then softmax, 8 of 64 experts,
       dropless token choice), 4.1.6 and 4.1.7 (loss weights 0.01 and 0.001).
  [X]  "Mixture-of-experts LLMs from scratch with OLMoE": section 2 "The router
       and the experts" (softmax over all experts then top-k, grouped dispatch,
       every-expert brute force, the renormalised router variant), section 3
       "OLMoE in PyTorch" (no renormalisation, float32 residual stream, RMSNorm)
       and section 5 "A smaller model for one kind of text" (pruned experts).

Readings taken where the pages are silent or disagree:
  * routing weights are the 64-way softmax probabilities of the chosen experts,
    NOT renormalised over the 8 ([X] sections 2-3 and [P] over [G]'s formula);
  * the 8 experts are the 8 largest logits; equal logits go to the lower expert
    id, and route_ids lists them by descending logit;
  * the load-balancing term is alpha*E*sum_e f_e*P_e with alpha applied once
    (as [G]'s code does), the z-loss is beta*mean_t(lse_t^2); both are returned
    separately and their sum is [G]'s total auxiliary loss;
  * for T = 0 both losses are 0 and nothing else is produced;
  * router variants (off by default): `renormalize` divides the chosen weights
    by their sum (the Mixtral / Qwen3 router of [X] section 2, equal to [G]'s
    softmax over the top-8 logits); `keep` prunes experts by giving them score
    -inf before the softmax ([X] section 5), so their probability, count and
    share of the load-balancing term are 0 and lse runs over the kept experts;
    at least k experts must be kept;
  * expert choice ([P] 4.1.4 names it, without its rules): the plainest reading
    consistent with the layer is taken. The same router and 64-way softmax;
    capacity C = ceil(k*T/E) tokens per expert (token choice's k*T pairs shared
    equally); each expert takes its C most probable tokens, equal
    probabilities to the lower token id; a token sums p[t,e] * Expert_e over
    the experts that took it (zero to E of them); z-loss as for token choice,
    load-balancing term with f_e = C / (k*T);
  * RMSNorm of the stack uses weight 1 and eps 1e-5 and its output is rounded
    to bf16 (round to nearest even), the type the layer takes.

Pins: every function here is checked in tests/test_oracle_pins.py against closed
forms, brute force, library routines or values the pages print.
"""
from __future__ import annotations

import numpy as np

ALPHA = 0.01   # [P] 4.1.6; [G] item 2
BETA = 0.001   # [P] 4.1.7; [G] item 3
RMS_EPS = 1e-5  # [X] section 3 (library default for the missing config key)


# ----------------------------------------------------------------- type helpers


def to_f64(a) -> np.ndarray:
    """bf16 bit patterns (uint16) or any float array -> float64, exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_to_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), directly
    from float64 (no double rounding through float32). Returns float64."""
    a = np.asarray(a, dtype=np.float64)
    out = np.zeros_like(a)
    nz = (a != 0) & np.isfinite(a)
    _, e = np.frexp(a[nz])                      # a = m * 2**e, 0.5 <= |m| < 1
    quantum = np.ldexp(1.0, np.maximum(e, -125) - 8)   # bf16 spacing in that binade
    out[nz] = np.rint(a[nz] / quantum) * quantum       # rint: ties to even
    out[~np.isfinite(a)] = a[~np.isfinite(a)]
    big = np.abs(out) > 3.3895313892515355e38
    out[big] = np.copysign(np.inf, out[big])
    return out


def bf16_bits(a64) -> np.ndarray:
    """Bit patterns of float64 values that are already exact bf16 values."""
    return (np.asarray(a64, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------- router


def router_logits(x, w_router) -> np.ndarray:
    """h(x) = W_g x for every token: [T,D] x [E,D] -> [T,E] ([G] item 1; [X] section 2)."""
    return to_f64(x) @ to_f64(w_router).T


def softmax_all(logits):
    """Softmax over all experts with its log-normaliser ([X] section 2: softmax first).

    Returns (lse [T], probs [T,E]); lse_t = log sum_e exp(h_te) ([G] item 3)."""
    m = logits.max(axis=-1, keepdims=True)
    s = np.exp(logits - m).sum(axis=-1, keepdims=True)
    lse = m + np.log(s)
    return lse[:, 0], np.exp(logits - lse)


def top_k(logits, k):
    """The k largest logits per token by a full sort on (-logit, expert id).

    Returns ids [T,k] (descending logit, ties -> lower id) and the gap between
    the k-th and (k+1)-th sorted logits (inf when k = E)."""
    T, E = logits.shape
    expert = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((expert, -logits), axis=-1)          # primary key: -logit
    ids = order[:, :k].astype(np.int64)
    srt = np.take_along_axis(logits, order, axis=-1)
    gap = srt[:, k - 1] - srt[:, k] if k < E else np.full(T, np.inf)
    return ids, gap


def mask_logits(logits, keep):
    """Pruning ([X] section 5): experts outside `keep` (bool [E]) get score -inf
    before the softmax, so the router can never choose them."""
    keep = np.asarray(keep, dtype=bool)
    return np.where(keep[None, :], logits, -np.inf)


def renormalize_top_k(probs):
    """The renormalised router ([X] section 2, Mixtral and Qwen3): the k chosen
    softmax weights divided by their sum."""
    return probs / probs.sum(axis=-1, keepdims=True)


# -------------------------------------------------------------------- dispatch


def dispatch(ids, n_experts):
    """Group the (token, slot) pairs by expert, keeping tokens in ascending order.

    counts[e]  = number of tokens that chose e
    offsets    = exclusive prefix sum of counts (length E+1)
    perm[p]    = token of the p-th row of the expert-contiguous order
    inv[t, j]  = row p holding (t, ids[t, j])
    ([X] section 2, grouped dispatch: sort pairs by expert, then count.)"""
    ids = np.asarray(ids)
    T, K = ids.shape
    counts = np.zeros(n_experts, dtype=np.int64)
    perm = np.zeros(T * K, dtype=np.int64)
    inv = np.zeros((T, K), dtype=np.int64)
    pos = 0
    for e in range(n_experts):
        toks, slots = np.nonzero(ids == e)      # row-major: tokens ascending
        n = toks.size
        counts[e] = n
        perm[pos:pos + n] = toks
        inv[toks, slots] = pos + np.arange(n)
        pos += n
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return counts, offsets, perm, inv


# ---------------------------------------------------------------------- experts


def silu(g):
    """SiLU / Swish with beta = 1: g * sigmoid(g) ([G] item 1; [X] section 2 uses F.silu)."""
    return g / (1.0 + np.exp(-g))


def swiglu_expert(X, w_gate_e, w_up_e, w_down_e) -> np.ndarray:
    """(SiLU(X W_gate^T) * (X W_up^T)) W_down^T; weights stored [out, in]
    ([G] item 1 and its SwiGLUExpert; [X] section 2, Experts.run)."""
    wg, wu, wd = to_f64(w_gate_e), to_f64(w_up_e), to_f64(w_down_e)
    X = to_f64(X)
    return (silu(X @ wg.T) * (X @ wu.T)) @ wd.T


def losses(probs, counts, lse, k, alpha=ALPHA, beta=BETA):
    """Switch load-balancing loss and router z-loss ([G] items 2-3).

    f_e = counts_e / (T k), P_e = mean_t p_te, aux = alpha * E * sum_e f_e P_e,
    z = beta * mean_t lse_t^2."""
    T, E = probs.shape
    if T == 0:
        return 0.0, 0.0
    f = counts / float(T * k)
    P = probs.mean(axis=0)
    return float(alpha * E * np.sum(f * P)), float(beta * np.mean(lse ** 2))


def moe_layer_ref(x, w_router, w_gate, w_up, w_down, k=8, forced_ids=None,
                  keep_y=False, renormalize=False, keep=None):
    """One MoE layer, grouped by expert ([X] section 2 dispatch; [P] "Pretraining
    architecture"; [G] item 1 for the weighted sum).

    x [T,D] bf16 bits or float; w_router [E,D]; w_gate, w_up [E,F,D];
    w_down [E,D,F]. forced_ids [T,k] replaces the router's choice (used where
    two routings are both correct within rounding). renormalize / keep select
    the router variants described in the module docstring.
    Returns a dict: out [T,D], ids, probs (route_probs [T,k]), p_all [T,E],
    logits, lse, gap, counts, offsets, perm, inv, aux, z (and y [Tk,D] if keep_y)."""
    x64 = to_f64(x)
    T, D = x64.shape
    E = np.asarray(w_router).shape[0]
    logits = router_logits(x64, w_router) if T else np.zeros((0, E))
    if keep is not None:
        if int(np.sum(np.asarray(keep, dtype=bool))) < k:
            raise ValueError("fewer than k experts kept")
        logits = mask_logits(logits, keep)
    if T:
        lse, p_all = softmax_all(logits)
    else:
        lse, p_all = np.zeros(0), np.zeros((0, E))
    if forced_ids is None:
        ids, gap = top_k(logits, k) if T else (np.zeros((0, k), np.int64), np.zeros(0))
    else:
        ids = np.asarray(forced_ids, dtype=np.int64).reshape(T, k)
        gap = np.full(T, np.nan)
    probs = np.take_along_axis(p_all, ids, axis=-1)          # not renormalised by default
    if renormalize and T:
        probs = renormalize_top_k(probs)
    counts, offsets, perm, inv = dispatch(ids, E)
    y = np.zeros((T * k, D))
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            y[a:b] = swiglu_expert(x64[perm[a:b]], w_gate[e], w_up[e], w_down[e])
    out = np.zeros((T, D))
    for j in range(k):                                         # weighted sum over the k slots
        out += probs[:, j:j + 1] * y[inv[:, j]]
    aux, z = losses(p_all, counts, lse, k)
    r = dict(out=out, ids=ids, probs=probs, p_all=p_all, logits=logits, lse=lse, gap=gap,
             counts=counts, offsets=offsets, perm=perm, inv=inv, aux=aux, z=z)
    if keep_y:
        r["y"] = y
    return r


# --------------------------------------------------------------- expert choice


def expert_capacity(T, k=8, E=64):
    """Tokens per expert under expert choice: the pair budget of token choice, k*T, shared
    equally by the E experts and rounded up, ceil(k*T/E)."""
    return -(-k * T // E)


def expert_choice_select(p, C):
    """Each expert takes the C tokens with the largest probability p[:, e]; equal
    probabilities go to the lower token id. Returns chosen [E,C] (ascending token ids) and the
    gap between the C-th and (C+1)-th sorted probability of each expert (inf when C >= T)."""
    T, E = p.shape
    chosen = np.zeros((E, C), dtype=np.int64)
    gap = np.full(E, np.inf)
    tok = np.arange(T)
    for e in range(E):
        order = np.lexsort((tok, -p[:, e]))                 # primary key: -p
        chosen[e] = np.sort(order[:C])
        if C < T:
            gap[e] = p[order[C - 1], e] - p[order[C], e] if C > 0 else np.inf
    return chosen, gap


def expert_choice_layer_ref(x, w_router, w_gate, w_up, w_down, k=8, forced_chosen=None):
    """The layer with expert-choice routing ([P] 4.1.4 names it as the alternative to token
    choice; the steps here are the plainest reading, as in the module docstring of the GPU
    path): the same router and 64-way softmax ([G] item 1), then every expert takes its
    C = ceil(k*T/E) most probable tokens, and each token sums p[t,e] * Expert_e(x_t) over the
    experts that took it. Losses: z as for token choice; the load-balancing term with f_e the
    expert's share of the k*T pairs. forced_chosen [E,C] replaces the selection (near ties).

    Returns dict(out, chosen [E,C], weights [E,C], token_counts [T], p_all, lse, gap, aux, z)."""
    x64 = to_f64(x)
    T, D = x64.shape
    E = np.asarray(w_router).shape[0]
    C = expert_capacity(T, k, E)
    logits = router_logits(x64, w_router) if T else np.zeros((0, E))
    lse, p = softmax_all(logits) if T else (np.zeros(0), np.zeros((0, E)))
    if forced_chosen is None:
        chosen, gap = expert_choice_select(p, C) if T else (np.zeros((E, 0), np.int64), np.full(E, np.inf))
    else:
        chosen = np.asarray(forced_chosen, dtype=np.int64).reshape(E, C)
        gap = np.full(E, np.nan)
    weights = np.take_along_axis(p.T, chosen, axis=1) if T else np.zeros((E, 0))
    out = np.zeros((T, D))
    for e in range(E):
        if C:
            y = swiglu_expert(x64[chosen[e]], w_gate[e], w_up[e], w_down[e])
            np.add.at(out, chosen[e], weights[e][:, None] * y)
    token_counts = np.bincount(chosen.ravel(), minlength=T) if T else np.zeros(0, np.int64)
    counts = np.full(E, C)
    aux, z = losses(p, counts, lse, k) if T else (0.0, 0.0)
    return dict(out=out, chosen=chosen, weights=weights, token_counts=token_counts, p_all=p, lse=lse,
                gap=gap, aux=aux, z=z, capacity=C)


# -------------------------------------------------------------------- backward


def silu_grad(g):
    """d/dg [g * sigma(g)] = sigma(g) * (1 + g * (1 - sigma(g)))."""
    sig = 1.0 / (1.0 + np.exp(-g))
    return sig * (1.0 + g * (1.0 - sig))


def moe_layer_backward_ref(x, w_router, w_gate, w_up, w_down, dout, g_aux=0.0, g_z=0.0, k=8,
                           forced_ids=None, magnitudes=False):
    """Gradients of  L = sum_t <dout_t, out_t> + g_aux * aux + g_z * z  for one layer with the
    default router (64-way softmax, top-k, not renormalised), by the chain rule through the
    forward steps of moe_layer_ref ([G] items 1-3; [X] section 2). The routing choice and the
    counts f_e are piecewise constant and carry no gradient.

    forced_ids fixes the routing as in moe_layer_ref (for near ties). magnitudes=True also
    returns mag_gate / mag_up / mag_down / mag_dx: the same contractions over |operands|
    (sums of |a| |b| over the terms of each element), which scale the rounding error any
    evaluation of those gradients in a finite precision can make.
    Returns dict(dx [T,D], dw_router [E,D], dw_gate [E,F,D], dw_up [E,F,D], dw_down [E,D,F],
    dw [T,k] (gradient of the routing weights), dlogits [T,E], fwd (the forward dict))."""
    fwd = moe_layer_ref(x, w_router, w_gate, w_up, w_down, k, keep_y=True, forced_ids=forced_ids)
    x64 = to_f64(x)
    g = to_f64(dout)
    T, D = x64.shape
    wr = to_f64(w_router)
    E = wr.shape[0]
    F = np.asarray(w_gate).shape[1]
    dx = np.zeros((T, D))
    dw_gate = np.zeros((E, F, D))
    dw_up = np.zeros((E, F, D))
    dw_down = np.zeros((E, D, F))
    dw = np.zeros((T, k))
    mags = dict(mag_gate=np.zeros((E, F, D)), mag_up=np.zeros((E, F, D)), mag_down=np.zeros((E, D, F)),
                mag_dx=np.zeros((T, D))) if magnitudes else None
    perm, inv, offsets, probs = fwd["perm"], fwd["inv"], fwd["offsets"], fwd["probs"]
    slot = np.zeros(T * k, dtype=np.int64)          # row -> slot j of its (token, slot) pair
    for j in range(k):
        slot[inv[:, j]] = j
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b == a:
            continue
        t = perm[a:b]
        j = slot[a:b]
        X = x64[t]
        wg, wu, wd = to_f64(w_gate[e]), to_f64(w_up[e]), to_f64(w_down[e])
        G = X @ wg.T
        U = X @ wu.T
        S = silu(G)
        H = S * U
        go = g[t]                                  # upstream gradient of each row's token
        dw[t, j] = np.sum(go * fwd["y"][a:b], axis=1)   # out = sum_j w_j Y_j
        dY = probs[t, j][:, None] * go
        dw_down[e] = dY.T @ H                      # Y = H W_down^T
        dH = dY @ wd
        dG = dH * U * silu_grad(G)                 # H = silu(G) * U
        dU = dH * S
        dw_gate[e] = dG.T @ X                      # G = X W_gate^T, U = X W_up^T
        dw_up[e] = dU.T @ X
        np.add.at(dx, t, dG @ wg + dU @ wu)
        if magnitudes:
            mags["mag_gate"][e] = np.abs(dG).T @ np.abs(X)
            mags["mag_up"][e] = np.abs(dU).T @ np.abs(X)
            mags["mag_down"][e] = np.abs(dY).T @ np.abs(H)
            np.add.at(mags["mag_dx"], t, np.abs(dG) @ np.abs(wg) + np.abs(dU) @ np.abs(wu))
    # router: probabilities of the chosen experts, the load-balancing term and the z-loss
    p = fwd["p_all"]
    dp = np.zeros((T, E))
    np.put_along_axis(dp, fwd["ids"], dw, axis=1)
    if T:
        f = fwd["counts"] / (k * T)
        dp += g_aux * ALPHA * E * f[None, :] / T     # aux = alpha E sum_e f_e mean_t p_te
    dlogits = p * (dp - np.sum(p * dp, axis=1, keepdims=True))     # softmax Jacobian
    if T:
        dlogits += g_z * BETA * (2.0 * fwd["lse"] / T)[:, None] * p   # z = beta mean_t lse_t^2
    dx += dlogits @ wr
    r = dict(dx=dx, dw_router=dlogits.T @ x64, dw_gate=dw_gate, dw_up=dw_up, dw_down=dw_down,
             dw=dw, dlogits=dlogits, fwd=fwd)
    if magnitudes:
        mags["mag_dx"] += np.abs(dlogits) @ np.abs(wr)
        r.update(mags)
    return r


def expert_choice_backward_ref(x, w_router, w_gate, w_up, w_down, dout, g_aux=0.0, g_z=0.0, k=8,
                               forced_chosen=None, magnitudes=False):
    """Gradients of  L = sum_t <dout_t, out_t> + g_aux * aux + g_z * z  for the expert-choice layer
    of expert_choice_layer_ref, by the chain rule through its steps (the same router, softmax,
    SwiGLU experts and losses as the token-choice backward: [G] items 1-3). Which tokens each
    expert takes, and the shares f_e = C/(kT), are piecewise constant and carry no gradient.

    forced_chosen fixes the selection (near ties); magnitudes=True also returns the contractions
    over |operands| as moe_layer_backward_ref does. Returns dict(dx, dw_router, dw_gate, dw_up,
    dw_down, dp [T,E] (gradient of the routing weight of every taken pair, 0 elsewhere, before the
    loss terms), dlogits, fwd)."""
    fwd = expert_choice_layer_ref(x, w_router, w_gate, w_up, w_down, k, forced_chosen=forced_chosen)
    x64 = to_f64(x)
    g = to_f64(dout)
    T, D = x64.shape
    wr = to_f64(w_router)
    E = wr.shape[0]
    F = np.asarray(w_gate).shape[1]
    C = fwd["capacity"]
    p = fwd["p_all"]
    dx = np.zeros((T, D))
    dw_gate = np.zeros((E, F, D))
    dw_up = np.zeros((E, F, D))
    dw_down = np.zeros((E, D, F))
    dw = np.zeros((T, E))
    mags = dict(mag_gate=np.zeros((E, F, D)), mag_up=np.zeros((E, F, D)), mag_down=np.zeros((E, D, F)),
                mag_dx=np.zeros((T, D))) if magnitudes else None
    for e in range(E):
        if C == 0:
            break
        t = fwd["chosen"][e]                       # distinct tokens
        X = x64[t]
        wg, wu, wd = to_f64(w_gate[e]), to_f64(w_up[e]), to_f64(w_down[e])
        G = X @ wg.T
        U = X @ wu.T
        S = silu(G)
        H = S * U
        go = g[t]
        dw[t, e] = np.sum(go * (H @ wd.T), axis=1)      # out_t = sum_e p[t,e] Y_e(x_t)
        dY = p[t, e][:, None] * go
        dw_down[e] = dY.T @ H
        dH = dY @ wd
        dG = dH * U * silu_grad(G)
        dU = dH * S
        dw_gate[e] = dG.T @ X
        dw_up[e] = dU.T @ X
        dx[t] += dG @ wg + dU @ wu
        if magnitudes:
            mags["mag_gate"][e] = np.abs(dG).T @ np.abs(X)
            mags["mag_up"][e] = np.abs(dU).T @ np.abs(X)
            mags["mag_down"][e] = np.abs(dY).T @ np.abs(H)
            mags["mag_dx"][t] += np.abs(dG) @ np.abs(wg) + np.abs(dU) @ np.abs(wu)
    dp = dw.copy()
    if T:
        dp += g_aux * ALPHA * E * (C / (k * T)) / T      # aux = alpha E sum_e f_e mean_t p_te
    dlogits = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    if T:
        dlogits += g_z * BETA * (2.0 * fwd["lse"] / T)[:, None] * p
    dx += dlogits @ wr
    r = dict(dx=dx, dw_router=dlogits.T @ x64, dw_gate=dw_gate, dw_up=dw_up, dw_down=dw_down, dp=dw,
             dlogits=dlogits, fwd=fwd)
    if magnitudes:
        mags["mag_dx"] += np.abs(dlogits) @ np.abs(wr)
        r.update(mags)
    return r


# ----------------------------------------------------------------- brute force


def moe_layer_dense_ref(x, w_router, w_gate, w_up, w_down, k=8):
    """The same layer the wasteful way: every expert on every token, outputs of
    unchosen experts multiplied by zero ([X] section 2, dense_run). Selection by
    pairwise comparison: expert e is chosen iff fewer than k experts beat it,
    where e' beats e if h_e' > h_e, or h_e' = h_e and e' < e. Tiny inputs only."""
    x64 = to_f64(x)
    T, D = x64.shape
    wr = to_f64(w_router)
    E = wr.shape[0]
    logits = np.zeros((T, E))
    for t in range(T):
        for e in range(E):
            logits[t, e] = sum(x64[t, d] * wr[e, d] for d in range(D)) if D <= 64 else x64[t] @ wr[e]
    rank = np.zeros((T, E), dtype=np.int64)
    for t in range(T):
        for e in range(E):
            rank[t, e] = sum(1 for e2 in range(E)
                             if logits[t, e2] > logits[t, e] or (logits[t, e2] == logits[t, e] and e2 < e))
    chosen = rank < k
    ids = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        for e in range(E):
            if chosen[t, e]:
                ids[t, rank[t, e]] = e
    z_t = np.array([np.log(np.sum(np.exp(logits[t]))) for t in range(T)])
    p = np.exp(logits - z_t[:, None])
    gate = np.where(chosen, p, 0.0)
    out = np.zeros((T, D))
    for e in range(E):
        ye = swiglu_expert(x64, w_gate[e], w_up[e], w_down[e])
        out += gate[:, e:e + 1] * ye
    counts = chosen.sum(axis=0)
    f = counts / (T * k)
    P = p.sum(axis=0) / T
    aux = ALPHA * E * sum(f[e] * P[e] for e in range(E))
    z = BETA * sum(v * v for v in z_t) / T
    return dict(out=out, ids=ids, counts=counts, aux=float(aux), z=float(z), probs_all=p)


# ------------------------------------------------------------------------ stack


def rmsnorm_bf16(h, eps=RMS_EPS) -> np.ndarray:
    """RMSNorm with weight 1, computed in float64, then rounded to bf16 (the
    layer's input type) ([X] section 3, RMSNorm). Returns float64 bf16 values."""
    h = np.asarray(h, dtype=np.float64)
    u = h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return round_to_bf16(u)


def moe_stack_ref(h0, layers, k=8, teacher_inputs=None, eps=RMS_EPS):
    """Residual stack h <- h + MoE_l(RMSNorm(h)), l = 0..L-1, h kept in float64
    ([X] section 3, Block.forward with the attention sublayer left out).

    layers: list of dicts with w_router / w_gate / w_up / w_down.
    teacher_inputs: optional per-layer bf16 inputs to use instead of RMSNorm(h)
    (runs each layer on given inputs, so every layer can be checked alone).
    Returns (h_final, per-layer list of dicts: x_in (bf16 bits), out, ids,
    counts, aux, z, gap)."""
    h = np.asarray(h0, dtype=np.float64).copy()
    per_layer = []
    for l, w in enumerate(layers):
        if teacher_inputs is not None:
            xin = to_f64(teacher_inputs[l])
        else:
            xin = rmsnorm_bf16(h, eps)
        r = moe_layer_ref(xin, w["w_router"], w["w_gate"], w["w_up"], w["w_down"], k)
        h = h + r["out"]
        per_layer.append(dict(x_in=bf16_bits(xin), out=r["out"], ids=r["ids"], counts=r["counts"],
                              aux=r["aux"], z=r["z"], gap=r["gap"]))
    return h, per_layer
