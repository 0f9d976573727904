"""GPU parity: the HIP library (through the C ABI) against the float64 oracle.

Small and ragged token counts run the whole oracle; the full-size workloads,
launched exactly as bench.py launches them, are checked in full for routing,
dispatch tables and losses and on sampled tokens for the output (every token's
output depends on its own row only, so the oracle can run on a subset).
"""
import time

import numpy as np
import pytest

import oracle
from sparse_mixture_experts_expert_amd import binding, inputs
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _log(msg):
    print(f"[gpu-parity] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    binding.lib()   # fail loudly if the HIP library is missing
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def weights():
    w = inputs.device_weights(seed=0, workload="parity")
    host = {k: (v.cpu().numpy() if v.dtype == torch.float32 else parity.bf16_tensor_to_bits(v))
            for k, v in w.items()}
    return w, host


def host_of(r):
    out = {}
    for k, v in r.items():
        if v is None or k == "workspace":
            continue
        out[k] = parity.bf16_tensor_to_bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()
    return out


def run_layer(x, w, **variant):
    r = binding.moe_forward(x, w["w_router"], w["w_gate"], w["w_up"], w["w_down"], **variant)
    torch.cuda.synchronize()
    T = x.shape[0]
    tables = binding.dispatch_tables(r["workspace"], T)
    h = host_of(r)
    h.update({k: v.cpu().numpy() for k, v in tables.items()})
    h["x"] = parity.bf16_tensor_to_bits(x)
    h["clip"] = binding.clip_count(r["workspace"])
    return h


def full_check(g, hw, label, renormalize=False, keep=None):
    """Whole-oracle comparison for one call (router variant as given)."""
    var = dict(renormalize=renormalize, keep=keep)
    ref = oracle.moe_layer_ref(g["x"], hw["w_router"], hw["w_gate"], hw["w_up"], hw["w_down"], 8, **var)
    ntie = parity.check_routing(g["route_ids"], g["route_probs"], ref, label, renormalize=renormalize)
    if ntie or not np.array_equal(g["route_ids"], ref["ids"]):
        ref = oracle.moe_layer_ref(g["x"], hw["w_router"], hw["w_gate"], hw["w_up"], hw["w_down"], 8,
                                   forced_ids=g["route_ids"], **var)
    parity.check_dispatch(g["route_ids"], g["expert_counts"], g["perm"], g["inv"], g["offsets"], label=label)
    rel, mx = parity.check_out(oracle.to_f64(g["out"]), ref["out"], label)
    parity.check_losses(float(g["aux_loss"][0]), float(g["z_loss"][0]), ref["aux"], ref["z"], label)
    assert g["clip"] == 0, f"{label}: {g['clip']} intermediates clipped"
    _log(f"{label}: ties={ntie} relL2={rel:.2e} maxabs/rms={mx:.2e} aux={float(g['aux_loss'][0]):.6f}")
    return ref


@pytest.mark.parametrize("T", [1, 7, 16, 31, 64, 100, 255, 257, 385, 600])
def test_layer_matches_oracle(weights, T):
    w, hw = weights
    _log(f"layer T={T}")
    x = inputs.device_x(T, seed=1, workload="parity")
    full_check(run_layer(x, w), hw, f"T={T}")


@pytest.mark.parametrize("T", [449, 641, 832, 833, 1024, 1025, 1536, 1537, 2049, 2560, 2561, 2600])
def test_layer_matches_oracle_large_tile_plans(weights, T):
    """Batches served by the 128-row (385 to 832 tokens), 192-row (to 1024), streaming 256-row (to
    1536), 384-row (to 2560) and MFMA-tuned 256-row tile plans, ragged tails included."""
    w, hw = weights
    _log(f"layer T={T}")
    x = inputs.device_x(T, seed=4, workload="parity")
    full_check(run_layer(x, w), hw, f"T={T}")


@pytest.mark.parametrize("T,renorm,n_keep", [(1, True, 64), (100, True, 64), (300, False, 48),
                                              (257, True, 16), (64, False, 8), (1500, True, 32)])
def test_router_variants(weights, T, renorm, n_keep):
    """Renormalised router and pruned experts ("Mixture-of-experts LLMs from scratch with
    OLMoE", sections 2 and 5) against the oracle's variants."""
    w, hw = weights
    rng = np.random.default_rng(T * 131 + n_keep)
    keep = np.zeros(64, bool)
    keep[rng.choice(64, n_keep, replace=False)] = True
    _log(f"variant T={T} renormalize={renorm} keep={n_keep}")
    x = inputs.device_x(T, seed=6, workload="parity")
    g = run_layer(x, w, renormalize=renorm, keep=None if n_keep == 64 else keep)
    kp = None if n_keep == 64 else keep
    full_check(g, hw, f"variant T={T} renorm={renorm} keep={n_keep}", renormalize=renorm, keep=kp)
    if kp is not None:
        assert (g["expert_counts"][~keep] == 0).all()
    if renorm:
        np.testing.assert_allclose(g["route_probs"].sum(1), 1.0, rtol=2e-6)


def test_scaled_rows_and_large_logits(weights):
    w, hw = weights
    x = inputs.device_x(512, seed=2, workload="prefill-4096", scaled_rows_frac=0.05)
    full_check(run_layer(x, w), hw, "scaled rows T=512")


@pytest.mark.parametrize("T", [300, 1000])
def test_skewed_routing(weights, T):
    w, hw = weights
    ws = inputs.device_weights(seed=3, workload="skew-16384", skew=True)
    ws = {k: (w[k] if k != "w_router" else ws["w_router"]) for k in w}
    hws = dict(hw)
    hws["w_router"] = ws["w_router"].cpu().numpy()
    x = inputs.device_x(T, seed=3, workload="skew-16384", skew=True)
    g = run_layer(x, ws)
    assert g["expert_counts"].max() > 4 * (8 * T / 64)
    full_check(g, hws, f"skew T={T}")


def test_every_token_to_the_same_experts(weights):
    # one expert set gets every token: T rows per expert, 56 experts empty
    w, hw = weights
    T = 700
    x = inputs.device_x(T, seed=4, workload="parity")
    x[:, 2047] = 1.0
    wr = w["w_router"].clone()
    wr[:8, 2047] = 40.0
    g = run_layer(x, dict(w, w_router=wr))
    assert (g["expert_counts"][:8] == T).all() and g["expert_counts"][8:].sum() == 0
    full_check(g, dict(hw, w_router=wr.cpu().numpy()), "all tokens to experts 0..7")


def test_zero_router_ties_go_to_lower_ids(weights):
    w, hw = weights
    T = 50
    x = inputs.device_x(T, seed=5, workload="parity")
    wr = torch.zeros_like(w["w_router"])
    g = run_layer(x, dict(w, w_router=wr))
    assert (g["route_ids"] == np.arange(8)).all()
    np.testing.assert_allclose(g["route_probs"], 1 / 64, rtol=1e-6)
    assert g["aux_loss"][0] == pytest.approx(0.01, rel=1e-5)
    assert g["z_loss"][0] == pytest.approx(0.001 * np.log(64) ** 2, rel=1e-5)
    ref = oracle.moe_layer_ref(g["x"], hw["w_router"] * 0, hw["w_gate"], hw["w_up"], hw["w_down"], 8)
    parity.check_out(oracle.to_f64(g["out"]), ref["out"], "zero router")


@pytest.mark.filterwarnings("ignore:overflow encountered in exp")
def test_activations_beyond_fp16_are_counted(weights):
    """Tokens scaled x256 drive their SwiGLU activations and expert outputs past fp16's range: the
    library stores them clipped and reports how many in the workspace's clip count instead of
    clipping silently; every other token still matches the oracle, and the next call with normal
    inputs on the same workspace reports 0."""
    w, hw = weights
    T = 64
    x = inputs.device_x(T, seed=8, workload="parity")
    big = [5, 17, 40]
    x[big] = (x[big].float() * 256.0).to(torch.bfloat16)   # exact in bf16
    ws = binding.make_workspace(T)
    r = binding.moe_forward(x, w["w_router"], w["w_gate"], w["w_up"], w["w_down"], workspace=ws)
    torch.cuda.synchronize()
    n = binding.clip_count(ws)
    assert n > 0
    g = host_of(r)
    xb = parity.bf16_tensor_to_bits(x)
    rows = np.setdiff1d(np.arange(T), big)
    ref = oracle.moe_layer_ref(xb[rows], hw["w_router"], hw["w_gate"], hw["w_up"], hw["w_down"], 8,
                               forced_ids=g["route_ids"][rows])
    rel, mx = parity.check_out(oracle.to_f64(g["out"][rows]), ref["out"], "unscaled tokens beside clipped ones")
    # the scaled tokens' exact outputs lie far outside fp16
    ref_big = oracle.moe_layer_ref(xb[big], hw["w_router"], hw["w_gate"], hw["w_up"], hw["w_down"], 8,
                                   forced_ids=g["route_ids"][big], keep_y=True)
    assert np.abs(ref_big["y"]).max() > 65504
    x2 = inputs.device_x(T, seed=9, workload="parity")
    binding.moe_forward(x2, w["w_router"], w["w_gate"], w["w_up"], w["w_down"], workspace=ws)
    torch.cuda.synchronize()
    assert binding.clip_count(ws) == 0
    _log(f"clipped intermediates counted: {n}; other tokens relL2={rel:.2e} maxabs/rms={mx:.2e}")


def test_small_down_weights_convert_exactly(weights):
    """W_down scaled by 2^-12 puts most weights below fp16's normal range (2^-14): the down GEMM's
    scaled conversion keeps them exact down to 2^-18, so the layer still matches the oracle."""
    w, hw = weights
    T = 100
    wd = (w["w_down"].float() * 2.0 ** -12).to(torch.bfloat16)   # exact in bf16
    assert (wd.float().abs() < 2.0 ** -14).float().mean().item() > 0.9
    x = inputs.device_x(T, seed=10, workload="parity")
    g = run_layer(x, dict(w, w_down=wd))
    full_check(g, dict(hw, w_down=parity.bf16_tensor_to_bits(wd)), "W_down x 2^-12")


def test_zero_tokens(weights):
    w, _ = weights
    x = torch.empty((0, 2048), dtype=torch.bfloat16, device="cuda")
    counts = torch.full((64,), 7, dtype=torch.int32, device="cuda")
    aux = torch.full((1,), 3.0, device="cuda")
    z = torch.full((1,), 3.0, device="cuda")
    r = binding.moe_forward(x, w["w_router"], w["w_gate"], w["w_up"], w["w_down"], expert_counts=counts,
                            aux_loss=aux, z_loss=z)
    torch.cuda.synchronize()
    assert r["out"].shape == (0, 2048)
    assert counts.sum().item() == 0 and aux.item() == 0.0 and z.item() == 0.0


def test_bitwise_reproducible(weights):
    w, _ = weights
    for T in (40, 3000):
        x = inputs.device_x(T, seed=6, workload="parity")
        a = run_layer(x, w)
        b = run_layer(x, w)
        for k in ("out", "route_ids", "route_probs", "expert_counts", "aux_loss", "z_loss", "perm", "inv"):
            np.testing.assert_array_equal(a[k], b[k], err_msg=f"T={T} {k}")


def test_rmsnorm_and_residual_add():
    T = 300
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    h = torch.randn((T, 2048), generator=g, device="cuda") * 3
    x = binding.rmsnorm_bf16(h, 1e-5)
    y = torch.randn((T, 2048), generator=g, device="cuda").to(torch.bfloat16)
    h_host = h.cpu().numpy()
    ref = oracle.rmsnorm_bf16(h_host.astype(np.float64), 1e-5)
    got = oracle.to_f64(parity.bf16_tensor_to_bits(x))
    # fp32 on the GPU vs fp64 here: the bf16 results may differ by one unit at rounding boundaries
    ulp = np.abs(ref) * 2.0 ** -7
    assert (np.abs(got - ref) <= ulp + 1e-30).all()
    assert (got != ref).mean() < 1e-3
    binding.residual_add(h, y)
    torch.cuda.synchronize()
    expect = h_host + oracle.to_f64(parity.bf16_tensor_to_bits(y)).astype(np.float32)
    np.testing.assert_array_equal(h.cpu().numpy(), expect)


def test_fused_residual_epilogue(weights):
    """olmoe_moe_forward_residual: h += layer output in fp32 and x_next = bf16(RMSNorm(h)),
    x_next aliasing x (the stack's use)."""
    w, hw = weights
    T = 300
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    h = torch.randn((T, 2048), generator=g, device="cuda") * 2
    x = binding.rmsnorm_bf16(h, 1e-5)
    x_bits = parity.bf16_tensor_to_bits(x)
    h_old = h.cpu().numpy().astype(np.float64)
    ids = torch.empty((T, 8), dtype=torch.int32, device="cuda")
    counts = torch.empty(64, dtype=torch.int32, device="cuda")
    binding.moe_forward_residual(x, w["w_router"], w["w_gate"], w["w_up"], w["w_down"], h, x_next=x,
                                 eps=1e-5, route_ids=ids, expert_counts=counts)
    torch.cuda.synchronize()
    ids = ids.cpu().numpy()
    ref = oracle.moe_layer_ref(x_bits, hw["w_router"], hw["w_gate"], hw["w_up"], hw["w_down"], 8,
                               forced_ids=ids)
    np.testing.assert_array_equal(counts.cpu().numpy(), ref["counts"])
    h_new = h.cpu().numpy().astype(np.float64)
    rel, mx = parity.check_out(h_new - h_old, ref["out"], "fused residual update")
    # the next input is RMSNorm of the updated residual, within one bf16 unit of fp64
    want = oracle.rmsnorm_bf16(h_new, 1e-5)
    got = oracle.to_f64(parity.bf16_tensor_to_bits(x))
    assert (np.abs(got - want) <= np.abs(want) * 2.0 ** -7 + 1e-30).all()
    assert (got != want).mean() < 1e-3
    _log(f"fused residual: relL2={rel:.2e} maxabs/rms={mx:.2e}")


@pytest.mark.parametrize("fused", [True, False])
def test_stack_teacher_forced_and_free_running(fused):
    T, L = 64, 3
    layers = [inputs.device_weights(seed=10 + l, workload="stack-16x8192", layer=l) for l in range(L)]
    hw = [{k: (v.cpu().numpy() if v.dtype == torch.float32 else parity.bf16_tensor_to_bits(v))
           for k, v in w.items()} for w in layers]
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    h0 = torch.randn((T, 2048), generator=g, device="cuda")
    h0_host = h0.cpu().numpy()
    r = binding.moe_stack_forward(h0.clone(), layers, keep_inputs=True, keep_states=True, fused=fused)
    torch.cuda.synchronize()
    xs = [parity.bf16_tensor_to_bits(x) for x in r["inputs"]]
    states = [h0_host.astype(np.float64)] + [st.cpu().numpy().astype(np.float64) for st in r["states"]]
    # teacher forcing: each layer checked on the GPU's own input and its own residual update
    for l in range(L):
        ids = r["route_ids"][l].cpu().numpy()
        ref = oracle.moe_layer_ref(xs[l], hw[l]["w_router"], hw[l]["w_gate"], hw[l]["w_up"], hw[l]["w_down"], 8,
                                   forced_ids=ids)
        np.testing.assert_array_equal(r["expert_counts"][l].cpu().numpy(), ref["counts"])
        parity.check_losses(float(r["aux_loss"][l]), float(r["z_loss"][l]), ref["aux"], ref["z"], f"layer {l}")
        parity.check_out(states[l + 1] - states[l], ref["out"], f"layer {l} residual update")
        if l + 1 < L:   # the next input is RMSNorm of this state
            want = oracle.rmsnorm_bf16(states[l + 1], 1e-5)
            got = oracle.to_f64(xs[l + 1])
            assert (np.abs(got - want) <= np.abs(want) * 2.0 ** -7 + 1e-30).all()
    # free running against the oracle's own stack.  A token whose top-8 flips at a near tie
    # (either routing is correct) follows a different path from then on, so the update is
    # checked on the tokens routed identically at every layer; the flipped ones must be few.
    h_ref, per_ref = oracle.moe_stack_ref(h0_host, hw, k=8)
    hg = r["h"].cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(hg - h_ref) / np.linalg.norm(h_ref)
    same = np.ones(T, bool)
    for l in range(L):
        same &= (np.sort(r["route_ids"][l].cpu().numpy(), 1) == np.sort(per_ref[l]["ids"], 1)).all(1)
    du, dr = (hg - h0_host)[same], (h_ref - h0_host)[same]
    upd = np.linalg.norm(du - dr) / np.linalg.norm(dr)
    _log(f"stack free-running rel L2 {rel:.2e}, update rel L2 {upd:.2e} on {same.sum()}/{T} tokens")
    assert rel <= 1e-2 and (~same).sum() <= max(2, T // 10) and upd <= 1e-2


# ------------------------------------------------------------------ full sizes


def oracle_routing(x_bits, wr):
    logits = oracle.router_logits(x_bits, wr)
    lse, p_all = oracle.softmax_all(logits)
    ids, gap = oracle.top_k(logits, 8)
    return dict(logits=logits, lse=lse, p_all=p_all, ids=ids, gap=gap)


def sampled_check(g, hw, ref_rt, n, seed, label, extra_rows=()):
    T = g["route_ids"].shape[0]
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([rng.choice(T, size=min(n, T), replace=False),
                                     np.asarray(extra_rows, dtype=np.int64)])).astype(np.int64)
    ref = oracle.moe_layer_ref(g["x"][rows], hw["w_router"], hw["w_gate"], hw["w_up"], hw["w_down"], 8,
                               forced_ids=g["route_ids"][rows])
    rel, mx = parity.check_out(oracle.to_f64(g["out"][rows]), ref["out"], label)
    return rel, mx


def full_size_layer(name, tokens=None):
    wl = inputs.WORKLOADS[name]
    t0 = time.time()
    d = inputs.device_workload(name, seed=0, tokens=tokens)
    g = run_layer(d["x"], d)
    hw = {k: (d[k].cpu().numpy() if d[k].dtype == torch.float32 else parity.bf16_tensor_to_bits(d[k]))
          for k in ("w_router", "w_gate", "w_up", "w_down")}
    ref = oracle_routing(g["x"], hw["w_router"])
    ntie = parity.check_routing(g["route_ids"], g["route_probs"], ref, name)
    parity.check_dispatch(g["route_ids"], g["expert_counts"], g["perm"], g["inv"], g["offsets"], label=name)
    assert g["clip"] == 0, f"{name}: {g['clip']} intermediates clipped"
    counts = np.bincount(g["route_ids"].ravel(), minlength=64)
    aux, z = oracle.losses(ref["p_all"], counts, ref["lse"], 8)
    parity.check_losses(float(g["aux_loss"][0]), float(g["z_loss"][0]), aux, z, name)
    extra = np.nonzero(ref["gap"] < parity.GAP_TOL)[0][:8]
    if wl.scaled_rows_frac:
        T_run = g["route_ids"].shape[0]
        extra = np.concatenate([extra, inputs._scaled_rows(0, name, T_run, wl.scaled_rows_frac)[:8]])
    rel, mx = sampled_check(g, hw, ref, 40, 1, name, extra)
    _log(f"{name}: ties={ntie} max count={counts.max()} empty={int((counts == 0).sum())} "
         f"sampled relL2={rel:.2e} maxabs/rms={mx:.2e} ({time.time() - t0:.1f}s)")
    return g


@pytest.mark.parametrize("name", ["tiny-32", "decode-256", "prefill-4096", "skew-16384"])
def test_full_size_workload(name):
    _log(f"full size {name}")
    g = full_size_layer(name)
    if name == "skew-16384":
        assert g["expert_counts"].max() > 4 * (8 * 16384 / 64)


def test_largest_batch():
    """65,536 tokens (the row indices, tile lists and workspace at 16x the prefill batch): routing,
    dispatch tables and losses in full, the output on sampled tokens."""
    _log("largest batch 65536")
    g = full_size_layer("prefill-4096", tokens=65536)
    assert g["expert_counts"].sum() == 8 * 65536


def test_full_size_stack():
    """The 16-layer stack at 8192 tokens through the fused path the bench times ("Mixture-of-experts
    LLMs from scratch with OLMoE", section 3: h <- h + MoE(RMSNorm(h)), fp32 residual).  Per layer:
    routing ids and probabilities of every token against the oracle run on the GPU's own input
    x_l, counts and losses; on sampled rows, the fused residual update h_{l+1} - h_l against the
    oracle layer on those rows (the GPU's ids forced), and x_{l+1} = bf16(RMSNorm(h_{l+1}))."""
    name = "stack-16x8192"
    _log("full size stack")
    t0 = time.time()
    d = inputs.device_workload(name, seed=0)
    T = d["h0"].shape[0]
    rng = np.random.default_rng(2)
    rows = np.sort(rng.choice(T, size=24, replace=False))
    rows_t = torch.from_numpy(rows).to("cuda")
    h0_rows = d["h0"][rows_t].cpu().numpy().astype(np.float64)
    r = binding.moe_stack_forward(d["h0"].clone(), d["layers"], keep_inputs=True, keep_states=True,
                                  keep_probs=True, state_rows=rows_t)
    torch.cuda.synchronize()
    states = [h0_rows] + [st.cpu().numpy().astype(np.float64) for st in r["states"]]
    np.testing.assert_array_equal(states[-1], r["h"][rows_t].cpu().numpy().astype(np.float64))
    nl = len(d["layers"])
    for l, w in enumerate(d["layers"]):
        hw = {k: (w[k].cpu().numpy() if w[k].dtype == torch.float32 else parity.bf16_tensor_to_bits(w[k]))
              for k in ("w_router", "w_gate", "w_up", "w_down")}
        xb = parity.bf16_tensor_to_bits(r["inputs"][l])
        ids = r["route_ids"][l].cpu().numpy()
        probs = r["route_probs"][l].cpu().numpy()
        ref = oracle_routing(xb, hw["w_router"])
        ntie = parity.check_routing(ids, probs, ref, f"stack layer {l}")
        counts = np.bincount(ids.ravel(), minlength=64)
        np.testing.assert_array_equal(r["expert_counts"][l].cpu().numpy(), counts)
        aux, z = oracle.losses(ref["p_all"], counts, ref["lse"], 8)
        parity.check_losses(float(r["aux_loss"][l]), float(r["z_loss"][l]), aux, z, f"stack layer {l}")
        # the fused epilogue's fp32 update of the residual on the sampled rows
        ref_o = oracle.moe_layer_ref(xb[rows], hw["w_router"], hw["w_gate"], hw["w_up"], hw["w_down"], 8,
                                     forced_ids=ids[rows])
        rel, mx = parity.check_out(states[l + 1] - states[l], ref_o["out"], f"stack layer {l} residual update")
        if l == 0:   # the first input is RMSNorm of h0
            want = oracle.rmsnorm_bf16(h0_rows, 1e-5)
            assert (np.abs(oracle.to_f64(xb[rows]) - want) <= np.abs(want) * 2.0 ** -7 + 1e-30).all()
        if l + 1 < nl:   # the next input, written by the same epilogue, is RMSNorm of this state
            want = oracle.rmsnorm_bf16(states[l + 1], 1e-5)
            got = oracle.to_f64(parity.bf16_tensor_to_bits(r["inputs"][l + 1])[rows])
            assert (np.abs(got - want) <= np.abs(want) * 2.0 ** -7 + 1e-30).all(), f"layer {l + 1} input"
            assert (got != want).mean() < 1e-2
        _log(f"stack layer {l}: ties={ntie} update relL2={rel:.2e} maxabs/rms={mx:.2e} ({time.time() - t0:.1f}s)")


def test_stage_timing_on_a_sample_of_calls(weights):
    """olmoe_timing_every(n) brackets calls 0, n, 2n, ... of those that follow it."""
    w, _ = weights
    x = inputs.device_x(64, seed=11, workload="parity")
    binding.timing_enable(["gateup", "down"])
    binding.timing_every(3)
    for _ in range(7):
        binding.moe_forward(x, w["w_router"], w["w_gate"], w["w_up"], w["w_down"])
    torch.cuda.synchronize()
    stats, calls = binding.timing_read()
    binding.timing_enable(False)
    assert calls == 3
    assert set(stats) == {"gateup", "down"} and stats["gateup"] > 0 and stats["down"] > 0


def test_concurrent_calls_on_two_streams(weights):
    """Two layer calls in flight at once on two streams (default priority), each with its own
    workspace and outputs, give the same bits as the same calls made one after the other: the
    library keeps no state shared between calls."""
    w, _ = weights
    ws = (w["w_router"], w["w_gate"], w["w_up"], w["w_down"])
    xs = [inputs.device_x(600, seed=21, workload="parity"), inputs.device_x(300, seed=22, workload="parity")]
    refs = [host_of(binding.moe_forward(x, *ws)) for x in xs]
    torch.cuda.synchronize()

    def buffers(T):
        return dict(out=torch.empty((T, 2048), dtype=torch.bfloat16, device="cuda"),
                    route_ids=torch.empty((T, 8), dtype=torch.int32, device="cuda"),
                    route_probs=torch.empty((T, 8), dtype=torch.float32, device="cuda"),
                    expert_counts=torch.empty(64, dtype=torch.int32, device="cuda"),
                    aux_loss=torch.empty(1, dtype=torch.float32, device="cuda"),
                    z_loss=torch.empty(1, dtype=torch.float32, device="cuda"),
                    workspace=binding.make_workspace(T))
    bufs = [buffers(x.shape[0]) for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(3):
        for x, b, s in zip(xs, bufs, streams):
            binding.moe_forward(x, *ws, stream=s, **b)
    torch.cuda.synchronize()
    for i, (b, ref) in enumerate(zip(bufs, refs)):
        got = host_of(b)
        for k in ("out", "route_ids", "route_probs", "expert_counts", "aux_loss", "z_loss"):
            np.testing.assert_array_equal(got[k], ref[k], err_msg=f"call {i}: {k}")


def test_forward_captured_in_a_graph_replays_exactly(weights):
    """Three layer calls (small, streaming and large tile plans) captured in one HIP graph: every
    replay gives the eager calls' bits, with the outputs poisoned and eager work of other sizes on
    the same workspaces between the replays.  Nothing the forward enqueues is a memset: the clip
    count and the other per-call zeroing are done by its kernels."""
    w, _ = weights
    ws = (w["w_router"], w["w_gate"], w["w_up"], w["w_down"])
    sizes = (256, 1024, 4096)
    xs = [inputs.device_x(T, seed=60 + i, workload="parity") for i, T in enumerate(sizes)]
    names = ("out", "route_ids", "route_probs", "expert_counts", "aux_loss", "z_loss")

    def buffers(T):
        return dict(out=torch.empty((T, 2048), dtype=torch.bfloat16, device="cuda"),
                    route_ids=torch.empty((T, 8), dtype=torch.int32, device="cuda"),
                    route_probs=torch.empty((T, 8), dtype=torch.float32, device="cuda"),
                    expert_counts=torch.empty(64, dtype=torch.int32, device="cuda"),
                    aux_loss=torch.empty(1, dtype=torch.float32, device="cuda"),
                    z_loss=torch.empty(1, dtype=torch.float32, device="cuda"),
                    workspace=binding.make_workspace(T))
    bufs = [buffers(x.shape[0]) for x in xs]
    for x, b in zip(xs, bufs):   # eager calls first (also outside any capture)
        binding.moe_forward(x, *ws, **b)
    torch.cuda.synchronize()
    refs = [{k: b[k].clone() for k in names} for b in bufs]
    clip0 = [binding.clip_count(b["workspace"]) for b in bufs]
    assert clip0 == [0, 0, 0]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for x, b in zip(xs, bufs):
            binding.moe_forward(x, *ws, stream=s, **b)
    for rep in range(3):
        for b in bufs:
            b["out"].fill_(float("nan"))
            b["route_probs"].fill_(float("nan"))
            b["route_ids"].fill_(-7)
            b["expert_counts"].fill_(-7)
        # eager work of another size on the same workspaces between the replays
        other = inputs.device_x(100 + rep, seed=70 + rep, workload="parity")
        for b in bufs:
            binding.moe_forward(other, *ws, workspace=b["workspace"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (b, ref) in enumerate(zip(bufs, refs)):
            for k in names:
                assert torch.equal(b[k], ref[k]), (rep, sizes[i], k)
            assert binding.clip_count(b["workspace"]) == 0, (rep, sizes[i])
