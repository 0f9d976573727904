"""Host-side logic of bench.py, on the CPU: the one-GPU guard, the algorithmic work model behind
roofline.achieved, the kernel-name -> stage map used by the profile summaries, and the rule that
counter-derived traffic is reported only for the kernel sources it was measured on."""
import json
import os
import shutil
import subprocess
import sys

import pytest

import bench
from sparse_mixture_experts_expert_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, env=env)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "single" in r.stderr and "--gpus 1" in r.stderr


def test_a_multi_rank_launch_exits_with_a_message():
    r = _run_bench([], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "single" in r.stderr


def test_work_model_matches_the_layer_shapes():
    # one expert's three matrices and the router, as the input generator builds them (reduced T)
    h = inputs.host_layer(4, seed=0, workload="custom")
    n_router = h["w_router"].size
    n_expert = (h["w_gate"][0].size + h["w_up"][0].size + h["w_down"][0].size)
    assert bench.FLOP_PER_TOKEN == 2 * (n_router + bench.K * n_expert)
    assert bench.EXPERT_BYTES == h["w_gate"][0].nbytes + h["w_up"][0].nbytes + h["w_down"][0].nbytes
    assert bench.GATEUP_EXPERT_BYTES == h["w_gate"][0].nbytes + h["w_up"][0].nbytes
    assert bench.DOWN_EXPERT_BYTES == h["w_down"][0].nbytes


@pytest.mark.parametrize("T", [1, 32, 256, 4096, 16384])
def test_stage_flops_add_up_to_the_layer(T):
    # the three contractions of the layer carry all of its FLOP; the combine's weighted sum is extra
    total = sum(bench.stage_model(s, T, 64)[0] for s in ("router", "gateup", "down"))
    assert total == T * bench.FLOP_PER_TOKEN
    assert bench.stage_model("combine", T, 64)[0] == 2 * bench.K * T * bench.D


def test_stage_bytes_count_each_touched_expert_once():
    for touched in (1, 17, 64):
        gu = bench.stage_model("gateup", 256, touched)[1]
        dn = bench.stage_model("down", 256, touched)[1]
        assert gu - bench.stage_model("gateup", 256, 0)[1] == touched * bench.GATEUP_EXPERT_BYTES
        assert dn - bench.stage_model("down", 256, 0)[1] == touched * bench.DOWN_EXPERT_BYTES
    # small batches are weight-bound, large ones matrix-bound, against the published ridge
    f, b = bench.stage_model("gateup", 256, 64)
    assert f / b < bench.RIDGE
    f, b = bench.stage_model("gateup", 4096, 64)
    assert f / b > bench.RIDGE


@pytest.mark.parametrize("name,stage", [
    ("void olmoe::(anonymous namespace)::grouped_gemm_kernel<olmoe::(anonymous namespace)::Cfg<64, 128, 2, 4, "
     "true, 2, 64, 1, true, false> >(unsigned short const*)", "gateup"),
    ("void olmoe::(anonymous namespace)::grouped_gemm_kernel<olmoe::(anonymous namespace)::Cfg<256, 256, 2, 4, "
     "false, 2, 64, 0, false, false> >(unsigned short const*)", "down"),
    ("void olmoe::(anonymous namespace)::router_partial_f32_kernel<16>(unsigned short const*)", "router"),
    ("olmoe::(anonymous namespace)::router_prep_kernel(float const*, unsigned short*)", "router"),
    ("olmoe::(anonymous namespace)::scan_permute_kernel(olmoe::ScanArgs, olmoe::PermuteArgs)", "dispatch"),
    ("olmoe::(anonymous namespace)::permute_kernel(olmoe::PermuteArgs)", "dispatch"),
    ("void olmoe::(anonymous namespace)::combine_kernel<false>(olmoe::CombineArgs)", "combine"),
    ("void olmoe::(anonymous namespace)::dgrad_kernel<olmoe::(anonymous namespace)::DCfg<64, 256, 2, 4, 3, 0> >"
     "(olmoe::BwdDgradArgs)", "backward"),
    ("olmoe::(anonymous namespace)::bwd_wrouter_partial_kernel(olmoe::BwdSmallArgs)", "backward"),
    ("void olmoe::(anonymous namespace)::ec_choose_kernel<256, 1>(olmoe::EcArgs)", "expert_choice"),
    ("void at::native::vectorized_elementwise_kernel<4>(int)", None),
])
def test_kernel_names_map_to_stages(name, stage):
    assert bench._stage_of(name) == stage


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(tmp_path, monkeypatch):
    csrc = tmp_path / "sparse_mixture_experts_expert_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("grouped_gemm.hip", "router.hip", "common.hpp", "kernels.hpp"):
        shutil.copy(os.path.join(ROOT, "sparse_mixture_experts_expert_amd", "csrc", f), csrc / f)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profiles("decode-256", "gateup") is None          # no summary
    rec = {"source_hash": bench.kernel_source_hash("gateup"), "hbm_bytes_per_launch": 5.47e8}
    (tmp_path / "profiles" / "traffic_gateup_decode-256.json").write_text(json.dumps(rec))
    assert bench.traffic_from_profiles("decode-256", "gateup") == 5.47e8
    # a change to a source of another stage leaves it valid, one to its own sources does not
    (csrc / "router.hip").write_text("// changed\n")
    assert bench.traffic_from_profiles("decode-256", "gateup") == 5.47e8
    with open(csrc / "grouped_gemm.hip", "a") as fh:
        fh.write("// changed\n")
    assert bench.traffic_from_profiles("decode-256", "gateup") is None


def test_committed_traffic_summaries_are_well_formed():
    d = os.path.join(ROOT, "profiles")
    files = [f for f in os.listdir(d) if f.startswith("traffic_") and f.endswith(".json")]
    assert files
    for f in files:
        rec = json.load(open(os.path.join(d, f)))
        assert len(rec["source_hash"]) == 16
        assert rec["hbm_bytes_per_launch"] is None or rec["hbm_bytes_per_launch"] >= 0
