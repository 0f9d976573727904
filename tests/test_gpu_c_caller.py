"""A plain C program (tests/c/forward_c.c, built by build()) drives olmoe_moe_forward through the
HIP runtime's C API, with no Python or torch in its process; its outputs are checked against the
float64 oracle to the same bar as the Python-driven parity tests."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from sparse_mixture_experts_expert_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu

CALLER = os.path.join(os.path.dirname(__file__), "c", "forward_c")


@pytest.mark.parametrize("T", [300])
def test_forward_from_c(tmp_path, T):
    if not os.path.exists(CALLER):
        pytest.fail(f"{CALLER} is missing: run __graft_entry__.build() first")
    h = inputs.host_layer(T, seed=5, workload="parity")
    files = {"x.bin": h["x"], "wr.bin": h["w_router"], "wg.bin": h["w_gate"], "wu.bin": h["w_up"],
             "wd.bin": h["w_down"]}
    for name, a in files.items():
        np.ascontiguousarray(a).tofile(tmp_path / name)
    print(f"[c-caller] T={T}", flush=True)
    r = subprocess.run([CALLER, str(T), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"forward_c exit {r.returncode}\n{r.stdout}\n{r.stderr}"
    assert "ok" in r.stdout
    out = np.fromfile(tmp_path / "out.bin", np.uint16).reshape(T, 2048)
    ids = np.fromfile(tmp_path / "ids.bin", np.int32).reshape(T, 8)
    probs = np.fromfile(tmp_path / "probs.bin", np.float32).reshape(T, 8)
    counts = np.fromfile(tmp_path / "counts.bin", np.int32)
    aux, z = np.fromfile(tmp_path / "losses.bin", np.float32)

    ref = oracle.moe_layer_ref(h["x"], h["w_router"], h["w_gate"], h["w_up"], h["w_down"], 8)
    ntie = parity.check_routing(ids, probs, ref, "C caller")
    if ntie or not np.array_equal(ids, ref["ids"]):
        ref = oracle.moe_layer_ref(h["x"], h["w_router"], h["w_gate"], h["w_up"], h["w_down"], 8,
                                   forced_ids=ids.astype(np.int64))
    np.testing.assert_array_equal(counts, oracle.dispatch(ids.astype(np.int64), 64)[0])
    parity.check_out(oracle.to_f64(out), ref["out"], "C caller")
    parity.check_losses(float(aux), float(z), ref["aux"], ref["z"], "C caller")
