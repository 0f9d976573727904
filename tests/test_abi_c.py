"""The C ABI from plain C: the header compiles as C11 with gcc, the library links, and the
host-side entry points behave as documented (no device needed)."""
import os
import shutil
import subprocess

import pytest

from sparse_mixture_experts_expert_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_caller_host_paths(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    binding.lib()   # the library must be built
    exe = tmp_path / "abi_host"
    libdir = os.path.dirname(binding.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host.c"), "-L", libdir, "-lolmoe_moe", f"-Wl,-rpath,{libdir}",
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "passed" in r.stdout
