"""Build libolmoe_moe.so (the HIP library behind include/olmoe_moe.h) for gfx950.

    python -m sparse_mixture_experts_expert_amd.build        # compile + link in-tree

Each csrc/*.hip is compiled to an object under _build/ (in parallel), then
linked into sparse_mixture_experts_expert_amd/libolmoe_moe.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libolmoe_moe.so")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-result",
    # packed fp32 instructions stay off (the compiler may still use plain fp32 ops)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the target feature above; keep other warnings visible
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stderr or "").splitlines() if ln.strip() and noise not in ln
            and "warnings generated" not in ln and "warning generated" not in ln]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = True, extra: list[str] | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra or []), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


C_CALLER_SRC = os.path.join(ROOT, "tests", "c", "forward_c.c")
C_CALLER = os.path.join(ROOT, "tests", "c", "forward_c")


def build_c_caller(verbose: bool = True) -> str:
    """The plain-C test program that drives olmoe_moe_forward through the HIP runtime's C API
    (gcc; the HIP headers need the platform macro that hipcc would define)."""
    rocm = os.path.dirname(os.path.dirname(hipcc()))
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
           "-I", os.path.join(ROOT, "include"), C_CALLER_SRC, "-L", PKG, "-lolmoe_moe",
           "-Wl,-rpath,$ORIGIN/../../sparse_mixture_experts_expert_amd", "-L", os.path.join(rocm, "lib"),
           "-lamdhip64", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-o", C_CALLER]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C caller build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {C_CALLER}")
    return C_CALLER


if __name__ == "__main__":
    build()
    build_c_caller()
