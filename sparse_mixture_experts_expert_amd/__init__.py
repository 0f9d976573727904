"""OLMoE mixture-of-experts feed-forward layer on MI355X (gfx950).

The layer runs in the HIP library libolmoe_moe.so behind the C ABI of
include/olmoe_moe.h; `binding` is its thin ctypes wrapper (torch provides
device memory and streams) and `inputs` draws the seeded synthetic workloads.
"""
from . import inputs  # noqa: F401
from .binding import (  # noqa: F401
    OlmoeError, abi_version, dispatch_tables, make_workspace, moe_forward, moe_stack_forward,
    residual_add, rmsnorm_bf16, timing_enable, timing_read, workspace_bytes, workspace_layout,
)
