"""Thin ctypes binding of libolmoe_moe.so (include/olmoe_moe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
torch supplies device memory and the current stream.  If the library has not
been built, every call raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libolmoe_moe.so")

D, F, E, K = 2048, 1024, 64, 8
OK, EINVAL, EWORKSPACE, EHIP, ENODEVICE = range(5)
ROUTE_RENORMALIZE = 1
KEEP_ALL = (1 << 64) - 1
EC_MAX_TOKENS = 1 << 16
STATUS_NAMES = {0: "OLMOE_OK", 1: "OLMOE_EINVAL", 2: "OLMOE_EWORKSPACE", 3: "OLMOE_EHIP", 4: "OLMOE_ENODEVICE"}

_lib = None


class OlmoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the HIP library (once); raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_mixture_experts_expert_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, sz, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    L.olmoe_abi_version.restype = i32
    L.olmoe_abi_version.argtypes = []
    L.olmoe_last_error.restype = ctypes.c_char_p
    L.olmoe_last_error.argtypes = []
    L.olmoe_moe_workspace_bytes.restype = sz
    L.olmoe_moe_workspace_bytes.argtypes = [i64]
    L.olmoe_moe_workspace_layout.restype = i32
    L.olmoe_moe_workspace_layout.argtypes = [i64, ctypes.POINTER(sz), ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.olmoe_moe_forward.restype = i32
    L.olmoe_moe_forward.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.olmoe_moe_forward_ex.restype = i32
    L.olmoe_moe_forward_ex.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp,
                                       ctypes.c_uint32, ctypes.c_uint64, vp, sz, vp]
    L.olmoe_moe_forward_noalloc.restype = i32
    L.olmoe_moe_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp]
    L.olmoe_moe_forward_residual.restype = i32
    L.olmoe_moe_forward_residual.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp, ctypes.c_float, vp, vp, vp, vp,
                                             vp, ctypes.c_uint32, ctypes.c_uint64, vp, sz, vp]
    L.olmoe_moe_backward_workspace_bytes.restype = sz
    L.olmoe_moe_backward_workspace_bytes.argtypes = [i64]
    L.olmoe_moe_backward.restype = i32
    L.olmoe_moe_backward.argtypes = [vp, vp, vp, vp, vp, i64, vp, ctypes.c_float, ctypes.c_float, vp, vp, vp, vp,
                                     vp, vp, sz, vp]
    L.olmoe_moe_ec_workspace_bytes.restype = sz
    L.olmoe_moe_ec_workspace_bytes.argtypes = [i64]
    L.olmoe_moe_forward_expert_choice.restype = i32
    L.olmoe_moe_forward_expert_choice.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.olmoe_moe_ec_backward_workspace_bytes.restype = sz
    L.olmoe_moe_ec_backward_workspace_bytes.argtypes = [i64]
    L.olmoe_moe_backward_expert_choice.restype = i32
    L.olmoe_moe_backward_expert_choice.argtypes = [vp, vp, vp, vp, vp, i64, vp, ctypes.c_float, ctypes.c_float, vp,
                                                   vp, vp, vp, vp, vp, sz, vp]
    L.olmoe_moe_saved_bytes.restype = sz
    L.olmoe_moe_saved_bytes.argtypes = [i64]
    L.olmoe_moe_forward_train.restype = i32
    L.olmoe_moe_forward_train.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.olmoe_moe_backward_saved.restype = i32
    L.olmoe_moe_backward_saved.argtypes = [vp, vp, vp, vp, vp, i64, vp, ctypes.c_float, ctypes.c_float, vp, vp, vp,
                                           vp, vp, vp, sz, vp]
    L.olmoe_moe_ec_saved_bytes.restype = sz
    L.olmoe_moe_ec_saved_bytes.argtypes = [i64]
    L.olmoe_moe_forward_expert_choice_train.restype = i32
    L.olmoe_moe_forward_expert_choice_train.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.olmoe_moe_backward_expert_choice_saved.restype = i32
    L.olmoe_moe_backward_expert_choice_saved.argtypes = [vp, vp, vp, vp, vp, i64, vp, ctypes.c_float, ctypes.c_float,
                                                         vp, vp, vp, vp, vp, vp, sz, vp]
    L.olmoe_moe_backward_ex.restype = i32
    L.olmoe_moe_backward_ex.argtypes = [vp, vp, vp, vp, vp, i64, vp, ctypes.c_float, ctypes.c_float, vp, vp, vp, vp,
                                        vp, vp, sz, ctypes.c_uint32, vp]
    L.olmoe_rmsnorm_bf16.restype = i32
    L.olmoe_rmsnorm_bf16.argtypes = [vp, ctypes.c_float, i64, vp, vp]
    L.olmoe_residual_add.restype = i32
    L.olmoe_residual_add.argtypes = [vp, vp, i64, vp]
    L.olmoe_timing_enable.restype = i32
    L.olmoe_timing_enable.argtypes = [i32]
    L.olmoe_timing_read.restype = i32
    L.olmoe_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), i32, ctypes.POINTER(i32)]
    L.olmoe_timing_every.restype = i32
    L.olmoe_timing_every.argtypes = [i32]
    L.olmoe_timing_stage_name.restype = ctypes.c_char_p
    L.olmoe_timing_stage_name.argtypes = [i32]
    _lib = L
    return L


def _check(status: int):
    if status != OK:
        raise OlmoeError(status, lib().olmoe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr() or None)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t, name, dtype, shape):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on the GPU, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def abi_version() -> int:
    return lib().olmoe_abi_version()


def workspace_bytes(T: int) -> int:
    return int(lib().olmoe_moe_workspace_bytes(int(T)))


def workspace_layout(T: int):
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().olmoe_moe_workspace_layout(int(T), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return {"perm": a.value, "inv": b.value, "offsets": c.value}


def make_workspace(T: int, device="cuda"):
    import torch
    return torch.empty(max(workspace_bytes(T), 256), dtype=torch.uint8, device=device)


def keep_mask_bits(keep) -> int:
    """A keep mask as the ABI's 64-bit integer (bit e set: expert e may be chosen).
    Accepts None (every expert), an int, a boolean array of 64 entries, or expert ids."""
    import numpy as np
    if keep is None:
        return KEEP_ALL
    if isinstance(keep, int):
        return keep & KEEP_ALL
    arr = np.asarray(keep.cpu() if hasattr(keep, "cpu") else keep)
    if arr.dtype == bool:
        if arr.shape != (E,):
            raise ValueError(f"boolean keep mask must have {E} entries, got {arr.shape}")
        arr = np.flatnonzero(arr)
    return sum(1 << int(e) for e in set(arr.ravel().tolist()))


def moe_forward(x, w_router, w_gate, w_up, w_down, *, out=None, route_ids=None, route_probs=None,
                expert_counts=None, aux_loss=None, z_loss=None, workspace=None, stream=None,
                want_routing=True, renormalize=False, keep=None):
    """One MoE layer (olmoe_moe_forward, or olmoe_moe_forward_ex for the router
    variants: renormalize=True, keep = experts that may be chosen).  Tensors are
    torch CUDA tensors: x bf16 [T,2048], w_router fp32 [64,2048], w_gate / w_up
    bf16 [64,1024,2048], w_down bf16 [64,2048,1024].  Missing outputs are
    allocated (routing outputs only when want_routing).  Returns a dict of the
    output tensors."""
    import torch
    T = x.shape[0]
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, D))
    _need(w_router, "w_router", torch.float32, (E, D))
    _need(w_gate, "w_gate", torch.bfloat16, (E, F, D))
    _need(w_up, "w_up", torch.bfloat16, (E, F, D))
    _need(w_down, "w_down", torch.bfloat16, (E, D, F))
    if out is None:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    if want_routing:
        route_ids = route_ids if route_ids is not None else torch.empty((T, K), dtype=torch.int32, device=dev)
        route_probs = route_probs if route_probs is not None else torch.empty((T, K), dtype=torch.float32, device=dev)
        expert_counts = expert_counts if expert_counts is not None else torch.empty(E, dtype=torch.int32, device=dev)
        aux_loss = aux_loss if aux_loss is not None else torch.empty(1, dtype=torch.float32, device=dev)
        z_loss = z_loss if z_loss is not None else torch.empty(1, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = make_workspace(T, dev)
    if renormalize or keep is not None:
        _check(lib().olmoe_moe_forward_ex(
            _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), int(T), _ptr(out),
            _ptr(route_ids), _ptr(route_probs), _ptr(expert_counts), _ptr(aux_loss), _ptr(z_loss),
            ROUTE_RENORMALIZE if renormalize else 0, keep_mask_bits(keep),
            _ptr(workspace), workspace.numel(), _stream(stream)))
    else:
        _check(lib().olmoe_moe_forward(
            _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), int(T), _ptr(out),
            _ptr(route_ids), _ptr(route_probs), _ptr(expert_counts), _ptr(aux_loss), _ptr(z_loss),
            _ptr(workspace), workspace.numel(), _stream(stream)))
    return {"out": out, "route_ids": route_ids, "route_probs": route_probs,
            "expert_counts": expert_counts, "aux_loss": aux_loss, "z_loss": z_loss,
            "workspace": workspace}


NOALLOC_MAX_TOKENS = 1024
NOALLOC_SCRATCH_BYTES = 60 << 20


def moe_forward_noalloc(x, w_router, w_gate, w_up, w_down, *, out=None, route_ids=None, route_probs=None,
                        expert_counts=None, aux_loss=None, z_loss=None, stream=None):
    """The layer with the library-owned scratch instead of a workspace
    (olmoe_moe_forward_noalloc, at most NOALLOC_MAX_TOKENS tokens).  Missing
    outputs are allocated here by torch, not by the library; pass them all to
    make the call allocation-free.  Calls that overlap on one GPU race."""
    import torch
    T = x.shape[0]
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, D))
    if out is None:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    _check(lib().olmoe_moe_forward_noalloc(
        _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), int(T), _ptr(out),
        _ptr(route_ids), _ptr(route_probs), _ptr(expert_counts), _ptr(aux_loss), _ptr(z_loss),
        _stream(stream)))
    return {"out": out, "route_ids": route_ids, "route_probs": route_probs, "expert_counts": expert_counts,
            "aux_loss": aux_loss, "z_loss": z_loss}


def backward_workspace_bytes(T: int) -> int:
    return int(lib().olmoe_moe_backward_workspace_bytes(int(T)))


def moe_backward(x, w_router, w_gate, w_up, w_down, dout, *, g_aux: float = 1.0, g_z: float = 1.0,
                 dx=None, dw_router=None, dw_gate=None, dw_up=None, dw_down=None, workspace=None,
                 stream=None):
    """Gradients of <dout, out> + g_aux * aux + g_z * z (olmoe_moe_backward) for the default
    router.  dout bf16 [T,2048]; outputs (allocated when missing) are fp32: dx [T,2048],
    dw_router [64,2048], dw_gate / dw_up [64,1024,2048], dw_down [64,2048,1024]."""
    import torch
    T = x.shape[0]
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, D))
    _need(dout, "dout", torch.bfloat16, (T, D))
    _need(w_router, "w_router", torch.float32, (E, D))
    _need(w_gate, "w_gate", torch.bfloat16, (E, F, D))
    _need(w_up, "w_up", torch.bfloat16, (E, F, D))
    _need(w_down, "w_down", torch.bfloat16, (E, D, F))
    f32 = torch.float32
    dx = dx if dx is not None else torch.empty((T, D), dtype=f32, device=dev)
    dw_router = dw_router if dw_router is not None else torch.empty((E, D), dtype=f32, device=dev)
    dw_gate = dw_gate if dw_gate is not None else torch.empty((E, F, D), dtype=f32, device=dev)
    dw_up = dw_up if dw_up is not None else torch.empty((E, F, D), dtype=f32, device=dev)
    dw_down = dw_down if dw_down is not None else torch.empty((E, D, F), dtype=f32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(backward_workspace_bytes(T), 256), dtype=torch.uint8, device=dev)
    _check(lib().olmoe_moe_backward(
        _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), int(T), _ptr(dout),
        ctypes.c_float(g_aux), ctypes.c_float(g_z), _ptr(dx), _ptr(dw_router), _ptr(dw_gate), _ptr(dw_up),
        _ptr(dw_down), _ptr(workspace), workspace.numel(), _stream(stream)))
    return {"dx": dx, "dw_router": dw_router, "dw_gate": dw_gate, "dw_up": dw_up, "dw_down": dw_down,
            "workspace": workspace}


def ec_capacity(T: int) -> int:
    """Tokens each expert takes under expert choice: ceil(8T / 64)."""
    return -(-K * int(T) // E)


def ec_workspace_bytes(T: int) -> int:
    return int(lib().olmoe_moe_ec_workspace_bytes(int(T)))


def moe_forward_expert_choice(x, w_router, w_gate, w_up, w_down, *, out=None, choice_tokens=None,
                              choice_probs=None, token_counts=None, aux_loss=None, z_loss=None,
                              workspace=None, stream=None, want_routing=True):
    """One MoE layer with expert-choice routing (olmoe_moe_forward_expert_choice): every
    expert takes its C = ceil(8T/64) most probable tokens.  Tensors as moe_forward; the
    routing outputs are choice_tokens int32 [64,C] (ascending per expert), choice_probs
    fp32 [64,C], token_counts int32 [T], aux_loss / z_loss fp32 [1], allocated when missing
    (only when want_routing).  Returns a dict of the output tensors."""
    import torch
    T = x.shape[0]
    dev = x.device
    C = ec_capacity(T)
    _need(x, "x", torch.bfloat16, (T, D))
    _need(w_router, "w_router", torch.float32, (E, D))
    _need(w_gate, "w_gate", torch.bfloat16, (E, F, D))
    _need(w_up, "w_up", torch.bfloat16, (E, F, D))
    _need(w_down, "w_down", torch.bfloat16, (E, D, F))
    if out is None:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    if want_routing:
        i32, f32 = torch.int32, torch.float32
        choice_tokens = choice_tokens if choice_tokens is not None else torch.empty((E, C), dtype=i32, device=dev)
        choice_probs = choice_probs if choice_probs is not None else torch.empty((E, C), dtype=f32, device=dev)
        token_counts = token_counts if token_counts is not None else torch.empty(T, dtype=i32, device=dev)
        aux_loss = aux_loss if aux_loss is not None else torch.empty(1, dtype=f32, device=dev)
        z_loss = z_loss if z_loss is not None else torch.empty(1, dtype=f32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(ec_workspace_bytes(T), 256), dtype=torch.uint8, device=dev)
    _check(lib().olmoe_moe_forward_expert_choice(
        _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), int(T), _ptr(out),
        _ptr(choice_tokens), _ptr(choice_probs), _ptr(token_counts), _ptr(aux_loss), _ptr(z_loss),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return {"out": out, "choice_tokens": choice_tokens, "choice_probs": choice_probs,
            "token_counts": token_counts, "aux_loss": aux_loss, "z_loss": z_loss, "workspace": workspace}


def saved_bytes(T: int) -> int:
    return int(lib().olmoe_moe_saved_bytes(int(T)))


def moe_forward_train(x, w_router, w_gate, w_up, w_down, *, saved=None, out=None, route_ids=None,
                      route_probs=None, expert_counts=None, aux_loss=None, z_loss=None, stream=None):
    """olmoe_moe_forward_train: the layer's forward, keeping its state in `saved` (allocated
    when missing, olmoe_moe_saved_bytes(T)) for moe_backward_saved.  Returns a dict of the
    outputs and `saved`."""
    import torch
    T = x.shape[0]
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, D))
    _need(w_router, "w_router", torch.float32, (E, D))
    _need(w_gate, "w_gate", torch.bfloat16, (E, F, D))
    _need(w_up, "w_up", torch.bfloat16, (E, F, D))
    _need(w_down, "w_down", torch.bfloat16, (E, D, F))
    out = out if out is not None else torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    if saved is None:
        saved = torch.empty(max(saved_bytes(T), 256), dtype=torch.uint8, device=dev)
    _check(lib().olmoe_moe_forward_train(
        _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), int(T), _ptr(out), _ptr(route_ids),
        _ptr(route_probs), _ptr(expert_counts), _ptr(aux_loss), _ptr(z_loss), _ptr(saved), saved.numel(),
        _stream(stream)))
    return {"out": out, "route_ids": route_ids, "route_probs": route_probs, "expert_counts": expert_counts,
            "aux_loss": aux_loss, "z_loss": z_loss, "saved": saved}


def moe_backward_saved(x, w_router, w_gate, w_up, w_down, dout, saved, *, g_aux: float = 1.0, g_z: float = 1.0,
                       dx=None, dw_router=None, dw_gate=None, dw_up=None, dw_down=None, stream=None):
    """olmoe_moe_backward_saved: the gradients of moe_backward from the state moe_forward_train left
    in `saved` for the same x and weights (which this call consumes)."""
    import torch
    T = x.shape[0]
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, D))
    _need(dout, "dout", torch.bfloat16, (T, D))
    f32 = torch.float32
    dx = dx if dx is not None else torch.empty((T, D), dtype=f32, device=dev)
    dw_router = dw_router if dw_router is not None else torch.empty((E, D), dtype=f32, device=dev)
    dw_gate = dw_gate if dw_gate is not None else torch.empty((E, F, D), dtype=f32, device=dev)
    dw_up = dw_up if dw_up is not None else torch.empty((E, F, D), dtype=f32, device=dev)
    dw_down = dw_down if dw_down is not None else torch.empty((E, D, F), dtype=f32, device=dev)
    _check(lib().olmoe_moe_backward_saved(
        _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), int(T), _ptr(dout),
        ctypes.c_float(g_aux), ctypes.c_float(g_z), _ptr(dx), _ptr(dw_router), _ptr(dw_gate), _ptr(dw_up),
        _ptr(dw_down), _ptr(saved), saved.numel(), _stream(stream)))
    return {"dx": dx, "dw_router": dw_router, "dw_gate": dw_gate, "dw_up": dw_up, "dw_down": dw_down}


def ec_saved_bytes(T: int) -> int:
    return int(lib().olmoe_moe_ec_saved_bytes(int(T)))


def moe_forward_expert_choice_train(x, w_router, w_gate, w_up, w_down, *, saved=None, out=None, choice_tokens=None,
                                    choice_probs=None, token_counts=None, aux_loss=None, z_loss=None, stream=None):
    """olmoe_moe_forward_expert_choice_train: the expert-choice forward, keeping its state in `saved`
    (allocated when missing) for moe_backward_expert_choice_saved."""
    import torch
    T = x.shape[0]
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, D))
    out = out if out is not None else torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    if saved is None:
        saved = torch.empty(max(ec_saved_bytes(T), 256), dtype=torch.uint8, device=dev)
    _check(lib().olmoe_moe_forward_expert_choice_train(
        _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), int(T), _ptr(out), _ptr(choice_tokens),
        _ptr(choice_probs), _ptr(token_counts), _ptr(aux_loss), _ptr(z_loss), _ptr(saved), saved.numel(),
        _stream(stream)))
    return {"out": out, "choice_tokens": choice_tokens, "choice_probs": choice_probs, "token_counts": token_counts,
            "aux_loss": aux_loss, "z_loss": z_loss, "saved": saved}


def moe_backward_expert_choice_saved(x, w_router, w_gate, w_up, w_down, dout, saved, *, g_aux: float = 1.0,
                                     g_z: float = 1.0, dx=None, dw_router=None, dw_gate=None, dw_up=None,
                                     dw_down=None, stream=None):
    """olmoe_moe_backward_expert_choice_saved: moe_backward_expert_choice's gradients from the state
    moe_forward_expert_choice_train left in `saved`."""
    import torch
    T = x.shape[0]
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, D))
    _need(dout, "dout", torch.bfloat16, (T, D))
    f32 = torch.float32
    dx = dx if dx is not None else torch.empty((T, D), dtype=f32, device=dev)
    dw_router = dw_router if dw_router is not None else torch.empty((E, D), dtype=f32, device=dev)
    dw_gate = dw_gate if dw_gate is not None else torch.empty((E, F, D), dtype=f32, device=dev)
    dw_up = dw_up if dw_up is not None else torch.empty((E, F, D), dtype=f32, device=dev)
    dw_down = dw_down if dw_down is not None else torch.empty((E, D, F), dtype=f32, device=dev)
    _check(lib().olmoe_moe_backward_expert_choice_saved(
        _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), int(T), _ptr(dout),
        ctypes.c_float(g_aux), ctypes.c_float(g_z), _ptr(dx), _ptr(dw_router), _ptr(dw_gate), _ptr(dw_up),
        _ptr(dw_down), _ptr(saved), saved.numel(), _stream(stream)))
    return {"dx": dx, "dw_router": dw_router, "dw_gate": dw_gate, "dw_up": dw_up, "dw_down": dw_down}


def ec_backward_workspace_bytes(T: int) -> int:
    return int(lib().olmoe_moe_ec_backward_workspace_bytes(int(T)))


def moe_backward_expert_choice(x, w_router, w_gate, w_up, w_down, dout, *, g_aux: float = 1.0, g_z: float = 1.0,
                               dx=None, dw_router=None, dw_gate=None, dw_up=None, dw_down=None, workspace=None,
                               stream=None):
    """Gradients of <dout, out> + g_aux * aux + g_z * z for the expert-choice layer
    (olmoe_moe_backward_expert_choice); tensors and outputs as moe_backward."""
    import torch
    T = x.shape[0]
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, D))
    _need(dout, "dout", torch.bfloat16, (T, D))
    _need(w_router, "w_router", torch.float32, (E, D))
    _need(w_gate, "w_gate", torch.bfloat16, (E, F, D))
    _need(w_up, "w_up", torch.bfloat16, (E, F, D))
    _need(w_down, "w_down", torch.bfloat16, (E, D, F))
    f32 = torch.float32
    dx = dx if dx is not None else torch.empty((T, D), dtype=f32, device=dev)
    dw_router = dw_router if dw_router is not None else torch.empty((E, D), dtype=f32, device=dev)
    dw_gate = dw_gate if dw_gate is not None else torch.empty((E, F, D), dtype=f32, device=dev)
    dw_up = dw_up if dw_up is not None else torch.empty((E, F, D), dtype=f32, device=dev)
    dw_down = dw_down if dw_down is not None else torch.empty((E, D, F), dtype=f32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(ec_backward_workspace_bytes(T), 256), dtype=torch.uint8, device=dev)
    _check(lib().olmoe_moe_backward_expert_choice(
        _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), int(T), _ptr(dout),
        ctypes.c_float(g_aux), ctypes.c_float(g_z), _ptr(dx), _ptr(dw_router), _ptr(dw_gate), _ptr(dw_up),
        _ptr(dw_down), _ptr(workspace), workspace.numel(), _stream(stream)))
    return {"dx": dx, "dw_router": dw_router, "dw_gate": dw_gate, "dw_up": dw_up, "dw_down": dw_down,
            "workspace": workspace}


BWD_SAVED = 1 << 0            # OLMOE_BWD_SAVED: workspace is the training forward's saved state
BWD_EXPERT_CHOICE = 1 << 1    # OLMOE_BWD_EXPERT_CHOICE: the expert-choice layer
BWD_GRAD_BF16 = 1 << 2        # OLMOE_BWD_GRAD_BF16: dW_gate / dW_up / dW_down in bf16


def moe_backward_ex(x, w_router, w_gate, w_up, w_down, dout, *, flags: int = 0, g_aux: float = 1.0,
                    g_z: float = 1.0, dx=None, dw_router=None, dw_gate=None, dw_up=None, dw_down=None,
                    workspace=None, stream=None):
    """olmoe_moe_backward_ex: any backward variant chosen by `flags` (BWD_SAVED, BWD_EXPERT_CHOICE,
    BWD_GRAD_BF16).  The expert weight gradients are bf16 with BWD_GRAD_BF16, else fp32; dx and
    dw_router are fp32.  With BWD_SAVED, `workspace` is the training forward's `saved` buffer;
    otherwise it is allocated when missing."""
    import torch
    T = x.shape[0]
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, D))
    _need(dout, "dout", torch.bfloat16, (T, D))
    f32 = torch.float32
    wg = torch.bfloat16 if flags & BWD_GRAD_BF16 else f32
    dx = dx if dx is not None else torch.empty((T, D), dtype=f32, device=dev)
    dw_router = dw_router if dw_router is not None else torch.empty((E, D), dtype=f32, device=dev)
    dw_gate = dw_gate if dw_gate is not None else torch.empty((E, F, D), dtype=wg, device=dev)
    dw_up = dw_up if dw_up is not None else torch.empty((E, F, D), dtype=wg, device=dev)
    dw_down = dw_down if dw_down is not None else torch.empty((E, D, F), dtype=wg, device=dev)
    if workspace is None:
        if flags & BWD_SAVED:
            raise ValueError("BWD_SAVED needs the saved buffer of the training forward as workspace")
        nbytes = ec_backward_workspace_bytes(T) if flags & BWD_EXPERT_CHOICE else backward_workspace_bytes(T)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _check(lib().olmoe_moe_backward_ex(
        _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), int(T), _ptr(dout),
        ctypes.c_float(g_aux), ctypes.c_float(g_z), _ptr(dx), _ptr(dw_router), _ptr(dw_gate), _ptr(dw_up),
        _ptr(dw_down), _ptr(workspace), workspace.numel(), ctypes.c_uint32(flags), _stream(stream)))
    return {"dx": dx, "dw_router": dw_router, "dw_gate": dw_gate, "dw_up": dw_up, "dw_down": dw_down,
            "workspace": workspace}


CLIP_COUNT_OFFSET = 0


def clip_count(workspace) -> int:
    """Number of fp16 intermediates (SwiGLU activations and expert outputs) the last call that used
    this workspace (or `saved` buffer) stored clipped to +-65504 because they were out of range or
    NaN; 0 in normal use.  Synchronises with the device."""
    import torch
    return int(workspace[CLIP_COUNT_OFFSET:CLIP_COUNT_OFFSET + 4].view(torch.int32).item())


def dispatch_tables(workspace, T: int):
    """Views of perm [8T], inv [T,8], offsets [65] inside a workspace after a call."""
    import torch
    lay = workspace_layout(T)
    def view(off, n):
        return workspace[off:off + 4 * n].view(torch.int32)
    return {"perm": view(lay["perm"], 8 * T), "inv": view(lay["inv"], 8 * T).view(T, K),
            "offsets": view(lay["offsets"], E + 1)}


def rmsnorm_bf16(h, eps: float = 1e-5, x_out=None, stream=None):
    import torch
    T = h.shape[0]
    _need(h, "h", torch.float32, (T, D))
    if x_out is None:
        x_out = torch.empty((T, D), dtype=torch.bfloat16, device=h.device)
    _check(lib().olmoe_rmsnorm_bf16(_ptr(h), float(eps), int(T), _ptr(x_out), _stream(stream)))
    return x_out


def residual_add(h, y, stream=None):
    import torch
    T = h.shape[0]
    _need(h, "h", torch.float32, (T, D))
    _need(y, "y", torch.bfloat16, (T, D))
    _check(lib().olmoe_residual_add(_ptr(h), _ptr(y), int(T), _stream(stream)))
    return h


def moe_forward_residual(x, w_router, w_gate, w_up, w_down, h, *, x_next=None, eps: float = 1e-5,
                         route_ids=None, route_probs=None, expert_counts=None, aux_loss=None,
                         z_loss=None, workspace=None, stream=None, renormalize=False, keep=None):
    """One layer of the residual stack with the fused epilogue
    (olmoe_moe_forward_residual): h (fp32 [T,2048]) += the layer's output of x,
    and x_next (bf16 [T,2048], may be x itself) = bf16(RMSNorm(h)) if given."""
    import torch
    T = x.shape[0]
    _need(x, "x", torch.bfloat16, (T, D))
    _need(h, "h", torch.float32, (T, D))
    if x_next is not None:
        _need(x_next, "x_next", torch.bfloat16, (T, D))
    if workspace is None:
        workspace = make_workspace(T, x.device)
    _check(lib().olmoe_moe_forward_residual(
        _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down), int(T), _ptr(h), _ptr(x_next),
        ctypes.c_float(eps), _ptr(route_ids), _ptr(route_probs), _ptr(expert_counts), _ptr(aux_loss),
        _ptr(z_loss), ROUTE_RENORMALIZE if renormalize else 0, keep_mask_bits(keep),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return h


def moe_stack_forward(h, layers, eps: float = 1e-5, keep_inputs: bool = False, keep_states: bool = False,
                      workspace=None, stream=None, fused: bool = True, keep_probs: bool = False,
                      state_rows=None):
    """Residual stack h <- h + MoE_l(RMSNorm(h)) over `layers` (dicts of weight
    tensors), in place on the fp32 residual `h` [T,2048].  fused: each layer's
    combine also updates h and writes the next layer's input
    (olmoe_moe_forward_residual); otherwise RMSNorm, layer and residual add run
    as separate calls (the layer output then passes through bf16).  Returns h
    and, per layer, expert counts / aux / z / route ids, plus the bf16 layer
    inputs (keep_inputs), h after each layer (keep_states; only the rows in
    the index tensor state_rows when it is given, h itself is always whole) and
    the route probabilities (keep_probs, as "route_probs" [L,T,8])."""
    import torch
    T = h.shape[0]
    dev = h.device
    workspace = workspace if workspace is not None else make_workspace(T, dev)
    xbuf = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    ybuf = None if fused else torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    counts = torch.empty((len(layers), E), dtype=torch.int32, device=dev)
    aux = torch.empty(len(layers), dtype=torch.float32, device=dev)
    z = torch.empty(len(layers), dtype=torch.float32, device=dev)
    ids = torch.empty((len(layers), T, K), dtype=torch.int32, device=dev)
    probs = torch.empty((len(layers), T, K), dtype=torch.float32, device=dev) if keep_probs else None
    inputs, states = [], []
    rmsnorm_bf16(h, eps, xbuf, stream)
    for l, w in enumerate(layers):
        if keep_inputs:
            inputs.append(xbuf.clone())
        last = l == len(layers) - 1
        pl = probs[l] if keep_probs else None
        if fused:
            moe_forward_residual(xbuf, w["w_router"], w["w_gate"], w["w_up"], w["w_down"], h,
                                 x_next=None if last else xbuf, eps=eps, route_ids=ids[l], route_probs=pl,
                                 expert_counts=counts[l], aux_loss=aux[l:l + 1], z_loss=z[l:l + 1],
                                 workspace=workspace, stream=stream)
        else:
            moe_forward(xbuf, w["w_router"], w["w_gate"], w["w_up"], w["w_down"], out=ybuf,
                        route_ids=ids[l], route_probs=pl, expert_counts=counts[l],
                        aux_loss=aux[l:l + 1], z_loss=z[l:l + 1], workspace=workspace, stream=stream,
                        want_routing=False)
            residual_add(h, ybuf, stream)
            if not last:
                rmsnorm_bf16(h, eps, xbuf, stream)
        if keep_states:
            states.append(h.clone() if state_rows is None else h[state_rows].clone())
    return {"h": h, "expert_counts": counts, "aux_loss": aux, "z_loss": z, "route_ids": ids,
            "route_probs": probs, "inputs": inputs, "states": states}


TIMING_STAGES = ("router", "dispatch", "gateup", "down", "combine")


def timing_enable(stages=True):
    """Bracket stages of later forward calls with HIP events: True = every stage,
    False = off, or an iterable of stage names."""
    if stages is True:
        mask = (1 << len(TIMING_STAGES)) - 1
    elif not stages:
        mask = 0
    else:
        mask = 0
        for name in stages:
            mask |= 1 << TIMING_STAGES.index(name)
    _check(lib().olmoe_timing_enable(mask))
    global _timing_mask
    _timing_mask = mask


_timing_mask = 0


def timing_every(n):
    """Bracket only every n-th later forward call (the next one first); timing_enable resets it to 1."""
    _check(lib().olmoe_timing_every(int(n)))


def timing_read():
    """Summed milliseconds of each bracketed stage and the number of timed calls since
    timing_enable."""
    buf = (ctypes.c_double * 16)()
    calls = ctypes.c_int()
    n = lib().olmoe_timing_read(buf, 16, ctypes.byref(calls))
    if n < 0:
        raise OlmoeError(EHIP, lib().olmoe_last_error().decode())
    names = [lib().olmoe_timing_stage_name(i).decode() for i in range(n)]
    return {names[i]: buf[i] for i in range(n) if _timing_mask >> i & 1}, calls.value
