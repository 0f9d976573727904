"""olmoe_moe_forward_noalloc (the layer with the library-owned scratch, for callers that cannot
allocate) against olmoe_moe_forward on the same inputs: the same kernels run, so every output
must be equal bit for bit, on two calls in a row, the second with fewer tokens."""
import numpy as np
import pytest

from sparse_mixture_experts_expert_amd import binding, inputs

torch = pytest.importorskip("torch")


def _log(msg):
    print(f"[no-alloc] {msg}", flush=True)


@pytest.mark.gpu
def test_forward_noalloc_matches_forward_on_two_calls():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    binding.lib()
    w = inputs.device_weights(seed=0, workload="parity")
    ws = (w["w_router"], w["w_gate"], w["w_up"], w["w_down"])
    dev = "cuda"
    for T in (binding.NOALLOC_MAX_TOKENS, 300, 37):
        _log(f"T={T}")
        x = inputs.device_x(T, seed=40 + T, workload="parity")
        ref = binding.moe_forward(x, *ws)
        outs = dict(out=torch.empty((T, 2048), dtype=torch.bfloat16, device=dev),
                    route_ids=torch.empty((T, 8), dtype=torch.int32, device=dev),
                    route_probs=torch.empty((T, 8), dtype=torch.float32, device=dev),
                    expert_counts=torch.empty(64, dtype=torch.int32, device=dev),
                    aux_loss=torch.empty(1, dtype=torch.float32, device=dev),
                    z_loss=torch.empty(1, dtype=torch.float32, device=dev))
        got = binding.moe_forward_noalloc(x, *ws, **outs)
        torch.cuda.synchronize()
        for k in ("out", "route_ids", "route_probs", "expert_counts", "aux_loss", "z_loss"):
            a, b = ref[k], got[k]
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            np.testing.assert_array_equal(b.cpu().numpy(), a.cpu().numpy(), err_msg=f"T={T} {k}")
    # more tokens than the scratch holds: rejected before anything is enqueued
    x = inputs.device_x(binding.NOALLOC_MAX_TOKENS + 1, seed=3, workload="parity")
    with pytest.raises(binding.OlmoeError) as ei:
        binding.moe_forward_noalloc(x, *ws)
    assert ei.value.status == binding.EINVAL


@pytest.mark.gpu
def test_forward_noalloc_replays_in_a_graph():
    """The allocation-free forward captured in a HIP graph (the use it exists for): every replay
    equals the plain forward bit for bit, with eager allocation-free calls of other sizes in
    between that overwrite the shared scratch."""
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    binding.lib()
    w = inputs.device_weights(seed=0, workload="parity")
    ws = (w["w_router"], w["w_gate"], w["w_up"], w["w_down"])
    dev = "cuda"
    T = 256
    x = inputs.device_x(T, seed=77, workload="parity")
    ref = binding.moe_forward(x, *ws)
    torch.cuda.synchronize()
    outs = dict(out=torch.empty((T, 2048), dtype=torch.bfloat16, device=dev),
                route_ids=torch.empty((T, 8), dtype=torch.int32, device=dev),
                route_probs=torch.empty((T, 8), dtype=torch.float32, device=dev),
                expert_counts=torch.empty(64, dtype=torch.int32, device=dev),
                aux_loss=torch.empty(1, dtype=torch.float32, device=dev),
                z_loss=torch.empty(1, dtype=torch.float32, device=dev))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        binding.moe_forward_noalloc(x, *ws, stream=s, **outs)   # first call on the device outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        binding.moe_forward_noalloc(x, *ws, stream=s, **outs)
    for rep, other_T in enumerate((600, 31, 1024)):
        _log(f"replay {rep} after an eager call of {other_T} tokens")
        for t in outs.values():
            t.fill_(-3)
        binding.moe_forward_noalloc(inputs.device_x(other_T, seed=80 + rep, workload="parity"), *ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k], ref[k]), (rep, k)
