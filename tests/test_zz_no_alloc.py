"""moe_layer_decode_noalloc (workspace in the library's own device array)
against moe_layer_decode with a caller workspace, through the C ABI: two
calls in a row, the second with fewer tokens, each bit for bit equal to the
workspace call on the same inputs; a layer whose workspace exceeds the array
is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest

import synth
from layer_fixture import device_layer, x_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    assert torch.cuda.is_available(), "GPU test needs a GPU"
    from bit_quantized_moe_02_amd import qmoe
    return qmoe


def _bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits.astype(np.uint16).view(np.int16))).view(torch.bfloat16).cuda()


def _both(q, layer, xb, k):
    """(idx, w, y) of the no-alloc call and of the workspace call."""
    import torch
    T, H = xb.shape
    x = _bf16(xb)
    out = []
    for noalloc in (True, False):
        idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
        w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
        y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            q.moe_layer_decode_noalloc(layer.w, layer.router, layer.bias, x, T, k, idx, w, y)
        else:
            ws = torch.full((q.moe_layer_decode_workspace_bytes(layer.w, T, k),), 0xFF, dtype=torch.uint8,
                            device="cuda")
            q.moe_layer_decode(layer.w, layer.router, layer.bias, x, T, k, idx, w, y, ws)
        torch.cuda.synchronize()
        out.append((idx.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()))
    return out


def test_noalloc_matches_workspace_call(q):
    import torch
    wl = synth.WORKLOADS["decode_b16_hot"]
    xb16, _ = x_bits(wl, 16, step=21)
    xb1, _ = x_bits(wl, 1, step=22)
    # experts the two steps route to (the router needs no expert weights)
    router_only = device_layer(wl, experts=[])
    need = set()
    for xb in (xb16, xb1):
        T = xb.shape[0]
        idx = torch.empty((T, wl.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, wl.top_k), dtype=torch.float32, device="cuda")
        ws = torch.empty(q.moe_route_workspace_bytes(T, wl.n_experts), dtype=torch.uint8, device="cuda")
        q.moe_route(_bf16(xb), router_only.router, router_only.bias, T, wl.hidden, wl.n_experts, wl.top_k, idx,
                    w, ws)
        need |= set(idx.cpu().numpy().reshape(-1).tolist())
    layer = device_layer(wl, experts=need)
    print(f"16-token step then 1-token step, {len(need)} experts", flush=True)
    for xb in (xb16, xb1):
        (ia, wa, ya), (ib, wb, yb) = _both(q, layer, xb, wl.top_k)
        assert np.array_equal(ia, ib), "top-k indices differ"
        assert np.array_equal(wa, wb), "top-k weights differ"
        assert np.array_equal(ya, yb), "outputs differ"
        assert np.all(np.isfinite(ya))
        print(f"T={xb.shape[0]}: identical (max |y| {np.abs(ya).max():.3e})", flush=True)


def test_noalloc_refuses_oversize(q):
    """K4, H = 8192, 16 tokens of 16 choices: the workspace is over 8 MiB."""
    import torch
    wl = synth.Workload("noalloc_big", 8192, 64, 16, 16, 0, "k4", "k4", "k4", seed=30, tokens=16)
    layer = device_layer(wl, experts=[])
    T, k, H = 16, 16, 8192
    assert q.moe_layer_decode_workspace_bytes(layer.w, T, k) > q.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), -7.0, dtype=torch.float32, device="cuda")
    y = torch.full((T, H), -7.0, dtype=torch.float32, device="cuda")
    rc = q.lib.moe_layer_decode_noalloc(ctypes.byref(layer.w), layer.router.data_ptr(), None, x.data_ptr(), T, k,
                                        idx.data_ptr(), w.data_ptr(), y.data_ptr(), None)
    torch.cuda.synchronize()
    assert rc == q.MOE_ERR_WORKSPACE
    assert "8388608" in q.moe_last_error()
    assert torch.all(idx == -7) and torch.all(w == -7.0) and torch.all(y == -7.0)
