"""GPU parity of expert streaming: the decode step run through an HBM expert
cache smaller than the layer (moe_layer_decode_streamed: route, choices to
the host, plan, copies of the missing experts, expert FFN over the cache)
gives the same choices, weights and outputs, bit for bit, as the resident
layer's moe_layer_decode, over sequences of steps with hits, misses and
evictions; also with the copies on a stream of their own, and through the
separate plan / fetch / expert-FFN calls.  (Reading of the osrepos summary,
"SSD Streaming for Large Models": routed experts loaded on demand into a
cache of a set size; host memory stands in for the disk.)
"""
import dataclasses

import numpy as np
import pytest

import oracle as O
import synth

from layer_fixture import device_layer, register, x_bits
from oracle.expert_cache import LruExpertCache

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


def _resident(q, layer, xb, k):
    import torch
    T, H = xb.shape
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(q.moe_layer_decode_workspace_bytes(layer.w, T, k), dtype=torch.uint8, device="cuda")
    q.moe_layer_decode(layer.w, layer.router, layer.bias, _bf16(xb), T, k, idx, w, y, ws)
    torch.cuda.synchronize()
    return idx, w, y


def _cache_for(q, wl, layer, n_slots, keep):
    t = layer.tensors
    host = [t[n].cpu().numpy() for n in ("up", "gate", "down")]
    return q.ExpertCache(wl.n_experts, wl.hidden, wl.inter, wl.fmts, *host, n_slots=n_slots, keep=keep,
                         shared_from=layer)


def _streamed(q, cache, layer, xb, k, copy_stream=None):
    import torch
    T, H = xb.shape
    idx = torch.full((T, k), -9, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), -9.0, dtype=torch.float32, device="cuda")
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.randint(0, 256, (cache.decode_workspace_bytes(T, k),), dtype=torch.uint8, device="cuda")
    cache.decode(layer.router, layer.bias, _bf16(xb), T, k, idx, w, y, ws, copy_stream=copy_stream)
    torch.cuda.synchronize()
    return idx, w, y


def _steps(wl, T, order):
    return [x_bits(wl, T, step=s)[0] for s in order]


ODD_CB2 = register(synth.Workload("odd_cb2_test", 512, 160, 32, 5, 96, "cb2", "cb2", "k2", seed=13, tokens=1))
ODD_K4 = register(synth.Workload("odd_k4_test", 768, 96, 24, 3, 48, "k4", "k4", "k4", seed=14, tokens=1))
ODD_CB2_Q8 = register(dataclasses.replace(ODD_CB2, name="odd_cb2_q8_stream", fmt_shared="q8"))


# (with keep = 1 a cache must hold two steps' experts)
@pytest.mark.parametrize("wl,T,n_slots,keep", [(ODD_CB2, 1, 10, 1), (ODD_CB2, 2, 12, 0), (ODD_K4, 1, 6, 1),
                                               (ODD_CB2_Q8, 3, 16, 0), (ODD_K4, 4, 12, 0)],
                         ids=["cb2_T1", "cb2_T2", "k4_T1", "cb2_q8_T3", "k4_T4"])
def test_streamed_decode_equals_resident(q, wl, T, n_slots, keep):
    """Small layers, every expert packed: 8 steps (some repeated, so hits,
    misses and evictions all occur), streamed and resident outputs equal."""
    print(f"streamed {wl.name} T={T} slots={n_slots}", flush=True)
    layer = device_layer(wl)
    cache = _cache_for(q, wl, layer, n_slots, keep)
    ref = LruExpertCache(wl.n_experts, n_slots, keep)
    order = [0, 1, 0, 2, 3, 1, 4, 0]
    for s, xb in zip(order, _steps(wl, T, order)):
        ri, rw, ry = _resident(q, layer, xb, wl.top_k)
        si, sw, sy = _streamed(q, cache, layer, xb, wl.top_k)
        assert np.array_equal(si.cpu().numpy(), ri.cpu().numpy()), s
        assert np.array_equal(sw.cpu().numpy(), rw.cpu().numpy()), s
        assert np.array_equal(sy.cpu().numpy(), ry.cpu().numpy()), s
        ref.plan(ri.cpu().numpy().reshape(-1).tolist())
        eos, hits, misses = cache.state()
        assert sorted(e for e in eos.tolist() if e >= 0) == sorted(ref.resident)
    assert hits > 0 and misses > n_slots          # hits and evictions happened
    cache.close()


def test_streamed_decode_full_size_copy_stream(q):
    """decode_b1 (H = 4096, E = 256, k = 8) with 24 slots and the copies on a
    stream of their own: six steps, three of them repeats."""
    import torch
    wl = synth.WORKLOADS["decode_b1"]
    order = [0, 1, 0, 2, 1, 3]
    xs = _steps(wl, 1, order)
    need = set()
    for xb in xs:
        x64 = synth.bf16_bits_to_f32(xb).astype(np.float64)
        need |= set(O.route(x64, synth.router_weight(wl), None, wl.top_k)[0].reshape(-1).tolist())
    layer = device_layer(wl, experts=need)
    cache = _cache_for(q, wl, layer, 24, 1)
    cs = torch.cuda.Stream()
    for s, xb in zip(order, xs):
        ri, rw, ry = _resident(q, layer, xb, wl.top_k)
        si, sw, sy = _streamed(q, cache, layer, xb, wl.top_k, copy_stream=cs)
        assert torch.equal(si, ri) and torch.equal(sw, rw) and torch.equal(sy, ry), s
    _, hits, misses = cache.state()
    assert hits >= 16 and misses >= 24
    cache.close()


def test_plan_fetch_then_expert_ffn(q):
    """The separate calls: plan on the host, fetch on the stream, then
    moe_expert_ffn_decode over the cache's weight set with the slot ids."""
    import torch
    wl = ODD_CB2
    layer = device_layer(wl)
    cache = _cache_for(q, wl, layer, 10, 0)
    for s in range(4):
        xb = x_bits(wl, 2, step=s)[0]
        ri, rw, ry = _resident(q, layer, xb, wl.top_k)
        slots, me, ms = cache.plan(ri.cpu().numpy())
        cache.fetch(me, ms)
        y = torch.full_like(ry, float("nan"))
        ws = torch.empty(q.moe_ffn_workspace_bytes(cache.w, 2, wl.top_k, False), dtype=torch.uint8, device="cuda")
        q.moe_expert_ffn_decode(cache.w, _bf16(xb), 2, wl.top_k, torch.from_numpy(slots.reshape(2, -1)).cuda(), rw,
                                y, ws)
        torch.cuda.synchronize()
        assert torch.equal(y, ry), s
    cache.close()


def test_streamed_decode_refuses_overfull_step(q):
    """A step that needs more experts than the cache has slots is refused
    after routing: the choices and weights are written (they decide the
    refusal), y and the cache are untouched, and the next step that fits
    runs as the resident layer does."""
    import torch
    wl = ODD_CB2
    layer = device_layer(wl)
    xb = x_bits(wl, 2, step=5)[0]
    ri, rw, _ = _resident(q, layer, xb, wl.top_k)
    distinct = len(set(ri.cpu().numpy().reshape(-1).tolist()))
    assert distinct > wl.top_k                    # the two tokens share fewer than k experts
    n_slots = distinct - 1
    print(f"overfull step: {distinct} experts, {n_slots} slots", flush=True)
    cache = _cache_for(q, wl, layer, n_slots, 0)
    T, H = xb.shape
    idx = torch.full((T, wl.top_k), -9, dtype=torch.int32, device="cuda")
    w = torch.full((T, wl.top_k), -9.0, dtype=torch.float32, device="cuda")
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(cache.decode_workspace_bytes(T, wl.top_k), dtype=torch.uint8, device="cuda")
    with pytest.raises(q.QmoeError) as ei:
        cache.decode(layer.router, layer.bias, _bf16(xb), T, wl.top_k, idx, w, y, ws)
    torch.cuda.synchronize()
    assert ei.value.code == q.MOE_ERR_INVALID_ARG
    assert "slots" in q.moe_last_error()
    assert torch.equal(idx, ri) and torch.equal(w, rw)
    assert torch.isnan(y).all()
    eos, hits, misses = cache.state()
    assert (eos == -1).all() and hits == 0 and misses == 0
    # one token needs only k experts
    x1 = x_bits(wl, 1, step=6)[0]
    r1 = _resident(q, layer, x1, wl.top_k)
    s1 = _streamed(q, cache, layer, x1, wl.top_k)
    assert all(torch.equal(a, b) for a, b in zip(s1, r1))
    cache.close()
