"""Test fixtures: one MoE layer of a synth workload, built twice from the same
seeded fp32 draws -- packed by the library for the GPU, quantized by the
oracle for the fp64 reference.  Only experts in `experts` get real weights
(the others stay zero bytes, i.e. all-zero weights); a test that samples
tokens passes the union of their routed experts."""
from __future__ import annotations

import functools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle as O
import synth


@functools.lru_cache(maxsize=None)
def codebook():
    return O.codebook(0)


def oracle_expert(wl: synth.Workload, e: int):
    """fp64 dequantized (up, gate, down) of expert e, quantized by the oracle."""
    return _oracle_expert_cached(wl.name, e)


# (96 experts: a 16-token step's ~70 distinct experts stay cached between its
# fp64 and mirror sums; ~200 MB each at H = 4096, ~350 MB at H = 7168)
@functools.lru_cache(maxsize=96)
def _oracle_expert_cached(name: str, e: int):
    wl = synth.WORKLOADS[name] if name in synth.WORKLOADS else _CUSTOM[name]
    out = []
    for which, fmt in zip(("up", "gate", "down"), wl.fmts):
        w = synth.expert_weight(wl, which, e)
        f = O.quantize_matrix(fmt, w, codebook())
        out.append(O.dequantize_matrix(f, codebook(), k=w.shape[1]))
    return tuple(out)


def prefetch_oracle_experts(wl: synth.Workload, experts) -> None:
    """Quantizes the given experts in the oracle on a few threads (the C
    search and numpy's array operations release the GIL), so that the layer
    sums that follow find them cached; the values are those oracle_expert
    computes one by one."""
    todo = sorted(set(int(e) for e in np.asarray(experts).reshape(-1)) - {-1})
    if len(todo) > 1:
        with ThreadPoolExecutor(min(8, len(todo), os.cpu_count() or 1)) as ex:
            list(ex.map(lambda e: oracle_expert(wl, e), todo))


def down_k2_as_prefill(wl: synth.Workload, e: int):
    """Expert e's K2 down matrix as the grouped GEMM holds it: per sub-block
    fp16(d*sc) and fp16(-dmin*m), then fp16(q*fp16(d*sc) + fp16(-dmin*m))
    with one rounding (a fused multiply-add)."""
    return _down_k2_cached(wl.name, e)


@functools.lru_cache(maxsize=64)
def _down_k2_cached(name: str, e: int):
    wl = synth.WORKLOADS[name] if name in synth.WORKLOADS else _CUSTOM[name]
    assert wl.fmts[2] == "k2"
    w = synth.expert_weight(wl, "down", e)
    f = O.quantize_matrix("k2", w, codebook())
    q = f["q"].astype(np.float64)
    sc = np.repeat(f["sc"].astype(np.float64), 16, axis=1)
    m = np.repeat(f["m"].astype(np.float64), 16, axis=1)
    d = np.repeat(f["d"], 256, axis=1)
    dmin = np.repeat(f["dmin"], 256, axis=1)
    ds, nm = O.f16(d * sc), O.f16(-(dmin * m))
    return O.f16(q * ds + nm)[:, : w.shape[1]]      # q*ds + nm is exact in fp64


_CUSTOM: dict = {}


def register(wl: synth.Workload):
    """Make a workload defined inside a test known to the caches."""
    _CUSTOM[wl.name] = wl
    return wl


def oracle_shared(wl: synth.Workload, fold: bool = False):
    """fp64 (up, gate, down) of the shared expert: bf16 values, or the Q8
    format's d*q as the oracle quantizes them; fold=True rounds Q8 weights to
    fp16 once (the grouped GEMM's fp16(d*q) operands)."""
    if wl.shared_inter == 0:
        return None
    if wl.fmt_shared == "q8":
        return _oracle_shared_q8_cached(wl.name, fold)
    return tuple(synth.bf16_bits_to_f32(synth.shared_weight_bits(wl, w)).astype(np.float64)
                 for w in ("up", "gate", "down"))


@functools.lru_cache(maxsize=8)
def _oracle_shared_q8_cached(name: str, fold: bool):
    wl = synth.WORKLOADS[name] if name in synth.WORKLOADS else _CUSTOM[name]
    out = []
    for which in ("up", "gate", "down"):
        w = synth.shared_weight_f32(wl, which)
        d = O.dequantize_matrix(O.quantize_matrix("q8", w), k=w.shape[1])
        out.append(O.f16(d) if fold else d)
    return tuple(out)


def oracle_layer(wl: synth.Workload, x64: np.ndarray, round_h=None):
    """(y, idx, weights) of the fp64 oracle for tokens x64 [T, H]."""
    prefetch_oracle_experts(wl, O.route(x64, synth.router_weight(wl), synth.logit_bias(wl), wl.top_k)[0])
    return O.moe_layer(x64, synth.router_weight(wl), synth.logit_bias(wl), wl.top_k,
                       lambda e: oracle_expert(wl, e), shared=oracle_shared(wl), round_h=round_h)


def device_layer(wl: synth.Workload, experts=None, device="cuda"):
    """DeviceLayer with library-packed weights for `experts` (default: all)."""
    import torch
    from bit_quantized_moe_02_amd import qmoe
    E, H, I, Is = wl.n_experts, wl.hidden, wl.inter, wl.shared_inter
    experts = range(E) if experts is None else sorted(set(int(e) for e in experts))
    cb = qmoe.moe_codebook_generate(0)
    nb_up = qmoe.moe_packed_bytes(wl.fmt_up, I, H)
    nb_dn = qmoe.moe_packed_bytes(wl.fmt_down, H, I)
    up = np.zeros(E * nb_up, np.uint8)
    gate = np.zeros(E * nb_up, np.uint8)
    down = np.zeros(E * nb_dn, np.uint8)

    def pack(e):
        qmoe.moe_quantize_pack(wl.fmt_up, synth.expert_weight(wl, "up", e), cb, n_threads=2,
                               out=up[e * nb_up:(e + 1) * nb_up])
        qmoe.moe_quantize_pack(wl.fmt_gate, synth.expert_weight(wl, "gate", e), cb, n_threads=2,
                               out=gate[e * nb_up:(e + 1) * nb_up])
        qmoe.moe_quantize_pack(wl.fmt_down, synth.expert_weight(wl, "down", e), cb, n_threads=2,
                               out=down[e * nb_dn:(e + 1) * nb_dn])

    with ThreadPoolExecutor(8) as ex:
        list(ex.map(pack, experts))
    dev = lambda a: torch.from_numpy(a).to(device)
    sh = [None, None, None]
    if Is > 0:
        for i, which in enumerate(("up", "gate", "down")):
            if wl.fmt_shared == "q8":
                sh[i] = dev(qmoe.moe_quantize_pack("q8", synth.shared_weight_f32(wl, which)))
            else:
                wf = synth.bf16_bits_to_f32(synth.shared_weight_bits(wl, which))
                sh[i] = dev(qmoe.moe_quantize_pack("bf16", wf))
    router = dev(synth.router_weight(wl))
    bias = synth.logit_bias(wl)
    bias = dev(bias) if bias is not None else None
    cbd = dev(cb.reshape(-1).copy()) if "cb2" in wl.fmts else None
    return qmoe.DeviceLayer(E, H, I, Is, wl.fmts, dev(up), dev(gate), dev(down), codebook=cbd,
                            shared_up=sh[0], shared_gate=sh[1], shared_down=sh[2], router=router, bias=bias,
                            shared_fmt=wl.fmt_shared)


def x_bits(wl: synth.Workload, n: int, step: int = 0):
    """bf16 bits [n, H] of the workload's input and the same values in fp64."""
    b = synth.activations_bits(wl, n, step)
    return b, synth.bf16_bits_to_f32(b).astype(np.float64)


def rel_err(y: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """Per-token normwise error max|y - y_ref| / max|y_ref|."""
    return np.max(np.abs(y - y_ref), axis=1) / np.max(np.abs(y_ref), axis=1)


def near_tie_tokens(logits: np.ndarray, k: int, rel: float = 1e-5) -> np.ndarray:
    """Tokens whose k-th and (k+1)-th fp64 logits are closer than
    rel * max(1, |l_k|): there an fp32 router may legitimately pick either."""
    s = -np.sort(-logits, axis=1)
    if s.shape[1] <= k:
        return np.zeros(s.shape[0], bool)
    gap = s[:, k - 1] - s[:, k]
    return gap < rel * np.maximum(1.0, np.abs(s[:, k - 1]))
