"""Seeded synthetic workloads for the quantized routed-MoE layer.

This module is the only code shared by the fp64 oracle's tests and the HIP
path's tests and benchmark.  It holds shapes and seeded random draws and
nothing else: no quantization, no routing, no expert arithmetic.  Rounding a
draw to bf16 (the layer's activation and shared-expert storage type) is done
here with torch's own conversion, so the value handed to both sides is the
same bf16 number.

Every tensor comes from its own generator, ``numpy.random.default_rng([seed,
tag, index])``, so any expert or token can be regenerated alone, in any
order, on any machine with the same numpy version.

Workloads (sizes follow the layer the ds4 pages describe: routed experts
quantized, shared expert and router left in high precision -- ds4 digest,
"Model weights" section; prefill in 2048/8192-token chunks -- Korean user
blog, server log excerpts):

  tiny              H=256  I=128  E=8   k=2  no shared expert, 4 tokens
  decode_b1         H=4096 I=2048 E=256 k=8  bf16 shared expert I_s=2048,
                    1000 independent single-token steps
  decode_b16_hot    same layer, 16 tokens per step, 4 hot experts that take
                    about 40% of the assignments through a logit bias
  prefill_2048      same layer, 2048 tokens, router std 1/64 (logits ~N(0,1))
  k4_h7168          H=7168 I=2048 E=256 k=8, 4-bit K-quant experts,
                    8192-token prefill and 1000 single-token decode steps
  *_q8              decode_b1, prefill_2048 and the 4-bit decode with the
                    shared expert in the 8-bit Q8 format (upppp.jp article,
                    "asymmetric 2-bit quantization": shared experts at Q8_0;
                    osrepos summary, the "Q8Shared" model file name)
"""
from __future__ import annotations

import dataclasses

import numpy as np

# Stream tags: one generator per (seed, tag, index).
TAG_ROUTER = 1
TAG_UP = 2
TAG_GATE = 3
TAG_DOWN = 4
TAG_SHARED_UP = 5
TAG_SHARED_GATE = 6
TAG_SHARED_DOWN = 7
TAG_X = 8
TAG_HOT_SET = 9
TAG_BIAS_CALIB = 10
TAG_X_DECODE = 11
TAG_X_DRAFT = 12

WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    shared_inter: int
    fmt_up: str
    fmt_gate: str
    fmt_down: str
    seed: int
    router_std: float = WEIGHT_STD
    tokens: int = 1          # tokens per step (decode) or per chunk (prefill)
    steps: int = 1           # independent steps drawn for the workload
    hot_experts: int = 0     # size of the hot set (skewed routing), 0 = none
    hot_bias: float = 0.0    # logit bias added to the hot set
    x_tag: int = TAG_X
    fmt_shared: str = "bf16"  # shared-expert storage: "bf16" or "q8"

    @property
    def fmts(self):
        return (self.fmt_up, self.fmt_gate, self.fmt_down)


# Logit bias that makes the 4 hot experts take 40% of the top-8 assignments
# in expectation for decode_b16_hot.  Written by
# tests/golden/calibrate_hot_bias.py, which calls only the oracle's router.
HOT_BIAS_DECODE_B16 = 3.7216796875

WORKLOADS = {
    "tiny": Workload("tiny", 256, 128, 8, 2, 0, "cb2", "cb2", "k2", seed=0,
                     tokens=4),
    "decode_b1": Workload("decode_b1", 4096, 2048, 256, 8, 2048,
                          "cb2", "cb2", "k2", seed=1, tokens=1, steps=1000),
    "decode_b16_hot": Workload("decode_b16_hot", 4096, 2048, 256, 8, 2048,
                               "cb2", "cb2", "k2", seed=2, tokens=16,
                               steps=1000, hot_experts=4,
                               hot_bias=HOT_BIAS_DECODE_B16),
    "prefill_2048": Workload("prefill_2048", 4096, 2048, 256, 8, 2048,
                             "cb2", "cb2", "k2", seed=3, tokens=2048,
                             router_std=1.0 / 64.0),
    "k4_h7168_prefill": Workload("k4_h7168_prefill", 7168, 2048, 256, 8, 2048,
                                 "k4", "k4", "k4", seed=4, tokens=8192),
    "k4_h7168_decode": Workload("k4_h7168_decode", 7168, 2048, 256, 8, 2048,
                                "k4", "k4", "k4", seed=4, tokens=1,
                                steps=1000, x_tag=TAG_X_DECODE),
    # decode_b1's layer (same seed, same weights) without its shared expert:
    # the quantized expert bytes alone
    "decode_b1_noshared": Workload("decode_b1_noshared", 4096, 2048, 256, 8, 0,
                                   "cb2", "cb2", "k2", seed=1, tokens=1, steps=1000),
    # draft verification: decode_b1's layer, 1 + 2 drafted tokens per step
    "draft_verify_t3": Workload("draft_verify_t3", 4096, 2048, 256, 8, 2048,
                                "cb2", "cb2", "k2", seed=1, tokens=3, steps=1000,
                                x_tag=TAG_X_DRAFT),
    # the same layers with the shared expert stored in the 8-bit Q8 format
    # (its fp32 draw quantized directly, no bf16 rounding first)
    "decode_b1_q8": Workload("decode_b1_q8", 4096, 2048, 256, 8, 2048,
                             "cb2", "cb2", "k2", seed=1, tokens=1, steps=1000, fmt_shared="q8"),
    "prefill_2048_q8": Workload("prefill_2048_q8", 4096, 2048, 256, 8, 2048,
                                "cb2", "cb2", "k2", seed=3, tokens=2048,
                                router_std=1.0 / 64.0, fmt_shared="q8"),
    "k4_h7168_decode_q8": Workload("k4_h7168_decode_q8", 7168, 2048, 256, 8, 2048,
                                   "k4", "k4", "k4", seed=4, tokens=1,
                                   steps=1000, x_tag=TAG_X_DECODE, fmt_shared="q8"),
}


def rng(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, tag, index])


def normal_f32(seed: int, tag: int, index: int, shape, std: float) -> np.ndarray:
    """fp32 draw of N(0, std^2) from the (seed, tag, index) stream."""
    g = rng(seed, tag, index)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (torch's round-to-nearest-even conversion)
    and return the raw uint16 patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to the fp32 numbers they denote (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# Tensors of a workload


def router_weight(w: Workload) -> np.ndarray:
    """Router weights, fp32 [E, H]."""
    return normal_f32(w.seed, TAG_ROUTER, 0, (w.n_experts, w.hidden), w.router_std)


def expert_weight(w: Workload, which: str, e: int) -> np.ndarray:
    """fp32 weights of routed expert e before quantization.

    which = "up" / "gate": [I, H]; "down": [H, I]  (row-major [out, in])."""
    tag = {"up": TAG_UP, "gate": TAG_GATE, "down": TAG_DOWN}[which]
    shape = (w.inter, w.hidden) if which != "down" else (w.hidden, w.inter)
    return normal_f32(w.seed, tag, e, shape, WEIGHT_STD)


def shared_weight_f32(w: Workload, which: str) -> np.ndarray:
    """fp32 draw of the shared expert: up/gate [I_s, H], down [H, I_s] (the
    "q8" storage quantizes it directly, "bf16" rounds it: shared_weight_bits)."""
    if w.shared_inter == 0:
        raise ValueError(f"{w.name} has no shared expert")
    tag = {"up": TAG_SHARED_UP, "gate": TAG_SHARED_GATE, "down": TAG_SHARED_DOWN}[which]
    shape = (w.shared_inter, w.hidden) if which != "down" else (w.hidden, w.shared_inter)
    return normal_f32(w.seed, tag, 0, shape, WEIGHT_STD)


def shared_weight_bits(w: Workload, which: str) -> np.ndarray:
    """bf16 bit patterns of the shared expert: up/gate [I_s, H], down [H, I_s]."""
    if w.shared_inter == 0:
        raise ValueError(f"{w.name} has no shared expert")
    tag = {"up": TAG_SHARED_UP, "gate": TAG_SHARED_GATE, "down": TAG_SHARED_DOWN}[which]
    shape = (w.shared_inter, w.hidden) if which != "down" else (w.hidden, w.shared_inter)
    return to_bf16_bits(normal_f32(w.seed, tag, 0, shape, WEIGHT_STD))


def activations_bits(w: Workload, n_tokens: int, step: int = 0, scale: float = 1.0) -> np.ndarray:
    """bf16 bit patterns of the layer input x [n_tokens, H], N(0, scale^2)
    (the fp32 draw times `scale`, then rounded to bf16).

    Step s of a multi-step workload is an independent draw (index = step)."""
    return to_bf16_bits(normal_f32(w.seed, w.x_tag, step, (n_tokens, w.hidden), scale))


def activations_f32(w: Workload, n_tokens: int, step: int = 0) -> np.ndarray:
    """fp32 N(0, 1) layer input before bf16 rounding (oracle self-tests)."""
    return normal_f32(w.seed, w.x_tag, step, (n_tokens, w.hidden), 1.0)


def hot_set(w: Workload) -> np.ndarray:
    """Sorted indices of the hot experts (skewed-routing workloads)."""
    if w.hot_experts == 0:
        return np.zeros(0, dtype=np.int64)
    g = rng(w.seed, TAG_HOT_SET, 0)
    return np.sort(g.choice(w.n_experts, size=w.hot_experts, replace=False))


def logit_bias(w: Workload) -> np.ndarray | None:
    """fp32 [E] additive router bias (hot_bias on the hot set), or None."""
    if w.hot_experts == 0:
        return None
    b = np.zeros(w.n_experts, dtype=np.float32)
    b[hot_set(w)] = np.float32(w.hot_bias)
    return b


def random_codebook_free_rows(seed: int, rows: int, k: int, std: float = WEIGHT_STD) -> np.ndarray:
    """Generic fp32 matrix for format tests (tag 0 is never used by a workload)."""
    return normal_f32(seed, 0, rows * 100003 + k, (rows, k), std)
