"""Python binding of libqmoe (include/qmoe.h): the same calls under the same
names, with argument marshalling only -- torch tensors become device
pointers, the current torch stream becomes the hipStream_t, a nonzero status
becomes a QmoeError carrying moe_last_error().  Every computation happens in
the library's kernels or its host quantizer.

Import torch before this module (the library then shares torch's HIP
runtime); a missing libqmoe.so raises at import time.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4

MOE_FMT_BF16 = 0
MOE_FMT_CB2 = 1
MOE_FMT_K2 = 2
MOE_FMT_K4 = 3
FMT = {"bf16": MOE_FMT_BF16, "cb2": MOE_FMT_CB2, "k2": MOE_FMT_K2, "k4": MOE_FMT_K4}

EXPORTED = [
    "moe_codebook_generate", "moe_packed_bytes", "moe_quantize_pack",
    "moe_route_workspace_bytes", "moe_route", "moe_group_workspace_bytes",
    "moe_group_tokens", "moe_ffn_workspace_bytes", "moe_expert_ffn_decode",
    "moe_expert_ffn_prefill", "moe_layer_decode_workspace_bytes", "moe_layer_decode",
    "moe_debug_dequant", "moe_profile_next_launch", "moe_last_error",
]

MOE_KERNEL = {"route_logits": 0, "route_topk": 1, "decode_upgate": 2, "decode_down": 3,
              "decode_combine": 4, "group": 5, "prefill_upgate": 6, "prefill_down": 7,
              "prefill_combine": 8}


class QmoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libqmoe error {code}: {msg}")
        self.code = code


class MoeWeights(ctypes.Structure):
    """Mirror of struct moe_weights."""
    _fields_ = [
        ("n_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
        ("fmt_up", ctypes.c_int32), ("fmt_gate", ctypes.c_int32),
        ("fmt_down", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("up", ctypes.c_void_p), ("gate", ctypes.c_void_p), ("down", ctypes.c_void_p),
        ("codebook", ctypes.c_void_p),
        ("shared_up", ctypes.c_void_p), ("shared_gate", ctypes.c_void_p),
        ("shared_down", ctypes.c_void_p),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m bit_quantized_moe_02_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "moe_codebook_generate": (ctypes.c_int, [ctypes.c_uint64, vp]),
        "moe_packed_bytes": (sz, [ctypes.c_int, i64, i64]),
        "moe_quantize_pack": (ctypes.c_int, [ctypes.c_int, vp, i64, i64, vp, vp, sz, ctypes.c_int]),
        "moe_route_workspace_bytes": (sz, [i32, i32]),
        "moe_route": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, sz, vp]),
        "moe_group_workspace_bytes": (sz, [i32, i32, i32]),
        "moe_group_tokens": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]),
        "moe_ffn_workspace_bytes": (sz, [ctypes.POINTER(MoeWeights), i32, i32, ctypes.c_int]),
        "moe_expert_ffn_decode": (ctypes.c_int, [ctypes.POINTER(MoeWeights), vp, i32, i32, vp, vp, vp,
                                                 vp, sz, vp]),
        "moe_expert_ffn_prefill": (ctypes.c_int, [ctypes.POINTER(MoeWeights), vp, i32, i32, vp, vp, vp,
                                                  vp, vp, vp, vp, sz, vp]),
        "moe_layer_decode_workspace_bytes": (sz, [ctypes.POINTER(MoeWeights), i32, i32]),
        "moe_layer_decode": (ctypes.c_int, [ctypes.POINTER(MoeWeights), vp, vp, vp, i32, i32, vp, vp, vp,
                                            vp, sz, vp]),
        "moe_debug_dequant": (ctypes.c_int, [ctypes.c_int, vp, i64, i64, vp, vp, vp]),
        "moe_profile_next_launch": (ctypes.c_int, [ctypes.c_int, vp, vp]),
        "moe_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(rc):
    if rc != MOE_OK:
        raise QmoeError(rc, lib.moe_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------------------
# host-only calls


def moe_codebook_generate(seed: int = 0) -> np.ndarray:
    out = np.empty((256, 8), dtype=np.int8)
    _check(lib.moe_codebook_generate(seed, out.ctypes.data))
    return out


def moe_packed_bytes(fmt, rows: int, k: int) -> int:
    return int(lib.moe_packed_bytes(FMT.get(fmt, fmt), rows, k))


def moe_quantize_pack(fmt, w: np.ndarray, codebook: np.ndarray | None = None, n_threads: int = 0,
                      out: np.ndarray | None = None) -> np.ndarray:
    """fp32 host matrix [rows, k] -> packed uint8 bytes (host)."""
    f = FMT.get(fmt, fmt)
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, k = w.shape
    nbytes = moe_packed_bytes(f, rows, k)
    if out is None:
        out = np.empty(max(nbytes, 1), dtype=np.uint8)
    cb = None if codebook is None else np.ascontiguousarray(codebook, dtype=np.int8)
    _check(lib.moe_quantize_pack(f, w.ctypes.data, rows, k, None if cb is None else cb.ctypes.data,
                                 out.ctypes.data, out.nbytes, n_threads))
    return out[:nbytes]


# ---------------------------------------------------------------------------
# device calls (torch tensors on the current device)


def moe_route_workspace_bytes(T: int, E: int) -> int:
    return int(lib.moe_route_workspace_bytes(T, E))


def moe_route(x_bf16, w_router, logit_bias, T, H, E, k, topk_idx, topk_w, ws, stream=None):
    _check(lib.moe_route(_ptr(x_bf16), _ptr(w_router), _ptr(logit_bias), T, H, E, k, _ptr(topk_idx),
                         _ptr(topk_w), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_group_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(lib.moe_group_workspace_bytes(T, k, E))


def moe_group_tokens(topk_idx, T, k, E, expert_offsets, sorted_slots, slot_pos, ws, stream=None):
    _check(lib.moe_group_tokens(_ptr(topk_idx), T, k, E, _ptr(expert_offsets), _ptr(sorted_slots),
                                _ptr(slot_pos), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)))


def moe_ffn_workspace_bytes(w: MoeWeights, T: int, k: int, prefill: bool) -> int:
    return int(lib.moe_ffn_workspace_bytes(ctypes.byref(w), T, k, int(bool(prefill))))


def moe_expert_ffn_decode(w: MoeWeights, x_bf16, T, k, topk_idx, topk_w, y, ws, stream=None):
    _check(lib.moe_expert_ffn_decode(ctypes.byref(w), _ptr(x_bf16), T, k, _ptr(topk_idx), _ptr(topk_w),
                                     _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_layer_decode_workspace_bytes(w: MoeWeights, T: int, k: int) -> int:
    return int(lib.moe_layer_decode_workspace_bytes(ctypes.byref(w), T, k))


def moe_layer_decode(w: MoeWeights, w_router, logit_bias, x_bf16, T, k, topk_idx, topk_w, y, ws, stream=None):
    _check(lib.moe_layer_decode(ctypes.byref(w), _ptr(w_router), _ptr(logit_bias), _ptr(x_bf16), T, k,
                                _ptr(topk_idx), _ptr(topk_w), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)))


def moe_expert_ffn_prefill(w: MoeWeights, x_bf16, T, k, topk_idx, topk_w, expert_offsets, sorted_slots,
                           slot_pos, y, ws, stream=None):
    _check(lib.moe_expert_ffn_prefill(ctypes.byref(w), _ptr(x_bf16), T, k, _ptr(topk_idx), _ptr(topk_w),
                                      _ptr(expert_offsets), _ptr(sorted_slots), _ptr(slot_pos), _ptr(y),
                                      _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_debug_dequant(fmt, packed, rows, k, codebook, out, stream=None):
    _check(lib.moe_debug_dequant(FMT.get(fmt, fmt), _ptr(packed), rows, k, _ptr(codebook), _ptr(out),
                                 _stream(stream)))


def moe_profile_next_launch(kernel, start_event, stop_event):
    """Record torch.cuda.Event (or raw hipEvent_t) start/stop around the next
    launch of `kernel` (name or id) by this thread."""
    kid = MOE_KERNEL.get(kernel, kernel)
    ev = lambda e: None if e is None else (e.cuda_event if hasattr(e, "cuda_event") else e)
    _check(lib.moe_profile_next_launch(kid, ev(start_event), ev(stop_event)))


def moe_last_error() -> str:
    return lib.moe_last_error().decode()


# ---------------------------------------------------------------------------
# Convenience: a layer's weights resident in device memory.


class DeviceLayer:
    """Device copies of one layer's packed weights plus the MoeWeights view.

    up / gate / down: uint8 device tensors holding E packed matrices back to
    back; shared_*: BF16-format packed matrices or None; codebook: int8 device
    tensor [256*8] or None; router: fp32 device tensor [E, H]."""

    def __init__(self, n_experts, hidden, inter, shared_inter, fmts, up, gate, down, codebook=None,
                 shared_up=None, shared_gate=None, shared_down=None, router=None, bias=None):
        self.tensors = dict(up=up, gate=gate, down=down, codebook=codebook, shared_up=shared_up,
                            shared_gate=shared_gate, shared_down=shared_down, router=router, bias=bias)
        self.router = router
        self.bias = bias
        self.n_experts, self.hidden, self.inter, self.shared_inter = n_experts, hidden, inter, shared_inter
        self.w = MoeWeights(n_experts, hidden, inter, shared_inter, FMT[fmts[0]], FMT[fmts[1]], FMT[fmts[2]],
                            0, _ptr(up), _ptr(gate), _ptr(down), _ptr(codebook), _ptr(shared_up),
                            _ptr(shared_gate), _ptr(shared_down))
