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
# QMOE_LIB names another build of the same library (the host-sanitizer build
# the CPU tests load); by default the one built in this directory.
LIB_PATH = os.environ.get("QMOE_LIB") or os.path.join(_HERE, "libqmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4

MOE_FMT_BF16 = 0
MOE_FMT_CB2 = 1
MOE_FMT_K2 = 2
MOE_FMT_K4 = 3
MOE_FMT_Q8 = 4
FMT = {"bf16": MOE_FMT_BF16, "cb2": MOE_FMT_CB2, "k2": MOE_FMT_K2, "k4": MOE_FMT_K4, "q8": MOE_FMT_Q8}

EXPORTED = [
    "moe_codebook_generate", "moe_packed_bytes", "moe_quantize_pack",
    "moe_route_workspace_bytes", "moe_route", "moe_group_workspace_bytes",
    "moe_group_tokens", "moe_ffn_workspace_bytes", "moe_expert_ffn_decode",
    "moe_expert_ffn_prefill", "moe_layer_decode_workspace_bytes", "moe_layer_decode",
    "moe_debug_dequant", "moe_profile_next_launch", "moe_last_error", "moe_layer_decode_noalloc",
    "moe_measure_read", "moe_expert_cache_slot_bytes", "moe_expert_cache_create", "moe_expert_cache_destroy",
    "moe_expert_cache_weights", "moe_expert_cache_plan", "moe_expert_cache_fetch", "moe_expert_cache_state",
    "moe_layer_decode_streamed_workspace_bytes", "moe_layer_decode_streamed",
]
MOE_NOALLOC_SCRATCH_BYTES = 8 << 20

MOE_KERNEL = {"route_logits": 0, "route_topk": 1, "decode_upgate": 2, "decode_down": 3,
              "decode_combine": 4, "group": 5, "prefill_upgate": 6, "prefill_down": 7,
              "prefill_combine": 8, "read": 9}


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
        ("fmt_down", ctypes.c_int32), ("fmt_shared", ctypes.c_int32),
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
        "moe_layer_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(MoeWeights), vp, vp, vp, i32, i32, vp, vp, vp,
                                                    vp]),
        "moe_debug_dequant": (ctypes.c_int, [ctypes.c_int, vp, i64, i64, vp, vp, vp]),
        "moe_profile_next_launch": (ctypes.c_int, [ctypes.c_int, vp, vp]),
        "moe_measure_read": (ctypes.c_int, [vp, sz, vp, ctypes.c_int, vp]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_expert_cache_slot_bytes": (sz, [ctypes.POINTER(MoeWeights), i32]),
        "moe_expert_cache_create": (ctypes.c_int, [ctypes.POINTER(MoeWeights), i32, i32, vp, sz,
                                                   ctypes.POINTER(vp)]),
        "moe_expert_cache_destroy": (ctypes.c_int, [vp]),
        "moe_expert_cache_weights": (ctypes.c_int, [vp, ctypes.POINTER(MoeWeights)]),
        "moe_expert_cache_plan": (ctypes.c_int, [vp, vp, i32, vp, vp, vp, ctypes.POINTER(i32)]),
        "moe_expert_cache_fetch": (ctypes.c_int, [vp, vp, vp, i32, vp]),
        "moe_expert_cache_state": (ctypes.c_int, [vp, vp, ctypes.POINTER(i64), ctypes.POINTER(i64)]),
        "moe_layer_decode_streamed_workspace_bytes": (sz, [vp, i32, i32]),
        "moe_layer_decode_streamed": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, sz, vp, vp]),
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


def _dev(t, name, dtype, n=0, optional=False):
    """Device address of tensor `t` as a kernel argument, after the checks
    that keep a kernel from touching the wrong memory: a CUDA tensor of
    `dtype`, contiguous, with at least `n` elements.  None passes only where
    the call takes NULL (`optional`)."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements; the call needs {n}")
    return t.data_ptr()


def _ws(ws):
    """(address, bytes) of a uint8 device workspace; the library checks the size."""
    return _dev(ws, "ws", torch.uint8), ws.numel()


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
    _check(lib.moe_route(_dev(x_bf16, "x_bf16", torch.bfloat16, T * H), _dev(w_router, "w_router", torch.float32, E * H),
                         _dev(logit_bias, "logit_bias", torch.float32, E, optional=True), T, H, E, k,
                         _dev(topk_idx, "topk_idx", torch.int32, T * k), _dev(topk_w, "topk_w", torch.float32, T * k),
                         *_ws(ws), _stream(stream)))


def moe_group_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(lib.moe_group_workspace_bytes(T, k, E))


def moe_group_tokens(topk_idx, T, k, E, expert_offsets, sorted_slots, slot_pos, ws, stream=None):
    _check(lib.moe_group_tokens(_dev(topk_idx, "topk_idx", torch.int32, T * k), T, k, E,
                                _dev(expert_offsets, "expert_offsets", torch.int32, E + 1),
                                _dev(sorted_slots, "sorted_slots", torch.int32, T * k),
                                _dev(slot_pos, "slot_pos", torch.int32, T * k), *_ws(ws), _stream(stream)))


def moe_ffn_workspace_bytes(w: MoeWeights, T: int, k: int, prefill: bool) -> int:
    return int(lib.moe_ffn_workspace_bytes(ctypes.byref(w), T, k, int(bool(prefill))))


def moe_expert_ffn_decode(w: MoeWeights, x_bf16, T, k, topk_idx, topk_w, y, ws, stream=None):
    H = w.hidden
    _check(lib.moe_expert_ffn_decode(ctypes.byref(w), _dev(x_bf16, "x_bf16", torch.bfloat16, T * H), T, k,
                                     _dev(topk_idx, "topk_idx", torch.int32, T * k),
                                     _dev(topk_w, "topk_w", torch.float32, T * k),
                                     _dev(y, "y", torch.float32, T * H), *_ws(ws), _stream(stream)))


def moe_layer_decode_workspace_bytes(w: MoeWeights, T: int, k: int) -> int:
    return int(lib.moe_layer_decode_workspace_bytes(ctypes.byref(w), T, k))


def moe_layer_decode_noalloc(w: MoeWeights, w_router, logit_bias, x_bf16, T, k, topk_idx, topk_w, y, stream=None):
    """moe_layer_decode with the library's own device scratch (allocates nothing)."""
    E, H = w.n_experts, w.hidden
    _check(lib.moe_layer_decode_noalloc(ctypes.byref(w), _dev(w_router, "w_router", torch.float32, E * H),
                                        _dev(logit_bias, "logit_bias", torch.float32, E, optional=True),
                                        _dev(x_bf16, "x_bf16", torch.bfloat16, T * H), T, k,
                                        _dev(topk_idx, "topk_idx", torch.int32, T * k),
                                        _dev(topk_w, "topk_w", torch.float32, T * k),
                                        _dev(y, "y", torch.float32, T * H), _stream(stream)))


def moe_layer_decode(w: MoeWeights, w_router, logit_bias, x_bf16, T, k, topk_idx, topk_w, y, ws, stream=None):
    E, H = w.n_experts, w.hidden
    _check(lib.moe_layer_decode(ctypes.byref(w), _dev(w_router, "w_router", torch.float32, E * H),
                                _dev(logit_bias, "logit_bias", torch.float32, E, optional=True),
                                _dev(x_bf16, "x_bf16", torch.bfloat16, T * H), T, k,
                                _dev(topk_idx, "topk_idx", torch.int32, T * k),
                                _dev(topk_w, "topk_w", torch.float32, T * k),
                                _dev(y, "y", torch.float32, T * H), *_ws(ws), _stream(stream)))


def moe_expert_ffn_prefill(w: MoeWeights, x_bf16, T, k, topk_idx, topk_w, expert_offsets, sorted_slots,
                           slot_pos, y, ws, stream=None):
    E, H = w.n_experts, w.hidden
    _check(lib.moe_expert_ffn_prefill(ctypes.byref(w), _dev(x_bf16, "x_bf16", torch.bfloat16, T * H), T, k,
                                      _dev(topk_idx, "topk_idx", torch.int32, T * k),
                                      _dev(topk_w, "topk_w", torch.float32, T * k),
                                      _dev(expert_offsets, "expert_offsets", torch.int32, E + 1),
                                      _dev(sorted_slots, "sorted_slots", torch.int32, T * k),
                                      _dev(slot_pos, "slot_pos", torch.int32, T * k),
                                      _dev(y, "y", torch.float32, T * H), *_ws(ws), _stream(stream)))


def moe_debug_dequant(fmt, packed, rows, k, codebook, out, stream=None):
    f = FMT.get(fmt, fmt)
    kp = -(-k // 256) * 256
    _check(lib.moe_debug_dequant(f, _dev(packed, "packed", torch.uint8, moe_packed_bytes(f, rows, k)), rows, k,
                                 _dev(codebook, "codebook", torch.int8, 256 * 8, optional=True),
                                 _dev(out, "out", torch.float32, rows * kp), _stream(stream)))


def moe_profile_next_launch(kernel, start_event, stop_event):
    """Record torch.cuda.Event (or raw hipEvent_t) start/stop around the next
    launch of `kernel` (name or id) by this thread."""
    kid = MOE_KERNEL.get(kernel, kernel)
    ev = lambda e: None if e is None else (e.cuda_event if hasattr(e, "cuda_event") else e)
    _check(lib.moe_profile_next_launch(kid, ev(start_event), ev(stop_event)))


def moe_measure_read(src, out, blocks=0, stream=None):
    """Streaming read of the whole uint8 device tensor `src`; XOR of its words into out (int32 [1])."""
    _check(lib.moe_measure_read(_dev(src, "src", torch.uint8), src.numel(), _dev(out, "out", torch.int32, 1),
                                blocks, _stream(stream)))


def moe_last_error() -> str:
    return lib.moe_last_error().decode()


# ---------------------------------------------------------------------------
# Convenience: a layer's weights resident in device memory.


class DeviceLayer:
    """Device copies of one layer's packed weights plus the MoeWeights view.

    up / gate / down: uint8 device tensors holding E packed matrices back to
    back; shared_*: packed matrices in format `shared_fmt` ("bf16" or "q8")
    or None; codebook: int8 device tensor [256*8] or None; router: fp32
    device tensor [E, H]."""

    def __init__(self, n_experts, hidden, inter, shared_inter, fmts, up, gate, down, codebook=None,
                 shared_up=None, shared_gate=None, shared_down=None, router=None, bias=None,
                 shared_fmt="bf16"):
        self.tensors = dict(up=up, gate=gate, down=down, codebook=codebook, shared_up=shared_up,
                            shared_gate=shared_gate, shared_down=shared_down, router=router, bias=bias)
        self.router = router
        self.bias = bias
        self.n_experts, self.hidden, self.inter, self.shared_inter = n_experts, hidden, inter, shared_inter
        E, H, I, Is = n_experts, hidden, inter, shared_inter
        nb_up, nb_dn = moe_packed_bytes(fmts[0], I, H), moe_packed_bytes(fmts[2], H, I)
        u8 = torch.uint8
        shared = Is > 0
        sf = FMT[shared_fmt]
        self.w = MoeWeights(E, H, I, Is, FMT[fmts[0]], FMT[fmts[1]], FMT[fmts[2]], sf,
                            _dev(up, "up", u8, E * nb_up), _dev(gate, "gate", u8, E * nb_up),
                            _dev(down, "down", u8, E * nb_dn),
                            _dev(codebook, "codebook", torch.int8, 256 * 8, optional=True),
                            _dev(shared_up, "shared_up", u8, moe_packed_bytes(sf, Is, H) if shared else 0,
                                 optional=not shared),
                            _dev(shared_gate, "shared_gate", u8, moe_packed_bytes(sf, Is, H) if shared else 0,
                                 optional=not shared),
                            _dev(shared_down, "shared_down", u8, moe_packed_bytes(sf, H, Is) if shared else 0,
                                 optional=not shared))
        _dev(router, "router", torch.float32, E * H, optional=True)
        _dev(bias, "bias", torch.float32, E, optional=True)


# ---------------------------------------------------------------------------
# Expert streaming: an HBM cache of n_slots experts over a layer whose routed
# experts stay in host memory.


def _host(a, name, nbytes):
    """Address of a host buffer (numpy array or CPU tensor, page-locked for
    asynchronous copies) of at least `nbytes` bytes."""
    if isinstance(a, torch.Tensor):
        if a.is_cuda or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous host tensor")
        if a.numel() * a.element_size() < nbytes:
            raise ValueError(f"{name} holds fewer than {nbytes} bytes")
        return a.data_ptr()
    a = np.asarray(a)
    if not a.flags.c_contiguous or a.nbytes < nbytes:
        raise ValueError(f"{name} must be a contiguous host array of at least {nbytes} bytes")
    return a.ctypes.data


class ExpertCache:
    """moe_expert_cache over a layer whose up/gate/down are host buffers
    (`host_up`, `host_gate`, `host_down`: E packed experts each) and whose
    shared expert and codebook come from the device layer `shared_from`
    (a DeviceLayer, or None).  `slot_mem`: uint8 device tensor of at least
    moe_expert_cache_slot_bytes bytes (allocated here when None)."""

    def __init__(self, n_experts, hidden, inter, fmts, host_up, host_gate, host_down, n_slots, keep=0,
                 shared_from=None, slot_mem=None):
        E, H, I = n_experts, hidden, inter
        nb_up, nb_dn = moe_packed_bytes(fmts[0], I, H), moe_packed_bytes(fmts[2], H, I)
        self._keep_alive = [host_up, host_gate, host_down, shared_from]
        sw = shared_from.w if shared_from is not None else None
        self.host_w = MoeWeights(E, H, I, sw.shared_inter if sw else 0, FMT[fmts[0]], FMT[fmts[1]], FMT[fmts[2]],
                                 sw.fmt_shared if sw else 0,
                                 _host(host_up, "host_up", E * nb_up), _host(host_gate, "host_gate", E * nb_up),
                                 _host(host_down, "host_down", E * nb_dn),
                                 sw.codebook if sw else None, sw.shared_up if sw else None,
                                 sw.shared_gate if sw else None, sw.shared_down if sw else None)
        need = int(lib.moe_expert_cache_slot_bytes(ctypes.byref(self.host_w), n_slots))
        if need == 0:
            raise QmoeError(MOE_ERR_INVALID_ARG, "bad layer or n_slots")
        if slot_mem is None:
            slot_mem = torch.empty(need, dtype=torch.uint8, device="cuda")
        self.slot_mem = slot_mem
        self.ptr = ctypes.c_void_p()
        _check(lib.moe_expert_cache_create(ctypes.byref(self.host_w), n_slots, keep,
                                           _dev(slot_mem, "slot_mem", torch.uint8, need), slot_mem.numel(),
                                           ctypes.byref(self.ptr)))
        self.n_slots, self.n_experts, self.hidden = n_slots, E, H
        self.w = MoeWeights()
        _check(lib.moe_expert_cache_weights(self.ptr, ctypes.byref(self.w)))

    def plan(self, ids):
        ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
        slots = np.empty(ids.size, np.int32)
        me = np.empty(max(ids.size, 1), np.int32)
        ms = np.empty(max(ids.size, 1), np.int32)
        nm = ctypes.c_int32(0)
        _check(lib.moe_expert_cache_plan(self.ptr, ids.ctypes.data, ids.size, slots.ctypes.data, me.ctypes.data,
                                         ms.ctypes.data, ctypes.byref(nm)))
        return slots, me[:nm.value].copy(), ms[:nm.value].copy()

    def fetch(self, miss_experts, miss_slots, stream=None):
        me = np.ascontiguousarray(miss_experts, dtype=np.int32)
        ms = np.ascontiguousarray(miss_slots, dtype=np.int32)
        _check(lib.moe_expert_cache_fetch(self.ptr, me.ctypes.data, ms.ctypes.data, me.size, _stream(stream)))

    def state(self):
        eos = np.empty(self.n_slots, np.int32)
        h, m = ctypes.c_int64(0), ctypes.c_int64(0)
        _check(lib.moe_expert_cache_state(self.ptr, eos.ctypes.data, ctypes.byref(h), ctypes.byref(m)))
        return eos, h.value, m.value

    def decode_workspace_bytes(self, T, k):
        return int(lib.moe_layer_decode_streamed_workspace_bytes(self.ptr, T, k))

    def decode(self, w_router, logit_bias, x_bf16, T, k, topk_idx, topk_w, y, ws, stream=None, copy_stream=None):
        H = self.hidden
        _check(lib.moe_layer_decode_streamed(
            self.ptr, _dev(w_router, "w_router", torch.float32, self.n_experts * H),
            _dev(logit_bias, "logit_bias", torch.float32, self.n_experts, optional=True),
            _dev(x_bf16, "x_bf16", torch.bfloat16, T * H), T, k,
            _dev(topk_idx, "topk_idx", torch.int32, T * k), _dev(topk_w, "topk_w", torch.float32, T * k),
            _dev(y, "y", torch.float32, T * H), *_ws(ws), _stream(stream),
            None if copy_stream is None else _stream(copy_stream)))

    def close(self):
        if self.ptr:
            lib.moe_expert_cache_destroy(self.ptr)
            self.ptr = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
