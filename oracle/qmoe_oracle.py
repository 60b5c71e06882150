"""Plain, slow fp64 implementation of the quantized routed-MoE layer.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): used by tests/, the smoke
check and bench.py's cpu_baseline leg, never by the product path.

The layer (ds4 digest, "Model weights" section; upppp.jp article,
"asymmetric 2-bit quantization" section): only the routed experts are
quantized -- up/gate in a 2-bit codebook format, down in a 2-bit K-quant
format (a 4-bit K-quant variant exists for the larger model: osrepos summary,
"Q4KExperts" model file name) -- while the shared expert and the router stay
in high precision.  Sparse top-k activation of the experts is what makes the
model fast (ds4 digest, overview).

Functions, in the order a layer uses them:

  codebook(seed)                 SplitMix64 table of 256 signed 8-vectors
  cb2_quantize / cb2_dequantize  2-bit codebook format (CB2)
  kq_quantize / kq_dequantize    K-quant super-block formats (K2, K4)
  q8_quantize / q8_dequantize    8-bit blocks of 32 (Q8, shared expert)
  pack_* / unpack_*              byte layout of the 16x256 weight tiles
  route                          softmax over experts, top-k, renormalize
  group                          stable grouping of (token, slot) by expert
  expert_ffn                     SiLU(x Wg^T) * (x Wu^T) then Wd
  moe_layer                      sum_j w_tj FFN_{e_tj}(x_t) + shared(x_t)

Everything is fp64 except where a format fixes a precision (fp16 scales,
fp32 dequantized weights).  Readings of points the pages leave open are
listed where they are used.
"""
from __future__ import annotations

import ctypes
import math
import os
from fractions import Fraction

import numpy as np

__all__ = [
    "splitmix64", "codebook", "f16", "bf16_round", "f32_round",
    "cb2_quantize", "cb2_dequantize", "kq_params", "kq_quantize", "kq_dequantize",
    "q8_quantize", "q8_dequantize",
    "quantize_matrix", "dequantize_matrix", "pack_matrix", "unpack_matrix",
    "tile_bytes", "packed_bytes", "route", "group", "silu", "expert_ffn",
    "moe_layer", "dense_ffn", "cb2_search_numpy", "cb2_search",
]

MASK64 = (1 << 64) - 1

# ---------------------------------------------------------------------------
# Codebook: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
# number generators", OOPSLA 2014), 2048 draws, top two bits of each draw
# select a value in {-3, -1, +1, +3} (quarter units).  Draw i fills entry
# i // 8, dimension i % 8.


def splitmix64(seed: int, n: int) -> list[int]:
    """First n outputs of SplitMix64 started from `seed` (published algorithm:
    add the golden-ratio increment, then two xor-shift-multiply rounds and a
    final xor-shift)."""
    state = seed & MASK64
    out = []
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        out.append(z ^ (z >> 31))
    return out


_TOP2_VALUE = {0: -3, 1: -1, 2: 1, 3: 3}


def codebook(seed: int = 0) -> np.ndarray:
    """The CB2 table: int8 [256, 8], values in {-3, -1, 1, 3} (units of 1/4)."""
    draws = splitmix64(seed, 256 * 8)
    return np.array([_TOP2_VALUE[d >> 62] for d in draws], dtype=np.int8).reshape(256, 8)


# ---------------------------------------------------------------------------
# Rounding helpers


def f16(x) -> np.ndarray:
    """Round fp64 values to the nearest fp16 (ties to even), returned as fp64.
    numpy converts float64 -> float16 from the double's bits in one rounding."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def f32_round(x) -> np.ndarray:
    """Round exact fp64 values to fp32 (ties to even), returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """Round fp64 values to bf16 (8 significant bits, ties to even) in one
    rounding, returned as fp64.  Normal range only (|x| >= 2^-126 or 0)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                     # x = m * 2^e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0)                 # 8 significant bits, half to even
    return np.ldexp(r, e - 8)


# ---------------------------------------------------------------------------
# CB2: groups of 8 consecutive weights along K each hold an 8-bit index into
# the 256-entry codebook and 8 flip bits; one fp16 scale per 32 weights.
# Decoded weight j of a group: s * T[idx][j] / 4, negated when flip bit j is
# set.  Readings: the table entries are signed and a set bit flips the sign;
# s = fp16(max|w| / 0.75) over the 32-block (no refit); the index minimizes
# sum_j (|w_j| - s*|T[e][j]|/4)^2 summed in fp64 with j ascending, lowest
# index on ties; flip bit j = (w_j < 0) xor (T[idx][j] < 0), -0.0 counts as
# non-negative.


def cb2_search_numpy(absw: np.ndarray, s: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Brute-force index search.  absw fp64 [G, 8], s fp64 [G] -> uint8 [G]."""
    mag = np.abs(table.astype(np.float64)) / 4.0          # [256, 8], exact
    out = np.empty(absw.shape[0], dtype=np.uint8)
    step = 4096
    for g0 in range(0, absw.shape[0], step):
        a = absw[g0:g0 + step]
        sc = s[g0:g0 + step, None]
        err = np.zeros((a.shape[0], 256))
        for j in range(8):                                 # j ascending
            d = a[:, j:j + 1] - sc * mag[None, :, j]
            err = err + d * d
        out[g0:g0 + step] = np.argmin(err, axis=1)         # first minimum
    return out


_C_SEARCH = None


def _load_c_search():
    global _C_SEARCH
    if _C_SEARCH is None:
        path = os.path.join(os.path.dirname(__file__), "_cb2_search.so")
        if os.path.exists(path):
            lib = ctypes.CDLL(path)
            lib.cb2_search.restype = None
            lib.cb2_search.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
            _C_SEARCH = lib
        else:
            _C_SEARCH = False
    return _C_SEARCH or None


def cb2_search(absw: np.ndarray, s: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Same search as cb2_search_numpy; uses the plain C loop in
    cb2_search.c when it is built (identical arithmetic, just faster)."""
    lib = _load_c_search()
    if lib is None:
        return cb2_search_numpy(absw, s, table)
    absw = np.ascontiguousarray(absw, dtype=np.float64)
    s = np.ascontiguousarray(s, dtype=np.float64)
    mag = np.ascontiguousarray(np.abs(table.astype(np.float64)) / 4.0)
    out = np.empty(absw.shape[0], dtype=np.uint8)
    lib.cb2_search(absw.shape[0], absw.ctypes.data, s.ctypes.data, mag.ctypes.data,
                   out.ctypes.data)
    return out


def cb2_quantize(w: np.ndarray, table: np.ndarray) -> dict:
    """Quantize fp32 rows [R, K] (K % 32 == 0) to CB2 fields:
    idx uint8 [R, K/8], flip uint8 [R, K/8] (bit j = weight j of the group),
    scale fp64 [R, K/32] holding fp16 values."""
    w = np.asarray(w, dtype=np.float32)
    R, K = w.shape
    assert K % 32 == 0
    w64 = w.astype(np.float64)
    a = np.abs(w64).reshape(R, K // 32, 32).max(axis=2)
    s = f16(a / 0.75)
    s = np.where(s == 0, 0.0, s)                            # canonical +0
    groups = w64.reshape(R * K // 8, 8)
    s_g = np.repeat(s.reshape(-1), 4)
    idx = cb2_search(np.abs(groups), s_g, table)
    neg_w = groups < 0
    neg_t = table[idx] < 0
    flip_bits = (neg_w != neg_t).astype(np.uint8)
    flip = (flip_bits << np.arange(8, dtype=np.uint8)).sum(axis=1).astype(np.uint8)
    return {"idx": idx.reshape(R, K // 8), "flip": flip.reshape(R, K // 8), "scale": s}


def cb2_dequantize(f: dict, table: np.ndarray) -> np.ndarray:
    """CB2 fields -> fp64 [R, K].  Every value is exact in fp32."""
    idx, flip, s = f["idx"], f["flip"], f["scale"]
    R, G = idx.shape
    t = table[idx.reshape(-1)].astype(np.float64) / 4.0            # [R*G, 8]
    bits = (flip.reshape(-1, 1) >> np.arange(8, dtype=np.uint8)) & 1
    sign = np.where(bits == 1, -1.0, 1.0)
    s_g = np.repeat(s.reshape(-1), 4)[:, None]
    return (s_g * t * sign).reshape(R, G * 8)


# ---------------------------------------------------------------------------
# K-quant super-blocks of 256 weights along K.
#   K2: 16 sub-blocks of 16, q in 0..3, 4-bit sc and m.
#   K4: 8 sub-blocks of 32, q in 0..15, 6-bit sc and m.
# Weight = d*sc*q - dmin*m with fp16 d, dmin per super-block.
# Readings (the quantizer is not specified beyond the format): per sub-block
# lo = min(0, min w), hi = max w, a = (hi - lo)/Q, b = 0 - lo;
# d = fp16(max a / S), dmin = fp16(max b / S);
# sc = min(S, floor(a/d + 1/2)) (0 if d = 0), m likewise from b and dmin;
# q = clamp(floor((w + dmin*m)/(d*sc) + 1/2), 0, Q) (0 if d*sc = 0).


def kq_params(fmt: str):
    """(sub-block length B, max code Q, max scale S) of a K-quant format."""
    return {"k2": (16, 3, 15), "k4": (32, 15, 63)}[fmt]


def kq_quantize(w: np.ndarray, fmt: str) -> dict:
    """Quantize fp32 rows [R, K] (K % 256 == 0) to K-quant fields:
    q uint8 [R, K], sc/m uint8 [R, K/B], d/dmin fp64 [R, K/256] (fp16 values)."""
    B, Q, S = kq_params(fmt)
    w = np.asarray(w, dtype=np.float32)
    R, K = w.shape
    assert K % 256 == 0
    nsb = 256 // B
    x = w.astype(np.float64).reshape(R, K // 256, nsb, B)
    lo = np.minimum(0.0, x.min(axis=3))
    hi = x.max(axis=3)
    a = (hi - lo) / Q
    b = 0.0 - lo
    d = f16(a.max(axis=2) / S)
    dmin = f16(b.max(axis=2) / S)
    d = np.where(d == 0, 0.0, d)
    dmin = np.where(dmin == 0, 0.0, dmin)
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d[..., None] == 0, 0.0,
                      np.minimum(S, np.floor(a / d[..., None] + 0.5)))
        m = np.where(dmin[..., None] == 0, 0.0,
                     np.minimum(S, np.floor(b / dmin[..., None] + 0.5)))
        step = d[..., None] * sc                       # exact in fp64
        off = dmin[..., None] * m                      # exact in fp64
        q = np.where(step[..., None] == 0, 0.0,
                     np.clip(np.floor((x + off[..., None]) / step[..., None] + 0.5), 0, Q))
    return {
        "q": q.reshape(R, K).astype(np.uint8),
        "sc": sc.reshape(R, K // B).astype(np.uint8),
        "m": m.reshape(R, K // B).astype(np.uint8),
        "d": d, "dmin": dmin,
    }


def _exact_f32(dscq: np.ndarray, dm: np.ndarray, d: np.ndarray, dmin: np.ndarray) -> np.ndarray:
    """RNE_fp32(dscq - dm) where dscq = d*sc*q and dm = dmin*m are exact
    fp64 products.  The fp64 difference is exact unless d and dmin are more
    than 2^25 apart; those elements are redone with exact rationals."""
    out = f32_round(dscq - dm)
    with np.errstate(divide="ignore"):
        gap = np.abs(np.log2(np.where(d > 0, d, 1.0)) - np.log2(np.where(dmin > 0, dmin, 1.0)))
    far = (gap > 25) & (d > 0) & (dmin > 0)
    for i in zip(*np.nonzero(far)):
        exact = Fraction(float(dscq[i])) - Fraction(float(dm[i]))
        out[i] = float(np.float32(_round_fraction_to_f32(exact)))
    return out


def _round_fraction_to_f32(v: Fraction) -> float:
    """Nearest fp32 to an exact rational, ties to even (normal range)."""
    if v == 0:
        return 0.0
    sign = -1 if v < 0 else 1
    v = abs(v)
    e = math.floor(math.log2(v))
    while Fraction(2) ** e > v:
        e -= 1
    while Fraction(2) ** (e + 1) <= v:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    n = v / ulp
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * ulp)


def kq_dequantize(f: dict, fmt: str) -> np.ndarray:
    """K-quant fields -> fp64 [R, K] holding RNE_fp32(d*sc*q - dmin*m)."""
    B, Q, S = kq_params(fmt)
    q = f["q"].astype(np.float64)
    R, K = q.shape
    sc = np.repeat(f["sc"].astype(np.float64), B, axis=1)
    m = np.repeat(f["m"].astype(np.float64), B, axis=1)
    d = np.repeat(f["d"], 256, axis=1)
    dmin = np.repeat(f["dmin"], 256, axis=1)
    return _exact_f32(d * sc * q, dmin * m, d, dmin)


# ---------------------------------------------------------------------------
# Q8: the 8-bit format the pages keep for shared-expert tensors (upppp.jp
# article, "asymmetric 2-bit quantization": shared experts, projections and
# the output layer stay at Q8_0 or F16; osrepos summary, the "Q8Shared" model
# file name).  Blocks of 32 consecutive weights along K, one signed code q
# per weight and one fp16 scale d per block: weight = d * q.
# Readings (the pages name the format only): d = fp16(max|w| / 127) (fp64
# quotient, one rounding to fp16); q = sign(w) * min(127, floor(|w|/d + 1/2))
# with the quotient in fp64, i.e. the nearest code, ties away from zero,
# clamped to the symmetric range -127..127 (q = 0 when d = 0).


def q8_quantize(w: np.ndarray) -> dict:
    """Quantize fp32 rows [R, K] (K % 32 == 0) to Q8 fields:
    q int8 [R, K], d fp64 [R, K/32] (fp16 values)."""
    w = np.asarray(w, dtype=np.float32)
    R, K = w.shape
    assert K % 32 == 0
    x = w.astype(np.float64).reshape(R, K // 32, 32)
    d = f16(np.abs(x).max(axis=2) / 127.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        mag = np.where(d[..., None] == 0, 0.0,
                       np.minimum(127.0, np.floor(np.abs(x) / d[..., None] + 0.5)))
    q = np.where(x < 0, -mag, mag)
    return {"q": q.reshape(R, K).astype(np.int8), "d": d}


def q8_dequantize(f: dict) -> np.ndarray:
    """Q8 fields -> fp64 [R, K] holding d*q (exact: an 11-bit significand
    times a 7-bit integer, so also exact in fp32)."""
    q = f["q"].astype(np.float64)
    return q * np.repeat(f["d"], 32, axis=1)


# ---------------------------------------------------------------------------
# Whole matrices (rows = output features, K = reduction dimension).


def _pad_k(w: np.ndarray) -> np.ndarray:
    R, K = w.shape
    Kp = -(-K // 256) * 256
    if Kp == K:
        return np.asarray(w, dtype=np.float32)
    out = np.zeros((R, Kp), dtype=np.float32)
    out[:, :K] = w
    return out


def quantize_matrix(fmt: str, w: np.ndarray, table: np.ndarray | None = None) -> dict:
    """fp32 [R, K] -> fields of `fmt` (K zero-padded to a multiple of 256).
    fmt "bf16" keeps the values (they must already be bf16 numbers)."""
    w = _pad_k(w)
    if fmt == "cb2":
        f = cb2_quantize(w, table)
    elif fmt in ("k2", "k4"):
        f = kq_quantize(w, fmt)
    elif fmt == "q8":
        f = q8_quantize(w)
    elif fmt == "bf16":
        v = w.astype(np.float64)
        assert np.array_equal(bf16_round(v), v), "bf16 format takes bf16 values"
        f = {"w": v}
    else:
        raise ValueError(fmt)
    f["fmt"] = fmt
    return f


def dequantize_matrix(f: dict, table: np.ndarray | None = None, k: int | None = None) -> np.ndarray:
    """Fields -> fp64 weights [R, K] (K cut back to `k` when given)."""
    fmt = f["fmt"]
    if fmt == "cb2":
        w = cb2_dequantize(f, table)
    elif fmt in ("k2", "k4"):
        w = kq_dequantize(f, fmt)
    elif fmt == "q8":
        w = q8_dequantize(f)
    else:
        w = f["w"]
    return w if k is None else w[:, :k]


# ---------------------------------------------------------------------------
# Byte layout.  A matrix [R, K] (R % 16 == 0, K % 256 == 0) is stored as
# R/16 x K/256 tiles of 16 rows x 256 columns, row-tile major.  Inside a
# tile, row n in 0..15 and column kk in 0..255 split as kb = kk // 32,
# qq = (kk % 32) // 8, j = kk % 8, and lane c = 16*qq + n owns the 8 weights
# (n, kb, qq, j=0..7) of every kb.  The tile sizes and field orders are the
# ones include/qmoe.h defines.

TILE_BYTES = {"cb2": 1280, "k2": 1344, "k4": 2304, "bf16": 8192, "q8": 4352}


def tile_bytes(fmt: str) -> int:
    return TILE_BYTES[fmt]


def packed_bytes(fmt: str, rows: int, k: int) -> int:
    kp = -(-k // 256) * 256
    return (rows // 16) * (kp // 256) * TILE_BYTES[fmt]


def _lanes(a: np.ndarray, R: int, K: int) -> np.ndarray:
    """[R, K, ...] per-weight array -> [R/16, K/256, 64 lanes, 8 kb, 8 j, ...]."""
    rest = a.shape[2:]
    a = a.reshape((R // 16, 16, K // 256, 8, 4, 8) + rest)      # rt n kc kb qq j
    a = np.moveaxis(a, (0, 2, 4, 1, 3, 5), (0, 1, 2, 3, 4, 5))  # rt kc qq n kb j
    return a.reshape((R // 16, K // 256, 64, 8, 8) + rest)


def _unlanes(a: np.ndarray, R: int, K: int) -> np.ndarray:
    rest = a.shape[5:]
    a = a.reshape((R // 16, K // 256, 4, 16, 8, 8) + rest)      # rt kc qq n kb j
    a = np.moveaxis(a, (0, 1, 2, 3, 4, 5), (0, 2, 4, 1, 3, 5))  # rt n kc kb qq j
    return a.reshape((R, K) + rest)


def _f16_bits(v: np.ndarray) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def _f16_from_bits(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def pack_matrix(f: dict) -> np.ndarray:
    """Fields -> uint8 [R/16, K/256, tile_bytes]."""
    fmt = f["fmt"]
    if fmt == "cb2":
        R, G = f["idx"].shape
        K = G * 8
        # one 16-bit code per group: index in bits 0-7, flip bits in 8-15
        code = f["idx"].astype(np.uint16) | (f["flip"].astype(np.uint16) << 8)   # [R, K/8]
        per_w = np.repeat(code, 8, axis=1)                                       # [R, K]
        lanes = _lanes(per_w, R, K)[..., 0]                                      # j = 0
        codes = lanes.astype("<u2").view(np.uint8).reshape(R // 16, K // 256, 1024)
        sc = _f16_bits(f["scale"]).reshape(R // 16, 16, K // 256, 8)
        sc = np.moveaxis(sc, 2, 1).astype("<u2").view(np.uint8).reshape(R // 16, K // 256, 256)
        return np.concatenate([codes, sc], axis=2)
    if fmt == "k2":
        q = f["q"].astype(np.uint32)
        R, K = q.shape
        lanes = _lanes(q, R, K)                                  # [.., 64, kb, j]
        kb = np.arange(8)[:, None]
        j = np.arange(8)[None, :]
        shift = 2 * (4 * (kb % 2) + j // 2) + 16 * (j % 2)       # bit of (kb, j)
        dwords = np.zeros(lanes.shape[:3] + (4,), dtype=np.uint32)
        for kbi in range(8):
            for ji in range(8):
                dwords[..., kbi // 2] |= lanes[..., kbi, ji] << np.uint32(shift[kbi, ji])
        qb = dwords.astype("<u4").view(np.uint8).reshape(R // 16, K // 256, 1024)
        scm = (f["sc"].astype(np.uint8) | (f["m"].astype(np.uint8) << 4))      # [R, K/16]
        scm = np.moveaxis(scm.reshape(R // 16, 16, K // 256, 16), 2, 1).reshape(R // 16, K // 256, 256)
        dd = np.stack([_f16_bits(f["d"]), _f16_bits(f["dmin"])], axis=-1)     # [R, K/256, 2]
        dd = np.moveaxis(dd.reshape(R // 16, 16, K // 256, 2), 2, 1).astype("<u2")
        dd = dd.view(np.uint8).reshape(R // 16, K // 256, 64)
        return np.concatenate([qb, scm, dd], axis=2)
    if fmt == "k4":
        q = f["q"].astype(np.uint32)
        R, K = q.shape
        lanes = _lanes(q, R, K)
        j = np.arange(8)
        shift = 4 * (j // 2) + 16 * (j % 2)
        dwords = np.zeros(lanes.shape[:3] + (8,), dtype=np.uint32)   # dword per kb
        for kbi in range(8):
            for ji in range(8):
                dwords[..., kbi] |= lanes[..., kbi, ji] << np.uint32(shift[ji])
        # halves: kb 0-3 for all lanes, then kb 4-7
        halves = np.stack([dwords[..., 0:4], dwords[..., 4:8]], axis=2)     # [.., 2, 64, 4]
        qb = halves.astype("<u4").view(np.uint8).reshape(R // 16, K // 256, 2048)
        vals = np.concatenate([f["sc"].reshape(R, K // 256, 8), f["m"].reshape(R, K // 256, 8)],
                              axis=2).astype(np.uint8)                          # [R, K/256, 16]
        # 16 six-bit values as a little-endian bitstream: bit b of the stream
        # is bit b % 6 of value b // 6 and lands in byte b // 8, bit b % 8.
        bits = np.zeros((R, K // 256, 12), dtype=np.uint8)
        for b in range(96):
            bit = (vals[..., b // 6] >> (b % 6)) & 1
            bits[..., b // 8] |= (bit << (b % 8)).astype(np.uint8)
        scb = np.moveaxis(bits.reshape(R // 16, 16, K // 256, 12), 2, 1).reshape(R // 16, K // 256, 192)
        dd = np.stack([_f16_bits(f["d"]), _f16_bits(f["dmin"])], axis=-1)
        dd = np.moveaxis(dd.reshape(R // 16, 16, K // 256, 2), 2, 1).astype("<u2")
        dd = dd.view(np.uint8).reshape(R // 16, K // 256, 64)
        return np.concatenate([qb, scb, dd], axis=2)
    if fmt == "q8":
        q = f["q"].astype(np.int8)
        R, K = q.shape
        lanes = _lanes(q, R, K)                                      # [.., 64, kb, j]
        # 16-byte piece i of a lane holds k-blocks a and a + 2, a = 4*(i % 2) + i // 2
        pieces = np.stack([np.concatenate([lanes[..., a, :], lanes[..., a + 2, :]], axis=-1)
                           for a in (0, 4, 1, 5)], axis=2)           # [.., piece, 64, 16]
        qb = pieces.view(np.uint8).reshape(R // 16, K // 256, 4096)
        sc = _f16_bits(f["d"]).reshape(R // 16, 16, K // 256, 8)
        sc = np.moveaxis(sc, 2, 1).astype("<u2").view(np.uint8).reshape(R // 16, K // 256, 256)
        return np.concatenate([qb, sc], axis=2)
    if fmt == "bf16":
        w = f["w"]
        R, K = w.shape
        bits = (w.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        lanes = _lanes(bits, R, K)                                   # [.., 64, kb, j]
        lanes = np.moveaxis(lanes, 3, 2)                             # [.., kb, 64, j]
        return lanes.astype("<u2").view(np.uint8).reshape(R // 16, K // 256, 8192)
    raise ValueError(fmt)


def unpack_matrix(fmt: str, packed: np.ndarray, rows: int, k: int) -> dict:
    """uint8 bytes of a packed matrix -> fields (inverse of pack_matrix)."""
    K = -(-k // 256) * 256
    R = rows
    t = np.asarray(packed, dtype=np.uint8).reshape(R // 16, K // 256, TILE_BYTES[fmt])
    if fmt == "cb2":
        codes = t[..., :1024].copy().view("<u2").reshape(R // 16, K // 256, 64, 8)
        per_w = np.repeat(codes[..., None], 8, axis=-1)                  # [.., 64, kb, j]
        code = _unlanes(per_w, R, K)[:, ::8]                             # [R, K/8]
        idx = (code & 0xFF).astype(np.uint8)
        flip = (code >> 8).astype(np.uint8)
        sc = t[..., 1024:].copy().view("<u2").reshape(R // 16, K // 256, 16, 8)
        sc = np.moveaxis(sc, 1, 2).reshape(R, K // 32)
        return {"fmt": fmt, "idx": idx, "flip": flip, "scale": _f16_from_bits(sc)}
    if fmt == "k2":
        dw = t[..., :1024].copy().view("<u4").reshape(R // 16, K // 256, 64, 4)
        q = np.zeros((R // 16, K // 256, 64, 8, 8), dtype=np.uint8)
        for kbi in range(8):
            for ji in range(8):
                shift = 2 * (4 * (kbi % 2) + ji // 2) + 16 * (ji % 2)
                q[..., kbi, ji] = (dw[..., kbi // 2] >> np.uint32(shift)) & 3
        q = _unlanes(q, R, K)
        scm = np.moveaxis(t[..., 1024:1280].reshape(R // 16, K // 256, 16, 16), 1, 2).reshape(R, K // 16)
        dd = t[..., 1280:].copy().view("<u2").reshape(R // 16, K // 256, 16, 2)
        dd = np.moveaxis(dd, 1, 2).reshape(R, K // 256, 2)
        return {"fmt": fmt, "q": q, "sc": scm & 0xF, "m": scm >> 4,
                "d": _f16_from_bits(dd[..., 0]), "dmin": _f16_from_bits(dd[..., 1])}
    if fmt == "k4":
        dw = t[..., :2048].copy().view("<u4").reshape(R // 16, K // 256, 2, 64, 4)
        dw = np.moveaxis(dw, 2, 3).reshape(R // 16, K // 256, 64, 8)     # [.., lane, kb]
        q = np.zeros((R // 16, K // 256, 64, 8, 8), dtype=np.uint8)
        for ji in range(8):
            shift = 4 * (ji // 2) + 16 * (ji % 2)
            q[..., ji] = (dw >> np.uint32(shift)) & 15
        q = _unlanes(q, R, K)
        sb = np.moveaxis(t[..., 2048:2240].reshape(R // 16, K // 256, 16, 12), 1, 2).reshape(R, K // 256, 12)
        vals = np.zeros((R, K // 256, 16), dtype=np.uint8)
        for i in range(16):
            pos = 6 * i
            v = np.zeros((R, K // 256), dtype=np.uint32)
            for b in range(6):
                bit = pos + b
                v |= ((sb[..., bit // 8] >> (bit % 8)) & 1).astype(np.uint32) << b
            vals[..., i] = v
        dd = t[..., 2240:].copy().view("<u2").reshape(R // 16, K // 256, 16, 2)
        dd = np.moveaxis(dd, 1, 2).reshape(R, K // 256, 2)
        return {"fmt": fmt, "q": q, "sc": vals[..., :8].reshape(R, K // 32),
                "m": vals[..., 8:].reshape(R, K // 32),
                "d": _f16_from_bits(dd[..., 0]), "dmin": _f16_from_bits(dd[..., 1])}
    if fmt == "q8":
        pieces = t[..., :4096].copy().view(np.int8).reshape(R // 16, K // 256, 4, 64, 16)
        q = np.zeros((R // 16, K // 256, 64, 8, 8), dtype=np.int8)
        for i, a in enumerate((0, 4, 1, 5)):
            q[..., a, :] = pieces[:, :, i, :, :8]
            q[..., a + 2, :] = pieces[:, :, i, :, 8:]
        sc = t[..., 4096:].copy().view("<u2").reshape(R // 16, K // 256, 16, 8)
        sc = np.moveaxis(sc, 1, 2).reshape(R, K // 32)
        return {"fmt": fmt, "q": _unlanes(q, R, K), "d": _f16_from_bits(sc)}
    if fmt == "bf16":
        b = t.copy().view("<u2").reshape(R // 16, K // 256, 8, 64, 8)   # kb, lane, j
        b = np.moveaxis(b, 2, 3)                                         # lane, kb, j
        w = (_unlanes(b, R, K).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return {"fmt": fmt, "w": w}
    raise ValueError(fmt)


# ---------------------------------------------------------------------------
# Routing.  The pages keep the router unquantized and say nothing about its
# function; the reading taken: logits l = x Wr^T (+ bias), softmax over all
# experts, keep the k largest (ties: lower expert index first), renormalize
# over the kept k.  Softmax is monotone, so renormalizing the kept softmax
# values equals exp(l_j - l_0) / sum_i exp(l_i - l_0) over the kept logits.


def route(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray | None, k: int):
    """x [T, H], w_router [E, H], bias [E] or None -> (idx int64 [T, k],
    weights fp64 [T, k], logits fp64 [T, E]).  Order: descending logit."""
    x = np.asarray(x, dtype=np.float64)
    logits = x @ np.asarray(w_router, dtype=np.float64).T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int64)
    wts = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        order = np.argsort(-logits[t], kind="stable")[:k]   # ties keep index order
        idx[t] = order
        l = logits[t, order]
        p = np.exp(l - l[0])
        wts[t] = p / p.sum()
    return idx, wts, logits


def group(topk_idx: np.ndarray, n_experts: int):
    """Stable counting sort of the T*k slots (slot = t*k + j) by expert.
    Returns expert_offsets [E+1], sorted_slots [T*k], slot_pos [T*k]."""
    e_of_slot = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    sorted_slots = np.argsort(e_of_slot, kind="stable")
    counts = np.bincount(e_of_slot, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    slot_pos = np.empty_like(sorted_slots)
    slot_pos[sorted_slots] = np.arange(sorted_slots.size)
    return offsets.astype(np.int64), sorted_slots.astype(np.int64), slot_pos.astype(np.int64)


# ---------------------------------------------------------------------------
# Expert FFN: h = SiLU(x Wg^T) * (x Wu^T), y = h Wd^T, SiLU(z) = z / (1 + e^-z).


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_ffn(x: np.ndarray, w_up: np.ndarray, w_gate: np.ndarray, w_down: np.ndarray,
               round_h=None) -> np.ndarray:
    """x [n, H] -> y [n, H] for one expert (all fp64).  `round_h`, if given,
    is applied to h before the down projection (mirror checks)."""
    x = np.asarray(x, dtype=np.float64)
    u = x @ w_up.T
    g = x @ w_gate.T
    h = silu(g) * u
    if round_h is not None:
        h = round_h(h)
    return h @ w_down.T


def moe_layer(x: np.ndarray, w_router: np.ndarray, bias, k: int, expert_weights,
              shared=None, round_h=None):
    """The routed-MoE layer in fp64.

    expert_weights(e) -> (W_up [I, H], W_gate [I, H], W_down [H, I]) fp64;
    shared is (W_up, W_gate, W_down) fp64 or None.  Returns (y [T, H], idx,
    weights): y_t = sum_j w_tj FFN_{e_tj}(x_t) + shared(x_t), summed over j
    in route order, then the shared expert."""
    x = np.asarray(x, dtype=np.float64)
    idx, wts, _ = route(x, w_router, bias, k)
    T, H = x.shape
    offsets, sorted_slots, _ = group(idx, w_router.shape[0])
    y_slot = np.zeros((T * k, H))
    for e in range(w_router.shape[0]):
        slots = sorted_slots[offsets[e]:offsets[e + 1]]
        if slots.size == 0:
            continue
        wu, wg, wd = expert_weights(e)
        y_slot[slots] = expert_ffn(x[slots // k], wu, wg, wd, round_h)
    y = np.zeros((T, H))
    for j in range(k):
        y = y + wts[:, j:j + 1] * y_slot[j::k]
    if shared is not None:
        y = y + expert_ffn(x, *shared, round_h=round_h)
    return y, idx, wts


def dense_ffn(x: np.ndarray, w_up: np.ndarray, w_gate: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """Plain SwiGLU FFN written as explicit Python loops (tiny sizes only)."""
    x = np.asarray(x, dtype=np.float64)
    n, H = x.shape
    I = w_up.shape[0]
    y = np.zeros((n, w_down.shape[0]))
    for t in range(n):
        h = np.zeros(I)
        for i in range(I):
            u = 0.0
            g = 0.0
            for c in range(H):
                u += x[t, c] * w_up[i, c]
                g += x[t, c] * w_gate[i, c]
            h[i] = g / (1.0 + math.exp(-g)) * u
        for o in range(w_down.shape[0]):
            acc = 0.0
            for i in range(I):
                acc += h[i] * w_down[o, i]
            y[t, o] = acc
    return y
