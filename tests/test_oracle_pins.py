"""Pins of the fp64 oracle against facts that do not come from the oracle itself:
published generator outputs, hand-worked blocks, exact rational arithmetic,
brute-force searches written independently here, closed forms and invariants.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a double rounding) fails it.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16_hex(h):
    return float(np.array([int(h, 16)], dtype=np.uint16).view(np.float16)[0])


# ---------------------------------------------------------------------------
# Generator and rounding


def test_splitmix64_known_answers():
    g = _golden("splitmix64_seed0.json")
    got = O.splitmix64(g["seed"], len(g["outputs_hex"]))
    assert [f"{v:016x}" for v in got] == g["outputs_hex"]


def test_codebook_shape_values_and_balance():
    t = O.codebook(0)
    assert t.shape == (256, 8) and t.dtype == np.int8
    assert set(np.unique(t)) <= {-3, -1, 1, 3}
    counts = np.array([(t == v).sum() for v in (-3, -1, 1, 3)])
    # 2048 fair draws of 4 values: each count is 512 +- 3 sigma (sigma ~ 19.6)
    assert np.all(np.abs(counts - 512) < 60), counts
    # the table is the top two bits of each draw, entry-major
    draws = O.splitmix64(0, 16)
    assert [int(v) for v in t[:2].reshape(-1)] == [(-3, -1, 1, 3)[d >> 62] for d in draws]


def _nearest_ties_even(v: Fraction, candidates):
    best = None
    for c in candidates:
        dist = abs(Fraction(c) - v)
        if best is None or dist < best[0]:
            best = (dist, [c])
        elif dist == best[0]:
            best[1].append(c)
    return best[1]


def _nearest_f32(v: Fraction) -> Fraction:
    """Nearest fp32 to an exact rational, ties to even, found among the
    fp32 neighbours of numpy's conversion and compared exactly."""
    c = np.float32(float(v))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(abs(Fraction(float(x)) - v) for x in cands)
    win = [x for x in cands if abs(Fraction(float(x)) - v) == best]
    if len(win) > 1:
        win = [x for x in win if int(np.float32(x).view(np.uint32)) % 2 == 0]
    return Fraction(float(win[0]))


def _f16_neighbors(x: float):
    h = np.float16(x)
    lo = np.nextafter(h, np.float16(-np.inf))
    hi = np.nextafter(h, np.float16(np.inf))
    return [float(lo), float(h), float(hi)]


def test_f16_rounding_is_nearest_even_single_rounding():
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(3000) * 0.05) + list(rng.standard_normal(500) * 1e-5)
    # exact midpoints between fp16 neighbours, and values a hair off them
    for base in [1.0, 0.0625, 3.0, 2.0 ** -20, 1000.0]:
        h = np.float16(base)
        nxt = float(np.nextafter(h, np.float16(np.inf)))
        mid = (float(h) + nxt) / 2
        vals += [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)]
    for x in vals:
        got = float(O.f16(x))
        cands = _f16_neighbors(x)
        winners = _nearest_ties_even(Fraction(float(x)), cands)
        if len(winners) == 2:   # tie: the one with an even last mantissa bit
            winners = [w for w in winners if int(np.float16(w).view(np.uint16)) % 2 == 0]
        assert got == winners[0], (x, got, winners)


def test_bf16_rounding_exact():
    rng = np.random.default_rng(2)
    xs = rng.standard_normal(2000) * 3
    xs = np.concatenate([xs, [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)]])
    got = O.bf16_round(xs)
    for x, g in zip(xs, got):
        e = math.frexp(x)[1]
        ulp = Fraction(2) ** (e - 8)
        n = Fraction(float(x)) / ulp
        fl = math.floor(n)
        rem = n - fl
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
            fl += 1
        assert Fraction(float(g)) == fl * ulp, x
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1 (even)
    assert O.bf16_round(1.0 + 2.0 ** -8) == 1.0
    assert O.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6


# ---------------------------------------------------------------------------
# Worked examples


def test_worked_cb2_block():
    g = _golden("worked_examples.json")
    for ex in g["cb2"]:
        table = np.zeros((256, 8), dtype=np.int8)
        table[0] = 1
        table[7] = np.array(ex["entry"], dtype=np.int8)
        f = {"idx": np.array([[7, 7, 7, 7]], dtype=np.uint8),
             "flip": np.array([[ex["flip"]] * 4], dtype=np.uint8),
             "scale": np.array([[_f16_hex(ex["scale_f16_hex"])]])}
        w = O.cb2_dequantize(f, table)
        assert w.shape == (1, 32)
        assert list(w[0, :8]) == ex["decoded"]
        # re-quantizing returns the same scale and flip bits and the same values
        rq = O.cb2_quantize(w.astype(np.float32), table)
        assert float(rq["scale"][0, 0]) == _f16_hex(ex["scale_f16_hex"])
        assert np.array_equal(O.cb2_dequantize(rq, table), w)
        assert int(rq["idx"][0, 0]) == 7 and int(rq["flip"][0, 0]) == ex["flip"]


def test_worked_kquant_blocks():
    g = _golden("worked_examples.json")
    for ex in g["kquant"]:
        fmt = ex["fmt"]
        B, Q, S = KQ_FIELDS[fmt]
        q = np.zeros((1, 256), dtype=np.uint8)
        q[0, :len(ex["q"])] = ex["q"]
        f = {"q": q,
             "sc": np.full((1, 256 // B), ex["sc"], dtype=np.uint8),
             "m": np.full((1, 256 // B), ex["m"], dtype=np.uint8),
             "d": np.array([[_f16_hex(ex["d_f16_hex"])]]),
             "dmin": np.array([[_f16_hex(ex["dmin_f16_hex"])]])}
        w = O.kq_dequantize(f, fmt)
        assert list(w[0, :len(ex["q"])]) == ex["decoded"], ex["name"]


def test_worked_routing():
    g = _golden("worked_examples.json")
    for ex in g["route"]:
        E = len(ex["logits"])
        # x = identity rows, router = diag(logits) gives logits l exactly
        x = np.ones((1, E))
        wr = np.diag(ex["logits"])
        idx, w, _ = O.route(x, wr, None, ex["k"])
        assert list(idx[0]) == ex["idx"], ex["name"]
        assert np.allclose(w[0], ex["weights"], rtol=1e-14, atol=0), ex["name"]


# ---------------------------------------------------------------------------
# CB2 quantizer


def test_cb2_search_matches_independent_brute_force():
    table = O.codebook(0)
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((4, 64)) * 0.02).astype(np.float32)
    f = O.cb2_quantize(w, table)
    for r in range(4):
        for g in range(8):
            s = float(f["scale"][r, g // 4])
            grp = [float(v) for v in w[r, 8 * g:8 * g + 8]]
            errs = []
            for e in range(256):
                acc = 0.0
                for j in range(8):
                    dd = abs(grp[j]) - s * abs(int(table[e, j])) / 4.0
                    acc = acc + dd * dd
                errs.append(acc)
            best = min(range(256), key=lambda e: (errs[e], e))
            assert int(f["idx"][r, g]) == best
            exp_flip = sum(1 << j for j in range(8)
                           if (grp[j] < 0) != (int(table[best, j]) < 0))
            assert int(f["flip"][r, g]) == exp_flip


def test_cb2_c_search_equals_numpy_search():
    table = O.codebook(0)
    rng = np.random.default_rng(4)
    absw = np.abs(rng.standard_normal((5000, 8)) * 0.02)
    s = O.f16(absw.max(axis=1) / 0.75)
    assert np.array_equal(O.cb2_search_numpy(absw, s, table), O.cb2_search(absw, s, table))


def test_cb2_exactly_representable_roundtrip():
    table = O.codebook(0)
    rng = np.random.default_rng(5)
    has3 = np.nonzero((np.abs(table) == 3).any(axis=1))[0]
    R, K = 3, 256
    w = np.zeros((R, K))
    for r in range(R):
        for blk in range(K // 32):
            s = float(np.float16(rng.uniform(0.01, 0.1)))
            for g in range(4):
                e = int(rng.choice(has3))
                flips = rng.integers(0, 2, 8)
                w[r, blk * 32 + g * 8: blk * 32 + g * 8 + 8] = s * table[e] / 4.0 * np.where(flips, -1, 1)
    f = O.cb2_quantize(w.astype(np.float32), table)
    assert np.array_equal(O.cb2_dequantize(f, table), w)


def test_cb2_zero_and_edge_groups():
    table = O.codebook(0)
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 32:40] = [-0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0]
    w[0, 40] = 0.3
    f = O.cb2_quantize(w, table)
    dq = O.cb2_dequantize(f, table)
    assert np.all(dq[0, :32] == 0) and f["scale"][0, 0] == 0
    assert f["scale"][0, 1] == float(np.float16(0.3 / 0.75))
    # the group holding the single nonzero weight decodes to the table entry
    # of least squared error over all 256 (the table need not hold the ideal
    # magnitude pattern 3,1,1,1,1,1,1,1), with the weight's sign
    s = float(f["scale"][0, 1])
    grp = np.abs(w[0, 40:48].astype(np.float64))
    best = min(float(np.sum((grp - s * np.abs(table[e]) / 4.0) ** 2)) for e in range(256))
    got = float(np.sum((grp - np.abs(dq[0, 40:48])) ** 2))
    assert got == best and dq[0, 40] > 0


# ---------------------------------------------------------------------------
# K-quant quantizers

# (sub-block length, largest code, largest scale or min) that the packed
# fields hold, taken from the formats and not from the oracle: K2 has 2-bit
# codes and 4-bit scales and mins per 16 weights, K4 4-bit codes and 6-bit
# scales and mins per 32 weights.
KQ_FIELDS = {"k2": (16, 3, 15), "k4": (32, 15, 63)}


@pytest.mark.parametrize("fmt", ["k2", "k4"])
def test_kquant_codes_are_nearest_grid_points(fmt):
    B, Q, S = KQ_FIELDS[fmt]
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((3, 512)) * 0.02).astype(np.float32)
    f = O.kq_quantize(w, fmt)
    for r in range(3):
        for k in range(512):
            sb = k // B
            d = f["d"][r, k // 256]
            dmin = f["dmin"][r, k // 256]
            sc = int(f["sc"][r, sb])
            m = int(f["m"][r, sb])
            step = d * sc
            if step == 0:
                assert f["q"][r, k] == 0
                continue
            x = float(w[r, k])
            # nearest of the Q+1 grid values; ties go to the larger code
            dist = [abs(x - (step * qq - dmin * m)) for qq in range(Q + 1)]
            best = min(range(Q + 1), key=lambda qq: (dist[qq], -qq))
            qv = int(f["q"][r, k])
            assert qv == best or dist[qv] - dist[best] <= 1e-15 * (abs(x) + 1), (r, k, qv, best)


@pytest.mark.parametrize("fmt", ["k2", "k4"])
def test_kquant_scales_and_mins_are_nearest_codes(fmt):
    """Per sub-block, sc is the code in 0..S nearest to range/(Q d) and m the
    one nearest to -min(0, min w)/dmin (ties to the larger code), found by
    brute force; the sub-block with the largest range (offset) reaches S."""
    B, Q, S = KQ_FIELDS[fmt]
    rng = np.random.default_rng(16)
    w = (rng.standard_normal((4, 512)) * 0.02).astype(np.float32)
    f = O.kq_quantize(w, fmt)
    for r in range(4):
        for blk in range(2):
            d, dmin = f["d"][r, blk], f["dmin"][r, blk]
            assert d > 0 and dmin > 0
            for sb in range(256 // B):
                x = w[r, 256 * blk + sb * B: 256 * blk + (sb + 1) * B].astype(np.float64)
                lo, hi = min(0.0, x.min()), x.max()
                for code, target, unit in ((int(f["sc"][r, blk * (256 // B) + sb]), (hi - lo) / Q, d),
                                           (int(f["m"][r, blk * (256 // B) + sb]), -lo, dmin)):
                    dist = [abs(target - unit * c) for c in range(S + 1)]
                    best = min(range(S + 1), key=lambda c: (dist[c], -c))
                    assert code == best or dist[code] - dist[best] <= 1e-15, (r, blk, sb, code, best)
            n = 256 // B
            assert f["sc"][r, blk * n:(blk + 1) * n].max() == S
            assert f["m"][r, blk * n:(blk + 1) * n].max() == S


@pytest.mark.parametrize("fmt", ["k2", "k4"])
def test_kquant_error_bound(fmt):
    B, Q, S = KQ_FIELDS[fmt]
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((8, 512)) * 0.02).astype(np.float32)
    f = O.kq_quantize(w, fmt)
    dq = O.kq_dequantize(f, fmt)
    d = np.repeat(f["d"], 256, axis=1)
    dmin = np.repeat(f["dmin"], 256, axis=1)
    sc = np.repeat(f["sc"], B, axis=1).astype(float)
    # grid spacing/2 + scale rounding (Q*d/2) + offset rounding (dmin/2) + slack
    bound = d * sc / 2 + Q * d / 2 + dmin / 2 + 1e-7
    assert np.all(np.abs(dq - w) <= bound)


@pytest.mark.parametrize("fmt", ["k2", "k4"])
def test_kquant_exact_superblock_roundtrip(fmt):
    B, Q, S = KQ_FIELDS[fmt]
    rng = np.random.default_rng(8)
    d = 2.0 ** -8
    dmin = 2.0 ** -9
    sc = rng.integers(1, S + 1, 256 // B)
    m = rng.integers(0, S + 1, 256 // B)
    sc[0] = S      # the block maximum fixes d = max a / S exactly
    m[1] = S       # and dmin = max b / S
    q = rng.integers(0, Q + 1, 256)
    # each sub-block spans its full grid so that lo/hi reproduce sc, m
    for s in range(256 // B):
        q[s * B] = 0
        q[s * B + 1] = Q
    w = np.array([d * sc[k // B] * q[k] - dmin * m[k // B] for k in range(256)])
    # with m > 0 the sub-block minimum is negative and lo = min w; with m = 0,
    # lo = 0 = the grid's q = 0 value.  hi = d*sc*Q - dmin*m.
    f = O.kq_quantize(w[None, :].astype(np.float32), fmt)
    assert np.array_equal(O.kq_dequantize(f, fmt)[0], w)
    assert np.array_equal(f["q"][0], q) and np.array_equal(f["sc"][0], sc)


@pytest.mark.parametrize("fmt", ["k2", "k4"])
def test_kquant_edge_subblocks(fmt):
    B, Q, S = KQ_FIELDS[fmt]
    w = np.zeros((1, 256), dtype=np.float32)
    w[0, 0:B] = 0.05                  # constant positive: lo = 0, one grid point
    w[0, B:2 * B] = -0.05             # constant negative
    w[0, 2 * B:3 * B] = np.linspace(0.01, 0.04, B)    # all positive
    w[0, 3 * B:4 * B] = np.linspace(-0.04, -0.01, B)  # all negative
    # remaining sub-blocks zero
    f = O.kq_quantize(w, fmt)
    dq = O.kq_dequantize(f, fmt)[0]
    assert np.all(dq[4 * B:] == 0)
    assert np.all(f["q"][0, 4 * B:] == 0)
    d, dmin = f["d"][0, 0], f["dmin"][0, 0]
    assert np.all(np.abs(dq[:4 * B] - w[0, :4 * B]) <= d * S / 2 + Q * d + dmin)
    # an all-zero row gives d = dmin = +0 and zero codes
    z = O.kq_quantize(np.zeros((1, 256), np.float32), fmt)
    assert z["d"][0, 0] == 0 and z["dmin"][0, 0] == 0
    assert np.signbit(z["d"][0, 0]) == False and np.signbit(z["dmin"][0, 0]) == False  # noqa: E712


@pytest.mark.parametrize("fmt", ["k2", "k4"])
def test_kquant_dequant_exact_against_rationals(fmt):
    B, Q, S = KQ_FIELDS[fmt]
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((2, 256)) * rng.choice([1e-3, 0.02, 3.0])).astype(np.float32)
    f = O.kq_quantize(w, fmt)
    dq = O.kq_dequantize(f, fmt)
    for r in range(2):
        for k in range(0, 256, 7):
            exact = (Fraction(float(f["d"][r, 0])) * int(f["sc"][r, k // B]) * int(f["q"][r, k])
                     - Fraction(float(f["dmin"][r, 0])) * int(f["m"][r, k // B]))
            assert Fraction(float(dq[r, k])) == _nearest_f32(exact)
    # a block whose d and dmin are 2^39 apart takes the rational path
    f2 = {"q": np.full((1, 256), 1, np.uint8), "sc": np.full((1, 256 // B), 1, np.uint8),
          "m": np.full((1, 256 // B), 1, np.uint8), "d": np.array([[2.0 ** 15]]),
          "dmin": np.array([[2.0 ** -24]])}
    v = O.kq_dequantize(f2, fmt)[0, 0]
    assert Fraction(float(v)) == _nearest_f32(Fraction(2 ** 15) - Fraction(1, 2 ** 24)) == 32768


# ---------------------------------------------------------------------------
# Q8 (8-bit blocks of 32, shared expert)


def test_worked_q8_blocks():
    g = _golden("worked_examples.json")
    for ex in g["q8"]:
        w = np.zeros((1, 32), dtype=np.float32)
        if "w" in ex:
            w[0, :len(ex["w"])] = ex["w"]
        else:
            w[0, :len(ex["w_units_2^-25"])] = [v * 2.0 ** -25 for v in ex["w_units_2^-25"]]
        f = O.q8_quantize(w)
        n = len(ex["q"])
        assert float(f["d"][0, 0]) == _f16_hex(ex["d_f16_hex"]), ex["name"]
        assert list(f["q"][0, :n]) == ex["q"], ex["name"]
        assert not f["q"][0, n:].any()
        assert list(O.q8_dequantize(f)[0, :n]) == ex["decoded"], ex["name"]


def _q8_blocks():
    """Blocks of 32 with normal and fp16-subnormal scales, exact ties, zeros."""
    rng = np.random.default_rng(21)
    rows = [rng.standard_normal(32) * 0.02, rng.standard_normal(32) * 3.0,
            rng.standard_normal(32) * 1e-6, rng.standard_normal(32) * 3e-7,
            np.zeros(32), np.r_[np.zeros(31), -1e-3]]
    # a block whose elements sit exactly on half steps of its own scale
    d = float(np.float16(0.5 / 127))
    ties = np.array([0.5] + [d * (k + 0.5) * (-1) ** k for k in range(31)])
    rows.append(ties)
    return np.array(rows).astype(np.float32)


def test_q8_scale_is_nearest_fp16_of_max_over_127():
    """d is the fp16 nearest to max|w|/127 among its fp16 neighbours (exact
    rational distances), ties to the even significand."""
    w = _q8_blocks()
    f = O.q8_quantize(w)
    for r in range(w.shape[0]):
        target = Fraction(float(np.abs(w[r].astype(np.float64)).max())) / 127
        cands = _f16_neighbors(float(target))
        win = _nearest_ties_even(target, cands)
        if len(win) == 2:
            win = [c for c in win if int(np.float16(c).view(np.uint16)) % 2 == 0]
        assert float(f["d"][r, 0]) == win[0], r


def test_q8_codes_are_nearest_of_all_codes():
    """Brute force over the 255 codes: q minimizes |w - d c| exactly, ties
    to the code of larger magnitude; with a normal scale the largest |w| of
    a block takes |q| = 127."""
    w = _q8_blocks()
    f = O.q8_quantize(w)
    for r in range(w.shape[0]):
        d = Fraction(float(f["d"][r, 0]))
        for k in range(32):
            x = Fraction(float(w[r, k]))
            if d == 0:
                assert f["q"][r, k] == 0
                continue
            best = min(range(-127, 128), key=lambda c: (abs(x - d * c), -abs(c)))
            assert int(f["q"][r, k]) == best, (r, k, int(f["q"][r, k]), best)
        if d >= Fraction(2) ** -14:
            assert np.abs(f["q"][r].astype(int)).max() == 127, r


def test_q8_error_bound_and_exact_roundtrip():
    rng = np.random.default_rng(22)
    w = (rng.standard_normal((6, 512)) * 0.02).astype(np.float32)
    f = O.q8_quantize(w)
    dq = O.q8_dequantize(f)
    d = np.repeat(f["d"], 32, axis=1)
    assert np.all(np.abs(dq - w) <= d / 2)
    # values already on the grid, with the code 127 in each block, come back unchanged
    g = O.q8_quantize(dq.astype(np.float32))
    assert np.array_equal(g["q"], f["q"]) and np.array_equal(g["d"], f["d"])
    # dequantized values are exact fp32 numbers
    assert np.array_equal(dq.astype(np.float32).astype(np.float64), dq)


# ---------------------------------------------------------------------------
# Byte layout


def test_layout_single_weight_positions():
    """Move one weight and check which byte/bit of the tile changes, against
    the positions include/qmoe.h documents."""
    R, K = 32, 512
    r, k = 21, 300           # row-tile 1, n = 5; chunk 1, kk = 44: kb 1, qq 1, j 4
    lane = 16 * 1 + 5
    # CB2: code of the group holding k; flip bit j=4 -> code bit 12
    f = {"fmt": "cb2", "idx": np.zeros((R, K // 8), np.uint8),
         "flip": np.zeros((R, K // 8), np.uint8), "scale": np.zeros((R, K // 32))}
    f["flip"][r, k // 8] = 1 << 4
    f["idx"][r, k // 8] = 0xAB
    p = O.pack_matrix(f).reshape(-1)
    base = (1 * (K // 256) + 1) * 1280
    code_off = base + lane * 16 + 2 * 1
    code = int(p[code_off]) | (int(p[code_off + 1]) << 8)
    assert code == 0xAB | (1 << 12)
    assert np.count_nonzero(p) == 2
    # CB2 scale of block (r, k // 32) at 1024 + n*16 + kb*2
    f["flip"][:] = 0
    f["idx"][:] = 0
    f["scale"][r, k // 32] = 1.0
    p = O.pack_matrix(f).reshape(-1)
    assert p[base + 1024 + 5 * 16 + 2 * 1 + 1] == 0x3C and np.count_nonzero(p) == 1
    # K2: q of (kb=1, j=4) -> dword 0, bit 2*(4*1 + 2) + 0 = 12
    g = {"fmt": "k2", "q": np.zeros((R, K), np.uint8), "sc": np.zeros((R, K // 16), np.uint8),
         "m": np.zeros((R, K // 16), np.uint8), "d": np.zeros((R, K // 256)),
         "dmin": np.zeros((R, K // 256))}
    g["q"][r, k] = 3
    p = O.pack_matrix(g).reshape(-1)
    base = (1 * (K // 256) + 1) * 1344
    dw = int(p[base + lane * 16: base + lane * 16 + 4].view("<u4")[0])
    assert dw == 3 << 12 and np.count_nonzero(p) == 1
    g["q"][r, k] = 0
    g["sc"][r, k // 16] = 0xA          # sub-block kk // 16 = 2
    g["m"][r, k // 16] = 0x7
    p = O.pack_matrix(g).reshape(-1)
    assert p[base + 1024 + 5 * 16 + 2] == 0x7A and np.count_nonzero(p) == 1
    # K4: q of (kb=1, j=4) -> half 0, dword 1, bit 4*2 + 0 = 8
    h = {"fmt": "k4", "q": np.zeros((R, K), np.uint8), "sc": np.zeros((R, K // 32), np.uint8),
         "m": np.zeros((R, K // 32), np.uint8), "d": np.zeros((R, K // 256)),
         "dmin": np.zeros((R, K // 256))}
    h["q"][r, k] = 9
    p = O.pack_matrix(h).reshape(-1)
    base = (1 * (K // 256) + 1) * 2304
    dw = int(p[base + lane * 16 + 4: base + lane * 16 + 8].view("<u4")[0])
    assert dw == 9 << 8 and np.count_nonzero(p) == 1
    # K4 scales: m of sub-block 1 is value 9 of the 6-bit stream, bits 54..59
    h["q"][r, k] = 0
    h["m"][r, k // 32] = 0b101101
    p = O.pack_matrix(h).reshape(-1)
    sb = p[base + 2048 + 5 * 12: base + 2048 + 6 * 12]
    stream = int.from_bytes(bytes(sb), "little")
    assert stream == 0b101101 << 54 and np.count_nonzero(p) == 2
    # BF16: element at kb*1024 + lane*16 + j*2
    b = {"fmt": "bf16", "w": np.zeros((R, K))}
    b["w"][r, k] = 1.0
    p = O.pack_matrix(b).reshape(-1)
    base = (1 * (K // 256) + 1) * 8192
    off = base + 1 * 1024 + lane * 16 + 4 * 2
    assert p[off] == 0x80 and p[off + 1] == 0x3F and np.count_nonzero(p) == 2
    # Q8: (kb=1, j=4) sits in 16-byte piece 2 (k-blocks 1 and 3), first half:
    # byte 2*1024 + lane*16 + 4; the scale of (n, kb) at 4096 + n*16 + kb*2
    c = {"fmt": "q8", "q": np.zeros((R, K), np.int8), "d": np.zeros((R, K // 32))}
    c["q"][r, k] = -5
    c["d"][r, k // 32] = 1.0
    p = O.pack_matrix(c).reshape(-1)
    base = (1 * (K // 256) + 1) * 4352
    assert p[base + 2 * 1024 + lane * 16 + 4] == 0xFB
    assert p[base + 4096 + 5 * 16 + 2 * 1 + 1] == 0x3C and np.count_nonzero(p) == 2
    c["q"][r, k] = 0
    c["q"][r, k + 64] = 7                # kb = 3: piece 2, second half
    p = O.pack_matrix(c).reshape(-1)
    assert p[base + 2 * 1024 + lane * 16 + 8 + 4] == 7
    c["q"][r, k + 64] = 0
    c["q"][r, k + 128] = 9               # kb = 5: piece 3, first half
    p = O.pack_matrix(c).reshape(-1)
    assert p[base + 3 * 1024 + lane * 16 + 4] == 9


@pytest.mark.parametrize("fmt", ["cb2", "k2", "k4", "bf16", "q8"])
def test_pack_unpack_roundtrip(fmt):
    rng = np.random.default_rng(10)
    table = O.codebook(0)
    w = (rng.standard_normal((48, 768)) * 0.02).astype(np.float32)
    if fmt == "bf16":
        w = O.bf16_round(w.astype(np.float64)).astype(np.float32)
    f = O.quantize_matrix(fmt, w, table)
    p = O.pack_matrix(f)
    assert p.size == O.packed_bytes(fmt, 48, 768)
    u = O.unpack_matrix(fmt, p, 48, 768)
    for key in f:
        if key != "fmt":
            assert np.array_equal(f[key], u[key]), key
    assert np.array_equal(O.dequantize_matrix(u, table), O.dequantize_matrix(f, table))


def test_k_padding_to_superblock():
    table = O.codebook(0)
    w = (np.random.default_rng(11).standard_normal((16, 128)) * 0.02).astype(np.float32)
    f = O.quantize_matrix("k2", w, table)
    assert f["q"].shape == (16, 256)
    dq = O.dequantize_matrix(f, table)
    assert np.all(dq[:, 128:] == 0)
    # padding never changes the kept half's scales: same as quantizing the
    # row with explicit zeros
    wz = np.zeros((16, 256), np.float32)
    wz[:, :128] = w
    assert np.array_equal(O.dequantize_matrix(O.quantize_matrix("k2", wz, table), table), dq)


# ---------------------------------------------------------------------------
# Routing and grouping


def test_route_invariants_and_brute_force():
    rng = np.random.default_rng(12)
    T, H, E, k = 16, 32, 12, 3
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((E, H)) * 0.3
    bias = rng.standard_normal(E)
    idx, w, logits = O.route(x, wr, bias, k)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-12)
    for t in range(T):
        l = [sum(x[t, h] * wr[e, h] for h in range(H)) + bias[e] for e in range(E)]
        order = sorted(range(E), key=lambda e: (-l[e], e))[:k]
        assert list(idx[t]) == order
        p = [math.exp(v) for v in l]
        full = [p[e] / sum(p) for e in range(E)]       # softmax over all experts
        kept = [full[e] for e in order]
        assert np.allclose(w[t], np.array(kept) / sum(kept), rtol=1e-12)
    # k = E gives the full softmax
    _, wf, lf = O.route(x, wr, bias, E)
    sm = np.exp(lf - lf.max(axis=1, keepdims=True))
    sm /= sm.sum(axis=1, keepdims=True)
    idx_f, _, _ = O.route(x, wr, bias, E)
    assert np.allclose(np.take_along_axis(sm, idx_f, axis=1), wf, rtol=1e-12)


def test_group_is_stable_permutation():
    rng = np.random.default_rng(13)
    T, k, E = 40, 4, 9
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    off, ss, pos = O.group(idx, E)
    flat = idx.reshape(-1)
    assert sorted(ss) == list(range(T * k))
    assert list(off) == [0] + list(np.cumsum([np.sum(flat == e) for e in range(E)]))
    for e in range(E):
        seg = ss[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)   # stable
    assert np.all(ss[pos] == np.arange(T * k))


# ---------------------------------------------------------------------------
# Whole layer


def _tiny_layer():
    wl = synth.WORKLOADS["tiny"]
    table = O.codebook(0)
    experts = []
    for e in range(wl.n_experts):
        mats = []
        for which, fmt in zip(("up", "gate", "down"), wl.fmts):
            w = synth.expert_weight(wl, which, e)
            f = O.quantize_matrix(fmt, w, table)
            mats.append(O.dequantize_matrix(f, table, k=w.shape[1]))
        experts.append(tuple(mats))
    return wl, experts


def test_layer_equals_dense_brute_force_on_tiny():
    wl, experts = _tiny_layer()
    x = synth.activations_f32(wl, wl.tokens).astype(np.float64)
    wr = synth.router_weight(wl)
    y, idx, wts = O.moe_layer(x, wr, None, wl.top_k, lambda e: experts[e])
    # dense: every expert on every token with gate weight zero off the top-k
    logits = [[sum(float(x[t, h]) * float(wr[e, h]) for h in range(wl.hidden))
               for e in range(wl.n_experts)] for t in range(wl.tokens)]
    y_dense = np.zeros_like(y)
    for t in range(wl.tokens):
        order = sorted(range(wl.n_experts), key=lambda e: (-logits[t][e], e))
        keep = order[:wl.top_k]
        z = sum(math.exp(logits[t][e] - logits[t][keep[0]]) for e in keep)
        for e in range(wl.n_experts):
            gate = math.exp(logits[t][e] - logits[t][keep[0]]) / z if e in keep else 0.0
            y_dense[t] += gate * O.dense_ffn(x[t:t + 1], *experts[e])[0]
    assert np.max(np.abs(y - y_dense)) <= 1e-12 * np.max(np.abs(y_dense))


def test_layer_special_cases():
    rng = np.random.default_rng(14)
    H, I = 16, 8
    x = rng.standard_normal((5, H))
    wu, wg, wd = (rng.standard_normal((I, H)) * 0.3, rng.standard_normal((I, H)) * 0.3,
                  rng.standard_normal((H, I)) * 0.3)
    sh = (rng.standard_normal((I, H)) * 0.3, rng.standard_normal((I, H)) * 0.3,
          rng.standard_normal((H, I)) * 0.3)
    # one expert, k = 1: the plain SwiGLU FFN
    y, _, _ = O.moe_layer(x, rng.standard_normal((1, H)), None, 1, lambda e: (wu, wg, wd))
    assert np.allclose(y, O.dense_ffn(x, wu, wg, wd), rtol=1e-12, atol=1e-14)
    # identical experts: routing weights sum to 1, so FFN(x) + shared(x)
    y, _, _ = O.moe_layer(x, rng.standard_normal((6, H)), None, 3, lambda e: (wu, wg, wd), shared=sh)
    assert np.allclose(y, O.dense_ffn(x, wu, wg, wd) + O.dense_ffn(x, *sh), rtol=1e-12, atol=1e-14)
    # x = 0 gives y = 0
    y, _, _ = O.moe_layer(np.zeros((2, H)), rng.standard_normal((6, H)), None, 2,
                          lambda e: (wu, wg, wd), shared=sh)
    assert np.all(y == 0)


def test_silu_closed_forms():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(O.silu(np.array([-40.0]))[0]) < 1e-15
    assert abs(O.silu(np.array([40.0]))[0] - 40.0) < 1e-12
