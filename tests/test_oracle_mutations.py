"""Planted mistakes in the oracle: each mutation below changes one plausible
detail (a constant, a sign, an index, a dropped term, a transposed operand,
a rounding, a tie rule) in a copy of the oracle's source loaded as a module
of its own, and the oracle pins must reject every one of them.  The oracle
package itself is never modified; the copy lives only inside these tests.
"""
import os
import types

import pytest

import oracle as O_real
import test_oracle_pins as P

SRC_PATH = os.path.join(os.path.dirname(O_real.__file__), "qmoe_oracle.py")

# name -> (exact source text, replacement); each text occurs once
MUTATIONS = {
    # generator and rounding
    "splitmix_shift": ("z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64",
                       "z = ((z ^ (z >> 31)) * 0xBF58476D1CE4E5B9) & MASK64"),
    "codebook_value_map": ("_TOP2_VALUE = {0: -3, 1: -1, 2: 1, 3: 3}", "_TOP2_VALUE = {0: -3, 1: 1, 2: -1, 3: 3}"),
    "f16_double_rounding": ("return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)",
                            "return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float16)"
                            ".astype(np.float64)"),
    "bf16_ties_away": ("r = np.rint(m * 256.0)", "r = np.sign(m) * np.floor(np.abs(m) * 256.0 + 0.5)"),
    # CB2
    "cb2_scale_divisor": ("s = f16(a / 0.75)", "s = f16(a / 0.7)"),
    "cb2_search_last_minimum": ("out[g0:g0 + step] = np.argmin(err, axis=1)",
                                "out[g0:g0 + step] = 255 - np.argmin(err[:, ::-1], axis=1)"),
    "cb2_search_dropped_square": ("err = err + d * d", "err = err + np.abs(d)"),
    "cb2_flip_inverted": ("flip_bits = (neg_w != neg_t)", "flip_bits = (neg_w == neg_t)"),
    "cb2_table_unit": ("t = table[idx.reshape(-1)].astype(np.float64) / 4.0",
                       "t = table[idx.reshape(-1)].astype(np.float64) / 2.0"),
    "cb2_flip_bit_order": ("bits = (flip.reshape(-1, 1) >> np.arange(8, dtype=np.uint8)) & 1",
                           "bits = (flip.reshape(-1, 1) >> np.arange(7, -1, -1, dtype=np.uint8)) & 1"),
    # K-quants
    "kq_k4_scale_range": ('return {"k2": (16, 3, 15), "k4": (32, 15, 63)}[fmt]',
                          'return {"k2": (16, 3, 15), "k4": (32, 15, 31)}[fmt]'),
    "kq_lo_not_clamped": ("lo = np.minimum(0.0, x.min(axis=3))", "lo = x.min(axis=3)"),
    "kq_min_truncated": ("np.minimum(S, np.floor(b / dmin[..., None] + 0.5)))",
                         "np.minimum(S, np.floor(b / dmin[..., None])))"),
    "kq_code_offset_sign": ("np.clip(np.floor((x + off[..., None]) / step[..., None] + 0.5), 0, Q))",
                            "np.clip(np.floor((x - off[..., None]) / step[..., None] + 0.5), 0, Q))"),
    "kq_dequant_min_sign": ("return _exact_f32(d * sc * q, dmin * m, d, dmin)",
                            "return _exact_f32(d * sc * q, -(dmin * m), d, dmin)"),
    "kq_dequant_no_f32_rounding": ("out = f32_round(dscq - dm)", "out = dscq - dm"),
    "kq_dequant_scale_per_superblock": ("sc = np.repeat(f[\"sc\"].astype(np.float64), B, axis=1)",
                                        "sc = np.repeat(f[\"sc\"].astype(np.float64)[:, ::-1], B, axis=1)"),
    # Q8
    "q8_scale_divisor": ("d = f16(np.abs(x).max(axis=2) / 127.0)", "d = f16(np.abs(x).max(axis=2) / 128.0)"),
    "q8_ties_to_even": ("np.minimum(127.0, np.floor(np.abs(x) / d[..., None] + 0.5)))",
                        "np.minimum(127.0, np.rint(np.abs(x) / d[..., None])))"),
    "q8_truncated_codes": ("np.minimum(127.0, np.floor(np.abs(x) / d[..., None] + 0.5)))",
                           "np.minimum(127.0, np.floor(np.abs(x) / d[..., None])))"),
    "q8_clamp_128": ("np.minimum(127.0, np.floor(np.abs(x) / d[..., None] + 0.5)))",
                     "np.minimum(128.0, np.floor(np.abs(x) / d[..., None] + 0.5)))"),
    "q8_sign_dropped": ("q = np.where(x < 0, -mag, mag)", "q = mag"),
    "q8_dequant_block_16": ('return q * np.repeat(f["d"], 32, axis=1)', 'return q * np.repeat(f["d"], 16, axis=1)[:, :q.shape[1]]'),
    # packing
    "pack_q8_piece_order": ("for a in (0, 4, 1, 5)], axis=2)", "for a in (0, 1, 4, 5)], axis=2)"),
    "pack_k2_code_shift": ("shift = 2 * (4 * (kb % 2) + j // 2) + 16 * (j % 2)       # bit of (kb, j)",
                           "shift = 2 * (4 * (kb % 2) + j // 2) + 8 * (j % 2)       # bit of (kb, j)"),
    "pack_k4_scale_bit_order": ("bits[..., b // 8] |= (bit << (b % 8)).astype(np.uint8)",
                                "bits[..., b // 8] |= (bit << (7 - b % 8)).astype(np.uint8)"),
    "pack_cb2_index_flip_swapped": (
        'code = f["idx"].astype(np.uint16) | (f["flip"].astype(np.uint16) << 8)   # [R, K/8]',
        'code = f["flip"].astype(np.uint16) | (f["idx"].astype(np.uint16) << 8)   # [R, K/8]'),
    "pack_k2_scale_min_nibbles_swapped": (
        'scm = (f["sc"].astype(np.uint8) | (f["m"].astype(np.uint8) << 4))      # [R, K/16]',
        'scm = (f["m"].astype(np.uint8) | (f["sc"].astype(np.uint8) << 4))      # [R, K/16]'),
    "pack_k4_code_nibble_order": ("shift = 4 * (j // 2) + 16 * (j % 2)\n        dwords = np.zeros(lanes.shape[:3] + (8,)",
                                  "shift = 8 * (j // 2) + 4 * (j % 2)\n        dwords = np.zeros(lanes.shape[:3] + (8,)"),
    "pack_bf16_kb_lane_order": ("lanes = np.moveaxis(lanes, 3, 2)                             # [.., kb, 64, j]",
                                "lanes = lanes                                               # [.., kb, 64, j]"),
    # routing and grouping
    "route_ties_to_higher_index": ('order = np.argsort(-logits[t], kind="stable")[:k]   # ties keep index order',
                                   'order = np.argsort(logits[t], kind="stable")[::-1][:k]'),
    "route_not_renormalized": ("wts[t] = p / p.sum()", "wts[t] = p / np.exp(logits[t] - l[0]).sum()"),
    "route_bias_dropped": ("logits = logits + np.asarray(bias, dtype=np.float64)[None, :]", "logits = logits"),
    "group_slot_pos_not_inverted": ("slot_pos[sorted_slots] = np.arange(sorted_slots.size)",
                                    "slot_pos[:] = sorted_slots"),
    "group_offsets_inclusive": ("offsets = np.concatenate([[0], np.cumsum(counts)])",
                                "offsets = np.concatenate([np.cumsum(counts), [e_of_slot.size]])"),
    # expert FFN and combine
    "silu_sign": ("return z / (1.0 + np.exp(-z))", "return z / (1.0 + np.exp(z))"),
    "ffn_up_gate_swapped": ("h = silu(g) * u", "h = silu(u) * g"),
    "ffn_down_layout_misread": ("return h @ w_down.T", "return h @ w_down.reshape(w_down.shape[1], w_down.shape[0])"),
    "combine_wrong_slot": ("y = y + wts[:, j:j + 1] * y_slot[j::k]", "y = y + wts[:, j:j + 1] * y_slot[j * T:(j + 1) * T]"),
    "combine_first_weight_only": ("y = y + wts[:, j:j + 1] * y_slot[j::k]", "y = y + wts[:, 0:1] * y_slot[j::k]"),
    "combine_shared_dropped": ("y = y + expert_ffn(x, *shared, round_h=round_h)", "y = y"),
}


def _mutant(old=None, new=None):
    src = open(SRC_PATH).read()
    if old is not None:
        assert src.count(old) == 1, f"mutation text not found exactly once: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = SRC_PATH
    exec(compile(src, SRC_PATH + " (mutant)", "exec"), mod.__dict__)
    return mod


def _pins():
    """(name, zero-argument call) for every pin, parametrized cases expanded."""
    for name in sorted(n for n in dir(P) if n.startswith("test_")):
        f = getattr(P, name)
        params = [m for m in getattr(f, "pytestmark", []) if m.name == "parametrize"]
        if params:
            argname, values = params[0].args[:2]
            for v in values:
                yield f"{name}[{v}]", (lambda f=f, a=argname, v=v: f(**{a: v}))
        else:
            yield name, f


def _failing_pins(mod, stop_at_first):
    saved = P.O
    P.O = mod
    failed = []
    try:
        for name, call in _pins():
            try:
                call()
            except Exception:          # an assertion, or an error the mistake causes
                failed.append(name)
                if stop_at_first:
                    break
    finally:
        P.O = saved
    return failed


def test_unmutated_copy_passes_every_pin():
    """The harness itself: a faithful copy of the oracle fails no pin."""
    assert _failing_pins(_mutant(), stop_at_first=False) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_reject_planted_mistake(name):
    old, new = MUTATIONS[name]
    failed = _failing_pins(_mutant(old, new), stop_at_first=True)
    assert failed, f"no oracle pin rejects the planted mistake {name!r}"
