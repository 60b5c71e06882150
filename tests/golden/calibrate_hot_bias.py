"""Find the logit bias that gives the hot experts of decode_b16_hot a 40% share
of the top-k assignments in expectation, and print it.

Calls only the oracle's router.  The printed value is stored as
synth.HOT_BIAS_DECODE_B16 (rounded to a multiple of 2^-10 so that it is an
exact fp32 number).  Run from the repository root:

    python tests/golden/calibrate_hot_bias.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import oracle as O  # noqa: E402
import synth  # noqa: E402

TARGET_SHARE = 0.40
N_TOKENS = 20000


def hot_share(x, wr, hot, beta, k):
    bias = np.zeros(wr.shape[0])
    bias[hot] = beta
    idx, _, _ = O.route(x, wr, bias, k)
    return np.isin(idx, hot).mean()


def main():
    wl = synth.WORKLOADS["decode_b16_hot"]
    wr = synth.router_weight(wl)
    hot = synth.hot_set(wl)
    x = synth.normal_f32(wl.seed, synth.TAG_BIAS_CALIB, 0, (N_TOKENS, wl.hidden), 1.0)
    x = synth.bf16_bits_to_f32(synth.to_bf16_bits(x))
    lo, hi = 0.0, 8.0
    for _ in range(14):
        mid = (lo + hi) / 2
        if hot_share(x, wr, hot, mid, wl.top_k) < TARGET_SHARE:
            lo = mid
        else:
            hi = mid
    beta = round((lo + hi) / 2 * 1024) / 1024
    print(f"hot set {list(hot)}  bias {beta!r}  share {hot_share(x, wr, hot, beta, wl.top_k):.4f}")


if __name__ == "__main__":
    main()
