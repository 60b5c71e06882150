"""Benchmark of the routed 2-bit MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_b1]

A step is one pass of the whole hot path over one batch: route (router GEMV,
top-k) and the expert FFN (decode: up/gate + SiLU, down, combine; prefill:
grouping, grouped up/gate GEMM, grouped down GEMM, combine).  Inputs and
weights are resident in HBM before timing starts.  Decode workloads rotate
over --instances copies of the layer's weights so that consecutive steps do
not find the previous step's experts in the 256 MB last-level cache.

Prints one JSON line: whole-layer tokens/s, the dominant kernel's roofline
(HBM for decode, MFMA for prefill; its duration measured with HIP events
around that kernel on its stream inside the timed region) and the fp64 CPU
oracle's tokens/s on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "MoE-layer tokens/s (decode b=1, prefill 2048) + % HBM BW / % MFMA peak"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0

# HBM bytes per launch (read + written) of the dominant kernels, from two
# rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE) scaled by the counts the same
# counters gave for an elementwise pass of known size (FETCH x 2.0, WRITE x 1.0);
# the summaries are profiles/<workload>_counters.md.  Each entry holds a digest
# of the kernel sources it was measured on: when the sources differ, the figure
# no longer describes the kernel and "traffic" is reported as null.
MEASURED_TRAFFIC = {
    ("decode_b1", "decode_upgate"): ("abb06f880411c12b:66c6882cc36e9a40", 76.28e6 + 0.049e6),
    ("decode_b1", "decode_down"): ("abb06f880411c12b:66c6882cc36e9a40", 39.33e6 + 0.016e6),
    ("prefill_2048", "prefill_upgate"): ("073ea6d28936fe05:66c6882cc36e9a40", 1761.42e6 + 75.497e6),
    ("prefill_2048", "prefill_down"): ("073ea6d28936fe05:66c6882cc36e9a40", 1015.51e6 + 301.990e6),
}
TRAFFIC_SOURCES = {"decode": ["k_decode1.hip", "device_common.hpp"], "prefill": ["k_prefill.hip", "device_common.hpp"]}


def source_digest(kind):
    import hashlib
    d = os.path.join(ROOT, "bit_quantized_moe_02_amd", "csrc")
    return ":".join(hashlib.sha256(open(os.path.join(d, f), "rb").read()).hexdigest()[:16]
                    for f in TRAFFIC_SOURCES[kind])


# The decode call runs the single-token kernels once per token up to this
# many tokens (kDecPerTokenMax in csrc/abi.hip).
DEC_PER_TOKEN_MAX = 3
DECODE = {"decode_b1", "decode_b16_hot", "k4_h7168_decode", "decode_b1_noshared", "draft_verify_t3"}
PREFILL = {"prefill_2048", "k4_h7168_prefill"}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="decode_b1", choices=sorted(DECODE | PREFILL))
    p.add_argument("--instances", type=int, default=None,
                   help="layer copies rotated over the decode steps (default 4 for decode, 1 for prefill)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-kernel-events", action="store_true",
                   help="time the steps without the per-kernel events")
    p.add_argument("--eager", action="store_true",
                   help="launch every step from Python instead of replaying one captured HIP graph "
                        "(decode workloads; prefill always runs eagerly)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="also run one elementwise pass (torch.neg) over MIB MiB: a kernel of known "
                        "traffic that the hardware byte counters are scaled by")
    return p.parse_args()


# ---------------------------------------------------------------------------
# Layer set-up (host quantization with the library, upload, replication)


def build_layer(wl, instances):
    import torch
    from bit_quantized_moe_02_amd import qmoe
    E, H, I, Is = wl.n_experts, wl.hidden, wl.inter, wl.shared_inter
    cb = qmoe.moe_codebook_generate(0)
    nb_up = qmoe.moe_packed_bytes(wl.fmt_up, I, H)
    nb_dn = qmoe.moe_packed_bytes(wl.fmt_down, H, I)
    up = np.empty(E * nb_up, np.uint8)
    gate = np.empty(E * nb_up, np.uint8)
    down = np.empty(E * nb_dn, np.uint8)

    def pack(job):
        which, e = job
        fmt = {"up": wl.fmt_up, "gate": wl.fmt_gate, "down": wl.fmt_down}[which]
        dst, nb = {"up": (up, nb_up), "gate": (gate, nb_up), "down": (down, nb_dn)}[which]
        qmoe.moe_quantize_pack(fmt, synth.expert_weight(wl, which, e), cb, n_threads=1,
                               out=dst[e * nb:(e + 1) * nb])

    t0 = time.time()
    jobs = [(w, e) for e in range(E) for w in ("up", "gate", "down")]
    n_workers = min(32, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(n_workers) as ex:
        list(ex.map(pack, jobs))
    log(f"[bench] quantized {E} experts of {wl.name} in {time.time() - t0:.1f} s ({n_workers} threads)")
    dev = lambda a: torch.from_numpy(a).cuda()
    sh = [None, None, None]
    if Is > 0:
        for i, which in enumerate(("up", "gate", "down")):
            sh[i] = dev(qmoe.moe_quantize_pack("bf16", synth.bf16_bits_to_f32(synth.shared_weight_bits(wl, which))))
    router = dev(synth.router_weight(wl))
    bias = synth.logit_bias(wl)
    bias = dev(bias) if bias is not None else None
    cbd = dev(cb.reshape(-1).copy()) if "cb2" in wl.fmts else None
    layers = []
    d_up, d_gate, d_down = dev(up), dev(gate), dev(down)
    for i in range(instances):
        if i > 0:
            d_up, d_gate, d_down = d_up.clone(), d_gate.clone(), d_down.clone()
            sh = [s.clone() if s is not None else None for s in sh]
            router = router.clone()
        layers.append(qmoe.DeviceLayer(E, H, I, Is, wl.fmts, d_up, d_gate, d_down, codebook=cbd,
                                       shared_up=sh[0], shared_gate=sh[1], shared_down=sh[2], router=router,
                                       bias=bias))
    torch.cuda.synchronize()
    return layers, (nb_up, nb_dn)


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle as it stands, on a bounded sample


def cpu_baseline(wl, seconds):
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    cb = O.codebook(0)
    wr = synth.router_weight(wl)
    bias = synth.logit_bias(wl)
    shared = None
    if wl.shared_inter:
        shared = tuple(synth.bf16_bits_to_f32(synth.shared_weight_bits(wl, w)).astype(np.float64)
                       for w in ("up", "gate", "down"))
    # sample tokens: the workload's own inputs, in order
    if wl.name in DECODE:
        per_step = wl.tokens
        xs = [synth.bf16_bits_to_f32(synth.activations_bits(wl, wl.tokens, step=s)).astype(np.float64)
              for s in range(8)]
    else:
        full = synth.bf16_bits_to_f32(synth.activations_bits(wl, wl.tokens)).astype(np.float64)
        per_step = 1
        xs = [full[i:i + 1] for i in range(8)]
    fields = {}

    def fields_of(e):   # oracle quantization of an expert (set-up, not timed)
        if e not in fields:
            fields[e] = tuple(O.quantize_matrix(fmt, synth.expert_weight(wl, which, e), cb)
                              for which, fmt in zip(("up", "gate", "down"), wl.fmts))
        return fields[e]

    def experts_of(e):  # dequantize when used, no caching (timed)
        f = fields[e]
        return (O.dequantize_matrix(f[0], cb, k=wl.hidden), O.dequantize_matrix(f[1], cb, k=wl.hidden),
                O.dequantize_matrix(f[2], cb, k=wl.inter))

    done_tokens, elapsed, n_steps = 0, 0.0, 0
    for x in xs:
        idx, _, _ = O.route(x, wr, bias, wl.top_k)
        for e in set(idx.reshape(-1).tolist()):
            fields_of(e)
        t0 = time.perf_counter()
        O.moe_layer(x, wr, bias, wl.top_k, experts_of, shared=shared)
        elapsed += time.perf_counter() - t0
        done_tokens += x.shape[0]
        n_steps += 1
        if elapsed >= seconds:
            break
    what = (f"first {n_steps} step(s) of {wl.name} ({done_tokens} tokens)" if wl.name in DECODE
            else f"first {done_tokens} tokens of the {wl.tokens}-token {wl.name} chunk, one at a time")
    return {"value": done_tokens / elapsed, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": what + "; numpy fp64, routed experts dequantized when used; "
                             f"{elapsed:.1f} s of CPU time, os.cpu_count()={os.cpu_count()}"}


# ---------------------------------------------------------------------------


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    from bit_quantized_moe_02_amd import qmoe
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = synth.WORKLOADS[args.workload]
    decode = wl.name in DECODE
    steps = args.steps if args.steps is not None else (1000 if decode else 20)
    warmup = args.warmup if args.warmup is not None else (50 if decode else 3)
    instances = args.instances if args.instances is not None else (4 if decode else 1)
    E, H, I, Is, k, T = wl.n_experts, wl.hidden, wl.inter, wl.shared_inter, wl.top_k, wl.tokens

    layers, (nb_up, nb_dn) = build_layer(wl, instances)
    # inputs: one independent draw per step (decode), one chunk (prefill)
    n_x = min(steps + warmup, wl.steps) if decode else 1
    xs = torch.stack([torch.from_numpy(synth.activations_bits(wl, T, step=s).view(np.int16)).view(torch.bfloat16)
                      for s in range(n_x)]).cuda()
    n_total = steps + warmup
    idx_all = torch.empty((n_total, T, k), dtype=torch.int32, device="cuda")
    w_all = torch.empty((n_total, T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    rws = torch.empty(qmoe.moe_route_workspace_bytes(T, E), dtype=torch.uint8, device="cuda")
    if decode:     # the whole decode step in one call (router, top-k, experts, combine)
        ws = torch.empty(qmoe.moe_layer_decode_workspace_bytes(layers[0].w, T, k), dtype=torch.uint8, device="cuda")
    else:
        ws = torch.empty(qmoe.moe_ffn_workspace_bytes(layers[0].w, T, k, True), dtype=torch.uint8, device="cuda")
    if not decode:
        off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        ss = torch.empty(T * k, dtype=torch.int32, device="cuda")
        sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
        gws = torch.zeros(qmoe.moe_group_workspace_bytes(T, k, E), dtype=torch.uint8, device="cuda")
    kernels = ["decode_upgate", "decode_down"] if decode else ["prefill_upgate", "prefill_down"]
    ev = {kn: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
          for kn in kernels}
    for kn in kernels:       # torch creates the HIP event on its first record
        for a, b in ev[kn]:
            a.record()
            b.record()

    def step(s, timed_kernel):
        layer = layers[s % instances]
        x = xs[s % n_x]
        if not decode:
            qmoe.moe_route(x, layer.router, layer.bias, T, H, E, k, idx_all[s], w_all[s], rws)
        if timed_kernel is not None:
            for kn in kernels:
                qmoe.moe_profile_next_launch(kn, *ev[kn][timed_kernel])
        if decode:
            qmoe.moe_layer_decode(layer.w, layer.router, layer.bias, x, T, k, idx_all[s], w_all[s], y, ws)
        else:
            qmoe.moe_group_tokens(idx_all[s], T, k, E, off, ss, sp, gws)
            qmoe.moe_expert_ffn_prefill(layer.w, x, T, k, idx_all[s], w_all[s], off, ss, sp, y, ws)

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)          # reads and writes MIB MiB once each
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calibrate_copy} MiB done")
        del src, dst
    for s in range(warmup):
        step(s, None)
    torch.cuda.synchronize()
    use_graph = decode and not args.eager
    eager_tps = None
    if use_graph:
        # The K timed steps are captured back to back into one HIP graph (each
        # step: route + expert FFN of its own token, with its own input row,
        # layer copy and output slots), so host launch overhead -- which a
        # whole-model decode graph spreads over all its layers -- stays out of
        # the per-layer figure.  One untimed replay uploads the graph first.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                step(warmup + i, None)
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if not args.no_kernel_events:
            # Events recorded inside a graph carry no usable timestamps, so the
            # kernel durations come from a second timed region: the same K
            # steps launched one by one, with HIP events around each kernel on
            # the stream it runs on.
            te0 = time.perf_counter()
            for i in range(steps):
                step(warmup + i, i)
            torch.cuda.synchronize()
            eager_tps = steps * T / (time.perf_counter() - te0)
    else:
        t0 = time.perf_counter()
        for i in range(steps):
            step(warmup + i, None if args.no_kernel_events else i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    tokens_per_s = steps * T / (t1 - t0)

    # dominant kernel: algorithmic work per launch from the routing each step made
    idx_h = idx_all[warmup:].cpu().numpy()
    roof, per_kernel = None, None
    if not args.no_kernel_events:
        durs = {kn: np.array([a.elapsed_time(b) for a, b in ev[kn]]) * 1e-3 for kn in kernels}   # s
        # algorithmic work per launch, from the routing each step made
        if decode:
            work = {kn: [] for kn in kernels}
            for s in range(steps):
                # up to DEC_PER_TOKEN_MAX tokens the library runs the single-token
                # kernels once per token and the events time the first token's
                # launch; beyond, one launch covers the whole batch
                Tl = 1 if T <= DEC_PER_TOKEN_MAX else T
                d = len(np.unique(idx_h[s][:Tl]))
                # up/gate: both matrices of the distinct routed experts + shared, x in, h out
                work["decode_upgate"].append(d * 2 * nb_up + 2 * Is * H * 2 + Tl * H * 2 + Tl * k * I * 2 + Tl * Is * 2)
                # down: the distinct routed down matrices + shared, h in, y out
                work["decode_down"].append(d * nb_dn + H * Is * 2 + Tl * k * I * 2 + Tl * Is * 2 + Tl * H * 4)
            unit, peak, bound, scale = "GB/s", HBM_PEAK_GBS, "hbm", 1e9
        else:
            work = {"prefill_upgate": [2.0 * 2 * (T * k) * I * H + 2.0 * 2 * T * Is * H] * steps,
                    "prefill_down": [2.0 * (T * k) * I * H + 2.0 * T * Is * H] * steps}
            unit, peak, bound, scale = "TFLOP/s", MFMA_F16_PEAK_TFLOPS, "mfma", 1e12
        per_kernel = {}
        for kn in kernels:
            w = np.array(work[kn], dtype=np.float64)
            ach = w.sum() / durs[kn].sum() / scale
            per_kernel[kn] = {"avg_us": round(float(durs[kn].mean()) * 1e6, 2), "achieved": round(ach, 1),
                              "frac": round(ach / peak, 4), "work_per_launch": float(w.mean())}
        dom = max(kernels, key=lambda kn: durs[kn].sum())
        traffic = None
        rec = MEASURED_TRAFFIC.get((wl.name, dom))
        if rec is not None and rec[0] == source_digest("decode" if decode else "prefill"):
            traffic = rec[1]
        roof = {"bound": bound, "achieved": per_kernel[dom]["achieved"], "peak": peak, "unit": unit,
                "frac": per_kernel[dom]["frac"], "traffic": traffic, "traffic_unit": "bytes per launch",
                "kernel": dom,
                "avg_us": per_kernel[dom]["avg_us"],
                ("bytes_per_launch" if decode else "flops_per_launch"): per_kernel[dom]["work_per_launch"]}

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": wl.name, "hidden": H, "inter": I, "experts": E, "top_k": k, "shared_inter": Is,
                   "tokens_per_step": T, "formats": "/".join(f.upper() for f in wl.fmts),
                   "layer_instances": instances, "launch": "hip_graph" if use_graph else "eager",
                   **({"entry": "moe_layer_decode",
                       "decode_kernels": "single-token, once per token" if T <= DEC_PER_TOKEN_MAX else "batched"}
                      if decode else {})},
        "roofline": roof,
        "kernels": per_kernel,
        "kernel_events_pass": None if per_kernel is None else {
            "launch": "eager" if use_graph else "same as timed region",
            "tokens_per_s": None if eager_tps is None else round(eager_tps, 1)},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
