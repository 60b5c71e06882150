"""Benchmark of the routed 2-bit MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload headline]

The headline metric is MoE-layer tokens/s at batch-1 decode and at a
2048-token prefill chunk, each with its roofline fraction (HBM for decode,
MFMA for prefill).  The default run (--workload headline) measures both and
prints them in ONE JSON line:

  value / ms_per_step / roofline   decode_b1: K single-token steps, each one
                                   moe_layer_decode call (router, top-k, expert
                                   FFN, combine), replayed from one captured
                                   HIP graph; the dominant kernel's roofline
                                   over the bytes it streams (routed experts +
                                   bf16 shared expert), against 8 TB/s and
                                   against a measured streaming read of the
                                   same byte count.
  decode_quantized_only            the same layer and tokens without the shared
                                   expert (I_s = 0): %HBM over the quantized
                                   expert bytes alone.
  prefill_2048                     the 2048-token chunk: route, group, grouped
                                   GEMMs, combine; tokens/s and the dominant
                                   GEMM's MFMA fraction.
  cpu_baseline                     the fp64 CPU oracle on a bounded sample.

A step is one pass of the whole hot path over one batch.  Inputs and weights
are resident in HBM before timing starts.  Decode rotates over --instances
copies of the weights so that a step never finds the previous step's experts
in the 256 MB last-level cache.  Kernel durations come from HIP events that
hipExtLaunchKernel records at each kernel dispatch's start and end (the
library's moe_profile_next_launch hook), in a pass that launches the same
steps one by one on the stream the kernels run on; events captured into a
graph carry no timestamps.  --workload W measures one other workload alone
(the *_q8 workloads store the shared expert in the 8-bit Q8 format).
"""
from __future__ import annotations

import argparse
import json
import os
import re
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
# the summaries are under profiles/.  Each entry names the source file that
# defines the kernel and holds a digest of that file, of abi.hip (which sets
# the launch) and of every header the two reach through their #include lines
# (kernel_digest): when any of them differs, the figure no longer describes
# the kernel and "traffic" is reported as null.
MEASURED_TRAFFIC = {
    ("decode_b1", "decode_upgate"): ("k_decode1.hip", "b85a1305e51cfb66", 7.632e+07),
    ("decode_b1", "decode_down"): ("k_decode1.hip", "b85a1305e51cfb66", 3.933e+07),
    ("prefill_2048", "prefill_upgate"): ("k_prefill.hip", "f22f902d45e073d1", 1.839e+09),
    ("prefill_2048", "prefill_down"): ("k_prefill.hip", "f22f902d45e073d1", 1.317e+09),
}
CSRC = os.path.join(ROOT, "bit_quantized_moe_02_amd", "csrc")


def kernel_sources(kernel_file):
    """kernel_file and abi.hip with every file they include ("..." includes,
    followed transitively), as paths sorted by their name under the
    repository root."""
    seen = set()

    def visit(path):
        path = os.path.normpath(path)
        if path in seen:
            return
        seen.add(path)
        with open(path) as f:
            for line in f:
                m = re.match(r'\s*#\s*include\s+"([^"]+)"', line)
                if m:
                    visit(os.path.join(os.path.dirname(path), m.group(1)))

    for name in ("abi.hip", kernel_file):
        visit(os.path.join(CSRC, name))
    return sorted(seen, key=lambda f: os.path.relpath(f, ROOT))


def kernel_digest(kernel_file):
    import hashlib
    h = hashlib.sha256()
    for f in kernel_sources(kernel_file):
        h.update(os.path.relpath(f, ROOT).encode())
        h.update(b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# The decode call runs the single-token kernels once per token up to this
# many tokens (kDecPerTokenMax in csrc/abi.hip).
DEC_PER_TOKEN_MAX = 3
DECODE = {"decode_b1", "decode_b16_hot", "k4_h7168_decode", "decode_b1_noshared", "draft_verify_t3",
          "decode_b1_q8", "k4_h7168_decode_q8"}
PREFILL = {"prefill_2048", "k4_h7168_prefill", "prefill_2048_q8"}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None, help="timed decode steps (prefill: at most 50)")
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="headline", choices=["headline"] + sorted(DECODE | PREFILL))
    p.add_argument("--instances", type=int, default=None,
                   help="layer copies rotated over the decode steps (default 4 for decode, 1 for prefill)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--skip-prefill", action="store_true", help="headline: decode parts only")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--stream-slots", type=int, default=0, metavar="N",
                   help="decode workloads: also time the step with the routed experts streamed from host "
                        "memory through an HBM cache of N experts (moe_layer_decode_streamed)")
    p.add_argument("--stream-keep", type=int, default=1, help="cache steps kept from eviction (with --stream-slots)")
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
            if wl.fmt_shared == "q8":
                sh[i] = dev(qmoe.moe_quantize_pack("q8", synth.shared_weight_f32(wl, which)))
            else:
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
                                       bias=bias, shared_fmt=wl.fmt_shared))
    torch.cuda.synchronize()
    return layers, (nb_up, nb_dn)


def without_shared(layer, wl):
    """The same routed experts and router with the shared expert left out."""
    from bit_quantized_moe_02_amd import qmoe
    t = layer.tensors
    return qmoe.DeviceLayer(wl.n_experts, wl.hidden, wl.inter, 0, wl.fmts, t["up"], t["gate"], t["down"],
                            codebook=t["codebook"], router=t["router"], bias=t["bias"])


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle as it stands, on a bounded sample


def cpu_baseline(wl, seconds, max_tokens=8):
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    cb = O.codebook(0)
    wr = synth.router_weight(wl)
    bias = synth.logit_bias(wl)
    shared = None
    if wl.shared_inter and wl.fmt_shared == "q8":
        shared = tuple(O.dequantize_matrix(O.quantize_matrix("q8", synth.shared_weight_f32(wl, w)),
                                           k=wl.hidden if w != "down" else wl.shared_inter)
                       for w in ("up", "gate", "down"))
    elif wl.shared_inter:
        shared = tuple(synth.bf16_bits_to_f32(synth.shared_weight_bits(wl, w)).astype(np.float64)
                       for w in ("up", "gate", "down"))
    # sample tokens: the workload's own inputs, in order
    if wl.name in DECODE:
        xs = [synth.bf16_bits_to_f32(synth.activations_bits(wl, wl.tokens, step=s)).astype(np.float64)
              for s in range(max_tokens)]
    else:
        full = synth.bf16_bits_to_f32(synth.activations_bits(wl, wl.tokens)).astype(np.float64)
        xs = [full[i:i + 1] for i in range(max_tokens)]
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
# Timing


class Events:
    """Reusable torch events for the per-kernel dispatch timestamps."""

    def __init__(self, names, n):
        import torch
        self.ev = {kn: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                        for _ in range(n)] for kn in names}
        for kn in names:          # torch creates the HIP event on its first record
            for a, b in self.ev[kn]:
                a.record()
                b.record()

    def arm(self, i):
        from bit_quantized_moe_02_amd import qmoe
        for kn, lst in self.ev.items():
            qmoe.moe_profile_next_launch(kn, *lst[i])

    def seconds(self, kn):
        return np.array([a.elapsed_time(b) for a, b in self.ev[kn]]) * 1e-3


def time_decode(wl, layers, steps, warmup, label):
    """K steps of moe_layer_decode replayed from one HIP graph, then the same
    steps launched one by one with dispatch events on every kernel."""
    import torch
    from bit_quantized_moe_02_amd import qmoe
    E, H, k, T = wl.n_experts, wl.hidden, wl.top_k, wl.tokens
    inst = len(layers)
    n_x = min(steps + warmup, wl.steps)
    xs = torch.stack([torch.from_numpy(synth.activations_bits(wl, T, step=s).view(np.int16)).view(torch.bfloat16)
                      for s in range(n_x)]).cuda()
    n_total = steps + warmup
    idx_all = torch.empty((n_total, T, k), dtype=torch.int32, device="cuda")
    w_all = torch.empty((n_total, T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(qmoe.moe_layer_decode_workspace_bytes(layers[0].w, T, k), dtype=torch.uint8, device="cuda")
    kernels = ["route_logits", "decode_upgate", "decode_down"]
    ev = Events(kernels, steps)

    def step(s, timed):
        layer = layers[s % inst]
        if timed is not None:
            ev.arm(timed)
        qmoe.moe_layer_decode(layer.w, layer.router, layer.bias, xs[s % n_x], T, k, idx_all[s], w_all[s], y, ws)

    for s in range(warmup):
        step(s, None)
    torch.cuda.synchronize()
    # The K timed steps are captured back to back into one HIP graph (each
    # step: route + expert FFN of its own token, with its own input row, layer
    # copy and output slots), so host launch overhead -- which a whole-model
    # decode graph spreads over all its layers -- stays out of the per-layer
    # figure.  One untimed replay uploads the graph first.
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
    log(f"[bench] {label}: {steps} steps in {1e3 * (t1 - t0):.2f} ms (graph)")
    te0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i, i)
    torch.cuda.synchronize()
    te1 = time.perf_counter()
    del graph
    return {"seconds": t1 - t0, "durs": {kn: ev.seconds(kn) for kn in kernels},
            "idx": idx_all[warmup:].cpu().numpy(), "eager_tps": steps * T / (te1 - te0)}


def time_streamed(wl, layer, n_slots, keep, steps, warmup):
    """Decode steps with the routed experts in page-locked host memory and an
    HBM cache of n_slots experts: each step is one moe_layer_decode_streamed
    call (route, choices to the host, plan, copies of the misses on a copy
    stream, expert FFN over the cache), launched eagerly (the call waits for
    the routing on the host, so it cannot be captured in a graph)."""
    import torch
    from bit_quantized_moe_02_amd import qmoe
    E, H, k, T = wl.n_experts, wl.hidden, wl.top_k, wl.tokens
    t = layer.tensors
    host = []
    for n in ("up", "gate", "down"):
        h = torch.empty(t[n].numel(), dtype=torch.uint8, pin_memory=True)
        h.copy_(t[n])
        host.append(h)
    cache = qmoe.ExpertCache(E, H, wl.inter, wl.fmts, *host, n_slots=n_slots, keep=keep, shared_from=layer)
    n_x = min(steps + warmup, wl.steps)
    xs = torch.stack([torch.from_numpy(synth.activations_bits(wl, T, step=s).view(np.int16)).view(torch.bfloat16)
                      for s in range(n_x)]).cuda()
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(cache.decode_workspace_bytes(T, k), dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream()
    for s in range(warmup):
        cache.decode(layer.router, layer.bias, xs[s % n_x], T, k, idx, w, y, ws, copy_stream=cs)
    torch.cuda.synchronize()
    _, h0, m0 = cache.state()
    t0 = time.perf_counter()
    for i in range(steps):
        cache.decode(layer.router, layer.bias, xs[(warmup + i) % n_x], T, k, idx, w, y, ws, copy_stream=cs)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    _, h1, m1 = cache.state()
    nb = 2 * qmoe.moe_packed_bytes(wl.fmt_up, wl.inter, H) + qmoe.moe_packed_bytes(wl.fmt_down, H, wl.inter)
    hits, misses = h1 - h0, m1 - m0
    cache.close()
    return {"n_slots": n_slots, "keep": keep, "cache_bytes": n_slots * nb, "steps": steps,
            "tokens_per_s": round(steps * T / (t1 - t0), 1), "ms_per_step": round((t1 - t0) / steps * 1e3, 4),
            "hit_rate": round(hits / max(1, hits + misses), 4),
            "copied_bytes_per_token": round(misses * nb / (steps * T), 1),
            "host_to_device_GBs": round(misses * nb / (t1 - t0) / 1e9, 2),
            "entry": "moe_layer_decode_streamed", "host_memory": "page-locked", "launch": "eager"}


def shared_bytes(wl):
    """Packed bytes of the shared expert's up (= gate) and down matrices."""
    if wl.shared_inter == 0:
        return 0, 0
    from bit_quantized_moe_02_amd import qmoe
    return (qmoe.moe_packed_bytes(wl.fmt_shared, wl.shared_inter, wl.hidden),
            qmoe.moe_packed_bytes(wl.fmt_shared, wl.hidden, wl.shared_inter))


def decode_work(wl, idx_h, nb_up, nb_dn):
    """Algorithmic bytes per timed launch of the up/gate and down kernels and
    the quantized expert bytes alone, from the routing each step made."""
    T, k, H, I, Is = wl.tokens, wl.top_k, wl.hidden, wl.inter, wl.shared_inter
    nb_su, nb_sd = shared_bytes(wl)
    w = {"decode_upgate": [], "decode_down": [], "route_logits": [], "quant_upgate": [], "quant_down": []}
    for s in range(idx_h.shape[0]):
        # up to DEC_PER_TOKEN_MAX tokens the library runs the single-token
        # kernels once per token and the events time the first token's
        # launch; beyond, one launch covers the whole batch
        Tl = 1 if T <= DEC_PER_TOKEN_MAX else T
        d = len(np.unique(idx_h[s][:Tl]))
        w["quant_upgate"].append(d * 2 * nb_up)
        w["quant_down"].append(d * nb_dn)
        # up/gate: both matrices of the distinct routed experts + shared, x in, h out
        w["decode_upgate"].append(d * 2 * nb_up + 2 * nb_su + Tl * H * 2 + Tl * k * I * 2 + Tl * Is * 2)
        # down: the distinct routed down matrices + shared, h in, y out
        w["decode_down"].append(d * nb_dn + nb_sd + Tl * k * I * 2 + Tl * Is * 2 + Tl * H * 4)
        # router: fp32 weights + x in, logits out
        w["route_logits"].append(wl.n_experts * H * 4 + T * H * 2 + T * wl.n_experts * 4)
    return {kn: np.array(v, dtype=np.float64) for kn, v in w.items()}


def kernel_stats(durs, work, scale, peak):
    ach = work.sum() / durs.sum() / scale
    return {"avg_us": round(float(durs.mean()) * 1e6, 2), "achieved": round(float(ach), 1),
            "frac": round(float(ach / peak), 4), "work_per_launch": float(work.mean())}


def read_ceiling(nbytes, reps=24):
    """Rate of the library's streaming-read kernel over `nbytes` (rounded to
    16), rotating over enough buffers that the 256 MB last-level cache holds
    none of them, timed with dispatch events: GB/s (best grid of 2, 4 or 8
    workgroups per compute unit)."""
    import torch
    from bit_quantized_moe_02_amd import qmoe
    nbytes = (int(nbytes) + 15) // 16 * 16
    nbuf = max(2, -(-(512 << 20) // nbytes))
    bufs = [torch.full((nbytes,), i + 1, dtype=torch.uint8, device="cuda") for i in range(nbuf)]
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    best = None
    for per_cu in (2, 4, 8):
        ev = Events(["read"], reps)
        for i in range(4):                                   # warm-up
            qmoe.moe_measure_read(bufs[i % nbuf], out, per_cu * cus)
        for i in range(reps):
            ev.arm(i)
            qmoe.moe_measure_read(bufs[(i + 4) % nbuf], out, per_cu * cus)
        torch.cuda.synchronize()
        d = ev.seconds("read")
        gbs = nbytes / d.mean() / 1e9
        if best is None or gbs > best["GB/s"]:
            best = {"GB/s": round(float(gbs), 1), "avg_us": round(float(d.mean()) * 1e6, 2), "bytes": nbytes,
                    "workgroups_per_cu": per_cu}
    del bufs
    return best


def time_prefill(wl, layer, steps, warmup):
    """Route, group and the prefill expert FFN of one chunk, K times, launched
    eagerly (a step is ~1.6 ms, so host launch cost stays out of the way),
    with dispatch events on the two GEMM kernels."""
    import torch
    from bit_quantized_moe_02_amd import qmoe
    E, H, k, T = wl.n_experts, wl.hidden, wl.top_k, wl.tokens
    x = torch.from_numpy(synth.activations_bits(wl, T).view(np.int16)).view(torch.bfloat16).cuda()
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    rws = torch.empty(qmoe.moe_route_workspace_bytes(T, E), dtype=torch.uint8, device="cuda")
    ws = torch.empty(qmoe.moe_ffn_workspace_bytes(layer.w, T, k, True), dtype=torch.uint8, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    ss = torch.empty(T * k, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    gws = torch.zeros(qmoe.moe_group_workspace_bytes(T, k, E), dtype=torch.uint8, device="cuda")
    kernels = ["prefill_upgate", "prefill_down"]
    ev = Events(kernels, steps)

    def step(timed):
        qmoe.moe_route(x, layer.router, layer.bias, T, H, E, k, idx, w, rws)
        qmoe.moe_group_tokens(idx, T, k, E, off, ss, sp, gws)
        if timed is not None:
            ev.arm(timed)
        qmoe.moe_expert_ffn_prefill(layer.w, x, T, k, idx, w, off, ss, sp, y, ws)

    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    I, Is = wl.inter, wl.shared_inter
    work = {"prefill_upgate": np.full(steps, 2.0 * 2 * (T * k) * I * H + 2.0 * 2 * T * Is * H),
            "prefill_down": np.full(steps, 2.0 * (T * k) * I * H + 2.0 * T * Is * H)}
    per = {kn: kernel_stats(ev.seconds(kn), work[kn], 1e12, MFMA_F16_PEAK_TFLOPS) for kn in kernels}
    dom = max(kernels, key=lambda kn: per[kn]["avg_us"])
    roof = {"bound": "mfma", "achieved": per[dom]["achieved"], "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": per[dom]["frac"], "traffic": traffic_of(wl.name, dom), "traffic_unit": "bytes per launch",
            "kernel": dom, "avg_us": per[dom]["avg_us"], "flops_per_launch": per[dom]["work_per_launch"]}
    useful = work["prefill_upgate"][0] + work["prefill_down"][0]
    return {"value": round(steps * T / (t1 - t0), 1), "unit": "tokens/s", "steps": steps, "warmup": warmup,
            "ms_per_step": round((t1 - t0) * 1e3 / steps, 4), "launch": "eager",
            "mfma_frac_whole_step": round(useful / ((t1 - t0) / steps) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "roofline": roof, "kernels": per}


def traffic_of(workload, kernel):
    rec = MEASURED_TRAFFIC.get((workload, kernel))
    if rec is not None and rec[1] == kernel_digest(rec[0]):
        return rec[2]
    return None


def decode_config(wl, instances):
    return {"workload": wl.name, "hidden": wl.hidden, "inter": wl.inter, "experts": wl.n_experts,
            "top_k": wl.top_k, "shared_inter": wl.shared_inter, "tokens_per_step": wl.tokens,
            "formats": "/".join(f.upper() for f in wl.fmts),
            "shared_format": wl.fmt_shared.upper() if wl.shared_inter else None,
            "layer_instances": instances, "launch": "hip_graph",
            "entry": "moe_layer_decode",
            "decode_kernels": "single-token, once per token" if wl.tokens <= DEC_PER_TOKEN_MAX else "batched"}


def decode_report(wl, res, nb_up, nb_dn, steps, ceilings=None):
    work = decode_work(wl, res["idx"], nb_up, nb_dn)
    per = {kn: kernel_stats(res["durs"][kn], work[kn], 1e9, HBM_PEAK_GBS) for kn in res["durs"]}
    if ceilings:
        for kn, c in ceilings.items():
            per[kn]["read_ceiling_GBs"] = c["GB/s"]
            per[kn]["frac_of_ceiling"] = round(per[kn]["achieved"] / c["GB/s"], 4)
    return per, work


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)          # reads and writes MIB MiB once each
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calibrate_copy} MiB done")
        del src, dst
    name = args.workload
    head = name == "headline"
    dname = "decode_b1" if head else name
    out = None

    if head or name in DECODE:
        wl = synth.WORKLOADS[dname]
        steps = args.steps if args.steps is not None else 1000
        warmup = args.warmup if args.warmup is not None else 50
        instances = args.instances if args.instances is not None else 4
        layers, (nb_up, nb_dn) = build_layer(wl, instances)
        res = time_decode(wl, layers, steps, warmup, wl.name)
        per, work = decode_report(wl, res, nb_up, nb_dn, steps)
        dom = max(["decode_upgate", "decode_down"], key=lambda kn: res["durs"][kn].sum())
        ceil = read_ceiling(per[dom]["work_per_launch"])
        per[dom]["read_ceiling_GBs"] = ceil["GB/s"]
        per[dom]["frac_of_ceiling"] = round(per[dom]["achieved"] / ceil["GB/s"], 4)
        step_us = res["seconds"] / steps * 1e6
        out = {
            "metric": METRIC, "value": round(steps * wl.tokens / res["seconds"], 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": round(step_us * 1e-3, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
            "config": decode_config(wl, instances),
            "roofline": {"bound": "hbm", "achieved": per[dom]["achieved"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": per[dom]["frac"], "traffic": traffic_of(wl.name, dom),
                         "traffic_unit": "bytes per launch", "kernel": dom, "avg_us": per[dom]["avg_us"],
                         "bytes_per_launch": per[dom]["work_per_launch"],
                         "read_ceiling": ceil, "frac_of_read_ceiling": per[dom]["frac_of_ceiling"]},
            "kernels": per,
            "kernel_timing": {"events": "hipExtLaunchKernel dispatch start/end", "launch": "one by one",
                              "sum_of_kernel_us": round(sum(float(res["durs"][kn].mean()) for kn in res["durs"]) * 1e6,
                                                        2),
                              "graph_step_us": round(step_us, 2),
                              "eager_tokens_per_s": round(res["eager_tps"], 1)},
        }
        if head or wl.shared_inter == 0:
            # %HBM over the quantized expert bytes alone (no shared expert)
            if head:
                wq = synth.WORKLOADS["decode_b1_noshared"]
                qlayers = [without_shared(l, wl) for l in layers]
                rq = time_decode(wq, qlayers, steps, warmup, wq.name)
            else:
                wq, rq = wl, res
            wk = decode_work(wq, rq["idx"], nb_up, nb_dn)
            q = {}
            for kn, wkey in (("decode_upgate", "quant_upgate"), ("decode_down", "quant_down")):
                d = rq["durs"][kn]
                c = read_ceiling(wk[wkey].mean())
                ach = wk[wkey].sum() / d.sum() / 1e9
                q[kn] = {"avg_us": round(float(d.mean()) * 1e6, 2), "quantized_bytes": float(wk[wkey].mean()),
                         "achieved": round(float(ach), 1), "frac": round(float(ach / HBM_PEAK_GBS), 4),
                         "read_ceiling_GBs": c["GB/s"], "frac_of_ceiling": round(float(ach / c["GB/s"]), 4)}
            qb = wk["quant_upgate"].sum() + wk["quant_down"].sum()
            qs = rq["durs"]["decode_upgate"].sum() + rq["durs"]["decode_down"].sum()
            out["decode_quantized_only"] = {
                "workload": wq.name, "tokens_per_s": round(steps * wq.tokens / rq["seconds"], 1),
                "ms_per_step": round(rq["seconds"] / steps * 1e3, 5),
                "quantized_bytes_per_token": float(qb / steps),
                "frac_hbm_expert_kernels": round(float(qb / qs / 1e9 / HBM_PEAK_GBS), 4),
                "kernels": q}
        if args.stream_slots > 0 and not head:
            log(f"[bench] streaming through {args.stream_slots} cache slots ...")
            out["expert_streaming"] = time_streamed(wl, layers[0], args.stream_slots, args.stream_keep,
                                                    min(steps, 200), min(warmup, 20))
        if not args.no_cpu_baseline:
            log("[bench] timing the CPU oracle (decode) ...")
            out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
        del layers

    if (head and not args.skip_prefill) or name in PREFILL:
        pwl = synth.WORKLOADS["prefill_2048" if head else name]
        psteps = min(args.steps, 50) if args.steps is not None else 20
        pwarm = min(args.warmup, 5) if args.warmup is not None else 3
        players, _ = build_layer(pwl, 1)
        pre = time_prefill(pwl, players[0], psteps, pwarm)
        pre["config"] = {"workload": pwl.name, "hidden": pwl.hidden, "inter": pwl.inter, "experts": pwl.n_experts,
                         "top_k": pwl.top_k, "shared_inter": pwl.shared_inter, "tokens_per_step": pwl.tokens,
                         "formats": "/".join(f.upper() for f in pwl.fmts),
                         "shared_format": pwl.fmt_shared.upper() if pwl.shared_inter else None}
        if not args.no_cpu_baseline:
            log("[bench] timing the CPU oracle (prefill) ...")
            pre["cpu_baseline"] = cpu_baseline(pwl, min(args.cpu_seconds, 10.0), max_tokens=6)
        if head:
            out[pwl.name] = pre
        else:
            out = {"metric": METRIC, "value": pre["value"], "unit": "tokens/s", "n_gpus": 1, "steps": psteps,
                   "warmup": pwarm, "ms_per_step": pre["ms_per_step"], "higher_is_better": True, "scaling": "weak",
                   "vs_baseline": None, "dtype": "f16", "data": "synthetic", "config": pre.pop("config"),
                   "roofline": pre["roofline"], "kernels": pre["kernels"],
                   "mfma_frac_whole_step": pre["mfma_frac_whole_step"]}
            if "cpu_baseline" in pre:
                out["cpu_baseline"] = pre["cpu_baseline"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
