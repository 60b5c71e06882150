"""Checks on the gfx950 assembly of the library's kernels (CPU only: hipcc
cross-compiles), for two properties that the weight streaming relies on and
that no numerical test can see.

A wave's vector loads complete in order and a wait (s_waitcnt vmcnt(N)) is
a count of loads still in flight, so a kernel keeps its next items' weights
in flight while it computes only where the compiler can count the loads
issued after each payload.

* No flat memory instructions: a flat load counts as a vector load, so an
  LDS read that the compiler can only address as flat (a pointer rounded
  through an integer) makes every later wait a wait for all loads in flight.
* The decode kernels wait for one payload at a time: some wait before a
  multiply leaves the next items' loads in flight (the counts below are
  what each kernel's prefetch depth gives).  Issuing a prefetch on one path
  only, or leaving a payload unused on some path, turns those waits into
  vmcnt(0), as it did in the batched kernels before they were changed.
  The prefill GEMMs wait for all loads once per 256-column chunk by design
  (the next chunk is issued at the start of the current one) and are not
  checked here.
"""
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from bit_quantized_moe_02_amd import build as B  # noqa: E402

HIPCC = B.HIPCC if shutil.which(B.HIPCC) or os.path.exists(B.HIPCC) else None
pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


def _device_asm(src, out_dir):
    out = os.path.join(out_dir, os.path.splitext(src)[0] + ".s")
    subprocess.run([HIPCC] + B.HIP_FLAGS + ["-S", "--cuda-device-only", "-o", out,
                                            os.path.join(B.CSRC, src)],
                   check=True, capture_output=True)
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("asm"))
    with ThreadPoolExecutor(4) as ex:
        texts = list(ex.map(lambda s: _device_asm(s, d), B.DEVICE_SOURCES))
    return dict(zip(B.DEVICE_SOURCES, texts))


def _kernels(text):
    """{symbol: body} of every function in an assembly listing."""
    out, name, body = {}, None, []
    for line in text.splitlines():
        m = re.match(r"^(_Z\w+):(\s|$)", line)
        if m:
            if name:
                out[name] = "\n".join(body)
            name, body = m.group(1), []
        elif name:
            body.append(line)
            if "s_endpgm" in line:
                out[name] = "\n".join(body)
                name, body = None, []
    return out


def test_no_flat_memory_instructions(asm):
    for src, text in asm.items():
        for name, body in _kernels(text).items():
            flat = re.findall(r"^\s*(flat_\w+)", body, re.M)
            assert not flat, f"{src}: {name} uses {sorted(set(flat))}"


@pytest.mark.parametrize("src,kernel,n_inst,min_in_flight", [
    ("k_decodem.hip", "decm_upgate_kernel", 2, 8),
    ("k_decodem.hip", "decm_down_kernel", 2, 24),
    ("k_decode1.hip", "dec1_cb2_upgate_kernel", 4, 12),   # (with and without in-kernel ranking)
    ("k_decode1.hip", "dec1_down_k2d_kernel", 2, 20),
    ("k_decode1.hip", "dec1_k4_upgate_kernel", 2, 8),
    ("k_decode1.hip", "dec1_k4_down_kernel", 2, 24),
])
def test_decode_keeps_loads_in_flight(asm, src, kernel, n_inst, min_in_flight):
    ks = {n: b for n, b in _kernels(asm[src]).items() if kernel in n}
    assert len(ks) == n_inst, sorted(ks)                  # bf16 and Q8 shared expert instances
    for name, body in ks.items():
        counts = [int(c) for c in re.findall(r"s_waitcnt vmcnt\((\d+)\)", body)]
        assert counts and max(counts) >= min_in_flight, (name, sorted(set(counts)))
