"""Builds libqmoe.so in this package directory (gfx950).

The host translation unit (quantizer / packer, no HIP) is compiled by the
host C++ compiler with -ffp-contract=off so its fp64 quantization decisions
do not depend on fused multiply-adds; the device translation units are
compiled by hipcc for gfx950 with packed fp32 instructions disabled.

    python -m bit_quantized_moe_02_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqmoe.so")

ARCH = os.environ.get("QMOE_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX_HOST", shutil.which("g++") or "c++")

HOST_SOURCES = ["host_quant.cpp"]
DEVICE_SOURCES = ["abi.hip", "k_route.hip", "k_decode.hip", "k_decode1.hip", "k_decodem.hip", "k_prefill.hip", "k_misc.hip",
                  "expert_cache.hip"]

HIP_FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC, "-Wno-unused-result"]
HOST_FLAGS = ["-O3", "-fPIC", "-std=c++17", "-ffp-contract=off", "-Wall", "-Wextra",
              "-Wno-unused-parameter", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says
    # so once per file; that note is expected and dropped here.
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([CXX] + HOST_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    n = min(len(jobs), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=n) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs + ["-lpthread"])
    os.replace(tmp, LIB)
    return LIB


# Host-code sanitizer build: AddressSanitizer and UndefinedBehaviorSanitizer
# on the host side of every translation unit (the packer, and the argument
# checks, workspace layout and launch code of the C ABI); device code is
# built as usual.  Every sanitizer flag of a hipcc line carries -Xarch_host.
# The library needs clang's shared ASan runtime preloaded into the process
# (sanitizer_runtime() names it); CPU tests only, no GPU.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    clang = os.path.join(os.path.dirname(HIPCC), "..", "lib", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = shutil.which("amdclang++") or "/opt/rocm/llvm/bin/clang++"
    return subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                          text=True, check=True).stdout.strip()


def build_sanitized(out: str) -> str:
    """Builds the library with host-side ASan + UBSan into `out`."""
    obj_dir = os.path.join(BUILD, "san")
    os.makedirs(obj_dir, exist_ok=True)
    jobs, objs = [], []
    for src in HOST_SOURCES + DEVICE_SOURCES:
        obj = os.path.join(obj_dir, src + ".o")
        flags = HIP_FLAGS + ["-g", "-O1"] + SAN_FLAGS
        if src in HOST_SOURCES:
            flags = flags + ["-ffp-contract=off", "-x", "c++"]
        jobs.append([HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    n = min(len(jobs), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(_run, jobs))
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host", "-shared-libasan"] + SAN_FLAGS +
         ["-o", out + ".tmp"] + objs + ["-lpthread"])
    os.replace(out + ".tmp", out)
    return out


def build_oracle() -> str:
    """Compiles the oracle's plain C search loop (test infrastructure)."""
    src = os.path.join(ROOT, "oracle", "cb2_search.c")
    out = os.path.join(ROOT, "oracle", "_cb2_search.so")
    _run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", src, "-o", out + ".tmp"])
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_oracle())
