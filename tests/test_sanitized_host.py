"""The host code of the library (the packer; the C ABI's argument checks,
workspace layout and launch set-up) built with AddressSanitizer and
UndefinedBehaviorSanitizer, and the CPU tests of the library run against
that build in a child process: any out-of-bounds access, use after free or
undefined operation on those paths aborts the run.  CPU only (device code is
built as usual and never launched here)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from bit_quantized_moe_02_amd import build
    try:
        runtime = build.sanitizer_runtime()
    except (OSError, subprocess.CalledProcessError) as e:
        pytest.skip(f"no clang sanitizer runtime: {e}")
    if not os.path.exists(runtime):
        pytest.skip(f"no clang sanitizer runtime at {runtime}")
    lib = build.build_sanitized(str(tmp_path / "libqmoe_san.so"))
    env = dict(os.environ, QMOE_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_host_lib.py"),
                        os.path.join(ROOT, "tests", "test_expert_cache.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=900)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stdout[-3000:]
    assert "passed" in r.stdout
