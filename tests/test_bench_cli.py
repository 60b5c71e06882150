"""bench.py's one-GPU contract, checked on the CPU: asked for more than one
GPU (or started as one rank of several) it exits with status 2 and a message
before it touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_multi_rank_launch_is_refused():
    r = _run([], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "WORLD_SIZE 4" in r.stderr


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_traffic_digest_follows_includes(tmp_path):
    """The measured-traffic digest of a kernel covers its file, abi.hip and
    every header they reach through #include lines, and changes when any of
    them does (here: a copy of the sources with one header edited)."""
    import shutil
    b = _bench_module()
    names = {os.path.relpath(f, b.ROOT) for f in b.kernel_sources("k_decode1.hip")}
    for must in ("bit_quantized_moe_02_amd/csrc/k_decode1.hip", "bit_quantized_moe_02_amd/csrc/abi.hip",
                 "bit_quantized_moe_02_amd/csrc/device_common.hpp", "bit_quantized_moe_02_amd/csrc/route_common.hpp",
                 "bit_quantized_moe_02_amd/csrc/qmoe_internal.h", "include/qmoe.h"):
        assert must in names, must
    assert "bit_quantized_moe_02_amd/csrc/k_prefill.hip" not in names
    # every measured entry names a kernel file that exists
    for (wl, kern), (kf, dig, nbytes) in b.MEASURED_TRAFFIC.items():
        assert os.path.exists(os.path.join(b.CSRC, kf)) and len(dig) == 16 and nbytes > 0
    # a copy of the tree: editing a header reached only through includes changes the digest
    shutil.copytree(os.path.join(ROOT, "bit_quantized_moe_02_amd", "csrc"),
                    tmp_path / "bit_quantized_moe_02_amd" / "csrc")
    shutil.copytree(os.path.join(ROOT, "include"), tmp_path / "include")
    before = b.kernel_digest("k_decodem.hip")
    b.ROOT, b.CSRC = str(tmp_path), str(tmp_path / "bit_quantized_moe_02_amd" / "csrc")
    assert b.kernel_digest("k_decodem.hip") == before
    with open(tmp_path / "bit_quantized_moe_02_amd" / "csrc" / "decode_common.hpp", "a") as f:
        f.write("\n")
    assert b.kernel_digest("k_decodem.hip") != before
    assert b.kernel_digest("k_prefill.hip") == _bench_module().kernel_digest("k_prefill.hip")
