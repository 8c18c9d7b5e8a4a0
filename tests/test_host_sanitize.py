"""The C ABI host layer (api.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

tests/host_sanitize/ builds api.cpp with g++ against stub kernel launchers
that record the launch they are asked for (no HIP, no GPU), and a harness
that drives every entry point of include/decode_attn.h: each documented
rejection, the launch a valid call asks for, and a seeded fuzz over extreme
sizes in which a call must either be rejected or ask for a launch whose grid
and workspace fit what was validated.  Any sanitizer report fails the run.
The workspace sizes the sanitized build computes for a list of shapes must
equal the real library's (so the stubs' plan constants are the kernels')."""

import ctypes
import json
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
SOURCES = [os.path.join(ROOT, "decode_attention_folded_amd", "csrc", "api.cpp"),
           os.path.join(HERE, "stub_launchers.cpp"), os.path.join(HERE, "harness.cpp")]
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-static-libasan",
            "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    exe = str(tmp_path_factory.mktemp("host_sanitize") / "harness")
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-Wall", "-Werror", *SANITIZE, *SOURCES, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


def _run(exe, rounds):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.pop("LD_PRELOAD", None)
    return subprocess.run([exe, str(rounds)], capture_output=True, text=True, timeout=300, env=env)


def test_every_entry_point_clean_under_asan_and_ubsan(harness):
    r = _run(harness, 100000)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    assert r.stdout.strip().splitlines()[-1] == "ok"


def test_sanitized_build_sizes_match_the_library(harness):
    from decode_attention_folded_amd import _binding
    if not os.path.exists(_binding.library_path()):
        pytest.skip("the HIP library is not built")
    lib = _binding.load_library()
    r = _run(harness, 10)
    assert r.returncode == 0, r.stderr[-4000:]
    sizes = json.loads(r.stdout.strip().splitlines()[-2])
    for b, hkv, d, cap, hq, budget, st, want in sizes["attention"]:
        desc = _binding.KVCacheDesc()
        desc.k = desc.v = 1 << 20
        desc.batch, desc.num_kv_heads, desc.head_dim, desc.capacity = b, hkv, d, cap
        desc.page_size = 16
        out = ctypes.c_size_t()
        assert lib.da_workspace_size(ctypes.byref(desc), hq, budget, 0, ctypes.byref(out)) == st
        assert out.value == want, (b, hkv, d, cap, hq, budget)
