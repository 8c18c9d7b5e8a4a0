"""Build libdecode_attn.so in-tree with hipcc for gfx950.

``python -m decode_attention_folded_amd.build`` (or ``__graft_entry__.build()``)
compiles the HIP kernels and the C ABI layer into
``decode_attention_folded_amd/libdecode_attn.so``.  Always rebuilds.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libdecode_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

HIP_SOURCES = ["decode_kernel.hip", "decode_select.hip", "quest_kernels.hip", "repeat_kv.hip",
               "calibrate.hip", "noalloc.hip", "check.hip"]
HOST_SOURCES = ["api.cpp"]

# Packed-FP32 instructions are disabled for all device code.  The kernels'
# leading scalar arguments (at most 9) are preloaded into SGPRs at dispatch,
# so their first loads do not wait for a read of the kernel-argument segment.
DEVICE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-kernarg-preload-count=9",
    "-Wall", "-Wno-unused-function",
]


def _hipcc():
    cand = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")
    return cand


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines()
                    if "packed-fp32-ops" not in line and "not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + res.stdout)
    if verbose and out.strip():
        print(out)


def build(verbose=True, out_dir=None):
    """Compile every source and link the shared library; returns its path."""
    hipcc = _hipcc()
    out_dir = out_dir or os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        jobs.append(([hipcc, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    for src in HOST_SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        jobs.append(([hipcc, "-O2", "-std=c++17", "-fPIC", "-Wall", "-x", "c++", "-c",
                      os.path.join(CSRC, src), "-o", obj], obj))
    # the translation units compile independently: run them side by side
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd, _ in jobs]:
            f.result()
    objs = [obj for _, obj in jobs]
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
