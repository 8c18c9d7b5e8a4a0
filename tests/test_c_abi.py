"""The library driven from a plain C program through its C ABI alone
(tests/c_abi/c_abi_check.c, built by __graft_entry__.build()): dense decode
attention with an append, the Quest pipeline and the input check, each
against the program's own fp64 evaluation on the host."""

import os
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "c_abi_check")


def _run():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built: run __graft_entry__.build()")
    return subprocess.run([EXE], capture_output=True, text=True, timeout=120)


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful without a GPU")
def test_c_program_links_and_reports_no_device():
    if not os.path.exists(EXE):  # a CPU checkout that skipped build(): build it here
        import sys
        sys.path.insert(0, ROOT)
        from decode_attention_folded_amd import _binding, build
        if not os.path.exists(_binding.library_path()):
            build.build(verbose=False)
        import __graft_entry__
        __graft_entry__.build_c_abi_check(verbose=False)
    r = _run()
    assert r.returncode == 2, (r.stdout, r.stderr)
    assert "no HIP device" in r.stderr


@pytest.mark.gpu
def test_c_program_drives_every_step_through_the_c_abi():
    r = _run()
    print(r.stdout)
    assert r.returncode == 0, (r.stdout, r.stderr)
    assert r.stdout.strip().splitlines()[-1] == "c abi checks passed"
    assert r.stdout.count(" ok (") == 8
