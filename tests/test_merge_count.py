"""CPU check of decode's in-launch merge counter (csrc/merge_count.h): the
packed fields, the last-arriver rule, the one-XCD placement proof and the
stale-counter test, compiled for the host from the same header the kernel
uses."""

import os
import subprocess

import pytest

from prefill_attention_rmsnorm_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))


def test_merge_counter_host_check(tmp_path):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    exe = tmp_path / "merge_count_check"
    src = os.path.join(HERE, "native", "merge_count_check.cpp")
    cmd = [hipcc, "-std=c++17", "-O2", "--offload-arch=gfx950", "-I", B.CSRC,
           src, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-3000:]
