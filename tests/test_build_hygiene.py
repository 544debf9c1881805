"""Static checks of the HIP sources and their generated gfx950 code."""

import os
import re
import subprocess

import pytest

from prefill_attention_rmsnorm_amd import build as B


def test_no_bit_cast_of_vector_elements():
    # clang miscompiles __builtin_bit_cast(T, v[i]) on ext_vector elements
    # (the index is dropped); operands must go through a scalar first.
    pat = re.compile(r"__builtin_bit_cast\([^()]*\[[^\]]*\]\s*\)")
    for f in os.listdir(B.CSRC):
        text = open(os.path.join(B.CSRC, f)).read()
        assert not pat.search(text), f


@pytest.mark.parametrize("src", [s for s in B.SOURCES if s.endswith(".hip")])
def test_no_packed_fp32_instructions(src, tmp_path):
    # All device code is compiled with packed FP32 disabled; no v_pk_add/
    # mul/fma_f32 may appear in the generated assembly.
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path / (src + ".s")
    cmd = [hipcc] + B._flags() + ["--cuda-device-only", "-S",
                                  os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    assert "gfx950" in asm
    bad = re.findall(r"v_pk_(?:fma|add|mul)_f32", asm)
    assert not bad, f"{src}: {len(bad)} packed fp32 instructions"
