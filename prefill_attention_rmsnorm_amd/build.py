"""Build libqa.so (HIP, gfx950) in-tree with hipcc.

Every source under ``csrc/`` is compiled to an object under ``_build/`` and
linked into ``libqa.so`` next to this file.  Packed-FP32 instructions are
disabled (``-packed-fp32-ops``) for all device code.
"""

from __future__ import annotations

import hashlib
import json
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqa.so")
ARCH = "gfx950"

SOURCES = ["qa_api.cpp", "util.hip", "prefill.hip", "decode.hip", "verify.hip",
           "merge.hip", "rmsnorm.hip", "noalloc.hip", "epilogue.hip"]
HEADERS = ["qa_internal.h", "qa_device.h", "attn_tile.h", "rmsnorm.h",
           "verify_layout.h", "merge_count.h", "merge_inline.h"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm not installed?)")


def _flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


# Per-source extra flags.  prefill.hip: the prefill kernel claims its next
# q-tile with a one-lane atomic in the middle of the current one and reads the
# result only after it; the compiler's atomic optimizer would rewrite that
# into a wave-wide atomic whose result it spreads over the lanes at once,
# waiting for the round trip right there.
EXTRA_FLAGS = {"prefill.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = ([hipcc()] + _flags() + EXTRA_FLAGS.get(src, [])
           + ["-c", os.path.join(CSRC, src), "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n"
                           f"{r.stderr}")
    return obj


def _code_lines(text: str):
    """The lines of a source with // comments and blank lines removed, so that
    the hash below changes with the code only."""
    for line in text.splitlines():
        code = line.split("//", 1)[0].rstrip()
        if code:
            yield code


def _sha(files, read=None) -> str:
    h = hashlib.sha256()
    for f in files:
        if read is None:
            with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
                text = fh.read()
        else:
            text = read(f)
        for line in _code_lines(text):
            h.update(line.encode() + b"\n")
    return h.hexdigest()[:16]


DECODE_SOURCES = ["decode.hip", "merge.hip", "qa_device.h", "qa_internal.h",
                  "merge_count.h", "merge_inline.h"]


def _git(*args) -> str:
    try:
        r = subprocess.run(["git", "-C", ROOT] + list(args),
                           capture_output=True, text=True, timeout=10)
        return r.stdout.strip() if r.returncode == 0 else ""
    except (OSError, subprocess.SubprocessError):
        return ""


def _write_build_info():
    ver = subprocess.run([hipcc(), "--version"], capture_output=True,
                         text=True).stdout.splitlines()
    info = {
        "commit": _git("rev-parse", "HEAD") or "unknown",
        "dirty": _git("status", "--short", "--", "prefill_attention_rmsnorm_amd",
                      "include"),
        "hipcc": ver[0] if ver else "",
        "arch": ARCH,
        "decode_source_sha": _sha(DECODE_SOURCES),
        "prefill_source_sha": _sha(["prefill.hip", "attn_tile.h",
                                    "qa_device.h", "qa_internal.h"]),
        "verify_source_sha": _sha(["verify.hip", "attn_tile.h", "qa_device.h",
                                   "qa_internal.h", "verify_layout.h", "merge_count.h",
                                   "merge_inline.h", "merge.hip"]),
    }
    with open(os.path.join(BUILD, "BUILD_INFO.json"), "w") as f:
        json.dump(info, f, indent=1)


def build(verbose: bool = True) -> str:
    """Compile every source and link libqa.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] \
        + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    _write_build_info()
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
