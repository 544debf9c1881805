"""CPU checks of the C ABI: the library loads, exports every declared entry
point, and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

from prefill_attention_rmsnorm_amd import qa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(qa.LIB_PATH),
                                reason="libqa.so not built")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared()
    assert len(names) >= 13
    L = ctypes.CDLL(qa.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(qa.EXPORTS)


def test_status_strings():
    L = qa.lib()
    assert L.qa_status_str(0) == b"QA_OK"
    assert L.qa_status_str(-5) == b"QA_ERR_CAPACITY"
    assert L.qa_status_str(-8) == b"QA_ERR_DEVICE"


FAKE = 0x10000  # an aligned address that is never dereferenced


def _cache(batch=2, hkv=2, cap=64, hd=128):
    c = qa.QaCache()
    st = qa.lib().qa_cache_alloc(ctypes.byref(c), batch, hkv, cap, hd,
                                 ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE * 2))
    return st, c


def _params(hq=4, scale=0.088, theta=1e6, eps=1e-6):
    return qa.QaParams(hq, scale, theta, eps, None, None)


def test_cache_descriptor_with_caller_memory():
    st, c = _cache(2, 3, 50)
    assert st == 0 and c.owns == 0
    assert (c.stride_pos, c.stride_h, c.stride_b) == (128, 50 * 128, 3 * 50 * 128)
    assert qa.lib().qa_cache_free(ctypes.byref(c)) == 0
    assert c.k is None


@pytest.mark.parametrize("args,status", [
    ((2, 2, 64, 64), -3),    # head_dim
    ((0, 2, 64, 128), -2),   # batch
    ((2, 2, 0, 128), -2),    # capacity
])
def test_cache_alloc_rejects(args, status):
    st, _ = _cache(*args)
    assert st == status


def test_cache_alloc_rejects_half_memory_and_misalignment():
    c = qa.QaCache()
    L = qa.lib()
    assert L.qa_cache_alloc(ctypes.byref(c), 1, 1, 8, 128,
                            ctypes.c_void_p(FAKE), None) == -1
    assert L.qa_cache_alloc(ctypes.byref(c), 1, 1, 8, 128,
                            ctypes.c_void_p(FAKE + 2),
                            ctypes.c_void_p(FAKE)) == -4


def _decode(c, p, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, pos=FAKE, batch=2, max_ctx=64, out=FAKE,
             lse=None, ws=FAKE, ws_bytes=1 << 20)
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return qa.lib().qa_decode(ctypes.byref(c), ctypes.byref(p), vp(a["q"]),
                              vp(a["k"]), vp(a["v"]), vp(a["pos"]), a["batch"],
                              a["max_ctx"], vp(a["out"]), vp(a["lse"]),
                              vp(a["ws"]), a["ws_bytes"], None)


def test_decode_validation_paths():
    st, c = _cache(2, 2, 64)
    assert st == 0
    before = qa.counters()
    assert _decode(c, _params(hq=4), q=None) == -1
    assert _decode(c, _params(hq=3)) == -2               # Hq % Hkv
    assert _decode(c, _params(hq=32)) == -3              # group 16
    assert _decode(c, _params(hq=4), batch=3) == -2      # > cache batch
    assert _decode(c, _params(hq=4), max_ctx=65) == -5   # > capacity
    assert b"capacity" in qa.lib().qa_last_error()
    assert _decode(c, _params(hq=4), q=FAKE + 8) == -4   # alignment
    assert _decode(c, _params(hq=4), ws_bytes=100) == -6
    assert _decode(c, _params(hq=4, theta=-1.0)) == -2
    assert _decode(c, _params(hq=4, scale=float("nan"))) == -2
    assert qa.counters()[4] - before[4] == 9
    assert qa.counters()[1] == before[1]                 # nothing launched


def test_prefill_validation_paths():
    st, c = _cache(2, 2, 64)
    p = _params(hq=4)
    L = qa.lib()
    vp = ctypes.c_void_p

    def call(n_seq=2, T=10, max_seqlen=8, qs=512, kvs=256, ws=1 << 20, q=FAKE):
        return L.qa_prefill(ctypes.byref(c), ctypes.byref(p), vp(q), vp(FAKE),
                            vp(FAKE), qs, kvs, vp(FAKE), vp(FAKE), n_seq, T,
                            max_seqlen, vp(FAKE), None, vp(FAKE), ws, None)
    assert call(T=0, q=None) == 0                        # empty call: no-op
    assert call(n_seq=3) == -2
    assert call(max_seqlen=65) == -5
    assert call(qs=500) == -2
    assert call(qs=520 + 4) == -4
    assert call(ws=100) == -6


def test_verify_validation_paths():
    st, c = _cache(2, 2, 64)
    L = qa.lib()
    vp = ctypes.c_void_p

    def call(hq=4, n=16, max_ctx=64):
        p = _params(hq=hq)
        return L.qa_verify(ctypes.byref(c), ctypes.byref(p), vp(FAKE),
                           vp(FAKE), vp(FAKE), vp(FAKE), 2, n, max_ctx,
                           vp(FAKE), None, vp(FAKE), 1 << 24, None)
    assert call(hq=16, n=32) == -2       # 32 tokens x 8 heads > 128 rows
    assert call(n=0) == -2
    assert call(max_ctx=80) == -5


def test_workspace_sizes():
    L = qa.lib()
    # prefill: header + cos/sin table (64 float2 per token)
    assert L.qa_workspace_bytes(0, 4, 32, 8, 8192, 0) == 256 + 8192 * 512
    d = L.qa_workspace_bytes(1, 4, 32, 8, 2176, 0)
    v = L.qa_workspace_bytes(2, 4, 32, 8, 2064, 16)
    assert d > 0 and v > d
    assert L.qa_workspace_bytes(1, 4, 32, 7, 2176, 0) == 0   # bad group
    assert L.qa_workspace_bytes(2, 4, 32, 8, 2064, 64) == 0  # 256 rows


def _norm(x=FAKE, res=None, w=None, T=4, H=2560, eps=1e-6, out=FAKE * 3):
    return qa.lib().qa_rmsnorm_hidden(x, res, w, T, H, eps, out, None)


def test_rmsnorm_hidden_validation_paths():
    before = qa.counters()
    assert _norm(x=None) == -1
    assert _norm(out=None) == -1
    assert _norm(T=-1) == -2
    assert _norm(H=0) == -2
    assert _norm(H=2564) == -2                       # not a multiple of 8
    assert _norm(H=8200) == -3                       # more than 8192
    assert _norm(eps=-1.0) == -2
    assert _norm(eps=float("nan")) == -2
    assert _norm(x=FAKE + 8) == -4                   # alignment
    assert _norm(res=FAKE * 5 + 4) == -4
    assert _norm(w=FAKE * 7 + 2) == -4
    assert b"aligned" in qa.lib().qa_last_error()
    assert qa.counters()[4] - before[4] == 11
    assert qa.counters()[3] == before[3]             # nothing launched
    assert _norm(T=0) == 0                           # empty call: a no-op
    assert _norm(x=None, out=None, T=0) == 0         # (any pointers)
    assert qa.counters()[3] == before[3]
