"""ctypes binding of libqa (include/qa.h).

Argument marshalling only: torch tensors supply device memory and the
stream; every step of the attention path runs in the HIP kernels of
libqa.so.  There is no fallback: if the library is missing or a call is
rejected, a ``QaError`` is raised.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqa.so")

QA_OP_PREFILL, QA_OP_DECODE, QA_OP_VERIFY = 0, 1, 2
QA_DEVERR_POSITION, QA_DEVERR_SEQLENS, QA_DEVERR_MERGE = 1, 2, 4
HEAD_DIM = 128

EXPORTS = (
    "qa_cache_alloc", "qa_cache_free", "qa_workspace_bytes",
    "qa_workspace_init", "qa_prefill", "qa_decode", "qa_decode_noalloc",
    "qa_verify", "qa_copy",
    "qa_rmsnorm_hidden", "qa_attn_epilogue",
    "qa_status_str", "qa_last_error", "qa_get_counters", "qa_reset_counters",
    "qa_device_error", "qa_set_debug",
)


class QaError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name} ({status}): {detail}")
        self.status = status
        self.name = name
        self.detail = detail


class QaCache(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("capacity", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
        ("stride_pos", ctypes.c_int64), ("owns", ctypes.c_int32),
    ]


class QaParams(ctypes.Structure):
    _fields_ = [
        ("n_q_heads", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_double),
        ("q_norm_w", ctypes.c_void_p), ("k_norm_w", ctypes.c_void_p),
    ]


_lib = None
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, \
    ctypes.c_size_t


def lib():
    """The loaded libqa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise QaError(-100, "QA_NOT_BUILT",
                      f"{LIB_PATH} missing: run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    sig = {
        "qa_cache_alloc": (_i32, [P(QaCache), _i32, _i32, _i32, _i32, _vp, _vp]),
        "qa_cache_free": (_i32, [P(QaCache)]),
        "qa_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
        "qa_workspace_init": (_i32, [_vp, _sz, _vp]),
        "qa_prefill": (_i32, [P(QaCache), P(QaParams), _vp, _vp, _vp, _i64,
                              _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp,
                              _vp, _sz, _vp]),
        "qa_decode": (_i32, [P(QaCache), P(QaParams), _vp, _vp, _vp, _vp,
                             _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
        "qa_decode_noalloc": (_i32, [P(QaCache), P(QaParams), _vp, _vp, _vp,
                                     _vp, _i32, _i32, _vp, _vp, _vp, _vp]),
        "qa_verify": (_i32, [P(QaCache), P(QaParams), _vp, _vp, _vp, _vp,
                             _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
        "qa_copy": (_i32, [_vp, _vp, _sz, _vp]),
        "qa_rmsnorm_hidden": (_i32, [_vp, _vp, _vp, _i32, _i32, ctypes.c_double,
                                     _vp, _vp]),
        "qa_attn_epilogue": (_i32, [_vp, _i64, _vp, _vp, _vp, _i32, _i32, _i32,
                                    ctypes.c_double, _vp, _vp]),
        "qa_status_str": (ctypes.c_char_p, [_i32]),
        "qa_last_error": (ctypes.c_char_p, []),
        "qa_get_counters": (None, [P(ctypes.c_uint64)]),
        "qa_reset_counters": (None, []),
        "qa_device_error": (_i32, [_vp, _vp, P(ctypes.c_int32)]),
        "qa_set_debug": (None, [_i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        L = lib()
        raise QaError(status, L.qa_status_str(status).decode(),
                      L.qa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, numel=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")


# ---------------------------------------------------------------- objects


class Cache:
    """A qa_cache over caller-owned bf16 tensors k, v [B, Hkv, cap, 128].

    k and v may be strided views (a padded slot pitch, a token-major or a
    slot-major buffer viewed as [B, Hkv, cap, 128]) as long as the head_dim
    axis is dense, both share one set of strides, and every stride is a
    multiple of 8 elements; the descriptor carries the strides and the
    library validates them at every call.
    """

    def __init__(self, k: torch.Tensor, v: torch.Tensor):
        if k.shape != v.shape or k.dim() != 4 or k.shape[3] != HEAD_DIM:
            raise ValueError("k, v must be [batch, n_kv_heads, capacity, 128]")
        _need(k, "cache k", torch.bfloat16)
        _need(v, "cache v", torch.bfloat16)
        if k.stride() != v.stride() or k.stride(3) != 1:
            raise ValueError("cache k and v must share strides with a dense "
                             "head_dim axis")
        self.k, self.v = k, v
        B, H, cap, d = k.shape
        self.desc = QaCache()
        if k.is_contiguous():
            _check(lib().qa_cache_alloc(ctypes.byref(self.desc), B, H, cap, d,
                                        _ptr(k), _ptr(v)))
        else:
            sb, sh, sp, _ = k.stride()
            self.desc = QaCache(_ptr(k), _ptr(v), B, H, cap, d, sb, sh, sp, 0)

    @staticmethod
    def empty(batch, n_kv_heads, capacity, device="cuda", fill_bits=0x7FC1):
        """Cache with every slot set to a NaN bit pattern (unwritten marker)."""
        shape = (batch, n_kv_heads, capacity, HEAD_DIM)
        k = torch.full(shape, fill_bits, dtype=torch.int16,
                       device=device).view(torch.bfloat16)
        v = torch.full(shape, fill_bits, dtype=torch.int16,
                       device=device).view(torch.bfloat16)
        return Cache(k, v)

    @property
    def batch(self):
        return self.desc.batch

    @property
    def n_kv_heads(self):
        return self.desc.n_kv_heads

    @property
    def capacity(self):
        return self.desc.capacity


class Params:
    """qa_params; keeps the norm-weight tensors alive."""

    def __init__(self, n_q_heads, softmax_scale, rope_theta=1.0e6,
                 rms_eps=1.0e-6, q_norm_w=None, k_norm_w=None):
        for name, w in (("q_norm_w", q_norm_w), ("k_norm_w", k_norm_w)):
            if w is not None:
                _need(w, name, torch.bfloat16, HEAD_DIM)
        self.q_norm_w, self.k_norm_w = q_norm_w, k_norm_w
        self.desc = QaParams(int(n_q_heads), float(softmax_scale),
                             float(rope_theta), float(rms_eps),
                             _ptr(q_norm_w), _ptr(k_norm_w))


def workspace_bytes(op, batch, n_q_heads, n_kv_heads, max_ctx, block_len=0):
    return int(lib().qa_workspace_bytes(op, batch, n_q_heads, n_kv_heads,
                                        max_ctx, block_len))


def workspace(op, batch, n_q_heads, n_kv_heads, max_ctx, block_len=0,
              device="cuda", stream=None):
    """Allocate (torch) and clear (libqa fill kernel) a workspace."""
    n = workspace_bytes(op, batch, n_q_heads, n_kv_heads, max_ctx, block_len)
    if n <= 0:
        raise QaError(-2, "QA_ERR_SHAPE", "invalid workspace sizes")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    _check(lib().qa_workspace_init(_ptr(ws), n, _stream(stream)))
    return ws


# ---------------------------------------------------------------- calls


def prefill(cache: Cache, params: Params, q, k, v, cu_seqlens, positions,
            max_seqlen, out=None, lse=None, ws=None, stream=None):
    """qa_prefill on packed q [T, Hq, 128], k/v [T, Hkv, 128] (token-strided).

    Returns (out, lse, ws).
    """
    Hq, Hkv = params.desc.n_q_heads, cache.n_kv_heads
    T = q.shape[0]
    n_seq = cu_seqlens.numel() - 1
    if T == 0:
        return (out if out is not None else q.new_empty((0, Hq, HEAD_DIM))), \
            lse, ws
    for name, t, H in (("q", q, Hq), ("k", k, Hkv), ("v", v, Hkv)):
        _need(t, name, torch.bfloat16)
        if t.dim() != 3 or t.shape[0] != T or t.shape[1] != H \
                or t.shape[2] != HEAD_DIM or t.stride(2) != 1 \
                or t.stride(1) != HEAD_DIM:
            raise ValueError(f"{name} must be [T, {H}, 128] with dense heads")
    if k.stride(0) != v.stride(0):
        raise ValueError("k and v must share a token stride")
    _need(cu_seqlens, "cu_seqlens", torch.int32, n_seq + 1)
    _need(positions, "positions", torch.int32, T)
    if out is None:
        out = torch.empty((T, Hq, HEAD_DIM), dtype=torch.bfloat16,
                          device=q.device)
    _need(out, "out", torch.bfloat16, T * Hq * HEAD_DIM)
    if lse is not None:
        _need(lse, "lse", torch.float32, T * Hq)
    if ws is None:
        ws = workspace(QA_OP_PREFILL, cache.batch, Hq, Hkv, T,
                       device=q.device, stream=stream)
    _check(lib().qa_prefill(
        ctypes.byref(cache.desc), ctypes.byref(params.desc), _ptr(q), _ptr(k),
        _ptr(v), q.stride(0), k.stride(0), _ptr(cu_seqlens), _ptr(positions),
        n_seq, T, int(max_seqlen), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
        _stream(stream)))
    return out, lse, ws


def decode(cache: Cache, params: Params, q, k, v, positions, max_ctx,
           out=None, lse=None, ws=None, stream=None):
    """qa_decode on q [B, Hq, 128], k/v [B, Hkv, 128].  Returns (out, lse, ws)."""
    Hq, Hkv = params.desc.n_q_heads, cache.n_kv_heads
    B = q.shape[0]
    _need(q, "q", torch.bfloat16, B * Hq * HEAD_DIM)
    _need(k, "k", torch.bfloat16, B * Hkv * HEAD_DIM)
    _need(v, "v", torch.bfloat16, B * Hkv * HEAD_DIM)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _need(positions, "positions", torch.int32, B)
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.bfloat16,
                          device=q.device)
    _need(out, "out", torch.bfloat16, B * Hq * HEAD_DIM)
    if lse is not None:
        _need(lse, "lse", torch.float32, B * Hq)
    if ws is None:
        ws = workspace(QA_OP_DECODE, B, Hq, Hkv, max_ctx, device=q.device,
                       stream=stream)
    _check(lib().qa_decode(
        ctypes.byref(cache.desc), ctypes.byref(params.desc), _ptr(q), _ptr(k),
        _ptr(v), _ptr(positions), B, int(max_ctx), _ptr(out), _ptr(lse),
        _ptr(ws), ws.numel(), _stream(stream)))
    return out, lse, ws


def decode_noalloc(cache: Cache, params: Params, q, k, v, positions, max_ctx,
                   out, lse=None, dev_err=None, stream=None):
    """qa_decode_noalloc: qa_decode on the library's own scratch array (no
    workspace).  out must be given; dev_err is an optional int32 device
    tensor that collects QA_DEVERR_* bits.  Returns out."""
    Hq, Hkv = params.desc.n_q_heads, cache.n_kv_heads
    B = q.shape[0]
    _need(q, "q", torch.bfloat16, B * Hq * HEAD_DIM)
    _need(k, "k", torch.bfloat16, B * Hkv * HEAD_DIM)
    _need(v, "v", torch.bfloat16, B * Hkv * HEAD_DIM)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _need(positions, "positions", torch.int32, B)
    _need(out, "out", torch.bfloat16, B * Hq * HEAD_DIM)
    if lse is not None:
        _need(lse, "lse", torch.float32, B * Hq)
    if dev_err is not None:
        _need(dev_err, "dev_err", torch.int32, 1)
    _check(lib().qa_decode_noalloc(
        ctypes.byref(cache.desc), ctypes.byref(params.desc), _ptr(q), _ptr(k),
        _ptr(v), _ptr(positions), B, int(max_ctx), _ptr(out), _ptr(lse),
        _ptr(dev_err), _stream(stream)))
    return out


def verify(cache: Cache, params: Params, q, k, v, start_pos, max_ctx,
           out=None, lse=None, ws=None, stream=None):
    """qa_verify on q [B, n, Hq, 128], k/v [B, n, Hkv, 128]."""
    Hq, Hkv = params.desc.n_q_heads, cache.n_kv_heads
    B, n = q.shape[0], q.shape[1]
    _need(q, "q", torch.bfloat16, B * n * Hq * HEAD_DIM)
    _need(k, "k", torch.bfloat16, B * n * Hkv * HEAD_DIM)
    _need(v, "v", torch.bfloat16, B * n * Hkv * HEAD_DIM)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _need(start_pos, "start_pos", torch.int32, B)
    if out is None:
        out = torch.empty((B, n, Hq, HEAD_DIM), dtype=torch.bfloat16,
                          device=q.device)
    _need(out, "out", torch.bfloat16, B * n * Hq * HEAD_DIM)
    if lse is not None:
        _need(lse, "lse", torch.float32, B * n * Hq)
    if ws is None:
        ws = workspace(QA_OP_VERIFY, B, Hq, Hkv, max_ctx, n, device=q.device,
                       stream=stream)
    _check(lib().qa_verify(
        ctypes.byref(cache.desc), ctypes.byref(params.desc), _ptr(q), _ptr(k),
        _ptr(v), _ptr(start_pos), B, n, int(max_ctx), _ptr(out), _ptr(lse),
        _ptr(ws), ws.numel(), _stream(stream)))
    return out, lse, ws


def copy(src: torch.Tensor, dst: torch.Tensor, stream=None):
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    _check(lib().qa_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def rmsnorm_hidden(x, residual=None, weight=None, eps=1e-6, out=None,
                   stream=None):
    """qa_rmsnorm_hidden on x bf16 [T, H]; residual (bf16 [T, H], updated in
    place with bf16(x + residual)) and weight (bf16 [H]) are optional.
    Returns out."""
    if x.dim() != 2:
        raise ValueError("x must be [n_tokens, hidden]")
    T, H = x.shape
    _need(x, "x", torch.bfloat16, T * H)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16, T * H)
    if weight is not None:
        _need(weight, "weight", torch.bfloat16, H)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", torch.bfloat16, T * H)
    _check(lib().qa_rmsnorm_hidden(
        _ptr(x), None if residual is None else _ptr(residual),
        None if weight is None else _ptr(weight), T, H, float(eps), _ptr(out),
        _stream(stream)))
    return out


def attn_epilogue(o, w_o, residual, norm_w=None, eps=1e-6, out=None,
                  stream=None):
    """qa_attn_epilogue: o bf16 [T, in_dim] (a token-strided view is fine,
    e.g. a [T, Hq, 128] attention output reshaped), w_o bf16 [hidden, in_dim],
    residual bf16 [T, hidden] (updated in place with bf16(residual + o w_o^T)),
    norm_w bf16 [hidden] or None.  Returns out = the post-attention norm of the
    new residual."""
    if o.dim() == 3:
        o = o.reshape(o.shape[0], -1)
    if o.dim() != 2 or o.stride(1) != 1:
        raise ValueError("o must be [T, in_dim] with a dense in_dim axis")
    T, in_dim = o.shape
    _need(o, "o", torch.bfloat16)
    if w_o.dim() != 2 or w_o.shape[1] != in_dim or not w_o.is_contiguous():
        raise ValueError("w_o must be a dense [hidden, in_dim] tensor")
    hidden = w_o.shape[0]
    _need(w_o, "w_o", torch.bfloat16)
    if residual.shape != (T, hidden) or not residual.is_contiguous():
        raise ValueError("residual must be a dense [T, hidden] tensor")
    _need(residual, "residual", torch.bfloat16)
    if norm_w is not None:
        _need(norm_w, "norm_w", torch.bfloat16, hidden)
    if out is None:
        out = torch.empty_like(residual)
    _need(out, "out", torch.bfloat16, T * hidden)
    _check(lib().qa_attn_epilogue(
        _ptr(o), o.stride(0), _ptr(w_o), _ptr(residual), _ptr(norm_w), T, in_dim,
        hidden, float(eps), _ptr(out), _stream(stream)))
    return out


def device_error(ws: torch.Tensor, stream=None) -> int:
    code = ctypes.c_int32(0)
    _check(lib().qa_device_error(_ptr(ws), _stream(stream), ctypes.byref(code)))
    return int(code.value)


def set_debug(on: bool):
    """qa_set_debug: synchronise and check every call (QA_ERR_DEVICE on a set
    device error bit); also set by QA_DEBUG=1 in the environment."""
    lib().qa_set_debug(1 if on else 0)


def counters():
    buf = (ctypes.c_uint64 * 8)()
    lib().qa_get_counters(buf)
    return list(buf)


def reset_counters():
    lib().qa_reset_counters()
