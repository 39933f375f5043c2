"""ctypes wrapper around attn_oracle.c (plain C, fp64, OpenMP).

TEST INFRASTRUCTURE ONLY (see the package docstring).  The arithmetic lives in
attn_oracle.c; this module only builds it with gcc, marshals numpy float64
arrays and returns the results.

Definition followed (page "GPU 内核与 FlashAttention", sections 10, 11.1, 13.2):
for each batch b, head h and query i,
    s_ij = scale * <q_i, k_j>,  m_i = max_j s_ij,  l_i = sum_j exp(s_ij - m_i),
    O_i  = sum_j exp(s_ij - m_i) / l_i * v_j,  LSE_i = m_i + ln l_i.
Options of the same page's section 14: causal (s_ij = -inf for j > i, section 14.4)
and grouped K/V heads (k, v with heads_kv heads; query head h reads K/V head
h // (heads // heads_kv), section 14.2).  heads_kv is read off k's shape.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def library_path():
    return _LIB


def build(force=True):
    """Compile attn_oracle.c into oracle/liboracle.so with gcc (-O2 -fopenmp)."""
    global _lib
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    _lib = None
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [_D, _D, _D, _D, _D, _i64, _i64, _i64, _i64, _i64, _i64,
                                     ctypes.c_double, ctypes.c_int, _I64]
    lib.oracle_attention_rows.restype = ctypes.c_int
    lib.oracle_attention_rows.argtypes = [_D, _D, _D, _D, _D, _i64, _i64, _i64, _i64, _i64, _i64,
                                          ctypes.c_double, ctypes.c_int, _I64, _I64, _i64]
    lib.oracle_attention_online.restype = ctypes.c_int
    lib.oracle_attention_online.argtypes = [_D, _D, _D, _D, _D, _i64, _i64, _i64, _i64, _i64,
                                            ctypes.c_double, ctypes.c_int, _i64]
    lib.oracle_attention_bwd.restype = ctypes.c_int
    lib.oracle_attention_bwd.argtypes = [_D, _D, _D, _D, _D, _D, _D, _i64, _i64, _i64, _i64, _i64, _i64,
                                         ctypes.c_double, ctypes.c_int, _I64]
    lib.oracle_attention_bwd_rows.restype = ctypes.c_int
    lib.oracle_attention_bwd_rows.argtypes = [_D, _D, _D, _D, _i64, _i64, _i64, _i64, _i64, _i64,
                                              ctypes.c_double, ctypes.c_int, _I64, _I64, _i64, _D, _I64, _i64,
                                              _D, _D]
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(_LIB)
    return _lib


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_D)


def _shapes(q, k, v, cu_seqlens, max_seqlen):
    """-> (batch, nq, nk, heads, heads_kv, d, cu)"""
    if cu_seqlens is None:
        if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
            raise ValueError("dense q, k, v must be [B, N, H, D] with k and v alike")
        batch, nq, heads, d = q.shape
        hkv = k.shape[2]
        if k.shape[0] != batch or k.shape[3] != d or hkv < 1 or heads % hkv:
            raise ValueError("q and k disagree on batch or d, or k's heads do not divide q's")
        return batch, nq, k.shape[1], heads, hkv, d, None
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    if q.ndim != 3 or k.ndim != 3 or k.shape != v.shape or q.shape[0] != k.shape[0] or \
            q.shape[2] != k.shape[2] or k.shape[1] < 1 or q.shape[1] % k.shape[1]:
        raise ValueError("varlen q must be [total, H, D] and k, v [total, Hkv, D] with Hkv | H")
    batch = cu.shape[0] - 1
    if cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] != q.shape[0]:
        raise ValueError("cu_seqlens must start at 0, not decrease, and end at total")
    lmax = int(np.max(np.diff(cu))) if batch > 0 else 0
    if max_seqlen is None:
        max_seqlen = lmax
    if max_seqlen < lmax:
        raise ValueError("max_seqlen smaller than the longest sequence")
    return batch, max_seqlen, max_seqlen, q.shape[1], k.shape[1], q.shape[2], cu


def attention(q, k, v, scale, cu_seqlens=None, max_seqlen=None, causal=False, _lib_override=None):
    """Exact attention in fp64.

    Dense: q [B, Nq, H, D], k/v [B, Nk, Hkv, D] -> (O [B, Nq, H, D], LSE [B, H, Nq]).
    Varlen: q [total, H, D], k/v [total, Hkv, D] with cu_seqlens [B+1] -> (O [total, H, D],
    LSE [B, H, max_seqlen]); LSE rows past a sequence's length are NaN.
    causal masks key j > query i (indices within the sequence).
    """
    lib = _lib_override or _load()
    batch, nq, nk, heads, hkv, d, cu = _shapes(np.asarray(q), np.asarray(k), np.asarray(v),
                                               cu_seqlens, max_seqlen)
    q, qp = _f64(q)
    k, kp = _f64(k)
    v, vp = _f64(v)
    o = np.zeros(q.shape, dtype=np.float64)
    lse = np.full((batch, heads, nq), np.nan, dtype=np.float64)
    cup = cu.ctypes.data_as(_I64) if cu is not None else None
    rc = lib.oracle_attention(qp, kp, vp, o.ctypes.data_as(_D), lse.ctypes.data_as(_D),
                              batch, nq, nk, heads, hkv, d, float(scale), int(bool(causal)), cup)
    if rc != 0:
        raise MemoryError("oracle_attention failed")
    return o, lse


def attention_rows(q, k, v, scale, rows, cu_seqlens=None, max_seqlen=None, causal=False,
                   _lib_override=None):
    """O and LSE for selected (b, h, i) rows only: returns (O [n, D], LSE [n])."""
    lib = _lib_override or _load()
    batch, nq, nk, heads, hkv, d, cu = _shapes(np.asarray(q), np.asarray(k), np.asarray(v),
                                               cu_seqlens, max_seqlen)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    for b, h, i in rows:
        lq = (cu[b + 1] - cu[b]) if cu is not None else nq
        if not (0 <= b < batch and 0 <= h < heads and 0 <= i < lq):
            raise IndexError("row (%d, %d, %d) out of range" % (b, h, i))
    q, qp = _f64(q)
    k, kp = _f64(k)
    v, vp = _f64(v)
    n = rows.shape[0]
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    cup = cu.ctypes.data_as(_I64) if cu is not None else None
    rc = lib.oracle_attention_rows(qp, kp, vp, o.ctypes.data_as(_D), lse.ctypes.data_as(_D),
                                   batch, nq, nk, heads, hkv, d, float(scale), int(bool(causal)),
                                   cup, rows.ctypes.data_as(_I64), n)
    if rc != 0:
        raise MemoryError("oracle_attention_rows failed")
    return o, lse


def attention_online(q, k, v, scale, block, causal=False, _lib_override=None):
    """The blockwise one-pass recurrence in fp64 (dense layout, as many K/V heads as query
    heads), key blocks of `block`; with causal, blocks above the diagonal are skipped."""
    lib = _lib_override or _load()
    batch, nq, nk, heads, hkv, d, _ = _shapes(np.asarray(q), np.asarray(k), np.asarray(v), None, None)
    if hkv != heads:
        raise ValueError("attention_online takes as many K/V heads as query heads")
    q, qp = _f64(q)
    k, kp = _f64(k)
    v, vp = _f64(v)
    o = np.zeros(q.shape, dtype=np.float64)
    lse = np.zeros((batch, heads, nq), dtype=np.float64)
    rc = lib.oracle_attention_online(qp, kp, vp, o.ctypes.data_as(_D), lse.ctypes.data_as(_D),
                                     batch, nq, nk, heads, d, float(scale), int(bool(causal)),
                                     int(block))
    if rc != 0:
        raise ValueError("oracle_attention_online failed (block must be > 0)")
    return o, lse


def attention_bwd(q, k, v, dout, scale, cu_seqlens=None, max_seqlen=None, causal=False, _lib_override=None):
    """Gradients of exact attention in fp64 (page "GPU 内核与 FlashAttention", section 13.1).

    Same layouts as attention(); dout is shaped like q.  Returns (dQ like q, dK like k,
    dV like v).  Packed rows outside every sequence are left 0.
    """
    lib = _lib_override or _load()
    batch, nq, nk, heads, hkv, d, cu = _shapes(np.asarray(q), np.asarray(k), np.asarray(v),
                                               cu_seqlens, max_seqlen)
    if np.asarray(dout).shape != np.asarray(q).shape:
        raise ValueError("dout must be shaped like q")
    q, qp = _f64(q)
    k, kp = _f64(k)
    v, vp = _f64(v)
    dout, dop = _f64(dout)
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    cup = cu.ctypes.data_as(_I64) if cu is not None else None
    rc = lib.oracle_attention_bwd(qp, kp, vp, dop, dq.ctypes.data_as(_D), dk.ctypes.data_as(_D),
                                  dv.ctypes.data_as(_D), batch, nq, nk, heads, hkv, d, float(scale),
                                  int(bool(causal)), cup)
    if rc != 0:
        raise MemoryError("oracle_attention_bwd failed")
    return dq, dk, dv


def attention_bwd_rows(q, k, v, dout, scale, qrows=(), krows=(), cu_seqlens=None, max_seqlen=None,
                       causal=False, _lib_override=None):
    """Selected rows of the backward pass in fp64: dQ of query rows (b, h, i) and dK, dV of key
    rows (b, hk, j).  Returns (dQ [n_q, D], dK [n_k, D], dV [n_k, D]).  Key rows are best
    grouped by (b, hk): the per-row LSE and D of a (b, hk) are computed once per group."""
    lib = _lib_override or _load()
    batch, nq, nk, heads, hkv, d, cu = _shapes(np.asarray(q), np.asarray(k), np.asarray(v),
                                               cu_seqlens, max_seqlen)
    qr = np.ascontiguousarray(np.asarray(qrows, dtype=np.int64).reshape(-1, 3))
    kr = np.ascontiguousarray(np.asarray(krows, dtype=np.int64).reshape(-1, 3))
    for b, h, i in qr:
        lq = (cu[b + 1] - cu[b]) if cu is not None else nq
        if not (0 <= b < batch and 0 <= h < heads and 0 <= i < lq):
            raise IndexError("query row (%d, %d, %d) out of range" % (b, h, i))
    for b, hk, j in kr:
        lk = (cu[b + 1] - cu[b]) if cu is not None else nk
        if not (0 <= b < batch and 0 <= hk < hkv and 0 <= j < lk):
            raise IndexError("key row (%d, %d, %d) out of range" % (b, hk, j))
    q, qp = _f64(q)
    k, kp = _f64(k)
    v, vp = _f64(v)
    dout, dop = _f64(dout)
    dq = np.zeros((qr.shape[0], d), dtype=np.float64)
    dk = np.zeros((kr.shape[0], d), dtype=np.float64)
    dv = np.zeros((kr.shape[0], d), dtype=np.float64)
    cup = cu.ctypes.data_as(_I64) if cu is not None else None
    rc = lib.oracle_attention_bwd_rows(qp, kp, vp, dop, batch, nq, nk, heads, hkv, d, float(scale),
                                       int(bool(causal)), cup, qr.ctypes.data_as(_I64), qr.shape[0],
                                       dq.ctypes.data_as(_D), kr.ctypes.data_as(_I64), kr.shape[0],
                                       dk.ctypes.data_as(_D), dv.ctypes.data_as(_D))
    if rc != 0:
        raise MemoryError("oracle_attention_bwd_rows failed")
    return dq, dk, dv


def num_threads():
    """OpenMP threads the oracle runs with."""
    return int(_load().oracle_num_threads())


class Oracle:
    """The oracle bound to a given shared library (default: oracle/liboracle.so).

    Tests use this to run the same pins against a deliberately altered build
    of attn_oracle.c, to show each plausible mistake fails at least one pin.
    """

    def __init__(self, path=None):
        self._lib = _bind(path) if path else _load()

    def attention(self, *a, **kw):
        return attention(*a, _lib_override=self._lib, **kw)

    def attention_rows(self, *a, **kw):
        return attention_rows(*a, _lib_override=self._lib, **kw)

    def attention_online(self, *a, **kw):
        return attention_online(*a, _lib_override=self._lib, **kw)

    def attention_bwd(self, *a, **kw):
        return attention_bwd(*a, _lib_override=self._lib, **kw)

    def attention_bwd_rows(self, *a, **kw):
        return attention_bwd_rows(*a, _lib_override=self._lib, **kw)


def compile_source(src_text, out_path):
    """Compile C source text (a variant of attn_oracle.c) into a shared library at out_path."""
    c_path = out_path + ".c"
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", out_path, c_path, "-lm"])
    return out_path


def source_text():
    with open(_SRC) as f:
        return f.read()
