"""CPU oracle for the INT8 FlashAttention-style forward — TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The GPU library never calls it, and it
shares no code with the GPU library: the arithmetic lives in
``attn_oracle.cpp`` (plain C++17, no fast-math, no contraction) and this module
only marshals numpy arrays.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, invariants and the pages' formulas; none is
"parity unpinned" except the approximation-vs-exact error size, for which the
pages give only a relative claim (see the design notes).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib(path=None):
    """Load (building first if needed) the oracle library, or a variant at `path`."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        _lib = _bind(ctypes.CDLL(_build.ensure_built()))
    return _lib


def _bind(L):
    P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int
    L.oracle_half_to_float.argtypes = [P, P, I64]
    L.oracle_float_to_half.argtypes = [P, P, I64]
    L.oracle_quantize_rows.argtypes = [P, F, I64, I32, I64, P, P]
    L.oracle_quantize_cols.argtypes = [P, F, I64, I64, I32, P, P]
    L.oracle_quantize_rows_int4.argtypes = [P, F, I64, I32, P, P]
    L.oracle_quantize_rows_hadamard.argtypes = [P, F, I64, I32, I32, P, P]
    L.oracle_hadamard_rows.argtypes = [P, I64, I32, P]
    L.oracle_logits_i32.argtypes = [P, P, I32, I32, I32, I32, I32, I32, P, F]
    FL = ctypes.c_float
    L.oracle_attn_int8.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                   I32, I32, I32, I32, FL, P, I64, P, P, F]
    L.oracle_attn_int8_trace.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                         I32, I32, I32, I32, FL, I32, I32, I32, P, P, P, P, P, P,
                                         P, P]
    L.oracle_index_softmax_lut.argtypes = [I32, FL, P]
    L.oracle_attn_ref_f64.argtypes = [P, P, P, I32, I32, I32, I32, I32, I32, I32, P, I64, P, F]
    for fn in ("oracle_half_to_float", "oracle_float_to_half", "oracle_quantize_rows", "oracle_quantize_cols", "oracle_quantize_rows_int4", "oracle_quantize_rows_hadamard", "oracle_hadamard_rows",
               "oracle_logits_i32", "oracle_attn_int8", "oracle_attn_int8_trace",
               "oracle_attn_ref_f64", "oracle_index_softmax_lut"):
        getattr(L, fn).restype = ctypes.c_int
    return L


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def default_threads():
    """Worker threads when a call passes nthreads=0: the CPUs this process may
    run on, at most 16 (a GPU host may show many more CPUs than its share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _nt(nthreads):
    return nthreads if nthreads and nthreads > 0 else default_threads()


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle rejected the arguments of %s" % what)


def half_to_float(h, L=None):
    """binary16 (as np.float16 or uint16 bits) -> fp32, by the oracle's own decoder."""
    h = np.ascontiguousarray(h).view(np.uint16)
    out = np.empty(h.shape, np.float32)
    _check((L or lib()).oracle_half_to_float(_p(h), _p(out), h.size), "half_to_float")
    return out


def float_to_half(f, L=None):
    """fp32 -> binary16 bits (uint16), round to nearest even, by the oracle's encoder."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    _check((L or lib()).oracle_float_to_half(_p(f), _p(out), f.size), "float_to_half")
    return out


def quantize_rows(x, rows_per_scale=1, L=None):
    """Symmetric INT8 quantization of groups of `rows_per_scale` rows.

    x: np.float32 or np.float16 array whose last axis is the row.
    Returns (q int8 same shape, scales fp32 [n_rows // rows_per_scale]).
    """
    x = np.ascontiguousarray(x)
    n_cols = x.shape[-1]
    n_rows = x.size // n_cols
    is_half = x.dtype == np.float16
    if not is_half:
        x = x.astype(np.float32, copy=False)
    q = np.empty(x.shape, np.int8)
    s = np.empty(n_rows // rows_per_scale if rows_per_scale and n_rows % rows_per_scale == 0 else 0,
                 np.float32)
    _check((L or lib()).oracle_quantize_rows(_p(x), int(is_half), n_rows, n_cols, rows_per_scale,
                                             _p(q), _p(s)), "quantize_rows")
    return q, s


def quantize_rows_int4(x, L=None):
    """Per-token symmetric 4-bit quantization: codes in [-7, 7] (int8 array
    like x) and scales absmax / 7 [n_rows]."""
    x = np.ascontiguousarray(x)
    n_cols = x.shape[-1]
    n_rows = x.size // n_cols
    if x.dtype == np.float16:
        src, is_half = x.view(np.uint16), 1
    else:
        src, is_half = np.ascontiguousarray(x, np.float32), 0
    q = np.empty(x.shape, np.int8)
    s = np.empty(n_rows, np.float32)
    _check((L or lib()).oracle_quantize_rows_int4(_p(src), is_half, n_rows, n_cols, _p(q), _p(s)),
           "quantize_rows_int4")
    return q, s


def hadamard_rows(x, L=None):
    """Each row (last axis, a power of two) times the normalized Hadamard
    matrix, by the fast transform in fp32."""
    x = np.ascontiguousarray(x, np.float32)
    y = np.empty_like(x)
    n = x.shape[-1]
    _check((L or lib()).oracle_hadamard_rows(_p(x), x.size // n, n, _p(y)), "hadamard_rows")
    return y


def quantize_rows_hadamard(x, bits=8, L=None):
    """Rows rotated by the normalized Hadamard matrix, then per-token codes
    (bits 8: [-127, 127]; bits 4: [-7, 7]) and scales."""
    x = np.ascontiguousarray(x)
    n_cols = x.shape[-1]
    n_rows = x.size // n_cols
    if x.dtype == np.float16:
        src, is_half = x.view(np.uint16), 1
    else:
        src, is_half = np.ascontiguousarray(x, np.float32), 0
    q = np.empty(x.shape, np.int8)
    s = np.empty(n_rows, np.float32)
    _check((L or lib()).oracle_quantize_rows_hadamard(_p(src), is_half, n_rows, n_cols, bits, _p(q), _p(s)),
           "quantize_rows_hadamard")
    return q, s


def quantize_cols(x, rows_per_group, L=None):
    """Per-column symmetric INT8 quantization of groups of rows_per_group rows:
    x [..., n_cols] (fp32 or fp16) read as [n_groups, rows_per_group, n_cols].
    Returns (codes int8 like x, scales fp32 [n_groups * n_cols])."""
    x = np.ascontiguousarray(x)
    n_cols = x.shape[-1]
    n_rows = x.size // n_cols
    assert n_rows % rows_per_group == 0
    n_groups = n_rows // rows_per_group
    if x.dtype == np.float16:
        src, is_half = x.view(np.uint16), 1
    else:
        src, is_half = np.ascontiguousarray(x, np.float32), 0
    q = np.empty(x.shape, np.int8)
    s = np.empty(n_groups * n_cols, np.float32)
    _check((L or lib()).oracle_quantize_cols(_p(src), is_half, n_groups, rows_per_group, n_cols, _p(q), _p(s)),
           "quantize_cols")
    return q, s


def logits_i32(q, k, B, H, Hkv, Lq, Lkv, d, nthreads=0, L=None):
    """All INT32 logits [B,H,Lq,Lkv] (mask not applied)."""
    q = np.ascontiguousarray(q, np.int8)
    k = np.ascontiguousarray(k, np.int8)
    out = np.empty((B, H, Lq, Lkv), np.int32)
    _check((L or lib()).oracle_logits_i32(_p(q), _p(k), B, H, Hkv, Lq, Lkv, d, _p(out), _nt(nthreads)),
           "logits_i32")
    return out


def index_softmax_lut(bits, clip, L=None):
    """The IndexSoftmax table: 2^bits int32 entries for clipping threshold clip."""
    out = np.empty(1 << bits, np.int32) if 1 <= bits <= 8 else None
    _check((L or lib()).oracle_index_softmax_lut(int(bits), float(clip), _p(out)), "index_softmax_lut")
    return out


def _lut_args(index_softmax):
    return (0, 0.0) if index_softmax is None else (int(index_softmax[0]), float(index_softmax[1]))


def attn_int8(q, s_q, k, s_k, v, s_v, v_per_token, B, H, Hkv, Lq, Lkv, d, causal,
              kv_tile, kv_split_len=0, rows=None, nthreads=0, L=None, index_softmax=None):
    """Step-by-step INT8 attention forward. Returns (O fp32, lse fp32).

    v_per_token: the V scale mode, 0 (or False) one scale for the tensor, 1 (or
    True) one per token [B*Hkv*Lkv], 2 one per (batch, kv head) [B*Hkv], 3 one
    per (batch, kv head, channel) [B*Hkv*d].
    index_softmax: None (exp softmax) or (b, c): IndexSoftmax with a 2^b-entry
    table and clipping threshold c.
    O is [B,H,Lq,d] (rows None) or [len(rows), d]."""
    args = [np.ascontiguousarray(a) for a in (q, s_q, k, s_k, v, s_v)]
    for a, dt in zip(args, (np.int8, np.float32, np.int8, np.float32, np.int8, np.float32)):
        assert a.dtype == dt, (a.dtype, dt)
    if rows is None:
        o = np.empty((B, H, Lq, d), np.float32)
        lse = np.empty((B, H, Lq), np.float32)
        r, nr = None, 0
    else:
        r = np.ascontiguousarray(rows, np.int64)
        nr = r.size
        o = np.empty((nr, d), np.float32)
        lse = np.empty((nr,), np.float32)
    rc = (L or lib()).oracle_attn_int8(*(_p(a) for a in args), int(v_per_token), B, H, Hkv, Lq, Lkv,
                                       d, int(causal), kv_tile, kv_split_len,
                                       *_lut_args(index_softmax), _p(r), nr, _p(o), _p(lse), _nt(nthreads))
    _check(rc, "attn_int8")
    return o, lse


def attn_int8_trace(q, s_q, k, s_k, v, s_v, v_per_token, B, H, Hkv, Lq, Lkv, d, causal,
                    kv_tile, kv_split_len, b, h, i, L=None, index_softmax=None):
    """One row with its per-key trace: dict of o, lse, t (base-2 logit), m_tile, y (127 P_tilde),
    p_hat, w (multiplier of y), split_m."""
    args = [np.ascontiguousarray(a) for a in (q, s_q, k, s_k, v, s_v)]
    o = np.empty(d, np.float32)
    lse = np.empty(1, np.float32)
    t, mt, y, w, sm = (np.empty(Lkv, np.float32) for _ in range(5))
    ph = np.empty(Lkv, np.int32)
    rc = (L or lib()).oracle_attn_int8_trace(*(_p(a) for a in args), int(v_per_token), B, H, Hkv,
                                             Lq, Lkv, d, int(causal), kv_tile, kv_split_len,
                                             *_lut_args(index_softmax), b, h, i,
                                             _p(o), _p(lse), _p(t), _p(mt), _p(y), _p(ph), _p(w),
                                             _p(sm))
    _check(rc, "attn_int8_trace")
    return dict(o=o, lse=float(lse[0]), t=t, m_tile=mt, y=y, p_hat=ph, w=w, split_m=sm)


def attn_ref_f64(q, k, v, B, H, Hkv, Lq, Lkv, d, causal, rows=None, nthreads=0, L=None):
    """Exact softmax(Q K^T / sqrt(d)) V in fp64 on un-quantized fp32 inputs."""
    q, k, v = (np.ascontiguousarray(a, np.float32) for a in (q, k, v))
    if rows is None:
        o = np.empty((B, H, Lq, d), np.float64)
        r, nr = None, 0
    else:
        r = np.ascontiguousarray(rows, np.int64)
        nr = r.size
        o = np.empty((nr, d), np.float64)
    rc = (L or lib()).oracle_attn_ref_f64(_p(q), _p(k), _p(v), B, H, Hkv, Lq, Lkv, d, int(causal),
                                          _p(r), nr, _p(o), _nt(nthreads))
    _check(rc, "attn_ref_f64")
    return o


__all__ = ["lib", "half_to_float", "float_to_half", "quantize_rows", "quantize_rows_int4", "quantize_rows_hadamard", "hadamard_rows", "quantize_cols", "logits_i32", "index_softmax_lut", "attn_int8",
           "attn_int8_trace", "attn_ref_f64"]
