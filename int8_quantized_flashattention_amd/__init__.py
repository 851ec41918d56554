"""Python binding of libattn_int8 (INT8 FlashAttention-style forward, gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libattn_int8.so``; PyTorch supplies device memory and the stream.
The functions carry the names of the C ABI in ``include/attn_int8.h``.

Importing this package loads the library and raises ImportError when it has
not been built (``python int8_quantized_flashattention_amd/build.py``): there
is no fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn_int8.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3
ATTN_F32, ATTN_F16 = 0, 1
ATTN_VSCALE_PER_TENSOR, ATTN_VSCALE_PER_TOKEN, ATTN_VSCALE_PER_HEAD, ATTN_VSCALE_PER_CHANNEL = 0, 1, 2, 3

# every function the C header declares, with its ctypes signature
_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "attn_quantize_rows": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I32, _I64, _P, _P, _P]),
    "attn_quantize_cols": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I32, _P, _P, _P]),
    "attn_quantize_rows_int4": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I32, _P, _P, _P, _P]),
    "attn_int4qk_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int, _P, ctypes.c_int, _P,
                                       _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _SZ, _P]),
    "attn_int4qk_fwd_workspace_size": (_SZ, [_I32] * 7),
    "attn_kv_append_int4": (ctypes.c_int, [_P, ctypes.c_int, _I32, _I32, _I32, _I32, _P, _P, _I32, _I32, _P]),
    "attn_quantize_rows_hadamard": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I32, _I32, _P, _P, _P, _P]),
    "attn_int8_fwd_qfloat_hadamard": (ctypes.c_int, [_P, ctypes.c_int, _P, _P, _P, _P, ctypes.c_int, _P,
                                                     ctypes.c_int, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                                     _I32, _I32, _P, _SZ, _P]),
    "attn_kv_append": (ctypes.c_int, [_P, ctypes.c_int, _I32, _I32, _I32, _I32, _P, _P, _I32, _I32, _P]),
    "attn_int8_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int, _P, ctypes.c_int, _P,
                                     _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _SZ, _P]),
    "attn_int8_fwd_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int, _P, ctypes.c_int, _P,
                                             _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P]),
    "attn_int8_fwd_noalloc_max_scratch": (_SZ, []),
    "attn_int8_fwd_qfloat": (ctypes.c_int, [_P, ctypes.c_int, _P, _P, _P, _P, ctypes.c_int, _P,
                                            ctypes.c_int, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                            _I32, _I32, _P, _SZ, _P]),
    "attn_int8_fwd_index_softmax": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int, _P, ctypes.c_int,
                                                   _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                   ctypes.c_float, _P, _SZ, _P]),
    "attn_index_softmax_table": (ctypes.c_int, [_I32, ctypes.c_float, _P]),
    "attn_int8_fwd_workspace_size": (_SZ, [_I32] * 7),
    "attn_int8_fwd_schedule": (ctypes.c_int, [_I32] * 7 + [_P, _P]),
    "attn_int8_debug_logits": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                              _P, _P]),
    "attn_status_str": (ctypes.c_char_p, [ctypes.c_int]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libattn_int8.so is not built (%s); run "
                          "`python int8_quantized_flashattention_amd/build.py`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = _load()


class AttnError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s failed: %s (status %d)" % (fn, attn_status_str(status), status))
        self.status = status


def attn_status_str(status):
    return _lib.attn_status_str(int(status)).decode()


def _check(fn, status):
    if status != ATTN_OK:
        raise AttnError(fn, status)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t


def attn_quantize_rows(x, rows_per_scale=1, q=None, scales=None, stream=None):
    """Symmetric INT8 quantization of groups of `rows_per_scale` rows of x
    (fp16 or fp32, last axis = row). Returns (q int8 like x, scales fp32)."""
    _dev(x, "x")
    if x.dtype not in (torch.float16, torch.float32):
        raise TypeError("x must be float16 or float32")
    n_cols = x.shape[-1]
    n_rows = x.numel() // n_cols
    if q is None:
        q = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    if scales is None:
        n = n_rows // rows_per_scale if rows_per_scale > 0 else 0
        scales = torch.empty(max(n, 1), dtype=torch.float32, device=x.device)
    _dev(q, "q", torch.int8)
    _dev(scales, "scales", torch.float32)
    st = _lib.attn_quantize_rows(_ptr(x), ATTN_F16 if x.dtype == torch.float16 else ATTN_F32,
                                 n_rows, n_cols, rows_per_scale, _ptr(q), _ptr(scales), _stream(stream))
    _check("attn_quantize_rows", st)
    return q, scales


def attn_quantize_cols(x, rows_per_group, q=None, scales=None, stream=None):
    """Symmetric INT8 quantization with one scale per column of each group of
    `rows_per_group` rows of x (fp16 or fp32, last axis = columns), e.g. V
    [B,Hkv,Lkv,d] with rows_per_group = Lkv gives per-channel scales
    [B*Hkv*d]. Returns (q int8 like x, scales fp32)."""
    _dev(x, "x")
    if x.dtype not in (torch.float16, torch.float32):
        raise TypeError("x must be float16 or float32")
    n_cols = x.shape[-1]
    n_rows = x.numel() // n_cols
    if rows_per_group < 1 or n_rows % rows_per_group:
        raise ValueError("rows_per_group must divide the number of rows")
    n_groups = n_rows // rows_per_group
    if q is None:
        q = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty(n_groups * n_cols, dtype=torch.float32, device=x.device)
    _dev(q, "q", torch.int8)
    _dev(scales, "scales", torch.float32)
    st = _lib.attn_quantize_cols(_ptr(x), ATTN_F16 if x.dtype == torch.float16 else ATTN_F32, n_groups,
                                 rows_per_group, n_cols, _ptr(q), _ptr(scales), _stream(stream))
    _check("attn_quantize_cols", st)
    return q, scales


def attn_quantize_rows_int4(x, codes=True, packed=True, scales=None, stream=None):
    """Per-token 4-bit quantization of x (fp16/fp32, last axis = row). codes
    and packed: True (allocate), False (skip) or an output tensor. Returns
    (codes int8 like x or None, packed uint8 [..., d/2] or None, scales fp32
    [n_rows])."""
    _dev(x, "x")
    if x.dtype not in (torch.float16, torch.float32):
        raise TypeError("x must be float16 or float32")
    n_cols = x.shape[-1]
    n_rows = x.numel() // n_cols
    c = torch.empty(x.shape, dtype=torch.int8, device=x.device) if codes is True else codes
    p = torch.empty(tuple(x.shape[:-1]) + (n_cols // 2,), dtype=torch.uint8, device=x.device) \
        if packed is True else packed
    for t, n, dt in ((c, "codes", torch.int8), (p, "packed", torch.uint8)):
        if t is not None and t is not False:
            _dev(t, n, dt)
    c = c if c is not False else None
    p = p if p is not False else None
    if scales is None:
        scales = torch.empty(n_rows, dtype=torch.float32, device=x.device)
    _dev(scales, "scales", torch.float32)
    if scales.numel() != n_rows:
        raise ValueError("scales must hold one value per row")
    st = _lib.attn_quantize_rows_int4(_ptr(x), ATTN_F16 if x.dtype == torch.float16 else ATTN_F32, n_rows, n_cols,
                                      _ptr(c), _ptr(p), _ptr(scales), _stream(stream))
    _check("attn_quantize_rows_int4", st)
    return c, p, scales


def attn_quantize_rows_hadamard(x, bits=8, codes=True, packed=False, scales=None, stream=None):
    """Rows of x (fp16/fp32, last axis a power of two) rotated by the
    normalized Hadamard matrix, then per-token codes at 8 or 4 bits. codes /
    packed: True (allocate), False (skip) or an output tensor (packed only
    for bits 4). Returns (codes or None, packed or None, scales)."""
    _dev(x, "x")
    if x.dtype not in (torch.float16, torch.float32):
        raise TypeError("x must be float16 or float32")
    n_cols = x.shape[-1]
    n_rows = x.numel() // n_cols
    c = torch.empty(x.shape, dtype=torch.int8, device=x.device) if codes is True else codes
    p = torch.empty(tuple(x.shape[:-1]) + (n_cols // 2,), dtype=torch.uint8, device=x.device) \
        if packed is True else packed
    c = c if c is not False else None
    p = p if p is not False else None
    if c is not None:
        _dev(c, "codes", torch.int8)
    if p is not None:
        _dev(p, "packed", torch.uint8)
    if scales is None:
        scales = torch.empty(n_rows, dtype=torch.float32, device=x.device)
    _dev(scales, "scales", torch.float32)
    st = _lib.attn_quantize_rows_hadamard(_ptr(x), ATTN_F16 if x.dtype == torch.float16 else ATTN_F32, n_rows,
                                          n_cols, int(bits), _ptr(c), _ptr(p), _ptr(scales), _stream(stream))
    _check("attn_quantize_rows_hadamard", st)
    return c, p, scales


def attn_kv_append_int4(x, cache4, scales, pos, stream=None):
    """Per-token 4-bit codes of new tokens x [B,Hkv,T,d] (fp16/fp32) packed
    into rows pos .. pos+T-1 of cache4 [B,Hkv,L_max,d/2] (uint8) and scales
    [B,Hkv,L_max]."""
    _dev(x, "x")
    if x.dtype not in (torch.float16, torch.float32):
        raise TypeError("x must be float16 or float32")
    _dev(cache4, "cache4", torch.uint8)
    _dev(scales, "scales", torch.float32)
    B, Hkv, T, d = x.shape
    if cache4.dim() != 4 or tuple(cache4.shape[:2]) != (B, Hkv) or cache4.shape[3] != d // 2:
        raise ValueError("cache4 must be [B, Hkv, L_max, d/2] matching x")
    L_max = cache4.shape[2]
    if scales.numel() != B * Hkv * L_max:
        raise ValueError("scales must hold B * Hkv * L_max values")
    st = _lib.attn_kv_append_int4(_ptr(x), ATTN_F16 if x.dtype == torch.float16 else ATTN_F32, B, Hkv, T, d,
                                  _ptr(cache4), _ptr(scales), L_max, int(pos), _stream(stream))
    _check("attn_kv_append_int4", st)
    return cache4, scales


def attn_kv_append(x, cache, scales, pos, stream=None):
    """Per-token quantization of new tokens x [B,Hkv,T,d] (fp16/fp32) into rows
    pos .. pos+T-1 of the INT8 cache [B,Hkv,L_max,d] and its scales
    [B,Hkv,L_max]; the codes equal attn_quantize_rows(.., 1) of the same rows."""
    _dev(x, "x")
    if x.dtype not in (torch.float16, torch.float32):
        raise TypeError("x must be float16 or float32")
    _dev(cache, "cache", torch.int8)
    _dev(scales, "scales", torch.float32)
    B, Hkv, T, d = x.shape
    if cache.dim() != 4 or tuple(cache.shape[:2]) != (B, Hkv) or cache.shape[3] != d:
        raise ValueError("cache must be [B, Hkv, L_max, d] matching x")
    L_max = cache.shape[2]
    if scales.numel() != B * Hkv * L_max:
        raise ValueError("scales must hold B * Hkv * L_max values")
    st = _lib.attn_kv_append(_ptr(x), ATTN_F16 if x.dtype == torch.float16 else ATTN_F32, B, Hkv, T, d,
                             _ptr(cache), _ptr(scales), L_max, int(pos), _stream(stream))
    _check("attn_kv_append", st)
    return cache, scales


def attn_int8_fwd_workspace_size(B, H, Hkv, Lq, Lkv, d, causal):
    return int(_lib.attn_int8_fwd_workspace_size(B, H, Hkv, Lq, Lkv, d, int(causal)))


def attn_int8_fwd_schedule(B, H, Hkv, Lq, Lkv, d, causal):
    """(kv_tile, kv_split_len) the forward uses for this shape; 0 = no split."""
    t, s = ctypes.c_int32(), ctypes.c_int32()
    _check("attn_int8_fwd_schedule",
           _lib.attn_int8_fwd_schedule(B, H, Hkv, Lq, Lkv, d, int(causal), ctypes.byref(t),
                                       ctypes.byref(s)))
    return t.value, s.value


def _vmode(v_per_token):
    """V scale mode from False / True / "head" / "channel" (or 0 / 1 / 2 / 3)."""
    if isinstance(v_per_token, str):
        return {"tensor": ATTN_VSCALE_PER_TENSOR, "token": ATTN_VSCALE_PER_TOKEN,
                "head": ATTN_VSCALE_PER_HEAD, "channel": ATTN_VSCALE_PER_CHANNEL}[v_per_token]
    return int(v_per_token)


def _fwd_common(q, k, s_k, v, s_v, v_per_token, causal, o_dtype, return_lse, out, lse, workspace):
    """Shape checks and output / workspace allocation shared by both forwards."""
    for t, n in ((k, "k"), (v, "v")):
        _dev(t, n, torch.int8)
    for t, n in ((s_k, "s_k"), (s_v, "s_v")):
        _dev(t, n, torch.float32)
    B, H, Lq, d = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Lkv, d) or tuple(v.shape) != (B, Hkv, Lkv, d):
        raise ValueError("k and v must be [B, Hkv, Lkv, d] matching q")
    if s_k.numel() != B * Hkv * Lkv:
        raise ValueError("s_k size does not match k")
    mode = _vmode(v_per_token)
    if s_v.numel() != {ATTN_VSCALE_PER_TENSOR: 1, ATTN_VSCALE_PER_TOKEN: B * Hkv * Lkv,
                       ATTN_VSCALE_PER_HEAD: B * Hkv, ATTN_VSCALE_PER_CHANNEL: B * Hkv * d}.get(mode, -1):
        raise ValueError("s_v size does not match the V scale mode")
    if o_dtype not in (torch.float16, torch.float32):
        raise TypeError("o_dtype must be float16 or float32")
    if out is None:
        out = torch.empty((B, H, Lq, d), dtype=o_dtype, device=q.device)
    _dev(out, "out", o_dtype)
    if return_lse and lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32)
    if workspace is False:           # the no-allocation forward takes none
        return (B, H, Hkv, Lq, Lkv, d), out, lse, None, 0
    need = attn_int8_fwd_workspace_size(B, H, Hkv, Lq, Lkv, d, causal)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return (B, H, Hkv, Lq, Lkv, d), out, lse, workspace, ws_bytes


def attn_int8_fwd(q, s_q, k, s_k, v, s_v, v_per_token, causal, o_dtype=torch.float16,
                  return_lse=False, out=None, lse=None, workspace=None, stream=None):
    """Fused INT8 attention forward. q [B,H,Lq,d] int8, k/v [B,Hkv,Lkv,d] int8,
    s_q [B*H*Lq], s_k [B*Hkv*Lkv], s_v (fp32) [1] (v_per_token False),
    [B*Hkv*Lkv] (True), [B*Hkv] (v_per_token "head": one scale per (batch,
    kv head)) or [B*Hkv*d] ("channel": one per (batch, kv head, channel)).
    Returns O (and lse when return_lse)."""
    _dev(q, "q", torch.int8)
    _dev(s_q, "s_q", torch.float32)
    shape, out, lse, workspace, ws_bytes = _fwd_common(q, k, s_k, v, s_v, v_per_token, causal,
                                                       o_dtype, return_lse, out, lse, workspace)
    if s_q.numel() != shape[0] * shape[1] * shape[3]:
        raise ValueError("s_q size does not match q")
    st = _lib.attn_int8_fwd(_ptr(q), _ptr(s_q), _ptr(k), _ptr(s_k), _ptr(v), _ptr(s_v),
                            _vmode(v_per_token),
                            _ptr(out), ATTN_F16 if o_dtype == torch.float16 else ATTN_F32, _ptr(lse),
                            *shape, int(causal), _ptr(workspace), ws_bytes, _stream(stream))
    _check("attn_int8_fwd", st)
    return (out, lse) if return_lse else out


def attn_int8_fwd_noalloc(q, s_q, k, s_k, v, s_v, v_per_token, causal, o_dtype=torch.float16,
                          return_lse=False, out=None, lse=None, stream=None):
    """attn_int8_fwd without a workspace: decode-shaped problems keep their
    split-KV partials in the library's static per-GPU scratch, and the call
    allocates nothing in the library (pass `out` (and `lse`) to allocate
    nothing here either). Calls that overlap on one GPU race on that scratch.
    Returns O (and lse when return_lse)."""
    _dev(q, "q", torch.int8)
    _dev(s_q, "s_q", torch.float32)
    shape, out, lse, _, _ = _fwd_common(q, k, s_k, v, s_v, v_per_token, causal, o_dtype, return_lse, out, lse,
                                        workspace=False)
    if s_q.numel() != shape[0] * shape[1] * shape[3]:
        raise ValueError("s_q size does not match q")
    st = _lib.attn_int8_fwd_noalloc(_ptr(q), _ptr(s_q), _ptr(k), _ptr(s_k), _ptr(v), _ptr(s_v),
                                    _vmode(v_per_token), _ptr(out), ATTN_F16 if o_dtype == torch.float16 else ATTN_F32,
                                    _ptr(lse), *shape, int(causal), _stream(stream))
    _check("attn_int8_fwd_noalloc", st)
    return (out, lse) if return_lse else out


def attn_int8_fwd_noalloc_max_scratch():
    """Bytes of the per-GPU scratch of attn_int8_fwd_noalloc."""
    return int(_lib.attn_int8_fwd_noalloc_max_scratch())


def attn_int8_fwd_qfloat(q, k, s_k, v, s_v, v_per_token, causal, o_dtype=torch.float16,
                         return_lse=False, q_hat=None, s_q=None, out=None, lse=None, workspace=None,
                         stream=None, hadamard=False):
    """The forward with Q given in fp16/fp32 [B,H,Lq,d]: the kernels quantize
    each Q row per token themselves (the same codes and scales as
    attn_quantize_rows). q_hat (int8 like q) and s_q ([B*H*Lq] fp32), when
    given, receive them. hadamard=True rotates each Q row by the normalized
    Hadamard matrix first (attn_int8_fwd_qfloat_hadamard; K must carry the
    same rotation). Returns O (and lse when return_lse)."""
    _dev(q, "q")
    if q.dtype not in (torch.float16, torch.float32):
        raise TypeError("q must be float16 or float32")
    shape, out, lse, workspace, ws_bytes = _fwd_common(q, k, s_k, v, s_v, v_per_token, causal,
                                                       o_dtype, return_lse, out, lse, workspace)
    if q_hat is not None:
        _dev(q_hat, "q_hat", torch.int8)
        if tuple(q_hat.shape) != tuple(q.shape):
            raise ValueError("q_hat must have q's shape")
    if s_q is not None:
        _dev(s_q, "s_q", torch.float32)
        if s_q.numel() != shape[0] * shape[1] * shape[3]:
            raise ValueError("s_q size does not match q")
    fn = _lib.attn_int8_fwd_qfloat_hadamard if hadamard else _lib.attn_int8_fwd_qfloat
    st = fn(_ptr(q), ATTN_F16 if q.dtype == torch.float16 else ATTN_F32, _ptr(k), _ptr(s_k), _ptr(v), _ptr(s_v),
            _vmode(v_per_token), _ptr(out), ATTN_F16 if o_dtype == torch.float16 else ATTN_F32, _ptr(lse),
            _ptr(q_hat), _ptr(s_q), *shape, int(causal), _ptr(workspace), ws_bytes, _stream(stream))
    _check("attn_int8_fwd_qfloat_hadamard" if hadamard else "attn_int8_fwd_qfloat", st)
    return (out, lse) if return_lse else out


def attn_int8_fwd_index_softmax(q, s_q, k, s_k, v, s_v, v_per_token, causal, o_dtype=torch.float16,
                                lut_bits=5, clip=6.6, return_lse=False, out=None, lse=None, workspace=None,
                                stream=None):
    """The INT8 forward with IndexSoftmax (a 2^lut_bits-entry exponential
    table over distances clipped at `clip`) in place of the exp softmax.
    Arguments as attn_int8_fwd; V scales per tensor or per (batch, kv head)
    (v_per_token False or "head")."""
    _dev(q, "q", torch.int8)
    _dev(s_q, "s_q", torch.float32)
    shape, out, lse, workspace, ws_bytes = _fwd_common(q, k, s_k, v, s_v, v_per_token, causal,
                                                       o_dtype, return_lse, out, lse, workspace)
    if s_q.numel() != shape[0] * shape[1] * shape[3]:
        raise ValueError("s_q size does not match q")
    st = _lib.attn_int8_fwd_index_softmax(_ptr(q), _ptr(s_q), _ptr(k), _ptr(s_k), _ptr(v), _ptr(s_v),
                                          _vmode(v_per_token),
                                          _ptr(out), ATTN_F16 if o_dtype == torch.float16 else ATTN_F32,
                                          _ptr(lse), *shape, int(causal), int(lut_bits), float(clip),
                                          _ptr(workspace), ws_bytes, _stream(stream))
    _check("attn_int8_fwd_index_softmax", st)
    return (out, lse) if return_lse else out


def attn_index_softmax_table(lut_bits=5, clip=6.6):
    """The library's IndexSoftmax table (host bytes, 2^lut_bits entries)."""
    buf = (ctypes.c_uint8 * 256)()
    _check("attn_index_softmax_table", _lib.attn_index_softmax_table(int(lut_bits), float(clip), buf))
    return bytes(buf)[:1 << int(lut_bits)]


def attn_int4qk_fwd(q, s_q, k4, s_k, v, s_v, v_per_token, causal, o_dtype=torch.float16, return_lse=False,
                    out=None, lse=None, workspace=None, stream=None):
    """The forward with K in packed 4-bit codes k4 [B,Hkv,Lkv,d/2] (uint8;
    attn_quantize_rows_int4) and INT8 codes q. Other arguments as
    attn_int8_fwd."""
    _dev(q, "q", torch.int8)
    _dev(s_q, "s_q", torch.float32)
    _dev(k4, "k4", torch.uint8)
    _dev(v, "v", torch.int8)
    for t, n in ((s_k, "s_k"), (s_v, "s_v")):
        _dev(t, n, torch.float32)
    B, H, Lq, d = q.shape
    Hkv, Lkv = v.shape[1], v.shape[2]
    if tuple(k4.shape) != (B, Hkv, Lkv, d // 2) or tuple(v.shape) != (B, Hkv, Lkv, d):
        raise ValueError("k4 must be [B, Hkv, Lkv, d/2] and v [B, Hkv, Lkv, d], matching q")
    if s_q.numel() != B * H * Lq or s_k.numel() != B * Hkv * Lkv:
        raise ValueError("s_q / s_k sizes do not match q / k4")
    mode = _vmode(v_per_token)
    if s_v.numel() != {ATTN_VSCALE_PER_TENSOR: 1, ATTN_VSCALE_PER_TOKEN: B * Hkv * Lkv,
                       ATTN_VSCALE_PER_HEAD: B * Hkv, ATTN_VSCALE_PER_CHANNEL: B * Hkv * d}.get(mode, -1):
        raise ValueError("s_v size does not match the V scale mode")
    if o_dtype not in (torch.float16, torch.float32):
        raise TypeError("o_dtype must be float16 or float32")
    if out is None:
        out = torch.empty((B, H, Lq, d), dtype=o_dtype, device=q.device)
    _dev(out, "out", o_dtype)
    if return_lse and lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32)
    need = int(_lib.attn_int4qk_fwd_workspace_size(B, H, Hkv, Lq, Lkv, d, int(causal)))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.attn_int4qk_fwd(_ptr(q), _ptr(s_q), _ptr(k4), _ptr(s_k), _ptr(v), _ptr(s_v), mode, _ptr(out),
                              ATTN_F16 if o_dtype == torch.float16 else ATTN_F32, _ptr(lse), B, H, Hkv, Lq, Lkv, d,
                              int(causal), _ptr(workspace), ws_bytes, _stream(stream))
    _check("attn_int4qk_fwd", st)
    return (out, lse) if return_lse else out


def attn_int4qk_fwd_workspace_size(B, H, Hkv, Lq, Lkv, d, causal):
    return int(_lib.attn_int4qk_fwd_workspace_size(B, H, Hkv, Lq, Lkv, d, int(causal)))


def attn_int8_debug_logits(q, k, causal, out=None, stream=None):
    """INT32 logits of every visible pair from the prefill kernel's tile code;
    masked pairs keep out's previous contents (out defaults to zeros)."""
    _dev(q, "q", torch.int8)
    _dev(k, "k", torch.int8)
    B, H, Lq, d = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.zeros((B, H, Lq, Lkv), dtype=torch.int32, device=q.device)
    _dev(out, "out", torch.int32)
    st = _lib.attn_int8_debug_logits(_ptr(q), _ptr(k), B, H, Hkv, Lq, Lkv, d, int(causal), _ptr(out),
                                     _stream(stream))
    _check("attn_int8_debug_logits", st)
    return out


def int8_attention(q, k, v, causal, v_per_token=False, o_dtype=torch.float16, return_lse=False):
    """The whole path from fp16/fp32 Q, K, V: per-token quantization of K,
    per-tensor or per-token quantization of V, then the forward, which
    quantizes Q per token as it loads it."""
    d = q.shape[-1]
    kh, sk = attn_quantize_rows(k, 1)
    vh, sv = attn_quantize_rows(v, 1 if v_per_token else v.numel() // d)
    return attn_int8_fwd_qfloat(q, kh, sk, vh, sv, v_per_token, causal, o_dtype, return_lse)


__all__ = ["attn_quantize_rows", "attn_quantize_cols", "attn_quantize_rows_int4", "attn_kv_append",
           "attn_int4qk_fwd", "attn_int4qk_fwd_workspace_size", "attn_kv_append_int4", "attn_quantize_rows_hadamard", "attn_int8_fwd", "attn_int8_fwd_qfloat",
           "attn_int8_fwd_index_softmax", "attn_index_softmax_table", "attn_int8_fwd_workspace_size",
           "attn_int8_fwd_schedule", "attn_int8_debug_logits", "attn_status_str", "int8_attention",
           "AttnError", "LIB_PATH", "SIGNATURES"]
