"""The C-ABI library loads, exports every function include/attn_int8.h declares,
and rejects every invalid request on the host before any launch (no GPU needed:
the rejected calls never reach the HIP runtime, so fake addresses are safe)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_int8.h")

import int8_quantized_flashattention_amd as m  # noqa: E402

OK, INVALID, UNSUPPORTED = m.ATTN_OK, m.ATTN_ERR_INVALID_ARG, m.ATTN_ERR_UNSUPPORTED
L = m._lib
A = 0x100000  # a 256-byte aligned fake device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(m.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(m.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for s in (OK, INVALID, UNSUPPORTED, m.ATTN_ERR_HIP):
        assert m.attn_status_str(s) and m.attn_status_str(s) != "unknown status"
    assert m.attn_status_str(99) == "unknown status"


def fwd(**kw):
    args = dict(q=A, s_q=A, k=A, s_k=A, v=A, s_v=A, v_mode=0, o=A, o_dt=1, lse=None, B=1, H=2, Hkv=1,
                Lq=8, Lkv=8, d=64, causal=0, ws=None, ws_bytes=0, stream=None)
    args.update(kw)
    p = lambda x: ctypes.c_void_p(x) if x is not None else None
    return L.attn_int8_fwd(p(args["q"]), p(args["s_q"]), p(args["k"]), p(args["s_k"]), p(args["v"]),
                           p(args["s_v"]), args["v_mode"], p(args["o"]), args["o_dt"], p(args["lse"]),
                           args["B"], args["H"], args["Hkv"], args["Lq"], args["Lkv"], args["d"],
                           args["causal"], p(args["ws"]), args["ws_bytes"], p(args["stream"]))


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(s_q=None), INVALID), (dict(k=None), INVALID),
    (dict(s_k=None), INVALID), (dict(v=None), INVALID), (dict(s_v=None), INVALID),
    (dict(o=None), INVALID),
    (dict(v_mode=4), INVALID), (dict(o_dt=5), INVALID),
    (dict(B=0), INVALID), (dict(H=0), INVALID), (dict(Hkv=0), INVALID), (dict(Lq=0), INVALID),
    (dict(Lkv=-3), INVALID), (dict(d=0), INVALID),
    (dict(H=3, Hkv=2), INVALID), (dict(causal=2), INVALID), (dict(causal=1, Lq=9, Lkv=8), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(q=A + 8), INVALID), (dict(k=A + 4), INVALID), (dict(v=A + 1), INVALID),
    (dict(o=A + 2), INVALID), (dict(s_q=A + 2), INVALID), (dict(lse=A + 1), INVALID),
    (dict(B=1024, H=64, Hkv=64, Lq=4096, Lkv=4096, d=128), UNSUPPORTED),
])
def test_fwd_rejects_before_launch(kw, expect):
    assert fwd(**kw) == expect


def fwdq(**kw):
    args = dict(q=A, q_dt=1, k=A, s_k=A, v=A, s_v=A, v_mode=0, o=A, o_dt=1, lse=None, q_hat=None,
                s_q=None, B=1, H=2, Hkv=1, Lq=8, Lkv=8, d=64, causal=0, ws=None, ws_bytes=0)
    args.update(kw)
    p = lambda x: ctypes.c_void_p(x) if x is not None else None
    return L.attn_int8_fwd_qfloat(p(args["q"]), args["q_dt"], p(args["k"]), p(args["s_k"]),
                                  p(args["v"]), p(args["s_v"]), args["v_mode"], p(args["o"]),
                                  args["o_dt"], p(args["lse"]), p(args["q_hat"]), p(args["s_q"]),
                                  args["B"], args["H"], args["Hkv"], args["Lq"], args["Lkv"],
                                  args["d"], args["causal"], p(args["ws"]), args["ws_bytes"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(q_dt=4), INVALID), (dict(k=None), INVALID),
    (dict(s_v=None), INVALID), (dict(o=None), INVALID), (dict(v_mode=4), INVALID),
    (dict(q=A + 8), INVALID), (dict(q_hat=A + 4), INVALID), (dict(s_q=A + 2), INVALID),
    (dict(H=3, Hkv=2), INVALID), (dict(causal=1, Lq=9, Lkv=8), INVALID), (dict(d=32), UNSUPPORTED),
    (dict(B=1, H=2, Hkv=1, Lq=1, Lkv=4096), INVALID),   # decode schedule needs a workspace
])
def test_fwd_qfloat_rejects_before_launch(kw, expect):
    assert fwdq(**kw) == expect


def fwdlut(**kw):
    args = dict(q=A, s_q=A, k=A, s_k=A, v=A, s_v=A, v_mode=0, o=A, o_dt=1, lse=None, B=1, H=2, Hkv=1,
                Lq=8, Lkv=8, d=64, causal=0, bits=5, clip=6.6, ws=None, ws_bytes=0)
    args.update(kw)
    p = lambda x: ctypes.c_void_p(x) if x is not None else None
    return L.attn_int8_fwd_index_softmax(p(args["q"]), p(args["s_q"]), p(args["k"]), p(args["s_k"]),
                                         p(args["v"]), p(args["s_v"]), args["v_mode"], p(args["o"]),
                                         args["o_dt"], p(args["lse"]), args["B"], args["H"], args["Hkv"],
                                         args["Lq"], args["Lkv"], args["d"], args["causal"], args["bits"],
                                         args["clip"], p(args["ws"]), args["ws_bytes"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(s_q=None), INVALID), (dict(s_v=None), INVALID), (dict(o=None), INVALID),
    (dict(bits=0), INVALID), (dict(bits=9), INVALID), (dict(bits=-1), INVALID),
    (dict(clip=0.0), INVALID), (dict(clip=-1.0), INVALID), (dict(clip=float("inf")), INVALID),
    (dict(clip=float("nan")), INVALID), (dict(clip=5e-4), INVALID), (dict(clip=2e3), INVALID),
    (dict(v_mode=1), UNSUPPORTED), (dict(v_mode=4), INVALID), (dict(o_dt=5), INVALID),
    (dict(H=3, Hkv=2), INVALID), (dict(causal=1, Lq=9, Lkv=8), INVALID), (dict(d=96), UNSUPPORTED),
    (dict(q=A + 8), INVALID), (dict(o=A + 2), INVALID),
    (dict(B=1, H=2, Hkv=1, Lq=1, Lkv=4096), INVALID),   # decode schedule needs a workspace
])
def test_fwd_index_softmax_rejects_before_launch(kw, expect):
    assert fwdlut(**kw) == expect


def test_index_softmax_table_query():
    import oracle
    for bits, clip in ((5, 6.6), (1, 1e-3), (8, 1e3), (3, 2.0)):
        got = m.attn_index_softmax_table(bits, clip)
        assert list(got) == list(oracle.index_softmax_lut(bits, float(np.float32(clip))))
    buf = (ctypes.c_uint8 * 256)()
    assert L.attn_index_softmax_table(0, 6.6, buf) == INVALID
    assert L.attn_index_softmax_table(5, 0.0, buf) == INVALID
    assert L.attn_index_softmax_table(5, 6.6, None) == INVALID


def test_kv_append_rejects_before_launch():
    p = ctypes.c_void_p
    f = lambda **kw: L.attn_kv_append(
        p(kw.get("x", A)), kw.get("dt", 1), kw.get("B", 2), kw.get("Hkv", 2), kw.get("T", 1),
        kw.get("d", 128), p(kw.get("c", A)), p(kw.get("s", A)), kw.get("L", 16), kw.get("pos", 15), None)
    assert f(x=None) == INVALID
    assert f(c=None) == INVALID
    assert f(s=None) == INVALID
    assert f(dt=3) == INVALID
    assert f(T=0) == INVALID
    assert f(pos=-1) == INVALID
    assert f(pos=16) == INVALID            # pos + T > L_max
    assert f(T=2, pos=15) == INVALID
    assert f(d=60) == UNSUPPORTED          # not a multiple of 8
    assert f(d=4096) == UNSUPPORTED        # wider than one team handles
    assert f(B=4096, Hkv=64, L=8192) == UNSUPPORTED
    assert f(x=A + 8) == INVALID
    assert f(c=A + 4) == INVALID
    assert f(s=A + 2) == INVALID


def test_quantize_rejects_before_launch():
    p = ctypes.c_void_p
    q = lambda **kw: L.attn_quantize_rows(
        p(kw.get("x", A)), kw.get("dt", 1), kw.get("n_rows", 16), kw.get("n_cols", 64),
        kw.get("rps", 1), p(kw.get("q", A)), p(kw.get("s", A)), None)
    assert q(x=None) == INVALID
    assert q(q=None) == INVALID
    assert q(s=None) == INVALID
    assert q(dt=7) == INVALID
    assert q(n_rows=0) == INVALID
    assert q(n_cols=0) == INVALID
    assert q(rps=0) == INVALID
    assert q(rps=5) == INVALID          # 16 rows not divisible by 5
    assert q(n_cols=60) == UNSUPPORTED  # not a multiple of 8
    assert q(x=A + 8) == INVALID
    assert q(q=A + 4) == INVALID
    assert q(s=A + 2) == INVALID


def test_quantize_cols_rejects_before_launch():
    p = ctypes.c_void_p
    q = lambda **kw: L.attn_quantize_cols(
        p(kw.get("x", A)), kw.get("dt", 1), kw.get("g", 4), kw.get("rows", 16), kw.get("n_cols", 64),
        p(kw.get("q", A)), p(kw.get("s", A)), None)
    assert q(x=None) == INVALID
    assert q(q=None) == INVALID
    assert q(s=None) == INVALID
    assert q(dt=7) == INVALID
    assert q(g=0) == INVALID
    assert q(rows=0) == INVALID
    assert q(n_cols=0) == INVALID
    assert q(n_cols=60) == UNSUPPORTED            # not a multiple of 8
    assert q(n_cols=4096) == UNSUPPORTED          # wider than one workgroup's columns
    assert q(g=1 << 21, n_cols=2048) == UNSUPPORTED   # 2^32 scales
    assert q(g=1 << 40, rows=1 << 30) == INVALID  # element count overflows
    assert q(x=A + 8) == INVALID
    assert q(q=A + 4) == INVALID
    assert q(s=A + 2) == INVALID


def test_int4_entry_points_reject_before_launch():
    p = ctypes.c_void_p
    q4 = lambda **kw: L.attn_quantize_rows_int4(
        p(kw.get("x", A)), kw.get("dt", 1), kw.get("n_rows", 16), kw.get("n_cols", 64), p(kw.get("c", A)),
        p(kw.get("pk", A)), p(kw.get("s", A)), None)
    assert q4(x=None) == INVALID and q4(s=None) == INVALID and q4(c=None, pk=None) == INVALID
    assert q4(dt=5) == INVALID and q4(n_rows=0) == INVALID and q4(n_cols=0) == INVALID
    assert q4(n_cols=60) == UNSUPPORTED and q4(n_cols=4096) == UNSUPPORTED
    assert q4(x=A + 8) == INVALID and q4(c=A + 4) == INVALID and q4(pk=A + 2) == INVALID and q4(s=A + 2) == INVALID
    ap = lambda **kw: L.attn_kv_append_int4(
        p(kw.get("x", A)), kw.get("dt", 1), kw.get("B", 2), kw.get("Hkv", 2), kw.get("T", 1), kw.get("d", 128),
        p(kw.get("c", A)), p(kw.get("s", A)), kw.get("L", 16), kw.get("pos", 15), None)
    assert ap(x=None) == INVALID and ap(c=None) == INVALID and ap(pos=16) == INVALID and ap(T=0) == INVALID
    assert ap(d=60) == UNSUPPORTED and ap(B=4096, Hkv=64, L=8192) == UNSUPPORTED
    assert ap(c=A + 2) == INVALID and ap(x=A + 8) == INVALID
    f = lambda **kw: L.attn_int4qk_fwd(
        p(kw.get("q", A)), p(kw.get("sq", A)), p(kw.get("k", A)), p(kw.get("sk", A)), p(kw.get("v", A)),
        p(kw.get("sv", A)), kw.get("vm", 0), p(kw.get("o", A)), kw.get("odt", 1), None, kw.get("B", 1),
        kw.get("H", 2), kw.get("Hkv", 1), kw.get("Lq", 8), kw.get("Lkv", 8), kw.get("d", 64), kw.get("causal", 0),
        p(kw.get("ws", None)), kw.get("wsb", 0), None)
    for kw in (dict(q=None), dict(k=None), dict(sv=None), dict(o=None), dict(vm=4), dict(odt=3), dict(H=3, Hkv=2),
               dict(causal=1, Lq=9, Lkv=8), dict(k=A + 8), dict(q=A + 4), dict(sk=A + 2)):
        assert f(**kw) == INVALID, kw
    assert f(d=96) == UNSUPPORTED
    # decode shape without its workspace; prefill shape without room for the widened K
    assert f(B=1, H=2, Hkv=1, Lq=1, Lkv=4096) == INVALID
    assert f(B=1, H=1, Hkv=1, Lq=64, Lkv=64) == INVALID
    assert f(B=1, H=1, Hkv=1, Lq=64, Lkv=64, ws=A, wsb=64 * 64 - 256) == INVALID
    assert m.attn_int4qk_fwd_workspace_size(1, 1, 1, 64, 64, 64, 0) == 64 * 64
    assert m.attn_int4qk_fwd_workspace_size(2, 8, 2, 1, 700, 128, 0) == \
        m.attn_int8_fwd_workspace_size(2, 8, 2, 1, 700, 128, 0) > 0


def test_fwd_qfloat_hadamard_rejects_before_launch():
    p = ctypes.c_void_p
    f = lambda **kw: L.attn_int8_fwd_qfloat_hadamard(
        p(kw.get("q", A)), kw.get("qdt", 1), p(A), p(A), p(A), p(A), kw.get("vm", 0), p(kw.get("o", A)), 1, None,
        None, None, 1, 2, 1, kw.get("Lq", 8), kw.get("Lkv", 8), kw.get("d", 64), 0, None, 0, None)
    assert f(q=None) == INVALID and f(qdt=3) == INVALID and f(o=None) == INVALID and f(vm=4) == INVALID
    assert f(d=96) == UNSUPPORTED and f(q=A + 8) == INVALID
    assert f() == INVALID                            # decode shape without its workspace


def test_quantize_hadamard_rejects_before_launch():
    p = ctypes.c_void_p
    f = lambda **kw: L.attn_quantize_rows_hadamard(
        p(kw.get("x", A)), kw.get("dt", 1), kw.get("n_rows", 16), kw.get("n_cols", 128), kw.get("bits", 8),
        p(kw.get("c", A)), p(kw.get("pk", None)), p(kw.get("s", A)), None)
    assert f(x=None) == INVALID and f(s=None) == INVALID and f(dt=4) == INVALID
    assert f(c=None) == INVALID                      # bits 8 needs codes
    assert f(pk=A) == INVALID                        # bits 8 has no packed form
    assert f(bits=4, c=None) == INVALID              # bits 4 needs codes or packed
    assert f(bits=5) == INVALID and f(n_rows=0) == INVALID and f(n_cols=0) == INVALID
    assert f(n_cols=96) == UNSUPPORTED and f(n_cols=4) == UNSUPPORTED and f(n_cols=4096) == UNSUPPORTED
    assert f(x=A + 8) == INVALID and f(c=A + 4) == INVALID and f(s=A + 2) == INVALID
    assert f(bits=4, pk=A + 2) == INVALID


def test_debug_logits_rejects_before_launch():
    p = ctypes.c_void_p
    f = lambda **kw: L.attn_int8_debug_logits(
        p(kw.get("q", A)), p(kw.get("k", A)), kw.get("B", 1), kw.get("H", 1), kw.get("Hkv", 1),
        kw.get("Lq", 8), kw.get("Lkv", 8), kw.get("d", 64), kw.get("causal", 0),
        p(kw.get("s", A)), None)
    assert f(q=None) == INVALID
    assert f(s=None) == INVALID
    assert f(d=32) == UNSUPPORTED
    assert f(causal=1, Lq=9) == INVALID
    assert f(s=A + 4) == INVALID
    assert f(B=64, H=64, Hkv=64, Lq=1024, Lkv=1024) == UNSUPPORTED


def test_schedule_and_workspace_queries():
    t, s = m.attn_int8_fwd_schedule(4, 32, 32, 4096, 4096, 128, 1)
    assert t > 0 and t % 32 == 0 and s >= 0 and (s == 0 or s % t == 0)
    assert m.attn_int8_fwd_workspace_size(1, 3, 2, 8, 8, 64, 0) == 0   # invalid -> 0
    with pytest.raises(m.AttnError):
        m.attn_int8_fwd_schedule(1, 1, 1, 8, 8, 48, 0)
    assert L.attn_int8_fwd_schedule(1, 1, 1, 8, 8, 64, 0, None, None) == INVALID


PROBE_HEADER = os.path.join(ROOT, "include", "attn_probes.h")
PROBE_LIB = os.path.join(ROOT, "int8_quantized_flashattention_amd", "libattn_probes.so")


def test_probe_library_exports_and_rejects_bad_arguments():
    # the benchmark's measurement kernels (include/attn_probes.h): every
    # declared symbol is exported, and invalid arguments return 1 before any
    # launch
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(attn_probe_[a-z0-9_]+)\s*\(", text)))
    assert names == ["attn_probe_hbm_read", "attn_probe_lds_patterns", "attn_probe_mfma_i8"]
    lib = ctypes.CDLL(PROBE_LIB)
    for n in names:
        assert hasattr(lib, n), n
    lib.attn_probe_mfma_i8.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p]
    assert lib.attn_probe_mfma_i8(0, 10, A, None) == 1
    assert lib.attn_probe_mfma_i8(4, 0, A, None) == 1
    assert lib.attn_probe_mfma_i8(4, 10, None, None) == 1
    assert lib.attn_probe_hbm_read(A, 1 << 20, 8, 0, None, None) == 1
    assert lib.attn_probe_hbm_read(A, 100, 8, 0, A, None) == 1          # not a multiple of 16
    assert lib.attn_probe_hbm_read(A + 4, 1 << 20, 8, 1, A, None) == 1  # misaligned source
    assert lib.attn_probe_hbm_read(A, 1 << 20, 0, 0, A, None) == 1
    lib.attn_probe_lds_patterns.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_void_p]
    assert lib.attn_probe_lds_patterns(4, A, 8, 10, A, None) == 1       # no such pattern
    assert lib.attn_probe_lds_patterns(-1, A, 8, 10, A, None) == 1
    assert lib.attn_probe_lds_patterns(0, None, 8, 10, A, None) == 1
    assert lib.attn_probe_lds_patterns(3, A + 8, 8, 10, A, None) == 1   # misaligned source
    assert lib.attn_probe_lds_patterns(1, A, 0, 10, A, None) == 1
    assert lib.attn_probe_lds_patterns(2, A, 8, 0, A, None) == 1
    assert lib.attn_probe_lds_patterns(2, A, 8, 10, None, None) == 1


def test_noalloc_forward_rejects_before_any_hip_call():
    # arguments are checked before the per-GPU scratch is looked up, so these
    # return their status with no HIP call at all (this host has no GPU)
    f = L.attn_int8_fwd_noalloc
    args = [A, A, A, A, A, A, 0, A, 1, None, 1, 2, 1, 8, 8, 64, 0, None]
    bad = list(args)
    bad[0] = None                                   # q
    assert f(*bad) == INVALID
    bad = list(args)
    bad[15] = 96                                    # d
    assert f(*bad) == UNSUPPORTED
    bad = list(args)
    bad[9] = A + 2                                  # misaligned lse
    assert f(*bad) == INVALID
    # a decode shape whose split-KV partials exceed the scratch
    big = [A, A, A, A, A, A, 1, A, 1, None, 4096, 16, 16, 1, 8, 128, 0, None]
    assert m.attn_int8_fwd_workspace_size(4096, 16, 16, 1, 8, 128, 0) > L.attn_int8_fwd_noalloc_max_scratch()
    assert f(*big) == UNSUPPORTED
    assert L.attn_int8_fwd_noalloc_max_scratch() == 32 << 20
