"""Hadamard-rotated quantization ("incoherent processing", FlashAttention-3
page) on the GPU: the rotated codes and scales bit for bit against the
oracle (the fast transform's butterflies in one fixed order), the forwards on
rotated Q and K against the oracle on the same codes, and on the
outlier-channel configuration the rotated path's output closer to exact
attention than the unrotated one."""
import numpy as np
import pytest
import torch

import int4_format
import oracle
from gpu_parity import compare_o, dev, host, log, o_errors, quantize_both, quantize_cols_both
from workloads import WORKLOADS, gaussian

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import int8_quantized_flashattention_amd as m
    return m


def rotated_both(lib, x, bits=8):
    c, p, s = lib.attn_quantize_rows_hadamard(dev(x), bits, codes=True, packed=(bits == 4))
    qo, so = oracle.quantize_rows_hadamard(x, bits)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32)), "rotated scales differ"
    if not np.array_equal(host(c), qo):
        raise AssertionError("rotated codes differ at %s" % np.argwhere(host(c) != qo)[:5].tolist())
    if bits == 4:
        assert np.array_equal(host(p), int4_format.pack(qo))
    return qo, so, c, p, s


def run_rotated(lib, q, k, v, causal, vmode, odt, tag="", measure=None):
    """The rotated path on the GPU against the oracle: Q and K rotated and
    quantized (codes and scales bit-exact), V per tensor, token, head or
    channel; the forward on the rotated codes, and the forward that rotates
    and quantizes fp16/fp32 Q in its Q load, which must return the same codes,
    scales, O and lse bit for bit. measure: if a dict, the O and lse errors
    are stored in it instead of being asserted (the bit-exact checks still
    assert)."""
    B, H, Lq, d = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    log("[%s] B=%d H=%d Hkv=%d Lq=%d Lkv=%d d=%d causal=%d v=%s o=%s" % (tag, B, H, Hkv, Lq, Lkv, d, causal, vmode, odt))
    qh, sq, qd, _, sqd = rotated_both(lib, q)
    kh, sk, kd, _, skd = rotated_both(lib, k)
    if vmode == "channel":
        vh, sv, vd, svd = quantize_cols_both(lib, v, Lkv)
    else:
        vh, sv, vd, svd = quantize_both(lib, v, {"tensor": v.size // d, "token": 1, "head": Lkv}[vmode])
    vp = {"tensor": False, "token": True, "head": "head", "channel": "channel"}[vmode]
    tdt = torch.float16 if odt == "f16" else torch.float32
    o1, l1 = lib.attn_int8_fwd(qd, sqd, kd, skd, vd, svd, vp, causal, tdt, return_lse=True)
    qh2, sq2 = torch.empty_like(qd), torch.empty_like(sqd)
    o2, l2 = lib.attn_int8_fwd_qfloat(dev(q), kd, skd, vd, svd, vp, causal, tdt, return_lse=True,
                                      q_hat=qh2, s_q=sq2, hadamard=True)
    assert torch.equal(qh2, qd) and torch.equal(sq2.view(torch.int32), sqd.view(torch.int32)), "fused rotated Q codes"
    iv = torch.int16 if tdt == torch.float16 else torch.int32
    assert torch.equal(o2.view(iv), o1.view(iv)) and torch.equal(l2.view(torch.int32), l1.view(torch.int32)), \
        "fused rotated-Q forward differs"
    tile, split = lib.attn_int8_fwd_schedule(B, H, Hkv, Lq, Lkv, d, causal)
    mode = {"tensor": 0, "token": 1, "head": 2, "channel": 3}[vmode]
    oo, lo = oracle.attn_int8(qh, sq, kh, sk, vh, sv, mode, B, H, Hkv, Lq, Lkv, d, causal, tile, split)
    og, lg = host(o1).astype(np.float32).reshape(-1, d), host(l1).reshape(-1)
    lo = lo.reshape(-1)
    lse_err = float(np.max(np.abs(lg - lo) / np.maximum(1.0, np.abs(lo)))) if lo.size else 0.0
    if measure is not None:
        measure["max_abs"], measure["rel_fro"], measure["finite"] = o_errors(og, oo.reshape(-1, d))
        measure["lse_err"] = lse_err
        return
    compare_o(og, oo.reshape(-1, d), tag)
    assert lse_err <= 1e-4


@pytest.mark.parametrize("rows,cols,bits,dt", [(7, 64, 8, np.float16), (4096, 128, 8, np.float16),
                                               (3, 2048, 8, np.float32), (33, 8, 8, np.float32),
                                               (1000, 128, 4, np.float16), (65, 256, 4, np.float32)])
def test_rotated_quantizer_matches_oracle(lib, rows, cols, bits, dt):
    log("rotated quantize rows=%d cols=%d bits=%d %s" % (rows, cols, bits, np.dtype(dt).name))
    r = np.random.Generator(np.random.PCG64(rows + cols * 3 + bits))
    x = (r.standard_normal((rows, cols)) * r.uniform(0.01, 40.0, size=(rows, 1))).astype(dt)
    x[:, cols // 3] *= dt(20)
    x[min(1, rows - 1)] = 0
    rotated_both(lib, x, bits)


@pytest.mark.parametrize("B,H,Hkv,Lq,Lkv,d,causal,o", [
    (2, 4, 2, 77, 130, 128, 1, "f16"), (2, 8, 2, 1, 1500, 128, 0, "f32"), (1, 3, 3, 300, 300, 64, 1, "f32"),
])
def test_forward_on_rotated_codes(lib, B, H, Hkv, Lq, Lkv, d, causal, o):
    seed = B * 101 + Lq + Lkv
    q = gaussian((B, H, Lq, d), seed, np.float16)
    k = gaussian((B, Hkv, Lkv, d), seed + 1, np.float16)
    v = gaussian((B, Hkv, Lkv, d), seed + 2, np.float16)
    qh, sq, qd, _, sqd = rotated_both(lib, q)
    kh, sk, kd, _, skd = rotated_both(lib, k)
    vh, sv, vd, svd = quantize_both(lib, v, v.size // d)
    tdt = torch.float16 if o == "f16" else torch.float32
    og = lib.attn_int8_fwd(qd, sqd, kd, skd, vd, svd, False, causal, tdt)
    tile, split = lib.attn_int8_fwd_schedule(B, H, Hkv, Lq, Lkv, d, causal)
    oo, _ = oracle.attn_int8(qh, sq, kh, sk, vh, sv, 0, B, H, Hkv, Lq, Lkv, d, causal, tile, split)
    compare_o(host(og).astype(np.float32), oo, "rotated")


def test_rotation_reduces_error_with_outlier_channels(lib):
    # the outlier-channel configuration's first head group at L = 1024: the GPU
    # output on rotated Q, K is closer to exact attention than on unrotated
    w = WORKLOADS["l4096_outlier"]
    q, k, v = (x[:1, :4, :1024].copy() for x in w.inputs())
    B, H, L, d = q.shape
    exact = oracle.attn_ref_f64(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), B, H, H, L, L, d,
                                True)
    vd, svd = lib.attn_quantize_rows(dev(v), v.size // d)
    errs = {}
    for name in ("plain", "rotated"):
        if name == "plain":
            qd, sqd = lib.attn_quantize_rows(dev(q), 1)
            kd, skd = lib.attn_quantize_rows(dev(k), 1)
        else:
            qd, _, sqd = lib.attn_quantize_rows_hadamard(dev(q))
            kd, _, skd = lib.attn_quantize_rows_hadamard(dev(k))
        og = host(lib.attn_int8_fwd(qd, sqd, kd, skd, vd, svd, False, True, torch.float32))
        errs[name] = float(np.linalg.norm(og - exact) / np.linalg.norm(exact))
    log("relative error vs exact: %s" % errs)
    assert errs["rotated"] < 0.6 * errs["plain"]


@pytest.mark.parametrize("B,H,Hkv,Lq,Lkv,d,causal,qdt", [
    (2, 4, 2, 77, 130, 128, 1, np.float16), (1, 3, 3, 300, 300, 64, 0, np.float32),
    (2, 8, 2, 1, 1500, 128, 0, np.float16), (1, 8, 1, 2, 520, 64, 1, np.float32),
])
def test_fused_rotated_q_equals_separate(lib, B, H, Hkv, Lq, Lkv, d, causal, qdt):
    # Q rotated and quantized in the kernels' Q load: the rotated quantizer's
    # codes and scales, and O and lse bit for bit those of the forward fed with
    # them (prefill and split-KV decode shapes)
    seed = B * 313 + Lq + Lkv
    q = gaussian((B, H, Lq, d), seed, qdt)
    q[..., 3] *= qdt(20)
    k = gaussian((B, Hkv, Lkv, d), seed + 1, np.float16)
    v = gaussian((B, Hkv, Lkv, d), seed + 2, np.float16)
    qh, sq, qd, _, sqd = rotated_both(lib, q)
    kh, sk, kd, _, skd = rotated_both(lib, k)
    vh, sv, vd, svd = quantize_both(lib, v, v.size // d)
    o1, l1 = lib.attn_int8_fwd(qd, sqd, kd, skd, vd, svd, False, causal, torch.float32, return_lse=True)
    qh2, sq2 = torch.empty_like(qd), torch.empty_like(sqd)
    o2, l2 = lib.attn_int8_fwd_qfloat(dev(q), kd, skd, vd, svd, False, causal, torch.float32, return_lse=True,
                                      q_hat=qh2, s_q=sq2, hadamard=True)
    assert torch.equal(qh2, qd) and torch.equal(sq2.view(torch.int32), sqd.view(torch.int32))
    assert torch.equal(o2.view(torch.int32), o1.view(torch.int32))
    assert torch.equal(l2.view(torch.int32), l1.view(torch.int32))
    tile, split = lib.attn_int8_fwd_schedule(B, H, Hkv, Lq, Lkv, d, causal)
    oo, _ = oracle.attn_int8(qh, sq, kh, sk, vh, sv, 0, B, H, Hkv, Lq, Lkv, d, causal, tile, split)
    compare_o(host(o2), oo, "fused rotated Q")


@pytest.mark.parametrize("vmode", ["tensor", "token", "head", "channel"])
@pytest.mark.parametrize("B,H,Hkv,Lq,Lkv,d,causal,odt", [
    (2, 4, 2, 150, 333, 128, 1, "f16"), (2, 8, 2, 1, 2100, 64, 0, "f32")])
def test_rotated_path_every_v_mode(lib, B, H, Hkv, Lq, Lkv, d, causal, odt, vmode):
    # rotated Q and K with each V granularity, prefill and split-KV decode
    # shapes, one outlier channel in Q and K: codes bit-exact, the fused
    # rotated-Q forward bit-identical, O against the oracle
    seed = 17000 + Lq + Lkv
    q = gaussian((B, H, Lq, d), seed, np.float16, [5])
    k = gaussian((B, Hkv, Lkv, d), seed + 1, np.float16, [5])
    v = gaussian((B, Hkv, Lkv, d), seed + 2, np.float16)
    run_rotated(lib, q, k, v, causal, vmode, odt, tag="rot_%s" % vmode)
