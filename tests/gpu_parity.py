"""Helpers of the GPU parity tests: run one problem through the HIP path and
through the oracle on the same bytes, and compare.

Tolerance for O (fp32 or fp16 output): max-abs error <= 2e-2 and relative
Frobenius error <= 1e-2 against the oracle run with the GPU's KV schedule.
The quantized tensors, their scales and the INT32 logits must be bit-exact.
The forward that quantizes fp16/fp32 Q itself must return the quantizer's
codes and scales and the same O and lse, bit for bit, as the forward fed with
them.
"""
import sys

import numpy as np
import torch

import oracle

O_MAX_ABS = 2e-2
O_REL_FRO = 1e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def quantize_both(lib, x, rows_per_scale):
    """Quantize host array x on the GPU and with the oracle; assert bit-exact.
    Returns the (shared) host codes and scales plus the device copies."""
    qd, sd = lib.attn_quantize_rows(dev(x), rows_per_scale)
    qg, sg = host(qd), host(sd)
    qo, so = oracle.quantize_rows(x, rows_per_scale)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32)), "scales differ"
    if not np.array_equal(qg, qo):
        bad = np.argwhere(qg != qo)[:5]
        raise AssertionError("codes differ at %s" % bad.tolist())
    return qo, so, qd, sd


def quantize_cols_both(lib, x, rows_per_group):
    """Per-column quantization on the GPU and with the oracle; bit-exact."""
    qd, sd = lib.attn_quantize_cols(dev(x), rows_per_group)
    qg, sg = host(qd), host(sd)
    qo, so = oracle.quantize_cols(x, rows_per_group)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32)), "column scales differ"
    if not np.array_equal(qg, qo):
        bad = np.argwhere(qg != qo)[:5]
        raise AssertionError("column codes differ at %s" % bad.tolist())
    return qo, so, qd, sd


def o_errors(o_gpu, o_ref):
    """(max-abs error, relative Frobenius error, all finite) of o_gpu against o_ref."""
    o_gpu = np.asarray(o_gpu, np.float32)
    o_ref = np.asarray(o_ref, np.float32)
    assert o_gpu.shape == o_ref.shape
    finite = bool(np.all(np.isfinite(o_gpu)))
    diff = o_gpu.astype(np.float64) - o_ref.astype(np.float64)
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    den = float(np.linalg.norm(o_ref.astype(np.float64)))
    rel = float(np.linalg.norm(diff) / den) if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel, finite


def compare_o(o_gpu, o_ref, what=""):
    max_abs, rel, finite = o_errors(o_gpu, o_ref)
    assert finite, "non-finite output " + what
    log("  %s max_abs=%.3e rel_fro=%.3e" % (what, max_abs, rel))
    assert max_abs <= O_MAX_ABS and rel <= O_REL_FRO, (what, max_abs, rel)
    return max_abs, rel


def quantize_subset(lib, x, batches):
    """Per-token quantization on the GPU over all of x; the oracle quantizes the
    selected batch entries, which must match bit for bit."""
    qd, sd = lib.attn_quantize_rows(dev(x), 1)
    qo, so = oracle.quantize_rows(np.ascontiguousarray(x[batches]), 1)
    qg = host(qd)[batches]
    sg = host(sd).reshape(x.shape[:-1])[batches].reshape(-1)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32)), "scales differ"
    assert np.array_equal(qg, qo), "codes differ"
    return qo, so, qd, sd


def run_problem(lib, q, k, v, causal, v_per_token, o_dtype, rows=None, check_lse=True, tag="",
                batches=None, measure=None):
    """Full path on the GPU vs the oracle. q/k/v are host fp16/fp32 arrays.
    rows: optional flat row ids to compare (default: every row).
    batches: optional batch indices; the oracle then quantizes and attends only
    those entries (per-token V only, where batch entries are independent).
    measure: if a dict, the O and lse errors are stored in it instead of being
    asserted against the tolerance (the bit-exact checks still assert)."""
    B, H, Lq, d = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    # V scales: "head" one per (batch, kv head), "channel" one per (batch, kv
    # head, channel), else a truth value: per token / per tensor
    v_per_token = v_per_token if isinstance(v_per_token, str) and v_per_token in ("head", "channel") \
        else bool(v_per_token)
    log("[%s] B=%d H=%d Hkv=%d Lq=%d Lkv=%d d=%d causal=%d vpt=%s o=%s" %
        (tag, B, H, Hkv, Lq, Lkv, d, causal, v_per_token, o_dtype))
    if batches is None:
        qh, sq, qd, sqd = quantize_both(lib, q, 1)
        kh, sk, kd, skd = quantize_both(lib, k, 1)
        if v_per_token == "channel":
            vh, sv, vd, svd = quantize_cols_both(lib, v, Lkv)
        else:
            vh, sv, vd, svd = quantize_both(lib, v, 1 if v_per_token is True else
                                            Lkv if v_per_token == "head" else v.size // d)
    else:
        assert v_per_token is True and rows is None
        batches = np.asarray(batches)
        qh, sq, qd, sqd = quantize_subset(lib, q, batches)
        kh, sk, kd, skd = quantize_subset(lib, k, batches)
        vh, sv, vd, svd = quantize_subset(lib, v, batches)
    tdt = torch.float16 if o_dtype == "f16" else torch.float32
    o, lse = lib.attn_int8_fwd(qd, sqd, kd, skd, vd, svd, v_per_token, causal, tdt, return_lse=True)
    # the same problem with Q given in floating point (quantized in the kernel)
    qh2 = torch.empty_like(qd)
    sq2 = torch.empty_like(sqd)
    o2, lse2 = lib.attn_int8_fwd_qfloat(dev(q), kd, skd, vd, svd, v_per_token, causal, tdt,
                                        return_lse=True, q_hat=qh2, s_q=sq2)
    assert torch.equal(qh2, qd), "fused Q codes differ from the quantizer's"
    assert torch.equal(sq2.view(torch.int32), sqd.view(torch.int32)), "fused s_Q differs"
    assert torch.equal(o2.view(torch.int16 if tdt == torch.float16 else torch.int32),
                       o.view(torch.int16 if tdt == torch.float16 else torch.int32)), "fused-Q O differs"
    assert torch.equal(lse2.view(torch.int32), lse.view(torch.int32)), "fused-Q lse differs"
    del o2, lse2, qh2, sq2
    og = host(o).astype(np.float32)
    lg = host(lse)
    tile, split = lib.attn_int8_fwd_schedule(B, H, Hkv, Lq, Lkv, d, causal)
    if batches is not None:
        og, lg, B = og[batches], lg[batches], len(batches)
    mode = {"head": 2, "channel": 3}.get(v_per_token, None) if isinstance(v_per_token, str) else int(v_per_token)
    oo, lo = oracle.attn_int8(qh, sq, kh, sk, vh, sv, mode, B, H, Hkv, Lq, Lkv, d, causal,
                              tile, split, rows=rows)
    og_sel = og if rows is None else og.reshape(-1, d)[rows]
    lg_sel = lg.reshape(-1) if rows is None else lg.reshape(-1)[rows]
    lo_f = lo.reshape(-1)
    lse_err = float((np.abs(lg_sel - lo_f) / np.maximum(1.0, np.abs(lo_f))).max()) if lo_f.size else 0.0
    if measure is not None:
        measure["max_abs"], measure["rel_fro"], measure["finite"] = o_errors(og_sel, oo)
        measure["lse_err"] = lse_err
        return og, oo
    compare_o(og_sel, oo, tag)
    if check_lse:
        assert lse_err <= 1e-4, ("lse", lse_err)
    return og, oo
