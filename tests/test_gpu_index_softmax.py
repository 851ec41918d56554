"""IndexSoftmax forward (IntAttention §3.1-3.2: clipped distance, 2^b-entry
exponential table, integer row sum) on the GPU vs the oracle's IndexSoftmax
mode, run with the GPU's KV schedule on the same quantized bytes.

Bar: O within the path's tolerance (max-abs 2e-2, relative Frobenius 1e-2).
The table indices are the same fp32 operations on both sides (u = S_int s_K,
the running max of u, one fma, floor), so the codes agree and only the
rescale factors and sums round differently: O is also held to relative
Frobenius 2e-5 (fp32 out) or 1e-3 (fp16 out), and lse to 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_parity import compare_o, host, log, o_errors, quantize_both, quantize_cols_both
from workloads import WORKLOADS, gaussian

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import int8_quantized_flashattention_amd as m
    return m


def run_lut(lib, q, k, v, causal, vmode, odt, bits, clip, rows=None, tag="", measure=None):
    """IndexSoftmax forward on the GPU against the oracle with the same table
    and schedule. measure: if a dict, the errors are stored in it (max_abs,
    rel_fro, finite, lse_err, and strict: relative Frobenius within 2e-5 for
    fp32 O, 1e-3 for fp16) instead of being asserted."""
    B, H, Lq, d = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    c32 = float(np.float32(clip))
    log("[%s] B=%d H=%d Hkv=%d Lq=%d Lkv=%d d=%d causal=%d v=%s o=%s b=%d c=%g" %
        (tag, B, H, Hkv, Lq, Lkv, d, causal, vmode, odt, bits, c32))
    qh, sq, qd, sqd = quantize_both(lib, q, 1)
    kh, sk, kd, skd = quantize_both(lib, k, 1)
    if vmode == "channel":
        vh, sv, vd, svd = quantize_cols_both(lib, v, Lkv)
    else:
        vh, sv, vd, svd = quantize_both(lib, v, Lkv if vmode == "head" else v.size // d)
    tdt = torch.float16 if odt == "f16" else torch.float32
    o, lse = lib.attn_int8_fwd_index_softmax(qd, sqd, kd, skd, vd, svd, vmode, causal, tdt, bits, c32,
                                             return_lse=True)
    og, lg = host(o).astype(np.float32), host(lse)
    tile, split = lib.attn_int8_fwd_schedule(B, H, Hkv, Lq, Lkv, d, causal)
    mode = {"tensor": 0, "head": 2, "channel": 3}[vmode]
    oo, lo = oracle.attn_int8(qh, sq, kh, sk, vh, sv, mode, B, H, Hkv, Lq, Lkv, d, causal, tile, split, rows=rows,
                              index_softmax=(bits, c32))
    og = og.reshape(-1, d) if rows is None else og.reshape(-1, d)[rows]
    lg = lg.reshape(-1) if rows is None else lg.reshape(-1)[rows]
    oo = oo.reshape(-1, d)
    if measure is not None:
        measure["max_abs"], measure["rel_fro"], measure["finite"] = o_errors(og, oo)
        measure["strict"] = measure["rel_fro"] <= (1e-3 if odt == "f16" else 2e-5)
        lo_ = lo.reshape(-1)
        measure["lse_err"] = float(np.max(np.abs(lg - lo_) / np.maximum(1.0, np.abs(lo_)))) if lo_.size else 0.0
        return
    _, rel = compare_o(og, oo, tag)
    assert rel <= (1e-3 if odt == "f16" else 2e-5), ("codes differ?", rel)
    lo = lo.reshape(-1)
    assert float(np.max(np.abs(lg - lo) / np.maximum(1.0, np.abs(lo)))) <= 1e-5


@pytest.mark.parametrize("bits,clip", [(5, 6.6), (3, 2.0), (8, 7.7)])
def test_small_workload_all_rows(lib, bits, clip):
    w = WORKLOADS["l1024_causal"]
    q, k, v = w.inputs()
    run_lut(lib, q, k, v, w.causal, "tensor", "f32", bits, clip, tag="l1024_causal")


def test_full_size_workload_sampled_rows(lib):
    # the configuration the benchmark times (B4 H32 L4096 d128 causal, outlier
    # channels), every head's first and last rows plus a seeded sample
    w = WORKLOADS["l4096_outlier"]
    q, k, v = w.inputs()
    r = np.random.Generator(np.random.PCG64(5))
    rows = []
    for bh in np.unique(np.concatenate([[0, w.B * w.H - 1], r.choice(w.B * w.H, 4, replace=False)])):
        ids = np.unique(np.concatenate([np.arange(16), np.arange(w.Lq - 64, w.Lq),
                                        r.choice(w.Lq, 256, replace=False)]))
        rows.append(bh * w.Lq + ids)
    rows = np.concatenate(rows).astype(np.int64)
    run_lut(lib, q, k, v, w.causal, "tensor", w.o_dtype, 5, 6.6, rows=rows, tag="l4096_outlier")


SWEEP = [  # B, H, Hkv, Lq, Lkv, d, causal, V scale, o, b, c
    (1, 1, 1, 128, 128, 64, 0, "tensor", "f32", 5, 6.6), (2, 4, 2, 77, 130, 128, 1, "tensor", "f16", 5, 6.6),
    (1, 3, 3, 300, 300, 64, 1, "head", "f32", 3, 2.0), (2, 4, 2, 130, 257, 128, 1, "head", "f32", 8, 7.7),
    (1, 2, 2, 256, 640, 128, 1, "tensor", "f32", 4, 1.5), (1, 1, 1, 1, 1, 64, 1, "tensor", "f16", 5, 6.6),
    (3, 8, 1, 129, 65, 128, 0, "tensor", "f32", 1, 0.5), (1, 2, 2, 300, 50, 64, 0, "head", "f32", 5, 6.6),
    # split-KV decode shapes, GQA groups up to 16 rows
    (2, 8, 2, 1, 1500, 128, 0, "tensor", "f16", 5, 6.6), (1, 8, 1, 2, 520, 64, 1, "head", "f32", 3, 2.0),
    (1, 16, 1, 1, 333, 128, 0, "tensor", "f32", 5, 6.6), (1, 4, 1, 4, 700, 128, 1, "tensor", "f32", 2, 0.5),
    (4, 32, 8, 1, 4096, 128, 0, "head", "f32", 5, 6.6), (1, 34, 2, 1, 300, 128, 0, "tensor", "f32", 5, 6.6),
    # V scales per (batch, kv head, channel)
    (2, 4, 2, 130, 257, 128, 1, "channel", "f32", 5, 6.6), (2, 8, 2, 1, 1500, 128, 0, "channel", "f16", 8, 7.7),
]


@pytest.mark.parametrize("B,H,Hkv,Lq,Lkv,d,causal,vmode,odt,bits,clip", SWEEP)
def test_shape_sweep(lib, B, H, Hkv, Lq, Lkv, d, causal, vmode, odt, bits, clip):
    seed = B * 1000 + H * 100 + Lq * 7 + Lkv + bits
    q = gaussian((B, H, Lq, d), seed, np.float16)
    q[0, 0, 0] = 0                                    # an all-zero query row
    k = gaussian((B, Hkv, Lkv, d), seed + 1, np.float16)
    v = gaussian((B, Hkv, Lkv, d), seed + 2, np.float16)
    run_lut(lib, q, k, v, causal, vmode, odt, bits, clip, tag="sweep")


def test_growing_logits(lib):
    # keys whose norm grows along the sequence: the running max rises tile
    # after tile, so every rescale path runs
    r = np.random.Generator(np.random.PCG64(77))
    B, H, L, d = 1, 2, 700, 128
    q = (r.standard_normal((B, H, L, d)) * 6).astype(np.float32)
    k = r.standard_normal((B, H, L, d)).astype(np.float32) * np.linspace(1, 8, L, dtype=np.float32)[:, None]
    v = r.standard_normal((B, H, L, d)).astype(np.float32)
    run_lut(lib, q, k, v, True, "tensor", "f32", 5, 6.6, tag="growing")
    run_lut(lib, q[:, :, -1:].copy(), k, v, False, "tensor", "f32", 5, 6.6, tag="growing-decode")


def _random_shapes(n, seed):
    """Seeded random problems for the table kernels: prefill and decode
    shapes, table sizes b = 1 .. 8 (pair table up to b = 5, byte table above),
    clips 0.5 .. 8, V per tensor, head or channel."""
    import random
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        d = rng.choice([64, 128])
        causal = int(rng.random() < 0.6)
        hkv = rng.choice([1, 2, 4])
        h = hkv * rng.choice([1, 2, 4])
        lq = rng.randint(1, 16 // (h // hkv)) if rng.random() < 0.3 else rng.randint(1, 500)
        lkv = rng.randint(lq if causal else 1, 900)
        out.append((rng.choice([1, 2]), h, hkv, lq, lkv, d, causal, rng.choice(["tensor", "head", "channel"]),
                    rng.choice(["f16", "f32"]), rng.randint(1, 8), round(rng.uniform(0.5, 8.0), 2)))
    return out


@pytest.mark.parametrize("i,shape", list(enumerate(_random_shapes(32, 20261205))))
def test_random_shapes(lib, i, shape):
    B, H, Hkv, Lq, Lkv, d, causal, vmode, odt, bits, clip = shape
    seed = 11000 + 3 * i
    q = gaussian((B, H, Lq, d), seed, np.float16)
    k = gaussian((B, Hkv, Lkv, d), seed + 1, np.float16)
    v = gaussian((B, Hkv, Lkv, d), seed + 2, np.float16)
    run_lut(lib, q, k, v, causal, vmode, odt, bits, clip, tag="random%d" % i)
