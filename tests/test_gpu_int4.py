"""INT4 Q.K on the GPU vs the oracle: per-token 4-bit codes (absmax / 7) and
their packed form bit for bit, quantize-on-append into a packed K cache, and
the forward with packed K (read directly by the split-KV decode kernel;
widened to INT8 in the workspace for prefill shapes) against the oracle run
on the same 4-bit codes with the GPU's schedule (the path's tolerance)."""
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


def quantize4_both(lib, x):
    c, p, s = lib.attn_quantize_rows_int4(dev(x))
    qo, so = oracle.quantize_rows_int4(x)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32)), "4-bit scales differ"
    assert np.array_equal(host(c), qo), "4-bit codes differ"
    assert np.array_equal(host(p), int4_format.pack(qo)), "packed codes differ"
    return qo, so, c, p, s


@pytest.mark.parametrize("rows,cols,dt", [(7, 64, np.float16), (1000, 128, np.float32), (3, 2048, np.float16),
                                          (33, 24, np.float32), (4097, 512, np.float16)])
def test_quantize_int4_matches_oracle(lib, rows, cols, dt):
    log("int4 quantize rows=%d cols=%d %s" % (rows, cols, np.dtype(dt).name))
    r = np.random.Generator(np.random.PCG64(rows + cols))
    x = (r.standard_normal((rows, cols)) * r.uniform(0.01, 40.0, size=(rows, 1))).astype(dt)
    x[min(2, rows - 1)] = 0
    quantize4_both(lib, x)


def test_kv_append_int4_matches_oracle(lib):
    B, Hkv, T, d, L, pos = 4, 8, 3, 128, 300, 97
    x = gaussian((B, Hkv, T, d), 611, np.float16)
    cache = torch.full((B, Hkv, L, d // 2), 0x63, dtype=torch.uint8, device="cuda")
    sc = torch.full((B * Hkv * L,), 7.0, dtype=torch.float32, device="cuda")
    lib.attn_kv_append_int4(dev(x), cache, sc, pos)
    qo, so = oracle.quantize_rows_int4(x)
    c, s = host(cache), host(sc).reshape(B, Hkv, L)
    assert np.array_equal(c[:, :, pos:pos + T], int4_format.pack(qo))
    assert np.array_equal(s[:, :, pos:pos + T].reshape(-1).view(np.uint32), so.view(np.uint32))
    keep = np.ones(L, bool)
    keep[pos:pos + T] = False
    assert np.all(c[:, :, keep] == 0x63) and np.all(s[:, :, keep] == 7.0)


def run_int4(lib, q, k, v, causal, vmode, odt, rows=None, tag="", measure=None):
    """INT4 Q.K forward on the GPU against the oracle on the same 4-bit codes
    (codes, scales and packed bytes checked bit for bit). measure: if a dict,
    the O and lse errors are stored in it instead of being asserted."""
    B, H, Lq, d = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    log("[%s] B=%d H=%d Hkv=%d Lq=%d Lkv=%d d=%d causal=%d v=%s o=%s" % (tag, B, H, Hkv, Lq, Lkv, d, causal, vmode, odt))
    qh, sq, qd, _, sqd = quantize4_both(lib, q)
    kh, sk, _, kp, skd = quantize4_both(lib, k)
    if vmode == "channel":
        vh, sv, vd, svd = quantize_cols_both(lib, v, Lkv)
    else:
        vh, sv, vd, svd = quantize_both(lib, v, {"tensor": v.size // d, "token": 1, "head": Lkv}[vmode])
    tdt = torch.float16 if odt == "f16" else torch.float32
    o, lse = lib.attn_int4qk_fwd(qd, sqd, kp, skd, vd, svd, vmode, causal, tdt, return_lse=True)
    tile, split = lib.attn_int8_fwd_schedule(B, H, Hkv, Lq, Lkv, d, causal)
    mode = {"tensor": 0, "token": 1, "head": 2, "channel": 3}[vmode]
    oo, lo = oracle.attn_int8(qh, sq, kh, sk, vh, sv, mode, B, H, Hkv, Lq, Lkv, d, causal, tile, split, rows=rows)
    og, lg = host(o).astype(np.float32).reshape(-1, d), host(lse).reshape(-1)
    if rows is not None:
        og, lg = og[rows], lg[rows]
    lo = lo.reshape(-1)
    lse_err = float(np.max(np.abs(lg - lo) / np.maximum(1.0, np.abs(lo)))) if lo.size else 0.0
    if measure is not None:
        measure["max_abs"], measure["rel_fro"], measure["finite"] = o_errors(og, oo.reshape(-1, d))
        measure["lse_err"] = lse_err
        return split
    compare_o(og, oo.reshape(-1, d), tag)
    assert lse_err <= 1e-4
    return split


SWEEP = [  # B, H, Hkv, Lq, Lkv, d, causal, V scale, o
    (2, 8, 2, 1, 1500, 128, 0, "tensor", "f16"), (1, 8, 1, 2, 520, 64, 1, "token", "f32"),
    (1, 16, 1, 1, 333, 128, 0, "head", "f32"), (4, 32, 8, 1, 4096, 128, 0, "channel", "f32"),
    (1, 4, 1, 4, 700, 128, 1, "token", "f16"), (1, 1, 1, 1, 1, 64, 1, "tensor", "f32"),
    # prefill shapes (K widened in the workspace)
    (2, 4, 2, 77, 130, 128, 1, "tensor", "f16"), (1, 3, 3, 300, 300, 64, 1, "head", "f32"),
    (1, 34, 2, 1, 300, 128, 0, "token", "f32"),
]


@pytest.mark.parametrize("B,H,Hkv,Lq,Lkv,d,causal,vmode,odt", SWEEP)
def test_int4qk_forward(lib, B, H, Hkv, Lq, Lkv, d, causal, vmode, odt):
    seed = B * 7919 + H * 31 + Lq * 7 + Lkv
    q = gaussian((B, H, Lq, d), seed, np.float16)
    k = gaussian((B, Hkv, Lkv, d), seed + 1, np.float16)
    v = gaussian((B, Hkv, Lkv, d), seed + 2, np.float16)
    run_int4(lib, q, k, v, causal, vmode, odt, tag="int4")


@pytest.mark.timeout(400)
def test_int4qk_decode_workload_sampled_rows(lib):
    # the decode configuration (B64 H32 Hkv8 L8192, per-token V): the whole
    # packed cache goes through the kernel; the oracle checks every head of a
    # seeded set of batch entries
    w = WORKLOADS["decode"]
    q, k, v = w.inputs()
    rows = np.concatenate([b * w.H + np.arange(w.H) for b in (0, 21, 63)]).astype(np.int64)
    split = run_int4(lib, q, k, v, w.causal, "token", w.o_dtype, rows=rows, tag="int4 decode")
    assert split > 0


def _random_shapes(n, seed):
    """Seeded random INT4 Q.K problems: mostly decode shapes (the packed-K
    kernel), some prefill shapes (K widened in the workspace)."""
    import random
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        g = rng.choice([1, 2, 4, 8])
        hkv = rng.choice([1, 2, 4])
        lq = rng.randint(1, 16 // g) if rng.random() < 0.7 else rng.randint(17, 300)
        causal = int(rng.random() < 0.5)
        out.append((rng.choice([1, 2]), hkv * g, hkv, lq, rng.randint(lq, 3000), rng.choice([64, 128]), causal,
                    rng.choice(["tensor", "token", "head", "channel"]), rng.choice(["f16", "f32"])))
    return out


@pytest.mark.parametrize("i,shape", list(enumerate(_random_shapes(24, 20261206))))
def test_random_shapes(lib, i, shape):
    B, H, Hkv, Lq, Lkv, d, causal, vmode, odt = shape
    seed = 13000 + 3 * i
    q = gaussian((B, H, Lq, d), seed, np.float16)
    k = gaussian((B, Hkv, Lkv, d), seed + 1, np.float16)
    v = gaussian((B, Hkv, Lkv, d), seed + 2, np.float16)
    run_int4(lib, q, k, v, causal, vmode, odt, tag="random%d" % i)
