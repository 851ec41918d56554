"""Fused INT8 attention on the GPU vs the oracle run with the GPU's schedule.

Every workload compares every output row, the full-size ones (the sizes the
benchmark times) included, and the decode workload every batch entry.
Quantized tensors and scales are compared bit for bit on the full tensors
along the way.
"""
import numpy as np
import pytest

from gpu_parity import log, run_problem
from workloads import WORKLOADS, gaussian

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import int8_quantized_flashattention_amd as m
    return m


@pytest.mark.parametrize("name", ["tiny", "l1024", "l1024_causal"])
def test_small_workloads_all_rows(lib, name):
    w = WORKLOADS[name]
    q, k, v = w.inputs()
    for odt in ({w.o_dtype} | {"f32"}):
        run_problem(lib, q, k, v, w.causal, w.v_per_token, odt, tag="%s/%s" % (name, odt))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["l4096_outlier", "l4096_gauss", "l16384"])
def test_full_size_workloads_all_rows(lib, name):
    # every row of B4 H32 L4096 (outlier channels and plain Gaussian) and of
    # B1 H32 L16384, in the launch configuration the benchmark times
    w = WORKLOADS[name]
    q, k, v = w.inputs()
    run_problem(lib, q, k, v, w.causal, w.v_per_token, w.o_dtype, tag=name)


@pytest.mark.timeout(600)
def test_decode_workload_all_batches(lib):
    # the full 1 GB KV cache, every batch entry, head and row
    w = WORKLOADS["decode"]
    q, k, v = w.inputs()
    run_problem(lib, q, k, v, w.causal, w.v_per_token, w.o_dtype, tag="decode")


def test_wide_outlier_problem(lib):
    # B3 H16 Hkv2 Lq1003 Lkv2228 d64 causal, per-tensor V, fp32 O, channels 3
    # and 59 of Q and K x20: logits of several hundred in magnitude and rows
    # peaked on a few keys, where one P_hat code that the kernel rounds
    # differently from the oracle moves O by ~0.02
    B, H, Hkv, Lq, Lkv, d = 3, 16, 2, 1003, 2228, 64
    ch = [3, 59]
    q = gaussian((B, H, Lq, d), 50008, outlier_channels=ch)
    k = gaussian((B, Hkv, Lkv, d), 50009, outlier_channels=ch)
    v = gaussian((B, Hkv, Lkv, d), 50010)
    run_problem(lib, q, k, v, True, False, "f32", tag="wide_outlier")


def test_per_token_v_tie_problem(lib):
    # B2 H11 Hkv11 Lq296 Lkv1127 d64 causal, per-token V, fp16 in and out,
    # channel 37 of Q and K x20 (problem 446 of the random sweep). In rows
    # peaked on key 881 that key's y is 127 and 127 s_V[j] / s_t lies within
    # 5e-6 of 102.5: a multiplier formed as s_V[j] * (1 / s_t), one ulp above
    # the quotient, rounds the code to 103 instead of 102 and moves O by 0.02
    B, H, Hkv, Lq, Lkv, d = 2, 11, 11, 296, 1127, 64
    q = gaussian((B, H, Lq, d), 104460, outlier_channels=[37])
    k = gaussian((B, Hkv, Lkv, d), 104461, outlier_channels=[37])
    v = gaussian((B, Hkv, Lkv, d), 104462)
    run_problem(lib, q, k, v, True, True, "f16", tag="per_token_v_tie")


def test_exact_rounding_tie_problem(lib):
    # B2 H12 Hkv3 Lq1177 Lkv2608 d64, not causal, per-token V, fp32 inputs,
    # fp16 O, channel 11 of Q and K x20 (problem 1958 of the random sweep). In
    # the peaked row (b 0, h 1, query 711) key 882's fp32 product y * w is
    # exactly 40.5: the oracle rounds it to the even code 40, and an exponential
    # one ulp higher gives 41, which moves that row by ~0.018, inside the
    # tolerance (the one way the exact logits leave for a code to differ)
    B, H, Hkv, Lq, Lkv, d = 2, 12, 3, 1177, 2608, 64
    q = gaussian((B, H, Lq, d), 119580, np.float32, [11])
    k = gaussian((B, Hkv, Lkv, d), 119581, np.float32, [11])
    v = gaussian((B, Hkv, Lkv, d), 119582, np.float32)
    run_problem(lib, q, k, v, False, True, "f16", tag="exact_tie")


@pytest.mark.parametrize("neg", [False, True])
@pytest.mark.parametrize("B,H,Hkv,Lq,Lkv,d,causal,vpt,odt", [
    (1, 4, 2, 300, 333, 128, 1, 0, "f32"), (1, 4, 2, 300, 333, 64, 0, 1, "f16"),
    (2, 8, 2, 1, 700, 128, 0, 0, "f32"), (1, 8, 1, 2, 520, 64, 1, 1, "f16")])
def test_huge_logits(lib, B, H, Hkv, Lq, Lkv, d, causal, vpt, odt, neg):
    # Q and K x200: row maxima of ~10^5 (base 2 about 2^17), where the fp32
    # spacing of the running max is 2^-7..2^-6 and the exponent bias has to
    # keep the dominant key's code within a signed byte (a code of 128 would
    # read as -128 and flip that key's V row). neg: |Q| against -|K|, so every
    # logit and every row max is negative (about -2^18; the bias steps toward
    # zero). V x1/4: a code that rounds the other way at a tie moves O by at
    # most |V|/127 < 1e-2.
    q = gaussian((B, H, Lq, d), 50200 + d, np.float32) * np.float32(200.0)
    k = gaussian((B, Hkv, Lkv, d), 50201 + d, np.float32) * np.float32(200.0)
    v = gaussian((B, Hkv, Lkv, d), 50202 + d, np.float32) * np.float32(0.25)
    if neg:
        q, k = np.abs(q), -np.abs(k)
    run_problem(lib, q, k, v, bool(causal), bool(vpt), odt, tag="huge_logits_neg" if neg else "huge_logits")


# ragged and degenerate shapes: Lq/Lkv not multiples of the tiles, Lq != Lkv,
# GQA ratios, single rows/keys
SWEEP = [  # B, H, Hkv, Lq, Lkv, d, causal, v_per_token, o
    (1, 1, 1, 1, 1, 64, 0, 0, "f32"), (1, 1, 1, 1, 1, 128, 1, 1, "f16"),
    (2, 4, 2, 77, 130, 128, 1, 0, "f16"), (1, 2, 1, 1, 200, 128, 0, 1, "f32"),
    (1, 3, 3, 300, 300, 64, 1, 1, "f32"), (1, 2, 2, 50, 190, 64, 1, 0, "f16"),
    (3, 8, 1, 129, 65, 128, 0, 0, "f16"), (1, 8, 2, 257, 1000, 128, 1, 1, "f16"),
    (2, 16, 4, 16, 700, 128, 0, 1, "f16"), (1, 4, 4, 640, 640, 128, 1, 0, "f32"),
    (1, 32, 8, 3, 333, 64, 0, 1, "f32"), (2, 2, 2, 1000, 1001, 64, 1, 0, "f16"),
    # schedule boundaries: 16 rows per KV head (the largest decode-path group),
    # 17 (the smallest prefill-path one), more queries than keys (non-causal)
    (1, 16, 1, 1, 333, 128, 0, 1, "f32"), (1, 8, 1, 2, 333, 64, 1, 0, "f16"),
    (1, 34, 2, 1, 300, 128, 0, 0, "f32"), (1, 2, 2, 300, 50, 64, 0, 1, "f16"),
    # V scales per (batch, kv head)
    (2, 8, 2, 77, 130, 128, 1, "head", "f16"), (2, 16, 4, 1, 700, 128, 0, "head", "f32"),
    (3, 4, 4, 300, 300, 64, 1, "head", "f32"),
    # V scales per (batch, kv head, channel)
    (2, 8, 2, 77, 130, 128, 1, "channel", "f16"), (2, 16, 4, 1, 700, 128, 0, "channel", "f32"),
    (1, 3, 3, 300, 300, 64, 1, "channel", "f32"), (1, 8, 1, 2, 520, 64, 1, "channel", "f16"),
    # 1 .. 6 KV tiles of 64 keys around the two-tile steps of the prefill's stage ring
    (1, 2, 1, 130, 127, 128, 0, 0, "f16"), (1, 2, 1, 130, 129, 128, 0, 0, "f16"),
    (1, 2, 2, 64, 192, 64, 0, 0, "f32"), (1, 2, 2, 64, 193, 128, 0, 1, "f16"),
    (1, 2, 2, 200, 256, 128, 1, 0, "f16"), (1, 2, 2, 100, 321, 128, 0, 0, "f32"),
    (1, 2, 2, 40, 64, 128, 0, 0, "f16"), (1, 2, 2, 300, 384, 64, 1, "head", "f16"),
]


@pytest.mark.parametrize("B,H,Hkv,Lq,Lkv,d,causal,vpt,odt", SWEEP)
def test_shape_sweep(lib, B, H, Hkv, Lq, Lkv, d, causal, vpt, odt):
    seed = (B * 7 + H) * 1000003 + Lq * 1009 + Lkv
    q = gaussian((B, H, Lq, d), seed, np.float16)
    k = gaussian((B, Hkv, Lkv, d), seed + 1, np.float16)
    v = gaussian((B, Hkv, Lkv, d), seed + 2, np.float16)
    run_problem(lib, q, k, v, causal, vpt, odt, tag="sweep")


def test_degenerate_inputs(lib):
    r = np.random.Generator(np.random.PCG64(9))
    B, H, L, d = 1, 2, 200, 128
    base = [gaussian((B, H, L, d), 900 + i, np.float16) for i in range(3)]
    q0 = np.zeros_like(base[0])                     # zero queries: uniform weights
    run_problem(lib, q0, base[1], base[2], True, False, "f32", tag="zero-q")
    v0 = np.zeros_like(base[2])                     # zero values: s_V = 0, O = 0
    og, _ = run_problem(lib, base[0], base[1], v0, False, False, "f32", tag="zero-v")
    assert np.all(og == 0)
    keq = np.repeat(base[1][:, :, :1], L, axis=2)   # identical keys
    run_problem(lib, base[0], keq, base[2], False, True, "f32", tag="equal-k")
    big = (r.standard_normal((B, H, L, d)) * 60).astype(np.float16)  # peaked softmax
    run_problem(lib, big, big, base[2], True, False, "f16", tag="peaked")


def test_per_block_v_via_per_token_scales(lib):
    # per-block V scales (one per 64-key block, the KV tile): quantize V with
    # rows_per_scale = 64 and repeat each block's scale over its keys; the
    # per-token forward then uses that block's scale for the whole tile
    # (w_j = 127 s / s), which the oracle's per-token mode states
    import torch
    from gpu_parity import compare_o, dev, host, quantize_both
    import oracle
    B, H, Hkv, L, d = 2, 8, 2, 640, 128
    q = gaussian((B, H, L, d), 811, np.float16)
    k = gaussian((B, Hkv, L, d), 812, np.float16)
    v = gaussian((B, Hkv, L, d), 813, np.float16) * np.linspace(0.2, 3.0, L, dtype=np.float16)[:, None]
    qh, sq, qd, sqd = quantize_both(lib, q, 1)
    kh, sk, kd, skd = quantize_both(lib, k, 1)
    vh, sb, vd, sbd = quantize_both(lib, v, 64)
    assert sb.size == B * Hkv * L // 64
    svd = torch.repeat_interleave(sbd, 64).contiguous()
    sv = np.repeat(sb, 64)
    q1h, sq1, q1d, sq1d = quantize_both(lib, np.ascontiguousarray(q[:, :, -1:]), 1)   # a decode shape
    for Lq, causal in ((L, True), (L, False), (1, False)):
        qa, sa, qb, sbq = (qh, sq, qd, sqd) if Lq == L else (q1h, sq1, q1d, sq1d)
        o = lib.attn_int8_fwd(qb, sbq, kd, skd, vd, svd, True, causal, torch.float32)
        tile, split = lib.attn_int8_fwd_schedule(B, H, Hkv, Lq, L, d, causal)
        assert tile == 64 and split % 64 == 0
        oo, _ = oracle.attn_int8(qa, sa, kh, sk, vh, sv, 1, B, H, Hkv, Lq, L, d, causal, tile, split)
        compare_o(host(o), oo, "per-block V Lq=%d causal=%d" % (Lq, causal))


def _random_shapes(n, seed):
    """Seeded random problems: GQA ratios 1, 2, 4; Lq up to 600 and Lkv up to
    900 (Lq <= Lkv when causal); every V scale granularity; fp16 and fp32 O."""
    import random
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        d = rng.choice([64, 128])
        causal = int(rng.random() < 0.6)
        hkv = rng.choice([1, 2, 4])
        h = hkv * rng.choice([1, 2, 4])
        b = rng.choice([1, 2])
        lq = rng.randint(1, 600)
        lkv = rng.randint(lq if causal else 1, 900)
        out.append((b, h, hkv, lq, lkv, d, causal, rng.choice([0, 1, "head", "channel"]), rng.choice(["f16", "f32"])))
    return out


@pytest.mark.parametrize("i,shape", list(enumerate(_random_shapes(48, 20261203))))
def test_random_shapes(lib, i, shape):
    B, H, Hkv, Lq, Lkv, d, causal, vpt, odt = shape
    seed = 7000 + 3 * i
    q = gaussian((B, H, Lq, d), seed, np.float16)
    k = gaussian((B, Hkv, Lkv, d), seed + 1, np.float16)
    v = gaussian((B, Hkv, Lkv, d), seed + 2, np.float16)
    run_problem(lib, q, k, v, causal, vpt, odt, tag="random%d" % i)


def _random_decode_shapes(n, seed):
    """Seeded random decode-shaped problems (at most 16 query rows per KV
    head, so the split-KV kernel and the chunk merge run): Lkv up to 5000."""
    import random
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        g = rng.choice([1, 2, 4, 8])
        lq = rng.randint(1, 16 // g)
        causal = int(rng.random() < 0.5)
        hkv = rng.choice([1, 2, 8])
        out.append((rng.choice([1, 3]), hkv * g, hkv, lq, rng.randint(lq, 5000), rng.choice([64, 128]), causal,
                    rng.choice([0, 1, "head", "channel"]), rng.choice(["f16", "f32"])))
    return out


@pytest.mark.parametrize("i,shape", list(enumerate(_random_decode_shapes(24, 20261204))))
def test_random_decode_shapes(lib, i, shape):
    B, H, Hkv, Lq, Lkv, d, causal, vpt, odt = shape
    seed = 9000 + 3 * i
    q = gaussian((B, H, Lq, d), seed, np.float16)
    k = gaussian((B, Hkv, Lkv, d), seed + 1, np.float16)
    v = gaussian((B, Hkv, Lkv, d), seed + 2, np.float16)
    run_problem(lib, q, k, v, causal, vpt, odt, tag="random_decode%d" % i)
