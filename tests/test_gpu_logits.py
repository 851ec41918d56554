"""INT32 logits from the fused prefill kernel (its dump instance: the same
grid, K staging ring, barriers and Q.K^T tile code) == exact integer products.
Visible pairs must match bit for bit; masked pairs must be left untouched.
The cases include one head of the headline shape (L = 4096, d = 128, causal:
64 KV tiles through the four-stage ring) and a ragged d = 128 problem."""
import numpy as np
import pytest
import torch

import oracle
from gpu_parity import dev, host, log

pytestmark = pytest.mark.gpu
SENTINEL = np.iinfo(np.int32).min


@pytest.fixture(scope="module")
def lib():
    import int8_quantized_flashattention_amd as m
    return m


CASES = [  # B, H, Hkv, Lq, Lkv, d, causal
    (1, 1, 1, 128, 128, 64, 0), (1, 8, 8, 1024, 1024, 64, 1), (1, 8, 8, 1024, 1024, 64, 0),
    (2, 4, 2, 77, 130, 128, 1), (1, 2, 1, 1, 200, 128, 0), (1, 1, 1, 300, 300, 128, 1),
    (1, 2, 2, 50, 190, 64, 1), (3, 8, 1, 129, 65, 128, 0), (1, 1, 1, 1, 1, 64, 1),
    (1, 1, 1, 4096, 4096, 128, 1), (1, 2, 1, 2047, 3001, 128, 1), (2, 4, 4, 1000, 1000, 128, 0),
]


@pytest.mark.parametrize("B,H,Hkv,Lq,Lkv,d,causal", CASES)
def test_logits_bit_exact(lib, B, H, Hkv, Lq, Lkv, d, causal):
    log("logits B=%d H=%d Hkv=%d Lq=%d Lkv=%d d=%d causal=%d" % (B, H, Hkv, Lq, Lkv, d, causal))
    r = np.random.Generator(np.random.PCG64(B * 1000 + Lq * 7 + Lkv))
    q = r.integers(-127, 128, size=(B, H, Lq, d)).astype(np.int8)
    k = r.integers(-127, 128, size=(B, Hkv, Lkv, d)).astype(np.int8)
    q[0, 0, 0, :] = 127
    k[0, 0, 0, :] = -127          # extreme product -127*127*d
    out = torch.full((B, H, Lq, Lkv), SENTINEL, dtype=torch.int32, device="cuda")
    lib.attn_int8_debug_logits(dev(q), dev(k), causal, out=out)
    got = host(out)
    ref = oracle.logits_i32(q, k, B, H, Hkv, Lq, Lkv, d)
    vis = np.ones((Lq, Lkv), bool)
    if causal:
        vis = np.arange(Lkv)[None, :] <= (np.arange(Lq)[:, None] + (Lkv - Lq))
    vis = np.broadcast_to(vis, got.shape)
    assert np.array_equal(got[vis], ref[vis])
    assert np.all(got[~vis] == SENTINEL)
    assert got[0, 0, 0, 0] == -127 * 127 * d
