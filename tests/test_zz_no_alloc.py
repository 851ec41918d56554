"""The forward that allocates nothing (attn_int8_fwd_noalloc, split-KV
partials in the library's static per-GPU scratch) returns what attn_int8_fwd
returns with a caller workspace, bit for bit, on two calls in a row (the
second smaller, reusing the scratch the first one filled), and within the
oracle tolerance of the oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_parity import compare_o, dev, host, log, quantize_both
from workloads import gaussian

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import int8_quantized_flashattention_amd as m
    return m


def _problem(lib, B, H, Hkv, Lq, Lkv, d, causal, vpt, seed):
    q = gaussian((B, H, Lq, d), seed)
    k = gaussian((B, Hkv, Lkv, d), seed + 1)
    v = gaussian((B, Hkv, Lkv, d), seed + 2)
    qh, sq, qd, sqd = quantize_both(lib, q, 1)
    kh, sk, kd, skd = quantize_both(lib, k, 1)
    vh, sv, vd, svd = quantize_both(lib, v, 1 if vpt else v.size // d)
    return (qh, sq, kh, sk, vh, sv), (qd, sqd, kd, skd, vd, svd)


CASES = [  # B, H, Hkv, Lq, Lkv, d, causal, per-token V, O dtype
    (16, 32, 8, 1, 5000, 128, 0, True, torch.float16),      # decode shape, several KV chunks
    (2, 8, 2, 3, 700, 64, 1, False, torch.float32),         # smaller, causal, reuses the scratch
]


def test_noalloc_matches_workspace_forward_twice(lib):
    assert lib.attn_int8_fwd_noalloc_max_scratch() == 32 << 20
    for i, (B, H, Hkv, Lq, Lkv, d, causal, vpt, odt) in enumerate(CASES):
        log("noalloc call %d: B=%d H=%d Hkv=%d Lq=%d Lkv=%d d=%d causal=%d" % (i, B, H, Hkv, Lq, Lkv, d, causal))
        need = lib.attn_int8_fwd_workspace_size(B, H, Hkv, Lq, Lkv, d, causal)
        assert 0 < need <= lib.attn_int8_fwd_noalloc_max_scratch()
        hostt, devt = _problem(lib, B, H, Hkv, Lq, Lkv, d, causal, vpt, 9100 + 10 * i)
        qd, sqd, kd, skd, vd, svd = devt
        o_na = torch.empty((B, H, Lq, d), dtype=odt, device="cuda")
        l_na = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
        lib.attn_int8_fwd_noalloc(qd, sqd, kd, skd, vd, svd, vpt, causal, odt, out=o_na, lse=l_na)
        o_ws, l_ws = lib.attn_int8_fwd(qd, sqd, kd, skd, vd, svd, vpt, causal, odt, return_lse=True)
        torch.cuda.synchronize()
        bits = torch.int16 if odt == torch.float16 else torch.int32
        assert torch.equal(o_na.view(bits), o_ws.view(bits)), "O differs from the workspace forward"
        assert torch.equal(l_na.view(torch.int32), l_ws.view(torch.int32)), "lse differs"
        qh, sq, kh, sk, vh, sv = hostt
        tile, split = lib.attn_int8_fwd_schedule(B, H, Hkv, Lq, Lkv, d, causal)
        oo, _ = oracle.attn_int8(qh, sq, kh, sk, vh, sv, int(vpt), B, H, Hkv, Lq, Lkv, d, causal, tile, split)
        compare_o(host(o_na).astype(np.float32), oo, "noalloc%d" % i)


def test_noalloc_prefill_shape_needs_no_scratch(lib):
    B, H, Hkv, Lq, Lkv, d = 1, 4, 2, 300, 300, 128
    assert lib.attn_int8_fwd_workspace_size(B, H, Hkv, Lq, Lkv, d, 1) == 0
    _, devt = _problem(lib, B, H, Hkv, Lq, Lkv, d, 1, False, 9200)
    qd, sqd, kd, skd, vd, svd = devt
    o_na = lib.attn_int8_fwd_noalloc(qd, sqd, kd, skd, vd, svd, False, True, torch.float32)
    o_ws = lib.attn_int8_fwd(qd, sqd, kd, skd, vd, svd, False, True, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_na.view(torch.int32), o_ws.view(torch.int32))
