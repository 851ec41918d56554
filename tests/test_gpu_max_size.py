"""The largest tensors the ABI accepts: K and V of [1, 1, 16777215, 128]
(2^31 - 128 elements each, a ragged last tile), so the kernels' byte offsets
run up to their 32-bit limit. K and V are quantized once (GPU and oracle, bit
for bit over the whole tensors); then a decode-shaped problem (4 query heads
on the KV head, split-KV path) and a prefill-shaped causal one (17 query rows,
past the 16-row limit of the decode path) are checked against the oracle on
every row, through both forward entry points."""
import numpy as np
import pytest
import torch

import oracle
from gpu_parity import compare_o, dev, host, log, quantize_both
from workloads import gaussian, gaussian_chunked

pytestmark = pytest.mark.gpu

LKV = (2 ** 31 - 1) // 128          # 16777215 keys: K has 2147483520 elements
D = 128


@pytest.fixture(scope="module")
def lib():
    import int8_quantized_flashattention_amd as m
    return m


@pytest.fixture(scope="module")
def kv(lib):
    out = []
    for name, seed in (("K", 702), ("V", 703)):
        log("max-size: drawing %s [1, 1, %d, %d] fp32" % (name, LKV, D))
        x = gaussian_chunked((1, 1, LKV, D), seed)
        assert 2 ** 31 - 256 < x.size < 2 ** 31
        log("max-size: quantizing %s (GPU and oracle)" % name)
        qh, s, qd, sd = quantize_both(lib, x, 1)          # per token, bit-exact over the whole tensor
        del x
        out.append((qh, s, qd, sd))
    log("max-size: K and V ready")
    return out


def check(lib, kv, q, causal, odt, tag):
    (kh, sk, kd, skd), (vh, sv, vd, svd) = kv
    B, H, Lq, _ = q.shape
    log("[%s] H=%d Lq=%d causal=%d" % (tag, H, Lq, causal))
    qh, sq, qd, sqd = quantize_both(lib, q, 1)
    tdt = torch.float16 if odt == "f16" else torch.float32
    o, lse = lib.attn_int8_fwd(qd, sqd, kd, skd, vd, svd, True, causal, tdt, return_lse=True)
    o2, lse2 = lib.attn_int8_fwd_qfloat(dev(q), kd, skd, vd, svd, True, causal, tdt, return_lse=True)
    iv = torch.int16 if tdt == torch.float16 else torch.int32
    assert torch.equal(o2.view(iv), o.view(iv)) and torch.equal(lse2.view(torch.int32), lse.view(torch.int32))
    tile, split = lib.attn_int8_fwd_schedule(B, H, 1, Lq, LKV, D, causal)
    log("[%s] schedule tile=%d split=%d; oracle" % (tag, tile, split))
    oo, lo = oracle.attn_int8(qh, sq, kh, sk, vh, sv, True, B, H, 1, Lq, LKV, D, causal, tile, split)
    compare_o(host(o).astype(np.float32), oo, tag)
    lg = host(lse).reshape(-1)
    assert float(np.max(np.abs(lg - lo.reshape(-1)) / np.maximum(1.0, np.abs(lo.reshape(-1))))) <= 1e-4
    return split


@pytest.mark.timeout(900)
def test_max_size_decode(lib, kv):
    split = check(lib, kv, gaussian((1, 4, 1, D), 701, np.float16), False, "f32", "max-size decode")
    assert split > 0


@pytest.mark.timeout(900)
def test_max_size_prefill_causal(lib, kv):
    split = check(lib, kv, gaussian((1, 1, 17, D), 704, np.float16), True, "f16", "max-size prefill")
    assert split == 0
