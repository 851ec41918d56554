"""An exact rounding tie inside the attention path, on the oracle (CPU).

Problem 1958 of the random wide sweep (B2 H12 Hkv3 Lq1177 Lkv2608 d64, not
causal, per-token V, fp32 inputs, channel 11 of Q and K x20) has a row that is
peaked on few keys, where the code of key 882 is decided on an fp32 product
y * w of exactly 40.5. P_hat is round-to-nearest-even of that product
("IntAttention" §3.2, the prior-methods scheme, read with ties to even), so the
code is 40; rounding half away from zero would give 41. The GPU test of the
same problem (test_gpu_attention.test_exact_rounding_tie_problem) bounds the
effect of an exponential that lands one ulp off on such a tie.
"""
import numpy as np

import oracle
from workloads import gaussian


def test_row_has_an_exact_tie_rounded_to_even():
    B, H, Hkv, Lq, Lkv, d = 2, 12, 3, 1177, 2608, 64
    q = gaussian((B, H, Lq, d), 119580, np.float32, [11])
    k = gaussian((B, Hkv, Lkv, d), 119581, np.float32, [11])
    v = gaussian((B, Hkv, Lkv, d), 119582, np.float32)
    qh, sq = oracle.quantize_rows(q, 1)
    kh, sk = oracle.quantize_rows(k, 1)
    vh, sv = oracle.quantize_rows(v, 1)
    tr = oracle.attn_int8_trace(qh, sq, kh, sk, vh, sv, 1, B, H, Hkv, Lq, Lkv, d, False, 64, 0, 0, 1, 711)
    z = np.float32(tr["y"][882]) * np.float32(tr["w"][882])
    assert z == np.float32(40.5)
    assert tr["p_hat"][882] == 40
    # every other code of the row is the nearest integer of its product
    zz = tr["y"].astype(np.float32) * tr["w"].astype(np.float32)
    assert np.array_equal(tr["p_hat"], np.rint(zz).astype(np.int32))
