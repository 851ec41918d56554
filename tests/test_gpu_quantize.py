"""GPU quantizer == oracle quantizer, bit for bit (codes and scales)."""
import numpy as np
import pytest

from gpu_parity import quantize_cols_both, log, quantize_both

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import int8_quantized_flashattention_amd as m
    return m


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# (rows, cols, rows_per_scale, dtype): covers every team width, the
# register-chunk variant, the two-pass large-group path and ragged grids
CASES = [
    (1, 8, 1, np.float32), (7, 64, 1, np.float16), (1000, 128, 1, np.float16),
    (257, 64, 1, np.float32), (33, 256, 1, np.float16), (12, 128, 4, np.float32),
    (100, 128, 10, np.float16), (3, 2048, 1, np.float16), (2, 4096, 1, np.float32),
    (64, 128, 64, np.float16), (4096, 64, 4096, np.float32), (6, 24, 3, np.float16),
    (4 * 1024, 64, 1024, np.float16),
]


@pytest.mark.parametrize("rows,cols,rps,dt", CASES)
def test_quantize_matches_oracle(lib, rows, cols, rps, dt):
    log("quantize rows=%d cols=%d rps=%d %s" % (rows, cols, rps, np.dtype(dt).name))
    r = _rng(rows * 31 + cols)
    x = (r.standard_normal((rows, cols)) * r.uniform(0.01, 30)).astype(dt)
    if rows > 2:
        x[1] = 0                      # an all-zero row
    quantize_both(lib, x, rps)


def test_quantize_ties_and_integers(lib):
    r = _rng(5)
    x = r.integers(-127, 128, size=(64, 64)).astype(np.float32)
    x[:, 0] = 127.0
    x[::2, 1:9] += 0.5                # exact half-way cases (scale 1)
    x = np.clip(x, -127, 127)
    q, s, _, _ = quantize_both(lib, x, 1)
    assert np.all(s == 1.0)
    x2 = (r.integers(-254, 255, size=(32, 128)) / 2.0).astype(np.float16)
    quantize_both(lib, x2, 1)
    quantize_both(lib, x2, 32)


def test_quantize_all_zero_tensor(lib):
    x = np.zeros((16, 128), np.float16)
    q, s, _, _ = quantize_both(lib, x, 16)
    assert np.all(q == 0) and np.all(s == 0)


# One fp16 group of 2-3 M values (the two-pass path with hundreds of
# workgroups per group): a ragged last workgroup, the largest magnitude at the
# last element, negative zeros, ties at scale 1, and an all-zero tensor of that
# size.
def test_quantize_large_tensor_group(lib):
    r = _rng(77)
    x = (r.standard_normal((23457, 128)) * 3).astype(np.float16)
    x[-1, -1] = -1000.0
    x[5, :7] = -0.0
    quantize_both(lib, x, x.shape[0])
    y = r.integers(-127, 128, size=(16411, 128)).astype(np.float16)
    y[::3, ::5] += np.float16(0.5)
    y[0, 0] = 127.0
    q, s, _, _ = quantize_both(lib, np.clip(y, -127, 127).astype(np.float16), y.shape[0])
    assert s[0] == 1.0
    z = np.zeros((20000, 128), np.float16)
    q, s, _, _ = quantize_both(lib, z, z.shape[0])
    assert np.all(q == 0) and np.all(s == 0)


# quantize-on-append into an INT8 cache: (B, Hkv, T, d, L_max, pos, dtype)
APPEND = [
    (2, 3, 1, 128, 40, 39, np.float16), (1, 8, 5, 64, 16, 0, np.float32),
    (3, 2, 7, 128, 100, 50, np.float16), (1, 1, 33, 2048, 33, 0, np.float32),
    (64, 8, 1, 128, 8192, 8191, np.float16),
]


@pytest.mark.parametrize("B,Hkv,T,d,L,pos,dt", APPEND)
def test_kv_append_matches_oracle(lib, B, Hkv, T, d, L, pos, dt):
    import torch
    import oracle
    log("kv append B=%d Hkv=%d T=%d d=%d L_max=%d pos=%d %s" % (B, Hkv, T, d, L, pos, np.dtype(dt).name))
    r = _rng(B * 7 + T * 13 + d)
    x = (r.standard_normal((B, Hkv, T, d)) * r.uniform(0.1, 10)).astype(dt)
    x[0, 0, 0] = 0                                          # an all-zero token
    cache = torch.full((B, Hkv, L, d), 99, dtype=torch.int8, device="cuda")   # sentinel
    scales = torch.full((B, Hkv, L), -1.0, dtype=torch.float32, device="cuda")
    lib.attn_kv_append(torch.from_numpy(x).cuda(), cache, scales, pos)
    c, s = cache.cpu().numpy(), scales.cpu().numpy()
    qo, so = oracle.quantize_rows(x, 1)
    assert np.array_equal(c[:, :, pos:pos + T], qo)
    assert np.array_equal(s[:, :, pos:pos + T].reshape(-1).view(np.uint32), so.view(np.uint32))
    keep = np.ones(L, bool)
    keep[pos:pos + T] = False
    assert np.all(c[:, :, keep] == 99) and np.all(s[:, :, keep] == -1.0)


# (groups, rows, cols, dtype): one scale per column of each group of rows,
# from one row to the V tensor of the long-context shape, every column width
COLS = [
    (5, 1, 8, np.float16), (3, 37, 24, np.float32), (4, 130, 128, np.float16), (2, 700, 64, np.float32),
    (2, 3, 2048, np.float16), (128, 4096, 128, np.float16), (1, 100000, 64, np.float32),
]


@pytest.mark.parametrize("groups,rows,cols,dt", COLS)
def test_quantize_cols_matches_oracle(lib, groups, rows, cols, dt):
    log("quantize cols groups=%d rows=%d cols=%d %s" % (groups, rows, cols, np.dtype(dt).name))
    r = _rng(groups * 131 + rows + cols)
    x = (r.standard_normal((groups, rows, cols)) * r.uniform(0.01, 30.0, size=(groups, 1, cols))).astype(dt)
    x[0, :, cols // 2] = 0             # an all-zero column
    quantize_cols_both(lib, x, rows)
