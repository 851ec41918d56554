"""The packed 4-bit K layout, written from its definition (test helper): per
group of 8 codes of a row, byte j holds code[j] + 8 in its low nibble and
code[j + 4] + 8 in its high nibble."""
import numpy as np


def pack(codes):
    c = np.asarray(codes, np.int16) + 8
    assert c.min() >= 0 and c.max() <= 15
    g = c.reshape(c.shape[:-1] + (c.shape[-1] // 8, 8))
    b = g[..., :4] | (g[..., 4:] << 4)
    return b.reshape(c.shape[:-1] + (c.shape[-1] // 2,)).astype(np.uint8)


def unpack(packed):
    p = np.asarray(packed, np.uint8).astype(np.int16)
    g = p.reshape(p.shape[:-1] + (p.shape[-1] // 4, 4))
    lo, hi = g & 15, g >> 4
    c = np.concatenate([lo, hi], axis=-1) - 8
    return c.reshape(p.shape[:-1] + (p.shape[-1] * 2,)).astype(np.int8)
