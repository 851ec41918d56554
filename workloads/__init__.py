"""Seeded synthetic inputs and the workload table.

This module is the only thing the oracle side and the GPU side share: it draws
the input tensors and holds the shapes. It contains none of the attention
method's arithmetic (no quantization, no softmax, no products).

Recipe: numpy ``Generator(PCG64(seed)).standard_normal(dtype=float32)`` in the
tensor's row-major shape; for the outlier workload a seeded set of head-dim
channels is multiplied by 20 in fp32 (the same channels in Q and K, every
batch, head and token); finally the fp32 values are cast to the stored dtype
(fp16 by round-to-nearest-even, or kept fp32). The pages measure on language
and vision models over public datasets that are not available here; these
Gaussian tensors with the pages' sequence lengths and head dimension stand in
for them.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np


def gaussian(shape, seed, dtype=np.float16, outlier_channels=None, outlier_gain=20.0):
    """Return a seeded N(0,1) tensor of `shape` (last axis = head dim)."""
    x = np.random.Generator(np.random.PCG64(seed)).standard_normal(size=shape, dtype=np.float32)
    if outlier_channels is not None and len(outlier_channels):
        x[..., np.asarray(outlier_channels)] *= np.float32(outlier_gain)
    return x.astype(dtype)


def gaussian_chunked(shape, seed, chunk_rows=1 << 20, threads=16):
    """A seeded N(0,1) fp32 tensor drawn in parallel: the rows (last axis) are
    cut into chunks of `chunk_rows`, chunk i drawn from its own PCG64 stream
    spawned from SeedSequence(seed) (the same values for any thread count).
    For tensors of ~2^31 elements, where one stream takes about a minute."""
    from concurrent.futures import ThreadPoolExecutor
    n = int(np.prod(shape))
    per = chunk_rows * shape[-1]
    out = np.empty(n, np.float32)
    seqs = np.random.SeedSequence(seed).spawn((n + per - 1) // per)

    def fill(i):
        np.random.Generator(np.random.PCG64(seqs[i])).standard_normal(
            out=out[i * per:(i + 1) * per], dtype=np.float32)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, range(len(seqs))))
    return out.reshape(shape)


def outlier_channels(d, seed, fraction=0.01):
    """The seeded head-dim channels scaled for the outlier workload:
    max(1, round(fraction * d)) distinct channels."""
    n = max(1, int(round(fraction * d)))
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.sort(rng.choice(d, size=n, replace=False))


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    Lq: int
    Lkv: int
    d: int
    causal: bool
    v_per_token: bool
    in_dtype: str            # "f16" or "f32"
    o_dtype: str             # "f16" or "f32"
    seeds: Tuple[int, int, int]
    outlier_seed: Optional[int] = None
    # K/V live in an INT8 cache quantized once; a step appends one new token
    kv_cache: bool = False
    note: str = field(default="", compare=False)

    @property
    def np_in_dtype(self):
        return np.float16 if self.in_dtype == "f16" else np.float32

    def shapes(self):
        return ((self.B, self.H, self.Lq, self.d), (self.B, self.Hkv, self.Lkv, self.d),
                (self.B, self.Hkv, self.Lkv, self.d))

    def inputs(self):
        """(q, k, v) host arrays in the stored input dtype."""
        sq, sk, sv = self.shapes()
        oc = outlier_channels(self.d, self.outlier_seed) if self.outlier_seed is not None else None
        q = gaussian(sq, self.seeds[0], self.np_in_dtype, oc)
        k = gaussian(sk, self.seeds[1], self.np_in_dtype, oc)
        v = gaussian(sv, self.seeds[2], self.np_in_dtype)
        return q, k, v

    def visible_pairs(self):
        """Number of unmasked (query, key) pairs over the whole batch."""
        if not self.causal:
            n = self.Lq * self.Lkv
        else:
            off = self.Lkv - self.Lq
            # query i sees keys 0..i+off
            n = sum(min(self.Lkv, i + off + 1) for i in range(self.Lq))
        return self.B * self.H * n

    def ops(self):
        """Algorithmic INT8 ops: 2 ops per MAC, d MACs for Q.K and d for P.V per pair."""
        return 4 * self.d * self.visible_pairs()

    def replace(self, **kw):
        from dataclasses import replace
        return replace(self, **kw)


W = Workload
WORKLOADS = {
    # tiny reference case, fp32 inputs and output
    "tiny": W("tiny", 1, 1, 1, 128, 128, 64, False, False, "f32", "f32", (101, 102, 103)),
    # B1 H8 L1024 d64, both mask settings
    "l1024": W("l1024", 1, 8, 8, 1024, 1024, 64, False, False, "f16", "f16", (201, 202, 203)),
    "l1024_causal": W("l1024_causal", 1, 8, 8, 1024, 1024, 64, True, False, "f16", "f16",
                      (201, 202, 203)),
    # headline: B4 H32 L4096 d128 causal, 1% outlier channels x20 in Q and K
    "l4096_outlier": W("l4096_outlier", 4, 32, 32, 4096, 4096, 128, True, False, "f16", "f16",
                       (301, 302, 303), 304),
    "l4096_gauss": W("l4096_gauss", 4, 32, 32, 4096, 4096, 128, True, False, "f16", "f16",
                     (301, 302, 303)),
    # long context, per-token V
    "l16384": W("l16384", 1, 32, 32, 16384, 16384, 128, True, True, "f16", "f16", (401, 402, 403)),
    # decode-shaped GQA over an int8 KV cache with per-token scales
    "decode": W("decode", 64, 32, 8, 1, 8192, 128, False, True, "f16", "f16", (501, 502, 503), kv_cache=True),
}
# causal prefill over context lengths 1K .. 16K (B1 H32 d128, per-tensor V)
for _i, _L in enumerate((1024, 2048, 4096, 8192, 16384)):
    _s = 600 + _i
    WORKLOADS["sweep_%dk" % (_L // 1024)] = W("sweep_%dk" % (_L // 1024), 1, 32, 32, _L, _L, 128, True, False,
                                               "f16", "f16", (_s, _s + 10, _s + 20))

__all__ = ["gaussian", "gaussian_chunked", "outlier_channels", "Workload", "WORKLOADS"]
