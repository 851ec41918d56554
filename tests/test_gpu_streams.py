"""The stream argument of the C ABI: work goes on the given stream, and calls
on different streams over disjoint outputs do not interact. The same problems
run on the default stream, on one side stream, and concurrently on two side
streams (prefill and split-KV decode at once, each with its own workspace);
every result must equal the default-stream result bit for bit."""
import numpy as np
import pytest
import torch

from gpu_parity import dev
from workloads import gaussian

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import int8_quantized_flashattention_amd as m
    return m


def problem(lib, B, H, Hkv, Lq, Lkv, d, seed):
    q = dev(gaussian((B, H, Lq, d), seed, np.float16))
    k = dev(gaussian((B, Hkv, Lkv, d), seed + 1, np.float16))
    v = dev(gaussian((B, Hkv, Lkv, d), seed + 2, np.float16))
    kh, sk = lib.attn_quantize_rows(k, 1)
    vh, sv = lib.attn_quantize_rows(v, 1)
    return q, kh, sk, vh, sv


def run(lib, p, causal, stream):
    q, kh, sk, vh, sv = p
    B, H, Lq, d = q.shape
    n = lib.attn_int8_fwd_workspace_size(B, H, kh.shape[1], Lq, kh.shape[2], d, causal)
    with torch.cuda.stream(stream):
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda") if n else None
        out = torch.empty((B, H, Lq, d), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    lib.attn_int8_fwd_qfloat(q, kh, sk, vh, sv, True, causal, torch.float32, return_lse=True, out=out, lse=lse,
                             workspace=ws, stream=stream)
    return out, lse, ws


def test_side_streams_give_the_default_stream_results(lib):
    pre = problem(lib, 2, 8, 2, 300, 700, 128, 41)
    dec = problem(lib, 8, 32, 8, 1, 3000, 128, 51)
    torch.cuda.synchronize()
    base = [run(lib, pre, 1, torch.cuda.current_stream()), run(lib, dec, 0, torch.cuda.current_stream())]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    one = [run(lib, pre, 1, s1), run(lib, dec, 0, s1)]
    s1.synchronize()
    both = [run(lib, pre, 1, s1), run(lib, dec, 0, s2)]
    s1.synchronize()
    s2.synchronize()
    for got in (one, both):
        for (o, l, _), (ob, lb, _) in zip(got, base):
            assert torch.equal(o.view(torch.int32), ob.view(torch.int32))
            assert torch.equal(l.view(torch.int32), lb.view(torch.int32))
