"""Random sweep of wide attention problems, GPU path against the oracle.

Run by hand on a GPU host (not collected by pytest):

    python tests/sweep_random_wide.py --n 300 --log sweep.log
    python tests/sweep_random_wide.py --decode --n 1000 --log sweep_decode.log
    python tests/sweep_random_wide.py --lut --n 1000 --log sweep_lut.log
    python tests/sweep_random_wide.py --int4 --n 1000 --log sweep_int4.log
    python tests/sweep_random_wide.py --hadamard --n 1000 --log sweep_hadamard.log

Problem i draws its shape and options from PCG64(70000 + i): B 1-3, query
heads 1-16 with 1, 2, 4 or 8 query heads per KV head, Lq up to 2000 and Lkv
up to 3000 (Lq <= Lkv when causal), d 64 or 128, causal or not, each V scale
granularity, fp16 or fp32 O, fp16 or fp32 inputs, and for half of the
problems outlier channels (1-2 % of d, the same in Q and K) scaled x20.
Problem 0 is the fixed wide outlier case of test_gpu_attention.py. Every row
is compared. A problem that misses the O tolerance (max-abs 2e-2 and relative
Frobenius 1e-2) or the lse bound (1e-4) is recorded and the sweep goes on; a
mismatch of a bit-exact check (codes, scales, the fused-Q forward) is
recorded too. The last line summarises the count and the worst case.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

from gpu_parity import O_MAX_ABS, O_REL_FRO, run_problem  # noqa: E402
from workloads import gaussian  # noqa: E402
from test_gpu_index_softmax import run_lut  # noqa: E402
from test_gpu_int4 import run_int4  # noqa: E402
from test_gpu_hadamard import run_rotated  # noqa: E402


def problem(i):
    if i == 0:
        return dict(B=3, H=16, Hkv=2, Lq=1003, Lkv=2228, d=64, causal=True, vmode=False, o="f32",
                    dt="f16", outliers=[3, 59], seeds=(50008, 50009, 50010))
    r = np.random.Generator(np.random.PCG64(70000 + i))
    d = int(r.choice([64, 128]))
    g = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.integers(1, 17 // g + 1)) if g < 16 else 1
    H = Hkv * g
    B = int(r.integers(1, 4))
    causal = bool(r.integers(0, 2))
    Lkv = int(r.integers(1, 3001))
    Lq = int(r.integers(1, min(2000, Lkv) + 1)) if causal else int(r.integers(1, 2001))
    vmode = [False, True, "head", "channel"][int(r.integers(0, 4))]
    o = ["f16", "f32"][int(r.integers(0, 2))]
    dt = ["f16", "f32"][int(r.integers(0, 2))]
    outliers = None
    if r.integers(0, 2):
        n = int(r.integers(1, max(1, round(0.02 * d)) + 1))
        outliers = sorted(int(c) for c in r.choice(d, size=n, replace=False))
    base = 100000 + 10 * i
    return dict(B=B, H=H, Hkv=Hkv, Lq=Lq, Lkv=Lkv, d=d, causal=causal, vmode=vmode, o=o, dt=dt,
                outliers=outliers, seeds=(base, base + 1, base + 2))


def decode_problem(i):
    """Problem i of the decode-shaped sweep, from PCG64(90000 + i): at most 16
    query rows per KV head (the split-KV path): B 1-8, 1-8 KV heads with 1, 2,
    4 or 8 query heads each, Lq 1-4 (causal or not when Lq > 1), Lkv 1-20000,
    d 64 or 128, each V granularity, fp16 or fp32 inputs and O, half of the
    problems with 1-2 % of the channels of Q and K x20."""
    r = np.random.Generator(np.random.PCG64(90000 + i))
    d = int(r.choice([64, 128]))
    g = int(r.choice([1, 2, 4, 8]))
    Lq = int(r.integers(1, 16 // g + 1)) if g < 16 else 1
    Lq = min(Lq, 4)
    Hkv = int(r.integers(1, 9))
    B = int(r.integers(1, 9))
    Lkv = int(r.integers(max(Lq, 1), 20001))
    causal = bool(r.integers(0, 2)) and Lq > 1
    vmode = [False, True, "head", "channel"][int(r.integers(0, 4))]
    o = ["f16", "f32"][int(r.integers(0, 2))]
    dt = ["f16", "f32"][int(r.integers(0, 2))]
    outliers = None
    if r.integers(0, 2):
        n = int(r.integers(1, max(1, round(0.02 * d)) + 1))
        outliers = sorted(int(c) for c in r.choice(d, size=n, replace=False))
    base = 200000 + 10 * i
    return dict(B=B, H=Hkv * g, Hkv=Hkv, Lq=Lq, Lkv=Lkv, d=d, causal=causal, vmode=vmode, o=o, dt=dt,
                outliers=outliers, seeds=(base, base + 1, base + 2))


def lut_problem(i):
    """Problem i of the IndexSoftmax sweep, from PCG64(110000 + i): prefill
    shapes (Lq up to 2000, Lkv up to 3000) and, for 30 % of the problems,
    decode shapes (at most 16 query rows per KV head); B 1-3, 1-8 KV heads with
    GQA 1-8, d 64 or 128, causal or not, table bits 1-8 and clip 0.5-8, V per
    tensor, head or channel, fp16 or fp32 inputs and O, half of the problems
    with 1-2 % of the channels of Q and K x20."""
    r = np.random.Generator(np.random.PCG64(110000 + i))
    d = int(r.choice([64, 128]))
    g = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.integers(1, 9))
    B = int(r.integers(1, 4))
    causal = bool(r.integers(0, 2))
    if r.random() < 0.3:
        Lq = int(r.integers(1, 16 // g + 1))
        Lkv = int(r.integers(Lq, 12001))
    else:
        Lkv = int(r.integers(1, 3001))
        Lq = int(r.integers(1, min(2000, Lkv) + 1)) if causal else int(r.integers(1, 2001))
    vmode = ["tensor", "head", "channel"][int(r.integers(0, 3))]
    o = ["f16", "f32"][int(r.integers(0, 2))]
    dt = ["f16", "f32"][int(r.integers(0, 2))]
    bits = int(r.integers(1, 9))
    clip = round(float(r.uniform(0.5, 8.0)), 2)
    outliers = None
    if r.integers(0, 2):
        n = int(r.integers(1, max(1, round(0.02 * d)) + 1))
        outliers = sorted(int(c) for c in r.choice(d, size=n, replace=False))
    base = 300000 + 10 * i
    return dict(B=B, H=Hkv * g, Hkv=Hkv, Lq=Lq, Lkv=Lkv, d=d, causal=causal, vmode=vmode, o=o, dt=dt,
                bits=bits, clip=clip, outliers=outliers, seeds=(base, base + 1, base + 2))


def int4_problem(i):
    """Problem i of the INT4 Q.K sweep, from PCG64(130000 + i): 70 % decode
    shapes (the packed-K split-KV kernel, Lkv up to 12000), 30 % prefill shapes
    (K widened in the workspace, Lq up to 1000, Lkv up to 3000); B 1-3, 1-8 KV
    heads with GQA 1-8, d 64 or 128, causal or not, V per tensor, token, head
    or channel, fp16 or fp32 inputs and O, half with outlier channels."""
    r = np.random.Generator(np.random.PCG64(130000 + i))
    d = int(r.choice([64, 128]))
    g = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.integers(1, 9))
    B = int(r.integers(1, 4))
    causal = bool(r.integers(0, 2))
    if r.random() < 0.7:
        Lq = int(r.integers(1, 16 // g + 1))
        Lkv = int(r.integers(Lq, 12001))
    else:
        Lkv = int(r.integers(1, 3001))
        Lq = int(r.integers(1, min(1000, Lkv) + 1)) if causal else int(r.integers(1, 1001))
    vmode = ["tensor", "token", "head", "channel"][int(r.integers(0, 4))]
    o = ["f16", "f32"][int(r.integers(0, 2))]
    dt = ["f16", "f32"][int(r.integers(0, 2))]
    outliers = None
    if r.integers(0, 2):
        n = int(r.integers(1, max(1, round(0.02 * d)) + 1))
        outliers = sorted(int(c) for c in r.choice(d, size=n, replace=False))
    base = 400000 + 10 * i
    return dict(B=B, H=Hkv * g, Hkv=Hkv, Lq=Lq, Lkv=Lkv, d=d, causal=causal, vmode=vmode, o=o, dt=dt,
                outliers=outliers, seeds=(base, base + 1, base + 2))


def hadamard_problem(i):
    """Problem i of the Hadamard sweep, from PCG64(150000 + i): Q and K rotated
    before quantization; 30 % decode shapes (Lkv up to 12000), 70 % prefill
    shapes (Lq up to 2000, Lkv up to 3000); B 1-3, 1-8 KV heads with GQA 1-8,
    d 64 or 128, causal or not, V per tensor, token, head or channel, fp16 or
    fp32 inputs and O, half with outlier channels."""
    p = int4_problem(i)
    r = np.random.Generator(np.random.PCG64(150000 + i))
    g = p["H"] // p["Hkv"]
    causal = bool(r.integers(0, 2))
    if r.random() < 0.3:
        Lq = int(r.integers(1, 16 // g + 1))
        Lkv = int(r.integers(Lq, 12001))
    else:
        Lkv = int(r.integers(1, 3001))
        Lq = int(r.integers(1, min(2000, Lkv) + 1)) if causal else int(r.integers(1, 2001))
    base = 500000 + 10 * i
    return dict(p, Lq=Lq, Lkv=Lkv, causal=causal, seeds=(base, base + 1, base + 2))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--n", type=int, default=300, help="random problems after the fixed one")
    ap.add_argument("--log", default=None, help="also append the lines to this file")
    ap.add_argument("--decode", action="store_true",
                    help="decode-shaped problems (at most 16 query rows per KV head: split-KV path)")
    ap.add_argument("--hadamard", action="store_true",
                    help="Q and K rotated by the normalized Hadamard matrix (quantizer and fused-Q forward)")
    ap.add_argument("--int4", action="store_true",
                    help="INT4 Q.K problems (attn_int4qk_fwd against the oracle on the same 4-bit codes)")
    ap.add_argument("--lut", action="store_true",
                    help="IndexSoftmax problems (attn_int8_fwd_index_softmax against the oracle's table path)")
    args = ap.parse_args()
    import int8_quantized_flashattention_amd as lib

    out = open(args.log, "a") if args.log else None

    def emit(line):
        print(line, flush=True)
        if out:
            out.write(line + "\n")
            out.flush()

    n_ok = 0
    worst = None
    t0 = time.time()
    for i in range(args.n + 1):
        p = (lut_problem(i) if args.lut else int4_problem(i) if args.int4 else hadamard_problem(i) if args.hadamard
             else decode_problem(i) if args.decode else problem(i))
        dt = np.float16 if p["dt"] == "f16" else np.float32
        sq_, sk_, sv_ = p["seeds"]
        q = gaussian((p["B"], p["H"], p["Lq"], p["d"]), sq_, dt, p["outliers"])
        k = gaussian((p["B"], p["Hkv"], p["Lkv"], p["d"]), sk_, dt, p["outliers"])
        v = gaussian((p["B"], p["Hkv"], p["Lkv"], p["d"]), sv_, dt)
        m = {}
        err = None
        try:
            if args.lut:
                run_lut(lib, q, k, v, p["causal"], p["vmode"], p["o"], p["bits"], p["clip"], tag="lut%d" % i,
                        measure=m)
            elif args.int4:
                run_int4(lib, q, k, v, p["causal"], p["vmode"], p["o"], tag="int4_%d" % i, measure=m)
            elif args.hadamard:
                run_rotated(lib, q, k, v, p["causal"], p["vmode"], p["o"], tag="rot%d" % i, measure=m)
            else:
                run_problem(lib, q, k, v, p["causal"], p["vmode"], p["o"], tag="sweep%d" % i, measure=m)
        except AssertionError as e:          # a bit-exact check failed
            err = "bit-exact: %r" % (e.args,)
        ok = (err is None and m["finite"] and m["max_abs"] <= O_MAX_ABS and m["rel_fro"] <= O_REL_FRO
              and m["lse_err"] <= (1e-5 if args.lut else 1e-4) and m.get("strict", True))
        n_ok += ok
        rec = dict(i=i, ok=bool(ok), err=err, **{k_: v_ for k_, v_ in p.items() if k_ != "seeds"}, **m)
        if m and (worst is None or m["max_abs"] > worst["max_abs"]):
            worst = rec
        emit(json.dumps(rec))
    emit("SUMMARY %s" % json.dumps(dict(problems=args.n + 1, passed=n_ok, failed=args.n + 1 - n_ok,
                                        worst_max_abs=worst, seconds=round(time.time() - t0, 1))))
    return 0


if __name__ == "__main__":
    sys.exit(main())
