"""Benchmark of the INT8 attention forward hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input that is
already resident in HBM: per-token INT8 quantization of K, INT8 quantization
of V (per tensor or per token, as the workload says), and the fused attention
forward, which quantizes Q per token as it loads it (`--q-path separate`
quantizes Q in its own pass and feeds the INT8 forward instead). For the
decode workload K and V sit in an INT8 cache quantized once, before timing; a
step appends the newest token's K and V to the cache (quantize-on-append) and
runs the forward over the whole cache. `value` is algorithmic INT8 ops (4 d per visible
query-key pair) per second of step time, in TOPS.

Also reported on the same JSON line:
  roofline      the fused attention launch alone (prefill kernel, or split-KV
                decode kernel plus chunk merge): its average duration from HIP
                events around each launch in the timed region, against the
                dense INT8 MFMA peak (5.0 POP/s) or, for decode shapes, HBM
                (8 TB/s); `traffic` is the HBM bytes per launch measured with
                rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled by a copy of known
                size), read from profiles/ and given only while the kernel
                sources still match the ones measured
  cpu_baseline  the oracle (plain C++, all host threads given to it) timed on
                a bounded, seeded sample of the workload's query rows
  kernels       per-kernel times (quantize passes, attention) in the timed
                region: mean, median and interquartile range of the HIP-event
                durations
  clocks        shader and memory clocks (MHz) read from the driver's sysfs
                during the timed region
  roofline_int8_q  (prefill, Q quantized in the kernel) the same forward on
                INT8 codes of Q (attn_int8_fwd), timed right after the timed
                region in steps of the separate-Q path: the attention kernel
                without the Q quantization that the fused step moves into its
                prologue
  measured_peaks  second denominators measured on this GPU right after the
                timed region: an INT8 MFMA loop (TOP/s) and a streaming HBM
                read of 2 GiB (GB/s), from libattn_probes

The GPU's clocks ramp up over the first ~100 ms of load, so before the W
warm-up steps the forward runs back to back for --settle-ms of wall time
(untimed, not counted as steps): with a handful of warm-up steps the timed
steps would otherwise land in the ramp.

`--qk int4` times the step with INT4 Q.K: Q and K in per-token 4-bit codes,
K packed two codes per byte (the decode cache is then a packed K cache), Q
quantized in its own pass. `--hadamard` rotates Q and K by the normalized Hadamard matrix as they are
quantized (outlier handling; the attention is unchanged in exact arithmetic);
Q is then rotated inside the attention kernels' Q load.
`--softmax index` times the same step with IndexSoftmax (a 2^b-entry
exponential table, `--lut-bits`, `--lut-clip`) in place of the exp softmax; that
forward takes INT8 Q, so Q is then quantized in its own pass.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--q-path fused|separate] [--softmax exp|index]
       python bench.py --copy-calibration     (1 GiB device copies, for the
                                               HBM counter scale)
       python bench.py --lds-patterns         (the prefill tile's four LDS access
                                               patterns, one launch each, for the
                                               LDS counters of each pattern)
"""
import hashlib
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import WORKLOADS  # noqa: E402

METRIC = "INT8 attention fwd TOPS & % INT8 MFMA peak (B4 H32 L4096 d128, causal)"
PEAK_INT8_TOPS = 5000.0      # MI355X dense INT8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first (the clocks settle over the first tens of ms)")
    ap.add_argument("--workload", default="l4096_outlier", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the oracle sample (0 disables the CPU baseline)")
    ap.add_argument("--q-path", choices=["fused", "separate"], default="fused",
                    help="quantize Q inside the attention kernels (fused) or in its own pass")
    ap.add_argument("--softmax", choices=["exp", "index"], default="exp",
                    help="exp softmax, or IndexSoftmax (table lookup; INT8 Q from its own pass)")
    ap.add_argument("--qk", choices=["int8", "int4"], default="int8",
                    help="INT8 Q.K, or INT4 Q.K: 4-bit codes, K packed two per byte (Q from its own pass)")
    ap.add_argument("--hadamard", action="store_true",
                    help="rotate Q and K by the normalized Hadamard matrix before quantizing them")
    ap.add_argument("--lut-bits", type=int, default=5, help="IndexSoftmax table bits b")
    ap.add_argument("--lut-clip", type=float, default=6.6, help="IndexSoftmax clipping threshold c")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="run the forward back to back this long before the warm-up steps (clock ramp)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the MFMA-loop and HBM-read probes")
    ap.add_argument("--attn-only", action="store_true",
                    help="time only the fused attention launches (for profiling runs)")
    ap.add_argument("--lds-patterns", action="store_true",
                    help="run the prefill tile's LDS access patterns (libattn_probes) once each and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run five 1 GiB device-to-device copies and exit")
    return ap.parse_args()


CSRC = os.path.join(ROOT, "int8_quantized_flashattention_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def code_of(text):
    """C/C++ source without its comments and with runs of whitespace folded,
    so that a change to comments alone leaves the hash below unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":                  # string or character literal
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_sources_hash(names):
    """Hash of the kernel sources' code (comments and layout excluded)."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), encoding="utf-8") as f:
            h.update(code_of(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel_files):
    """HBM bytes per launch from the committed counter summary of this
    workload, or None when there is none or the kernel changed since."""
    path = os.path.join(PROFILES, "traffic_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("kernel_sources_sha256") != kernel_sources_hash(kernel_files):
        return None
    return float(kv["traffic_bytes_per_launch"])


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)


def read_clocks():
    """Current shader / memory clock levels (MHz) from the amdgpu sysfs files,
    or {} where the driver does not expose them."""
    import glob
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        for key, name in (("sclk_mhz", "pp_dpm_sclk"), ("mclk_mhz", "pp_dpm_mclk")):
            try:
                with open(os.path.join(dev, name)) as f:
                    for line in f:
                        if "*" in line:
                            out[key] = float(line.split(":")[1].strip().split("M")[0].split("m")[0])
            except (OSError, ValueError, IndexError):
                pass
        if out:
            break
    return out


class ClockSampler:
    """Samples read_clocks() every few ms on a host thread while the timed
    region runs; reports the median and range of each clock."""

    def __init__(self):
        import threading
        self.samples = []
        self.stop = threading.Event()
        self.th = threading.Thread(target=self.run, daemon=True)

    def run(self):
        while not self.stop.is_set():
            c = read_clocks()
            if not c:
                return
            self.samples.append(c)
            self.stop.wait(0.002)

    def __enter__(self):
        self.th.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        self.th.join()

    def summary(self):
        if not self.samples:
            return {"source": "sysfs pp_dpm_sclk / pp_dpm_mclk not readable"}
        out = {"source": "amdgpu sysfs pp_dpm_sclk / pp_dpm_mclk during the timed region",
               "samples": len(self.samples)}
        for key in ("sclk_mhz", "mclk_mhz"):
            v = [c[key] for c in self.samples if key in c]
            if v:
                out[key] = float(np.median(v))
                out[key + "_range"] = [min(v), max(v)]
        return out


def measured_peaks(torch):
    """INT8 MFMA-loop rate and streaming HBM read rate of this GPU (median of
    five launches each, after one warm-up launch)."""
    import ctypes
    path = os.path.join(ROOT, "int8_quantized_flashattention_amd", "libattn_probes.so")
    lib = ctypes.CDLL(path)
    lib.attn_probe_mfma_i8.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def timed(fn, reps=5):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    n_blocks, iters = 512, 2000                      # two 4-wavefront groups per CU
    mout = torch.empty(n_blocks * 256 * 16, dtype=torch.int32, device="cuda")

    def mfma():
        assert lib.attn_probe_mfma_i8(n_blocks, iters, ctypes.c_void_p(mout.data_ptr()), sp) == 0

    t_m = timed(mfma)
    mfma_ops = n_blocks * 4 * iters * 4 * 65536
    nbytes = 2 << 30                                 # 2 GiB: far past the 256 MB last-level cache
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    best = (0.0, None)
    for hb in (1024, 2048, 4096):                    # workgroups; each streams one contiguous slice
        for nt in (0, 1):
            hout = torch.empty(hb * 256, dtype=torch.int32, device="cuda")

            def hbm():
                assert lib.attn_probe_hbm_read(ctypes.c_void_p(src.data_ptr()), nbytes, hb, nt,
                                               ctypes.c_void_p(hout.data_ptr()), sp) == 0

            gbs = nbytes / timed(hbm) / 1e9
            if gbs > best[0]:
                best = (gbs, (hb, nt))
    del src
    return {"mfma_i8_tops": round(mfma_ops / t_m / 1e12, 1),
            "hbm_read_gbs": round(best[0], 1),
            "probe": "libattn_probes: 512 groups x 4 wavefronts x 2000 rounds of 4 independent "
                     "v_mfma_i32_32x32x32_i8; a 2 GiB read in contiguous slices with 16-byte loads, best of "
                     "1024/2048/4096 workgroups with and without the non-temporal policy (%d, nt=%d); "
                     "medians of 5 launches" % best[1]}


def lds_patterns():
    """One launch per LDS access pattern of the prefill tile (K operand reads,
    transposing V reads, scale reads, LDS-destination loads): 512 workgroups x
    200 rounds each, so a counter run sees each pattern alone."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "int8_quantized_flashattention_amd", "libattn_probes.so"))
    lib.attn_probe_lds_patterns.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_void_p]
    src = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    out = torch.empty(512 * 256, dtype=torch.int32, device="cuda")
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    names = ["k_operand_ds_read_b128", "v_operand_ds_read_b64_tr_b8", "scale_ds_read_b128", "stage_buffer_load_lds"]
    for mode, name in enumerate(names):
        assert lib.attn_probe_lds_patterns(mode, ctypes.c_void_p(src.data_ptr()), 512, 200,
                                           ctypes.c_void_p(out.data_ptr()), sp) == 0
    torch.cuda.synchronize()
    print(json.dumps({"lds_patterns": names, "workgroups": 512, "rounds": 200}), flush=True)


def host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(w, q, k, v, target_s, index_softmax=None, q4=False):
    """Time the oracle's INT8 attention on a seeded sample of rows, scaled so
    the timed call lasts about target_s seconds."""
    import oracle
    rps_v = 1 if w.v_per_token else v.size // w.d
    quant = oracle.quantize_rows_int4 if q4 else (lambda x: oracle.quantize_rows(x, 1))
    qh, sq = quant(q)
    kh, sk = quant(k)
    vh, sv = oracle.quantize_rows(v, rps_v)
    import int8_quantized_flashattention_amd as m
    tile, split = m.attn_int8_fwd_schedule(w.B, w.H, w.Hkv, w.Lq, w.Lkv, w.d, w.causal)
    nth = host_threads()
    total_rows = w.B * w.H * w.Lq
    rng = np.random.Generator(np.random.PCG64(12345))

    def ops_of(rows):
        i = rows % w.Lq
        keys = np.minimum(w.Lkv, i + (w.Lkv - w.Lq) + 1) if w.causal else np.full(rows.shape, w.Lkv)
        return float(4 * w.d * keys.sum())

    n = min(total_rows, 64 * nth)
    while True:
        rows = np.sort(rng.choice(total_rows, size=n, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        oracle.attn_int8(qh, sq, kh, sk, vh, sv, w.v_per_token, w.B, w.H, w.Hkv, w.Lq, w.Lkv, w.d,
                         w.causal, tile, split, rows=rows, nthreads=nth, index_softmax=index_softmax)
        dt = time.perf_counter() - t0
        if dt >= 0.5 * target_s or n >= total_rows:
            break
        n = int(min(total_rows, max(2 * n, n * target_s / max(dt, 1e-3))))
    return {"value": ops_of(rows) / dt / 1e12, "unit": "TOPS", "cores": nth, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": "%d of %d query rows (seeded uniform sample), INT8 attention step only "
                      "(quantization excluded)%s, %d host threads"
                      % (rows.size, total_rows, ", IndexSoftmax" if index_softmax else ", INT4 Q.K codes" if q4 else "",
                         nth)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import int8_quantized_flashattention_amd as m

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.lds_patterns:
        lds_patterns()
        return
    w = WORKLOADS[args.workload]
    q, k, v = w.inputs()
    dq, dk, dv = (torch.from_numpy(a).cuda() for a in (q, k, v))
    d = w.d
    rps_v = 1 if w.v_per_token else v.size // d
    # outputs and quantized buffers allocated once, outside the timed region
    qh = torch.empty(dq.shape, dtype=torch.int8, device="cuda")
    kh = torch.empty(dk.shape, dtype=torch.int8, device="cuda")
    vh = torch.empty(dv.shape, dtype=torch.int8, device="cuda")
    sq = torch.empty(dq.numel() // d, dtype=torch.float32, device="cuda")
    sk = torch.empty(dk.numel() // d, dtype=torch.float32, device="cuda")
    sv = torch.empty(dv.numel() // d // rps_v, dtype=torch.float32, device="cuda")
    odt = torch.float16 if w.o_dtype == "f16" else torch.float32
    o = torch.empty((w.B, w.H, w.Lq, d), dtype=odt, device="cuda")
    ws_n = m.attn_int8_fwd_workspace_size(w.B, w.H, w.Hkv, w.Lq, w.Lkv, d, w.causal)
    ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device="cuda") if ws_n else None
    stream = torch.cuda.current_stream()

    lut = args.softmax == "index"
    lut_args = (args.lut_bits, float(np.float32(args.lut_clip))) if lut else None
    if lut and w.v_per_token:
        print("IndexSoftmax takes V scales constant along the keys; workload %s has per-token V"
              % w.name, file=sys.stderr)
        sys.exit(2)
    q4 = args.qk == "int4"
    if lut and q4:
        print("IndexSoftmax and INT4 Q.K are separate forwards", file=sys.stderr)
        sys.exit(2)
    rot = args.hadamard
    if rot and w.kv_cache:
        print("--hadamard rotates K as it is quantized; the decode cache appends unrotated tokens", file=sys.stderr)
        sys.exit(2)
    fused_q = args.q_path == "fused" and not lut and not q4   # these take INT8 codes of Q
    if q4:
        kh = torch.empty(dk.shape[:-1] + (d // 2,), dtype=torch.uint8, device="cuda")   # packed 4-bit K
        ws_n = m.attn_int4qk_fwd_workspace_size(w.B, w.H, w.Hkv, w.Lq, w.Lkv, d, w.causal)
        ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device="cuda") if ws_n else None
    if w.kv_cache:
        assert w.v_per_token, "an appendable cache has per-token V scales"
        # the cache holds every token; each step re-appends the newest one
        # (position Lkv - 1) with the same values
        if q4:
            m.attn_quantize_rows_int4(dk, codes=False, packed=kh, scales=sk)
        else:
            m.attn_quantize_rows(dk, 1, kh, sk)
        m.attn_quantize_rows(dv, 1, vh, sv)
        k_new, v_new = dk[:, :, -1:].contiguous(), dv[:, :, -1:].contiguous()

    def quantize():
        if rot:
            bits = 4 if q4 else 8
            if not fused_q:
                m.attn_quantize_rows_hadamard(dq, bits, codes=qh, packed=False, scales=sq)
            m.attn_quantize_rows_hadamard(dk, bits, codes=False if q4 else kh, packed=kh if q4 else False, scales=sk)
            m.attn_quantize_rows(dv, rps_v, vh, sv)
            return
        if q4:
            m.attn_quantize_rows_int4(dq, codes=qh, packed=False, scales=sq)
        elif not fused_q:
            m.attn_quantize_rows(dq, 1, qh, sq)
        if w.kv_cache:
            if q4:
                m.attn_kv_append_int4(k_new, kh, sk, w.Lkv - 1)
            else:
                m.attn_kv_append(k_new, kh, sk, w.Lkv - 1)
            m.attn_kv_append(v_new, vh, sv, w.Lkv - 1)
            return
        if q4:
            m.attn_quantize_rows_int4(dk, codes=False, packed=kh, scales=sk)
        else:
            m.attn_quantize_rows(dk, 1, kh, sk)
        m.attn_quantize_rows(dv, rps_v, vh, sv)

    def attend():
        if q4:
            m.attn_int4qk_fwd(qh, sq, kh, sk, vh, sv, w.v_per_token, w.causal, odt, out=o, workspace=ws)
        elif lut:
            m.attn_int8_fwd_index_softmax(qh, sq, kh, sk, vh, sv, w.v_per_token, w.causal, odt, lut_args[0],
                                          lut_args[1], out=o, workspace=ws)
        elif fused_q:
            m.attn_int8_fwd_qfloat(dq, kh, sk, vh, sv, w.v_per_token, w.causal, odt, out=o, workspace=ws,
                                   hadamard=rot)
        else:
            m.attn_int8_fwd(qh, sq, kh, sk, vh, sv, w.v_per_token, w.causal, odt, out=o, workspace=ws)

    quantize()
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(8):
            attend()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        if not args.attn_only:
            quantize()
        attend()
    quantize()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        for e0, e1, e2 in ev:
            e0.record(stream)
            if not args.attn_only:
                quantize()
            e1.record(stream)
            attend()
            e2.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    step_ms = wall * 1e3 / args.steps
    attn_t = np.array([e1.elapsed_time(e2) for _, e1, e2 in ev])
    quant_t = np.array([e0.elapsed_time(e1) for e0, e1, _ in ev])
    attn_ms = float(np.mean(attn_t))
    quant_ms = float(np.mean(quant_t))

    def stats(t):
        q1, med, q3 = np.percentile(t, [25, 50, 75])
        return {"mean": round(float(np.mean(t)), 4), "median": round(float(med), 4),
                "iqr": [round(float(q1), 4), round(float(q3), 4)]}

    ops = float(w.ops())
    value = ops / (step_ms * 1e-3) / 1e12
    kernel_tops = ops / (attn_ms * 1e-3) / 1e12
    tile, split = m.attn_int8_fwd_schedule(w.B, w.H, w.Hkv, w.Lq, w.Lkv, d, w.causal)
    kv_bytes = (1.5 if q4 else 2) * w.B * w.Hkv * w.Lkv * d + 4 * 2 * w.B * w.Hkv * w.Lkv
    q_bytes = q.nbytes if fused_q else q.size + 4 * w.B * w.H * w.Lq
    o_bytes = w.B * w.H * w.Lq * d * (2 if w.o_dtype == "f16" else 4)
    attn_bytes = q_bytes + kv_bytes + o_bytes      # compulsory HBM bytes
    # quantize passes, compulsory bytes: read x once, write codes and scales
    # (one scale for a per-tensor V; its absmax pass re-reads V, mostly from
    # the last-level cache, and that re-read is not counted)
    quantized = [k, v] if not w.kv_cache else [k[:, :, -1:], v[:, :, -1:]]
    if not fused_q:
        quantized.append(q)
    quant_bytes = sum(x.nbytes + x.size + 4 * (x.size // d) for x in quantized)
    if q4:      # K's codes are half a byte each
        quant_bytes -= quantized[0].size // 2
    if not w.v_per_token:
        quant_bytes -= 4 * (v.size // d) - 4

    bound_mfma = ops / attn_bytes > PEAK_INT8_TOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if bound_mfma:
        roof = {"bound": "mfma", "achieved": round(kernel_tops, 2), "peak": PEAK_INT8_TOPS,
                "unit": "TOP/s", "frac": round(kernel_tops / PEAK_INT8_TOPS, 4), "traffic": None}
    else:
        gbs = attn_bytes / (attn_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
    decode = m.attn_int8_fwd_workspace_size(w.B, w.H, w.Hkv, w.Lq, w.Lkv, d, w.causal) > 0
    if decode:
        roof["kernel"] = "attn_decode_kernel + attn_decode_combine"
        kfiles = ["attn_decode.hip", "cdna4_ops.h", "attn_internal.h"]
    else:
        roof["kernel"] = "attn_fwd_kernel"
        kfiles = ["attn_fwd.hip", "cdna4_ops.h", "attn_internal.h"]
    if lut:
        roof["kernel"] += " (IndexSoftmax)"
    if q4:
        roof["kernel"] += " (INT4 Q.K, packed K)" if decode else " (INT4 Q.K: K widened, then the INT8 kernel)"
    if rot:
        roof["kernel"] += " (Hadamard-rotated Q and K)"
    roof["traffic"] = measured_traffic(w.name + ("_index_softmax" if lut else "_int4qk" if q4 else "_hadamard" if rot
                                                 else "" if fused_q else "_separate_q"), kfiles)
    roof["kernel_ms"] = round(attn_ms, 4)
    roof["algorithmic_per_launch"] = ops if bound_mfma else attn_bytes
    # the same forward on INT8 codes of Q: steps of the separate-Q path (K, V
    # and Q quantized in their own passes, then attn_int8_fwd), run right after
    # the timed region with events around the forward alone. This is the
    # attention kernel without the Q quantization in its prologue. (Launched
    # back to back with no quantize passes between them, the forwards run
    # slower: the clock drops under the sustained matrix-core load.)
    int8_q = None
    if fused_q and bound_mfma and not rot and not args.attn_only:
        def step8():
            quantize()
            m.attn_quantize_rows(dq, 1, qh, sq)
        ev8 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for _ in range(max(args.warmup, 10)):
            step8()
            m.attn_int8_fwd(qh, sq, kh, sk, vh, sv, w.v_per_token, w.causal, odt, out=o, workspace=ws)
        for e1, e2 in ev8:
            step8()
            e1.record(stream)
            m.attn_int8_fwd(qh, sq, kh, sk, vh, sv, w.v_per_token, w.causal, odt, out=o, workspace=ws)
            e2.record(stream)
        torch.cuda.synchronize()
        t8 = np.array([e1.elapsed_time(e2) for e1, e2 in ev8])
        tops8 = ops / (float(np.mean(t8)) * 1e-3) / 1e12
        int8_q = {"kernel": "attn_fwd_kernel on INT8 Q (attn_int8_fwd), timed in steps of the separate-Q "
                            "path (quantize K, V and Q, then the forward); not the step timed above",
                  "kernel_ms": round(float(np.mean(t8)), 4), "times_ms": stats(t8),
                  "achieved": round(tops8, 2), "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                  "frac": round(tops8 / PEAK_INT8_TOPS, 4)}
    peaks = None if args.no_peaks else measured_peaks(torch)
    if peaks:
        mp = peaks["mfma_i8_tops"] if bound_mfma else peaks["hbm_read_gbs"]
        roof["measured_peak"] = mp
        roof["frac_of_measured_peak"] = round(roof["achieved"] / mp, 4)
        if int8_q:
            int8_q["frac_of_measured_peak"] = round(int8_q["achieved"] / mp, 4)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "Lq": w.Lq, "Lkv": w.Lkv,
                   "d": d, "causal": bool(w.causal),
                   "v_scale": "per_token" if w.v_per_token else "per_tensor",
                   "inputs": "%s N(0,1)%s" % (w.in_dtype, ", 1 percent of head-dim channels x20 in Q and K"
                                              if w.outlier_seed is not None else ""),
                   "o_dtype": w.o_dtype, "kv_tile": tile, "kv_split_len": split,
                   "kv_cache": bool(w.kv_cache),
                   "softmax": "index_softmax(b=%d, c=%g)" % lut_args if lut else "exp",
                   "qk": args.qk, "hadamard_qk": bool(rot),
                   "step": ("attention only" if args.attn_only else
                            ("append the new token's K,V to the %s cache" % ("INT4-K/INT8-V" if q4 else "INT8")
             if w.kv_cache else "quantize K,V")
                            + (" + fused attention (Q quantized in the kernel)" if fused_q else
                               " + quantize Q + fused attention"))},
        "roofline": roof,
        "roofline_int8_q": int8_q,
        "kernels": {"attention_ms": round(attn_ms, 4), "quantize_ms": round(quant_ms, 4),
                    "attention": stats(attn_t), "quantize": stats(quant_t),
                    "attention_tops": round(kernel_tops, 2),
                    "quantize_gbs": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1)
                    if quant_ms > 0 and not args.attn_only else None},
        "clocks": clk.summary(),
        "settle_ms": args.settle_ms,
    }
    if peaks:
        out["measured_peaks"] = peaks
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds, lut_args, q4)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
