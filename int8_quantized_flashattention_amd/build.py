"""Builds libattn_int8.so (HIP for gfx950) in-tree.

Every source under csrc/ is compiled by hipcc for gfx950 only, then linked
into one shared library next to this file. Packed-fp32 instruction selection
is switched off for device code. The measurement kernels under probes/ (the
benchmark's MFMA-loop and HBM-read peaks) go into libattn_probes.so.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libattn_int8.so")
PROBES = os.path.join(HERE, "probes")
PROBE_LIB = os.path.join(HERE, "libattn_probes.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = ["-std=c++17", "-O3", "-fPIC", "--offload-arch=" + ARCH, "-I" + INCLUDE, "-I" + CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]


# Per-source code generation options. The fused attention kernel keeps its
# MFMA results in VGPRs: its softmax reads every logit with VALU instructions,
# and accumulator-register results would need a copy per value.
EXTRA = {"attn_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    return obj, out


def _link(objs, lib):
    tmp = lib + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, *objs], check=True)
    os.replace(tmp, lib)


def build(verbose=False):
    """Compile every csrc source for gfx950 and link libattn_int8.so; compile
    the probes into libattn_probes.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    probes = sorted(glob.glob(os.path.join(PROBES, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probes))) as ex:
        results = list(ex.map(_compile, srcs + probes))
    for _, out in results:
        if verbose and out.strip():
            print(out)
    _link([o for o, _ in results[:len(srcs)]], LIB)
    _link([o for o, _ in results[len(srcs):]], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
