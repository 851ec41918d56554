"""Builds the CPU emulation driver of libattn_int8 (test infrastructure).

The library's HIP sources are compiled unchanged as host C++ against the
stand-in headers in this folder, with AddressSanitizer and UBSan, into one
executable (emu_driver.cpp calls the C ABI on exact-size host buffers). A
second build uses ThreadSanitizer instead: the emulated lanes are threads that
meet at std::barrier for every wavefront and workgroup barrier, so an LDS or
cross-lane access that the kernels do not order by a barrier is a data race.
"""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "int8_quantized_flashattention_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "emu_driver")
OUT_TSAN = os.path.join(ROOT, "_build", "emu_driver_tsan")
CXX = os.environ.get("EMU_CXX", "/opt/rocm/llvm/bin/clang++")


def inputs():
    return (sorted(glob.glob(os.path.join(CSRC, "*"))) + sorted(glob.glob(os.path.join(HERE, "*.cpp")))
            + sorted(glob.glob(os.path.join(HERE, "hip", "*.h")))
            + [os.path.join(ROOT, "include", "attn_int8.h")])


def build(tsan=False):
    hips = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    cpps = sorted(glob.glob(os.path.join(CSRC, "*.cpp"))) + [os.path.join(HERE, "emu_driver.cpp")]
    out = OUT_TSAN if tsan else OUT
    os.makedirs(os.path.dirname(out), exist_ok=True)
    san = ["-fsanitize=thread"] if tsan else ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    cmd = [CXX, "-std=c++20", "-O1", "-g", *san, "-ffp-contract=off", "-pthread", "-Wno-psabi",
           "-I" + HERE, "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           "-x", "c++", *hips, "-x", "none", *cpps, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def ensure_built(tsan=False):
    out = OUT_TSAN if tsan else OUT
    if not os.path.exists(out) or os.path.getmtime(out) < max(os.path.getmtime(p) for p in inputs()):
        build(tsan)
    return out


if __name__ == "__main__":
    print(build())
