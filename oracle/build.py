"""Builds the CPU oracle shared library (test infrastructure only).

The oracle is plain C++17 compiled by the host compiler with no fast-math and
no floating-point contraction, so every fp32 step is rounded as written.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")

FLAGS = ["-std=c++17", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-pthread"]


# AddressSanitizer + UBSan build (tests only; load it with the host's
# libasan preloaded)
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(out=LIB, plant=None, extra=(), sanitize=False):
    """Compile the oracle into `out`. `plant` names a deliberate mistake, used
    only by the tests that show the pins catch such mistakes; `sanitize`
    builds it with AddressSanitizer and UBSan."""
    cmd = ["g++", *FLAGS, *(SANITIZE if sanitize else ()), *extra]
    if plant is not None:
        cmd.append('-DORACLE_PLANT="%s"' % plant)
    cmd += [SRC, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def ensure_built():
    """Build if the library is missing or older than its source."""
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    return LIB


if __name__ == "__main__":
    print(build(*(sys.argv[1:2] or [LIB])))
