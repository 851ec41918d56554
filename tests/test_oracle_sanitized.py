"""The oracle built with AddressSanitizer and UBSan passes every pin: no pin
input makes it read or write outside a buffer, overflow a signed integer or
hit other undefined behaviour. The pins run in a child process with the
host's libasan preloaded (the sanitized library cannot be loaded otherwise)."""
import os
import subprocess
import sys

from oracle import build as obuild

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

CHILD = r'''
import sys
sys.path[:0] = [%r, %r]
import numpy as np
import oracle
from oracle_pins import ALL_PINS
L = oracle.lib(%r)
maps = open("/proc/self/maps").read()
assert "libasan" in maps and "libubsan" in maps, "sanitizer runtimes not loaded"
print("sanitizers loaded", flush=True)
with np.errstate(all="ignore"):
    for pin in ALL_PINS:
        pin(L)
        print("ok", pin.__name__, flush=True)
'''


def test_pins_pass_under_asan_and_ubsan(tmp_path):
    path = obuild.build(out=os.path.join(str(tmp_path), "liboracle_asan.so"), sanitize=True)
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", CHILD % (ROOT, HERE, path)], env=env, capture_output=True,
                       text=True, timeout=1200)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    from oracle_pins import ALL_PINS
    assert "sanitizers loaded" in r.stdout
    assert r.stdout.count("ok ") == len(ALL_PINS)
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
