"""The kernels' emulation under ThreadSanitizer (CPU).

The same host build of the HIP sources as test_cpu_emulation.py, with
ThreadSanitizer in place of AddressSanitizer: every emulated lane is a thread,
and the lanes of a workgroup meet at std::barrier wherever the kernels have a
wavefront or workgroup barrier (or an s_waitcnt, which the emulation treats as
a wavefront meeting point). An LDS or cross-lane access that no such barrier
orders against another lane's access to the same bytes is reported as a data
race and fails the run (ThreadSanitizer's exit code). Each case is a small
problem that still runs the stage ring over several tiles, ragged tails and
the split-KV merge; the results are checked against the oracle as in the
AddressSanitizer tests.
"""
import os
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "cpu_emu"))

import build_emu  # noqa: E402
import test_cpu_emulation as emu  # noqa: E402

F16, F32 = emu.F16, emu.F32


@pytest.fixture(scope="module")
def exe():
    return build_emu.ensure_built(tsan=True)


@pytest.mark.parametrize("B,H,Hkv,Lq,Lkv,d,causal,vpt,odt,gain", [
    (1, 2, 1, 130, 200, 128, 1, 0, F16, 1),      # prefill, causal, ragged, per-tensor V, four-stage ring
    (1, 2, 2, 77, 330, 64, 0, 1, F32, 4),        # per-token V, growing logits (folds and rescales)
    (1, 2, 1, 65, 130, 128, 1, 3, F32, 1),       # per-channel V
    (1, 8, 2, 1, 700, 128, 0, 0, F16, 1),        # split-KV decode and the merge
])
def test_tsan_attention(exe, tmp_path, B, H, Hkv, Lq, Lkv, d, causal, vpt, odt, gain):
    emu.test_emulated_attention(exe, tmp_path, B, H, Hkv, Lq, Lkv, d, causal, vpt, odt, gain)


def test_tsan_attention_float_q(exe, tmp_path):
    # Q quantized inside the kernel (the lane pair's permlane32_swap maximum)
    emu.test_emulated_attention_float_q(exe, tmp_path, 1, 2, 1, 130, 200, 128, 1, 0, __import__("numpy").float16)


def test_tsan_attention_index_softmax(exe, tmp_path):
    # IndexSoftmax with the pair table built in LDS by the whole workgroup
    emu.test_emulated_attention_index_softmax(exe, tmp_path, 1, 2, 2, 256, 640, 128, 1, 0, F32, 4, 1.5, 12)


@pytest.mark.parametrize("rows,cols,rps", [(100, 128, 10), (64, 128, 64), (257, 64, 1)])
def test_tsan_quantize(exe, tmp_path, rows, cols, rps):
    # per-token teams and the large-group absmax (LDS reduction, atomic max)
    emu.test_emulated_quantize(exe, tmp_path, rows, cols, rps, __import__("numpy").float16)
