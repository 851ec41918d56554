"""Host-side logic of bench.py that needs no GPU: the code hash that keys the
committed traffic summaries, the traffic lookup, and the refusal of more than
one GPU."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FWD = ["attn_fwd.hip", "cdna4_ops.h", "attn_internal.h"]


def test_code_of_drops_comments_and_keeps_literals():
    src = 'int a = 1; // one\n/* two\n three */ const char* s = "// kept /* too */";\nchar c = \'/\';'
    assert bench.code_of(src) == 'int a = 1; const char* s = "// kept /* too */"; char c = \'/\';'
    # layout only: the same code
    assert bench.code_of("int  a=1;\n\n\tint b;") == bench.code_of("int a=1; int b;")
    # an escaped quote does not end the literal
    assert bench.code_of('s = "a\\" // b"; // c') == 's = "a\\" // b";'


def test_code_hash_ignores_comment_edits_only():
    with open(os.path.join(bench.CSRC, "attn_fwd.hip"), encoding="utf-8") as f:
        text = f.read()
    edited = text.replace("\n", "\n// an added comment line\n", 3)
    assert bench.code_of(edited) == bench.code_of(text)
    changed = text.replace("kStages = 4", "kStages = 3", 1)
    assert changed != text and bench.code_of(changed) != bench.code_of(text)


def test_traffic_lookup_follows_the_hash(tmp_path, monkeypatch):
    h = bench.kernel_sources_hash(FWD)
    (tmp_path / "traffic_w.txt").write_text(
        "# x\nkernel_sources: %s\nkernel_sources_sha256: %s\ntraffic_bytes_per_launch: 123\n" % (" ".join(FWD), h))
    (tmp_path / "traffic_stale.txt").write_text(
        "kernel_sources_sha256: 0000000000000000\ntraffic_bytes_per_launch: 456\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("w", FWD) == 123.0
    assert bench.measured_traffic("stale", FWD) is None
    assert bench.measured_traffic("absent", FWD) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "one GPU" in r.stdout, (r.stdout, r.stderr)
