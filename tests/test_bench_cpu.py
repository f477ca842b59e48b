"""Host logic of bench.py: the code digest that decides whether committed HBM counter figures
still describe the kernel."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _write(tmp_path, name, text):
    p = tmp_path / name
    p.write_text(text)
    return str(p)


def test_digest_ignores_comments_and_blank_lines(tmp_path):
    a = _write(tmp_path, "a.hip", "int f(int x) {\n  return x + 1;   // one\n}\n")
    b = _write(tmp_path, "b.hip", "/* header\n   more */\nint f(int x) {\n\n  return x + 1;\n}\n")
    assert bench.source_digest([a]) == bench.source_digest([b])


def test_digest_changes_with_code(tmp_path):
    a = _write(tmp_path, "a.hip", "int f(int x) { return x + 1; }\n")
    b = _write(tmp_path, "b.hip", "int f(int x) { return x + 2; }\n")
    assert bench.source_digest([a]) != bench.source_digest([b])


def test_committed_traffic_matches_current_code():
    """The committed counter summary was taken on the code that is in the tree."""
    t = bench.counter_traffic("gemm_fp8_mx16_kernel")
    q = bench.counter_traffic("quantize_tensorwise_kernel")
    assert t is not None and t["bytes"] > 0
    assert q is not None and q["bytes"] > 0
