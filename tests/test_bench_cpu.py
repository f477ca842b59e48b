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


def test_committed_traffic_is_used_only_for_its_code(tmp_path, monkeypatch):
    """A summary whose digest matches the sources gives its bytes; a stale one gives None."""
    src = _write(tmp_path, "k.hip", "__global__ void k() {}\n")
    good = bench.source_digest([src])

    def summary(digest):
        f = tmp_path / f"traffic_{digest}.txt"
        f.write_text(f"# header\nkernel k\nsources {src}\ncode_sha256 {digest}\n"
                     "fetch_kib_mean 100.0\nwrite_kib_mean 50.0\n"
                     "fetch_factor 2.0\nwrite_factor 1.0\n")
        return str(f)

    monkeypatch.setattr(bench, "TRAFFIC_FILE", summary(good))
    t = bench.counter_traffic("k")
    assert t == {"bytes": 200 * 1024 + 50 * 1024, "read_bytes": 200 * 1024,
                 "write_bytes": 50 * 1024}
    assert bench.counter_traffic("other") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", summary("0" * 16))
    assert bench.counter_traffic("k") is None


def test_more_than_one_gpu_exits_with_a_message():
    """The hot path runs on one device: --gpus 2 is refused before anything touches a GPU."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_traffic_file_names_existing_sources():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    text = open(os.path.join(root, "profiles", "hbm_traffic_mlp_8192x4096x14336.txt")).read()
    srcs = [ln.split()[1:] for ln in text.splitlines() if ln.startswith("sources ")]
    assert len(srcs) == 2
    for files in srcs:
        for f in files:
            assert os.path.exists(os.path.join(root, f)), f


def test_cpu_baseline_slab_quantize_is_the_oracle():
    """The baseline's quantize in row slabs on threads gives the oracle's codes and transposed
    codes byte for byte (slabs of unequal size included)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import workloads
    from oracle.quantize import amax, quantize_tensorwise
    from oracle.scaling import scale_from_amax
    x = workloads.bf16_tensor("student_t", (100, 48), 3, 99, 0, nu=3)
    _, si = scale_from_amax(amax(x))
    q, q_t, _ = quantize_tensorwise(x, si)
    with ThreadPoolExecutor(3) as pool:
        for slabs in (1, 3, 7):
            sq, sq_t = bench._oracle_quantize_slabs(x, si, pool, slabs)
            assert np.array_equal(sq, q) and np.array_equal(sq_t, q_t), slabs


def test_bench_functions_name_only_defined_names():
    """Every bare name a function of bench.py reads is bound somewhere it can see: its own
    parameters and assignments, an enclosing function's, the module's, or a builtin (the GPU
    paths of bench.py cannot run here, so a missing helper would only show on the GPU)."""
    import ast
    import builtins
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())

    def bound(node):
        names = set()
        for n in ast.walk(node):
            if isinstance(n, ast.Name) and isinstance(n.ctx, (ast.Store, ast.Del)):
                names.add(n.id)
            elif isinstance(n, (ast.FunctionDef, ast.ClassDef)):
                names.add(n.name)
            elif isinstance(n, (ast.Import, ast.ImportFrom)):
                names.update((a.asname or a.name).split(".")[0] for a in n.names)
            elif isinstance(n, ast.arg):
                names.add(n.arg)
            elif isinstance(n, ast.ExceptHandler) and n.name:
                names.add(n.name)
        return names

    module_names = bound(tree) | set(dir(builtins))
    missing = []
    for fn in [n for n in ast.walk(tree) if isinstance(n, ast.FunctionDef)]:
        visible = module_names | bound(fn)
        for n in ast.walk(fn):
            if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load) and n.id not in visible:
                missing.append((fn.name, n.id, n.lineno))
    assert not missing, missing
