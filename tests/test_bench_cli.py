"""bench.py's host side, without a GPU: the one-GPU guard, the work model it
reports, and the code-only hash that keys the committed counter summary."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_work_model():
    # FLUX-2048, window 16x16, 256 memory tokens: 4*H*n*(m+G)*D flops
    assert bench.window_flops(1, 24, 16384, 256, 256, 128) == 4 * 24 * 16384 * 512 * 128
    assert bench.window_flops(1, 24, 16384, 256, 256, 128) == 103079215104
    assert bench.dense_flops(1, 24, 16384, 128) == 4 * 24 * 16384 ** 2 * 128
    # theoretical speedups n/m and n/(m+G)
    assert bench.dense_flops(1, 1, 16384, 128) / bench.window_flops(1, 1, 16384, 256, 0, 128) == 64
    assert bench.dense_flops(1, 1, 16384, 128) / bench.window_flops(1, 1, 16384, 256, 256, 128) == 32


def test_kernel_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f() {  // one\n  return 1;\n}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["k.hip"])
    h1 = bench.kernel_hash()
    src.write_text("// header\nint f() {  // two\n\n    return 1;\n}\n")
    assert bench.kernel_hash() == h1
    src.write_text("int f() {\n  return 2;\n}\n")
    assert bench.kernel_hash() != h1
