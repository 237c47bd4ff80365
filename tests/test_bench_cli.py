"""bench.py's command line on the CPU: a request for more than one GPU is
refused with a message (the path runs on one GPU), before any workload is
built or any device is touched."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def test_counter_records_follow_the_kernel_code_not_its_comments(tmp_path):
    """bench.py keeps a kernel's committed counter figures while only its
    comments change, and drops them once its code changes."""
    sys.path.insert(0, ROOT)
    import bench
    a = tmp_path / "a.hip"
    a.write_text("__global__ void k(float* x) {\n  x[0] = 1.0f;  // one\n}\n")
    b = tmp_path / "b.hip"
    b.write_text("// a header\n__global__ void k(float* x) {\n\n  x[0] = 1.0f;  // another comment\n}\n")
    c = tmp_path / "c.hip"
    c.write_text("__global__ void k(float* x) {\n  x[0] = 2.0f;  // one\n}\n")
    assert bench.code_digest(str(a)) == bench.code_digest(str(b))
    assert bench.code_digest(str(a)) != bench.code_digest(str(c))
