"""Host-side behaviour of bench.py that needs no GPU: the one-GPU guard, the
source hash that ties stored counter readings to the kernel code, and the
lookup of stored traffic."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_source_hash_ignores_comments_and_layout():
    a = "int f(int x) {\n    return x + 1;  // one more\n}\n/* block\n comment */\n"
    b = "int f(int x) { return x + 1; }\n"
    strip = lambda t: " ".join(bench._COMMENT.sub(" ", t).split())
    assert strip(a) == strip(b)
    assert strip("return x + 2;") != strip("return x + 1;")
    h = bench.kernel_source_hash("das_bi_rows_kernel")
    assert len(h) == 16 and h == bench.kernel_source_hash("das_bi_rows_kernel")
    # each kernel's readings depend on its own source: the hashes differ
    hashes = {bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES}
    assert len(hashes) == len(bench.KERNEL_SOURCES)


def test_stored_traffic_is_none_for_an_unmeasured_workload():
    assert bench.stored_traffic("das_bi_staged_kernel", "no-such-workload") is None
    assert bench.stored_traffic("no_such_kernel", "main") is None


def test_pick_bound():
    import bench
    # algorithmic bytes slower than the flops: HBM
    assert bench.pick_bound(2.0, 1.0, None, None) == "hbm"
    # counted bytes keep HBM at 48% while the VALU is 83% busy: ALU
    assert bench.pick_bound(0.3, 2.0, 0.48, 0.83) == "alu"
    # counted bytes keep HBM busier than the VALU: HBM
    assert bench.pick_bound(0.3, 2.0, 0.9, 0.6) == "hbm"
    # no counters on these sources: the algorithmic rule alone
    assert bench.pick_bound(0.3, 2.0, 0.9, None) == "alu"
    assert bench.pick_bound(0.3, 2.0, None, 0.6) == "alu"
