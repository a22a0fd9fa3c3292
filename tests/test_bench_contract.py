"""The benchmark's host-side contract and measurement helpers (no GPU needed).

`bench.py --gpus N` with N above 1 exits with a message (the step runs on one GPU's share of a batch), and
the attention figure counts launches that overlap on two streams once: `busy_us` is the length of the
union of (start, end) intervals, checked here against a brute-force count over a fine grid.
"""
import os
import random
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""


def test_busy_time_is_the_union_of_the_intervals():
    assert bench.busy_us([]) == 0.0
    assert bench.busy_us([(3.0, 5.0)]) == 2.0
    assert bench.busy_us([(0.0, 10.0), (2.0, 4.0)]) == 10.0      # nested
    assert bench.busy_us([(0.0, 4.0), (4.0, 6.0)]) == 6.0        # touching
    assert bench.busy_us([(5.0, 9.0), (0.0, 2.0)]) == 6.0        # unsorted, disjoint
    rng = random.Random(7)
    for _ in range(50):
        iv = []
        for _ in range(rng.randint(1, 8)):
            a = rng.randint(0, 200)
            iv.append((a / 4.0, (a + rng.randint(0, 60)) / 4.0))
        # brute force on the quarter-unit grid the endpoints lie on
        covered = sum(1 for t in range(0, 1040) if any(a <= t / 4.0 < b for a, b in iv))
        assert abs(bench.busy_us(iv) - covered / 4.0) < 1e-9
