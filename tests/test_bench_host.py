"""Host-side logic of bench.py: the one-GPU guard, the count of (query, key)
pairs the masks keep (against brute force over tiny sequences), and the CPU
baseline's record on a bounded sample."""
import os
import subprocess
import sys

import numpy as np

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _brute_pairs(lengths, targets=None):
    n = 0
    for i, s in enumerate(lengths):
        t = 0 if targets is None else min(max(int(targets[i]), 0), s)
        hist = s - t
        for r in range(s):
            for c in range(r + 1):
                if targets is None or c < hist or c == r:
                    n += 1
    return n


def test_seen_pairs_matches_brute_force():
    lengths = [0, 1, 5, 33, 70]
    case = workloads.make_case(lengths, 1, 64, "fp32", seed=1)
    assert bench.seen_pairs(case) == _brute_pairs(lengths)
    for tg in ([0, 1, 2, 40, 3], [0, 0, 5, 33, -2]):
        case.num_targets = np.array(tg, np.int32)
        assert bench.seen_pairs(case) == _brute_pairs(lengths, tg)


def test_cpu_baseline_record():
    case = workloads.make_case([64, 100], 2, 64, "fp32", seed=2)
    rec = bench.cpu_baseline(case, 0.5)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert "sequences" in rec["sample"]
