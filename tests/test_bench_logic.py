"""Measurement logic of bench.py, on the CPU: work counting and the one-GPU contract."""
import os
import subprocess
import sys

import numpy as np

import workloads as wl
from oracle import visible_pairs_ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_visible_pairs_closed_form_matches_the_mask():
    rng = np.random.default_rng(0)
    for _ in range(30):
        _, _, _, cu_q, cu_k, qo, ko = wl.random_pack(rng, int(rng.integers(0, 6)), 200, 1, 1, 1,
                                                     dtype="fp32")
        assert bench.visible_pairs(cu_q, cu_k, qo, ko) == visible_pairs_ref(cu_q, cu_k, qo, ko)
    # the benchmarked share: pairs per head, as derived for seed 0
    pieces = wl.lengths_for("cp4_share", 0)
    cu = wl.cu_from_lengths(pieces)
    total = sum(bench.visible_pairs(cu, cu, [3 * p for p in pieces], [c * p for p in pieces])
                for c in range(4))
    assert total == 45_386_359


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=60)
    assert out.returncode == 2 and "one GPU" in out.stderr


def test_launch_chain_durations_tile_the_timed_region():
    """One event after each launch: a launch's duration runs from the previous event to its
    own, so the durations of all labels together sum to the span of the chain."""
    import bench

    clock = [0.0]

    class FakeEvent:
        def record(self, stream):
            self.t = clock[0]

        def elapsed_time(self, other):
            return other.t - self.t

    ch = bench.LaunchChain(FakeEvent, 1 + 3 * 2)
    ch.mark("start", None)
    for step in range(3):
        clock[0] += 5.0          # attention launch
        ch.mark("attn", None)
        clock[0] += 1.5          # merge launch
        ch.mark("merge", None)
    assert ch.durations_ms("attn") == [5.0, 5.0, 5.0]
    assert ch.durations_ms("merge") == [1.5, 1.5, 1.5]
    assert sum(ch.durations_ms("attn")) + sum(ch.durations_ms("merge")) == clock[0]
