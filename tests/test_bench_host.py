"""Host-side logic of bench.py (no GPU): the one-GPU rule, the guard that
reports a counter-based HBM traffic figure only while the kernel source it
was measured on is unchanged, and the FLOP counts of the window and packed
workloads against a brute-force count of the (query, key) pairs a row sees.
"""

import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line


def test_traffic_reported_only_for_the_measured_source(monkeypatch):
    name = "c3_bf16_d128"
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.txt")
    stored = [line.split(":", 1)[1].strip() for line in open(path)
              if line.startswith("hbm_bytes_per_launch:")]
    assert stored, "the headline traffic summary holds a byte count"
    assert bench._traffic(name, "bf16") == float(stored[0])
    # any change to the kernel sources (a different hash) withdraws it
    monkeypatch.setattr(bench, "_src_hash", lambda rels: "0" * 64)
    assert bench._traffic(name, "bf16") is None
    assert bench._traffic("no_such_workload", "bf16") is None


def _brute_pairs(Nq, Nk, causal, window):
    # key j is seen by query i iff it lies in the band around the
    # bottom-right-aligned diagonal i + Nk - Nq
    n = 0
    for i in range(Nq):
        diag = i + Nk - Nq
        for j in range(Nk):
            if causal and j > diag:
                continue
            if window is not None:
                left, right = window
                if left is not None and left >= 0 and j < diag - left:
                    continue
                if not causal and right is not None and right >= 0 and j > diag + right:
                    continue
            n += 1
    return n


@pytest.mark.parametrize("Nq,Nk,causal,window", [
    (37, 37, True, (5, 0)),
    (20, 45, True, (7, 0)),
    (30, 30, False, (4, 9)),
    (13, 50, False, (100, 3)),
    (40, 25, False, (6, 6)),
])
def test_window_flops_match_brute_force(Nq, Nk, causal, window):
    w = workloads.ALL["local_b1_h16_n16k_w4096_d128"].with_(B=2, H=3, Nq=Nq, Nk=Nk,
                                                            causal=causal, window=window)
    assert bench.window_flops(w) == 4.0 * 2 * 3 * w.d * _brute_pairs(Nq, Nk, causal, window)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_flops_match_brute_force(causal):
    w = workloads.ALL["varlen_s16_h16_d128_lognormal_causal"].with_(causal=causal)
    lens = [5, 1, 17, 64, 9]
    pairs = sum(_brute_pairs(n, n, False, None) for n in lens)
    if causal:
        # the causal count halves the square, as for the other causal
        # workloads (their FLOP rates use N^2 / 2 pairs)
        expect = 4.0 * w.H * w.d * pairs * 0.5
    else:
        expect = 4.0 * w.H * w.d * pairs
    assert bench.varlen_flops(w, np.array(lens)) == expect
