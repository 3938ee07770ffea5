"""Host-side checks of bench.py's accounting and entry behaviour (CPU only):
the flop count of the frame window equals the oracle's visible pairs, the
causal and dense counts are the closed forms, and a multi-GPU request is
refused with a message."""
import os
import subprocess
import sys

import numpy as np

import bench
import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_window_pair_count_matches_oracle_mask():
    for window, S, qv, kvv in [((100, 3, 1, 2), 2000, 2000, 2000), ((64, 2, 0, 0), 1024, 900, 300),
                               ((3072, 5, 1, 1), 104448, 104448, 104448)]:
        wl = workloads.Workload("w", 1, S, S, 2, qv, kvv, True, True, 0, window=window)
        rows = np.arange(qv) if S <= 4096 else np.random.default_rng(0).choice(S, 300, replace=False)
        want = oracle.window_visible(rows, np.arange(kvv), *window).sum(axis=1)
        assert np.array_equal(bench.window_keys_per_row(wl, rows), want), window
    wl = workloads.Workload("w", 1, 2000, 2000, 3, 2000, 2000, True, True, 0, window=(100, 3, 1, 2))
    pairs = oracle.window_visible(np.arange(2000), np.arange(2000), 100, 3, 1, 2).sum()
    assert bench.step_flops(wl) == 4.0 * pairs * 128 * 3


def test_dense_and_causal_flops_closed_forms():
    wl = workloads.WORKLOADS["full"]
    assert bench.step_flops(wl) == 4.0 * 104448 * 104448 * 128 * 6
    wc = workloads.VARIANT_WORKLOADS["full_causal"]
    assert bench.step_flops(wc) == 4.0 * (104448 * 104449 // 2) * 128 * 6
    wd = workloads.VARIANT_WORKLOADS["full_d64"]
    assert bench.step_flops(wd) == 4.0 * 104448 * 104448 * 64 * 12


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
