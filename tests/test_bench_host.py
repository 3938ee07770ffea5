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


def test_config_work_matches_the_tabulated_figures():
    """Valid-pair flops and compulsory attention bytes of the five
    configurations, as tabulated for the measurement: Padded counts its
    30720 valid rows and keys, Cross its 300 valid keys (and is the one
    whose compulsory bytes outlast its flops at the nominal peaks)."""
    W = workloads.WORKLOADS
    assert bench.step_flops(W["padded"]) == 4.0 * 30720 * 30720 * 128 * 8
    assert bench.step_flops(W["cross"]) == 4.0 * 32760 * 300 * 128 * 8
    assert bench.attention_bytes(W["cross"]) == 2 * 128 * 8 * (32760 + 2 * 300 + 32760)
    assert round(bench.attention_bytes(W["cross"]) / 1e6, 1) == 135.4
    assert bench.attention_bytes(W["full"]) == 4 * 104448 * 6 * 256
    assert bench.attention_bytes(W["padded"]) == 2 * 128 * 8 * (30720 + 2 * 30720 + 32768)
    for name, wl in W.items():
        t_mfma = bench.step_flops(wl) / (bench.PEAK_BF16_TFLOPS * 1e12)
        t_hbm = bench.attention_bytes(wl) / (bench.PEAK_HBM_GBS * 1e9)
        assert (t_hbm > t_mfma) == (name in ("cross", "tiny")), name


def test_timing_stats():
    s = bench.stats([1.0, 2.0, 3.0, 10.0])
    assert s["median"] == 2.5 and s["min"] == 1.0 and s["max"] == 10.0 and s["n"] == 4
    assert abs(s["cv"] - np.std([1, 2, 3, 10]) / 4.0) < 1e-4
    h = bench.host_info()
    assert h["host_cores"] == len(os.sched_getaffinity(0))


def test_attend_kernel_names_follow_the_launcher():
    """The bench names the kernels from the library's own schedule of each
    workload (256 compute units)."""
    W = {**workloads.WORKLOADS, **workloads.VARIANT_WORKLOADS}

    def name(wl):
        return bench.attend_kernels(wl, bench.attend_schedule(wl, cus=256))

    assert name(W["cross"]).startswith("attn_resident_kernel")
    assert name(W["full"]) == "attn_fwd_kernel<128, 3, false> + attn_merge_kernel<128, 3> (96 tiles split)"
    assert name(W["mid"]) == "attn_fwd_kernel<128, 2, false>"
    assert name(W["tiny"]) == "attn_fwd_kernel<128, 2, false>"
    assert name(W["full_causal"]) == "attn_fwd_kernel<128, 3, false> (general mode)"
    assert name(W["full_window"]) == "attn_fwd_kernel<128, 3, true> (general mode)"
    assert name(W["full_d64"]).startswith("attn_fwd_kernel<64, 4, false>")
    assert name(W["full_d256"]).startswith("attn_fwd_kernel<256, 2, false>")
    assert name(W["full_window_d64"]) == "attn_fwd_kernel<64, 4, true> (general mode)"
    wl = workloads.Workload("w", 1, 4096, 321, 2, 4096, 321, True, False, 0)
    assert name(wl).startswith("attn_fwd_kernel<128")      # 11 sub-tiles: the ring kernel
    wl = workloads.Workload("w", 1, 4096, 320, 2, 4096, 320, True, False, 0)
    assert name(wl).startswith("attn_resident_kernel")
