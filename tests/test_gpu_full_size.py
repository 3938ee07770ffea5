"""Full-size parity: every attention launch the benchmark times, at its real
size and in the launch configuration it times, against the fp64 oracle.

Coverage:
- padded and cross: every row of every head (the oracle takes seconds);
- full, full_causal, full_gqa, full_window, full_d64, full_d256,
  full_window_d64 and batch_varlen: seeded rows in every (item, head, query block) tile of the
  launch: one in every 128-row block, so at least one in every query block
  of whichever tiling the launch takes (128 to 512 rows), plus the
  first, last, last-valid and first-tail rows (and frame edges for the
  window). The oracle computes each chosen row for every head, so every tile
  the launch runs, whole, split or remapped by the tile orders, has checked
  rows.
- Every output buffer starts filled with NaN, and every element must come
  out finite: no tile, row or channel may be left unwritten. Rows at or past
  an item's q_valid must be exactly +0.0.

Bars: max-abs <= 2e-2 and relative RMS <= 5e-3 on the checked rows (the
tolerance the step is specified to), and relative L2 <= 1e-2 on every checked row.
"""
import functools
import math

import numpy as np
import pytest
import torch

import oracle_par
import workloads
from gpu_util import DevInputs, assert_all_written, check_metrics, nan_like, say, to_dev, to_host

import oracle

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
              pytest.mark.timeout(600)]

ALL = {**workloads.WORKLOADS, **workloads.VARIANT_WORKLOADS}


@pytest.fixture(scope="module")
def h3():
    from video_dit_dense_amd import h3attn
    h3attn.load_library()
    return h3attn


@functools.lru_cache(maxsize=2)
def inputs(name):
    return workloads.make_workload_inputs(ALL[name])


def run_gpu(h3, wl, inp):
    """The benchmark's launch of workload wl into a NaN-filled output."""
    d = DevInputs(inp)
    cos = sin = None
    if wl.rope:
        cos, sin = h3.rope_tables(max(wl.Sq, wl.Sk), wl.theta)
    lengths = torch.tensor(wl.lengths, dtype=torch.int32, device="cuda:0") if wl.lengths else None
    gate = to_dev(workloads.make_gate(wl.B, wl.Sq, wl.H, seed=wl.seed)) if wl.gate else None
    o = nan_like(d.q)
    h3.forward(d.q, d.k, d.v, d.w_q if wl.norm else None, d.w_k if wl.norm else None, wl.eps, cos, sin,
               q_valid=None if wl.lengths else wl.q_valid, kv_valid=None if wl.lengths else wl.kv_valid,
               scale=wl.scale, out=o, causal=wl.causal, valid_lengths=lengths, window=wl.window or None,
               gate=gate)
    torch.cuda.synchronize()
    return to_host(o)


def run_oracle(wl, inp, rows):
    lengths = wl.item_lengths()
    gate = workloads.make_gate(wl.B, wl.Sq, wl.H, seed=wl.seed) if wl.gate else None
    return oracle_par.forward(inp, wl.H, wl.kv_heads, rows=rows, gate_bits=gate, eps=wl.eps,
                              theta=wl.theta if wl.rope else None, scale=wl.scale,
                              q_valid=[l[0] for l in lengths], kv_valid=[l[1] for l in lengths],
                              norm=wl.norm, causal=wl.causal, window=wl.window or None)


def assert_tails_zero(got, wl):
    for b, (qv, _) in enumerate(wl.item_lengths()):
        assert np.all(got[b, qv:] == 0), f"{wl.name}: rows of item {b} at or past {qv} must be +0.0"


@pytest.mark.parametrize("name", ["padded", "cross"])
def test_every_row(h3, name):
    wl = ALL[name]
    say("every row", name, wl.description)
    inp = inputs(name)
    got = run_gpu(h3, wl, inp)
    assert_all_written(got, name)
    assert_tails_zero(got, wl)
    ref = run_oracle(wl, inp, None)
    check_metrics(oracle.compare(got, ref), f"{name} (all {wl.Sq} rows x {wl.H} heads)")


@pytest.mark.parametrize("name,per_tile", [
    ("full", 1), ("full_causal", 1), ("full_gqa", 1), ("full_window", 1),
    ("full_d64", 1), ("full_d256", 1), ("full_window_d64", 1), ("batch_varlen", 1),
])
def test_every_tile(h3, name, per_tile):
    wl = ALL[name]
    say("every tile", name, wl.description)
    inp = inputs(name)
    got = run_gpu(h3, wl, inp)
    assert_all_written(got, name)
    assert_tails_zero(got, wl)
    # 128-row blocks: every query block of every tiling (128, 256, 384 or
    # 512 rows) holds at least one of them whole
    tile = 128
    q_max = max(l[0] for l in wl.item_lengths())
    rows = workloads.tile_rows(wl.Sq, q_max, tile, per_tile, wl.seed)
    if wl.window:
        F, C = wl.window[0], wl.window[1]
        edges = np.array([F - 1, F, F + C * F - 1, F + C * F, wl.Sq - C * F, wl.Sq // 2])
        rows = np.unique(np.concatenate([rows, edges[(edges >= 0) & (edges < wl.Sq)]]))
    blocks = len(np.unique(rows[rows < q_max] // tile))
    assert blocks == math.ceil(q_max / tile), (blocks, q_max, tile)
    ref = run_oracle(wl, inp, rows)
    check_metrics(oracle.compare(got[:, rows], ref),
                  f"{name} ({len(rows)} rows: every one of the {blocks} query blocks x {wl.H} heads x {wl.B} items)")
