"""GPU parity of the frame-window attention with the softmax gate (SGLang
PR #37903, "Modifications", hybrid_window_attn_h3) through h3attn_forward_ex,
against the fp64 oracle on the same seeded inputs. Bar: max-abs <= 2e-2 and
relative RMS <= 5e-3 on the bf16 outputs, as for the dense step."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import DevInputs, check_metrics, say, to_dev, to_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

MAX_ABS = 2e-2
REL_RMS = 5e-3
SCALE = 1 / math.sqrt(128)


@pytest.fixture(scope="module")
def h3():
    from video_dit_dense_amd import h3attn
    h3attn.load_library()
    return h3attn


def check(metrics, label):
    check_metrics(metrics, label, MAX_ABS, REL_RMS)


def run(h3, inp, window, gate_bits=None, q_valid=None, kv_valid=None, lengths=None):
    d = DevInputs(inp)
    S = max(inp.q.shape[1], inp.k.shape[1])
    cos, sin = h3.rope_tables(S)
    lt = None if lengths is None else torch.tensor(lengths, dtype=torch.int32, device="cuda:0")
    gate = None if gate_bits is None else to_dev(gate_bits)
    o = h3.forward(d.q, d.k, d.v, d.w_q, d.w_k, 1e-6, cos, sin, q_valid=q_valid, kv_valid=kv_valid,
                   scale=SCALE, valid_lengths=lt, window=window, gate=gate)
    torch.cuda.synchronize()
    return to_host(o)


def ref(inp, window, gate_bits=None, q_valid=None, kv_valid=None, rows=None):
    return oracle.forward(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, 1e-6, 1e4, SCALE, q_valid=q_valid,
                          kv_valid=kv_valid, rows=rows, window=window, gate_bits=gate_bits)


# (B, S, H, Hkv, window, gate, label): 256-row tiles aligned with frames and
# chunks (the fast schedule), frames that do not align with 32-key sub-tiles
# or tiles (every step masked), tiles straddling chunks without anchors and
# radius 0 (rows that see nothing in the tile's first sub-tile), grouped heads.
CASES = [
    (1, 4096, 2, 2, (256, 2, 1, 1), True, "aligned frames, gate"),
    (1, 4096, 2, 2, (256, 2, 1, 1), False, "aligned frames, no gate"),
    (1, 2000, 2, 2, (100, 3, 1, 2), True, "frames of 100 rows"),
    (1, 1536, 2, 2, (96, 2, 0, 0), True, "no anchors, radius 0, tiles straddle chunks"),
    (2, 1800, 4, 2, (128, 5, 1, 1), True, "grouped heads, batch 2"),
    (1, 3000, 2, 2, (64, 1, 2, 3), True, "chunks of one frame, radius 2, 3 anchors"),
]


@pytest.mark.parametrize("B,S,H,Hkv,window,gate,label", CASES)
def test_window(h3, B, S, H, Hkv, window, gate, label):
    say("window", label)
    inp = workloads.make_inputs(B, S, S, H, seed=70 + S % 97, Hkv=Hkv)
    g = workloads.make_gate(B, S, H, seed=S) if gate else None
    check(oracle.compare(run(h3, inp, window, g), ref(inp, window, g)), label)


def test_window_with_padding_and_lengths(h3):
    say("window with padding and per-item lengths")
    B, S, H = 2, 2304, 2
    window = (192, 2, 1, 1)
    inp = workloads.make_inputs(B, S, S, H, seed=81)
    g = workloads.make_gate(B, S, H, seed=81)
    got = run(h3, inp, window, g, q_valid=2000, kv_valid=1700)
    check(oracle.compare(got, ref(inp, window, g, q_valid=2000, kv_valid=1700)), "uniform padding")
    lengths = [[2304, 2304], [1500, 1100]]
    got = run(h3, inp, window, g, lengths=lengths)
    want = np.concatenate([ref(workloads.Inputs(inp.q[b:b + 1], inp.k[b:b + 1], inp.v[b:b + 1], inp.w_q, inp.w_k),
                               window, g[b:b + 1], q_valid=lengths[b][0], kv_valid=lengths[b][1])
                           for b in range(B)])
    check(oracle.compare(got, want), "per-item lengths")


def test_rows_without_keys_are_zero(h3):
    """No anchors, radius 0 and keys cut at kv_valid: rows whose chunk lies
    past the keys see nothing and are written as zeros."""
    say("window rows without keys")
    S, H = 1024, 2
    window = (64, 2, 0, 0)
    inp = workloads.make_inputs(1, S, S, H, seed=82)
    got = run(h3, inp, window, kv_valid=300)
    want = ref(inp, window, kv_valid=300)
    check(oracle.compare(got, want), "rows without keys")
    assert np.all(got[0, 384:] == 0)


@pytest.mark.parametrize("D", [128, 256])
def test_first_keys_far_below_zero(h3, D):
    """Rows that see no key in their tile's first sub-tile (no anchors,
    radius 0, tiles straddling chunks) take their offset from the first keys
    they meet. Here every score is about -204 in exp2 units (q = 40 e_0,
    k = -40 e_0 on raw inputs), so the rescale of such a row must not form
    exp2(+204) (fp32 overflow); each row is the mean of v over its chunk."""
    say("window first keys far below zero", D)
    S, H = 1024, 2
    window = (64, 1, 0, 0)
    inp = workloads.make_inputs(1, S, S, H, seed=83, D=D)
    big = np.uint16(0x4220)            # 40.0 in bf16
    q = np.zeros_like(inp.q)
    k = np.zeros_like(inp.k)
    q[..., 0] = big
    k[..., 0] = big | np.uint16(0x8000)
    d = DevInputs(workloads.Inputs(q, k, inp.v, inp.w_q, inp.w_k))
    o = h3.forward(d.q, d.k, d.v, scale=SCALE, window=window)
    torch.cuda.synchronize()
    want = oracle.forward(q, k, inp.v, None, None, 1e-6, None, SCALE, norm=False, window=window)
    check(oracle.compare(to_host(o), want), f"D={D} first keys far below zero")


def test_gate_in_uniform_schedule(h3):
    """The gate alone, on the dense schedule whose last round is split over
    workgroups and merged (4096 rows x 8 heads: 128 tiles)."""
    say("gate, dense split schedule")
    S, H = 4096, 8
    inp = workloads.make_inputs(1, S, S, H, seed=83)
    g = workloads.make_gate(1, S, H, seed=83)
    d = DevInputs(inp)
    cos, sin = h3.rope_tables(S)
    o = h3.forward(d.q, d.k, d.v, d.w_q, d.w_k, 1e-6, cos, sin, scale=SCALE, gate=to_dev(g))
    torch.cuda.synchronize()
    check(oracle.compare(to_host(o), oracle.forward(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, 1e-6, 1e4, SCALE,
                                                    gate_bits=g)), "gate on split tiles")


def test_gate_on_resident_keys(h3):
    """The gate on the resident-key kernel (300 valid text keys stay in LDS;
    the gate values are read with each tile's query prefetch), two batch
    items, a zero tail and a partial last query tile."""
    say("gate, resident keys")
    B, Sq, Sk, H = 2, 1000, 512, 3
    inp = workloads.make_inputs(B, Sq, Sk, H, seed=86)
    g = workloads.make_gate(B, Sq, H, seed=86)
    assert h3.schedule(B, Sq, Sk, H, q_valid=900, kv_valid=300)["kernel"] == "resident"
    d = DevInputs(inp)
    o = h3.forward(d.q, d.k, d.v, d.w_q, d.w_k, 1e-6, None, None, q_valid=900, kv_valid=300, scale=SCALE,
                   gate=to_dev(g))
    torch.cuda.synchronize()
    got = to_host(o)
    check(oracle.compare(got, oracle.forward(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, 1e-6, None, SCALE,
                                             q_valid=900, kv_valid=300, gate_bits=g)), "gate on resident keys")
    assert np.all(got[:, 900:] == 0), "rows past q_valid are +0.0"


def test_window_repeatable(h3):
    inp = workloads.make_inputs(1, 2000, 2000, 2, seed=84)
    g = workloads.make_gate(1, 2000, 2, seed=84)
    a = run(h3, inp, (100, 3, 1, 2), g)
    b = run(h3, inp, (100, 3, 1, 2), g)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("D,H", [(64, 8), (128, 8), (256, 4)])
def test_window_longest_first_every_tile(h3, D, H):
    """A window geometry whose tiles are uneven enough that the launcher
    hands the query blocks out longest first (frames of 1024 rows, chunks of
    five, radius 1, one anchor frame; S = 24576 gives 768 tiles of four
    lengths on 256 CUs), on a seeded row of every query block of every head,
    the anchor frame and chunk edges."""
    say("window longest first, every tile", D)
    S, window = 24576, (1024, 5, 1, 1)
    inp = workloads.make_inputs(1, S, S, H, seed=85, D=D)
    d = DevInputs(inp)
    if D == 128:
        cos, sin = h3.rope_tables(S)
        o = h3.forward(d.q, d.k, d.v, d.w_q, d.w_k, 1e-6, cos, sin, scale=SCALE, window=window)
    else:
        o = h3.forward(d.q, d.k, d.v, scale=SCALE, window=window)
    torch.cuda.synchronize()
    F, C = window[0], window[1]
    edges = [0, F - 1, F, F + C * F - 1, F + C * F, S - C * F, S - 1]
    rows = np.unique(np.concatenate([workloads.tile_rows(S, S, 128 if D == 256 else 256, 1, 85), edges]))
    if D == 128:
        want = ref(inp, window, rows=rows)
    else:
        want = oracle.forward(inp.q, inp.k, inp.v, None, None, 1e-6, None, SCALE, norm=False, rows=rows,
                              window=window)
    check(oracle.compare(to_host(o)[:, rows], want), f"D={D} window longest first")


def test_window_cross_lengths(h3):
    """Queries and keys of different lengths share one frame grid."""
    say("window, Sq != Sk")
    inp = workloads.make_inputs(1, 1000, 700, 2, seed=85)
    window = (64, 2, 1, 1)
    d = DevInputs(inp)
    o = h3.forward(d.q, d.k, d.v, d.w_q, d.w_k, 1e-6, None, None, scale=SCALE, window=window)
    torch.cuda.synchronize()
    want = oracle.forward(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, 1e-6, None, SCALE, window=window)
    check(oracle.compare(to_host(o), want), "window Sq=1000 Sk=700")


def test_gate_saturation(h3):
    """Gates of +-1000: sigmoid 1 leaves the output bit for bit, sigmoid 0
    zeroes it."""
    say("gate saturation")
    S, H = 512, 2
    inp = workloads.make_inputs(1, S, S, H, seed=86)
    window = (128, 2, 1, 1)
    base = run(h3, inp, window)
    up = np.full((1, S, H), 0x447A, dtype=np.uint16)     # bf16 1000.0
    down = np.full((1, S, H), 0xC47A, dtype=np.uint16)   # bf16 -1000.0
    assert np.array_equal(run(h3, inp, window, up), base)
    assert np.all(oracle.bf16_bits_to_f64(run(h3, inp, window, down)) == 0.0)
