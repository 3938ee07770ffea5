"""GPU parity of the two head-dim-128 tilings of the attention kernel: two or
three 16-row query tiles per wave (query blocks of 256 or 384 rows), which
the launcher chooses per launch and h3attn_forward_args.query_tiles can
force. Every row's arithmetic is the same at either count (the same
matrix-core instructions over the same key sub-tiles in the same order; a
larger block only adds sub-tiles that the row's causal mask or frame window
masks, which add exact zeros), so launches whose tiles all run whole give
bit-identical outputs, and both match the fp64 oracle at the step's bar
(max-abs <= 2e-2, relative RMS <= 5e-3, per-row relative L2 <= 1e-2). Where
the uniform schedule splits the last round, the two tilings divide the keys
differently and are each held to the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import DevInputs, check_metrics, say, to_dev, to_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SCALE = 1 / math.sqrt(128)


@pytest.fixture(scope="module")
def h3():
    from video_dit_dense_amd import h3attn
    h3attn.load_library()
    return h3attn


def run(h3, d, qt, *, norm=True, causal=False, lengths=None, window=None, q_valid=None, kv_valid=None):
    Sq, Sk = d.q.shape[1], d.k.shape[1]
    cos, sin = h3.rope_tables(max(Sq, Sk)) if norm else (None, None)
    lt = None if lengths is None else torch.tensor(lengths, dtype=torch.int32, device="cuda:0")
    o = h3.forward(d.q, d.k, d.v, d.w_q if norm else None, d.w_k if norm else None, 1e-6, cos, sin,
                   q_valid=q_valid, kv_valid=kv_valid, scale=SCALE, causal=causal, valid_lengths=lt,
                   window=window, query_tiles=qt)
    torch.cuda.synchronize()
    return to_host(o)


def plan(h3, inp, qt, **kw):
    B, Sq, H, _ = inp.q.shape
    return h3.schedule(B, Sq, inp.k.shape[1], H, inp.k.shape[2], query_tiles=qt, **kw)


CASES = {
    # general mode: one workgroup per query block, nothing split
    "causal": dict(B=1, Sq=2000, Sk=2000, H=3, kw=dict(causal=True)),
    "window": dict(B=1, Sq=2304, Sk=2304, H=2, kw=dict(window=(192, 2, 1, 1))),
    "lengths": dict(B=3, Sq=1500, Sk=1500, H=2, kw=dict(lengths=[[1500, 1500], [900, 1400], [1333, 257]])),
    # uniform mode with 16 key sub-tiles: every tile whole (no split), the ring kernel
    "dense_whole": dict(B=1, Sq=3000, Sk=500, H=4, kw=dict()),
}


@pytest.mark.parametrize("case", list(CASES))
def test_whole_tiles_are_bit_identical_across_tilings(h3, case):
    c = CASES[case]
    say("query tiles 2 vs 3", case)
    inp = workloads.make_inputs(c["B"], c["Sq"], c["Sk"], c["H"], seed=900 + len(case))
    d = DevInputs(inp)
    kw = dict(c["kw"])
    pk = dict(causal=kw.get("causal", False), per_item_lengths="lengths" in kw, window=kw.get("window"))
    for qt in (2, 3):
        p = plan(h3, inp, qt, **pk)
        assert p["kernel"] == "ring" and p["query_tiles"] == qt and p["split_tiles"] == 0, p
    two = run(h3, d, 2, **kw)
    three = run(h3, d, 3, **kw)
    assert np.array_equal(two, three), case
    lengths = kw.pop("lengths", None)
    qv = kvv = None
    if lengths is not None:
        qv = [min(max(a, 0), c["Sq"]) for a, _ in lengths]
        kvv = [min(max(b, 0), c["Sk"]) for _, b in lengths]
    want = oracle.forward(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, 1e-6, 1e4, SCALE, q_valid=qv, kv_valid=kvv,
                          causal=kw.get("causal", False), window=kw.get("window"))
    check_metrics(oracle.compare(three, want), f"{case} at three query tiles")


@pytest.mark.parametrize("norm", [True, False])
def test_split_schedules_match_the_oracle(h3, norm):
    """A uniform launch whose last round splits at both tilings (the key
    ranges of the split tiles differ between them); without the norm the
    score bound comes from the data."""
    B, Sq, Sk, H = 1, 5000, 4000, 3
    say("query tiles split", norm)
    inp = workloads.make_inputs(B, Sq, Sk, H, seed=950 + norm)
    d = DevInputs(inp)
    want = oracle.forward(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, 1e-6, 1e4 if norm else None, SCALE, norm=norm)
    for qt in (2, 3):
        p = plan(h3, inp, qt)
        assert p["query_tiles"] == qt and p["split_tiles"] > 0, p
        got = run(h3, d, qt, norm=norm)
        check_metrics(oracle.compare(got, want), f"split schedule, {qt} query tiles, norm={norm}")


def test_automatic_choice_is_one_of_the_tilings(h3):
    """The default (0) runs whichever tiling the schedule query names, and
    its output equals that tiling forced."""
    inp = workloads.make_inputs(1, 2000, 2000, 3, seed=970)
    d = DevInputs(inp)
    qt = plan(h3, inp, 0, causal=True)["query_tiles"]
    assert qt in (2, 3)
    assert np.array_equal(run(h3, d, 0, causal=True), run(h3, d, qt, causal=True))


# (B, Sq, Sk, H, kwargs): the ring kernel's online path (norm weights whose
# score bound is over the limit) in the uniform schedule with a split last
# round, with ragged valid lengths, under the causal mask, and in the frame
# window with the gate.
ONLINE = [
    (1, 3000, 3000, 3, {}),
    (2, 1000, 777, 2, {"q_valid": 900, "kv_valid": 700}),
    (1, 1500, 1500, 2, {"causal": True}),
    (1, 2000, 2000, 2, {"window": (100, 3, 1, 2), "gate": True}),
]


@pytest.mark.parametrize("qt", [2, 3])
@pytest.mark.parametrize("B,Sq,Sk,H,kw", ONLINE)
def test_online_path_at_both_counts(h3, B, Sq, Sk, H, kw, qt):
    """Weights large enough that the a priori bound exceeds its limit (one
    channel's weight 4, zeroed in the data so the scores stay moderate): the
    running maximum and the rescale run, at either tiling."""
    kw = dict(kw)
    base = workloads.make_inputs(B, Sq, Sk, H, seed=980 + Sq)
    w_q, w_k = base.w_q.copy(), base.w_k.copy()
    w_q[3] = w_k[100] = 4.0
    q, k = base.q.copy(), base.k.copy()
    q[..., 3] = 0
    k[..., 100] = 0
    inp = workloads.Inputs(q, k, base.v, w_q, w_k)
    gate_bits = workloads.make_gate(B, Sq, H, seed=Sq) if kw.pop("gate", False) else None
    say("online path", qt, B, Sq, Sk, H, kw)
    d = DevInputs(inp)
    cos, sin = h3.rope_tables(max(Sq, Sk))
    gate = None if gate_bits is None else to_dev(gate_bits)
    o = h3.forward(d.q, d.k, d.v, d.w_q, d.w_k, 1e-6, cos, sin, scale=SCALE, gate=gate, query_tiles=qt, **kw)
    torch.cuda.synchronize()
    want = oracle.forward(inp.q, inp.k, inp.v, w_q, w_k, 1e-6, 1e4, SCALE, kw.get("q_valid"), kw.get("kv_valid"),
                          causal=kw.get("causal", False), window=kw.get("window"), gate_bits=gate_bits)
    check_metrics(oracle.compare(to_host(o), want), f"online path, {qt} query tiles, {B}x{Sq}x{Sk}x{H} {kw}")
