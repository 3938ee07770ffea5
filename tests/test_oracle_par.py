"""CPU checks of the helpers the full-size GPU parity tests use: the
threaded per-(head, row chunk) run of the oracle assembles the oracle's own
result, and the per-tile row sampler hits every query block."""
import math

import numpy as np
import pytest

import oracle
import oracle_par
import workloads


@pytest.mark.parametrize("kw", [
    dict(B=1, Sq=300, Sk=200, H=4, Hkv=4, q_valid=[250], kv_valid=[190], theta=1e4, norm=True),
    dict(B=2, Sq=257, Sk=257, H=4, Hkv=2, q_valid=[257, 100], kv_valid=[257, 31], theta=None, norm=True,
         causal=True),
    dict(B=1, Sq=400, Sk=400, H=2, Hkv=1, q_valid=[400], kv_valid=[400], theta=1e4, norm=False,
         window=(50, 2, 1, 1), gate=True),
])
def test_parallel_oracle_equals_oracle(kw):
    kw = dict(kw)
    B, Sq, Sk, H, Hkv = (kw.pop(x) for x in ("B", "Sq", "Sk", "H", "Hkv"))
    gate = workloads.make_gate(B, Sq, H, seed=3) if kw.pop("gate", False) else None
    inp = workloads.make_inputs(B, Sq, Sk, H, seed=Sq + H, Hkv=Hkv)
    common = dict(eps=1e-6, scale=1 / math.sqrt(128), **kw)
    rows = np.array([0, 3, 77, Sq - 1, 128, 129])
    for r in (None, rows):
        want = oracle.forward(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, rows=r, gate_bits=gate, **common)
        got = oracle_par.forward(inp, H, Hkv, rows=r, gate_bits=gate, chunk=64, **common)
        assert got.shape == want.shape
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("S,valid,tile,per", [(104448, 104448, 256, 2), (32768, 30720, 256, 1),
                                              (1000, 777, 128, 3), (5, 5, 256, 1), (300, 0, 256, 1)])
def test_tile_rows_hit_every_block(S, valid, tile, per):
    rows = workloads.tile_rows(S, valid, tile, per, seed=4)
    assert np.all(np.diff(rows) > 0) and rows.min() >= 0 and rows.max() < S
    for t0 in range(0, valid, tile):
        inside = rows[(rows >= t0) & (rows < min(t0 + tile, valid))]
        assert len(inside) >= min(per, min(tile, valid - t0))
    assert {0, S - 1} <= set(rows.tolist())
    assert np.array_equal(rows, workloads.tile_rows(S, valid, tile, per, seed=4))
