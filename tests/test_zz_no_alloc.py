"""GPU test of h3attn_forward_noalloc, the entry point for callers that
cannot allocate: through the C-ABI it must give what h3attn_forward gives
with a caller workspace (the same kernels and schedule, so bit for bit), on
two calls in a row where the second is smaller and so finds the first call's
contents in the static workspace, and meet the oracle's bar. Sizes beyond
the static array are refused before anything runs."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import DevInputs, check_metrics, nan_like, say, to_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def h3():
    from video_dit_dense_amd import h3attn
    h3attn.load_library()
    return h3attn


# (B, Sq, Sk, H, q_valid, kv_valid, rope): the mid configuration (158 MB of
# workspace, whole rounds of tiles), then a smaller ragged shape whose last
# round is split (partial records in the array) and whose valid lengths cut
# both ends; then cross-attention (177 MB) and a tiny one.
PAIRS = [
    ((1, 8192, 8192, 8, 8192, 8192, True), (2, 3000, 2500, 3, 2900, 2333, True)),
    ((1, 32760, 512, 8, 32760, 300, False), (1, 700, 300, 2, 650, 1, True)),
]


def run_both(h3, shape):
    B, Sq, Sk, H, qv, kvv, rope = shape
    inp = workloads.make_inputs(B, Sq, Sk, H, seed=Sq + 3 * Sk + H)
    d = DevInputs(inp)
    cos = sin = None
    if rope:
        cos, sin = h3.rope_tables(max(Sq, Sk))
    scale = 1 / math.sqrt(128)
    want = h3.forward(d.q, d.k, d.v, d.w_q, d.w_k, 1e-6, cos, sin, q_valid=qv, kv_valid=kvv, scale=scale)
    got = nan_like(d.q)
    h3.forward_noalloc(d.q, d.k, d.v, got, d.w_q, d.w_k, 1e-6, cos, sin, q_valid=qv, kv_valid=kvv, scale=scale)
    torch.cuda.synchronize()
    return inp, to_host(want), to_host(got)


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_forward_on_two_calls(h3, first, second):
    for shape in (first, second):
        say("no-alloc forward", shape)
        B, Sq, Sk, H, qv, kvv, rope = shape
        inp, want, got = run_both(h3, shape)
        assert np.array_equal(got, want), f"{shape}: differs from h3attn_forward"
        rows = workloads.tile_rows(Sq, qv, 256, 1, seed=Sq)
        ref = oracle.forward(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, 1e-6, 1e4 if rope else None,
                             1 / math.sqrt(128), qv, kvv, rows=rows)
        check_metrics(oracle.compare(got[:, rows], ref), f"no-alloc {shape}")
        assert np.all(got[:, qv:] == 0)


def test_noalloc_refuses_sizes_beyond_the_array(h3):
    wl = workloads.WORKLOADS["padded"]
    assert h3.workspace_bytes(wl.B, wl.Sq, wl.Sk, wl.H) > h3.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(wl.B, wl.Sq, wl.H, 128, dtype=torch.bfloat16, device="cuda:0")
    o = nan_like(q)
    with pytest.raises(h3.H3AttnError, match="ERR_WORKSPACE"):
        h3.forward_noalloc(q, q.clone(), q.clone(), o)
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all()   # nothing ran
