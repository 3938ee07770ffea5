"""Guard bands around the attention output: a launch writes its own
[B, Sq, H, D] output and nothing else. The output is a window into a larger
buffer; the bands before and after it hold a sentinel bit pattern, and the
window starts out NaN. After the launch the bands must be unchanged bit for
bit, every element of the window written and finite, and the window equal
bit for bit to the output of the same launch into a fresh tensor.

The cases cover every output path: the resident-key kernel (its stores go
through a buffer resource whose range ends at the item's last row, so rows
of the last tile past Sq are dropped), the ring kernel with tiles split over
the chip and merged, the general mode (causal mask, per-item lengths), the
frame window with the gate, and head dims 64 and 256."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import DevInputs, assert_all_written, say, to_dev, to_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

GUARD = 32768                 # bf16 elements (64 KB) on each side of the output
SENTINEL = 0x7E5A             # a NaN payload the kernels never write
NAN = 0x7FC0

# name, B, Sq, Sk, H, D, launch options
CASES = [
    ("resident ragged rows", 2, 1000, 300, 3, 128, dict(kv_valid=300)),
    ("resident zero tail", 1, 1300, 200, 2, 128, dict(q_valid=1100, kv_valid=170)),
    ("ring split and merge", 1, 3000, 2000, 3, 128, dict(q_valid=2900, kv_valid=1900)),
    ("ring causal", 2, 1500, 1500, 2, 128, dict(causal=True)),
    ("ring per-item lengths", 2, 1200, 1100, 2, 128, dict(lengths=[[1200, 1100], [700, 900]])),
    ("window with gate", 1, 1000, 1000, 2, 128, dict(window=(100, 3, 1, 1), gate=True)),
    ("head dim 64", 1, 2000, 1000, 2, 64, dict()),
    ("head dim 256", 1, 700, 900, 2, 256, dict()),
]


@pytest.fixture(scope="module")
def h3():
    from video_dit_dense_amd import h3attn
    h3attn.load_library()
    return h3attn


def launch(h3, d, B, Sq, Sk, H, D, opts, out):
    norm_rope = D == 128
    cos = sin = None
    if norm_rope:
        cos, sin = h3.rope_tables(max(Sq, Sk))
    lengths = opts.get("lengths")
    lt = None if lengths is None else torch.tensor(lengths, dtype=torch.int32, device="cuda:0")
    gate = None
    if opts.get("gate"):
        gate = to_dev(workloads.make_gate(B, Sq, H, seed=7))
    h3.forward(d.q, d.k, d.v, d.w_q if norm_rope else None, d.w_k if norm_rope else None, 1e-6, cos, sin,
               q_valid=opts.get("q_valid"), kv_valid=opts.get("kv_valid"), scale=D ** -0.5, out=out,
               causal=opts.get("causal", False), valid_lengths=lt, window=opts.get("window"), gate=gate)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,B,Sq,Sk,H,D,opts", CASES, ids=[c[0] for c in CASES])
def test_output_guard_bands(h3, name, B, Sq, Sk, H, D, opts):
    say("guard bands:", name)
    d = DevInputs(workloads.make_inputs(B, Sq, Sk, H, seed=91, D=D))
    n = B * Sq * H * D
    buf = torch.full((GUARD + n + GUARD,), SENTINEL, dtype=torch.int16, device="cuda:0")
    buf[GUARD:GUARD + n] = NAN
    out = buf[GUARD:GUARD + n].view(torch.bfloat16).view(B, Sq, H, D)
    launch(h3, d, B, Sq, Sk, H, D, opts, out)
    host = buf.cpu().numpy().view(np.uint16)
    assert np.all(host[:GUARD] == SENTINEL), f"{name}: band before the output overwritten"
    assert np.all(host[GUARD + n:] == SENTINEL), f"{name}: band after the output overwritten"
    got = host[GUARD:GUARD + n]
    assert_all_written(got, name)
    fresh = torch.empty(B, Sq, H, D, dtype=torch.bfloat16, device="cuda:0")
    launch(h3, d, B, Sq, Sk, H, D, opts, fresh)
    assert np.array_equal(got, to_host(fresh).ravel()), f"{name}: output differs from a fresh tensor's"
