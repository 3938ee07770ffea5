"""The largest tensors a call takes: one head-dim-128 attention step whose q,
output and prepared-query workspace each hold more than 2^31 elements (over
4 GiB), so every row, element and byte offset past 2^31 has to be formed in
64 bits:
- the prologue reading q and writing the prepared rows;
- the attention kernel's Q loads and output stores;
- the zeroed tail.

The key range is short (300 valid keys of 512, the cross-attention shape), so
the launch takes milliseconds. With an item's output above 2^31 bytes the
keys do not stay resident in LDS and the ring kernel runs; the test checks
that schedule.

Checked against the fp64 oracle:
- seeded rows in every 128-row block of the sequence, each row's norm and
  rotary at its own position;
- the rows on both sides of the 2^30- and 2^31-element output boundaries,
  and the last valid row;
- every output element finite (a NaN-filled output, reduced on the GPU);
- the tail rows past q_valid exactly +0.0."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import check_metrics, f32_dev, say, to_dev, to_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
              pytest.mark.timeout(600)]

SQ = (1 << 21) + 1000         # rows: SQ * H * 128 > 2^31 output elements
H = 8
SK = 512
KV_VALID = 300
Q_VALID = SQ - 37
EPS = 1e-6
THETA = 1e4
SEED = 2031


@pytest.fixture(scope="module")
def h3():
    from video_dit_dense_amd import h3attn
    h3attn.load_library()
    return h3attn


def test_output_past_2_31_elements(h3):
    D = 128
    assert SQ * H * D > 1 << 31
    plan = h3.schedule(1, SQ, SK, H, q_valid=Q_VALID, kv_valid=KV_VALID)
    assert plan["kernel"] == "ring", plan
    say(f"max size: B=1 Sq={SQ} Sk={SK} H={H} q_valid={Q_VALID} kv_valid={KV_VALID}, schedule {plan}")
    q_bits = workloads.normal_bf16_rows(1, SQ, H, seed=SEED)
    small = workloads.make_inputs(1, 1, SK, H, seed=SEED + 1)
    q, k, v = to_dev(q_bits), to_dev(small.k), to_dev(small.v)
    w_q, w_k = f32_dev(small.w_q), f32_dev(small.w_k)
    cos, sin = h3.rope_tables(SQ, THETA)
    o = torch.full_like(q, float("nan"))
    h3.forward(q, k, v, w_q, w_k, EPS, cos, sin, q_valid=Q_VALID, kv_valid=KV_VALID, scale=D ** -0.5, out=o)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()), "output elements unwritten or not finite"
    assert bool((o[:, Q_VALID:].view(torch.int16) == 0).all()), "tail rows must be +0.0"

    rows = workloads.tile_rows(SQ, Q_VALID, 128, 1, SEED)
    edges = np.array([(1 << 20) - 1, 1 << 20, (1 << 21) - 1, 1 << 21, (1 << 21) + 1, Q_VALID - 1])
    rows = np.unique(np.concatenate([rows, edges]))
    rows = rows[rows < Q_VALID]
    got = to_host(o[:, torch.from_numpy(rows).to("cuda:0")])
    del o, q
    torch.cuda.empty_cache()

    # The oracle's prologue and attention on the sampled rows, each at its
    # own position (the step oracle.forward takes, for a subset of rows).
    qn = oracle.apply_rope(oracle.rms_norm(oracle.bf16_bits_to_f64(q_bits[:, rows]), small.w_q, EPS), rows, THETA)
    kn = oracle.apply_rope(oracle.rms_norm(oracle.bf16_bits_to_f64(small.k), small.w_k, EPS), np.arange(SK), THETA)
    ref = oracle.attention(qn, kn, oracle.bf16_bits_to_f64(small.v), D ** -0.5, kv_valid=KV_VALID)
    check_metrics(oracle.compare(got, ref), f"max size ({len(rows)} rows x {H} heads)")
