"""GPU parity of the attention kernels at head dims 64 and 256 (FastVideo PR
#1799, "Implementation": validated head dims 64, 128 and 256) through
h3attn_forward_ex, against the fp64 oracle on the same seeded inputs. The Q/K
norm and rotary prologue are H3's and defined on 128 channels, so these run
without them. Bar: max-abs <= 2e-2 and relative RMS <= 5e-3, as for 128."""
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


@pytest.fixture(scope="module")
def h3():
    from video_dit_dense_amd import h3attn
    h3attn.load_library()
    return h3attn


def check(metrics, label):
    check_metrics(metrics, label, MAX_ABS, REL_RMS)


def gpu(h3, inp, D, **kw):
    d = DevInputs(inp)
    lengths = kw.pop("lengths", None)
    lt = None if lengths is None else torch.tensor(lengths, dtype=torch.int32, device="cuda:0")
    gate = kw.pop("gate_bits", None)
    o = h3.forward(d.q, d.k, d.v, scale=1 / math.sqrt(D), valid_lengths=lt,
                   gate=None if gate is None else to_dev(gate), **kw)
    torch.cuda.synchronize()
    return to_host(o)


def ref(inp, D, rows=None, **kw):
    return oracle.forward(inp.q, inp.k, inp.v, None, None, 1e-6, None, 1 / math.sqrt(D), norm=False, rows=rows,
                          **kw)


# (B, Sq, Sk, H, Hkv, kwargs, label): the dense schedule with split last
# round, padding, causal, grouped heads, per-item lengths, a frame window.
CASES = [
    (1, 2048, 2048, 4, 4, {}, "dense"),
    (1, 1000, 777, 2, 2, {"q_valid": 900, "kv_valid": 700}, "padding, ragged"),
    (1, 1300, 1300, 2, 2, {"causal": True}, "causal"),
    (2, 600, 900, 4, 2, {}, "grouped heads"),
    (1, 1500, 1500, 2, 1, {"window": (100, 3, 1, 1)}, "frame window, one kv head"),
]


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("B,Sq,Sk,H,Hkv,kw,label", CASES)
def test_head_dim(h3, D, B, Sq, Sk, H, Hkv, kw, label):
    say("head dim", D, label)
    inp = workloads.make_inputs(B, Sq, Sk, H, seed=90 + D + Sq % 13, Hkv=Hkv, D=D)
    check(oracle.compare(gpu(h3, inp, D, **kw), ref(inp, D, **kw)), f"D={D} {label}")


@pytest.mark.parametrize("D", [64, 256])
def test_head_dim_lengths_and_gate(h3, D):
    say("head dim", D, "per-item lengths and gate")
    B, S, H = 2, 700, 2
    inp = workloads.make_inputs(B, S, S, H, seed=95 + D, D=D)
    g = workloads.make_gate(B, S, H, seed=95 + D)
    lengths = [[700, 650], [333, 100]]
    got = gpu(h3, inp, D, lengths=lengths, gate_bits=g)
    want = np.concatenate([ref(workloads.Inputs(inp.q[b:b + 1], inp.k[b:b + 1], inp.v[b:b + 1], inp.w_q, inp.w_k),
                               D, q_valid=lengths[b][0], kv_valid=lengths[b][1], gate_bits=g[b:b + 1])
                           for b in range(B)])
    check(oracle.compare(got, want), f"D={D} lengths + gate")


@pytest.mark.parametrize("D", [64, 256])
def test_head_dim_fused_qkv_views(h3, D):
    """q, k, v as slices of one [B, S, 3H, D] projection output equal the
    dense call bit for bit."""
    say("head dim", D, "fused QKV views")
    B, S, H = 1, 800, 2
    inp = workloads.make_inputs(B, S, S, H, seed=97 + D, D=D)
    d = DevInputs(inp)
    qkv = torch.cat([d.q, d.k, d.v], dim=2).contiguous()
    q, k, v = qkv[:, :, :H], qkv[:, :, H:2 * H], qkv[:, :, 2 * H:]
    o1 = h3.forward(q, k, v, scale=1 / math.sqrt(D))
    o2 = h3.forward(d.q, d.k, d.v, scale=1 / math.sqrt(D))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_head_dim_rejections(h3):
    inp = workloads.make_inputs(1, 64, 64, 1, seed=1, D=64)
    d = DevInputs(inp)
    with pytest.raises(ValueError, match="head_dim 128 only"):
        h3.forward(d.q, d.k, d.v, d.w_q, d.w_k)
    with pytest.raises(ValueError, match="D in"):
        h3.forward(d.q[..., :32].contiguous(), d.k[..., :32].contiguous(), d.v[..., :32].contiguous())


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("B,Sq,Sk,H,kw", [
    (1, 1, 1, 1, {}),
    (2, 5, 3, 3, {"kv_valid": 1}),
    (1, 300, 40, 2, {"q_valid": 0}),
    (3, 257, 257, 1, {"causal": True, "kv_valid": 200}),
])
def test_head_dim_degenerate(h3, D, B, Sq, Sk, H, kw):
    say("head dim degenerate", D, B, Sq, Sk, H, kw)
    inp = workloads.make_inputs(B, Sq, Sk, H, seed=7 + Sq, D=D)
    got = gpu(h3, inp, D, **kw)
    want = ref(inp, D, **kw)
    if kw.get("q_valid") == 0:
        assert np.all(got == 0)
        return
    check(oracle.compare(got, want), f"D={D} degenerate {B}x{Sq}x{Sk}x{H} {kw}")


@pytest.mark.parametrize("Sk", [32, 64, 96, 128, 160, 200, 330])
def test_head_dim_256_key_lengths(h3, Sk):
    """Head dim 256 pipelines QK^T two sub-tiles ahead of PV: key lengths of
    1 to 11 sub-tiles cover the prologue alone, the last step without a
    QK^T, whole blocks of ring steps and ragged tails, in the uniform (split
    last round) and per-item-length (one tile per block) schedules."""
    say("head dim 256 key length", Sk)
    inp = workloads.make_inputs(1, 300, Sk, 2, seed=300 + Sk, D=256)
    check(oracle.compare(gpu(h3, inp, 256), ref(inp, 256)), f"D=256 Sk={Sk}")
    got = gpu(h3, inp, 256, lengths=[[300, Sk]])
    check(oracle.compare(got, ref(inp, 256)), f"D=256 Sk={Sk} per-item lengths")


@pytest.mark.parametrize("D,qt", [(64, 0), (128, 0), (128, 3), (256, 0)])
def test_rising_row_maxima(h3, D, qt):
    """Keys whose magnitude grows along the sequence, so each row's running
    maximum rises by many units at several steps and the accumulator is
    rescaled there. q has entries in {-1, 0, 1} and key j entries in
    {-c, 0, c} with c = 1 + j // 256, and the scale is ln 2: q * scale *
    log2(e) stays an exact small integer in bf16, so the scores (exp2 units)
    are exact integers however large, and only v and the output are
    rounded. At head dim 128 also with three query tiles per wave forced."""
    say("rising row maxima", D, qt)
    Sq, Sk, H = 512, 2048, 2
    rng = np.random.default_rng(330 + D)
    qv = rng.integers(-1, 2, size=(1, Sq, H, D)).astype(np.float32)
    c = (1 + np.arange(Sk) // 256).astype(np.float32)
    kv = rng.integers(-1, 2, size=(1, Sk, H, D)).astype(np.float32) * c[None, :, None, None]
    bits = lambda x: (x.view(np.uint32) >> 16).astype(np.uint16)   # exact: small integers
    inp = workloads.make_inputs(1, Sq, Sk, H, seed=330 + D, D=D)
    q, k = bits(qv), bits(kv)
    scale = math.log(2.0)
    d = DevInputs(workloads.Inputs(q, k, inp.v, inp.w_q, inp.w_k))
    o = h3.forward(d.q, d.k, d.v, scale=scale, query_tiles=qt)
    torch.cuda.synchronize()
    want = oracle.forward(q, k, inp.v, None, None, 1e-6, None, scale, norm=False)
    check(oracle.compare(to_host(o), want), f"D={D} rising maxima, query tiles {qt or 'auto'}")
