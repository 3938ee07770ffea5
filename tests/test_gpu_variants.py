"""GPU parity of the attention variants (FastVideo PR #1799, "Implementation":
MHA and GQA, causal attention, padding and causal masks combined), per-item
valid lengths and strided q/k/v views, through h3attn_forward_ex, against the
fp64 oracle on the same seeded inputs. Bar: max-abs <= 2e-2 and relative RMS
<= 5e-3 on the bf16 outputs, as for the dense step."""
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


def gpu(h3, d, *, causal=False, q_valid=None, kv_valid=None, lengths=None, norm=True, rope=True, views=None):
    q, k, v = views if views is not None else (d.q, d.k, d.v)
    cos = sin = None
    if rope:
        cos, sin = h3.rope_tables(max(q.shape[1], k.shape[1]))
    lt = None if lengths is None else torch.tensor(lengths, dtype=torch.int32, device="cuda:0")
    o = h3.forward(q, k, v, d.w_q if norm else None, d.w_k if norm else None, 1e-6, cos, sin,
                   q_valid=q_valid, kv_valid=kv_valid, scale=SCALE, causal=causal, valid_lengths=lt)
    torch.cuda.synchronize()
    return to_host(o)


def ref(inp, *, causal=False, q_valid=None, kv_valid=None, norm=True, rope=True, rows=None):
    return oracle.forward(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, 1e-6, 1e4 if rope else None, SCALE,
                          q_valid=q_valid, kv_valid=kv_valid, norm=norm, rows=rows, causal=causal)


@pytest.mark.parametrize("B,S,H,seed", [(1, 256, 2, 31), (1, 1000, 3, 32), (2, 2085, 2, 33)])
def test_causal_self_attention(h3, B, S, H, seed):
    say("causal", B, S, H)
    inp = workloads.make_inputs(B, S, S, H, seed)
    got = gpu(h3, DevInputs(inp), causal=True)
    check(oracle.compare(got, ref(inp, causal=True)), f"causal B={B} S={S} H={H}")


@pytest.mark.parametrize("Sq,Sk,qv,kvv", [(1536, 1536, 1200, 1100), (1536, 1536, 1100, 1300),
                                          (700, 1300, 650, 1300), (1300, 700, 1300, 333)])
def test_causal_with_padding_and_unequal_lengths(h3, Sq, Sk, qv, kvv):
    say("causal+padding", Sq, Sk, qv, kvv)
    inp = workloads.make_inputs(1, Sq, Sk, 2, 34 + Sq + Sk)
    d = DevInputs(inp)
    got = gpu(h3, d, causal=True, q_valid=qv, kv_valid=kvv)
    check(oracle.compare(got, ref(inp, causal=True, q_valid=qv, kv_valid=kvv)), "causal+padding")
    assert np.all(got[:, qv:] == 0)
    # keys past kv_valid are never read: poisoning them changes nothing
    kp, vp = d.k.clone(), d.v.clone()
    kp[:, kvv:] = float("nan")
    vp[:, kvv:] = float("inf")
    got2 = gpu(h3, d, causal=True, q_valid=qv, kv_valid=kvv, views=(d.q, kp, vp))
    assert np.array_equal(got, got2)


@pytest.mark.parametrize("B,S,Hq,Hkv,causal", [(1, 4096, 8, 2, False), (1, 1000, 6, 1, False),
                                               (2, 777, 4, 2, True), (1, 2048, 8, 1, True)])
def test_grouped_heads(h3, B, S, Hq, Hkv, causal):
    # (1, 4096, 8, 2): 128 query tiles on 256 compute units, so the uniform
    # schedule splits every tile's key steps and merges partial results.
    say("gqa", B, S, Hq, Hkv, causal)
    inp = workloads.make_inputs(B, S, S, Hq, 40 + S, Hkv=Hkv)
    got = gpu(h3, DevInputs(inp), causal=causal)
    check(oracle.compare(got, ref(inp, causal=causal)), f"gqa Hq={Hq} Hkv={Hkv} causal={causal}")


def _clamp(v, hi):
    return max(0, min(int(v), hi))


@pytest.mark.parametrize("causal", [False, True])
def test_per_item_valid_lengths(h3, causal):
    B, S, H = 4, 1000, 2
    lengths = [[1000, 1000], [300, 1000], [1000, 37], [-5, 99999]]
    say("per-item lengths", lengths, causal)
    inp = workloads.make_inputs(B, S, S, H, 50)
    got = gpu(h3, DevInputs(inp), causal=causal, lengths=lengths)
    qv = [_clamp(a, S) for a, _ in lengths]
    kvv = [_clamp(b, S) for _, b in lengths]
    want = ref(inp, causal=causal, q_valid=qv, kv_valid=kvv)
    check(oracle.compare(got, want), f"per-item causal={causal}")
    assert np.all(got[1, 300:] == 0) and np.all(got[3] == 0)


def test_item_without_keys_writes_zeros(h3):
    inp = workloads.make_inputs(2, 300, 300, 2, 51)
    got = gpu(h3, DevInputs(inp), lengths=[[300, 0], [300, 300]])
    assert np.all(got[0] == 0)
    check(oracle.compare(got[1:], ref(workloads.Inputs(inp.q[1:], inp.k[1:], inp.v[1:], inp.w_q, inp.w_k))),
          "second item")


@pytest.mark.parametrize("Hq,Hkv,causal", [(4, 4, False), (6, 2, True)])
def test_fused_qkv_views(h3, Hq, Hkv, causal):
    """q, k, v as slices of one [B, S, Hq + 2*Hkv, 128] projection output."""
    B, S = 2, 1111
    say("fused qkv", Hq, Hkv, causal)
    inp = workloads.make_inputs(B, S, S, Hq, 60, Hkv=Hkv)
    d = DevInputs(inp)
    x = torch.cat([d.q, d.k, d.v], dim=2)
    views = (x[:, :, :Hq], x[:, :, Hq:Hq + Hkv], x[:, :, Hq + Hkv:])
    assert not views[0].is_contiguous()
    got = gpu(h3, d, causal=causal, views=views)
    check(oracle.compare(got, ref(inp, causal=causal)), "fused views")
    dense = gpu(h3, d, causal=causal)
    assert np.array_equal(got, dense)   # the layout changes no arithmetic


def test_variant_repeat_runs_are_bitwise_identical(h3):
    inp = workloads.make_inputs(3, 1500, 1500, 4, 70, Hkv=2)
    d = DevInputs(inp)
    lengths = [[1500, 1500], [900, 1400], [1333, 257]]
    a = gpu(h3, d, causal=True, lengths=lengths)
    b = gpu(h3, d, causal=True, lengths=lengths)
    assert np.array_equal(a, b)
