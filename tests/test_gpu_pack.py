"""GPU parity of the prologue fused with the destination-major Ulysses pack
(h3attn_qkv_pack; TeleFuser PR #37, "2.2 Fuse Q/K RMSNorm, RoPE, and Ulysses
Pack") through the C-ABI, against oracle.ulysses_pack on the same seeded
inputs: every element of the q and k send buffers within half a bf16 ulp of
the exact value (the prologue's bar) and v bit for bit, for P = 1, 2, 3, 4
and 8, ragged shard lengths, two batch items, with and without norm and
rotary, nonzero row offsets and the full shard shape. A simulated
all-to-all of P packed shards must give every rank the stand-alone
prologue of the whole sequence for its heads, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import DevInputs, assert_prologue_rounding, say, to_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def h3():
    from video_dit_dense_amd import h3attn
    h3attn.load_library()
    return h3attn


def run_pack(h3, inp, P, rank, norm, rope, theta=1e4):
    d = DevInputs(inp)
    S = inp.q.shape[1]
    cos = sin = None
    if rope:
        cos, sin = h3.rope_tables((rank + 1) * S, theta)
    qs, ks, vs = h3.qkv_pack(d.q, d.k, d.v, P, row_offset=rank * S, w_q=d.w_q if norm else None,
                             w_k=d.w_k if norm else None, rope_cos=cos, rope_sin=sin)
    torch.cuda.synchronize()
    return to_host(qs), to_host(ks), to_host(vs)


def check_pack(inp, got, P, rank, norm, rope, label):
    S = inp.q.shape[1]
    rq, rk, rv = oracle.ulysses_pack(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, 1e-6, 1e4 if rope else None, P,
                                     row_offset=rank * S, norm=norm)
    assert_prologue_rounding(got[0], rq, f"{label} q")
    assert_prologue_rounding(got[1], rk, f"{label} k")
    assert np.array_equal(got[2], rv), f"{label} v"


@pytest.mark.parametrize("B,S,H,P,rank,norm,rope", [
    (1, 64, 8, 1, 0, True, True),
    (1, 777, 8, 2, 1, True, True),
    (2, 100, 12, 4, 3, True, True),
    (1, 13, 16, 8, 7, True, False),
    (1, 300, 6, 3, 2, False, True),
    (2, 33, 4, 4, 1, False, False),
])
def test_pack_matches_oracle(h3, B, S, H, P, rank, norm, rope):
    say("pack", B, S, H, P, rank, norm, rope)
    inp = workloads.make_inputs(B, S, S, H, seed=700 + S + P)
    got = run_pack(h3, inp, P, rank, norm, rope)
    check_pack(inp, got, P, rank, norm, rope, f"B={B} S={S} H={H} P={P} rank={rank}")


def test_pack_full_shard(h3):
    wl = workloads.PACK_WORKLOADS["pack_shard"]
    say("pack full shard", wl.description)
    inp = workloads.make_pack_inputs(wl)
    got = run_pack(h3, inp, wl.P, wl.rank, True, True, wl.theta)
    check_pack(inp, got, wl.P, wl.rank, True, True, wl.name)


@pytest.mark.parametrize("P,S_local,H", [(8, 1000, 16), (4, 333, 8), (2, 2048, 6)])
def test_simulated_all_to_all_equals_whole_sequence_prologue(h3, P, S_local, H):
    """Rank r receives chunk r of every rank's send buffers in rank order;
    for B = 1 that is the dense [1, S, H/P, 128] of its heads, which must
    equal h3attn_qk_prologue of the whole sequence bit for bit."""
    say("all-to-all", P, S_local, H)
    S = P * S_local
    inp = workloads.make_inputs(1, S, S, H, seed=800 + P)
    d = DevInputs(inp)
    cos, sin = h3.rope_tables(S)
    qo, ko = h3.qk_prologue(d.q, d.k, d.w_q, d.w_k, 1e-6, cos, sin)
    sends = [h3.qkv_pack(d.q[:, r * S_local:(r + 1) * S_local].contiguous(),
                         d.k[:, r * S_local:(r + 1) * S_local].contiguous(),
                         d.v[:, r * S_local:(r + 1) * S_local].contiguous(), P, row_offset=r * S_local,
                         w_q=d.w_q, w_k=d.w_k, rope_cos=cos, rope_sin=sin) for r in range(P)]
    Hl = H // P
    rq, rk = oracle.qk_prologue(inp.q, inp.k, inp.w_q, inp.w_k, 1e-6, 1e4)
    for r in range(P):
        heads = slice(r * Hl, (r + 1) * Hl)
        for t, (whole, exact) in enumerate(((qo, rq), (ko, rk), (d.v, None))):
            recv = torch.cat([sends[src][t][r] for src in range(P)], dim=1)   # [1, S, Hl, 128]
            if exact is not None:
                assert_prologue_rounding(to_host(recv), exact[:, :, heads], f"rank {r} tensor {t}")
            assert torch.equal(recv.view(torch.int16), whole[:, :, heads].contiguous().view(torch.int16)), (r, t)
    torch.cuda.synchronize()
