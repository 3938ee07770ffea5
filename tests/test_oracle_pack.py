"""Pins of the oracle's destination-major Ulysses pack (oracle.ulysses_pack,
TeleFuser PR #37, "2.2 Fuse Q/K RMSNorm, RoPE, and Ulysses Pack", step 4;
the all-to-all of section 2.1), independent of its own code:

- scalar brute force: every element of every destination chunk against a
  pure-Python RMSNorm + rotary of the source element at its global
  position, and v bit for bit;
- a simulated all-to-all: a whole sequence split into P shards, each packed
  with its own row offset; rank r collects chunk r of every shard in shard
  order and must hold exactly the whole-sequence prologue of its heads;
- P = 1 is the plain prologue at the shard's positions; heads that do not
  split evenly are refused.
A dropped row offset, a transposed destination index or heads taken in the
wrong order each fail one of these."""
import math

import numpy as np
import pytest

import oracle
import workloads


def brute_prologue_elem(x_row, w, eps, theta, pos, c):
    """Channel c of one 128-channel row after RMSNorm and the rotary
    embedding on channels 0..95 (pairs (j, j+48), angle pos * theta^(-j/48))."""
    xs = [float(oracle.bf16_bits_to_f64(b)) for b in x_row]
    r = math.sqrt(math.fsum(x * x for x in xs) / 128.0 + eps)
    y = [xs[i] / r * float(w[i]) for i in range(128)]
    if theta is None or c >= 96:
        return y[c]
    j = c % 48
    phi = pos * theta ** (-2.0 * j / 96.0)
    a, b = y[j], y[j + 48]
    return a * math.cos(phi) - b * math.sin(phi) if c < 48 else b * math.cos(phi) + a * math.sin(phi)


def test_pack_against_scalar_brute_force():
    B, S, H, P, off = 2, 3, 4, 2, 5
    inp = workloads.make_inputs(B, S, S, H, seed=501)
    qs, ks, vs = oracle.ulysses_pack(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, 1e-6, 1e4, P, row_offset=off)
    Hl = H // P
    assert qs.shape == ks.shape == vs.shape == (P, B, S, Hl, 128)
    rng = np.random.default_rng(7)
    for p in range(P):
        for b in range(B):
            for s in range(S):
                for j in range(Hl):
                    h = p * Hl + j
                    assert np.array_equal(vs[p, b, s, j], inp.v[b, s, h])
                    for c in rng.choice(128, 12, replace=False).tolist() + [0, 47, 48, 95, 96, 127]:
                        want_q = brute_prologue_elem(inp.q[b, s, h], inp.w_q, 1e-6, 1e4, off + s, c)
                        want_k = brute_prologue_elem(inp.k[b, s, h], inp.w_k, 1e-6, 1e4, off + s, c)
                        assert abs(qs[p, b, s, j, c] - want_q) <= 1e-12 * max(1.0, abs(want_q)), (p, b, s, j, c)
                        assert abs(ks[p, b, s, j, c] - want_k) <= 1e-12 * max(1.0, abs(want_k)), (p, b, s, j, c)


@pytest.mark.parametrize("P,S_local,H,rope,norm", [(4, 7, 8, True, True), (2, 33, 6, False, True),
                                                   (8, 5, 8, True, False), (3, 11, 9, True, True)])
def test_simulated_all_to_all_gives_each_rank_its_heads(P, S_local, H, rope, norm):
    S = P * S_local
    inp = workloads.make_inputs(1, S, S, H, seed=600 + P)
    theta = 1e4 if rope else None
    full_q, full_k = oracle.qk_prologue(inp.q, inp.k, inp.w_q, inp.w_k, 1e-6, theta, norm=norm)
    shards = []
    for rank in range(P):
        rows = slice(rank * S_local, (rank + 1) * S_local)
        shards.append(oracle.ulysses_pack(inp.q[:, rows], inp.k[:, rows], inp.v[:, rows], inp.w_q, inp.w_k, 1e-6,
                                          theta, P, row_offset=rank * S_local, norm=norm))
    Hl = H // P
    for r in range(P):
        # Rank r receives chunk r of every source rank, in source order.
        got_q = np.concatenate([shards[src][0][r] for src in range(P)], axis=1)
        got_k = np.concatenate([shards[src][1][r] for src in range(P)], axis=1)
        got_v = np.concatenate([shards[src][2][r] for src in range(P)], axis=1)
        heads = slice(r * Hl, (r + 1) * Hl)
        assert np.array_equal(got_q, full_q[:, :, heads])
        assert np.array_equal(got_k, full_k[:, :, heads])
        assert np.array_equal(got_v, inp.v[:, :, heads])


def test_single_rank_is_the_prologue_at_the_shard_positions():
    inp = workloads.make_inputs(2, 9, 9, 3, seed=602)
    qs, ks, vs = oracle.ulysses_pack(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, 1e-6, 1e4, 1, row_offset=40)
    q0, k0 = oracle.qk_prologue(inp.q, inp.k, inp.w_q, inp.w_k, 1e-6, 1e4, row_offset=40)
    assert np.array_equal(qs[0], q0) and np.array_equal(ks[0], k0) and np.array_equal(vs[0], inp.v)
    # the row offset is a shift of the rotary positions: rows 40.. of a longer sequence
    big = workloads.make_inputs(2, 49, 49, 3, seed=603)
    big.q[:, 40:], big.k[:, 40:] = inp.q, inp.k
    qb, kb = oracle.qk_prologue(big.q, big.k, inp.w_q, inp.w_k, 1e-6, 1e4)
    assert np.array_equal(qb[:, 40:], q0) and np.array_equal(kb[:, 40:], k0)


def test_uneven_heads_are_refused():
    inp = workloads.make_inputs(1, 4, 4, 6, seed=604)
    with pytest.raises(ValueError):
        oracle.ulysses_pack(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, 1e-6, 1e4, 4)
