"""Pins of the fp64 oracle to things other than itself: closed forms written
out by hand (tests/golden), brute force with scalar loops on tiny inputs,
invariants that the mathematics fixes, and torch's CPU float64 SDPA as an
independent library routine. CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _vec(spec, default=0.0, n=128):
    out = np.full(n, spec.get("default", default) if isinstance(spec, dict) else default)
    for key, val in spec.items():
        if key != "default":
            out[int(key)] = val
    return out


# ---------------------------------------------------------------- bf16 inputs

def test_bf16_roundtrip_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(10000).astype(np.float32) * 7,
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38, 1e-40, np.inf, -np.inf],
                 dtype=np.float32),
        # exact ties between two bf16 values, both parities
        (np.arange(1, 200, dtype=np.float32) * 2 + 1) * np.float32(2.0 ** -8) + 1.0,
    ]).astype(np.float32)
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = oracle.bf16_bits_to_f64(ours)
    ref_back = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, ref_back)


def test_bf16_bits_closed_forms():
    vals = oracle.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x3F81], dtype=np.uint16))
    assert list(vals[:5]) == [1.0, -2.0, 0.0, -0.0, math.inf]
    assert vals[5] == 1.0 + 2.0 ** -7


def test_generator_is_deterministic_and_distributed():
    a = workloads.make_inputs(1, 300, 200, 2, seed=7)
    b = workloads.make_inputs(1, 300, 200, 2, seed=7)
    c = workloads.make_inputs(1, 300, 200, 2, seed=8)
    for f in ("q", "k", "v", "w_q", "w_k"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert not np.array_equal(a.q, c.q)
    q = oracle.bf16_bits_to_f64(a.q)
    assert abs(q.mean()) < 0.02 and abs(q.std() - 1.0) < 0.02
    # weights are bf16-representable and near 1 +- 0.1
    assert np.array_equal(workloads.f32_to_bf16_bits(a.w_q), workloads.f32_to_bf16_bits(a.w_q))
    assert np.array_equal(oracle.bf16_bits_to_f64(workloads.f32_to_bf16_bits(a.w_q)), a.w_q.astype(np.float64))
    assert 0.05 < a.w_q.std() < 0.15 and abs(a.w_q.mean() - 1.0) < 0.05


# ------------------------------------------------------------------- RMSNorm

def test_rmsnorm_hand_example():
    g = _load("rmsnorm_hand.json")
    x = _vec(g["x"]).reshape(1, 1, 1, 128)
    w = _vec(g["w"])
    y = oracle.rms_norm(x, w, g["eps"]).reshape(128)
    assert np.allclose(y, _vec(g["y"]), rtol=0, atol=1e-13)


def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5, 2, 128)) * 3
    eps = 1e-2
    y = oracle.rms_norm(x, np.ones(128), eps)
    ms = np.mean(x * x, axis=-1)
    # with w = 1: mean(y^2) = ms / (ms + eps)
    assert np.allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-13, atol=0)
    # zero row maps to zero, eps keeps it finite
    z = oracle.rms_norm(np.zeros((1, 1, 1, 128)), np.ones(128), 1e-6)
    assert np.all(z == 0.0)
    # scale invariance with eps -> 0
    y1 = oracle.rms_norm(x, np.ones(128), 0.0)
    y2 = oracle.rms_norm(7.5 * x, np.ones(128), 0.0)
    assert np.allclose(y1, y2, rtol=1e-13, atol=1e-13)


def test_rmsnorm_brute_force():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 4, 2, 128))
    w = 1 + 0.1 * rng.standard_normal(128)
    eps = 1e-6
    y = oracle.rms_norm(x, w, eps)
    for s in range(4):
        for h in range(2):
            row = [float(t) for t in x[0, s, h]]
            r = math.sqrt(math.fsum(t * t for t in row) / 128.0 + eps)
            for c in range(128):
                assert abs(y[0, s, h, c] - row[c] / r * w[c]) <= 1e-13 * max(1.0, abs(y[0, s, h, c]))


# ---------------------------------------------------------------------- RoPE

def test_rope_inv_freq_closed_forms():
    f = oracle.rope_inv_freq(1e4)
    assert f.shape == (48,)
    assert f[0] == 1.0
    assert abs(f[24] - 0.01) < 1e-16
    assert abs(f[47] - 1e4 ** (-47.0 / 48.0)) < 1e-18
    assert np.all(np.diff(f) < 0)


def test_rope_hand_unit_vectors():
    g = _load("rope_hand.json")
    for case in g["cases"]:
        p = case["position"]
        y = np.zeros((1, p + 1, 1, 128))
        y[0, p, 0, case["channel"]] = 1.0
        out = oracle.apply_rope(y, np.arange(p + 1), g["theta"])[0, p, 0]
        want = _vec(case["out"])
        assert np.allclose(out, want, rtol=0, atol=1e-15), case


def test_rope_invariants():
    rng = np.random.default_rng(3)
    S = 40
    y = rng.standard_normal((2, S, 3, 128))
    pos = np.arange(S)
    r = oracle.apply_rope(y, pos, 1e4)
    # pair norms preserved
    n0 = y[..., :48] ** 2 + y[..., 48:96] ** 2
    n1 = r[..., :48] ** 2 + r[..., 48:96] ** 2
    assert np.allclose(n0, n1, rtol=1e-13, atol=1e-13)
    # position 0 is the identity; channels 96..127 untouched
    assert np.array_equal(r[:, 0], y[:, 0])
    assert np.array_equal(r[..., 96:], y[..., 96:])
    # composition: rotating by p then by p' equals rotating by p + p'
    a = oracle.apply_rope(oracle.apply_rope(y, pos, 1e4), pos * 2, 1e4)
    b = oracle.apply_rope(y, pos * 3, 1e4)
    assert np.allclose(a, b, rtol=1e-11, atol=1e-11)
    # relative position: q(p+D).k(s+D) == q(p).k(s)
    q = rng.standard_normal((1, S, 1, 128))
    k = rng.standard_normal((1, S, 1, 128))
    d0 = np.einsum("bshd,bthd->st", oracle.apply_rope(q, pos, 1e4), oracle.apply_rope(k, pos, 1e4))
    d1 = np.einsum("bshd,bthd->st", oracle.apply_rope(q, pos + 1234, 1e4), oracle.apply_rope(k, pos + 1234, 1e4))
    assert np.allclose(d0, d1, rtol=1e-9, atol=1e-9)


def test_rope_brute_force():
    rng = np.random.default_rng(4)
    S = 6
    y = rng.standard_normal((1, S, 2, 128))
    r = oracle.apply_rope(y, np.arange(S), 1e4)
    for s in range(S):
        for h in range(2):
            for j in range(48):
                phi = s * (1e4 ** (-(2.0 * j) / 96.0))
                a, b = y[0, s, h, j], y[0, s, h, j + 48]
                assert abs(r[0, s, h, j] - (a * math.cos(phi) - b * math.sin(phi))) < 1e-14
                assert abs(r[0, s, h, j + 48] - (b * math.cos(phi) + a * math.sin(phi))) < 1e-14


# ----------------------------------------------------------------- attention

def test_attention_two_key_closed_form():
    g = _load("attention_two_keys.json")
    q = np.zeros((1, 1, 1, 128)); q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 2, 1, 128)); k[0, 1, 0, 0] = g["L"]
    v = np.zeros((1, 2, 1, 128)); v[0, 0, 0] = _vec(g["v0"]); v[0, 1, 0] = _vec(g["v1"])
    o = oracle.attention(q, k, v, g["scale"])[0, 0, 0]
    assert np.allclose(o, _vec(g["o_all"]), rtol=0, atol=1e-13)
    o1 = oracle.attention(q, k, v, g["scale"], kv_valid=1)[0, 0, 0]
    assert np.allclose(o1, _vec(g["o_kv_valid_1"]), rtol=0, atol=0)
    o0 = oracle.attention(q, k, v, g["scale"], q_valid=0)
    assert np.all(o0 == 0.0)


def _sdpa(q, k, v, scale, kv_valid):
    qt = torch.from_numpy(q).transpose(1, 2)
    kt = torch.from_numpy(k).transpose(1, 2)
    vt = torch.from_numpy(v).transpose(1, 2)
    mask = torch.zeros(q.shape[1], k.shape[1], dtype=torch.bool)
    mask[:, :kv_valid] = True
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.transpose(1, 2).numpy()


@pytest.mark.parametrize("B,Sq,Sk,H,kv_valid,block", [
    (1, 300, 300, 2, 300, 256),
    (2, 257, 700, 3, 513, 64),
    (1, 1000, 37, 1, 1, 128),
])
def test_attention_matches_torch_sdpa_fp64(B, Sq, Sk, H, kv_valid, block):
    rng = np.random.default_rng(B * 1000 + Sq)
    q = rng.standard_normal((B, Sq, H, 128)) * 1.5
    k = rng.standard_normal((B, Sk, H, 128)) * 1.5
    v = rng.standard_normal((B, Sk, H, 128))
    o = oracle.attention(q, k, v, 1 / math.sqrt(128), kv_valid=kv_valid, block=block)
    ref = _sdpa(q, k, v, 1 / math.sqrt(128), kv_valid)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_attention_brute_force():
    rng = np.random.default_rng(6)
    B, Sq, Sk, H = 1, 7, 9, 2
    q = rng.standard_normal((B, Sq, H, 128))
    k = rng.standard_normal((B, Sk, H, 128))
    v = rng.standard_normal((B, Sk, H, 128))
    scale, qv, kvv = 0.11, 5, 6
    o = oracle.attention(q, k, v, scale, q_valid=qv, kv_valid=kvv)
    for h in range(H):
        for i in range(Sq):
            if i >= qv:
                assert np.all(o[0, i, h] == 0.0)
                continue
            s = [scale * math.fsum(q[0, i, h, c] * k[0, j, h, c] for c in range(128)) for j in range(kvv)]
            m = max(s)
            e = [math.exp(t - m) for t in s]
            z = math.fsum(e)
            for c in range(128):
                ref = math.fsum(e[j] * v[0, j, h, c] for j in range(kvv)) / z
                assert abs(o[0, i, h, c] - ref) < 1e-13


def test_attention_invariants():
    rng = np.random.default_rng(7)
    B, S, H = 1, 96, 2
    scale = 1 / math.sqrt(128)
    q = rng.standard_normal((B, S, H, 128))
    k = rng.standard_normal((B, S, H, 128))
    v = rng.standard_normal((B, S, H, 128))
    o = oracle.attention(q, k, v, scale)
    # (1) softmax rows sum to 1: V = identity (Sk <= 128) returns P itself
    eye = np.zeros((B, S, H, 128)); eye[0, np.arange(S), :, np.arange(S)] = 1.0
    p = oracle.attention(q, k, eye, scale)
    assert np.allclose(p[..., :S].sum(-1), 1.0, rtol=0, atol=1e-13)
    assert np.all(p[..., :S] > 0) and np.all(p[..., S:] == 0)
    # (2) constant V gives V
    cv = np.broadcast_to(rng.standard_normal((1, 1, H, 128)), v.shape).copy()
    assert np.allclose(oracle.attention(q, k, cv, scale), cv, rtol=0, atol=1e-13)
    # (3) one valid key returns its value
    assert np.allclose(oracle.attention(q, k, v, scale, kv_valid=1), np.broadcast_to(v[:, :1], o.shape), atol=0)
    # (4) joint K/V row permutation leaves O unchanged
    perm = rng.permutation(S)
    assert np.allclose(oracle.attention(q, k[:, perm], v[:, perm], scale), o, rtol=1e-12, atol=1e-13)
    # (5) masked keys have no effect, even when NaN
    kk, vv = k.copy(), v.copy()
    kk[:, 50:] = np.nan; vv[:, 50:] = 1e4
    a = oracle.attention(q, kk, vv, scale, kv_valid=50)
    b = oracle.attention(q, k[:, :50], v[:, :50], scale)
    assert np.array_equal(a, b)
    # (6) Q = 0 gives the mean of the valid values
    z = oracle.attention(np.zeros_like(q), k, v, scale, kv_valid=64)
    assert np.allclose(z, np.broadcast_to(v[:, :64].mean(axis=1, keepdims=True), z.shape), atol=1e-14)
    # (7) rows past q_valid are exactly zero, rows before are unchanged
    t = oracle.attention(q, k, v, scale, q_valid=40)
    assert np.all(t[:, 40:] == 0.0) and np.array_equal(t[:, :40], o[:, :40])
    # (8) linear in V
    v2 = rng.standard_normal(v.shape)
    lin = oracle.attention(q, k, 2 * v - 3 * v2, scale)
    assert np.allclose(lin, 2 * o - 3 * oracle.attention(q, k, v2, scale), atol=1e-12)
    # rows subset equals the full computation at those rows
    rows = np.array([0, 5, 17, 95])
    assert np.allclose(oracle.attention(q, k, v, scale, rows=rows), o[:, rows], rtol=1e-13, atol=1e-14)


def test_forward_composes_prologue_and_attention():
    inp = workloads.make_inputs(1, 64, 48, 2, seed=11)
    qn, kn = oracle.qk_prologue(inp.q, inp.k, inp.w_q, inp.w_k, 1e-6, 1e4)
    # prologue = rope(norm(x)) step by step
    q64 = oracle.bf16_bits_to_f64(inp.q)
    want = oracle.apply_rope(oracle.rms_norm(q64, inp.w_q, 1e-6), np.arange(64), 1e4)
    assert np.array_equal(qn, want)
    o = oracle.forward(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, 1e-6, 1e4, 1 / math.sqrt(128),
                       q_valid=60, kv_valid=40)
    ref = _sdpa(qn, kn, oracle.bf16_bits_to_f64(inp.v), 1 / math.sqrt(128), 40)
    ref[:, 60:] = 0
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)
    rows = np.array([0, 33, 59, 60, 63])
    o_rows = oracle.forward(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, 1e-6, 1e4, 1 / math.sqrt(128),
                            q_valid=60, kv_valid=40, rows=rows)
    assert np.allclose(o_rows, o[:, rows], rtol=1e-13, atol=1e-14)


def test_compare_metrics():
    ref = np.array([1.0, 2.0, -4.0, 0.5])
    got = workloads.f32_to_bf16_bits((ref + np.array([2 ** -8, 0, 0, 0])).astype(np.float32))
    m = oracle.compare(got, ref)
    assert m["nonfinite"] == 0
    assert m["max_abs"] <= 2 ** -7
    assert m["max_ulp"] <= 1.0


# ------------------------------------------- attention variants: causal, GQA, per-batch lengths

def test_attention_variants_brute_force():
    """Causal mask composed with key padding, grouped heads and per-item valid
    lengths, against scalar loops (FastVideo PR #1799, "Implementation")."""
    rng = np.random.default_rng(21)
    B, Sq, Sk, H, Hkv = 2, 7, 9, 4, 2
    q = rng.standard_normal((B, Sq, H, 128))
    k = rng.standard_normal((B, Sk, Hkv, 128))
    v = rng.standard_normal((B, Sk, Hkv, 128))
    scale, qv, kvv = 0.13, [5, 7], [6, 3]
    o = oracle.attention(q, k, v, scale, q_valid=qv, kv_valid=kvv, causal=True)
    for b in range(B):
        for h in range(H):
            hk = h // (H // Hkv)
            for i in range(Sq):
                if i >= qv[b]:
                    assert np.all(o[b, i, h] == 0.0)
                    continue
                keys = [j for j in range(Sk) if j < kvv[b] and j <= i]
                s = [scale * math.fsum(q[b, i, h, c] * k[b, j, hk, c] for c in range(128)) for j in keys]
                m = max(s)
                e = [math.exp(t - m) for t in s]
                z = math.fsum(e)
                for c in range(128):
                    ref = math.fsum(e[n] * v[b, j, hk, c] for n, j in enumerate(keys)) / z
                    assert abs(o[b, i, h, c] - ref) < 1e-13


def _sdpa_masked(q, k, v, scale, mask, gqa):
    """torch CPU float64 SDPA with a boolean [B, 1, Sq, Sk] mask (True = attend)."""
    qt = torch.from_numpy(q).transpose(1, 2)
    kt = torch.from_numpy(k).transpose(1, 2)
    vt = torch.from_numpy(v).transpose(1, 2)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask),
                                                         scale=scale, enable_gqa=gqa)
    return o.transpose(1, 2).numpy()


@pytest.mark.parametrize("B,Sq,Sk,H,Hkv,qv,kvv,causal", [
    (1, 300, 300, 2, 2, 300, 300, True),        # causal self-attention
    (1, 300, 300, 2, 2, 300, 211, True),        # causal composed with key padding
    (2, 257, 257, 4, 1, [257, 130], [257, 90], True),   # per-item lengths, one kv head (MQA)
    (2, 129, 400, 6, 2, [129, 77], [400, 1], False),    # GQA cross-attention, per-item lengths
])
def test_attention_variants_match_torch_sdpa_fp64(B, Sq, Sk, H, Hkv, qv, kvv, causal):
    rng = np.random.default_rng(Sq * 7 + Sk + H)
    q = rng.standard_normal((B, Sq, H, 128)) * 1.5
    k = rng.standard_normal((B, Sk, Hkv, 128)) * 1.5
    v = rng.standard_normal((B, Sk, Hkv, 128))
    scale = 1 / math.sqrt(128)
    o = oracle.attention(q, k, v, scale, q_valid=qv, kv_valid=kvv, causal=causal, block=64)
    qvl = qv if isinstance(qv, list) else [qv] * B
    kvl = kvv if isinstance(kvv, list) else [kvv] * B
    mask = np.zeros((B, 1, Sq, Sk), dtype=bool)
    for b in range(B):
        mask[b, 0, :, :kvl[b]] = True
    if causal:
        mask &= torch.tril(torch.ones(Sq, Sk, dtype=torch.bool)).numpy()[None, None]
    ref = _sdpa_masked(q, k, v, scale, mask, Hkv != H)
    for b in range(B):
        ref[b, qvl[b]:] = 0.0
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_attention_variant_invariants():
    rng = np.random.default_rng(22)
    B, S, H, Hkv = 1, 80, 4, 2
    scale = 1 / math.sqrt(128)
    q = rng.standard_normal((B, S, H, 128))
    k = rng.standard_normal((B, S, Hkv, 128))
    v = rng.standard_normal((B, S, Hkv, 128))
    o = oracle.attention(q, k, v, scale, causal=True)
    # causal row 0 sees only key 0: returns v_0 of its kv head
    assert np.array_equal(o[0, 0], v[0, 0, np.arange(H) // 2])
    # keys and values after position t do not change rows <= t (finite values:
    # a causally masked key still meets a zero weight, and 0 * NaN is NaN)
    t = 37
    k2, v2 = k.copy(), v.copy()
    k2[:, t + 1:] = rng.standard_normal(k2[:, t + 1:].shape) * 5
    v2[:, t + 1:] = rng.standard_normal(v2[:, t + 1:].shape) * 1e6
    o2 = oracle.attention(q, k2, v2, scale, causal=True)
    assert np.array_equal(o2[:, :t + 1], o[:, :t + 1])
    # grouped heads equal multi-head attention with each kv head repeated
    rep_k, rep_v = np.repeat(k, H // Hkv, axis=2), np.repeat(v, H // Hkv, axis=2)
    assert np.array_equal(oracle.attention(q, rep_k, rep_v, scale, causal=True), o)
    # causal with kv_valid = 1: every row returns v_0
    o1 = oracle.attention(q, k, v, scale, kv_valid=1, causal=True)
    assert np.array_equal(o1, np.broadcast_to(v[:, :1, np.arange(H) // 2], o1.shape))
    # per-item lengths: each item equals a one-item call with its own lengths
    qb = rng.standard_normal((3, 50, H, 128))
    kb = rng.standard_normal((3, 70, Hkv, 128))
    vb = rng.standard_normal((3, 70, Hkv, 128))
    qv, kvv = [50, 11, 30], [70, 5, 64]
    ob = oracle.attention(qb, kb, vb, scale, q_valid=qv, kv_valid=kvv, causal=True)
    for b in range(3):
        one = oracle.attention(qb[b:b + 1], kb[b:b + 1], vb[b:b + 1], scale, q_valid=qv[b], kv_valid=kvv[b],
                               causal=True)
        assert np.array_equal(ob[b:b + 1], one)
    # rows subset equals the full causal computation at those rows
    rows = np.array([0, 1, 37, 79])
    assert np.allclose(oracle.attention(q, k, v, scale, rows=rows, causal=True), o[:, rows], rtol=1e-13, atol=1e-14)


# ------------------------------------------- frame-window attention with the softmax gate

def _ranges(spec):
    spec = spec if isinstance(spec[0], list) else [spec]
    return sorted(j for lo, hi in spec for j in range(lo, hi))


def test_window_visibility_hand():
    g = _load("window_hand.json")
    for case in g["cases"]:
        vis = oracle.window_visible(np.arange(case["S"]), np.arange(case["S"]),
                                    case["F"], case["C"], case["R"], case["A"])
        for row, spec in case["visible"].items():
            assert list(np.flatnonzero(vis[int(row)])) == _ranges(spec), (case, row)
    for x, want in g["gate"]["sigmoid"].items():
        assert abs(oracle.sigmoid(float(x)) - want) < 1e-15


def _window_keys_constructive(i, S, F, C, R, A):
    """The visible keys of row i built from frame lists: every key of a dense
    row; else the anchor frames' rows and the rows of every frame in chunks
    c-R .. c+R (chunk c covers frames A + cC .. A + cC + C - 1)."""
    n_frames = (S + F - 1) // F
    f = i // F
    if f < A:
        return set(range(S))
    c = (f - A) // C
    frames = set(range(min(A, n_frames)))
    for cc in range(c - R, c + R + 1):
        for ff in range(A + cc * C, A + cc * C + C):
            if A <= ff < n_frames:
                frames.add(ff)
    return {j for ff in frames for j in range(ff * F, min(S, ff * F + F))}


@pytest.mark.parametrize("F,C,R,A,S", [(3, 2, 1, 1, 40), (4, 5, 1, 2, 61), (5, 1, 0, 0, 33), (2, 3, 2, 0, 50),
                                       (7, 2, 0, 3, 70)])
def test_window_visibility_constructive(F, C, R, A, S):
    vis = oracle.window_visible(np.arange(S), np.arange(S), F, C, R, A)
    for i in range(S):
        assert set(np.flatnonzero(vis[i]).tolist()) == _window_keys_constructive(i, S, F, C, R, A), i


def _window_mask(B, Sq, Sk, F, C, R, A, qvl, kvl):
    mask = np.zeros((B, 1, Sq, Sk), dtype=bool)
    for b in range(B):
        for i in range(Sq):
            for j in _window_keys_constructive(i, max(Sq, Sk), F, C, R, A):
                if j < kvl[b]:
                    mask[b, 0, i, j] = True
    return mask


@pytest.mark.parametrize("B,S,H,Hkv,F,C,R,A,qv,kvv", [
    (1, 96, 2, 2, 8, 2, 1, 1, 96, 96),
    (2, 130, 4, 2, 10, 3, 1, 2, [130, 77], [130, 101]),
    (1, 150, 3, 1, 6, 5, 0, 0, 150, 150),
])
def test_window_attention_matches_torch_sdpa_fp64(B, S, H, Hkv, F, C, R, A, qv, kvv):
    rng = np.random.default_rng(S + F * 3 + R)
    q = rng.standard_normal((B, S, H, 128)) * 1.5
    k = rng.standard_normal((B, S, Hkv, 128)) * 1.5
    v = rng.standard_normal((B, S, Hkv, 128))
    gate = rng.standard_normal((B, S, H)) * 2
    scale = 1 / math.sqrt(128)
    o = oracle.attention(q, k, v, scale, q_valid=qv, kv_valid=kvv, window=(F, C, R, A), gate=gate, block=64)
    qvl = qv if isinstance(qv, list) else [qv] * B
    kvl = kvv if isinstance(kvv, list) else [kvv] * B
    mask = _window_mask(B, S, S, F, C, R, A, qvl, kvl)
    ref = _sdpa_masked(q, k, v, scale, mask, Hkv != H)
    ref = ref * (1.0 / (1.0 + np.exp(-gate)))[..., None]
    for b in range(B):
        ref[b, qvl[b]:] = 0.0
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_window_attention_invariants():
    rng = np.random.default_rng(23)
    B, S, H = 1, 120, 2
    F, C, R, A = 6, 2, 1, 1
    scale = 1 / math.sqrt(128)
    q = rng.standard_normal((B, S, H, 128))
    k = rng.standard_normal((B, S, H, 128))
    v = rng.standard_normal((B, S, H, 128))
    dense = oracle.attention(q, k, v, scale)
    # a radius covering every chunk is dense attention
    assert np.array_equal(oracle.attention(q, k, v, scale, window=(F, C, 100, A)), dense)
    # anchor frames covering the whole sequence: every row is a dense row
    assert np.array_equal(oracle.attention(q, k, v, scale, window=(F, C, 0, 100)), dense)
    o = oracle.attention(q, k, v, scale, window=(F, C, R, A))
    # rows of the anchor frame are dense rows
    assert np.array_equal(o[:, :F], dense[:, :F])
    # keys outside a row's window do not affect it: chunk 0 = frames 1-2 sees
    # frames 0-4 (rows 0..29); rewrite rows 30.. of k and v
    k2, v2 = k.copy(), v.copy()
    k2[:, 30:] = rng.standard_normal(k2[:, 30:].shape) * 9
    v2[:, 30:] = 1e6
    o2 = oracle.attention(q, k2, v2, scale, window=(F, C, R, A))
    assert np.array_equal(o2[:, F:3 * F], o[:, F:3 * F])
    # gate 0 halves the output exactly; a gate of 40 leaves it to 1e-17
    g0 = np.zeros((B, S, H))
    assert np.array_equal(oracle.attention(q, k, v, scale, window=(F, C, R, A), gate=g0), o * 0.5)
    g40 = np.full((B, S, H), 40.0)
    assert np.allclose(oracle.attention(q, k, v, scale, window=(F, C, R, A), gate=g40), o, rtol=1e-16, atol=1e-17)
    # q = 0: each row is the mean of the v rows it sees
    q0 = np.zeros_like(q)
    o0 = oracle.attention(q0, k, v, scale, window=(F, C, R, A))
    vis = oracle.window_visible(np.arange(S), np.arange(S), F, C, R, A)
    for i in (0, 7, 40, 119):
        assert np.allclose(o0[0, i], v[0, vis[i]].mean(axis=0), rtol=1e-13, atol=1e-14)
    # no anchors, radius 0, keys cut at kv_valid: a row whose chunk lies past
    # kv_valid sees nothing and is 0
    oz = oracle.attention(q, k, v, scale, kv_valid=20, window=(F, C, 0, 0))
    assert np.all(oz[0, 24:] == 0.0) and np.all(np.isfinite(oz))
    # sigmoid: symmetry and no overflow at the extremes
    x = np.array([-1000.0, -3.0, 0.0, 3.0, 1000.0])
    sg = oracle.sigmoid(x)
    assert np.allclose(sg + oracle.sigmoid(-x), 1.0, rtol=0, atol=4e-16)
    assert sg[0] == 0.0 and sg[-1] == 1.0


@pytest.mark.parametrize("D", [64, 256])
def test_attention_head_dims_match_torch_sdpa_fp64(D):
    """The oracle's attention at the backend's other head dims (FastVideo PR
    #1799, "Implementation": 64, 128 and 256), with padding, grouped heads
    and the causal mask, against torch's CPU float64 SDPA."""
    rng = np.random.default_rng(D)
    B, Sq, Sk, H, Hkv = 2, 150, 170, 4, 2
    q = rng.standard_normal((B, Sq, H, D))
    k = rng.standard_normal((B, Sk, Hkv, D))
    v = rng.standard_normal((B, Sk, Hkv, D))
    scale = 1 / math.sqrt(D)
    for causal in (False, True):
        o = oracle.attention(q, k, v, scale, q_valid=[150, 99], kv_valid=[170, 120], causal=causal, block=64)
        mask = np.zeros((B, 1, Sq, Sk), dtype=bool)
        mask[0, 0, :, :170] = True
        mask[1, 0, :, :120] = True
        if causal:
            mask &= torch.tril(torch.ones(Sq, Sk, dtype=torch.bool)).numpy()[None, None]
        ref = _sdpa_masked(q, k, v, scale, mask, True)
        ref[1, 99:] = 0.0
        assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)
