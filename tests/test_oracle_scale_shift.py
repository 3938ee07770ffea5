"""Pins of the RMSNorm + indexed scale/shift oracle to things other than
itself: a row worked by hand (tests/golden/scale_shift_hand.json), torch's CPU
bf16 conversion and bf16 tensor arithmetic as independent implementations of
the rounding steps, exact rational arithmetic for the per-row factor, and
invariants. CPU only."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import scale_shift as ss

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(values):
    return torch.tensor(values, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _torch_bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _torch_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def test_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "scale_shift_hand.json")))
    x = _bits(g["x"])[None]
    scale = _bits(g["scale"])[None]
    shift = _bits(g["shift"])[None]
    index = np.array([g["index"]], dtype=np.int32)
    w = np.array(g["w"], dtype=np.float32)
    y = ss.rmsnorm_scale_shift(x, w, g["eps"], scale, shift, index)
    assert np.array_equal(ss.bf16_to_f32(y)[0], np.array(g["y"], dtype=np.float32))
    # The factor is exactly one half.
    assert ss.inv_rms(x, g["eps"])[0][0, 0] == np.float32(0.5)


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(11)
    f = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),          # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895e38, 3.3961e38, -3.3961e38, 3.4028235e38,
                  1.00390625, 1.01171875, -1.00390625], dtype=np.float32),
        # every tie between neighbouring bf16 values around 1, 2 and 1e-3
        ((np.arange(0, 256, dtype=np.float32) * 2 + 1) * np.float32(2.0 ** -8) + np.float32(1.0)),
        ((np.arange(0, 256, dtype=np.float32) * 2 + 1) * np.float32(2.0 ** -7) + np.float32(2.0)),
    ]).astype(np.float32)
    ours = ss.bf16_rne(f)
    ref = _torch_bits(torch.from_numpy(f).to(torch.bfloat16))
    assert np.array_equal(ours, ref)
    nan = ss.bf16_rne(np.array([np.nan, -np.nan], dtype=np.float32))
    assert np.all(np.isnan(ss.bf16_to_f32(nan)))


def test_bf16_to_f32_closed_forms():
    v = ss.bf16_to_f32(np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F80], dtype=np.uint16))
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == np.float32(3.140625)
    assert v[3] == np.float32(2.0 ** -133) and np.isinf(v[4])


@pytest.mark.parametrize("spread", [1.0, 1e4])
def test_modulate_matches_torch_bf16_arithmetic(spread):
    """t, u and y are bf16 tensor arithmetic; torch's CPU bf16 kernels compute
    each operation in fp32 and round, independently of this code."""
    rng = np.random.default_rng(12)
    shape = (64, 257)
    def draw(s):
        mag = np.exp(rng.uniform(-np.log(s), np.log(s), shape)) if s > 1 else 1.0
        return _bits((rng.standard_normal(shape) * mag).astype(np.float32))
    n, sc, sh = draw(spread), draw(spread), draw(spread)
    ours = ss.modulate(n, sc, sh)
    tn, tsc, tsh = _torch_bf16(n), _torch_bf16(sc), _torch_bf16(sh)
    ref = _torch_bits(tn * (1 + tsc) + tsh)
    assert np.array_equal(ours, ref)


def test_norm_rounding_matches_torch_bf16_cast():
    """n = bf16(fp32(x * r) * w): two fp32 products and one cast, as torch
    computes them on float32 tensors."""
    rng = np.random.default_rng(13)
    x = _bits(rng.standard_normal((40, 96)).astype(np.float32))
    r = rng.uniform(0.1, 4.0, (40, 1)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(96)).astype(np.float32)
    ours = ss.norm_bf16(x, r, w)
    tx = _torch_bf16(x).float()
    ref = _torch_bits((tx * torch.from_numpy(r) * torch.from_numpy(w)).to(torch.bfloat16))
    assert np.array_equal(ours, ref)
    ref_now = _torch_bits((tx * torch.from_numpy(r)).to(torch.bfloat16))
    assert np.array_equal(ss.norm_bf16(x, r, None), ref_now)


def test_inv_rms_matches_exact_rational():
    rng = np.random.default_rng(14)
    for D, eps, mag in [(4, 1e-6, 1.0), (8, 0.5, 1.0), (64, 1e-6, 1e-3), (128, 1e-5, 30.0), (96, 0.0, 1.0)]:
        x = _bits((rng.standard_normal((12, D)) * mag).astype(np.float32))
        r, amb, lo, hi = ss.inv_rms(x, eps)
        for i in range(x.shape[0]):
            exact = ss.inv_rms_exact(x[i], eps)
            if amb[i]:
                assert exact in (lo[i], hi[i])
            else:
                assert r[i] == exact, (D, eps, i)


def test_inv_rms_closed_forms():
    # constant row c: r = 1 / sqrt(c^2 + eps)
    x = _bits(np.full((1, 256), 2.0, dtype=np.float32))
    assert ss.inv_rms(x, 0.0)[0][0] == np.float32(0.5)
    assert ss.inv_rms(x, 12.0)[0][0] == np.float32(0.25)
    # a zero row with eps = 1/4 gives r = 2
    z = np.zeros((1, 16), dtype=np.uint16)
    assert ss.inv_rms(z, 0.25)[0][0] == np.float32(2.0)


def test_ambiguity_detection():
    """A value placed on an fp32 midpoint is flagged, and its two candidates
    are the neighbouring fp32 values."""
    mid = np.float64(np.float32(1.0)) + 2.0 ** -24          # halfway between 1 and 1 + 2^-23
    lo, hi = ss._f32_neighbours(np.array([mid]), ss.AMBIGUITY_REL)
    assert lo[0] == np.float32(1.0) and hi[0] == np.nextafter(np.float32(1.0), np.float32(2.0))
    lo, hi = ss._f32_neighbours(np.array([1.25]), ss.AMBIGUITY_REL)
    assert lo[0] == hi[0] == np.float32(1.25)


def test_norm_agrees_with_fp64_rmsnorm():
    """With no modulation (scale 0, shift 0) the step is the bf16 rounding of
    RMSNorm; the attention prologue's fp64 RMSNorm, rounded, agrees to within
    one bf16 ulp (two roundings against one)."""
    rng = np.random.default_rng(15)
    D = 128
    x = _bits(rng.standard_normal((1, 50, D)).astype(np.float32))
    w = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    zero = np.zeros((1, 1, D), dtype=np.uint16)
    y = ss.rmsnorm_scale_shift(x, w, 1e-6, zero, zero, None)
    ref = oracle.rms_norm(oracle.bf16_bits_to_f64(x), w.astype(np.float64), 1e-6)
    ref_bits = ss.bf16_rne(ref.astype(np.float32))
    diff = np.abs(y.astype(np.int32) - ref_bits.astype(np.int32))
    assert diff.max() <= 1 and (diff == 0).mean() > 0.99


def test_invariants():
    rng = np.random.default_rng(16)
    B, S, D, M = 2, 30, 64, 5
    x = _bits(rng.standard_normal((B, S, D)).astype(np.float32))
    scale = _bits((0.3 * rng.standard_normal((B, M, D))).astype(np.float32))
    shift = _bits((0.3 * rng.standard_normal((B, M, D))).astype(np.float32))
    index = rng.integers(0, M, (B, S)).astype(np.int32)
    y = ss.rmsnorm_scale_shift(x, None, 1e-6, scale, shift, index)
    # identity modulation returns the norm
    zero = np.zeros((B, M, D), dtype=np.uint16)
    r = ss.inv_rms(x, 1e-6)[0]
    n = ss.norm_bf16(x, r[..., None])
    assert np.array_equal(ss.rmsnorm_scale_shift(x, None, 1e-6, zero, zero, index), n)
    # scale = -1 zeroes the norm: the output is the shift
    m1 = np.full((B, M, D), 0xBF80, dtype=np.uint16)
    yk = ss.rmsnorm_scale_shift(x, None, 1e-6, m1, shift, index)
    assert np.array_equal(ss.bf16_to_f32(yk), ss.bf16_to_f32(ss.gather_rows(shift, index, M)))
    # permuting the modulation rows and remapping the index changes nothing
    perm = rng.permutation(M)
    inv = np.argsort(perm)
    yp = ss.rmsnorm_scale_shift(x, None, 1e-6, scale[:, perm], shift[:, perm], inv[index].astype(np.int32))
    assert np.array_equal(yp, y)
    # out-of-range indices clamp to the first / last row
    bad = index.copy()
    bad[0, :5] = -7
    bad[1, :5] = M + 9
    fixed = index.copy()
    fixed[0, :5] = 0
    fixed[1, :5] = M - 1
    assert np.array_equal(ss.rmsnorm_scale_shift(x, None, 1e-6, scale, shift, bad),
                          ss.rmsnorm_scale_shift(x, None, 1e-6, scale, shift, fixed))
    # no index: every token takes row 0
    assert np.array_equal(ss.rmsnorm_scale_shift(x, None, 1e-6, scale, shift, None),
                          ss.rmsnorm_scale_shift(x, None, 1e-6, scale, shift, np.zeros((B, S), np.int32)))
    # rows are independent: the result of one token does not depend on others
    y1 = ss.rmsnorm_scale_shift(x[:, 3:4], None, 1e-6, scale, shift, index[:, 3:4])
    assert np.array_equal(y1, y[:, 3:4])


def test_plausible_mistakes_fail_the_hand_example():
    """Each single-step mistake changes the hand example's output."""
    g = json.load(open(os.path.join(GOLDEN, "scale_shift_hand.json")))
    x = _bits(g["x"])[None]
    scale = _bits(g["scale"])[None]
    shift = _bits(g["shift"])[None]
    index = np.clip(np.array([g["index"]]), 0, 1)
    w = np.array(g["w"], dtype=np.float32)
    want = np.array(g["y"], dtype=np.float32)
    xf = ss.bf16_to_f32(x).astype(np.float64)
    sc = ss.bf16_to_f32(ss.gather_rows(scale, index, 2))
    sh = ss.bf16_to_f32(ss.gather_rows(shift, index, 2))
    ms = (xf * xf).mean(-1, keepdims=True)
    variants = {
        "eps outside root": 1 / np.sqrt(ms) + g["eps"],
        "sum not mean": 1 / np.sqrt((xf * xf).sum(-1, keepdims=True) + g["eps"]),
    }
    for name, r in variants.items():
        y = ss.modulate(ss.norm_bf16(x, r.astype(np.float32), w), ss.bf16_rne(sc), ss.bf16_rne(sh))
        assert not np.array_equal(ss.bf16_to_f32(y)[0], want), name
    r = np.float32(0.5)
    n_f32 = ss.bf16_to_f32(x) * r * w                           # no rounding of n
    fp32_chain = (n_f32 * (1 + sc) + sh).astype(np.float32)     # no rounding anywhere
    assert not np.array_equal(ss.bf16_to_f32(ss.bf16_rne(fp32_chain))[0], want)
    n = ss.bf16_to_f32(ss.norm_bf16(x, r, w))
    no_u = ss.bf16_rne(n * ss.bf16_to_f32(ss.bf16_rne(1 + sc)) + sh)   # u not rounded
    assert not np.array_equal(ss.bf16_to_f32(no_u)[0], want)
    no_t = ss.bf16_rne(ss.bf16_to_f32(ss.bf16_rne(n * (1 + sc))) + sh)  # t not rounded
    assert not np.array_equal(ss.bf16_to_f32(no_t)[0], want)
    t = ss.bf16_to_f32(ss.bf16_rne(1 + sc))
    no_n = ss.bf16_rne(ss.bf16_to_f32(ss.bf16_rne(n_f32 * t)) + sh)   # n not rounded
    assert not np.array_equal(ss.bf16_to_f32(no_n)[0], want)
