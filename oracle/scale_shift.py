"""Oracle of the fused RMSNorm + indexed AdaLN scale/shift step.

TEST INFRASTRUCTURE, like the rest of this package: only the tests, the smoke
check and the CPU-baseline leg of the benchmark use it, and it shares no code
with the HIP library.

What the step computes (TeleFuser PR #37, "2.5 Fuse RMSNorm with indexed
AdaLN modulation"): a DiT block's RMSNorm of the hidden states followed by
the AdaLN modulation x * (1 + scale) + shift, where each token takes its
scale/shift row by an index (one row per frame, say), with the bf16 rounding
boundaries of the unfused chain kept, so that fused and unfused results are
equal bit for bit.

The pages name the chain but print no formula, so the chain is read as the
plain bf16 PyTorch sequence, every elementwise operation computed in fp32 and
its result rounded to bf16 (round to nearest, ties to even):

  r  = fp32(1 / sqrt(mean_c x_c^2 + eps))   per row, correctly rounded
  n  = bf16(fp32(x * r) [* w])              the norm, stored in bf16
  t  = bf16(1 + scale[idx])                 bf16 tensor arithmetic
  u  = bf16(n * t)
  y  = bf16(u + shift[idx])

x, scale and shift are bf16; w (optional, absent in the usual DiT block
norm) is fp32; mean_c x_c^2 is the exact mean over the row's D channels; idx
is clamped to [0, M). Each fp32 step here uses NumPy float32 arithmetic,
which is IEEE round-to-nearest-even like the GPU's.

The per-row factor r is the one place where the GPU sums in a different
order: it accumulates the squares in fp64, so its r differs from the exact
one only when 1/sqrt(ms + eps) lies within ~2^-44 (relative) of a point
halfway between two fp32 values. `inv_rms` reports those rows and both fp32
candidates, and the parity tests accept either there.

Pinned in tests/test_oracle_pins.py: the bf16 rounding against torch's CPU
conversion, steps t, u, y against torch's CPU bf16 tensor arithmetic, r
against exact rational arithmetic, a hand-worked row (tests/golden), and
invariants (identity modulation, scale = -1, index permutation).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

# Relative distance from an fp32 rounding midpoint under which the GPU's
# fp64 accumulation may round r either way (its error is below 2^-48).
AMBIGUITY_REL = 2.0 ** -44


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns to their exact float32 values (bf16 is the upper
    half of an IEEE float32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_rne(x) -> np.ndarray:
    """float32 values to bf16 bit patterns, round to nearest, ties to even.
    A value past the largest bf16 rounds to infinity, as IEEE rounding does;
    NaN maps to the quiet NaN 0x7FC0."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    out = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def _f32_neighbours(r64: np.ndarray, rel: float):
    lo = (r64 * (1.0 - rel)).astype(np.float32)
    hi = (r64 * (1.0 + rel)).astype(np.float32)
    return lo, hi


def inv_rms(x_bits, eps: float):
    """Per-row r = fp32(1 / sqrt(mean_c x_c^2 + eps)) over the last axis.

    Returns (r, ambiguous, r_lo, r_hi): r is float32, computed from the fp64
    mean of squares (the squares of bf16 values are exact in fp64 and their
    sum is good to ~1e-16); `ambiguous` marks rows whose value is within
    AMBIGUITY_REL of an fp32 rounding midpoint, where r_lo and r_hi are the
    two fp32 values either rounding gives."""
    x = bf16_to_f32(x_bits).astype(np.float64)
    ms = np.mean(x * x, axis=-1)
    r64 = 1.0 / np.sqrt(ms + float(np.float32(eps)))
    r = r64.astype(np.float32)
    lo, hi = _f32_neighbours(r64, AMBIGUITY_REL)
    return r, (lo != hi) & np.isfinite(r64), lo, hi


def inv_rms_exact(row_bits, eps: float) -> np.float32:
    """r of one row in exact rational arithmetic: the mean of squares and eps
    as fractions, the square root bracketed by integer square roots at 2^-80
    resolution, then rounded to the nearest float32. For pinning inv_rms on
    small rows."""
    vals = [Fraction(float(v)) for v in bf16_to_f32(row_bits)]
    ms = sum(v * v for v in vals) / len(vals) + Fraction(float(np.float32(eps)))
    # 1/sqrt(ms) * 2^80 = sqrt(2^160 / ms) lies in [lo, lo + 1].
    lo = math.isqrt(((Fraction(2) ** 160) / ms).__floor__())
    a = _round_to_f32(Fraction(lo, 2 ** 80))
    b = _round_to_f32(Fraction(lo + 1, 2 ** 80))
    if a != b:
        raise ArithmeticError("row lies on an fp32 rounding midpoint to 2^-80")
    return a


def _round_to_f32(q: Fraction) -> np.float32:
    """A positive rational in float32's normal range, rounded to the nearest
    float32 (ties to even) with integer arithmetic only."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    scaled = q * Fraction(2) ** (23 - e)          # in [2^23, 2^24)
    m = scaled.__floor__()
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return np.float32(m * 2.0 ** (e - 23))


def gather_rows(mod_bits, index, M: int) -> np.ndarray:
    """mod[b, clamp(index[b, s], 0, M-1), :] for every token, shape [B, S, D].
    index None means row 0 for every token."""
    mod = np.asarray(mod_bits, dtype=np.uint16)
    B = mod.shape[0]
    if index is None:
        return np.broadcast_to(mod[:, :1, :], (B, 1, mod.shape[2]))
    idx = np.clip(np.asarray(index, dtype=np.int64), 0, M - 1)
    return mod[np.arange(B)[:, None], idx, :]


def modulate(n_bits, scale_bits, shift_bits) -> np.ndarray:
    """y = bf16(bf16(n * bf16(1 + scale)) + shift), each operation in fp32.
    Arguments broadcast against each other (bf16 bit patterns)."""
    one = np.float32(1.0)
    t = bf16_rne(one + bf16_to_f32(scale_bits))
    u = bf16_rne(bf16_to_f32(n_bits) * bf16_to_f32(t))
    return bf16_rne(bf16_to_f32(u) + bf16_to_f32(shift_bits))


def norm_bf16(x_bits, r, w=None) -> np.ndarray:
    """n = bf16(fp32(x * r) [* w]) with r per row (float32, shape [..., 1]
    broadcast) and w an optional fp32 [D] weight."""
    n = bf16_to_f32(x_bits) * np.asarray(r, dtype=np.float32)
    if w is not None:
        n = n * np.asarray(w, dtype=np.float32)
    return bf16_rne(n)


def rmsnorm_scale_shift(x_bits, w, eps: float, scale_bits, shift_bits, index=None, r=None):
    """The whole step on x [B, S, D] (bf16 bits) with scale / shift [B, M, D]
    (bf16 bits), index [B, S] (int) or None, w fp32 [D] or None. Returns the
    output bf16 bits [B, S, D]. `r` overrides the per-row factor (float32
    [B, S]) so that a test can evaluate the other candidate of an ambiguous
    row."""
    x = np.asarray(x_bits, dtype=np.uint16)
    M = np.asarray(scale_bits).shape[1]
    if r is None:
        r = inv_rms(x, eps)[0]
    n = norm_bf16(x, np.asarray(r, dtype=np.float32)[..., None], w)
    return modulate(n, gather_rows(scale_bits, index, M), gather_rows(shift_bits, index, M))
