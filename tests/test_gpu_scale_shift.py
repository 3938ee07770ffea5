"""GPU parity of the fused RMSNorm + indexed AdaLN scale/shift step
(TeleFuser PR #37, "2.5 Fuse RMSNorm with indexed AdaLN modulation") against
the oracle's bf16 chain on the same seeded inputs, through the C-ABI.

Bar: bit-exact on every element. The one decision the two sides may take
differently is the fp32 rounding of a row's factor r when 1/sqrt(ms + eps)
lies within 2^-44 of a midpoint between two floats (the GPU sums the
squares in another order); in such a row the GPU output must equal the chain
evaluated with one of the two candidates. NaN outputs compare as NaN."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import f32_dev, say, to_dev, to_host
from oracle import scale_shift as ss

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def h3():
    from video_dit_dense_amd import h3attn
    h3attn.load_library()
    return h3attn


def dev_inputs(inp):
    idx = None if inp.index is None else torch.from_numpy(np.ascontiguousarray(inp.index)).to("cuda:0")
    w = None if inp.w is None else f32_dev(inp.w)
    return to_dev(inp.x), to_dev(inp.scale), to_dev(inp.shift), idx, w


def run(h3, inp, eps, out_in_place=False):
    x, sc, sh, idx, w = dev_inputs(inp)
    y = h3.rmsnorm_scale_shift(x, sc, sh, idx, w, eps, out=x if out_in_place else None)
    torch.cuda.synchronize()
    return to_host(y)


def same(a, b):
    """Equal bits, or both NaN."""
    fa, fb = ss.bf16_to_f32(a), ss.bf16_to_f32(b)
    return (a == b) | (np.isnan(fa) & np.isnan(fb))


def check(got, inp, eps, label, row_chunk=1024):
    """Compares every element, `row_chunk` rows of the oracle at a time."""
    B, S, D = inp.x.shape
    n_amb = n_alt = 0
    for b in range(B):
        for s0 in range(0, S, row_chunk):
            s1 = min(S, s0 + row_chunk)
            xs = inp.x[b:b + 1, s0:s1]
            idx = None if inp.index is None else inp.index[b:b + 1, s0:s1]
            sc, sh = inp.scale[b:b + 1], inp.shift[b:b + 1]
            r, amb, lo, hi = ss.inv_rms(xs, eps)
            want = ss.rmsnorm_scale_shift(xs, inp.w, eps, sc, sh, idx, r=r)
            ok = same(got[b:b + 1, s0:s1], want).all(axis=-1)
            n_amb += int(amb.sum())
            for i in np.argwhere(~ok):
                row = tuple(i)
                assert amb[row], f"{label}: row b={b} s={s0 + row[1]} differs and is not ambiguous"
                other = np.where(r[row] == lo[row], hi[row], lo[row])
                r2 = r.copy()
                r2[row] = other
                alt = ss.rmsnorm_scale_shift(xs, inp.w, eps, sc, sh, idx, r=r2)
                assert same(got[b:b + 1, s0:s1][row], alt[row]).all(), f"{label}: row {row} matches neither"
                n_alt += 1
    say(f"{label}: bit-exact over {B}x{S}x{D}; ambiguous rows {n_amb}, of which took the other rounding {n_alt}")


@pytest.mark.parametrize("name", ["ss_tiny", "ss_mid"])
def test_workloads(h3, name):
    wl = workloads.SCALE_SHIFT_WORKLOADS[name]
    say("scale_shift", name)
    inp = workloads.make_scale_shift_inputs(wl)
    check(run(h3, inp, wl.eps), inp, wl.eps, name)


def test_full_shard(h3):
    """The shape the benchmark times: one GPU's 13056-row share at width 6144,
    every element compared, and four launches bitwise equal (a store whose
    data registers were rewritten too early once corrupted a few rows per
    launch, differently each time)."""
    wl = workloads.SCALE_SHIFT_WORKLOADS["ss_shard"]
    say("scale_shift ss_shard")
    inp = workloads.make_scale_shift_inputs(wl)
    x, sc, sh, idx, w = dev_inputs(inp)
    outs = []
    for _ in range(4):
        outs.append(to_host(h3.rmsnorm_scale_shift(x, sc, sh, idx, w, wl.eps)))
        torch.cuda.synchronize()
    for k in range(1, 4):
        assert np.array_equal(outs[k], outs[0]), f"launch {k} differs from launch 0"
    check(outs[0], inp, wl.eps, "ss_shard")


# Every register-blocking instantiation (chunks of 8 channels per lane: 1, 2,
# 4, 8, 12, 16, 24, 32) and ragged last chunks.
@pytest.mark.parametrize("D", [8, 56, 520, 1024, 2048, 4096, 6144, 6152, 8192, 12288, 16384])
@pytest.mark.parametrize("weight,index", [(False, "random"), (True, "frames"), (True, "none")])
def test_widths(h3, D, weight, index):
    wl = workloads.ScaleShiftWorkload("w", 2, 37, D, 1 if index == "none" else 3, 40 + D % 97,
                                      weight=weight, index=index)
    say("scale_shift width", D, weight, index)
    inp = workloads.make_scale_shift_inputs(wl)
    check(run(h3, inp, 1e-6), inp, 1e-6, f"D={D} weight={weight} index={index}")


@pytest.mark.parametrize("x_sigma,eps", [(1000.0, 1e-6), (1e-20, 1e-6), (1e-3, 0.0), (3.0, 0.5)])
def test_magnitudes(h3, x_sigma, eps):
    """Large and tiny rows (eps dominating), eps = 0 and a large eps."""
    wl = workloads.ScaleShiftWorkload("m", 1, 300, 768, 4, 50, weight=True, index="random", eps=eps)
    say("scale_shift magnitudes", x_sigma, eps)
    inp = workloads.make_scale_shift_inputs(wl, x_sigma=x_sigma)
    check(run(h3, inp, eps), inp, eps, f"x_sigma={x_sigma} eps={eps}")


def test_in_place_and_repeat(h3):
    wl = workloads.SCALE_SHIFT_WORKLOADS["ss_tiny"]
    say("scale_shift in place")
    inp = workloads.make_scale_shift_inputs(wl, seed=60)
    a = run(h3, inp, wl.eps)
    b = run(h3, inp, wl.eps)
    c = run(h3, inp, wl.eps, out_in_place=True)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_index_clamping_and_default(h3):
    wl = workloads.ScaleShiftWorkload("c", 2, 64, 256, 5, 61, index="random")
    say("scale_shift clamping")
    inp = workloads.make_scale_shift_inputs(wl)
    bad = inp.index.copy()
    bad[0, :10] = -3
    bad[1, :10] = 5 + 7
    bad[1, 10] = np.iinfo(np.int32).max
    bad[0, 10] = np.iinfo(np.int32).min
    clamped = np.clip(bad, 0, 4).astype(np.int32)
    got_bad = run(h3, workloads.ScaleShiftInputs(inp.x, inp.scale, inp.shift, bad, None), 1e-6)
    got_ok = run(h3, workloads.ScaleShiftInputs(inp.x, inp.scale, inp.shift, clamped, None), 1e-6)
    assert np.array_equal(got_bad, got_ok)
    none = workloads.ScaleShiftInputs(inp.x, inp.scale, inp.shift, None, None)
    zeros = workloads.ScaleShiftInputs(inp.x, inp.scale, inp.shift, np.zeros((2, 64), np.int32), None)
    assert np.array_equal(run(h3, none, 1e-6), run(h3, zeros, 1e-6))
    check(got_bad, workloads.ScaleShiftInputs(inp.x, inp.scale, inp.shift, bad, None), 1e-6, "clamped")


def test_special_rows(h3):
    """A zero row (eps > 0: the output is the shift; eps = 0: NaN), a row
    with an infinity (r = 0: the shift, NaN at that channel), a NaN row."""
    wl = workloads.ScaleShiftWorkload("z", 1, 8, 64, 2, 62, index="random")
    inp = workloads.make_scale_shift_inputs(wl)
    x = inp.x.copy()
    x[0, 0] = 0
    x[0, 1] = 0x8000                 # -0.0 everywhere
    x[0, 2, 5] = 0x7F80              # +inf
    x[0, 3, 9] = 0x7FC0              # NaN
    spec = workloads.ScaleShiftInputs(x, inp.scale, inp.shift, inp.index, None)
    for eps in (1e-6, 0.0):
        say("scale_shift special rows, eps", eps)
        with np.errstate(divide="ignore", invalid="ignore"):
            check(run(h3, spec, eps), spec, eps, f"special eps={eps}")


def test_single_row_and_single_modulation_row(h3):
    wl = workloads.ScaleShiftWorkload("one", 1, 1, 6144, 1, 63, weight=True, index="none")
    say("scale_shift one row")
    inp = workloads.make_scale_shift_inputs(wl)
    check(run(h3, inp, 1e-6), inp, 1e-6, "one row")
