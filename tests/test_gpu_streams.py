"""Calls on several streams at once, and from several host threads at once.
The library keeps no per-call state outside the caller's buffers (its only
globals are per-device caches of the CU count and of the frame window's tile
order, behind atomics and a lock), so launches that overlap on the GPU, or
whose host calls overlap, give the same bits as the same launches one after
another on one stream. Every stream is created at the default priority."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import workloads
from gpu_util import DevInputs, assert_all_written, say, to_dev, to_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# name, B, Sq, Sk, H, launch options: one case per kernel family
CASES = [
    ("resident keys", 2, 3000, 512, 4, dict(kv_valid=300)),
    ("ring split and merge", 1, 3000, 2000, 3, dict(q_valid=2900, kv_valid=1900)),
    ("causal", 2, 1500, 1500, 2, dict(causal=True)),
    ("window with gate", 1, 2000, 2000, 2, dict(window=(200, 3, 1, 1), gate=True)),
]


@pytest.fixture(scope="module")
def h3():
    from video_dit_dense_amd import h3attn
    h3attn.load_library()
    return h3attn


@pytest.fixture(scope="module")
def prepared(h3):
    out = []
    for i, (name, B, Sq, Sk, H, opts) in enumerate(CASES):
        d = DevInputs(workloads.make_inputs(B, Sq, Sk, H, seed=500 + i))
        cos, sin = h3.rope_tables(max(Sq, Sk))
        gate = to_dev(workloads.make_gate(B, Sq, H, seed=600 + i)) if opts.get("gate") else None
        out.append((name, d, cos, sin, gate, opts))
    return out


def launch(h3, case, o):
    name, d, cos, sin, gate, opts = case
    h3.forward(d.q, d.k, d.v, d.w_q, d.w_k, 1e-6, cos, sin, q_valid=opts.get("q_valid"),
               kv_valid=opts.get("kv_valid"), out=o, causal=opts.get("causal", False),
               window=opts.get("window"), gate=gate)


def sequential(h3, prepared):
    refs = []
    for case in prepared:
        o = torch.full_like(case[1].q, float("nan"))
        launch(h3, case, o)
        refs.append(o)
    torch.cuda.synchronize()
    return [to_host(o) for o in refs]


def test_overlapping_streams(h3, prepared):
    say("streams:", [c[0] for c in prepared])
    refs = sequential(h3, prepared)
    streams = [torch.cuda.Stream() for _ in prepared]
    for rep in range(2):
        outs = [torch.full_like(c[1].q, float("nan")) for c in prepared]
        torch.cuda.synchronize()
        for case, o, s in zip(prepared, outs, streams):
            with torch.cuda.stream(s):
                launch(h3, case, o)
        torch.cuda.synchronize()
        for case, o, ref in zip(prepared, outs, refs):
            got = to_host(o)
            assert_all_written(got, case[0])
            assert np.array_equal(got, ref), f"{case[0]}: stream launch {rep} differs from the sequential one"


def test_overlapping_host_threads(h3, prepared):
    refs = sequential(h3, prepared)
    outs = [torch.full_like(c[1].q, float("nan")) for c in prepared]
    torch.cuda.synchronize()

    def run(i):
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            for _ in range(3):
                launch(h3, prepared[i], outs[i])
        s.synchronize()

    with ThreadPoolExecutor(len(prepared)) as ex:
        list(ex.map(run, range(len(prepared))))
    torch.cuda.synchronize()
    for case, o, ref in zip(prepared, outs, refs):
        got = to_host(o)
        assert_all_written(got, case[0])
        assert np.array_equal(got, ref), f"{case[0]}: threaded launches differ from the sequential one"
