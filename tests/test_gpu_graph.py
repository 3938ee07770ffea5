"""HIP graph capture: the entry points enqueue kernels on the caller's stream
and nothing else (no allocation, no memset, no host synchronisation), so a
caller can capture an attention step once and replay it. Each case captures
its calls with static inputs and outputs, then replays the graph three times.
Before each replay, eager work writes new seeded inputs into the static
buffers and NaN into the outputs, and the host synchronises. Every replay
must equal, bit for bit, the same calls run eagerly into separate outputs and
workspaces (the kernels are deterministic)."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import DevInputs, assert_all_written, say, to_dev, to_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

REPLAYS = 3

# name, B, Sq, Sk, H, Hkv, D, launch options
CASES = [
    ("ring split and merge", 1, 3000, 2000, 3, 3, 128, dict(q_valid=2900, kv_valid=1900)),
    ("resident keys", 2, 1000, 512, 3, 3, 128, dict(kv_valid=300)),
    ("causal, grouped heads", 2, 1500, 1500, 4, 2, 128, dict(causal=True)),
    ("per-item lengths", 2, 1200, 1100, 2, 2, 128, dict(lengths=[[1200, 1100], [700, 900]])),
    ("window with gate", 1, 1000, 1000, 2, 2, 128, dict(window=(100, 3, 1, 1), gate=True)),
    ("head dim 64", 1, 2000, 1000, 2, 2, 64, dict()),
    ("head dim 256", 1, 700, 900, 2, 2, 256, dict()),
]


@pytest.fixture(scope="module")
def h3():
    from video_dit_dense_amd import h3attn
    h3attn.load_library()
    return h3attn


def bits(t: torch.Tensor) -> np.ndarray:
    return to_host(t).ravel()


class Static:
    """The buffers a captured forward reads and writes: inputs, weights,
    tables, per-item lengths, gate, output and workspace."""

    def __init__(self, h3, B, Sq, Sk, H, Hkv, D, opts):
        self.h3, self.D, self.opts = h3, D, opts
        self.q = torch.empty(B, Sq, H, D, dtype=torch.bfloat16, device="cuda:0")
        self.k = torch.empty(B, Sk, Hkv, D, dtype=torch.bfloat16, device="cuda:0")
        self.v = torch.empty_like(self.k)
        self.w_q = torch.empty(D, dtype=torch.float32, device="cuda:0")
        self.w_k = torch.empty_like(self.w_q)
        self.cos = self.sin = None
        if D == 128:
            self.cos, self.sin = h3.rope_tables(max(Sq, Sk))
        lengths = opts.get("lengths")
        self.lengths = None if lengths is None else torch.tensor(lengths, dtype=torch.int32, device="cuda:0")
        self.gate = torch.empty(B, Sq, H, dtype=torch.bfloat16, device="cuda:0") if opts.get("gate") else None
        self.o = torch.empty_like(self.q)
        n = max(h3.workspace_bytes(B, Sq, Sk, H),
                h3.forward_ex_workspace_bytes(B, Sq, Sk, H, Hkv, causal=opts.get("causal", False),
                                              per_item_lengths=lengths is not None,
                                              window=bool(opts.get("window")), head_dim=D))
        self.ws = torch.empty(n, dtype=torch.uint8, device="cuda:0")

    def fill(self, seed, B, Sq, Sk, H, Hkv):
        """New seeded inputs into the static buffers (eager copies)."""
        inp = workloads.make_inputs(B, Sq, Sk, H, seed=seed, Hkv=Hkv, D=self.D)
        d = DevInputs(inp)
        self.q.copy_(d.q)
        self.k.copy_(d.k)
        self.v.copy_(d.v)
        self.w_q.copy_(d.w_q)
        self.w_k.copy_(d.w_k)
        if self.gate is not None:
            self.gate.copy_(to_dev(workloads.make_gate(B, Sq, H, seed=seed + 1)))

    def launch(self, out, ws):
        norm_rope = self.D == 128
        o = self.opts
        self.h3.forward(self.q, self.k, self.v, self.w_q if norm_rope else None, self.w_k if norm_rope else None,
                        1e-6, self.cos, self.sin, q_valid=o.get("q_valid"), kv_valid=o.get("kv_valid"),
                        scale=self.D ** -0.5, out=out, workspace=ws, causal=o.get("causal", False),
                        valid_lengths=self.lengths, window=o.get("window"), gate=self.gate)


@pytest.mark.parametrize("name,B,Sq,Sk,H,Hkv,D,opts", CASES, ids=[c[0] for c in CASES])
def test_forward_graph_replays(h3, name, B, Sq, Sk, H, Hkv, D, opts):
    say("graph replays:", name)
    st = Static(h3, B, Sq, Sk, H, Hkv, D, opts)
    st.fill(300, B, Sq, Sk, H, Hkv)
    st.launch(st.o, st.ws)                       # eager warm-up before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.launch(st.o, st.ws)
    ref_o = torch.empty_like(st.o)
    ref_ws = torch.empty_like(st.ws)
    for r in range(REPLAYS):
        st.fill(301 + r, B, Sq, Sk, H, Hkv)
        st.o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = bits(st.o)
        st.launch(ref_o, ref_ws)
        torch.cuda.synchronize()
        want = bits(ref_o)
        assert_all_written(got, f"{name}, replay {r}")   # tail rows are written as zeros
        assert np.array_equal(got, want), f"{name}: replay {r} differs from the eager call"


def test_step_graph_replays(h3):
    """One captured step over the other entry points: the fused RMSNorm +
    scale/shift, the Q/K/V pack into destination-major send buffers, and the
    attention step with the library's static workspace (noalloc)."""
    B, S, H, M, D = 1, 1500, 4, 3, 128
    rng = np.random.default_rng(17)
    x = torch.empty(B, S, 2 * D, dtype=torch.bfloat16, device="cuda:0")
    scale = torch.empty(B, M, 2 * D, dtype=torch.bfloat16, device="cuda:0")
    shift = torch.empty_like(scale)
    index = torch.from_numpy(rng.integers(0, M, size=(B, S), dtype=np.int32)).to("cuda:0")
    y = torch.empty_like(x)
    q = torch.empty(B, S, H, D, dtype=torch.bfloat16, device="cuda:0")
    k, v = torch.empty_like(q), torch.empty_like(q)
    w_q = torch.empty(D, dtype=torch.float32, device="cuda:0")
    w_k = torch.empty_like(w_q)
    cos, sin = h3.rope_tables(S)
    P = 2
    send = tuple(torch.empty(P, B, S, H // P, D, dtype=torch.bfloat16, device="cuda:0") for _ in range(3))
    o = torch.empty_like(q)

    def fill(seed):
        inp = workloads.make_inputs(B, S, S, H, seed=seed)
        d = DevInputs(inp)
        q.copy_(d.q)
        k.copy_(d.k)
        v.copy_(d.v)
        w_q.copy_(d.w_q)
        w_k.copy_(d.w_k)
        r = np.random.default_rng(seed)
        for t in (x, scale, shift):
            t.copy_(torch.from_numpy(r.standard_normal(t.shape, dtype=np.float32)).to("cuda:0").bfloat16())

    def step(y_out, send_out, o_out, noalloc):
        h3.rmsnorm_scale_shift(x, scale, shift, index, None, 1e-6, out=y_out)
        h3.qkv_pack(q, k, v, P, 0, w_q, w_k, 1e-6, cos, sin, out=send_out)
        if noalloc:
            h3.forward_noalloc(q, k, v, o_out, w_q, w_k, 1e-6, cos, sin, kv_valid=S - 100)
        else:
            h3.forward(q, k, v, w_q, w_k, 1e-6, cos, sin, kv_valid=S - 100, out=o_out)

    fill(400)
    step(y, send, o, True)                       # eager warm-up (and the static workspace's set-up)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(y, send, o, True)
    ref_y = torch.empty_like(y)
    ref_send = tuple(torch.empty_like(t) for t in send)
    ref_o = torch.empty_like(o)
    for r in range(REPLAYS):
        fill(401 + r)
        for t in (y, o, *send):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [bits(t) for t in (y, *send, o)]
        step(ref_y, ref_send, ref_o, False)
        torch.cuda.synchronize()
        want = [bits(t) for t in (ref_y, *ref_send, ref_o)]
        for label, a, b in zip(("scale/shift", "q_send", "k_send", "v_send", "attention"), got, want):
            assert_all_written(a, f"{label}, replay {r}")
            assert np.array_equal(a, b), f"{label}: replay {r} differs from the eager call"
