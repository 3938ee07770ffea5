"""Host-side tests of the C-ABI library: it loads, exports every entry point
include/h3attn.h declares, and rejects bad arguments before touching the GPU.
No test here launches a kernel: every fake pointer below sits in a call that
fails validation (or, with no GPU present, the device gate)."""
import ctypes
import os
import re

import pytest
import torch

from video_dit_dense_amd import h3attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3attn.h")

OK, NULLP, SHAPE, ALIGN, ALIAS, VALUE, WS, DEVICE, HIP = range(9)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(h3attn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return h3attn.load_library()


def P(x):
    return ctypes.c_void_p(x)


A = 1 << 20   # fake, 16-byte aligned, never dereferenced (validation fails first)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names == sorted(h3attn.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(9):
        msg = h3attn.status_string(s)
        assert isinstance(msg, str) and msg
    assert "unknown" in h3attn.status_string(99)
    assert h3attn.status_string(DEVICE).find("gfx950") >= 0


def test_workspace_bytes(lib):
    # q rows padded to whole query blocks of every tiling a head-dim-128
    # launch may take (256 and 384 rows: the larger of the two round-ups),
    # k and v^T rows to 256; 256 bytes per row (bf16, 128 channels). Then
    # partial records for split tiles: 2 per split block, blocks =
    # min(256, tiles * steps / 16) counted with the smaller, 256-row tiles
    # and 32-key steps; a record is (96 + 6) x 512 floats, the larger
    # tiling's (each wave's 48 rows as three 16-row tiles: 48 x 128
    # accumulators over 64 lanes, then three row offsets and three partial
    # sums per lane). Then the key-norm maxima: one fp32 per 4096 padded keys
    # of each (b, head), padded to 256 bytes.
    rec = (96 + 6) * 512 * 4
    kn = lambda n: (n * 4 + 255) // 256 * 256   # noqa: E731
    # 104448 rows are whole blocks of both 256 and 384
    assert lib.h3attn_forward_workspace_bytes(1, 104448, 104448, 6) == 6 * 104448 * 256 * 3 + 2 * 256 * rec + kn(6 * 26)
    # 1000 query rows: 1024 by 256, 1152 by 384; 6 heads x 4 tiles x 10 steps = 240 steps -> 15 blocks
    assert lib.h3attn_forward_workspace_bytes(2, 1000, 300, 3) == 6 * (1152 + 2 * 512) * 256 + 2 * 15 * rec + kn(6)
    # 1 tile x 1 step: no split blocks; one query row pads to 384
    assert lib.h3attn_forward_workspace_bytes(1, 1, 1, 1) == (384 + 2 * 256) * 256 + kn(1)
    assert lib.h3attn_forward_workspace_bytes(0, 1, 1, 1) == 0
    assert lib.h3attn_forward_workspace_bytes(1, -5, 1, 1) == 0


def prologue(lib, q=A, k=2 * A, qo=3 * A, ko=4 * A, B=1, Sq=8, Sk=8, H=2, D=128,
             wq=5 * A, wk=5 * A + 512, eps=1e-6, rc=6 * A, rs=7 * A, rows=8):
    return lib.h3attn_qk_prologue(P(q), P(k), P(qo), P(ko), B, Sq, Sk, H, D, P(wq), P(wk), eps,
                                  P(rc), P(rs), rows, None)


def test_prologue_validation(lib):
    assert prologue(lib, q=0) == NULLP
    assert prologue(lib, ko=0) == NULLP
    assert prologue(lib, wk=0) == NULLP            # only one weight
    assert prologue(lib, rs=0) == NULLP            # only one table
    assert prologue(lib, D=64) == SHAPE
    assert prologue(lib, H=0) == SHAPE
    assert prologue(lib, Sq=0) == SHAPE
    assert prologue(lib, rows=7) == SHAPE          # tables shorter than S
    assert prologue(lib, eps=float("nan")) == VALUE
    assert prologue(lib, eps=-1.0) == VALUE
    assert prologue(lib, q=A + 2) == ALIGN
    assert prologue(lib, rc=6 * A + 4) == ALIGN
    assert prologue(lib, qo=2 * A) == ALIAS        # q_out on top of k
    assert prologue(lib, qo=A + 256) == ALIAS      # partial overlap with q
    assert prologue(lib, qo=3 * A, ko=3 * A + 256) == ALIAS
    assert prologue(lib, rs=6 * A + 16) == ALIAS   # cos and sin overlap


@pytest.mark.skipif(torch.cuda.is_available(), reason="device gate is checked on a machine without a GPU")
def test_prologue_device_gate_without_gpu(lib):
    assert prologue(lib) == DEVICE
    assert prologue(lib, qo=A, ko=2 * A) == DEVICE     # exact in-place passes validation
    assert prologue(lib, wq=0, wk=0, rc=0, rs=0, rows=0) == DEVICE


def forward(lib, q=A, k=2 * A, v=3 * A, o=4 * A, B=1, Sq=8, Sk=8, H=2, D=128, wq=5 * A, wk=5 * A + 512,
            eps=1e-6, rc=6 * A, rs=7 * A, rows=8, qv=-1, kvv=-1, scale=0.0883, ws=16 * A, wsb=None):
    if wsb is None:
        wsb = lib.h3attn_forward_workspace_bytes(B, Sq, Sk, H) if B > 0 and Sq > 0 and Sk > 0 and H > 0 else 0
    return lib.h3attn_forward(P(q), P(k), P(v), P(o), B, Sq, Sk, H, D, P(wq), P(wk), eps, P(rc), P(rs), rows,
                              qv, kvv, scale, P(ws), wsb, None)


def test_forward_validation(lib):
    assert forward(lib, v=0) == NULLP
    assert forward(lib, o=0) == NULLP
    assert forward(lib, wq=0) == NULLP
    assert forward(lib, D=256) == SHAPE
    assert forward(lib, qv=9) == SHAPE
    assert forward(lib, qv=-2) == SHAPE
    assert forward(lib, kvv=0) == SHAPE
    assert forward(lib, kvv=9) == SHAPE
    assert forward(lib, B=70000, H=1) == SHAPE
    assert forward(lib, scale=0.0) == VALUE
    assert forward(lib, scale=float("inf")) == VALUE
    assert forward(lib, o=4 * A + 8) == ALIGN
    assert forward(lib, ws=0) == WS
    assert forward(lib, wsb=1024) == WS
    assert forward(lib, ws=16 * A + 16) == ALIGN   # workspace must be 256-byte aligned
    assert forward(lib, o=A) == ALIAS              # o on top of q
    assert forward(lib, ws=3 * A) == ALIAS         # workspace on top of v
    assert forward(lib, rows=4) == SHAPE


@pytest.mark.skipif(torch.cuda.is_available(), reason="device gate is checked on a machine without a GPU")
def test_forward_device_gate_without_gpu(lib):
    assert forward(lib) == DEVICE
    assert forward(lib, wq=0, wk=0, rc=0, rs=0, rows=0, qv=0, kvv=1) == DEVICE
    assert lib.h3attn_rope_tables(P(A), P(2 * A), 16, 1e4, None) == DEVICE


def test_rope_tables_validation(lib):
    assert lib.h3attn_rope_tables(P(0), P(2 * A), 16, 1e4, None) == NULLP
    assert lib.h3attn_rope_tables(P(A), P(2 * A), 0, 1e4, None) == SHAPE
    assert lib.h3attn_rope_tables(P(A), P(2 * A), 16, float("nan"), None) == VALUE
    assert lib.h3attn_rope_tables(P(A), P(2 * A), 16, 0.5, None) == VALUE
    assert lib.h3attn_rope_tables(P(A + 4), P(2 * A), 16, 1e4, None) == ALIGN
    assert lib.h3attn_rope_tables(P(A), P(A + 64), 16, 1e4, None) == ALIAS


def test_python_wrapper_rejections():
    q = torch.zeros(1, 8, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        h3attn.forward(q, q, q)
    with pytest.raises(ValueError, match="GPU"):
        h3attn.qk_prologue(q, q, None, None)
    with pytest.raises(ValueError, match="GPU"):
        h3attn.forward(q.float(), q, q)
    with pytest.raises(TypeError):
        h3attn._check_bshd("q", q.numpy())


def test_python_wrapper_variant_rejections():
    """Argument checks of the binding's variants, before any device call."""
    q = torch.zeros(1, 8, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        h3attn.forward(q, q, q, window=(4, 2, 1, 1))
    x = torch.zeros(1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        h3attn.rmsnorm_scale_shift(x, x[:, :1], x[:, :1])
    with pytest.raises(ValueError, match="bfloat16"):
        h3attn.rmsnorm_scale_shift(x.float(), x[:, :1], x[:, :1])


def fwd_ex(lib, stages=3, ws=16 * A, wsb=None, **kw):
    """h3attn_forward_ex with a valid descriptor of fake pointers, then the
    fields in kw overridden; the call fails validation or the device gate."""
    a = h3attn.ForwardArgs()
    a.q, a.k, a.v, a.o = A, 2 * A, 3 * A, 4 * A
    a.B, a.Sq, a.Sk, a.Hq, a.Hkv, a.head_dim = 1, 8, 8, 4, 2, 128
    a.q_norm_w, a.k_norm_w, a.eps = 5 * A, 5 * A + 512, 1e-6
    a.rope_rows, a.rope_cos, a.rope_sin = 8, 6 * A, 7 * A
    a.q_valid, a.kv_valid, a.valid_lengths, a.causal, a.softmax_scale = -1, -1, None, 0, 0.0883
    for key, val in kw.items():
        if key.endswith("_stride"):
            getattr(a, key)[:] = val
        else:
            setattr(a, key, val)
    if wsb is None:
        wsb = lib.h3attn_forward_ex_workspace_bytes(ctypes.byref(a))
    return lib.h3attn_forward_ex(ctypes.byref(a), P(ws), wsb, stages, None)


def test_forward_ex_workspace_bytes(lib):
    # q rows for Hq heads, k and v^T rows for Hkv heads, partial records only
    # for the uniform schedule (no causal mask, no per-item lengths); at head
    # dim 128 a record is sized for three query tiles per wave (96
    # accumulators, three row offsets and three partial sums per lane); then
    # the key-norm maxima, one fp32 per 4096 padded keys of each (b, kv
    # head), padded to 256 bytes
    rec = (96 + 6) * 512 * 4
    kn = lambda n: (n * 4 + 255) // 256 * 256   # noqa: E731
    assert h3attn.forward_ex_workspace_bytes(1, 104448, 104448, 6, 2) == \
        (6 + 2 * 2) * 104448 * 256 + 2 * 256 * rec + kn(2 * 26)
    assert h3attn.forward_ex_workspace_bytes(1, 104448, 104448, 6, 2, causal=True) == \
        (6 + 2 * 2) * 104448 * 256 + kn(2 * 26)
    assert h3attn.forward_ex_workspace_bytes(2, 1000, 300, 4, 1, per_item_lengths=True) == \
        2 * (4 * 1152 + 2 * 1 * 512) * 256 + kn(2)
    assert h3attn.forward_ex_workspace_bytes(1, 104448, 104448, 6, 6, window=True) == \
        3 * 6 * 104448 * 256 + kn(6 * 26)
    # rows of 2 * head_dim bytes; split records per lane of 512: 64 accumulators (at head dim 64, 64
    # query rows x 64 channels over 64 lanes; at 256, 32 rows x 128 channels, each wave of a pair
    # holding half of the channels) and one row offset and one sum per 16-row query tile (four at 64,
    # two at 256). Query rows pad to 512 at head dim 64.
    assert h3attn.forward_ex_workspace_bytes(1, 4096, 4096, 8, 8, head_dim=64) == \
        3 * 8 * 4096 * 128 + 2 * 256 * (64 + 8) * 512 * 4 + kn(8)
    assert h3attn.forward_ex_workspace_bytes(1, 4100, 4100, 8, 8, head_dim=64) == \
        (8 * 4608 + 2 * 8 * 4352) * 128 + 2 * 256 * (64 + 8) * 512 * 4 + kn(8 * 2)
    assert h3attn.forward_ex_workspace_bytes(1, 4096, 4096, 8, 8, head_dim=256) == \
        3 * 8 * 4096 * 512 + 2 * 256 * (64 + 4) * 512 * 4 + kn(8)
    assert h3attn.forward_ex_workspace_bytes(1, 8, 8, 4, 4, head_dim=96) == 0
    assert h3attn.forward_ex_workspace_bytes(1, 8, 8, 6, 4) == 0      # 6 heads do not group into 4
    assert h3attn.forward_ex_workspace_bytes(1, 8, 8, 4, 0) == 0
    assert lib.h3attn_forward_ex_workspace_bytes(None) == 0


def far_apart(Sk):
    """Fields of an Sk-key call whose fake buffers are far enough apart not
    to overlap (the rotary tables grow with the key count)."""
    return dict(Sk=Sk, rope_rows=Sk, k=1 << 40, v=1 << 41, o=1 << 42, rope_cos=1 << 43, rope_sin=1 << 44,
                ws=1 << 45, wsb=1 << 40)


def test_forward_ex_validation(lib):
    assert lib.h3attn_forward_ex(None, P(16 * A), 1 << 20, 3, None) == NULLP
    assert fwd_ex(lib, v=None) == NULLP
    assert fwd_ex(lib, stages=0) == VALUE
    assert fwd_ex(lib, Hkv=3, wsb=1 << 30) == SHAPE            # 4 query heads do not group into 3
    assert fwd_ex(lib, Hkv=0, wsb=1 << 30) == SHAPE
    assert fwd_ex(lib, causal=2) == VALUE
    assert fwd_ex(lib, kv_valid=0) == SHAPE                    # uniform lengths need a valid key
    assert fwd_ex(lib, q_stride=[8 * 4 * 128, 4 * 128, -128]) == SHAPE
    assert fwd_ex(lib, k_stride=[2048, 260, 128]) == ALIGN     # rows must stay 16-byte aligned
    assert fwd_ex(lib, valid_lengths=9 * A + 2) == ALIGN
    assert fwd_ex(lib, valid_lengths=4 * A + 64) == ALIAS      # lengths inside o
    # a strided q whose rows reach over o
    assert fwd_ex(lib, q_stride=[0, 3 * A // 2, 128]) == ALIAS
    assert fwd_ex(lib, wsb=4096) == WS
    assert fwd_ex(lib, ws=0) == WS
    assert fwd_ex(lib, o=A + 1024) == ALIAS                    # o on top of q
    # frame window and gate
    assert fwd_ex(lib, window_frame_rows=-1) == VALUE
    assert fwd_ex(lib, window_chunk_frames=5) == VALUE         # window fields without a window
    assert fwd_ex(lib, window_frame_rows=4, window_chunk_frames=0) == VALUE
    assert fwd_ex(lib, window_frame_rows=4, window_chunk_frames=2, window_radius=-1) == VALUE
    assert fwd_ex(lib, window_frame_rows=4, window_chunk_frames=2, window_anchor_frames=-1) == VALUE
    assert fwd_ex(lib, window_frame_rows=4, window_chunk_frames=2, causal=1) == VALUE
    assert fwd_ex(lib, window_frame_rows=4, window_chunk_frames=2, Sq=1 << 28, Sk=1 << 28,
                  rope_rows=1 << 28, wsb=1 << 40) == SHAPE
    assert fwd_ex(lib, head_dim=96, wsb=1 << 30) == SHAPE
    assert fwd_ex(lib, head_dim=64, wsb=1 << 30) == SHAPE     # norm weights and rotary need 128
    assert fwd_ex(lib, head_dim=256, q_norm_w=None, k_norm_w=None, wsb=1 << 30) == SHAPE   # rotary still given
    assert fwd_ex(lib, gate=9 * A + 1) == ALIGN
    assert fwd_ex(lib, gate=4 * A + 256) == ALIAS               # gate inside o
    # one head's prepared keys reach 2 GB: past the 32-bit load offsets
    assert fwd_ex(lib, **far_apart(1 << 23)) == SHAPE


@pytest.mark.skipif(torch.cuda.is_available(), reason="device gate is checked on a machine without a GPU")
def test_forward_ex_device_gate_without_gpu(lib):
    assert fwd_ex(lib) == DEVICE
    assert fwd_ex(lib, **far_apart((1 << 23) - 512)) == DEVICE   # just under the per-head key limit
    assert fwd_ex(lib, causal=1) == DEVICE
    assert fwd_ex(lib, valid_lengths=9 * A, kv_valid=0) == DEVICE   # per-item lengths replace kv_valid
    assert fwd_ex(lib, q_stride=[8 * 12 * 128, 12 * 128, 128], k_stride=[8 * 12 * 128, 12 * 128, 128]) == DEVICE
    assert fwd_ex(lib, window_frame_rows=4, window_chunk_frames=2, window_radius=1, window_anchor_frames=1,
                  gate=9 * A + 2) == DEVICE
    assert fwd_ex(lib, window_frame_rows=1 << 30, window_chunk_frames=1 << 30, window_radius=1 << 30,
                  window_anchor_frames=1 << 30) == DEVICE          # huge geometry clamps, no overflow
    for d in (64, 256):
        assert fwd_ex(lib, head_dim=d, q_norm_w=None, k_norm_w=None, rope_cos=None, rope_sin=None,
                      rope_rows=0) == DEVICE


def scale_shift(lib, x=A, y=2 * A, B=1, S=8, D=64, w=3 * A, eps=1e-6, sc=4 * A, sh=5 * A, M=2, idx=6 * A):
    return lib.h3attn_rmsnorm_scale_shift(P(x), P(y), B, S, D, P(w), eps, P(sc), P(sh), M, P(idx), None)


def test_scale_shift_validation(lib):
    assert scale_shift(lib, x=0) == NULLP
    assert scale_shift(lib, y=0) == NULLP
    assert scale_shift(lib, sc=0) == NULLP
    assert scale_shift(lib, sh=0) == NULLP
    assert scale_shift(lib, B=0) == SHAPE
    assert scale_shift(lib, S=0) == SHAPE
    assert scale_shift(lib, M=0) == SHAPE
    assert scale_shift(lib, D=0) == SHAPE
    assert scale_shift(lib, D=60) == SHAPE            # not a multiple of 8
    assert scale_shift(lib, D=16384 + 8) == SHAPE     # past the largest row
    assert scale_shift(lib, B=1 << 16, S=1 << 15) == SHAPE   # B*S >= 2^31
    assert scale_shift(lib, eps=float("inf")) == VALUE
    assert scale_shift(lib, eps=-1e-6) == VALUE
    assert scale_shift(lib, x=A + 8) == ALIGN
    assert scale_shift(lib, sh=5 * A + 2) == ALIGN
    assert scale_shift(lib, w=3 * A + 4) == ALIGN
    assert scale_shift(lib, idx=6 * A + 2) == ALIGN
    assert scale_shift(lib, y=A + 512) == ALIAS       # partial overlap with x
    assert scale_shift(lib, y=4 * A + 128) == ALIAS   # on top of scale
    assert scale_shift(lib, y=5 * A) == ALIAS         # on top of shift
    assert scale_shift(lib, w=2 * A + 64) == ALIAS    # weight inside y
    assert scale_shift(lib, idx=2 * A + 16) == ALIAS  # index inside y


@pytest.mark.skipif(torch.cuda.is_available(), reason="device gate is checked on a machine without a GPU")
def test_scale_shift_device_gate_without_gpu(lib):
    assert scale_shift(lib) == DEVICE
    assert scale_shift(lib, y=A) == DEVICE                   # exact in place passes validation
    assert scale_shift(lib, w=0, idx=0) == DEVICE            # weight and index are optional
    assert scale_shift(lib, D=16384, w=0) == DEVICE
    assert scale_shift(lib, idx=6 * A + 4) == DEVICE         # 4-byte aligned index is enough


# ------------------------------------------------------------- microbenchmarks

MICRO_HEADER = os.path.join(ROOT, "include", "h3attn_micro.h")


def test_micro_exports_every_declared_symbol(lib):
    from video_dit_dense_amd import micro
    text = re.sub(r"/\*.*?\*/", "", open(MICRO_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(h3micro_\w+)\s*\(", text)))
    assert names == sorted(micro.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n


def test_micro_validation(lib):
    from video_dit_dense_amd import micro
    m = micro.load_library()
    assert m.h3micro_mfma_bf16(1, 1, None, P(2 * A), None) == NULLP
    assert m.h3micro_mfma_bf16(0, 1, P(A), P(2 * A), None) == SHAPE
    assert m.h3micro_mfma_bf16(1, 0, P(A), P(2 * A), None) == SHAPE
    assert m.h3micro_mfma_bf16(65537, 1, P(A), P(2 * A), None) == SHAPE
    assert m.h3micro_mfma_bf16(65536, 1 << 17, P(A), P(2 * A), None) == SHAPE   # > 2^32 block-iterations
    assert m.h3micro_mfma_bf16(4, 10, P(A), P(2 * A + 4), None) == ALIGN
    assert m.h3micro_mfma_bf16(4, 10, P(A), P(A + 1024), None) == ALIAS           # sink is 4 KB
    assert m.h3micro_exp(1, 1, None, None) == NULLP
    assert m.h3micro_exp(1, 1 << 25, P(A), None) == SHAPE
    assert m.h3micro_exp(1, 1, P(A + 2), None) == ALIGN
    assert m.h3micro_copy(None, P(A), 16, None) == NULLP
    assert m.h3micro_copy(P(A), P(2 * A), 0, None) == SHAPE
    assert m.h3micro_copy(P(A), P(2 * A), 24, None) == SHAPE
    assert m.h3micro_copy(P(A + 8), P(2 * A), 16, None) == ALIGN
    assert m.h3micro_copy(P(A), P(A + 16), 32, None) == ALIAS
    if not torch.cuda.is_available():   # valid arguments reach the device gate
        assert m.h3micro_mfma_bf16(4, 10, P(A), P(2 * A), None) == DEVICE
        assert m.h3micro_exp(4, 10, P(A), None) == DEVICE
        assert m.h3micro_copy(P(A), P(2 * A), 16, None) == DEVICE


# ---------------------------------------------------- no-allocation forward

G = 1 << 30   # fake pointers 1 GiB apart, so full-size tensors do not overlap


def noalloc(lib, q=A, k=2 * A, v=3 * A, o=4 * A, B=1, Sq=8, Sk=8, H=2, D=128, wq=5 * A, wk=5 * A + 512,
            eps=1e-6, rc=6 * A, rs=7 * A, rows=8, qv=-1, kvv=-1, scale=0.0883):
    return lib.h3attn_forward_noalloc(P(q), P(k), P(v), P(o), B, Sq, Sk, H, D, P(wq), P(wk), eps, P(rc), P(rs),
                                      rows, qv, kvv, scale, None)


def test_noalloc_validation(lib):
    assert h3attn.NOALLOC_SCRATCH_BYTES == 256 << 20
    assert noalloc(lib, q=0) == NULLP
    assert noalloc(lib, D=64) == SHAPE
    assert noalloc(lib, kvv=0) == SHAPE
    assert noalloc(lib, scale=-1.0) == VALUE
    assert noalloc(lib, o=4 * A + 8) == ALIGN
    assert noalloc(lib, o=2 * A) == ALIAS
    # Sizes whose workspace exceeds the static array: padded (309 MB) and the
    # full 104448 x 6 share (588 MB) are rejected before anything else runs.
    big = dict(q=G, k=2 * G, v=3 * G, o=4 * G, wq=5 * G, wk=5 * G + 512, rc=6 * G, rs=7 * G)
    assert lib.h3attn_forward_workspace_bytes(1, 32768, 32768, 8) > h3attn.NOALLOC_SCRATCH_BYTES
    assert noalloc(lib, B=1, Sq=32768, Sk=32768, H=8, rows=32768, **big) == WS
    assert noalloc(lib, B=1, Sq=104448, Sk=104448, H=6, rows=104448, **big) == WS
    # mid and cross fit
    assert lib.h3attn_forward_workspace_bytes(1, 8192, 8192, 8) <= h3attn.NOALLOC_SCRATCH_BYTES
    assert lib.h3attn_forward_workspace_bytes(1, 32760, 512, 8) <= h3attn.NOALLOC_SCRATCH_BYTES
    if not torch.cuda.is_available():   # valid arguments reach the device gate
        assert noalloc(lib) == DEVICE
        assert noalloc(lib, B=1, Sq=8192, Sk=8192, H=8, rows=8192, **big) == DEVICE


# ------------------------------------------------------ prologue + Ulysses pack

def pack(lib, q=A, k=2 * A, v=3 * A, qs=4 * A, ks=5 * A, vs=6 * A, B=1, S=8, H=4, Pr=2, D=128, off=0,
         wq=7 * A, wk=7 * A + 512, eps=1e-6, rc=8 * A, rs=9 * A, rows=8):
    return lib.h3attn_qkv_pack(P(q), P(k), P(v), P(qs), P(ks), P(vs), B, S, H, Pr, D, off, P(wq), P(wk), eps,
                               P(rc), P(rs), rows, None)


def test_pack_validation(lib):
    assert pack(lib, v=0) == NULLP
    assert pack(lib, vs=0) == NULLP
    assert pack(lib, wk=0) == NULLP
    assert pack(lib, Pr=3) == SHAPE             # 4 heads over 3 ranks
    assert pack(lib, Pr=0) == SHAPE
    assert pack(lib, D=64) == SHAPE
    assert pack(lib, off=-1) == SHAPE
    assert pack(lib, off=1) == SHAPE            # table rows 8 < 1 + 8
    assert pack(lib, eps=float("nan")) == VALUE
    assert pack(lib, ks=5 * A + 8) == ALIGN
    assert pack(lib, qs=A) == ALIAS             # no in-place form
    assert pack(lib, vs=4 * A + 256) == ALIAS   # send buffers overlap
    assert pack(lib, qs=8 * A) == ALIAS         # onto the cos table
    if not torch.cuda.is_available():
        assert pack(lib) == DEVICE
        assert pack(lib, off=2, rows=10) == DEVICE
        assert pack(lib, wq=0, wk=0, rc=0, rs=0, rows=0, off=1000) == DEVICE   # no rotary: any offset


def test_forward_ex_plan(lib):
    """The schedule query: host arithmetic on a checked descriptor, no device
    needed when the CU count is given."""
    sch = h3attn.schedule
    full = sch(1, 104448, 104448, 6, cus=256)
    assert full == {"kernel": "ring", "query_tiles": 3, "rows_per_tile": 384, "tiles": 1632, "whole_tiles": 1536,
                    "split_tiles": 96, "split_blocks": 256, "grid": 1792}
    # the same launch forced to two tiles per wave: 408 blocks of 256 rows per head
    two = sch(1, 104448, 104448, 6, query_tiles=2, cus=256)
    assert (two["rows_per_tile"], two["tiles"], two["whole_tiles"], two["split_tiles"]) == (256, 2448, 2304, 144)
    assert sch(1, 8192, 8192, 8, cus=256)["query_tiles"] == 2                 # one whole round of 256 tiles
    padded = sch(1, 32768, 32768, 8, q_valid=30720, kv_valid=30720, cus=256)
    assert (padded["query_tiles"], padded["tiles"], padded["grid"]) == (3, 640, 512 + 256 + 8 * 6)
    assert sch(1, 32760, 512, 8, kv_valid=300, cus=256)["kernel"] == "resident"
    # the resident kernel stores through a 32-bit buffer range per item: an item's output of 2^31 bytes or
    # more (here 1048576 rows x 8 heads x 256 B) takes the ring kernel instead
    assert sch(2, 1048575, 512, 8, kv_valid=300, cus=256)["kernel"] == "resident"
    assert sch(1, 1048576, 512, 8, kv_valid=300, cus=256)["kernel"] == "ring"
    causal = sch(1, 104448, 104448, 6, causal=True, cus=256)
    assert (causal["query_tiles"], causal["tiles"], causal["split_tiles"]) == (3, 1632, 0)
    assert sch(1, 104448, 104448, 12, head_dim=64, cus=256)["rows_per_tile"] == 512
    assert sch(1, 104448, 104448, 3, head_dim=256, cus=256)["rows_per_tile"] == 128
    # errors: no plan, a query-tile count the head dim does not have, bad sizes
    a = h3attn.ForwardArgs()
    a.q, a.k, a.v, a.o = A, 2 * A, 3 * A, 4 * A
    a.B, a.Sq, a.Sk, a.Hq, a.Hkv, a.head_dim = 1, 8, 8, 2, 2, 128
    a.q_valid, a.kv_valid, a.softmax_scale = -1, -1, 0.0883
    p = h3attn.Plan()
    assert lib.h3attn_forward_ex_plan(ctypes.byref(a), 256, None) == NULLP
    assert lib.h3attn_forward_ex_plan(None, 256, ctypes.byref(p)) == NULLP
    assert lib.h3attn_forward_ex_plan(ctypes.byref(a), 256, ctypes.byref(p)) == 0
    for qt, want in ((1, VALUE), (4, VALUE), (2, 0), (3, 0)):
        a.query_tiles = qt
        assert lib.h3attn_forward_ex_plan(ctypes.byref(a), 256, ctypes.byref(p)) == want, qt
    a.head_dim, a.query_tiles = 64, 3
    assert lib.h3attn_forward_ex_plan(ctypes.byref(a), 256, ctypes.byref(p)) == VALUE
    a.head_dim, a.query_tiles = 96, 0
    assert lib.h3attn_forward_ex_plan(ctypes.byref(a), 256, ctypes.byref(p)) == SHAPE
    assert fwd_ex(lib, query_tiles=5) == VALUE
