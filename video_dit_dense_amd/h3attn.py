"""ctypes binding of libh3attn.so: argument marshalling only.

Every computation runs in the library's HIP kernels. torch supplies device
memory (outputs, workspace) and the current stream. There is no CPU path: if
the library is missing or the device is not gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libh3attn.so")

HEAD_DIM = 128                 # H3's head dim: the Q/K norm and rotary prologue apply to it only
HEAD_DIMS = (64, 128, 256)     # head dims the attention kernels take
ROPE_PAIRS = 48

STATUS = {
    0: "OK", 1: "ERR_NULL_POINTER", 2: "ERR_BAD_SHAPE", 3: "ERR_BAD_ALIGNMENT",
    4: "ERR_ALIASING", 5: "ERR_BAD_VALUE", 6: "ERR_WORKSPACE",
    7: "ERR_UNSUPPORTED_DEVICE", 8: "ERR_HIP",
}

# Exported symbols and their C signatures (include/h3attn.h).
_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
SIGNATURES = {
    "h3attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "h3attn_rope_tables": (ctypes.c_int, [_P, _P, _I, ctypes.c_double, _P]),
    "h3attn_qk_prologue": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _F, _P, _P, _I, _P]),
    "h3attn_qkv_pack": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _F, _P, _P, _I,
                                       _P]),
    "h3attn_forward_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "h3attn_forward": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _F, _P, _P, _I,
                                      _I, _I, _F, _P, ctypes.c_size_t, _P]),
    "h3attn_forward_stages": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _F, _P, _P, _I,
                                             _I, _I, _F, _P, ctypes.c_size_t, ctypes.c_uint32, _P]),
    "h3attn_forward_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _F, _P, _P, _I,
                                              _I, _I, _F, _P]),
}

# Bytes of the library's static workspace used by h3attn_forward_noalloc
# (H3ATTN_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 256 << 20

STAGE_PREPARE = 1
STAGE_ATTEND = 2


class ForwardArgs(ctypes.Structure):
    """Mirror of h3attn_forward_args (include/h3attn.h)."""
    _fields_ = [
        ("q", _P), ("k", _P), ("v", _P), ("o", _P),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3), ("v_stride", ctypes.c_int64 * 3),
        ("B", _I), ("Sq", _I), ("Sk", _I), ("Hq", _I), ("Hkv", _I), ("head_dim", _I),
        ("q_norm_w", _P), ("k_norm_w", _P), ("eps", _F),
        ("rope_rows", _I), ("rope_cos", _P), ("rope_sin", _P),
        ("q_valid", _I), ("kv_valid", _I), ("valid_lengths", _P), ("causal", _I),
        ("softmax_scale", _F),
        ("window_frame_rows", _I), ("window_chunk_frames", _I), ("window_radius", _I),
        ("window_anchor_frames", _I), ("gate", _P), ("query_tiles", _I),
    ]


class Plan(ctypes.Structure):
    """Mirror of h3attn_plan (include/h3attn.h)."""
    _fields_ = [
        ("kernel", _I), ("query_tiles", _I), ("rows_per_tile", _I), ("reserved", _I),
        ("tiles", ctypes.c_int64), ("whole_tiles", ctypes.c_int64), ("split_tiles", ctypes.c_int64),
        ("split_blocks", ctypes.c_int64), ("grid", ctypes.c_int64),
    ]


SIGNATURES["h3attn_forward_ex_workspace_bytes"] = (ctypes.c_size_t, [ctypes.POINTER(ForwardArgs)])
SIGNATURES["h3attn_forward_ex_plan"] = (ctypes.c_int, [ctypes.POINTER(ForwardArgs), _I, ctypes.POINTER(Plan)])
SIGNATURES["h3attn_forward_ex"] = (ctypes.c_int, [ctypes.POINTER(ForwardArgs), _P, ctypes.c_size_t,
                                                  ctypes.c_uint32, _P])
SIGNATURES["h3attn_rmsnorm_scale_shift"] = (ctypes.c_int, [_P, _P, _I, _I, _I, _P, _F, _P, _P, _I, _P, _P])

_lib = None


class H3AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m video_dit_dense_amd.build` "
                              "(there is no CPU fallback)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().h3attn_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise H3AttnError(status, where)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_bshd(name: str, t: torch.Tensor, view: bool = False, dims=(HEAD_DIM,)) -> None:
    """A bf16 [B, S, H, D] GPU tensor with D in `dims`; contiguous, or with
    `view` any strided view whose channels are contiguous (e.g. a slice of a
    fused QKV projection)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16 (got {t.dtype}); the library is bf16-only")
    if t.dim() != 4 or t.shape[-1] not in dims:
        raise ValueError(f"{name} must be [B, S, H, D] with D in {dims} (got {tuple(t.shape)})")
    if view:
        if t.stride(-1) != 1 or min(t.stride()) < 0:
            raise ValueError(f"{name} must have contiguous channels and non-negative strides")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous BSHD")
    if t.requires_grad and torch.is_grad_enabled():
        raise RuntimeError(f"{name} requires grad: h3attn is inference-only (no backward)")


def _check_f32(name: str, t: torch.Tensor | None, numel: int | None = None) -> None:
    if t is None:
        return
    if t.device.type != "cuda" or t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 GPU tensor")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements (got {t.numel()})")


def rope_tables(rows: int, theta: float = 1e4, device="cuda") -> tuple[torch.Tensor, torch.Tensor]:
    """cos/sin tables [rows, 48] (fp32) for the 96/128 partial rotary embedding."""
    lib = load_library()
    cos = torch.empty((rows, ROPE_PAIRS), dtype=torch.float32, device=device)
    sin = torch.empty((rows, ROPE_PAIRS), dtype=torch.float32, device=device)
    _check(lib.h3attn_rope_tables(_ptr(cos), _ptr(sin), int(rows), float(theta), _stream(cos.device)),
           "h3attn_rope_tables")
    return cos, sin


def qk_prologue(q: torch.Tensor, k: torch.Tensor, w_q: torch.Tensor | None, w_k: torch.Tensor | None,
                eps: float = 1e-6, rope_cos: torch.Tensor | None = None, rope_sin: torch.Tensor | None = None,
                q_out: torch.Tensor | None = None, k_out: torch.Tensor | None = None):
    """Per-head RMSNorm + 96/128 partial rotary on q and k. Pass q_out=q,
    k_out=k to run in place. Returns (q_out, k_out)."""
    lib = load_library()
    _check_bshd("q", q)
    _check_bshd("k", k)
    _check_f32("w_q", w_q, HEAD_DIM)
    _check_f32("w_k", w_k, HEAD_DIM)
    _check_f32("rope_cos", rope_cos)
    _check_f32("rope_sin", rope_sin)
    B, Sq, H, D = q.shape
    if k.shape[0] != B or k.shape[2] != H:
        raise ValueError("q and k must share B and H")
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    _check_bshd("q_out", q_out)
    _check_bshd("k_out", k_out)
    rows = 0 if rope_cos is None else rope_cos.shape[0]
    st = lib.h3attn_qk_prologue(_ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), B, Sq, k.shape[1], H, D,
                                _ptr(w_q), _ptr(w_k), float(eps), _ptr(rope_cos), _ptr(rope_sin), rows,
                                _stream(q.device))
    _check(st, "h3attn_qk_prologue")
    return q_out, k_out


def qkv_pack(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: int, row_offset: int = 0,
             w_q: torch.Tensor | None = None, w_k: torch.Tensor | None = None, eps: float = 1e-6,
             rope_cos: torch.Tensor | None = None, rope_sin: torch.Tensor | None = None,
             out: tuple | None = None) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """h3attn_qkv_pack: one rank's sequence shard q, k, v [B, S_local, H, 128]
    (rows row_offset .. of the sequence) to destination-major send buffers
    [P, B, S_local, H/P, 128], q and k through the RMSNorm + rotary prologue,
    v copied. Returns (q_send, k_send, v_send); `out` may pass them in."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bshd(name, t)
    _check_f32("w_q", w_q, HEAD_DIM)
    _check_f32("w_k", w_k, HEAD_DIM)
    _check_f32("rope_cos", rope_cos)
    _check_f32("rope_sin", rope_sin)
    B, S, H, D = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    if P < 1 or H % P:
        raise ValueError("P must divide the head count")
    shape = (P, B, S, H // P, D)
    if out is None:
        out = tuple(torch.empty(shape, dtype=q.dtype, device=q.device) for _ in range(3))
    for name, t in zip(("q_send", "k_send", "v_send"), out):
        if (t.device.type != "cuda" or t.dtype != torch.bfloat16 or tuple(t.shape) != shape
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous bfloat16 GPU tensor {list(shape)}")
    rows = 0 if rope_cos is None else rope_cos.shape[0]
    st = lib.h3attn_qkv_pack(_ptr(q), _ptr(k), _ptr(v), *(_ptr(t) for t in out), B, S, H, int(P), D,
                             int(row_offset), _ptr(w_q), _ptr(w_k), float(eps), _ptr(rope_cos), _ptr(rope_sin),
                             rows, _stream(q.device))
    _check(st, "h3attn_qkv_pack")
    return out


def workspace_bytes(B: int, Sq: int, Sk: int, H: int) -> int:
    return int(load_library().h3attn_forward_workspace_bytes(B, Sq, Sk, H))


def make_workspace(B: int, Sq: int, Sk: int, H: int, device="cuda") -> torch.Tensor:
    n = workspace_bytes(B, Sq, Sk, H)
    if n == 0:
        raise ValueError("bad sizes for the workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            w_q: torch.Tensor | None = None, w_k: torch.Tensor | None = None, eps: float = 1e-6,
            rope_cos: torch.Tensor | None = None, rope_sin: torch.Tensor | None = None,
            q_valid: int | None = None, kv_valid: int | None = None, scale: float | None = None,
            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
            stages: int = STAGE_PREPARE | STAGE_ATTEND, causal: bool = False,
            valid_lengths: torch.Tensor | None = None, window: tuple | None = None,
            gate: torch.Tensor | None = None, query_tiles: int = 0) -> torch.Tensor:
    """The attention step: prologue on q/k (if weights/tables given), then
    softmax attention with key padding (kv_valid) and a zeroed query tail
    (q_valid). Returns o [B, Sq, Hq, D] bf16. D is 128 (H3), 64 or 256; the
    norm and rotary prologue apply to 128 only.

    k and v may have fewer heads than q (grouped heads: query head h reads
    kv head h // (Hq // Hkv)); q, k and v may be strided views with
    contiguous channels. `causal` masks key j for query row i when j > i.
    `valid_lengths`, an int32 GPU tensor [B, 2] of (q_valid, kv_valid) per
    batch item, replaces q_valid / kv_valid. `stages` selects the prepare
    and/or attend stage; a lone attend stage needs `workspace` from an earlier
    prepare call with the same arguments. `window` = (frame_rows,
    chunk_frames, radius, anchor_frames) restricts each row to its frame
    window (anchor-frame rows see every key); `gate`, a bf16 GPU tensor
    [B, Sq, Hq], multiplies each output row by sigmoid(gate). `query_tiles`
    (0: the library chooses) sets the attention kernel's 16-row query tiles
    per wave, 2 or 3 at head dim 128. Dense inputs without the variants go
    through h3attn_forward_stages, everything else through h3attn_forward_ex."""
    lib = load_library()
    a, o, plain = _forward_args(q, k, v, w_q, w_k, eps, rope_cos, rope_sin, q_valid, kv_valid, scale, out,
                                causal, valid_lengths, window, gate, query_tiles)
    if stages != (STAGE_PREPARE | STAGE_ATTEND) and workspace is None:
        raise ValueError("a single stage needs a caller-kept workspace")
    if plain:
        B, Sq, H, D = q.shape
        ws = make_workspace(B, Sq, k.shape[1], H, q.device) if workspace is None else workspace
        st = lib.h3attn_forward_stages(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, Sq, k.shape[1], H, D,
                                       _ptr(w_q), _ptr(w_k), float(eps), _ptr(rope_cos), _ptr(rope_sin),
                                       a.rope_rows, a.q_valid, a.kv_valid, a.softmax_scale, _ptr(ws),
                                       ws.numel() * ws.element_size(), int(stages), _stream(q.device))
        _check(st, "h3attn_forward_stages")
        return o
    if workspace is None:
        n = int(lib.h3attn_forward_ex_workspace_bytes(ctypes.byref(a)))
        if n == 0:
            raise ValueError("bad sizes for the workspace")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    st = lib.h3attn_forward_ex(ctypes.byref(a), _ptr(workspace), workspace.numel() * workspace.element_size(),
                               int(stages), _stream(q.device))
    _check(st, "h3attn_forward_ex")
    return o


def schedule(B: int, Sq: int, Sk: int, Hq: int, Hkv: int | None = None, head_dim: int = HEAD_DIM,
             q_valid: int = -1, kv_valid: int = -1, causal: bool = False, per_item_lengths: bool = False,
             window: tuple | None = None, query_tiles: int = 0, cus: int = 0) -> dict:
    """The schedule forward() launches for these sizes and variant on a
    device with `cus` compute units (0: the current device), from
    h3attn_forward_ex_plan: the kernel ("ring" or "resident"), query tiles
    per wave, rows per tile, the tiles with work, the uniform schedule's
    whole tiles, split tiles and split blocks, and the grid. Host arithmetic
    only; the descriptor's buffers are placeholders that are never touched."""
    a = ForwardArgs()
    a.q, a.k, a.v, a.o = 1 << 44, 2 << 44, 3 << 44, 4 << 44
    a.B, a.Sq, a.Sk, a.Hq, a.Hkv, a.head_dim = B, Sq, Sk, Hq, Hkv or Hq, head_dim
    a.eps, a.softmax_scale = 1e-6, 1.0 / math.sqrt(head_dim)
    a.q_valid, a.kv_valid = q_valid, kv_valid
    a.valid_lengths = (5 << 44) if per_item_lengths else None
    a.causal = 1 if causal else 0
    if window:
        a.window_frame_rows, a.window_chunk_frames, a.window_radius, a.window_anchor_frames = (
            int(x) for x in window)
    a.query_tiles = int(query_tiles)
    p = Plan()
    _check(load_library().h3attn_forward_ex_plan(ctypes.byref(a), int(cus), ctypes.byref(p)),
           "h3attn_forward_ex_plan")
    return {"kernel": "resident" if p.kernel else "ring", "query_tiles": p.query_tiles,
            "rows_per_tile": p.rows_per_tile, "tiles": p.tiles, "whole_tiles": p.whole_tiles,
            "split_tiles": p.split_tiles, "split_blocks": p.split_blocks, "grid": p.grid}


def _forward_args(q, k, v, w_q=None, w_k=None, eps=1e-6, rope_cos=None, rope_sin=None, q_valid=None,
                  kv_valid=None, scale=None, out=None, causal=False, valid_lengths=None, window=None,
                  gate=None, query_tiles=0):
    """Checks forward()'s arguments and fills h3attn_forward_args. Returns the
    descriptor, the output tensor (allocated when out is None) and whether the
    call is the plain dense one that h3attn_forward_stages takes."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bshd(name, t, view=True, dims=HEAD_DIMS)
    if q.shape[-1] != HEAD_DIM and any(x is not None for x in (w_q, w_k, rope_cos, rope_sin)):
        raise ValueError(f"the Q/K norm and rotary prologue are defined for head_dim {HEAD_DIM} only")
    _check_f32("w_q", w_q, HEAD_DIM)
    _check_f32("w_k", w_k, HEAD_DIM)
    _check_f32("rope_cos", rope_cos)
    _check_f32("rope_sin", rope_sin)
    B, Sq, H, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or H % Hkv != 0 or k.shape[3] != D:
        raise ValueError("k and v must be [B, Sk, Hkv, D] with q's B and D, and Hkv dividing q's heads")
    if valid_lengths is not None:
        if (valid_lengths.device.type != "cuda" or valid_lengths.dtype != torch.int32
                or tuple(valid_lengths.shape) != (B, 2) or not valid_lengths.is_contiguous()):
            raise ValueError("valid_lengths must be a contiguous int32 GPU tensor [B, 2]")
    if gate is not None:
        if (gate.device.type != "cuda" or gate.dtype != torch.bfloat16 or tuple(gate.shape) != (B, Sq, H)
                or not gate.is_contiguous()):
            raise ValueError("gate must be a contiguous bfloat16 GPU tensor [B, Sq, Hq]")
    if window is not None and len(window) != 4:
        raise ValueError("window is (frame_rows, chunk_frames, radius, anchor_frames)")
    o = torch.empty(B, Sq, H, D, dtype=q.dtype, device=q.device) if out is None else out
    _check_bshd("out", o, dims=(D,))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rows = 0 if rope_cos is None else rope_cos.shape[0]
    plain = (D == HEAD_DIM and Hkv == H and not causal and valid_lengths is None and window is None
             and gate is None and not query_tiles and q.is_contiguous() and k.is_contiguous()
             and v.is_contiguous())
    a = ForwardArgs()
    a.q, a.k, a.v, a.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()
    for field, t in (("q_stride", q), ("k_stride", k), ("v_stride", v)):
        getattr(a, field)[:] = [t.stride(0), t.stride(1), t.stride(2)]
    a.B, a.Sq, a.Sk, a.Hq, a.Hkv, a.head_dim = B, Sq, Sk, H, Hkv, D
    a.q_norm_w = None if w_q is None else w_q.data_ptr()
    a.k_norm_w = None if w_k is None else w_k.data_ptr()
    a.eps = float(eps)
    a.rope_rows = rows
    a.rope_cos = None if rope_cos is None else rope_cos.data_ptr()
    a.rope_sin = None if rope_sin is None else rope_sin.data_ptr()
    a.q_valid = -1 if q_valid is None else int(q_valid)
    a.kv_valid = -1 if kv_valid is None else int(kv_valid)
    a.valid_lengths = None if valid_lengths is None else valid_lengths.data_ptr()
    a.causal = 1 if causal else 0
    a.softmax_scale = scale
    if window is not None:
        a.window_frame_rows, a.window_chunk_frames, a.window_radius, a.window_anchor_frames = (
            int(x) for x in window)
    a.gate = None if gate is None else gate.data_ptr()
    a.query_tiles = int(query_tiles)
    return a, o, plain


def forward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                    w_q: torch.Tensor | None = None, w_k: torch.Tensor | None = None, eps: float = 1e-6,
                    rope_cos: torch.Tensor | None = None, rope_sin: torch.Tensor | None = None,
                    q_valid: int | None = None, kv_valid: int | None = None,
                    scale: float | None = None) -> torch.Tensor:
    """h3attn_forward_noalloc: the dense attention step of forward() with the
    library's static workspace, for callers that cannot allocate. The caller
    passes the output `out` [B, Sq, H, 128] bf16; nothing is allocated here
    either. Sizes whose workspace exceeds NOALLOC_SCRATCH_BYTES raise
    H3AttnError (ERR_WORKSPACE)."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_bshd(name, t)
    _check_f32("w_q", w_q, HEAD_DIM)
    _check_f32("w_k", w_k, HEAD_DIM)
    _check_f32("rope_cos", rope_cos)
    _check_f32("rope_sin", rope_sin)
    B, Sq, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != H or tuple(out.shape) != tuple(q.shape):
        raise ValueError("k and v must be [B, Sk, H, 128] and out like q")
    rows = 0 if rope_cos is None else rope_cos.shape[0]
    st = lib.h3attn_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Sq, k.shape[1], H, D,
                                    _ptr(w_q), _ptr(w_k), float(eps), _ptr(rope_cos), _ptr(rope_sin), rows,
                                    -1 if q_valid is None else int(q_valid),
                                    -1 if kv_valid is None else int(kv_valid),
                                    1.0 / math.sqrt(D) if scale is None else float(scale), _stream(q.device))
    _check(st, "h3attn_forward_noalloc")
    return out


def forward_ex_workspace_bytes(B: int, Sq: int, Sk: int, Hq: int, Hkv: int, causal: bool = False,
                               per_item_lengths: bool = False, window: bool = False,
                               head_dim: int = HEAD_DIM) -> int:
    """Workspace bytes h3attn_forward_ex needs for these sizes and variant."""
    a = ForwardArgs()
    a.B, a.Sq, a.Sk, a.Hq, a.Hkv, a.head_dim = B, Sq, Sk, Hq, Hkv, head_dim
    a.causal = 1 if causal else 0
    a.window_frame_rows = 1 if window else 0
    a.valid_lengths = 16 if per_item_lengths else None   # only NULL or not matters here
    return int(load_library().h3attn_forward_ex_workspace_bytes(ctypes.byref(a)))



def _check_bf16_3d(name: str, t: torch.Tensor) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda" or t.dtype != torch.bfloat16 or t.dim() != 3 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bfloat16 GPU tensor [B, rows, D] "
                         f"(got {t.dtype} {tuple(t.shape)} on {t.device})")
    if t.requires_grad and torch.is_grad_enabled():
        raise RuntimeError(f"{name} requires grad: h3attn is inference-only (no backward)")


def rmsnorm_scale_shift(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
                        index: torch.Tensor | None = None, norm_w: torch.Tensor | None = None,
                        eps: float = 1e-6, out: torch.Tensor | None = None) -> torch.Tensor:
    """Fused RMSNorm + indexed AdaLN scale/shift with the bf16 rounding of
    the unfused chain: y = bf16(bf16(n * bf16(1 + scale[i])) + shift[i]),
    n = bf16(x * r [* norm_w]), r = fp32(1/sqrt(mean x^2 + eps)), i =
    index[b, s] clamped to [0, M). x [B, S, D], scale and shift [B, M, D]
    (bf16), index int32 [B, S] or None (row 0), norm_w fp32 [D] or None.
    Pass out=x to run in place. Returns y [B, S, D] bf16."""
    lib = load_library()
    _check_bf16_3d("x", x)
    _check_bf16_3d("scale", scale)
    _check_bf16_3d("shift", shift)
    B, S, D = x.shape
    if scale.shape != shift.shape or scale.shape[0] != B or scale.shape[2] != D:
        raise ValueError("scale and shift must both be [B, M, D] with x's B and D")
    M = scale.shape[1]
    _check_f32("norm_w", norm_w, D)
    if index is not None:
        if (index.device.type != "cuda" or index.dtype != torch.int32 or tuple(index.shape) != (B, S)
                or not index.is_contiguous()):
            raise ValueError("index must be a contiguous int32 GPU tensor [B, S]")
    y = torch.empty_like(x) if out is None else out
    _check_bf16_3d("out", y)
    if y.shape != x.shape:
        raise ValueError("out must have x's shape")
    st = lib.h3attn_rmsnorm_scale_shift(_ptr(x), _ptr(y), B, S, D, _ptr(norm_w), float(eps), _ptr(scale),
                                        _ptr(shift), M, _ptr(index), _stream(x.device))
    _check(st, "h3attn_rmsnorm_scale_shift")
    return y
