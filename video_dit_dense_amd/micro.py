"""ctypes binding of the roofline-denominator microbenchmarks declared in
include/h3attn_micro.h (argument marshalling only; the kernels live in
libh3attn.so beside the attention step). torch supplies device memory and
the current stream; each call enqueues one launch and returns its buffers."""
from __future__ import annotations

import ctypes

import torch

from . import h3attn

_P = ctypes.c_void_p
_I = ctypes.c_int32
SIGNATURES = {
    "h3micro_mfma_bf16": (ctypes.c_int, [_I, _I, _P, _P, _P]),
    "h3micro_exp": (ctypes.c_int, [_I, _I, _P, _P]),
    "h3micro_copy": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _P]),
}

# Work per launch, as the header defines it.
MFMA_FLOP_PER_WAVE_ITER = 8 * 16 * 16 * 32 * 2   # eight 16x16x32 bf16 instructions
EXP_PER_LANE_ITER = 8                            # eight v_exp_f32 per lane per iteration
REFERENCE_CLOCK_HZ = 100e6                       # s_memrealtime ticks

_lib = None


def load_library() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        lib = h3attn.load_library()
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def mfma_bf16(blocks: int, iters: int, device="cuda:0", sink=None, clocks=None):
    """One launch of the matrix-core probe (blocks x 4 waves, iters rounds
    of eight 16x16x32 bf16 instructions per wave). Returns (sink fp32
    [blocks*256], clocks int64 [blocks*4, 2] of (shader cycles, 100 MHz
    ticks) per wave)."""
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=device) if sink is None else sink
    clocks = torch.empty((blocks * 4, 2), dtype=torch.int64, device=device) if clocks is None else clocks
    st = load_library().h3micro_mfma_bf16(int(blocks), int(iters), ctypes.c_void_p(sink.data_ptr()),
                                          ctypes.c_void_p(clocks.data_ptr()), _stream(sink.device))
    h3attn._check(st, "h3micro_mfma_bf16")
    return sink, clocks


def exp(blocks: int, iters: int, device="cuda:0", sink=None):
    """One launch of the exponential probe (blocks x 256 lanes, iters rounds
    of eight v_exp_f32 per lane). Returns the fp32 sink [blocks*256]."""
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=device) if sink is None else sink
    st = load_library().h3micro_exp(int(blocks), int(iters), ctypes.c_void_p(sink.data_ptr()), _stream(sink.device))
    h3attn._check(st, "h3micro_exp")
    return sink


def copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    """One launch of the streaming copy dst <- src (same byte size, 16-byte
    multiple, contiguous, disjoint)."""
    if src.device.type != "cuda" or dst.device.type != "cuda" or not src.is_contiguous() or not dst.is_contiguous():
        raise ValueError("copy needs contiguous device tensors")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("copy needs tensors of the same byte size")
    st = load_library().h3micro_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes,
                                     _stream(src.device))
    h3attn._check(st, "h3micro_copy")
