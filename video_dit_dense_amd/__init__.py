"""MI355X-native MiniMax-H3 attention step: a C-ABI HIP library
(libh3attn.so, declared in include/h3attn.h) and its thin Python binding.

    from video_dit_dense_amd import h3attn
    cos, sin = h3attn.rope_tables(S)
    o = h3attn.forward(q, k, v, w_q, w_k, 1e-6, cos, sin)
"""
from . import h3attn  # noqa: F401

__all__ = ["h3attn"]
