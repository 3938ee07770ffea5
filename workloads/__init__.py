"""Seeded synthetic workloads for the MiniMax-H3 attention step.

This module only draws random numbers and stores them in the formats the
library consumes (bf16 bit patterns, fp32 weights). It holds none of the
method's arithmetic: no normalisation, no rotary angles, no attention. The
fp64 oracle and the HIP library both receive the arrays it returns, and
neither imports the other.

The five workloads are the shapes on which the pages run the H3 attention
step: a tiny smoke case, an 8x32x32 latent grid, a valid-front/padded-tail
packed sequence (TeleFuser PR #37, "2.3 Add fixed-valid and valid-only
attention modes"), video-to-text cross-attention (FastVideo PR #1799,
"Implementation": dense self- and cross-attention) and one GPU's 6-head
share of the ~104k-row 345-frame packed sequence under Ulysses-8 (SGLang
PR #37903, "Motivation" table).

The scale/shift workloads at the end are the shapes of the DiT block's
RMSNorm + indexed AdaLN modulation step that feeds the QKV projection.
"""
from __future__ import annotations

import dataclasses

import numpy as np

HEAD_DIM = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Sq: int
    Sk: int
    H: int
    q_valid: int          # query rows >= q_valid produce zero output
    kv_valid: int         # keys >= kv_valid are masked out
    norm: bool            # Q/K RMSNorm on
    rope: bool            # 96/128 partial rotary embedding on
    seed: int
    eps: float = 1e-6
    theta: float = 1e4
    description: str = ""
    causal: bool = False  # key j visible to query row i only if j <= i
    Hkv: int = 0          # key/value heads (0: same as H)
    lengths: tuple = ()   # per-item (q_valid, kv_valid) pairs, replacing q_valid / kv_valid
    window: tuple = ()    # (frame_rows, chunk_frames, radius, anchor_frames) of a frame window
    gate: bool = False    # a softmax gate per (row, head)
    head_dim: int = HEAD_DIM   # 64 and 256 run without the Q/K norm and rotary prologue

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def D(self) -> int:
        return self.head_dim

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    def item_lengths(self) -> list:
        """(q_valid, kv_valid) of every batch item."""
        return list(self.lengths) if self.lengths else [(self.q_valid, self.kv_valid)] * self.B

    def attention_flops(self) -> float:
        """QK^T and PV at 2 flop per multiply-add: 4 * d * H per visible
        (query, key) pair, summed over the items' valid rows and keys; under
        the causal mask row i sees min(i + 1, kv_valid) keys."""
        if self.window:
            raise ValueError("the frame window's pair count is the benchmark's to compute")
        pairs = 0
        for qv, kvv in self.item_lengths():
            if self.causal:
                m = min(qv, kvv)   # rows 0..m-1 see i + 1 keys, the rest all kv_valid
                pairs += m * (m + 1) // 2 + (qv - m) * kvv
            else:
                pairs += qv * kvv
        return 4.0 * pairs * self.head_dim * self.H

    def nominal_flops(self) -> float:
        return 4.0 * self.Sq * self.Sk * self.head_dim * self.H * self.B

    def prologue_bytes(self) -> int:
        """Compulsory HBM bytes of the stand-alone Q/K prologue: read and write
        q and k in bf16, read the fp32 cos/sin tables (48 pairs per row) when
        rotary is on, and the two fp32 weight vectors."""
        qk = 2 * 2 * self.B * (self.Sq * self.H + self.Sk * self.kv_heads) * HEAD_DIM
        tables = 2 * 4 * 48 * max(self.Sq, self.Sk) if self.rope else 0
        return qk + tables + 2 * 4 * HEAD_DIM


WORKLOADS = {
    "tiny": Workload("tiny", 1, 512, 512, 2, 512, 512, True, True, 0,
                     description="B=1 S=512 H=2 d=128, prologue on, no mask"),
    "mid": Workload("mid", 1, 8192, 8192, 8, 8192, 8192, True, True, 1,
                    description="B=1 S=8192 (8x32x32 latent grid) H=8, prologue on, no mask"),
    "padded": Workload("padded", 1, 32768, 32768, 8, 30720, 30720, True, True, 2,
                       description="B=1 S=32768, first 30720 rows valid, tail masked and zeroed, H=8"),
    "cross": Workload("cross", 1, 32760, 512, 8, 32760, 300, True, False, 3,
                      description="B=1 Sq=32760 video queries, Sk=512 text keys (300 valid), H=8, "
                                  "Q/K RMSNorm, no rotary"),
    "full": Workload("full", 1, 104448, 104448, 6, 104448, 104448, True, True, 4,
                     description="B=1 S=104448 packed rows (345 frames at 1344x768), H=6, "
                                 "prologue on, no mask"),
}

# Attention variants of the FastVideo PR #1799 backend ("Implementation":
# GQA, causal attention, padding masks), at the full workload's shape or a
# batch of unequal items. Measured beside the workloads above; not H3's own
# shapes (H3 is non-causal multi-head attention).
VARIANT_WORKLOADS = {
    "full_causal": Workload("full_causal", 1, 104448, 104448, 6, 104448, 104448, True, True, 4,
                            description="full shape with the causal mask", causal=True),
    "full_gqa": Workload("full_gqa", 1, 104448, 104448, 6, 104448, 104448, True, True, 4,
                         description="full shape, 6 query heads on 2 key/value heads", Hkv=2),
    # VDN-H3's frame-window attention (SGLang PR #37903, "Modifications"):
    # chunks of 5 frames, radius 1, one anchor frame, with the softmax gate.
    # 34 frames of 3072 rows make the 104448 rows; the pages do not give the
    # frame size.
    "full_window": Workload("full_window", 1, 104448, 104448, 6, 104448, 104448, True, True, 4,
                            description="full shape, frame window: 34 frames of 3072 rows, chunks of 5 "
                                        "frames, radius 1, 1 anchor frame, softmax gate",
                            window=(3072, 5, 1, 1), gate=True),
    # The other head dims of the FastVideo PR #1799 backend ("Implementation":
    # head dims 64, 128 and 256), at the full sequence with the head count
    # that keeps the width of one GPU's share (6 x 128 = 768 channels). The
    # Q/K norm and rotary prologue are H3's, on 128 channels, so these run
    # without them.
    "full_d64": Workload("full_d64", 1, 104448, 104448, 12, 104448, 104448, False, False, 6,
                         description="full sequence at head dim 64, 12 heads, no prologue", head_dim=64),
    "full_d256": Workload("full_d256", 1, 104448, 104448, 3, 104448, 104448, False, False, 7,
                          description="full sequence at head dim 256, 3 heads, no prologue", head_dim=256),
    # The frame window and gate at head dim 64 (12 heads, no prologue): the
    # window kernel holds four query tiles' window bounds per wave there.
    "full_window_d64": Workload("full_window_d64", 1, 104448, 104448, 12, 104448, 104448, False, False, 8,
                                description="full sequence at head dim 64, 12 heads, no prologue, the "
                                            "full_window frame window and gate",
                                window=(3072, 5, 1, 1), gate=True, head_dim=64),
    "batch_varlen": Workload("batch_varlen", 4, 32768, 32768, 8, 32768, 32768, True, True, 5,
                             description="B=4 padded to 32768 rows, items valid for 32768, 24576, "
                                         "16384 and 8192 query rows and keys, H=8",
                             lengths=((32768, 32768), (24576, 24576), (16384, 16384), (8192, 8192))),
}


@dataclasses.dataclass(frozen=True)
class PackWorkload:
    """One rank's sequence shard for the prologue fused with the
    destination-major Ulysses pack (TeleFuser PR #37, "2.2 Fuse Q/K RMSNorm,
    RoPE, and Ulysses Pack"): q, k, v [B, S_local, H, 128] holding rows
    rank*S_local .. of the sequence, packed for P ranks."""
    name: str
    B: int
    S_local: int
    H: int
    P: int
    rank: int
    seed: int
    eps: float = 1e-6
    theta: float = 1e4
    description: str = ""

    @property
    def row_offset(self) -> int:
        return self.rank * self.S_local

    def bytes(self) -> int:
        """Compulsory HBM bytes: q, k, v read and their send buffers written
        (bf16), the fp32 cos/sin table rows of the shard and the two fp32
        weight vectors."""
        return 3 * 2 * 2 * self.B * self.S_local * self.H * HEAD_DIM + 2 * 4 * 48 * self.S_local + 2 * 4 * HEAD_DIM


PACK_WORKLOADS = {
    # The 104448-row sequence over 8 ranks: each holds 13056 rows of all 48
    # heads (the head count the 6-head-per-GPU share implies) and sends 6
    # heads to every rank. Rank 3 exercises the rotary row offset.
    "pack_shard": PackWorkload("pack_shard", 1, 13056, 48, 8, 3, 30,
                               description="one rank's 13056-row shard of the 104448-row sequence, 48 heads, "
                                           "packed for 8 ranks (6 heads each), rank 3"),
}


def make_pack_inputs(wl: PackWorkload) -> Inputs:
    return make_inputs(wl.B, wl.S_local, wl.S_local, wl.H, wl.seed)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns. NaN inputs map to a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding_bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + rounding_bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Inputs:
    q: np.ndarray        # uint16 bf16 bits [B, Sq, H, 128]
    k: np.ndarray        # uint16 bf16 bits [B, Sk, H, 128]
    v: np.ndarray        # uint16 bf16 bits [B, Sk, H, 128]
    w_q: np.ndarray      # float32 [128], bf16-representable
    w_k: np.ndarray      # float32 [128], bf16-representable


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def make_inputs(B: int, Sq: int, Sk: int, H: int, seed: int,
                weight_sigma: float = 0.1, Hkv: int | None = None, D: int = HEAD_DIM) -> Inputs:
    """Draw q [B, Sq, H, D], k and v [B, Sk, Hkv, D] (Hkv defaults to H) ~
    N(0,1) (float32, then RNE to bf16) and RMSNorm weights [D] 1 +
    weight_sigma*N(0,1) (float64, rounded to bf16-representable values and
    stored as float32), in that order, from numpy's PCG64 with `seed`."""
    rng = np.random.default_rng(seed)
    Hkv = H if Hkv is None else Hkv
    q = _normal_bf16(rng, (B, Sq, H, D))
    k = _normal_bf16(rng, (B, Sk, Hkv, D))
    v = _normal_bf16(rng, (B, Sk, Hkv, D))
    w = []
    for _ in range(2):
        w64 = 1.0 + weight_sigma * rng.standard_normal(D)
        w.append(bf16_bits_to_f32(f32_to_bf16_bits(w64.astype(np.float32))))
    return Inputs(q, k, v, w[0], w[1])


def normal_bf16_rows(B: int, S: int, H: int, seed: int, D: int = HEAD_DIM,
                     chunk_rows: int = 1 << 16) -> np.ndarray:
    """A [B, S, H, D] tensor ~ N(0,1) (float32, then RNE to bf16 bits) for
    tensors of several GiB: each chunk of chunk_rows sequence rows of each
    item is drawn from its own PCG64 stream, spawned in order from `seed`
    (numpy's SeedSequence), on a thread pool. No float32 draw is held whole."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    out = np.empty((B, S, H, D), dtype=np.uint16)
    spans = [(b, s0, min(S, s0 + chunk_rows)) for b in range(B) for s0 in range(0, S, chunk_rows)]
    seeds = np.random.SeedSequence(seed).spawn(len(spans))

    def draw(i):
        b, s0, s1 = spans[i]
        out[b, s0:s1] = _normal_bf16(np.random.default_rng(seeds[i]), (s1 - s0, H, D))

    with ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        list(ex.map(draw, range(len(spans))))
    return out


def make_workload_inputs(wl: Workload, seed: int | None = None) -> Inputs:
    return make_inputs(wl.B, wl.Sq, wl.Sk, wl.H, wl.seed if seed is None else seed, Hkv=wl.kv_heads,
                       D=wl.head_dim)


def tile_rows(S: int, valid: int, tile: int, per_tile: int, seed: int) -> np.ndarray:
    """A seeded, sorted set of query rows with `per_tile` distinct rows drawn
    in every `tile`-row block below `valid` (fewer in a short last block),
    plus the first and last rows, the last valid row and the first tail row.
    An oracle that computes these rows for every head covers every (head,
    query block) tile of a launch with `tile`-row query blocks."""
    rng = np.random.default_rng(20_000 + seed)
    rows = {0, S - 1, max(valid - 1, 0), min(valid, S - 1)}
    for t0 in range(0, valid, tile):
        n = min(tile, valid - t0)
        rows.update(int(t0 + r) for r in rng.choice(n, size=min(per_tile, n), replace=False))
    return np.array(sorted(rows), dtype=np.int64)


# ------------------------------------------------- RMSNorm + indexed scale/shift

@dataclasses.dataclass(frozen=True)
class ScaleShiftWorkload:
    """Shapes of the DiT block's RMSNorm + indexed AdaLN scale/shift step
    (TeleFuser PR #37, "2.5 Fuse RMSNorm with indexed AdaLN modulation"):
    hidden states [B, S, D], M modulation rows per batch item, one index per
    token."""
    name: str
    B: int
    S: int
    D: int
    M: int
    seed: int
    weight: bool = False   # an fp32 RMSNorm weight (the usual DiT block norm has none)
    index: str = "frames"  # "frames": token s takes row s*M//S; "random": uniform; "none": no index (row 0)
    eps: float = 1e-6
    description: str = ""

    def bytes(self) -> int:
        """Compulsory HBM bytes: x read and y written (bf16), the scale and
        shift rows read once, the int32 index and the fp32 weight."""
        xy = 2 * 2 * self.B * self.S * self.D
        mod = 2 * 2 * self.B * self.M * self.D
        idx = 4 * self.B * self.S if self.index != "none" else 0
        return xy + mod + idx + (4 * self.D if self.weight else 0)


SCALE_SHIFT_WORKLOADS = {
    "ss_tiny": ScaleShiftWorkload("ss_tiny", 2, 100, 520, 3, 20, weight=True, index="random",
                                  description="B=2 S=100 D=520 (a ragged last chunk), M=3, random index, weight"),
    "ss_mid": ScaleShiftWorkload("ss_mid", 1, 4096, 3072, 8, 21,
                                 description="B=1 S=4096 D=3072, 8 frames of 512 tokens"),
    "ss_shard": ScaleShiftWorkload("ss_shard", 1, 13056, 6144, 4, 22,
                                   description="one GPU's 13056-row share of the 104448-row sequence under "
                                               "8-way sequence parallelism, hidden width 6144 (48 heads x 128), "
                                               "4 frames of modulation"),
}


@dataclasses.dataclass
class ScaleShiftInputs:
    x: np.ndarray            # uint16 bf16 bits [B, S, D]
    scale: np.ndarray        # uint16 bf16 bits [B, M, D]
    shift: np.ndarray        # uint16 bf16 bits [B, M, D]
    index: np.ndarray | None  # int32 [B, S]
    w: np.ndarray | None     # float32 [D], bf16-representable


def make_scale_shift_inputs(wl: ScaleShiftWorkload, seed: int | None = None,
                            x_sigma: float = 1.0) -> ScaleShiftInputs:
    """Draw, in this order from PCG64 with `seed`: x ~ x_sigma*N(0,1), scale
    and shift ~ 0.2*N(0,1) (float32, then RNE to bf16), the weight 1 +
    0.1*N(0,1) (bf16-representable, stored as float32) when the workload has
    one, then a uniform index when the workload asks for a random one."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    x = f32_to_bf16_bits((rng.standard_normal((wl.B, wl.S, wl.D), dtype=np.float32)
                          * np.float32(x_sigma)).astype(np.float32))
    scale = f32_to_bf16_bits(rng.standard_normal((wl.B, wl.M, wl.D), dtype=np.float32) * np.float32(0.2))
    shift = f32_to_bf16_bits(rng.standard_normal((wl.B, wl.M, wl.D), dtype=np.float32) * np.float32(0.2))
    w = None
    if wl.weight:
        w64 = 1.0 + 0.1 * rng.standard_normal(wl.D)
        w = bf16_bits_to_f32(f32_to_bf16_bits(w64.astype(np.float32)))
    if wl.index == "random":
        index = rng.integers(0, wl.M, (wl.B, wl.S)).astype(np.int32)
    elif wl.index == "frames":
        index = np.broadcast_to((np.arange(wl.S, dtype=np.int64) * wl.M // wl.S).astype(np.int32),
                                (wl.B, wl.S)).copy()
    else:
        index = None
    return ScaleShiftInputs(x, scale, shift, index, w)


def make_gate(B: int, S: int, H: int, seed: int, sigma: float = 2.0) -> np.ndarray:
    """Softmax-gate pre-activations [B, S, H] ~ sigma*N(0,1), as bf16 bits,
    from PCG64 with seed 1000 + seed (a stream of its own, so adding a gate
    leaves q, k and v unchanged)."""
    rng = np.random.default_rng(1000 + seed)
    return f32_to_bf16_bits(rng.standard_normal((B, S, H), dtype=np.float32) * np.float32(sigma))
