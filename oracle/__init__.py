"""Plain fp64 CPU oracle for the MiniMax-H3 attention step.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this package. The HIP library never calls it, and
it shares no code, table or constant generator with the HIP library: it
computes its own rotary angles, its own normalisation and its own softmax from
the definitions, in float64, with NumPy.

What it computes, in the order the pages give (norm, then rotary, then
attention):

* Q/K RMSNorm per head over the 128 head channels (FastVideo PR #1832,
  "Summary" and "Preserve H3-specific attention behavior"; TeleFuser PR #37,
  "2.2 Fuse Q/K RMSNorm, RoPE, and Ulysses Pack", steps 1 and 3).
* Partial rotary embedding on 96 of the 128 channels, rotate-half pairs
  (j, j+48) (FastVideo PR #1832, "Preserve H3-specific attention behavior").
* Dense softmax attention over BSHD tensors at head_dim 128 (FastVideo PR
  #1832, "Summary"; non-causal for H3), with keys past a valid length
  excluded (FastVideo PR #1799, "Implementation": padding masks) and query
  rows past a valid length set to zero (TeleFuser PR #37, "2.3 Add
  fixed-valid and valid-only attention modes" and "2.4 Fuse valid-only gather
  with zero-tail merge").
* The attention variants of the FastVideo PR #1799 backend ("Implementation":
  MHA and GQA, causal attention, padding and causal masks combined): a causal
  mask (key j visible to query i iff j <= i, the lower-triangular mask of
  row indices), grouped heads (query head h reads key/value head
  h // (Hq / Hkv)), and valid lengths per batch item.
* The frame-window attention of VDN-H3 (SGLang PR #37903, "Modifications",
  hybrid_window_attn_h3: a chunk-5 / radius-1 window with anchor frames,
  dense-query rows against all keys, a softmax gate epilogue), read as a
  visibility rule over frame-major rows (`window_visible`) and a logistic
  gate per (row, head) on the attention output.

* The prologue fused with the destination-major Ulysses pack of one rank's
  sequence shard (TeleFuser PR #37, "2.2 Fuse Q/K RMSNorm, RoPE, and
  Ulysses Pack", step 4): `ulysses_pack`, rotary positions offset by the
  shard's first global row, each tensor laid out destination rank first.

Readings where the pages are silent (each pinned by a test in tests/):
per-head norm with one [128] weight shared by all heads, eps inside the square
root, weight multiplied as given; rotary frequency theta^(-2j/96) over the 96
rotated channels; 1-D positions 0..S-1; no rounding between steps. The same
holds for the frame-window geometry and the pack's chunk layout below. These
pins are worked by hand from the reading: the pages print no value for them,
so agreement with H3's own implementation on these points is parity unpinned.

The fused RMSNorm + indexed AdaLN scale/shift step has its own module,
`oracle.scale_shift`, with bf16 rounding boundaries instead of fp64 results.

Every function here is pinned by `tests/test_oracle_pins.py` against brute
force on tiny inputs, closed forms, invariants and torch's CPU float64 SDPA.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128
ROT_DIM = 96            # channels 0..95 are rotated, 96..127 pass through
HALF = ROT_DIM // 2     # 48 rotate-half pairs (j, j + 48)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns, as float64 (bf16 is the upper
    half of an IEEE float32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis (the 128 channels of one head):
    y_c = x_c / sqrt(mean_c(x_c^2) + eps) * w_c.

    Per-head extent and eps inside the root are readings of "Q/K RMSNorm"
    (FastVideo PR #1832, "Summary"); the pages print no formula."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * np.asarray(w, dtype=np.float64)


def rope_inv_freq(theta: float, rot_dim: int = ROT_DIM) -> np.ndarray:
    """Rotary frequencies theta^(-2j/rot_dim) for pairs j = 0 .. rot_dim/2-1."""
    j = np.arange(rot_dim // 2, dtype=np.float64)
    return float(theta) ** (-2.0 * j / rot_dim)


def rope_angles(positions, theta: float, rot_dim: int = ROT_DIM) -> np.ndarray:
    """phi[p, j] = position_p * theta^(-2j/rot_dim), shape [len(positions), rot_dim/2]."""
    pos = np.asarray(positions, dtype=np.float64)
    return np.multiply.outer(pos, rope_inv_freq(theta, rot_dim))


def apply_rope(y: np.ndarray, positions, theta: float, rot_dim: int = ROT_DIM) -> np.ndarray:
    """Partial rotary embedding on a [B, S, H, 128] tensor (FastVideo PR #1832,
    "Preserve H3-specific attention behavior": 96 of 128 channels rotated).

    Pair (a, b) = (y_j, y_{j+48}) at position p rotates by phi = p*theta^(-j/48):
    y'_j = a cos(phi) - b sin(phi), y'_{j+48} = b cos(phi) + a sin(phi).
    Channels rot_dim..127 are unchanged."""
    y = np.asarray(y, dtype=np.float64)
    half = rot_dim // 2
    phi = rope_angles(positions, theta, rot_dim)            # [S, half]
    c = np.cos(phi)[None, :, None, :]                       # broadcast over B and H
    s = np.sin(phi)[None, :, None, :]
    a = y[..., :half]
    b = y[..., half:rot_dim]
    out = y.copy()
    out[..., :half] = a * c - b * s
    out[..., half:rot_dim] = b * c + a * s
    return out


def qk_prologue(q_bits, k_bits, w_q, w_k, eps: float, theta: float | None,
                norm: bool = True, row_offset: int = 0):
    """The Q/K prologue of the attention step: RMSNorm, then rotary when
    `theta` is given, row s at position row_offset + s (0..S-1 for a whole
    sequence; a sequence shard starting at global row row_offset otherwise).
    Inputs are bf16 bit patterns [B, S, H, 128]; outputs are exact float64
    (no rounding)."""
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    if norm:
        q = rms_norm(q, w_q, eps)
        k = rms_norm(k, w_k, eps)
    if theta is not None:
        q = apply_rope(q, row_offset + np.arange(q.shape[1]), theta)
        k = apply_rope(k, row_offset + np.arange(k.shape[1]), theta)
    return q, k


def ulysses_pack(q_bits, k_bits, v_bits, w_q, w_k, eps: float, theta: float | None, P: int,
                 row_offset: int = 0, norm: bool = True):
    """The prologue fused with the destination-major Ulysses pack (TeleFuser
    PR #37, "2.2 Fuse Q/K RMSNorm, RoPE, and Ulysses Pack", step 4, feeding
    the all-to-all of section 2.1 that turns sequence shards into head
    shards). One rank holds rows row_offset .. row_offset + S - 1 of the
    sequence for all H heads (q, k, v bf16 bit patterns [B, S, H, 128]).
    Destination rank p gets heads p*H/P .. (p+1)*H/P - 1 of them, so each
    tensor is laid out with the destination outermost:

      send[p, b, s, j, :] = x[b, s, p*(H/P) + j, :],  x = prologue(q) or prologue(k) or v

    (the layout is a reading: the pages name the packing, not its layout).
    Returns (q_send, k_send) as exact float64 [P, B, S, H/P, 128] and v_send
    as the unchanged bf16 bit patterns in the same layout."""
    B, S, H, D = np.shape(q_bits)
    if P < 1 or H % P != 0:
        raise ValueError("the heads must split evenly over the P ranks")
    qn, kn = qk_prologue(q_bits, k_bits, w_q, w_k, eps, theta, norm=norm, row_offset=row_offset)

    def pack(x):
        return np.ascontiguousarray(np.asarray(x).reshape(B, S, P, H // P, D).transpose(2, 0, 1, 3, 4))

    return pack(qn), pack(kn), pack(np.asarray(v_bits, dtype=np.uint16))


def window_visible(rows, keys, F: int, C: int, R: int, A: int) -> np.ndarray:
    """Frame-window visibility [len(rows), len(keys)] (SGLang PR #37903,
    "Modifications", hybrid_window_attn_h3), read this way: row or key i lies
    in frame i // F; frames 0..A-1 are anchor frames; the frames after them
    form chunks of C frames, so frame f >= A is in chunk (f - A) // C (the
    chunk grid is shifted by the anchors). A query in an anchor frame is a
    dense-query row and sees every key. Any other query sees the anchor
    frames and the frames of the chunks within R of its own."""
    fi = np.asarray(rows, dtype=np.int64) // F
    fj = np.asarray(keys, dtype=np.int64) // F
    dense = fi < A
    ci = np.where(dense, 0, (fi - A) // C)
    anchor_key = fj < A
    cj = np.where(anchor_key, 0, (fj - A) // C)
    near = (~anchor_key)[None, :] & (np.abs(cj[None, :] - ci[:, None]) <= R)
    return dense[:, None] | anchor_key[None, :] | near


def sigmoid(x) -> np.ndarray:
    """The logistic function 1 / (1 + e^-x), in float64, without overflow."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def _per_batch(valid, B: int, full: int) -> list:
    """A valid length for every batch item: None means `full`, an int is
    shared by all items, a sequence gives one per item."""
    if valid is None:
        return [full] * B
    if np.ndim(valid) == 0:
        return [int(valid)] * B
    vals = [int(x) for x in valid]
    if len(vals) != B:
        raise ValueError("one valid length per batch item is needed")
    return vals


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              q_valid=None, kv_valid=None, rows=None, block: int = 256,
              causal: bool = False, window=None, gate=None) -> np.ndarray:
    """Softmax attention on BSHD float64 tensors, q [B, Sq, H, D] and k, v
    [B, Sk, Hkv, D] with H a multiple of Hkv (query head h reads key/value
    head h // (H // Hkv); Hkv = H is plain multi-head attention).

    For batch item b and query row i < q_valid[b]:
      o_i = sum_{j in V(i)} softmax_j(scale * q_i . k_j) v_j,
      V(i) = {j < kv_valid[b]}, and with `causal` also j <= i, and with
      `window` = (F, C, R, A) also window_visible(i, j); a row whose V(i)
      is empty is 0. With `gate` (float [B, Sq, H]) the output is multiplied
      by sigmoid(gate[b, i, h]) (the softmax gate epilogue);
    o_i = 0 for i >= q_valid[b]. q_valid / kv_valid are None (everything
    valid), one int for all items or one per item. With `rows` (absolute
    query row indices), only those rows are computed and the result has shape
    [B, len(rows), H, D]. Rows are processed `block` at a time so no Sq x Sk
    score matrix is held."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, H, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if H % Hkv != 0:
        raise ValueError("query heads must be a multiple of key/value heads")
    group = H // Hkv
    qv = _per_batch(q_valid, B, Sq)
    kvv = _per_batch(kv_valid, B, Sk)
    if min(kvv) < 1 and window is None:
        raise ValueError("attention needs at least one valid key")
    if causal and window is not None:
        raise ValueError("the frame window is not combined with the causal mask")
    row_idx = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, len(row_idx), H, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kh = np.ascontiguousarray(k[b, :kvv[b], h // group, :])
            vh = np.ascontiguousarray(v[b, :kvv[b], h // group, :])
            for start in range(0, len(row_idx), block):
                sel = row_idx[start:start + block]
                live = sel < qv[b]
                if not live.any():
                    continue
                qh = q[b, sel[live], h, :]
                s = (qh @ kh.T) * scale
                if causal:
                    # key j is visible to query row i iff j <= i
                    s = np.where(np.arange(kvv[b])[None, :] <= sel[live][:, None], s, -np.inf)
                if window is not None:
                    s = np.where(window_visible(sel[live], np.arange(kvv[b]), *window), s, -np.inf)
                seen = np.isfinite(s).any(axis=1) if s.shape[1] else np.zeros(len(s), dtype=bool)
                m = np.where(seen, s.max(axis=1, initial=-np.inf), 0.0)[:, None]
                p = np.exp(s - m)
                z = np.where(seen[:, None], p.sum(axis=1, keepdims=True), 1.0)
                o = np.where(seen[:, None], (p @ vh) / z, 0.0)
                if gate is not None:
                    o = o * sigmoid(np.asarray(gate, dtype=np.float64)[b, sel[live], h])[:, None]
                dst = np.arange(start, start + len(sel))[live]
                out[b, dst, h, :] = o
    return out


def forward(q_bits, k_bits, v_bits, w_q, w_k, eps: float, theta: float | None,
            scale: float, q_valid=None, kv_valid=None, norm: bool = True, rows=None,
            causal: bool = False, window=None, gate_bits=None) -> np.ndarray:
    """The whole attention step: prologue on q and k, then attention with v.
    Valid lengths, `rows`, `causal` and `window` are those of `attention`;
    `gate_bits` is the gate as bf16 bit patterns [B, Sq, H]."""
    qn, kn = qk_prologue(q_bits, k_bits, w_q, w_k, eps, theta, norm=norm)
    gate = None if gate_bits is None else bf16_bits_to_f64(gate_bits)
    return attention(qn, kn, bf16_bits_to_f64(v_bits), scale, q_valid, kv_valid,
                     rows=rows, causal=causal, window=window, gate=gate)


def compare(got_bits_or_f64, ref: np.ndarray) -> dict:
    """Error metrics of a bf16 (bit patterns) or float result against the
    fp64 reference: max-abs, relative RMS ||d||_2 / ||ref||_2, the largest
    distance in bf16 units in the last place, and the largest relative L2
    error of one row (the last axis: ||d_row||_2 / ||ref_row||_2, or
    ||d_row||_2 where the reference row is zero)."""
    got = np.asarray(got_bits_or_f64)
    if got.dtype == np.uint16:
        got = bf16_bits_to_f64(got)
    got = got.astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    nref = float(np.sqrt(np.sum(ref * ref)))
    rel_rms = float(np.sqrt(np.sum(d * d)) / nref) if nref > 0 else float(np.sqrt(np.sum(d * d)))
    # bf16 ulp of the reference value: 2^(floor(log2|x|) - 7), smallest normal spacing for 0.
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ulp = np.where(a > 0, np.exp2(np.maximum(e, -126.0) - 7.0), np.exp2(-133.0))
    dr = np.sqrt(np.sum(d * d, axis=-1)) if d.size else np.zeros(0)
    rr = np.sqrt(np.sum(ref * ref, axis=-1)) if d.size else np.zeros(0)
    row_rel = np.where(rr > 0, dr / np.where(rr > 0, rr, 1.0), dr)
    return {
        "max_abs": float(np.max(np.abs(d))) if d.size else 0.0,
        "rel_rms": rel_rms,
        "max_ulp": float(np.max(np.abs(d) / ulp)) if d.size else 0.0,
        "nonfinite": int(np.size(got) - np.count_nonzero(np.isfinite(got))),
        "row_rel_l2_max": float(np.max(row_rel)) if row_rel.size else 0.0,
    }
