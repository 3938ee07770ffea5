"""Runs the fp64 oracle on a thread pool for the full-size parity tests:
one task per (head, chunk of query rows), BLAS at one thread per worker.
Heads and rows are independent in every step the oracle computes (the norm
and rotary embedding are per head and per row, attention is per head and
per query row), so the assembled result is the oracle's own. Nothing here
computes any part of the method."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import threadpoolctl

import oracle


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def forward(inp, H: int, Hkv: int | None = None, rows=None, gate_bits=None, chunk: int = 4096, **kw):
    """oracle.forward(inp.q, inp.k, inp.v, inp.w_q, inp.w_k, rows=rows,
    gate_bits=gate_bits, **kw), computed per (head, row chunk) in threads.
    kw carries eps, theta, scale and the other keyword arguments of
    oracle.forward; the result is [B, len(rows) or Sq, H, D]."""
    Hkv = H if Hkv is None else Hkv
    group = H // Hkv
    Sq = inp.q.shape[1]
    all_rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    pieces = [all_rows[i:i + chunk] for i in range(0, len(all_rows), chunk)] or [all_rows]

    def one(task):
        h, r = task
        kv = slice(h // group, h // group + 1)
        g = None if gate_bits is None else gate_bits[:, :, h:h + 1]
        return oracle.forward(inp.q[:, :, h:h + 1], inp.k[:, :, kv], inp.v[:, :, kv], inp.w_q, inp.w_k,
                              rows=pieces[r], gate_bits=g, **kw)

    tasks = [(h, r) for h in range(H) for r in range(len(pieces))]
    with threadpoolctl.threadpool_limits(1, user_api="blas"):
        with ThreadPoolExecutor(workers()) as ex:
            parts = list(ex.map(one, tasks))
    heads = [np.concatenate(parts[h * len(pieces):(h + 1) * len(pieces)], axis=1) for h in range(H)]
    return np.concatenate(heads, axis=2)
