#!/usr/bin/env python3
"""Benchmark of the MiniMax-H3 attention step on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
already resident in HBM: the fused Q/K RMSNorm + partial-rotary prologue
(with the key-major copy of v) and the attention forward, through the C-ABI
(h3attn_forward_stages). The default workload is one GPU's 6-head share of
the 104,448-row packed sequence (B=1, S=104448, H=6, d=128, bf16);
--workload names the other configurations (tiny, mid, padded, cross), the
attention variants and the RMSNorm + scale/shift shapes.

Prints one JSON line. `value` is attention TFLOP/s over the whole step
(valid-pair flops / mean step time of K back-to-back steps between two
events). `roofline` is the attend stage alone (the attention kernel, plus
the small kernel that merges tiles the schedule splits across workgroups),
timed with HIP events on the stream it runs on, against the roofline that
bounds it (the bf16 matrix cores, or HBM where the compulsory bytes take
longer, as for cross-attention), with the other roofline beside it.
`timing` adds the protocol of repeated runs with the 256 MB last-level cache
flushed by a 512 MB write before each: median, min and coefficient of
variation. `achievable` holds what the chip sustains in this run on the
matrix-core, exponential and copy microbenchmarks, beside the nominal peaks.
`cpu_baseline` is the fp64 oracle timed on this host on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "attention fwd TFLOP/s + % bf16 MFMA peak at S=104448,H=6,d=128 (1 GPU)"
# The attention kernels' source: counter summaries under profiles/ are valid
# for the hash of these files only.
ATTN_SOURCES = [os.path.join(ROOT, "video_dit_dense_amd", "csrc", f) for f in ("attn_fwd.hip", "attn_sched.h")]
FLUSH_BYTES = 512 << 20        # twice the 256 MB last-level cache (MALL)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in ATTN_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_file(name: str) -> str:
    return os.path.join(ROOT, "profiles", f"attn_fwd_{name}_traffic.json")


def measured_traffic(name: str):
    """HBM bytes per attend stage of workload `name` from its committed
    rocprofv3 counter summary, or None when it is missing or the kernel
    source changed since the counters were taken."""
    try:
        with open(traffic_file(name)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def stats(xs) -> dict:
    """Median, min, mean, max and coefficient of variation of timings (ms)."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    mean = float(a.mean())
    return {"median": round(float(np.median(a)), 5), "min": round(float(a.min()), 5), "mean": round(mean, 5),
            "max": round(float(a.max()), 5), "cv": round(float(a.std() / mean) if mean > 0 else 0.0, 5), "n": len(a)}


def host_info() -> dict:
    """Cores this process may run on and the host CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_cores": len(os.sched_getaffinity(0)), "cpu_model": model}


def achievable(device="cuda:0") -> dict:
    """What the chip sustains in this run on the microbenchmarks of
    include/h3attn_micro.h: the bf16 matrix-core rate of 16x16x32
    instructions on every SIMD and the shader clock under that load, the
    v_exp_f32 rate (one exponential per attention score), and a streaming
    copy's read + write bandwidth. Each is the median of a few launches
    timed with events, after one untimed launch."""
    import numpy as np
    import torch
    from video_dit_dense_amd import micro

    def timed(fn, reps):
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3

    mb, mi = 1024, 100000            # 4 waves per SIMD, ~20 ms per launch
    sink = torch.empty(mb * 256, dtype=torch.float32, device=device)
    clocks = torch.empty((mb * 4, 2), dtype=torch.int64, device=device)
    t_mfma = timed(lambda: micro.mfma_bf16(mb, mi, sink=sink, clocks=clocks), 5)
    c = clocks.cpu().numpy().astype(np.float64)
    clock_ghz = float(np.median(c[:, 0] / c[:, 1])) * micro.REFERENCE_CLOCK_HZ / 1e9
    mfma_tflops = mb * 4 * mi * micro.MFMA_FLOP_PER_WAVE_ITER / t_mfma / 1e12
    eb, ei = 2048, 1000
    esink = torch.empty(eb * 256, dtype=torch.float32, device=device)
    t_exp = timed(lambda: micro.exp(eb, ei, sink=esink), 3)
    exp_rate = eb * 256 * ei * micro.EXP_PER_LANE_ITER / t_exp
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: micro.copy(src, dst), 10)
    del src, dst
    return {
        "mfma_bf16_tflops": round(mfma_tflops, 1),
        "mfma_bf16_frac_of_nominal": round(mfma_tflops / PEAK_BF16_TFLOPS, 4),
        "clock_ghz_under_mfma_load": round(clock_ghz, 3),
        "exp_per_s": float(f"{exp_rate:.4g}"),
        "copy_gbs": round(2 * n / t_copy / 1e9, 1),
        "copy_frac_of_nominal": round(2 * n / t_copy / 1e9 / PEAK_HBM_GBS, 4),
        "method": "h3micro_mfma_bf16 (1024 workgroups x 4 waves x 100000 x 8 v_mfma_f32_16x16x32_bf16; clock = "
                  "s_memtime cycles / s_memrealtime ticks x 100 MHz per wave, median), h3micro_exp (2048 x 256 lanes "
                  "x 1000 x 8 v_exp_f32), h3micro_copy (1 GiB, read + write bytes); median of 5, 3 and 10 launches",
    }


def attention_bytes(wl) -> int:
    """Compulsory HBM bytes of the attention (attend stage): the valid rows
    of q and the valid keys and values read once, and o written in full
    (rows past q_valid as zeros)."""
    D = wl.head_dim
    total = 0
    for qv, kvv in wl.item_lengths():
        total += 2 * D * (qv * wl.H + 2 * kvv * wl.kv_heads + wl.Sq * wl.H)
    return total


# Most key sub-tiles (32 keys each) whose K and V^T stay resident in LDS:
# dense head-dim-128 attention over at most this many runs in one kernel
# with no ring (the launcher's rule in attn_fwd.hip).
def attend_schedule(wl, cus: int = 0) -> dict:
    """The launcher's schedule of the attend stage for workload wl on a
    device with `cus` compute units (0: this device), from the library."""
    from video_dit_dense_amd import h3attn
    return h3attn.schedule(wl.B, wl.Sq, wl.Sk, wl.H, wl.kv_heads, wl.head_dim,
                           -1 if wl.lengths else wl.q_valid, -1 if wl.lengths else wl.kv_valid,
                           causal=wl.causal, per_item_lengths=bool(wl.lengths), window=wl.window or None, cus=cus)


def attend_kernels(wl, plan: dict) -> str:
    """The kernels the attend stage launches for workload wl under `plan`
    (attend_schedule): the general mode (causal mask, per-item lengths,
    frame window) runs one tile per workgroup with no split; the resident-key
    kernel serves short key ranges; every other launch runs whole rounds and
    merges the split last round, if any."""
    D = wl.head_dim
    if plan["kernel"] == "resident":
        return "attn_resident_kernel (keys resident in LDS)"
    qt = plan["query_tiles"]
    name = f"attn_fwd_kernel<{D}, {qt}, {'true' if wl.window else 'false'}>"
    if wl.causal or wl.lengths or wl.window:
        return name + " (general mode)"
    if plan["split_tiles"]:
        return f"{name} + attn_merge_kernel<{D}, {qt}> ({plan['split_tiles']} tiles split)"
    return name


def window_keys_per_row(wl, rows):
    """Visible keys of each query row under the workload's frame window: a
    row of an anchor frame sees all kv_valid keys; another row sees the
    anchor frames plus the frames of the chunks within R of its own, cut at
    kv_valid (the geometry h3attn_forward_args documents)."""
    import numpy as np
    F, C, R, A = wl.window
    kvv = wl.kv_valid
    f = np.asarray(rows, dtype=np.int64) // F
    c = np.maximum(f - A, 0) // C
    lo = np.minimum(F * (A + C * np.maximum(c - R, 0)), kvv)
    hi = np.minimum(F * (A + C * (c + R + 1)), kvv)
    return np.where(f < A, kvv, min(A * F, kvv) + np.maximum(hi - lo, 0))


def step_flops(wl) -> float:
    """Attention flops of one step: 4*d per visible (query, key) pair."""
    if wl.window:
        import numpy as np
        pairs = float(window_keys_per_row(wl, np.arange(wl.q_valid)).sum()) * wl.B
        return 4.0 * pairs * wl.head_dim * wl.H
    return wl.attention_flops()


def cpu_baseline(wl, inp, target_s: float):
    """Time the fp64 oracle (as it stands) on a bounded sample of the
    workload that takes about `target_s` seconds, and report attention
    TFLOP/s of that sample. The unit of work is one (item, query head): its
    valid query rows against its visible keys, prologue included. When one
    unit takes longer than target_s, the sample is a seeded subset of item
    0, head 0's query rows, sized from two probes; otherwise whole units in
    order (items, then heads), cycling over the workload again if it is
    done first, until target_s has passed."""
    import numpy as np
    import oracle
    import workloads
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([d.get("num_threads", 1) for d in info if d.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = None
    theta = wl.theta if wl.rope else None
    lengths = wl.item_lengths()
    gate_all = workloads.make_gate(wl.B, wl.Sq, wl.H, seed=wl.seed) if wl.gate else None
    group = wl.H // wl.kv_heads

    def run(b, h, rows):
        """Oracle on query head h of item b for `rows`: (seconds, flops)."""
        kvh = h // group
        q1 = inp.q[b:b + 1, :, h:h + 1].copy()
        k1, v1 = inp.k[b:b + 1, :, kvh:kvh + 1].copy(), inp.v[b:b + 1, :, kvh:kvh + 1].copy()
        gate1 = gate_all[b:b + 1, :, h:h + 1].copy() if gate_all is not None else None
        qv, kvv = lengths[b]
        t0 = time.perf_counter()
        oracle.forward(q1, k1, v1, inp.w_q, inp.w_k, wl.eps, theta, wl.scale, qv, kvv,
                       norm=wl.norm, rows=rows, causal=wl.causal, window=wl.window or None,
                       gate_bits=gate1)
        t = time.perf_counter() - t0
        if wl.window:
            keys = window_keys_per_row(wl, rows)
        else:
            keys = np.minimum(rows + 1, kvv) if wl.causal else np.full(len(rows), kvv)
        return t, 4.0 * float(np.minimum(keys, kvv).sum()) * wl.head_dim

    qv0 = lengths[0][0]

    def sample(n):
        return np.sort(np.random.default_rng(99).choice(qv0, size=n, replace=False))

    # Fixed cost (prologue over all rows of the head) plus a per-row cost:
    # fit t(n) = t0 + t1*n from two probes.
    n1, n2 = min(128, qv0), min(512, qv0)
    ta, _ = run(0, 0, sample(n1))
    tb, _ = run(0, 0, sample(n2))
    per_row = max((tb - ta) / max(n2 - n1, 1), 1e-7)
    fixed = max(ta - per_row * n1, 0.0)
    n = int(min(qv0, max(n2, (target_s - fixed) / per_row)))
    if n < qv0:
        t, flops = run(0, 0, sample(n))
        what = f"item 0, head 0 of {wl.H}, {n} of {qv0} query rows"
        units = 1
    else:
        units = []
        order = [(b, h) for b in range(wl.B) for h in range(wl.H) if lengths[b][0] > 0]
        t = flops = 0.0
        while t < target_s and len(units) < 100000:
            b, h = order[len(units) % len(order)]
            dt, df = run(b, h, np.arange(lengths[b][0]))
            t, flops = t + dt, flops + df
            units.append((b, h))
        per = len(order)
        what = (f"{len(units)} whole (item, head) units of the {per} with valid rows"
                + (f" ({len(units) / per:.1f} passes over the workload)" if len(units) > per else ""))
        units = len(units)
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": threads if threads is not None else len(os.sched_getaffinity(0)),
        "cores_meaning": "BLAS threads of the one oracle process (its matrix products); the rest runs on one",
        **host_info(),
        "kind": "oracle",
        "sample": f"fp64 NumPy oracle, {what}, each against "
                  f"{'its causal prefix of the' if wl.causal else 'its frame window of the' if wl.window else 'all'}"
                  f" valid keys, prologue included, {t:.1f} s wall",
        "seconds": t,
        "units": units,
    }


SS_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scale_shift_ss_shard_traffic.json")
SS_SOURCE = os.path.join(ROOT, "video_dit_dense_amd", "csrc", "scale_shift.hip")


def ss_measured_traffic():
    """HBM bytes per scale/shift launch from the committed counter summary,
    or None when it is missing or the kernel source changed since."""
    try:
        with open(SS_TRAFFIC_FILE) as f:
            t = json.load(f)
        with open(SS_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    return t.get("hbm_bytes_per_launch") if t.get("kernel_source_sha256") == sha else None


def ss_cpu_baseline(wl, inp, target_s: float):
    """Time the oracle's bf16 chain (as it stands) on the first rows of the
    workload, sized to take about `target_s` seconds; reports GB/s of the
    same per-row byte accounting as the GPU figure."""
    import numpy as np
    from oracle import scale_shift as ss

    def run(n):
        t0 = time.perf_counter()
        idx = None if inp.index is None else inp.index[:1, :n]
        ss.rmsnorm_scale_shift(inp.x[:1, :n], inp.w, wl.eps, inp.scale[:1], inp.shift[:1], idx)
        return time.perf_counter() - t0

    n = min(wl.S, 256)
    t = run(n)
    n = int(min(wl.S, max(n, n * target_s / max(t, 1e-6))))
    t = run(n)
    row_bytes = wl.bytes() / (wl.B * wl.S)
    return {
        "value": row_bytes * n / t / 1e9,
        "unit": "GB/s",
        "cores": 1,
        **host_info(),
        "kind": "oracle",
        "sample": f"NumPy bf16-chain oracle on the first {n} of {wl.B * wl.S} rows (D={wl.D}), {t:.1f} s wall; "
                  "bytes counted as the GPU figure counts them per row",
        "seconds": t,
    }


def bench_scale_shift(args, wl) -> int:
    """Times h3attn_rmsnorm_scale_shift on a scale/shift workload: `warmup`
    untimed launches, then `steps` back-to-back launches between two HIP
    events on the current stream (the stream the launches go to)."""
    import numpy as np
    import torch
    import workloads
    from video_dit_dense_amd import h3attn

    log(f"workload {wl.name}: {wl.description}")
    inp = workloads.make_scale_shift_inputs(wl)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")

    sc, sh = dev(inp.scale), dev(inp.shift)
    idx = None if inp.index is None else torch.from_numpy(inp.index).to("cuda:0")
    w = None if inp.w is None else torch.from_numpy(inp.w).to("cuda:0")
    # Launches rotate over copies of x and y that together are at least 1 GB,
    # four times the 256 MB last-level cache, so each launch reads x from and
    # writes y to HBM, and K launches run back to back between two events.
    n_sets = min(64, max(2, -(-(1 << 30) // (2 * inp.x.nbytes))))
    xs = [dev(inp.x) for _ in range(n_sets)]
    ys = [torch.empty_like(xs[0]) for _ in range(n_sets)]

    def step(k):
        h3attn.rmsnorm_scale_shift(xs[k % n_sets], sc, sh, idx, w, wl.eps, out=ys[k % n_sets])

    for k in range(args.warmup):
        step(k)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        step(k)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    gbs = wl.bytes() / (ms * 1e-3) / 1e9
    log(f"timed {args.steps} launches over {n_sets} input/output sets: {ms * 1e3:.1f} us each, {gbs:.0f} GB/s")
    result = {
        "metric": f"RMSNorm + indexed scale/shift GB/s + % HBM peak, {wl.name}: {wl.description}",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: B={wl.B} S={wl.S} D={wl.D} M={wl.M} index={wl.index} "
                        f"weight={wl.weight} eps={wl.eps}",
            "bytes_per_step": wl.bytes(),
            "step": "one h3attn_rmsnorm_scale_shift launch",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "scale_shift_kernel",
            "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": ss_measured_traffic() if wl.name == "ss_shard" else None,
            "avg_us": round(ms * 1e3, 2),
        },
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = ss_cpu_baseline(wl, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


PACK_SOURCES = [os.path.join(ROOT, "video_dit_dense_amd", "csrc", "qk_prologue.hip")]
PACK_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qkv_pack_pack_shard_traffic.json")


def pack_measured_traffic():
    """HBM bytes per pack launch from the committed counter summary, or None
    when it is missing or the kernel source changed since."""
    try:
        with open(PACK_TRAFFIC_FILE) as f:
            t = json.load(f)
        with open(PACK_SOURCES[0], "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    return t.get("hbm_bytes_per_launch") if t.get("kernel_source_sha256") == sha else None


def pack_cpu_baseline(wl, inp, target_s: float):
    """Time oracle.ulysses_pack (as it stands) on the shard's first rows, sized
    to take about `target_s` seconds; GB/s with the GPU figure's per-row
    byte accounting."""
    import oracle

    def run(n):
        t0 = time.perf_counter()
        oracle.ulysses_pack(inp.q[:, :n], inp.k[:, :n], inp.v[:, :n], inp.w_q, inp.w_k, wl.eps, wl.theta, wl.P,
                            row_offset=wl.row_offset)
        return time.perf_counter() - t0

    n = min(wl.S_local, 256)
    t = run(n)
    n = int(min(wl.S_local, max(n, n * target_s / max(t, 1e-6))))
    t = run(n)
    row_bytes = wl.bytes() / wl.S_local
    return {
        "value": row_bytes * n / t / 1e9,
        "unit": "GB/s",
        "cores": 1,
        **host_info(),
        "kind": "oracle",
        "sample": f"fp64 NumPy oracle (ulysses_pack) on the first {n} of {wl.S_local} shard rows x {wl.H} heads, "
                  f"{t:.1f} s wall; bytes counted as the GPU figure counts them per row",
        "seconds": t,
    }


def bench_pack(args, wl) -> int:
    """Times h3attn_qkv_pack on one rank's shard: `warmup` untimed launches,
    then `steps` back-to-back launches between two HIP events on the current
    stream, rotating over two input/output sets (each ~1 GB, four times the
    last-level cache) so every launch reads from and writes to HBM; then
    flushed repetitions as for the attention."""
    import numpy as np
    import torch
    import workloads
    from video_dit_dense_amd import h3attn

    log(f"workload {wl.name}: {wl.description}")
    inp = workloads.make_pack_inputs(wl)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")

    w_q = torch.from_numpy(inp.w_q).to("cuda:0")
    w_k = torch.from_numpy(inp.w_k).to("cuda:0")
    cos, sin = h3attn.rope_tables(wl.row_offset + wl.S_local, wl.theta)
    n_sets = 2
    ins = [(dev(inp.q), dev(inp.k), dev(inp.v)) for _ in range(n_sets)]
    shape = (wl.P, wl.B, wl.S_local, wl.H // wl.P, 128)
    outs = [tuple(torch.empty(shape, dtype=torch.bfloat16, device="cuda:0") for _ in range(3)) for _ in range(n_sets)]

    def step(i):
        q, k, v = ins[i % n_sets]
        h3attn.qkv_pack(q, k, v, wl.P, wl.row_offset, w_q, w_k, wl.eps, cos, sin, out=outs[i % n_sets])

    for i in range(args.warmup):
        step(i)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    gbs = wl.bytes() / (ms * 1e-3) / 1e9
    log(f"timed {args.steps} launches: {ms * 1e3:.1f} us each, {gbs:.0f} GB/s")
    flushed = None
    if args.flush_reps > 0:
        scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda:0")
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.flush_reps)]
        for i, (a, b) in enumerate(fev):
            scratch.fill_(i & 0xFF)
            a.record()
            step(i)
            b.record()
        torch.cuda.synchronize()
        flushed = stats([a.elapsed_time(b) for a, b in fev])
    result = {
        "metric": f"Q/K prologue + destination-major Ulysses pack GB/s + % HBM peak, {wl.name}: {wl.description}",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: B={wl.B} S_local={wl.S_local} H={wl.H} P={wl.P} rank={wl.rank} "
                        f"row_offset={wl.row_offset} eps={wl.eps} theta={wl.theta}",
            "bytes_per_step": wl.bytes(),
            "step": "one h3attn_qkv_pack launch (q, k RMSNorm + 96/128 rotary, v copy, destination-major layout)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "qkv_pack_kernel",
            "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": pack_measured_traffic(),
            "avg_us": round(ms * 1e3, 2),
        },
        "timing": {"mall_flushed_ms": flushed, "flush_bytes": FLUSH_BYTES if flushed else None},
    }
    if not args.no_achievable:
        ach = achievable()
        result["achievable"] = ach
        result["roofline"]["frac_of_achievable"] = round(gbs / ach["copy_gbs"], 4)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = pack_cpu_baseline(wl, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="full",
                    help="workload name (default: full); also the attention variants "
                         + ", ".join(sorted(__import__("workloads").VARIANT_WORKLOADS))
                         + ", the RMSNorm + scale/shift shapes "
                         + ", ".join(sorted(__import__("workloads").SCALE_SHIFT_WORKLOADS))
                         + " and the prologue + Ulysses pack shard "
                         + ", ".join(sorted(__import__("workloads").PACK_WORKLOADS)))
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-baseline duration")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prologue-reps", type=int, default=20)
    ap.add_argument("--flush-reps", type=int, default=None,
                    help="repetitions timed with the last-level cache flushed before each (default: --steps; "
                         "0 for profiler runs, so the kernel trace holds the back-to-back launches only)")
    ap.add_argument("--no-achievable", action="store_true", help="skip the microbenchmarks of the achievable peaks")
    ap.add_argument("--only", choices=["all", "attention", "copy"], default="all",
                    help="for profiler runs: 'attention' runs one prepare stage, then only the attention "
                         "stage (warmup + steps launches); 'copy' runs a plain 1 GiB device copy "
                         "(warmup + steps times) to calibrate HBM byte counters")
    args = ap.parse_args()
    if args.flush_reps is None:
        args.flush_reps = args.steps

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (no sharding or "
              "collectives); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np  # noqa: F401
    import torch
    import workloads
    from video_dit_dense_amd import h3attn

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    h3attn.load_library()
    if args.only == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                          "launches": args.warmup + args.steps}), flush=True)
        return 0
    if args.workload in workloads.SCALE_SHIFT_WORKLOADS:
        return bench_scale_shift(args, workloads.SCALE_SHIFT_WORKLOADS[args.workload])
    if args.workload in workloads.PACK_WORKLOADS:
        return bench_pack(args, workloads.PACK_WORKLOADS[args.workload])
    all_wl = {**workloads.WORKLOADS, **workloads.VARIANT_WORKLOADS}
    wl = all_wl[args.workload]
    variant = args.workload in workloads.VARIANT_WORKLOADS
    log(f"workload {wl.name}: {wl.description}")
    t0 = time.perf_counter()
    inp = workloads.make_workload_inputs(wl)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")

    def dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")

    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    w_q = torch.from_numpy(inp.w_q).to("cuda:0")
    w_k = torch.from_numpy(inp.w_k).to("cuda:0")
    cos = sin = None
    if wl.rope:
        cos, sin = h3attn.rope_tables(max(wl.Sq, wl.Sk), wl.theta)
    lengths = (torch.tensor(wl.lengths, dtype=torch.int32, device="cuda:0") if wl.lengths else None)
    gate = dev(workloads.make_gate(wl.B, wl.Sq, wl.H, seed=wl.seed)) if wl.gate else None
    if variant:
        nbytes = h3attn.forward_ex_workspace_bytes(wl.B, wl.Sq, wl.Sk, wl.H, wl.kv_heads, causal=wl.causal,
                                                   window=bool(wl.window), head_dim=wl.head_dim,
                                                   per_item_lengths=lengths is not None)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    else:
        ws = h3attn.make_workspace(wl.B, wl.Sq, wl.Sk, wl.H)
    o = torch.empty_like(q)

    def stage(st):
        h3attn.forward(q, k, v, w_q if wl.norm else None, w_k if wl.norm else None, wl.eps, cos, sin,
                       q_valid=None if wl.lengths else wl.q_valid, kv_valid=None if wl.lengths else wl.kv_valid,
                       scale=wl.scale, out=o, workspace=ws, stages=st, causal=wl.causal, valid_lengths=lengths,
                       window=wl.window or None, gate=gate)

    if args.only == "attention":
        stage(h3attn.STAGE_PREPARE)
        for _ in range(args.warmup + args.steps):
            stage(h3attn.STAGE_ATTEND)
        torch.cuda.synchronize()
        print(json.dumps({"only": "attention", "workload": wl.name, "flop_per_launch": step_flops(wl),
                          "launches": args.warmup + args.steps}), flush=True)
        return 0

    for _ in range(args.warmup):
        stage(h3attn.STAGE_PREPARE)
        stage(h3attn.STAGE_ATTEND)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # The timed steps: K back-to-back steps between two events, with events
    # between the stages of each step as well.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        ev[i][0].record()
        stage(h3attn.STAGE_PREPARE)
        ev[i][1].record()
        stage(h3attn.STAGE_ATTEND)
        ev[i][2].record()
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    prep_ms = [e[0].elapsed_time(e[1]) for e in ev]
    attn_ms = [e[1].elapsed_time(e[2]) for e in ev]
    attn_avg = sum(attn_ms) / len(attn_ms)
    prep_avg = sum(prep_ms) / len(prep_ms)
    flops = step_flops(wl)
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step, attend stage {attn_avg:.3f} ms "
        f"(min {min(attn_ms):.3f}, max {max(attn_ms):.3f}), prepare {prep_avg:.3f} ms")

    # The attend stage alone, K launches back to back between two events (the
    # prepared workspace stays resident, so each launch redoes the same
    # attention): the kernels' average launch duration, which the rooflines
    # use. The per-stage events above add a few microseconds of their own to
    # every interval, which a short attend stage would count as kernel time.
    a_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    a_ev[0].record()
    for _ in range(args.steps):
        stage(h3attn.STAGE_ATTEND)
    a_ev[1].record()
    torch.cuda.synchronize()
    attn_launch_ms = a_ev[0].elapsed_time(a_ev[1]) / args.steps
    log(f"attend stage alone, {args.steps} back-to-back launches: {attn_launch_ms:.4f} ms per launch")

    # Repetitions with the last-level cache flushed before each (a 512 MB
    # write, outside the events), so no repetition finds its inputs in the
    # 256 MB MALL that the previous one left there.
    flushed = None
    if args.flush_reps > 0:
        scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda:0")
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.flush_reps)]
        for i in range(args.flush_reps):
            scratch.fill_(i & 0xFF)
            fev[i][0].record()
            stage(h3attn.STAGE_PREPARE)
            fev[i][1].record()
            stage(h3attn.STAGE_ATTEND)
            fev[i][2].record()
        torch.cuda.synchronize()
        del scratch
        flushed = {"step_ms": stats([e[0].elapsed_time(e[2]) for e in fev]),
                   "prepare_ms": stats([e[0].elapsed_time(e[1]) for e in fev]),
                   "attend_ms": stats([e[1].elapsed_time(e[2]) for e in fev])}
        log(f"MALL-flushed repetitions: attend median {flushed['attend_ms']['median']:.4f} ms, "
            f"min {flushed['attend_ms']['min']:.4f}, cv {flushed['attend_ms']['cv']:.4f}")

    # Stand-alone prologue (h3attn_qk_prologue, BSHD in, BSHD out), HBM
    # roofline; measured on the workloads whose q and k share head count and
    # valid lengths (the stand-alone entry point's contract).
    prologue = None
    if wl.kv_heads == wl.H and not wl.lengths and wl.head_dim == 128:
        qo, ko = torch.empty_like(q), torch.empty_like(k)
        for _ in range(3):
            h3attn.qk_prologue(q, k, w_q if wl.norm else None, w_k if wl.norm else None, wl.eps, cos, sin, qo, ko)
        pe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        pe[0].record()
        for _ in range(args.prologue_reps):
            h3attn.qk_prologue(q, k, w_q if wl.norm else None, w_k if wl.norm else None, wl.eps, cos, sin, qo, ko)
        pe[1].record()
        torch.cuda.synchronize()
        pro_ms = pe[0].elapsed_time(pe[1]) / args.prologue_reps
        pro_gbs = wl.prologue_bytes() / (pro_ms * 1e-3) / 1e9
        log(f"prologue: {pro_ms * 1e3:.1f} us, {pro_gbs:.0f} GB/s")
        prologue = {
            "kernel": "qk_prologue_kernel (h3attn_qk_prologue, BSHD)",
            "bound": "hbm",
            "avg_us": round(pro_ms * 1e3, 2),
            "achieved": round(pro_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(pro_gbs / PEAK_HBM_GBS, 4),
            "bytes": wl.prologue_bytes(),
        }

    # The attend stage against both rooflines; the one whose time at peak is
    # longer bounds it.
    abytes = attention_bytes(wl)
    plan = attend_schedule(wl)
    tflops = flops / (attn_launch_ms * 1e-3) / 1e12
    gbs = abytes / (attn_launch_ms * 1e-3) / 1e9
    mfma_roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "work": flops}
    hbm_roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "work": abytes}
    hbm_bound = abytes / (PEAK_HBM_GBS * 1e9) > flops / (PEAK_BF16_TFLOPS * 1e12)
    main_roof, other_roof = (hbm_roof, mfma_roof) if hbm_bound else (mfma_roof, hbm_roof)
    roofline = {
        **{k: v for k, v in main_roof.items() if k != "work"},
        "kernel": attend_kernels(wl, plan) + ", attend stage",
        "schedule": plan,
        "traffic": measured_traffic(wl.name),
        "avg_ms": round(attn_launch_ms, 4),
        "avg_ms_method": f"{args.steps} back-to-back attend-stage launches between two HIP events on the stream",
        "work_per_launch": main_roof["work"],
        "work_unit": "bytes (q, k, v valid rows read once, o written)" if hbm_bound else "flop (4*d per valid pair)",
        "other": other_roof,
    }
    ach = None
    if not args.no_achievable:
        log("achievable peaks (microbenchmarks) ...")
        ach = achievable()
        roofline["frac_of_achievable"] = round(
            (gbs / ach["copy_gbs"]) if hbm_bound else (tflops / ach["mfma_bf16_tflops"]), 4)
        log(f"achievable: {ach}")
    result = {
        "metric": METRIC if wl.name == "full" else f"attention fwd TFLOP/s + % bf16 MFMA peak, {wl.name}: {wl.description}",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: B={wl.B} Sq={wl.Sq} Sk={wl.Sk} H={wl.H} Hkv={wl.kv_heads} d={wl.head_dim} "
                        + (f"lengths={list(wl.lengths)} " if wl.lengths else f"q_valid={wl.q_valid} kv_valid={wl.kv_valid} ")
                        + f"causal={wl.causal} norm={wl.norm} rope={'96/128' if wl.rope else 'off'}",
            "flop_per_step": flops,
            "nominal_flop_per_step": wl.nominal_flops() if not wl.window else None,
            "step": "prepare (RMSNorm+RoPE prologue, key-major v) + attention forward",
        },
        "roofline": roofline,
        "timing": {
            "back_to_back": {"step_ms": stats([a + b for a, b in zip(prep_ms, attn_ms)]),
                             "prepare_ms": stats(prep_ms), "attend_ms": stats(attn_ms)},
            "attend_launches_ms": round(attn_launch_ms, 5),
            "mall_flushed": flushed,
            "flush_bytes": FLUSH_BYTES if flushed else None,
        },
        "prologue": prologue,
        "prepare_stage_ms": round(prep_avg, 4),
        "achievable": ach,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle) ...")
        result["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
        log(f"cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
