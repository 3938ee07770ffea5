#!/usr/bin/env python3
"""Benchmark of the MiniMax-H3 attention step on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
already resident in HBM: the fused Q/K RMSNorm + partial-rotary prologue
(with the key-major copy of v) and the dense attention forward, through the
C-ABI (h3attn_forward_stages). The workload is one GPU's 6-head share of the
104,448-row packed sequence (B=1, S=104448, H=6, d=128, bf16).

Prints one JSON line. `value` is attention TFLOP/s over the whole step
(4*S^2*d*H flop per step / step time). `roofline` is the attend stage alone
(the attention kernel, plus the small kernel that merges tiles the schedule
splits across workgroups), timed with HIP events on the stream it runs on. `cpu_baseline` is the
fp64 oracle timed on this host on a bounded sample of the same workload.
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_full_traffic.json")
ATTN_SOURCE = os.path.join(ROOT, "video_dit_dense_amd", "csrc", "attn_fwd.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(ATTN_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, or None when it is missing or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


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
    """Time the fp64 oracle (as it stands) on one head and a seeded sample of
    query rows against all keys; scale the row count so the run takes about
    `target_s` seconds. Reports attention TFLOP/s of that sample."""
    import numpy as np
    import oracle
    import workloads
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([d.get("num_threads", 1) for d in info if d.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = None
    # Item 0, query head 0 and the key/value head it reads (head 0).
    q1, k1, v1 = inp.q[:1, :, :1].copy(), inp.k[:1, :, :1].copy(), inp.v[:1, :, :1].copy()
    gate1 = workloads.make_gate(wl.B, wl.Sq, wl.H, seed=wl.seed)[:1, :, :1].copy() if wl.gate else None
    theta = wl.theta if wl.rope else None
    qv0, kvv0 = wl.item_lengths()[0]

    def run(n_rows):
        rows = np.sort(np.random.default_rng(99).choice(qv0, size=n_rows, replace=False))
        t0 = time.perf_counter()
        oracle.forward(q1, k1, v1, inp.w_q, inp.w_k, wl.eps, theta, wl.scale, qv0, kvv0,
                       norm=wl.norm, rows=rows, causal=wl.causal, window=wl.window or None,
                       gate_bits=gate1)
        return time.perf_counter() - t0, rows

    # Fixed cost (prologue over all rows of the head) plus a per-row cost:
    # fit t(n) = t0 + t1*n from two probes, then size the timed run.
    n1, n2 = 128, 512
    ta, _ = run(n1)
    tb, _ = run(n2)
    per_row = max((tb - ta) / (n2 - n1), 1e-6)
    fixed = max(ta - per_row * n1, 0.0)
    n = int(min(qv0, max(n2, (target_s - fixed) / per_row)))
    t, rows = run(n)
    if wl.window:
        keys = window_keys_per_row(wl, rows)
    else:
        keys = np.minimum(rows + 1, kvv0) if wl.causal else np.full(len(rows), kvv0)
    flops = 4.0 * float(keys.sum()) * wl.head_dim
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": threads if threads is not None else len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"fp64 NumPy oracle, item 0, head 0 of {wl.H}, {n} of {qv0} query rows against "
                  f"{'their causal prefix of ' if wl.causal else 'their frame window of ' if wl.window else 'all '}"
                  f"{kvv0} keys, prologue included, "
                  f"{t:.1f} s wall",
        "seconds": t,
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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="full",
                    help="workload name (default: full); also the attention variants "
                         + ", ".join(sorted(__import__("workloads").VARIANT_WORKLOADS))
                         + " and the RMSNorm + scale/shift shapes "
                         + ", ".join(sorted(__import__("workloads").SCALE_SHIFT_WORKLOADS)))
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-baseline duration")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prologue-reps", type=int, default=20)
    ap.add_argument("--only", choices=["all", "attention", "copy"], default="all",
                    help="for profiler runs: 'attention' runs one prepare stage, then only the attention "
                         "stage (warmup + steps launches); 'copy' runs a plain 1 GiB device copy "
                         "(warmup + steps times) to calibrate HBM byte counters")
    args = ap.parse_args()

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

    achieved = flops / (attn_avg * 1e-3) / 1e12
    # The committed counters were taken on the full workload only.
    traffic = measured_traffic() if wl.name == "full" else None
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
            "step": "prepare (RMSNorm+RoPE prologue, key-major v) + attention forward",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_kernel + attn_merge_kernel (attend stage)",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "avg_ms": round(attn_avg, 4),
        },
        "prologue": prologue,
        "prepare_stage_ms": round(prep_avg, 4),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle) ...")
        result["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
        log(f"cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
