#!/usr/bin/env python3
"""Benchmark: fused attention forward on one MI355X.

One step = one attn_fwd launch over the whole workload (B x H heads of N x N
attention), i.e. every stage of the hot path: K/V streaming, QK^T, mask,
online softmax, rescale, PV, normalisation and LSE.

Default workload: B=2, H=16, N=16384, d=128, non-causal, bf16 Q/K/V ~ N(0,1)
from seed, scale = float32(1/sqrt(d)). Inputs are generated on the host,
uploaded once, and resident in HBM before timing starts.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value      = algorithmic TFLOP/s over exactly K timed steps (whole job);
  roofline   = the attention kernel's achieved MFMA rate (algorithmic flops per
               launch / mean launch duration from HIP events recorded on the
               launch stream) against MI355X's published dense bf16 peak;
  cpu_baseline = the fp64 oracle timed on this host on a bounded row sample
               of the same workload (a reported baseline, not a target).

--bwd times the attention backward (attn_bwd) on an attention workload: one
step = one call (three kernels), rate = 10*N^2*d*B*H algorithmic flops
(causal: visible pairs) per second against the bf16 MFMA peak.

--chunkscan times the Mamba2 ChunkScan entry (chunk_scan) on a ChunkScan
workload: one step = one call, rate = compulsory HBM bytes per second.

--mla times MLA decoding (mla_decode) on an MLA workload: one step = one call
(two kernels), rate = compulsory HBM bytes per second, MFMA rate beside it.

--decode times the split-KV decoding entry (attn_fwd_decode) on a decode
workload instead: one step = one call (partial kernel + merge kernel), and the
rate is compulsory HBM bytes per second against MI355X's 8 TB/s.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (bf16) and % of MI355X MFMA peak, N=16384 d=128"
PEAK_BF16_TFLOPS = 2500.0  # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0  # MI355X published HBM3E bandwidth
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the forward kernels and the device helpers they are built from
KERNEL_SRCS = [os.path.join(ROOT, "software_pipelined_amd", "csrc", f)
               for f in ("attn_fwd_kernels.h", "attn_fwd_variants.h", "attn_fwd_d64.hip", "attn_fwd_d128.hip",
                         "attn_fwd_d256.hip", "attn_common.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_cpu() -> dict:
    """The host the CPU baseline ran on: CPU model, logical CPUs, and the
    CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 0
    return {"cpu_model": model, "nproc": os.cpu_count() or 0, "usable_cpus": usable}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, q, k, v, target_s: float):
    """Time the fp64 oracle on a bounded, deterministic row sample."""
    import numpy as np
    from oracle import attn_oracle

    attn_oracle.build(force=False)
    threads = attn_oracle.max_threads()
    per_row_flops = 4 * cfg.d * (cfg.N if not cfg.causal else (cfg.N + 1) / 2)
    rng = np.random.default_rng(12345)
    total_rows = cfg.B * cfg.H * cfg.N
    # calibrate on a small sample, then size the timed sample to ~target_s
    calib = np.sort(rng.choice(total_rows, size=min(total_rows, 4 * threads), replace=False))
    t0 = time.perf_counter()
    attn_oracle.attn_fwd_rows(q, k, v, cfg.causal, cfg.scale, calib, threads=threads)
    dt = max(time.perf_counter() - t0, 1e-6)
    n = int(min(total_rows, max(threads, calib.size * target_s / dt)))
    rows = np.sort(rng.choice(total_rows, size=n, replace=False))
    t0 = time.perf_counter()
    attn_oracle.attn_fwd_rows(q, k, v, cfg.causal, cfg.scale, rows, threads=threads)
    dt = time.perf_counter() - t0
    if cfg.causal:
        flops = float(sum(4 * cfg.d * (int(r % cfg.N) + 1) for r in rows))
    else:
        flops = float(per_row_flops * n)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle", **host_cpu(),
            "sample": f"{n} of {total_rows} query rows (seeded uniform sample, all keys per row), "
                      f"fp64 C oracle, {dt:.1f} s wall"}


def decode_cpu_baseline(cfg, q, k, v, target_s: float):
    """Time the fp64 oracle's decoding entry on a bounded, deterministic sample
    of query rows; the rate is the compulsory bytes of those rows per second."""
    import numpy as np
    from oracle import attn_oracle

    attn_oracle.build(force=False)
    threads = attn_oracle.max_threads()
    rng = np.random.default_rng(12345)
    total_rows = cfg.B * cfg.H * cfg.Nq
    calib = np.sort(rng.choice(total_rows, size=min(total_rows, 4 * threads), replace=False))
    t0 = time.perf_counter()
    attn_oracle.attn_decode_rows(q, k, v, cfg.scale, calib, threads=threads)
    dt = max(time.perf_counter() - t0, 1e-6)
    n = int(min(total_rows, max(threads, calib.size * target_s / dt)))
    rows = np.sort(rng.choice(total_rows, size=n, replace=False))
    # a whole decode workload can take well under target_s: repeat the sample
    passes = 0
    t0 = time.perf_counter()
    while True:
        attn_oracle.attn_decode_rows(q, k, v, cfg.scale, rows, threads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= target_s:
            break
    nbytes = cfg.kv_bytes() * n / total_rows * passes
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle", **host_cpu(),
            "sample": f"{passes} pass(es) over {n} of {total_rows} query rows (seeded uniform sample, "
                      f"every cached key per row), fp64 C oracle, {dt:.1f} s wall"}


def bwd_cpu_baseline(cfg, q, k, v, do, target_s: float):
    """Time the fp64 oracle's backward on a bounded sample of query rows (dQ
    only), credited with the 6*N*d algorithmic flops of a row's dQ (S, dP and
    dQ rows; causal: visible keys only)."""
    import numpy as np
    from oracle import attn_oracle

    attn_oracle.build(force=False)
    threads = attn_oracle.max_threads()
    rng = np.random.default_rng(12345)
    total_rows = cfg.B * cfg.H * cfg.N
    calib = np.sort(rng.choice(total_rows, size=min(total_rows, 4 * threads), replace=False))
    none = np.zeros(0, dtype=np.int64)
    t0 = time.perf_counter()
    attn_oracle.attn_bwd_rows(q, k, v, do, cfg.causal, cfg.scale, calib, none, threads=threads)
    dt = max(time.perf_counter() - t0, 1e-6)
    n = int(min(total_rows, max(threads, calib.size * target_s / dt)))
    rows = np.sort(rng.choice(total_rows, size=n, replace=False))
    t0 = time.perf_counter()
    attn_oracle.attn_bwd_rows(q, k, v, do, cfg.causal, cfg.scale, rows, none, threads=threads)
    dt = time.perf_counter() - t0
    keys = [(int(r % cfg.N) + 1) if cfg.causal else cfg.N for r in rows]
    flops = float(sum(6 * cfg.d * kk for kk in keys))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle", **host_cpu(),
            "sample": f"dQ of {n} of {total_rows} query rows (seeded uniform sample), fp64 C oracle, "
                      f"{dt:.1f} s wall"}


def bwd_bench(args):
    """Attention backward (attn_bwd: statistics, dK/dV and dQ kernels) on an
    attention workload, with out and lse from attn_fwd and a seeded dO, all
    resident in HBM before timing."""
    import numpy as np
    import torch

    from software_pipelined_amd import attn, inputs

    cfg = {c.name: c for c in inputs.CONFIGS}[args.workload] if args.workload else inputs.HEADLINE
    log(f"backward workload {cfg.name}: generating inputs")
    q, k, v = inputs.gen_config(cfg)
    do = inputs.gen_dout(cfg.B, cfg.H, cfg.N, cfg.d, seed=cfg.seed)
    dev = torch.device("cuda:0")
    tq, tk, tv, tdo = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) for x in (q, k, v, do))
    scale = float(cfg.scale)
    out, lse = attn.attn_forward(tq, tk, tv, causal=cfg.causal, scale=scale)
    shape = (cfg.B, cfg.H, cfg.N, cfg.d)
    dq, dk, dv = (torch.empty(shape, dtype=torch.float32, device=dev) for _ in range(3))
    st, need = attn.attn_bwd_workspace_size(cfg.B, cfg.H, cfg.N, cfg.d)
    if st != 0:
        raise attn.AttnError(st)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)
    args_c = (tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), lse.data_ptr(), tdo.data_ptr(),
              dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cfg.B, cfg.H, cfg.N, cfg.d, int(cfg.causal), scale,
              ws.data_ptr(), ws.numel(), stream.cuda_stream)

    def step():
        st = attn.attn_bwd(*args_c)
        if st != 0:
            raise attn.AttnError(st)

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    events[0].record(stream)
    for i in range(args.steps):
        step()
        events[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    durs = [events[i].elapsed_time(events[i + 1]) for i in range(args.steps)]
    mean_ms = float(np.mean(durs))
    flops = inputs.bwd_flops(cfg)
    executed = flops * 14 // 10  # S and dP are formed in both main kernels
    achieved = flops / (mean_ms * 1e-3) / 1e12
    log(f"{cfg.name} backward: call mean {mean_ms:.3f} ms, median {float(np.median(durs)):.3f} ms; "
        f"{achieved:.1f} TFLOP/s algorithmic ({100 * achieved / PEAK_BF16_TFLOPS:.1f}% of "
        f"{PEAK_BF16_TFLOPS:.0f}); MFMA work executed {executed / (mean_ms * 1e-3) / 1e12:.1f} TFLOP/s")
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a row sample")
        cpu = bwd_cpu_baseline(cfg, q, k, v, do, args.cpu_seconds)
    print(json.dumps({
        "metric": "attention bwd TFLOP/s (bf16; algorithmic 2.5x the forward's flops) and % of MI355X "
                  "MFMA peak",
        "value": round(flops * args.steps / elapsed / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "N": cfg.N, "d": cfg.d, "causal": cfg.causal,
                   "flops_per_step": flops, "mfma_flops_executed_per_step": executed,
                   "workspace_bytes": need},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "unit_of_work": "one attn_bwd call (statistics, dK/dV and dQ kernels)",
                     "call_ms_mean": round(mean_ms, 4), "call_ms_median": round(float(np.median(durs)), 4)},
        "cpu_baseline": cpu}), flush=True)


def chunkscan_cpu_baseline(cfg, x, cb, dt, dacs, target_s: float):
    """Time the fp64 oracle's ChunkScan on a bounded, deterministic row sample;
    the rate is the compulsory bytes of those rows per second."""
    import numpy as np
    from oracle import attn_oracle

    attn_oracle.build(force=False)
    threads = attn_oracle.max_threads()
    rng = np.random.default_rng(12345)
    total_rows = cfg.B * cfg.S * cfg.H
    # grow a timed sample until it takes an eighth of target_s (small samples
    # cost more per row), then size the run for about target_s: one seeded
    # sample of rows, or whole passes over every row when they all take less
    n = min(total_rows, 64 * threads)
    while True:
        rows = np.sort(rng.choice(total_rows, size=n, replace=False))
        t0 = time.perf_counter()
        attn_oracle.chunk_scan_rows(x, cb, dt, dacs, cfg.L, rows, threads=threads)
        dt_s = max(time.perf_counter() - t0, 1e-6)
        if dt_s >= target_s / 8 or n == total_rows:
            break
        n = min(total_rows, n * 8)
    rows_per_s = n / dt_s
    passes = 1
    if total_rows / rows_per_s < target_s:
        n, passes = total_rows, max(1, int(round(target_s * rows_per_s / total_rows)))
        rows = None
    else:
        n = int(target_s * rows_per_s)
        rows = np.sort(rng.choice(total_rows, size=n, replace=False))
    t0 = time.perf_counter()
    for _ in range(passes):
        attn_oracle.chunk_scan_rows(x, cb, dt, dacs, cfg.L, rows, threads=threads)
    dt_s = time.perf_counter() - t0
    nbytes = cfg.hbm_bytes() * n / total_rows * passes
    what = (f"all {total_rows} output rows, {passes} passes" if rows is None else
            f"{n} of {total_rows} output rows (seeded uniform sample)")
    return {"value": nbytes / dt_s / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle", **host_cpu(),
            "sample": f"{what}, fp64 C oracle, {dt_s:.1f} s wall"}


def chunkscan_bench(args):
    """Mamba2 ChunkScan (chunk_scan): HBM-bound, so the rate is compulsory
    bytes (x, cb, dt, dA_cumsum read once; out written once) per call time."""
    import numpy as np
    import torch

    from software_pipelined_amd import attn, inputs

    cfgs = {c.name: c for c in inputs.CHUNKSCAN_CONFIGS}
    cfg = cfgs[args.workload] if args.workload else inputs.CHUNKSCAN_B64
    log(f"chunk scan workload {cfg.name}: generating inputs")
    x, cb, dt, dacs = inputs.gen_chunk_scan_config(cfg)
    dev = torch.device("cuda:0")
    tx, tcb = (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev) for a in (x, cb))
    tdt, tda = torch.from_numpy(dt).to(dev), torch.from_numpy(dacs).to(dev)
    out = torch.empty((cfg.B, cfg.S, cfg.H, cfg.P), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)
    args_c = (tx.data_ptr(), tcb.data_ptr(), tdt.data_ptr(), tda.data_ptr(), out.data_ptr(), cfg.B, cfg.S, cfg.H,
              cfg.P, cfg.L, stream.cuda_stream)

    def step():
        st = attn.chunk_scan(*args_c)
        if st != 0:
            raise attn.AttnError(st)

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    events[0].record(stream)
    for i in range(args.steps):
        step()
        events[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    durs = [events[i].elapsed_time(events[i + 1]) for i in range(args.steps)]
    mean_ms = float(np.mean(durs))
    nbytes = cfg.hbm_bytes()
    gbs = nbytes / (mean_ms * 1e-3) / 1e9
    log(f"{cfg.name}: call mean {mean_ms:.3f} ms, median {float(np.median(durs)):.3f} ms; {gbs:.0f} GB/s of "
        f"compulsory traffic ({100 * gbs / PEAK_HBM_GBS:.1f}% of {PEAK_HBM_GBS:.0f}); "
        f"{cfg.flops() / (mean_ms * 1e-3) / 1e12:.1f} TFLOP/s")
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a row sample")
        cpu = chunkscan_cpu_baseline(cfg, x, cb, dt, dacs, args.cpu_seconds)
    print(json.dumps({
        "metric": "Mamba2 ChunkScan: compulsory HBM bytes per second (x, cb, dt, dA_cumsum read once; out written)",
        "value": round(nbytes * args.steps / elapsed / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "S": cfg.S, "H": cfg.H, "P": cfg.P, "L": cfg.L,
                   "bytes_per_step": nbytes, "flops_per_step": cfg.flops()},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "call_ms_mean": round(mean_ms, 4), "call_ms_median": round(float(np.median(durs)), 4)},
        "cpu_baseline": cpu}), flush=True)


def mla_bench(args):
    """MLA decoding (mla_decode): reports compulsory HBM bytes per second (the
    shared cache read once) with the achieved MFMA rate beside it."""
    import numpy as np
    import torch

    from software_pipelined_amd import attn, inputs

    cfgs = {c.name: c for c in inputs.MLA_CONFIGS}
    cfg = cfgs[args.workload] if args.workload else inputs.MLA_B32
    log(f"mla workload {cfg.name}: generating inputs")
    q, kv = inputs.gen_mla(cfg.B, cfg.H, cfg.N, cfg.Dk, cfg.seed)
    dev = torch.device("cuda:0")
    tq, tkv = (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev) for a in (q, kv))
    out = torch.empty((cfg.B, cfg.H, cfg.Dv), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, cfg.H), dtype=torch.float32, device=dev)
    st, need = attn.mla_decode_workspace_size(cfg.B, cfg.H, cfg.N)
    if st != 0:
        raise attn.AttnError(st)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)
    args_c = (tq.data_ptr(), tkv.data_ptr(), out.data_ptr(), lse.data_ptr(), cfg.B, cfg.H, cfg.N, float(cfg.scale),
              ws.data_ptr(), ws.numel(), stream.cuda_stream)

    def step():
        st = attn.mla_decode(*args_c)
        if st != 0:
            raise attn.AttnError(st)

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    events[0].record(stream)
    for i in range(args.steps):
        step()
        events[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    durs = [events[i].elapsed_time(events[i + 1]) for i in range(args.steps)]
    mean_ms = float(np.mean(durs))
    nbytes = cfg.hbm_bytes()
    gbs = nbytes / (mean_ms * 1e-3) / 1e9
    tflops = cfg.flops() / (mean_ms * 1e-3) / 1e12
    log(f"{cfg.name}: call mean {mean_ms * 1e3:.1f} us, median {float(np.median(durs)) * 1e3:.1f} us; {gbs:.0f} GB/s "
        f"({100 * gbs / PEAK_HBM_GBS:.1f}% of {PEAK_HBM_GBS:.0f}); {tflops:.1f} TFLOP/s "
        f"({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of {PEAK_BF16_TFLOPS:.0f})")
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import attn_oracle
        attn_oracle.build(force=False)
        threads = attn_oracle.max_threads()
        # every head row; the whole workload takes well under the target on
        # the host, so it is evaluated repeatedly until about target seconds
        rows = np.arange(cfg.B * cfg.H)
        reps, t1 = 0, time.perf_counter()
        while True:
            attn_oracle.mla_decode_rows(q, kv, cfg.Dv, cfg.scale, rows, threads=threads)
            reps += 1
            dt_s = time.perf_counter() - t1
            if dt_s >= args.cpu_seconds:
                break
            if reps == 1 and dt_s * 2 > args.cpu_seconds:
                break
        cpu = {"value": cfg.hbm_bytes() * reps / dt_s / 1e9, "unit": "GB/s",
               "cores": int(threads), "kind": "oracle", **host_cpu(),
               "sample": f"all {rows.size} head rows, {reps} passes, fp64 C oracle, {dt_s:.1f} s wall"}
    print(json.dumps({
        "metric": "MLA decode: compulsory HBM bytes per second (q and the shared latent cache read once; out, lse "
                  "written)",
        "value": round(nbytes * args.steps / elapsed / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "N": cfg.N, "Dk": cfg.Dk, "Dv": cfg.Dv,
                   "bytes_per_step": nbytes, "flops_per_step": cfg.flops(), "workspace_bytes": need},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "mfma_tflops": round(tflops, 1), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "call_us_mean": round(mean_ms * 1e3, 2), "call_us_median": round(float(np.median(durs)) * 1e3, 2)},
        "cpu_baseline": cpu}), flush=True)


def sweep(cfg, attn, ptrs, out, lse, stream, args):
    """Time every variant for cfg's head dim. Parity gate: a variant's output
    must equal, bit for bit, that of the double-buffered simple schedule with
    the same key-block size (the per-row arithmetic depends only on that)."""
    import torch

    def run(vid):
        st = attn.attn_fwd_variant(vid, *ptrs)
        if st != 0:
            raise attn.AttnError(st)

    ids = [i for i in range(attn.attn_num_variants()) if attn.attn_variant_info(i)["head_dim"] == cfg.d]
    torch.cuda.synchronize()  # inputs were uploaded on torch's stream
    refs = {}
    for i in ids:
        name = attn.attn_variant_name(i)
        bn = attn.attn_variant_info(i)["block_n"]
        if "_st2_" in name and name.endswith("_simple") and bn not in refs:
            run(i)
            torch.cuda.synchronize()
            refs[bn] = (out.clone(), lse.clone())
            torch.cuda.synchronize()  # the clones run on torch's stream, the next kernel on ours
    flops = cfg.flops()
    results = []
    for i in ids:
        name = attn.attn_variant_name(i)
        bn = attn.attn_variant_info(i)["block_n"]
        out.fill_(float("nan"))
        torch.cuda.synchronize()  # the fill runs on torch's stream, the kernel on ours
        run(i)
        torch.cuda.synchronize()
        bad_o = int((out != refs[bn][0]).sum()) if bn in refs else -1
        bad_l = int((lse != refs[bn][1]).sum()) if bn in refs else -1
        ok = bad_o == 0 and bad_l == 0
        if not ok:
            log(f"{name}: {bad_o} O and {bad_l} LSE elements differ from the reference schedule")
            diff = (lse != refs[bn][1]).nonzero()
            log(f"  first differing LSE (b, h, row): {diff[:6].tolist()}; "
                f"got {lse[tuple(diff[0])].item() if diff.numel() else None}, "
                f"reference {refs[bn][1][tuple(diff[0])].item() if diff.numel() else None}")
        for _ in range(args.warmup):
            run(i)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(args.steps):
            run(i)
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / args.steps
        tf = flops / (ms * 1e-3) / 1e12
        log(f"{name:48s} {ms:8.4f} ms {tf:8.1f} TFLOP/s  parity {'ok' if ok else 'FAILED'}")
        results.append({"variant": name, "ms": round(ms, 4), "tflops": round(tf, 1), "parity": bool(ok)})
    good = [r for r in results if r["parity"]]
    best = max(good, key=lambda r: r["tflops"]) if good else None
    print(json.dumps({"sweep": cfg.name, "steps": args.steps, "warmup": args.warmup,
                      "default": attn.attn_variant_name(attn.attn_default_variant(cfg.d, cfg.causal)),
                      "best": best["variant"] if best else None, "results": results}), flush=True)
    if len(good) != len(results):
        sys.exit(1)


def decode_bench(args):
    """Split-KV decoding (attn_fwd_decode): HBM-bound, so the rate is compulsory
    bytes (q, k, v read once; out, lse written) per call over the call's time."""
    import numpy as np
    import torch

    from software_pipelined_amd import attn, inputs

    cfgs = {c.name: c for c in inputs.DECODE_CONFIGS}
    cfg = cfgs[args.workload] if args.workload else inputs.DECODE_B32
    log(f"decode workload {cfg.name}: generating inputs")
    q, k, v = inputs.gen_decode_config(cfg)
    dev = torch.device("cuda:0")
    dq, dk, dv = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) for x in (q, k, v))
    out = torch.empty((cfg.B, cfg.H, cfg.Nq, cfg.d), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, cfg.H, cfg.Nq), dtype=torch.float32, device=dev)
    # grouped K/V heads: the G query heads of a group are adjacent in q, out
    # and lse, so the call takes Hkv heads of G * Nq query rows
    G = cfg.H // cfg.kv_heads
    Hc, Nqc = cfg.kv_heads, G * cfg.Nq
    st, need = attn.attn_decode_workspace_size(cfg.B, Hc, Nqc, cfg.Nkv, cfg.d)
    if st != 0:
        raise attn.AttnError(st)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)
    args_c = (dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), out.data_ptr(), lse.data_ptr(),
              cfg.B, Hc, Nqc, cfg.Nkv, cfg.d, float(cfg.scale), ws.data_ptr(), ws.numel(),
              stream.cuda_stream)

    def step():
        st = attn.attn_fwd_decode(*args_c)
        if st != 0:
            raise attn.AttnError(st)

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    events[0].record(stream)
    for i in range(args.steps):
        step()
        events[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    durs = [events[i].elapsed_time(events[i + 1]) for i in range(args.steps)]
    mean_ms = float(np.mean(durs))
    nbytes = cfg.kv_bytes()
    gbs = nbytes / (mean_ms * 1e-3) / 1e9
    log(f"{cfg.name}: call mean {mean_ms * 1e3:.1f} us, median {float(np.median(durs)) * 1e3:.1f} us; "
        f"{gbs:.0f} GB/s of compulsory traffic ({100 * gbs / PEAK_HBM_GBS:.1f}% of {PEAK_HBM_GBS:.0f})")
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a row sample")
        cpu = decode_cpu_baseline(cfg, q.reshape(cfg.B, Hc, Nqc, cfg.d), k, v, args.cpu_seconds)
    print(json.dumps({
        "metric": "split-KV decode: compulsory HBM bytes per second (q, k, v read once; out, lse written)",
        "value": round(nbytes * args.steps / elapsed / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "Hkv": cfg.kv_heads, "Nq": cfg.Nq,
                   "Nkv": cfg.Nkv, "d": cfg.d,
                   "bytes_per_step": nbytes, "flops_per_step": cfg.flops(), "workspace_bytes": need},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "call_us_mean": round(mean_ms * 1e3, 2),
                     "call_us_median": round(float(np.median(durs)) * 1e3, 2),
                     "call_us_min": round(float(min(durs)) * 1e3, 2)},
        "cpu_baseline": cpu}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="workload name (default: the N=16384 d=128 one)")
    ap.add_argument("--variant", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="time every variant of the workload's head dim instead (the measured "
                         "sweep behind the defaults); each must first reproduce, bit for bit, "
                         "the double-buffered simple schedule of its key-block size")
    ap.add_argument("--decode", action="store_true",
                    help="time the split-KV decoding entry on a decode workload instead "
                         "(HBM-bound: reports GB/s of compulsory traffic)")
    ap.add_argument("--bwd", action="store_true",
                    help="time the attention backward (attn_bwd) on an attention workload instead")
    ap.add_argument("--chunkscan", action="store_true",
                    help="time the Mamba2 ChunkScan entry (chunk_scan) on a ChunkScan workload instead "
                         "(HBM-bound: reports GB/s of compulsory traffic)")
    ap.add_argument("--mla", action="store_true",
                    help="time MLA decoding (mla_decode) on an MLA workload instead")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of attention, run a plain device-to-device copy of this many "
                         "MiB per step (calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--mfma-probe", choices=("reg", "lds", "reg16", "lds16"), default=None,
                    help="instead of attention, time the library's matrix-core probe: a stream of bf16 "
                         "32x32x16 MFMAs with register operands only (reg) or one 1 KiB LDS read per MFMA (lds), "
                         "or of 16x16x32 MFMAs (reg16, lds16); two workgroups of 4 waves per CU "
                         "(--probe-blocks 256: one per CU, one wave per SIMD)")
    ap.add_argument("--probe-blocks", type=int, default=512, help="workgroups of the matrix-core probe")
    ap.add_argument("--gemm-ref", type=int, default=0,
                    help="instead of attention, time torch's bf16 matmul of two M x M matrices "
                         "(hipBLASLt): the practical MFMA ceiling on the same card and clock")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the benchmark runs on one GPU; --gpus must be 1 "
              "((batch, head) pairs would shard across GPUs with no exchange; that path is not built)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from software_pipelined_amd import attn, build as hip_build, inputs

    if args.copy_mib:
        # plain device copies: the counter calibration (fp32 -> fp32, as many
        # bytes read as written) and the practical HBM rates of the card for
        # that mix and for one byte read per two written (bf16 -> fp32, the
        # ChunkScan mix); not part of the product
        assert torch.cuda.is_available(), "bench needs a HIP device"
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        rates = {}
        src16 = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
        for name, a, nbytes in (("fp32_copy", src, 8 * n), ("bf16_to_fp32", src16, 6 * n)):
            for _ in range(args.warmup):
                dst.copy_(a)
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(args.steps):
                dst.copy_(a)
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1) / args.steps
            rates[name] = {"ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
        print(json.dumps({"copy_bytes_per_step": n * 4, "steps": args.warmup + args.steps, "rates": rates}),
              flush=True)
        return

    if args.mfma_probe:
        # the sustained matrix-core rate for a plain MFMA stream, with and
        # without LDS operand traffic, on the same card and clock as the
        # attention kernels; not part of the product path
        assert torch.cuda.is_available(), "bench needs a HIP device"
        mode = ("reg", "lds", "reg16", "lds16").index(args.mfma_probe)
        blocks, iters = args.probe_blocks, 4096
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
        stream = torch.cuda.Stream(device="cuda:0")

        def probe():
            st = attn.attn_probe_mfma(mode, blocks, iters, out.data_ptr(), stream.cuda_stream)
            if st != 0:
                raise attn.AttnError(st)

        torch.cuda.synchronize()
        for _ in range(args.warmup):
            probe()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(args.steps):
            probe()
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        flops = blocks * 4 * iters * 16 * (32768 if mode < 2 else 16384)
        tf = flops / (ms * 1e-3) / 1e12
        lds_bytes = blocks * 4 * iters * 16 * 1024 if mode in (1, 3) else 0
        print(json.dumps({"mfma_probe": args.mfma_probe, "blocks": blocks, "iters": iters, "ms": round(ms, 4),
                          "TFLOP/s": round(tf, 1), "frac_of_2500": round(tf / 2500.0, 4),
                          "lds_read_TB/s": round(lds_bytes / (ms * 1e-3) / 1e12, 2)}), flush=True)
        return

    if args.gemm_ref:
        # library GEMM reference for the MFMA roofline: same card, same power
        # and clock limits as the attention kernels; not part of the product
        assert torch.cuda.is_available(), "bench needs a HIP device"
        m = args.gemm_ref
        g = torch.Generator(device="cuda:0").manual_seed(7)
        a = torch.randn((m, m), device="cuda:0", generator=g).to(torch.bfloat16)
        b = torch.randn((m, m), device="cuda:0", generator=g).to(torch.bfloat16)
        c = torch.empty((m, m), device="cuda:0", dtype=torch.bfloat16)
        for _ in range(args.warmup):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            torch.matmul(a, b, out=c)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        tf = 2.0 * m ** 3 / (ms * 1e-3) / 1e12
        print(json.dumps({"gemm_ref": f"torch.matmul bf16 {m}x{m}x{m}", "ms_per_call": round(ms, 4),
                          "tflops": round(tf, 1), "frac_of_2500": round(tf / 2500.0, 4)}), flush=True)
        return

    if not os.path.exists(attn.LIB_PATH):
        hip_build.build_library()
    attn.load_library()
    assert torch.cuda.is_available(), "bench needs a HIP device"

    if args.decode:
        decode_bench(args)
        return
    if args.bwd:
        bwd_bench(args)
        return
    if args.chunkscan:
        chunkscan_bench(args)
        return
    if args.mla:
        mla_bench(args)
        return

    cfg = inputs.HEADLINE
    if args.workload:
        cfg = {c.name: c for c in inputs.CONFIGS}[args.workload]
    log(f"workload {cfg.name}: generating inputs")
    q, k, v = inputs.gen_config(cfg)
    dev = torch.device("cuda:0")
    dq, dk, dv = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) for x in (q, k, v))
    out = torch.empty((cfg.B, cfg.H, cfg.N, cfg.d), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)
    variant = args.variant if args.variant is not None else attn.attn_default_variant(cfg.d, cfg.causal)
    vname = attn.attn_variant_name(variant)
    scale = float(cfg.scale)
    ptrs = (dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), out.data_ptr(), lse.data_ptr(),
            cfg.B, cfg.H, cfg.N, cfg.d, int(cfg.causal), scale, stream.cuda_stream)

    if args.sweep:
        sweep(cfg, attn, ptrs, out, lse, stream, args)
        return

    def step():
        st = attn.attn_fwd_variant(variant, *ptrs)
        if st != 0:
            raise attn.AttnError(st)

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"variant {vname}: warmup done, timing {args.steps} steps")

    events = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    events[0].record(stream)
    for i in range(args.steps):
        step()
        events[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    durs = [events[i].elapsed_time(events[i + 1]) for i in range(args.steps)]  # ms
    mean_ms = float(np.mean(durs))

    flops = cfg.flops()
    value = flops * args.steps / elapsed / 1e12
    achieved = flops / (mean_ms * 1e-3) / 1e12
    log(f"{cfg.name}: {elapsed * 1e3 / args.steps:.3f} ms/step wall, kernel mean {mean_ms:.3f} ms "
        f"median {float(np.median(durs)):.3f} min {min(durs):.3f}; {achieved:.1f} TFLOP/s "
        f"({100 * achieved / PEAK_BF16_TFLOPS:.1f}% of {PEAK_BF16_TFLOPS:.0f})")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on host cores")
        cpu = cpu_baseline(cfg, q, k, v, args.cpu_seconds)
        log(f"cpu baseline: {cpu}")

    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "N": cfg.N, "d": cfg.d,
                   "causal": cfg.causal, "key_stress": cfg.key_stress, "seed": cfg.seed,
                   "variant": vname, "flops_per_step": flops, "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(cfg.name),
                     "kernel_ms_mean": round(mean_ms, 4),
                     "kernel_ms_median": round(float(np.median(durs)), 4),
                     "kernel_ms_min": round(float(min(durs)), 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
