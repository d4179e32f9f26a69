#!/usr/bin/env python3
"""Throughput of the exact-attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config C] [--gpus 1]

A step is one pass of the whole path over one batch of seeded synthetic
input: fa_forward (O and LSE), then the backward's three launches
(row dot products, dK/dV, dQ) when the workload trains.  The default
workload is the training step at N=8192, d=128 (B=2, H=32, bf16, causal);
--config 3 times the causal forward alone.  Inputs are resident in HBM
before the timed region starts.

Prints ONE JSON line with the throughput in credited TFLOP/s (forward
4 N^2 d per head, backward 10 N^2 d, halved for causal), the roofline of the
dominant kernel (its credited FLOPs per launch over its average duration,
timed with HIP events on the stream it runs on), and the fp64 CPU oracle
timed on a bounded sample of the same workload on this host.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s at N=8192,d=128 bf16; % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published
PEAK_F32_TFLOPS = 157.3          # MI355X fp32 MFMA, published
PEAK_FP8_TFLOPS = 5000.0         # MI355X dense fp8 MFMA, published
KV_LEN = None                    # key rows when they differ from the query rows
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ("fa_common.hpp", "fa_fwd.hip", "fa_bwd.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_io_aware_41_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, config_id: int):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when they are missing or were taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("kernel_source_hash") != kernel_source_hash():
        return None
    entry = data.get("kernels", {}).get(f"{kernel}@config{config_id}")
    if not entry:
        return None
    return entry.get("hbm_bytes_per_launch")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5])
    p.add_argument("--workload", default="attention", choices=["attention", "decode"],
                   help="attention: the --config workload (default, the headline metric); "
                        "decode: one query row per head against an 8192-position cache")
    p.add_argument("--dtype", default=None, choices=["bf16", "f16", "f32", "e4m3"],
                   help="run the --config workload in another element format (default: its "
                        "own); e4m3: FP8 inputs with per-tensor descale factors and a bf16 "
                        "output, forward workloads only")
    p.add_argument("--head-dim", type=int, default=None, choices=[64, 96, 128, 192, 256],
                   help="run the --config workload with another head dimension")
    p.add_argument("--kv-len", type=int, default=None, metavar="NK",
                   help="give keys and values NK rows instead of the queries' N (causal: query "
                        "i sees keys j <= i + NK - N)")
    p.add_argument("--packed", type=int, default=None, metavar="NSEQ",
                   help="pack NSEQ sequences of the --config workload's H, d and format, of "
                        "lengths uniform in [1, N] (one of exactly N), back to back without "
                        "padding, and time the packed entry points")
    p.add_argument("--decode-lengths", default=None, choices=[None, "zero_then_uniform"],
                   help="cached lengths of the decode workload (default: all full)")
    p.add_argument("--causal-forward-side", type=int, default=1, choices=[0, 1],
                   help="with the default training-step workload, also time the causal "
                        "B=1, H=32, N=8192 forward on its own (1, default) or not (0)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time for the oracle baseline sample (0 disables it)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="after timing, run one device-to-device copy of MIB MiB so that HBM "
                        "byte counters can be scaled against a kernel of known traffic")
    return p.parse_args()


def host_cpu():
    """(cores this process may run on, CPU model string)."""
    cores = len(os.sched_getaffinity(0))
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def blas_threads(n):
    """Context that sets the BLAS / OpenMP pools to n threads (a no-op
    context when threadpoolctl is missing)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=n)
    except ImportError:
        import contextlib
        return contextlib.nullcontext()


def timing_stats(ms):
    """Median and min of per-step (or per-launch) times in ms."""
    xs = sorted(ms)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"median": round(med, 4), "min": round(xs[0], 4), "mean": round(sum(xs) / n, 4)}


def measured_mfma(kernel: str, config_id: int):
    """MFMA utilisation of a kernel from the committed rocprofv3 counter runs
    (busy fraction of the MFMA units and executed MFMA TFLOP/s), or None when
    missing or taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("kernel_source_hash") != kernel_source_hash():
        return None
    entry = data.get("kernels", {}).get(f"{kernel}@config{config_id}") or {}
    if "mfma_busy_frac" not in entry:
        return None
    return {"mfma_busy_frac": entry["mfma_busy_frac"],
            "mfma_executed_tflops": entry.get("mfma_executed_tflops"),
            "effective_sclk_mhz": entry.get("effective_sclk_mhz")}


def cpu_baseline(cfg, inputs, budget_s):
    """Time the fp64 oracle (forward, plus backward when the workload trains)
    on whole heads of the workload until about budget_s seconds have passed."""
    import numpy as np

    import fa_inputs as fi
    import oracle

    cores, model = host_cpu()
    # batch index fastest, so that a short sample spans the batch's sequences
    # (with key lengths, not only the first sequence's heads)
    heads = [(b, h) for h in range(cfg.H) for b in range(cfg.B)]
    lengths = inputs.get("lengths")
    flops = 0
    elapsed = 0.0
    done = 0
    for (b, h) in heads:
        w = {n: fi.widen(inputs[n][b:b + 1, h:h + 1], cfg.dtype)
                * (fi.FP8_DESCALE[n] if cfg.dtype == "e4m3" else 1.0)
             for n in ("q", "k", "v", "do") if n in inputs}
        lb = None if lengths is None else np.asarray(lengths)[b:b + 1]
        t0 = time.perf_counter()
        with blas_threads(cores):
            o, lse = oracle.attention_materialised(w["q"], w["k"], w["v"], cfg.scale, cfg.causal,
                                                   lb)
            if cfg.backward:
                oracle.attention_backward(w["q"], w["k"], w["v"], o, w["do"], lse, cfg.scale,
                                          cfg.causal, lb)
        elapsed += time.perf_counter() - t0
        flops += step_flops(cfg, lb, heads=1, Nk=KV_LEN)
        done += 1
        if elapsed >= budget_s:
            break
    what = "forward+backward" if cfg.backward else "forward"
    res = {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(cores),
           "kind": "oracle", "cpu_model": model,
           "sample": f"{done} of {len(heads)} heads ({what}, fp64 materialised route, BLAS "
                     f"threads = {cores} cores of sched_getaffinity), {elapsed:.1f} s",
           "seconds": round(elapsed, 2)}
    if cfg.cid == 1 and cfg.H * cfg.B == 1:
        # the single-head workload once more on one thread
        t0 = time.perf_counter()
        with blas_threads(1):
            o, lse = oracle.attention_materialised(w["q"], w["k"], w["v"], cfg.scale, cfg.causal)
        one = time.perf_counter() - t0
        res["one_thread_value"] = flops / done / one / 1e12
    return res


def forward_bytes(cfg, Nk=None):
    """Algorithmic HBM bytes of one forward launch: Q, K and V read once, O
    and the fp32 LSE written once (K and V rows past a key length still
    counted: the padded tensors are the call's inputs)."""
    es = {"e4m3": 1, "f32": 4}.get(cfg.dtype, 2)
    out_es = 2 if cfg.dtype == "e4m3" else es
    nk = cfg.N if Nk is None else Nk
    rows_q, rows_k = cfg.B * cfg.H * cfg.N, cfg.B * cfg.H * nk
    return rows_q * cfg.d * es + 2 * rows_k * cfg.d * es + rows_q * cfg.d * out_es + rows_q * 4


def step_flops(cfg, lengths=None, heads=None, Nk=None):
    """Credited FLOPs of one step (all heads, or `heads` heads).  With Nk keys
    (Nk != N) every visible pair is counted."""
    import fa_inputs as fi
    H = cfg.H if heads is None else 1
    B = cfg.B if heads is None else heads
    if Nk is not None:
        f = fi.useful_flops(B, H, cfg.N, cfg.d, cfg.causal, lengths, Nk=Nk)
        if cfg.backward:
            f += fi.useful_flops(B, H, cfg.N, cfg.d, cfg.causal, lengths, backward=True, Nk=Nk)
        return f
    if lengths is not None:
        f = fi.useful_flops(B, H, cfg.N, cfg.d, cfg.causal, lengths)
        if cfg.backward:
            f += fi.useful_flops(B, H, cfg.N, cfg.d, cfg.causal, lengths, backward=True)
        return f
    f = fi.credited_flops(B, H, cfg.N, cfg.d, cfg.causal)
    if cfg.backward:
        f += fi.credited_flops(B, H, cfg.N, cfg.d, cfg.causal, backward=True)
    return f


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the attention path has no cross-GPU step "
              "(heads and batch shard with zero communication); run it with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_io_aware_41_amd as fa
    import fa_inputs as fi

    fa.load_library()                     # no library, no benchmark: fail loudly
    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    if args.workload == "decode":
        decode_main(args)
        return
    cfg = fi.CONFIGS[args.config]
    variant = {}
    if args.dtype is not None and args.dtype != cfg.dtype:
        variant["dtype"] = args.dtype
    if args.head_dim is not None and args.head_dim != cfg.d:
        variant["d"] = args.head_dim
    if variant:
        import dataclasses
        cfg = dataclasses.replace(cfg, **variant)
    if cfg.dtype == "e4m3" and cfg.backward:
        log("the FP8 path is a forward: use --config 1-4 with --dtype e4m3")
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.packed is not None:
        packed_main(args, cfg, dev)
        return

    t0 = time.perf_counter()
    inputs = fi.make_inputs(cfg)
    global KV_LEN
    KV_LEN = args.kv_len if args.kv_len is not None and args.kv_len != cfg.N else None
    if KV_LEN is not None:
        for n in ("k", "v"):
            inputs[n] = fi.make_tensor(cfg, n, 0, N=KV_LEN)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s: {cfg.name}"
        + (f", {KV_LEN} keys" if KV_LEN else ""))

    def up(a):
        if cfg.dtype in fi.HALF_DTYPES:
            half = torch.bfloat16 if cfg.dtype == "bf16" else torch.float16
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(half)
        return torch.from_numpy(a).to(dev)

    q, k, v = up(inputs["q"]), up(inputs["k"]), up(inputs["v"])
    do = up(inputs["do"]) if cfg.backward else None
    lens = None if inputs["lengths"] is None else torch.from_numpy(inputs["lengths"]).to(dev)
    fp8 = cfg.dtype == "e4m3"
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev) if fp8 else torch.empty_like(q)
    lse = torch.empty(cfg.B, cfg.H, cfg.N, dtype=torch.float32, device=dev)
    if cfg.backward:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
        delta = torch.empty(cfg.B, cfg.H, cfg.N, dtype=torch.float32, device=dev)

    n_ev = 5 if cfg.backward else 2

    def step(ev):
        ev[0].record()
        if fp8:
            fa.forward_fp8(q, k, v, fi.FP8_DESCALE["q"], fi.FP8_DESCALE["k"], fi.FP8_DESCALE["v"],
                           scale=cfg.scale, causal=cfg.causal, seqlens_k=lens, out=o, lse=lse)
        else:
            fa.forward(q, k, v, scale=cfg.scale, causal=cfg.causal, seqlens_k=lens, out=o,
                       lse=lse)
        ev[1].record()
        if cfg.backward:
            fa.backward_phases(q, k, v, o, do, lse, scale=cfg.scale, causal=cfg.causal,
                               seqlens_k=lens, dq=dq, dk=dk, dv=dv, delta=delta,
                               events=ev[1:5])

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for _ in range(args.warmup):
        step(mk())
    torch.cuda.synchronize()

    events = [mk() for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(events[i])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    step_ms = timing_stats([e[0].elapsed_time(e[-1]) for e in events])

    names = ["fwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq"][:n_ev - 1]
    per_kernel = {n: sum(e[i].elapsed_time(e[i + 1]) for e in events) / args.steps
                  for i, n in enumerate(names)}
    launch_ms = {n: timing_stats([e[i].elapsed_time(e[i + 1]) for e in events])
                 for i, n in enumerate(names)}
    log("per-launch ms: " + ", ".join(f"{n}={t:.4f}" for n, t in per_kernel.items())
        + f"; wall {wall * 1e3 / args.steps:.4f} ms/step")

    lengths = inputs["lengths"]
    flops = step_flops(cfg, lengths, Nk=KV_LEN)
    value = flops / (ms_per_step * 1e-3) / 1e12
    # bf16 and f16 share the dense MFMA peak; fp32 and fp8 run on their own MFMAs
    peak = {"e4m3": PEAK_FP8_TFLOPS, "f32": PEAK_F32_TFLOPS}.get(cfg.dtype, PEAK_BF16_TFLOPS)

    # credited FLOPs per launch of each compute kernel
    if KV_LEN is not None:
        fwd_f = fi.useful_flops(cfg.B, cfg.H, cfg.N, cfg.d, cfg.causal, lengths, Nk=KV_LEN)
    elif lengths is None:
        fwd_f = fi.credited_flops(cfg.B, cfg.H, cfg.N, cfg.d, cfg.causal)
    else:
        fwd_f = fi.useful_flops(cfg.B, cfg.H, cfg.N, cfg.d, cfg.causal, lengths)
    kernel_flops = {"fwd": fwd_f}
    if cfg.backward:
        kernel_flops["bwd_dkdv"] = 2 * fwd_f       # S recompute, dP, dV, dK
        kernel_flops["bwd_dq"] = fwd_f // 2        # dQ (its S/dP recompute is not credited)
    dominant = max(kernel_flops, key=lambda n: per_kernel[n])
    achieved = kernel_flops[dominant] / (per_kernel[dominant] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(achieved, 1),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": None if variant or KV_LEN else measured_traffic(dominant, args.config),
                "counters": None if variant or KV_LEN else measured_mfma(dominant, args.config)}
    # the forward's HBM rate on its algorithmic bytes (Q, K, V read once, O and
    # the LSE written once); the single-head fp32 workload (16.8 MFLOP against
    # 263 KB) is bound by latency and bytes, not by the MFMA, so its roofline
    # is the HBM one
    fwd_bytes = forward_bytes(cfg, Nk=KV_LEN)
    fwd_gbs = fwd_bytes / (per_kernel["fwd"] * 1e-3) / 1e9
    fwd_hbm = {"bytes_per_launch": fwd_bytes, "achieved_gbs": round(fwd_gbs, 1),
               "peak_gbs": PEAK_HBM_GBS, "frac": round(fwd_gbs / PEAK_HBM_GBS, 4),
               "latency_us": round(per_kernel["fwd"] * 1e3, 2)}
    if cfg.cid == 1 and not variant and KV_LEN is None:
        roofline = {"bound": "hbm", "kernel": "fwd", "achieved": fwd_hbm["achieved_gbs"],
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": fwd_hbm["frac"],
                    "traffic": measured_traffic("fwd", args.config)}

    counters = roofline.get("counters")
    extra = {
        "step_ms": step_ms,
        # the clock the dominant kernel ran at: GRBM_GUI_ACTIVE cycles per XCD
        # over the dispatch's duration in the committed counter run (the
        # runtime's clock query reports no live engine clock on this chip)
        "sclk": None if not counters else {"effective_mhz": counters.get("effective_sclk_mhz"),
                                           "kernel": dominant, "source": "rocprofv3 counters"},
        "per_launch_ms": {n: round(t, 4) for n, t in per_kernel.items()},
        "per_launch_stats_ms": launch_ms,
        "kernel_tflops": {n: round(kernel_flops[n] / (per_kernel[n] * 1e-3) / 1e12, 1)
                          for n in kernel_flops},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "fwd_hbm": fwd_hbm,
    }
    if cfg.backward:
        fwd_ms = per_kernel["fwd"]
        bwd_ms = sum(per_kernel[n] for n in names[1:])
        extra["fwd_tflops"] = round(fwd_f / (fwd_ms * 1e-3) / 1e12, 1)
        extra["bwd_tflops"] = round((flops - fwd_f) / (bwd_ms * 1e-3) / 1e12, 1)

    if args.calibrate_copy > 0:
        calibration_copy(torch, dev, args.calibrate_copy)

    if (args.config == 5 and not variant and KV_LEN is None and args.calibrate_copy == 0
            and args.causal_forward_side):
        # the causal N=8192 forward on its own (B=1, H=32): its own inputs and
        # timed region, reported beside the training step
        del inputs
        extra["causal_forward_N8192"] = causal_forward_side(args, torch, dev)

    cpu = None
    if args.cpu_seconds > 0:
        log("timing the fp64 CPU oracle on a sample ...")
        if "causal_forward_N8192" in extra:
            inputs = fi.make_inputs(cfg)
        cpu = cpu_baseline(cfg, inputs, args.cpu_seconds)

    workload = {1: "single-head non-causal forward", 2: "non-causal forward",
                3: "causal forward", 4: "causal forward with key lengths, Q x30",
                5: "causal training step (forward + backward)"}[cfg.cid]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded iid N(0,1) inputs)",
        "config": {"workload": workload, "B": cfg.B, "H": cfg.H, "N": cfg.N,
                   **({"kv_len": KV_LEN} if KV_LEN else {}), "d": cfg.d,
                   "causal": cfg.causal,
                   "key_lengths": None if lengths is None else [int(x) for x in lengths],
                   "credited_flops_per_step": flops},
        "roofline": roofline,
        "cpu_baseline": cpu,
        **extra,
    }
    print(json.dumps(line), flush=True)


def causal_forward_side(args, torch, dev):
    """Time fa_forward on the causal B=1, H=32, N=8192, d=128 bf16 workload
    with resident inputs: args.warmup untimed launches, then args.steps
    launches each bracketed by HIP events on the current stream."""
    import numpy as np

    import exact_io_aware_41_amd as fa
    import fa_inputs as fi

    cfg = fi.CONFIGS[3]
    inputs = fi.make_inputs(cfg)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
        torch.bfloat16)
    q, k, v = up(inputs["q"]), up(inputs["k"]), up(inputs["v"])
    del inputs
    o = torch.empty_like(q)
    lse = torch.empty(cfg.B, cfg.H, cfg.N, dtype=torch.float32, device=dev)

    def launch():
        fa.forward(q, k, v, scale=cfg.scale, causal=True, out=o, lse=lse)

    for _ in range(args.warmup):
        launch()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        launch()
        b.record()
    torch.cuda.synchronize()
    st = timing_stats([a.elapsed_time(b) for a, b in ev])
    flops = fi.credited_flops(cfg.B, cfg.H, cfg.N, cfg.d, True)
    tf = flops / (st["median"] * 1e-3) / 1e12
    target_ms = flops / (0.5 * PEAK_BF16_TFLOPS * 1e12) * 1e3
    log(f"causal N=8192 forward: median {st['median']:.4f} ms, min {st['min']:.4f} ms, "
        f"{tf:.1f} TFLOP/s")
    return {"config": {"B": cfg.B, "H": cfg.H, "N": cfg.N, "d": cfg.d, "causal": True,
                       "dtype": "bf16"},
            "credited_flops": flops, "launches": args.steps, "ms": st,
            "tflops_at_median": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "target_ms_at_half_peak": round(target_ms, 4),
            "counters": measured_mfma("fwd", 3)}


def packed_main(args, cfg, dev):
    """Packed batch of variable-length sequences: fa_forward_varlen (and
    fa_backward_varlen when the workload trains) over [H, total, d] tensors.
    Credited FLOPs count visible pairs only (4d forward, 10d backward), so
    the figure is comparable with the padded workload's."""
    import numpy as np
    import torch

    import exact_io_aware_41_amd as fa
    import fa_inputs as fi
    import oracle

    if args.packed < 1 or cfg.dtype == "e4m3":
        log("--packed needs at least one sequence and a bf16, f16 or f32 workload")
        sys.exit(2)
    lens = fi.packed_lengths(args.packed, cfg.N, seed=0, empty_first=False)
    cu = fi.offsets(lens)
    total = int(cu[-1])
    t0 = time.perf_counter()
    names = ["q", "k", "v"] + (["do"] if cfg.backward else [])
    host = {n: fi.make_packed(cfg, n, lens, 0) for n in names}
    log(f"packed inputs generated in {time.perf_counter() - t0:.1f} s: {len(lens)} sequences, "
        f"{total} rows per head, longest {int(lens.max())}")

    def up(a):
        if cfg.dtype in fi.HALF_DTYPES:
            half = torch.bfloat16 if cfg.dtype == "bf16" else torch.float16
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(half)
        return torch.from_numpy(a).to(dev)

    t = {n: up(host[n]) for n in names}
    cu_d = torch.from_numpy(cu).to(dev)
    mx = int(lens.max())
    o = torch.empty_like(t["q"])
    lse = torch.empty(cfg.H, total, dtype=torch.float32, device=dev)
    if cfg.backward:
        dq, dk, dv = (torch.empty_like(t["q"]) for _ in range(3))
        ws = torch.empty(max(fa.fa_backward_workspace_size(fa.FA_DTYPE_BF16, 1, cfg.H, total,
                                                           cfg.d), 16),
                         dtype=torch.uint8, device=dev)
    n_ev = 3 if cfg.backward else 2

    def step(ev):
        ev[0].record()
        fa.forward_varlen(t["q"], t["k"], t["v"], cu_d, cu_d, mx, mx, scale=cfg.scale,
                          causal=cfg.causal, out=o, lse=lse)
        ev[1].record()
        if cfg.backward:
            fa.backward_varlen(t["q"], t["k"], t["v"], o, t["do"], lse, cu_d, cu_d, mx, mx,
                               scale=cfg.scale, causal=cfg.causal, dq=dq, dk=dk, dv=dv,
                               workspace=ws)
            ev[2].record()

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for _ in range(args.warmup):
        step(mk())
    torch.cuda.synchronize()
    events = [mk() for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(events[i])
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    groups = ["fwd", "bwd"][:n_ev - 1]
    per = {g: sum(e[i].elapsed_time(e[i + 1]) for e in events) / args.steps
           for i, g in enumerate(groups)}

    fwd_f = sum(fi.useful_flops(1, cfg.H, int(n), cfg.d, cfg.causal) for n in lens)
    group_flops = {"fwd": fwd_f}
    if cfg.backward:
        group_flops["bwd"] = sum(fi.useful_flops(1, cfg.H, int(n), cfg.d, cfg.causal,
                                                 backward=True) for n in lens)
    flops = sum(group_flops.values())
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg.dtype in fi.HALF_DTYPES else PEAK_F32_TFLOPS
    dominant = max(per, key=per.get)
    achieved = group_flops[dominant] / (per[dominant] * 1e-3) / 1e12
    label = {"fwd": "fa_fwd (one launch)", "bwd": "backward (row dots + dK/dV + dQ launches)"}
    roofline = {"bound": "mfma", "kernel": label[dominant], "achieved": round(achieved, 1),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": None}

    cpu = None
    if args.cpu_seconds > 0:
        log("timing the fp64 CPU oracle on a sample ...")
        elapsed, done_f, done = 0.0, 0, 0
        for b, n in enumerate(lens):
            for h in range(cfg.H):
                sl = slice(int(cu[b]), int(cu[b + 1]))
                w = {x: fi.widen(host[x][h:h + 1, sl][None], cfg.dtype) for x in names}
                c0 = time.perf_counter()
                with blas_threads(len(os.sched_getaffinity(0))):
                    ro, rl = oracle.attention_materialised(w["q"], w["k"], w["v"], cfg.scale,
                                                           cfg.causal)
                    if cfg.backward:
                        oracle.attention_backward(w["q"], w["k"], w["v"], ro, w["do"], rl,
                                                  cfg.scale, cfg.causal)
                elapsed += time.perf_counter() - c0
                done_f += fi.useful_flops(1, 1, int(n), cfg.d, cfg.causal)
                if cfg.backward:
                    done_f += fi.useful_flops(1, 1, int(n), cfg.d, cfg.causal, backward=True)
                done += 1
                if elapsed >= args.cpu_seconds:
                    break
            if elapsed >= args.cpu_seconds:
                break
        threads, model = host_cpu()
        cpu = {"value": done_f / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads),
               "kind": "oracle", "cpu_model": model,
               "sample": f"{done} (sequence, head) pairs of {len(lens) * cfg.H}, "
                         f"{elapsed:.1f} s", "seconds": round(elapsed, 2)}

    what = "causal " if cfg.causal else ""
    what += "training step (forward + backward)" if cfg.backward else "forward"
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded iid N(0,1) inputs)",
        "config": {"workload": f"packed variable-length {what}", "sequences": len(lens),
                   "total_rows": total, "max_len": mx, "H": cfg.H, "d": cfg.d,
                   "causal": cfg.causal, "lengths": [int(x) for x in lens],
                   "credited_flops_per_step": flops},
        "roofline": roofline, "cpu_baseline": cpu,
        "per_launch_ms": {g: round(x, 4) for g, x in per.items()},
        "group_tflops": {g: round(group_flops[g] / (per[g] * 1e-3) / 1e12, 1) for g in per},
        "pct_of_peak": round(100.0 * value / peak, 2),
    }
    print(json.dumps(line), flush=True)


def calibration_copy(torch, dev, mib):
    """One device copy of known size, so that counter readings of the kernels
    can be scaled by what the same counters read for it."""
    nbytes = mib << 20
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration copy: {nbytes} bytes read and {nbytes} bytes written")


def decode_main(args):
    """One decode step per timed step: fa_decode (split kernel + merge) over
    the decode workload, reported as HBM GB/s of the minimum traffic."""
    import numpy as np
    import torch

    import exact_io_aware_41_amd as fa
    import fa_inputs as fi

    cfg = fi.DECODE
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    inputs = fi.make_decode_inputs(cfg, lengths=args.decode_lengths)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s: {cfg.name}")
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v = up(inputs["q"]), up(inputs["k"]), up(inputs["v"])
    lengths = inputs["lengths"]
    lens = None if lengths is None else torch.from_numpy(lengths).to(dev)
    B, H, N, d = cfg.shape
    o = torch.empty_like(q)
    lse = torch.empty(B, H, dtype=torch.float32, device=dev)
    ws_bytes = fa.fa_decode_workspace_size(fa.FA_DTYPE_BF16, B, H, N, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    parts = ws_bytes // (B * H * (d + 1) * 4)
    o_parts = ws[:B * H * parts * d * 4].view(torch.float32).view(B * H, parts, d)
    lse_parts = ws[B * H * parts * d * 4:].view(torch.float32).view(B * H, parts)

    def step():
        fa.decode(q, k, v, scale=cfg.scale, seqlens_k=lens, out=o, lse=lse, workspace=ws)

    def merge_only():
        fa.merge_states(o_parts, lse_parts, dtype=torch.bfloat16, out=o.view(B * H, d),
                        lse=lse.view(B * H))

    def timed(fn, steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    for _ in range(args.warmup):
        step()
    ms_per_step = timed(step, args.steps)
    merge_ms = timed(merge_only, args.steps)
    step()
    torch.cuda.synchronize()
    split_ms = ms_per_step - merge_ms
    if args.calibrate_copy > 0:
        calibration_copy(torch, dev, args.calibrate_copy)
    nbytes = fi.decode_bytes(B, H, N, d, 2, lengths)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (split_ms * 1e-3) / 1e9
    log(f"per-launch ms: decode_split={split_ms:.4f} (by difference), merge={merge_ms:.4f}; "
        f"{parts} parts per row")

    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        threads, model = host_cpu()
        qw, kw, vw = (fi.widen(inputs[n], "bf16") for n in ("q", "k", "v"))
        done_bytes, t_cpu, heads = 0, 0.0, 0
        for b in range(B):
            for h in range(H):
                sub = None if lengths is None else lengths[b:b + 1]
                t1 = time.perf_counter()
                with blas_threads(len(os.sched_getaffinity(0))):
                    oracle.attention_decode(qw[b:b + 1, h:h + 1], kw[b:b + 1, h:h + 1],
                                            vw[b:b + 1, h:h + 1], cfg.scale, sub)
                t_cpu += time.perf_counter() - t1
                done_bytes += fi.decode_bytes(1, 1, N, d, 2, sub)
                heads += 1
                if t_cpu >= args.cpu_seconds:
                    break
            if t_cpu >= args.cpu_seconds:
                break
        cpu = {"value": round(done_bytes / t_cpu / 1e9, 3), "unit": "GB/s", "cores": threads,
               "kind": "oracle", "cpu_model": model,
               "sample": f"{heads} of {B * H} heads (fp64 decode, one score row each), "
                         f"{t_cpu:.1f} s", "seconds": round(t_cpu, 2)}

    line = {
        "metric": "decode HBM GB/s (one query row per head, 8192-position cache, d=128 bf16)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1) inputs)",
        "config": {"workload": "decode against a key/value cache (split over keys + merge)",
                   "B": B, "H": H, "N": N, "d": d, "parts_per_row": int(parts),
                   "key_lengths": None if lengths is None else [int(x) for x in lengths],
                   "bytes_per_step": int(nbytes)},
        "roofline": {"bound": "hbm", "kernel": "decode_split", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None},
        "cpu_baseline": cpu,
        "per_launch_ms": {"decode_split": round(split_ms, 4), "merge": round(merge_ms, 4)},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
