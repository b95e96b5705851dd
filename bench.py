"""Benchmark: one data-parallel rank's ZeRO step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the W resident bf16 gradient slices of this rank's shard are reduced in
fp32 (the arithmetic of the reduce-scatter), AdamW updates the fp32 master
and moments, and the bf16 result is written straight into this rank's
positions of the flat all-gather buffer (the local half of the
all-gather).  All of it is one kernel launch of zs_step.  The layout is
built once, before timing, as a training job builds it once.

Default workload: the Llama-3-8B-shaped parameter list (291 tensors,
8,030,261,248 parameters) in 25 MiB buckets, W = 8 simulated ranks, rank 0's
shard of 1,003,782,656 parameters; gradients N(0, 1e-4) in bf16, master
N(0, 0.02), m = v = 0 at t = 1; AdamW lr 3e-4, betas 0.9/0.95, eps 1e-8,
wd 0.1.  Inputs are generated on the device before the timed region.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
PEAK_HBM_GBS = 8000.0                       # MI355X HBM3E, 8 TB/s
METRIC = ("optimizer-step params/s per GPU + achieved HBM GB/s (% of peak), "
          "8B W=8 shard")
STEP_SRC = os.path.join(ROOT, "zero_sharded_optimizer_shard_amd", "csrc",
                        "zs_step.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    return hashlib.sha256(open(STEP_SRC, "rb").read()).hexdigest()[:16]


def traffic_record(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    only if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256_16") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(W, seconds: float):
    """The oracle as it stands, single-threaded, on a bounded sample of the
    same workload: a 2^22-element window of the shard, stepped repeatedly
    until `seconds` have passed."""
    from oracle import step as O
    from synth import state as S
    n = 1 << 22
    G = S.cpu_grads(W, 0, n, 1, 1e-4)
    master, m, v = S.cpu_state(0, n, 0.02)
    hp = O.AdamW(**HP)
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.step(G, master, m, v, hp, reps + 1)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return dict(value=n * reps / el, unit="params/s", cores=1, kind="oracle",
                sample=f"{reps} steps over a {n}-element window of the rank-0 "
                       f"shard (W={W}), single-threaded C oracle, "
                       f"{el:.1f} s")


def ceiling(G, n, W, master, m, v, p, reps=10):
    """Same access pattern as the step, no arithmetic: the achievable
    bandwidth for this read/write mix on this device."""
    import torch
    import synth
    st = torch.cuda.current_stream()
    for _ in range(2):
        synth.dev_mix_stream(G, n, W, master, m, v, p, n, stream=st)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(st)
    for _ in range(reps):
        synth.dev_mix_stream(G, n, W, master, m, v, p, n, stream=st)
    ev[1].record(st)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    return (2 * W + 26) * n / (ms * 1e-3) / 1e9, ms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b",
                    choices=["llama8b", "dense7b", "gpt2", "tiny"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ceiling", action="store_true",
                    help="also time the same-mix copy kernel")
    ap.add_argument("--unfused", action="store_true",
                    help="also time step-to-shard + separate pack")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus "
              f"{args.gpus} is not supported (the W ranks are simulated on "
              f"one device)", file=sys.stderr)
        sys.exit(2)

    import torch
    import zero_sharded_optimizer_shard_amd as zs
    from synth import state as S
    from synth import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    w = wl.presets()[args.workload]
    W = w.world
    lay = zs.zs_layout_build(w.numels, W, w.rank)
    flat_n, n, nb, nc = zs.zs_layout_info(lay)
    log(f"workload {w.name}: W={W} shard={n} flat={flat_n} buckets={nb} "
        f"chunks={nc}")

    G = torch.empty((W, n), dtype=torch.bfloat16, device="cuda")
    master = torch.empty(n, dtype=torch.float32, device="cuda")
    m = torch.empty_like(master)
    v = torch.empty_like(master)
    flat = torch.zeros(flat_n, dtype=torch.bfloat16, device="cuda")
    S.dev_grads(G, W, n, 1, w.grad_sigma)
    S.dev_state(master, m, v, w.master_sigma)
    torch.cuda.synchronize()
    log("inputs resident")

    st = torch.cuda.current_stream()
    t = 0

    def one_step():
        nonlocal t
        t += 1
        zs.zs_step(lay, G, n, master, m, v, None, flat, step=t, stream=st,
                   **HP)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(st)
        one_step()
        b.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    ms_per_step = wall * 1e3 / K
    avg_ms = sum(kern_ms) / K
    bpp = 2 * W + 26
    achieved = bpp * n / (avg_ms * 1e-3) / 1e9
    log(f"zs_step: avg {avg_ms:.3f} ms  min {min(kern_ms):.3f} ms  "
        f"-> {achieved:.0f} GB/s ({achieved / PEAK_HBM_GBS:.1%} of 8 TB/s)")

    extra = {}
    if args.unfused:
        p = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for _ in range(2):
            zs.zs_step(lay, G, n, master, m, v, p, None, step=t, stream=st,
                       **HP)
            zs.zs_pack(lay, p, flat, stream=st)
        e[0].record(st)
        zs.zs_step(lay, G, n, master, m, v, p, None, step=t, stream=st, **HP)
        e[1].record(st)
        zs.zs_pack(lay, p, flat, stream=st)
        e[2].record(st)
        torch.cuda.synchronize()
        extra["unfused_ms"] = dict(step=e[0].elapsed_time(e[1]),
                                   pack=e[1].elapsed_time(e[2]))
        del p
    if args.ceiling:
        p = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        gbs, cms = ceiling(G, n, W, master, m, v, p)
        extra["same_mix_ceiling"] = dict(GBps=gbs, ms=cms,
                                         frac_of_peak=gbs / PEAK_HBM_GBS)
        log(f"same-mix ceiling: {gbs:.0f} GB/s ({cms:.3f} ms)")
        del p

    traffic = traffic_record(args.workload)
    out = {
        "metric": METRIC,
        "value": n / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name} rank-0 shard, W={W}",
                   "params_total": sum(w.numels), "shard_params": n,
                   "buckets": nb, "bucket_cap_mb": 25,
                   "bytes_per_param": bpp},
        "roofline": {"bound": "hbm", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic},
        "kernel_ms": {"avg": avg_ms, "min": min(kern_ms),
                      "max": max(kern_ms)},
        "achieved_GBps_per_step": bpp * n / (ms_per_step * 1e-3) / 1e9,
        **extra,
    }
    del G, master, m, v, flat
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(W, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
