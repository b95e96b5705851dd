"""Benchmark: one data-parallel rank's ZeRO step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the W resident bf16 gradient slices of this rank's shard are reduced in
fp32 (the arithmetic of the reduce-scatter), AdamW updates the fp32 master
and moments, and the bf16 result is written straight into this rank's
positions of the flat all-gather buffer (the local half of the
all-gather).  All of it is one kernel launch of zs_step.  The layout is
built once, before timing, as a training job builds it once.

Operand layouts: the optimizer state lives in the library's tiled layout
(per 8192-element tile, fp32 master | m | v), and the W gradient slices are
tile-interleaved (per tile, the W source ranks' 8192 values one after
another), the form a receive-side placement of the reduce-scatter's raw
slices would give.  The same step on plain [W][n] slices is timed too and
reported as "slices_layout".

Default workload: the Llama-3-8B-shaped parameter list (291 tensors,
8,030,261,248 parameters) in 25 MiB buckets, W = 8 simulated ranks, rank 0's
shard of 1,003,782,656 parameters; gradients N(0, 1e-4) in bf16, master
N(0, 0.02), m = v = 0 at t = 1; AdamW lr 3e-4, betas 0.9/0.95, eps 1e-8,
wd 0.1.  Inputs are generated on the device before the timed region.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
PEAK_HBM_GBS = 8000.0                       # MI355X HBM3E, 8 TB/s
METRIC_STEM = ("optimizer-step params/s per GPU + achieved HBM GB/s (% of "
               "peak), ")
SHARD_LABEL = {"llama8b": "8B W=8 shard", "dense7b": "7B dense W=64 shard",
               "gpt2": "GPT-2-small W=8 shard", "tiny": "tiny W=4 shard",
               "llama70b": "70B W=16 shard"}
METRIC = METRIC_STEM + SHARD_LABEL["llama8b"]


def metric_for(workload: str) -> str:
    """The step metric, labelled with the shard it was measured on."""
    return METRIC_STEM + SHARD_LABEL[workload]
KERNELS = os.path.join(ROOT, "zero_sharded_optimizer_shard_amd",
                       "libzs.kernels.json")
# the kernels whose HBM counters the roofline's traffic figure comes from,
# per workload: the tiled mixed-precision step in its work shape there
HEADLINE_KERNEL = ("_ZN12_GLOBAL__N_111step_kernelILi8ELb1ENS_5ShapeILi64ELi1E"
                   "Li8EEELb0EEEvNS_8StepArgsE")
STEP_KERNELS = {
    "llama8b": (HEADLINE_KERNEL, "step_kernel<8, true, Shape<64, 1, 8> >"),
    # the GPT-2-sized shard: the same kernel in a launch of 1899 tiles
    "gpt2": (HEADLINE_KERNEL, "step_kernel<8, true, Shape<64, 1, 8> >"),
    "dense7b": ("_ZN12_GLOBAL__N_111step_kernelILi64ELb1ENS_5ShapeILi64ELi1E"
                "Li64EEELb0EEEvNS_8StepArgsE",
                "step_kernel<64, true, Shape<64, 1, 64> >"),
    # the pure-bf16 step (record key <workload>_bf16)
    "llama8b_bf16": ("_ZN12_GLOBAL__N_111step_kernelILi8ELb1ENS_5ShapeILi64ELi1E"
                     "Li8EEELb1EEEvNS_8StepArgsE",
                     "step_kernel<8, true, Shape<64, 1, 8>, true>"),
    # the whole-tensor step: one group launch over the owned tensors
    "llama8b_tensors": ("_ZN12_GLOBAL__N_117group_step_kernelILi8ELb1ENS_5Shape"
                        "ILi64ELi1ELi4EEELb0EEEvNS_9GroupArgsE",
                        "group_step_kernel<8, true, Shape<64, 1, 4> >"),
    # the ZeRO-3 gather: traffic per forward (every unit's gather once)
    "llama8b_zero3": ("_ZN12_GLOBAL__N_113gather_kernelENS_10GatherArgsE",
                      "gather_kernel"),
    # the same forward on the whole-tensor layout: each tensor copied whole
    # from its owner's shard
    "llama8b_zero3_tensors": ("_ZN12_GLOBAL__N_120copy_segments_kernelENS_8"
                              "CopyArgsE", "copy_segments_kernel"),
    # gradient accumulation over k = 2 micro-batches: traffic per cycle
    # (the first-micro-batch launch and the last one); both kernels' digests
    # are checked
    "llama8b_accum": (("_ZN12_GLOBAL__N_112accum_kernelILi0EEEvNS_7AccArgsE",
                       "_ZN12_GLOBAL__N_112accum_kernelILi2EEEvNS_7AccArgsE"),
                      "accum_kernel<first> + accum_kernel<last>"),
    # the streaming step's bucket groups: traffic per full step (every
    # group launch of one pass over the buckets)
    "llama70b": ("_ZN12_GLOBAL__N_117group_step_kernelILi16ELb1ENS_5ShapeILi64"
                 "ELi1ELi16EEELb0EEEvNS_9GroupArgsE",
                 "group_step_kernel<16, true, Shape<64, 1, 16> >"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_digest(symbol: str):
    """sha256 prefix of the kernel's machine code in the built libzs.so
    (the build writes them beside the library), or None."""
    if not os.path.exists(KERNELS):
        return None
    return json.load(open(KERNELS)).get(symbol)


def traffic_record(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    only if the counters were taken on the kernel now built (same machine
    code)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    syms = rec.get("kernel_symbol", "")
    want = rec.get("kernel_sha256_16")
    if isinstance(syms, str):
        syms, want = [syms], [want]
    now = [kernel_digest(x) for x in syms]
    if None in now or now != want:
        return None
    return rec.get("bytes_per_launch")


def read_counter_csv(path: str, counter: str):
    """(kernel name, value) per dispatch from a rocprofv3 counter-collection
    CSV, in dispatch order."""
    import csv
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"],
                             float(r["Counter_Value"])))
    rows.sort()
    return [(k, v) for _, k, v in rows]


def record_traffic(fetch_csv: str, write_csv: str, n: int, W: int,
                   workload: str = "llama8b", per_step: int = 0,
                   out_path: str = None) -> dict:
    """HBM bytes per launch of the workload's step from two rocprofv3 --pmc
    runs of `bench.py --copy-calibration` (FETCH_SIZE, then WRITE_SIZE, KiB
    per dispatch), each scaled by what the same counter reads for the
    calibration copy of 4 GiB; written to profiles/traffic_<workload>.json
    with the digest of the kernel's machine code in the current build (the
    counters must have been taken on that build).  per_step > 0: the
    kernel is the streaming step's group kernel, launched per_step times per
    full step; the record is per full step (sums of per_step consecutive
    dispatches, averaged)."""
    symbol, kname = STEP_KERNELS[workload]
    pure = workload.endswith("_bf16")
    mode = workload.rsplit("_", 1)[1] if "_" in workload else ""
    if workload.endswith("_zero3_tensors"):
        mode = "zero3_tensors"
    fetch = read_counter_csv(fetch_csv, "FETCH_SIZE")
    write = read_counter_csv(write_csv, "WRITE_SIZE")
    copy_bytes = 4 << 30

    def pick(rows, pred):
        return [v for k, v in rows if pred(k)]

    is_copy = lambda k: "k_copy16" in k
    tiled = lambda k: (k.startswith("void (anonymous namespace)::step_kernel<"
                                    f"{W}, true,") and ("true>" in k) == pure)
    if mode == "zero3":         # (the profiler names a plain function
        tiled = lambda k: "(anonymous namespace)::gather_kernel(" in k
    elif mode == "zero3_tensors":
        tiled = lambda k: "(anonymous namespace)::copy_segments_kernel(" in k
    elif mode == "accum":       # without its return type)
        tiled = lambda k: "(anonymous namespace)::accum_kernel<" in k
    elif per_step or mode == "tensors":
        tiled = lambda k: (k.startswith("void (anonymous namespace)::"
                                        f"group_step_kernel<{W}, true,")
                           and "true>" not in k)
    plain = lambda k: (k.startswith("void (anonymous namespace)::step_kernel<"
                                    f"{W}, false,") and ("true>" in k) == pure)
    cf, cw = pick(fetch, is_copy), pick(write, is_copy)
    if len(cf) != 1 or len(cw) != 1:
        raise SystemExit("record-traffic: expected one calibration copy per "
                         "run")
    rs = copy_bytes / 1024 / cf[0]
    ws = copy_bytes / 1024 / cw[0]
    tf, tw = pick(fetch, tiled), pick(write, tiled)
    pf, pw = pick(fetch, plain), pick(write, plain)
    if not tf or not tw:
        raise SystemExit("record-traffic: no tiled step dispatches found")
    if per_step:
        if len(tf) % per_step or len(tw) % per_step:
            raise SystemExit(f"record-traffic: {len(tf)} / {len(tw)} group "
                             f"dispatches, not whole full steps of "
                             f"{per_step}")
        tf = [sum(tf[i:i + per_step]) for i in range(0, len(tf), per_step)]
        tw = [sum(tw[i:i + per_step]) for i in range(0, len(tw), per_step)]
    avg = lambda x: sum(x) / len(x)
    rd = avg(tf) * 1024 * rs
    wr = avg(tw) * 1024 * ws
    alg = (2 * W + (20 if pure else 26)) * n
    if mode in ("zero3", "zero3_tensors"):  # n: elements gathered per forward
        alg = 4 * n
        what = (f"zs_gather{' on the whole-tensor layout' if mode != 'zero3' else ''}, "
                f"bytes per forward of {per_step} unit gathers")
    elif mode == "accum":       # n: elements of the flat gradient buffer
        alg = (6 + 8) * n
        what = ("zs_accumulate, k = 2: bytes per cycle (first micro-batch "
                "and last)")
    elif mode == "tensors":
        what = ("zs_step on the whole-tensor layout: one group launch over "
                "the owned tensors, tiled gradients and state, flat output")
    elif per_step:
        what = ("zs_buckets_step, groups of 16 tiled buckets, tiled state, "
                f"flat output; bytes per full step of {per_step} launches")
    elif pure:
        what = ("zs_step_bf16, tiled gradients, tiled m|v state, bf16 "
                "parameters in place in the flat buffer")
    else:
        what = "zs_step, tiled gradients, tiled state, flat output"
    rec = {
        "kernel": f"{kname} ({what})",
        "workload": f"{workload}, W={W}, {n:,} elements",
        "kernel_symbol": symbol,
        "kernel_sha256_16": (kernel_digest(symbol) if isinstance(symbol, str)
                             else [kernel_digest(x) for x in symbol]),
        "copy_calibration": {"bytes_read": copy_bytes,
                             "bytes_written": copy_bytes,
                             "FETCH_SIZE_KiB": cf[0], "WRITE_SIZE_KiB": cw[0],
                             "read_scale": rs, "write_scale": ws},
        "FETCH_SIZE_KiB_per_launch": tf,
        "WRITE_SIZE_KiB_per_launch": tw,
        "bytes_read_per_launch": rd,
        "bytes_written_per_launch": wr,
        "bytes_per_launch": rd + wr,
        "algorithmic_bytes_per_launch": alg,
        "ratio_to_algorithmic": (rd + wr) / alg,
    }
    if pf and pw:
        prd, pwr = avg(pf) * 1024 * rs, avg(pw) * 1024 * ws
        rec["plain_slices"] = {"bytes_read_per_launch": prd,
                               "bytes_written_per_launch": pwr,
                               "ratio_to_algorithmic": (prd + pwr) / alg}
    if out_path is None:
        out_path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def copy_calibration():
    """One plain 4 GiB device copy (synth's k_copy16): the reference
    dispatch that scales rocprofv3's FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch
    import synth
    nbytes = 4 << 30
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    synth.dev_copy(dst, src, nbytes)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    log(f"copy calibration: {nbytes} bytes read and written")


def cpu_baseline(W, seconds: float, threads: int = 1):
    """The oracle as it stands on a bounded sample of the same workload:
    each of `threads` host threads steps its own 2^22-element window of the
    shard (windows one after another) with the single-threaded C oracle,
    repeatedly until `seconds` have passed; the oracle call holds no Python
    lock, so the threads run on separate cores."""
    import threading
    from oracle import step as O
    from synth import state as S
    n = 1 << 22
    hp = O.AdamW(**HP)
    data = [(S.cpu_grads(W, k * n, n, 1, 1e-4),
             *S.cpu_state(k * n, n, 0.02)) for k in range(threads)]
    reps = [0] * threads
    start = threading.Barrier(threads + 1)
    t_end = [0.0]

    def work(k):
        G, master, m, v = data[k]
        start.wait()
        while True:
            O.step(G, master, m, v, hp, reps[k] + 1)
            reps[k] += 1
            if time.perf_counter() >= t_end[0]:
                break

    ts = [threading.Thread(target=work, args=(k,)) for k in range(threads)]
    for t in ts:
        t.start()
    t0 = time.perf_counter()
    t_end[0] = t0 + seconds
    start.wait()
    for t in ts:
        t.join()
    el = time.perf_counter() - t0
    what = ("single-threaded C oracle" if threads == 1 else
            f"the single-threaded C oracle in {threads} host threads, one "
            f"window each")
    return dict(value=n * sum(reps) / el, unit="params/s", cores=threads,
                kind="oracle", cpu_model=cpu_model(),
                sample=f"{sum(reps)} steps over {threads} x {n}-element "
                       f"windows of the rank-0 shard (W={W}), {what}, "
                       f"{el:.1f} s")


def cpu_model() -> str:
    """The host CPU's model name, as the kernel reports it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores():
    """(threads for the all-cores oracle, cores in the affinity mask): every
    core of the process's affinity mask, capped by OMP_NUM_THREADS where the
    host sets a per-process thread share (a shared GPU node gives each GPU's
    jobs a slice of its cores and says so there)."""
    mask = len(os.sched_getaffinity(0))
    n = mask
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n), mask


def arena_views(parts):
    """Views carved, in the given order, from one device allocation.

    parts: (numel, dtype) pairs; each view starts on a 2 MiB boundary of the
    arena.  The step's bandwidth on MI355X depends on where its buffers land
    in HBM.  With the earlier form of the step (512-thread workgroups, plain
    non-temporal stores), over 19 processes on three devices, one arena
    holding the tiled gradients, then the state, then the flat buffer
    measured 78.8-81.3 % of peak (median 80.7 %).  Separate allocations
    measured 76.1-81.1 % over 14 processes (median 78.4 %), the lowest in
    processes started after others had used the device.  The other three
    region orders inside one arena measured 77.4-79.8 %."""
    import torch
    align = 2 << 20
    offs, total = [], 0
    for numel, dt in parts:
        offs.append(total)
        nbytes = numel * torch.empty((), dtype=dt).element_size()
        total += (nbytes + align - 1) // align * align
    arena = torch.empty(total, dtype=torch.uint8, device="cuda")
    return [arena[o:o + numel * torch.empty((), dtype=dt).element_size()]
            .view(dt) for o, (numel, dt) in zip(offs, parts)]


def _time_launches(fn, reps, st):
    import torch
    for _ in range(2):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(st)
    for _ in range(reps):
        fn()
    ev[1].record(st)
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / reps


def ceiling(Gt, state, flat, lay, W, n, reps=10):
    """Achievable bandwidths on this device: the step's exact access
    pattern (tiled gradients and state, flat output) with XORs in place of
    the arithmetic, a read-only stream over the tiled gradients, and a
    plain 4 GiB copy."""
    import torch
    import synth
    import zero_sharded_optimizer_shard_amd as zs
    st = torch.cuda.current_stream()
    buckets = zs.zs_layout_buckets(lay)
    b0 = buckets[0]
    args = (Gt, state, flat, W, b0.slice_numel, buckets[-1].slice_numel,
            b0.numel, len(buckets), st)
    ms = _time_launches(lambda: synth.dev_mix_stream(*args), reps, st)
    out = {"same_mix": dict(GBps=(2 * W + 26) * n / (ms * 1e-3) / 1e9,
                            ms=ms)}
    nb = Gt.numel() * 2 // 16 * 16
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    ms = _time_launches(lambda: synth.dev_read(Gt, nb, sink, stream=st),
                        reps, st)
    out["read_only"] = dict(GBps=nb / (ms * 1e-3) / 1e9, ms=ms, bytes=nb)
    cb = 4 << 30
    src = torch.empty(cb // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    ms = _time_launches(lambda: synth.dev_copy(dst, src, cb, stream=st),
                        reps, st)
    out["copy"] = dict(GBps=2 * cb / (ms * 1e-3) / 1e9, ms=ms, bytes=2 * cb)
    del src, dst
    for v in out.values():
        v["frac_of_peak"] = v["GBps"] / PEAK_HBM_GBS
    return out


def time_steps(fn, K, st):
    """K back-to-back launches of fn on stream st, bracketed by one pair of
    HIP events; returns the average kernel time (ms) and the wall time of
    the K launches (ms), both per launch."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(K):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / K
    return e0.elapsed_time(e1) / K, wall


def time_each(fn, K, st):
    """K launches of fn, each between its own pair of events (the events
    make every launch wait for the previous one's writes to be flushed)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def placement_draws(count, new_arena, first, lay, W, n, K, warmup, st,
                    first_frac):
    """The same step on further arenas: where the buffers land in HBM moves
    this stream's bandwidth by a few points, and the runtime gives no way to
    choose it.  Each new arena is allocated while the earlier ones are still
    alive, so each lands elsewhere; it gets a copy of the first arena's
    inputs and K timed launches after `warmup` untimed ones.  The first draw
    stays the reported value; this is its spread."""
    import torch
    import zero_sharded_optimizer_shard_amd as zs
    keep, fracs = [], [first_frac]
    t = 1 << 20                  # a step counter of their own
    for k in range(count):
        bufs = new_arena()
        for dst, src in zip(bufs, first):
            dst.copy_(src)
        keep.append(bufs)
        torch.cuda.synchronize()

        def one():
            nonlocal t
            t += 1
            zs.zs_step(lay, bufs[0], bufs[1], None, bufs[2],
                       grad_layout="tiled", step=t, stream=st, **HP)

        for _ in range(warmup):
            one()
        ms, _ = time_steps(one, K, st)
        fracs.append((2 * W + 26) * n / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS)
        log(f"  placement {k + 2}: {ms:.3f} ms per launch "
            f"({fracs[-1]:.1%} of 8 TB/s)")
    del keep
    torch.cuda.empty_cache()
    srt = sorted(fracs)
    mid = len(srt) // 2
    med = srt[mid] if len(srt) % 2 else (srt[mid - 1] + srt[mid]) / 2
    log(f"placements: first {first_frac:.1%}, min {srt[0]:.1%}, median "
        f"{med:.1%}, max {srt[-1]:.1%} over {len(fracs)} arenas")
    return {"arenas": len(fracs), "frac_of_peak": fracs, "first": first_frac,
            "min": srt[0], "median": med, "max": srt[-1],
            "note": "same inputs; each arena a separate allocation, all "
                    "alive at once; the first draw is the reported value"}


def bf16_main(args, w):
    """Pure-bf16 variant (12 B/param: bf16 parameter and gradient, fp32 m and
    v, no fp32 master): the step reads each parameter from this rank's
    positions of the flat bf16 buffer, updates it with the same AdamW
    statements in fp32 and writes the bf16 result back in place.  Tiled
    gradients, state tiled as [tile][m|v][8192].  2W + 20 bytes per
    element."""
    import torch
    import synth
    import zero_sharded_optimizer_shard_amd as zs
    from synth import state as S

    W, T = w.world, zs.ZS_TILE
    lay = zs.zs_layout_build(w.numels, W, w.rank)
    flat_n, n, nb, nc = zs.zs_layout_info(lay)
    n_tiles = zs.zs_layout_tiles(lay)
    log(f"workload {w.name} pure bf16: W={W} shard={n} buckets={nb}")
    Gt, state, flat = arena_views([(n_tiles * W * T, torch.bfloat16),
                                   (n_tiles * 2 * T, torch.float32),
                                   (flat_n, torch.bfloat16)])
    G = torch.empty((W, n), dtype=torch.bfloat16, device="cuda")
    S.dev_grads(G, W, n, 1, w.grad_sigma)
    zs.zs_grads_tile(lay, -1, G, n, Gt)
    del G
    zs.zs_state_mv_pack(lay, None, None, state)
    synth.dev_normal_bf16(flat, 0, synth.TAG_MASTER, 0, 0, 0, w.master_sigma)
    torch.cuda.synchronize()
    log("inputs resident")
    st = torch.cuda.current_stream()
    t = 0

    def one():
        nonlocal t
        t += 1
        zs.zs_step_bf16(lay, Gt, state, flat, params_flat=True,
                        grad_layout="tiled", step=t, stream=st, **HP)

    for _ in range(args.warmup):
        one()
    K = args.steps
    avg_ms, ms_per_step = time_steps(one, K, st)
    bpp = 2 * W + 20
    achieved = bpp * n / (avg_ms * 1e-3) / 1e9
    log(f"zs_step_bf16: {avg_ms:.3f} ms per launch -> {achieved:.0f} GB/s "
        f"({achieved / PEAK_HBM_GBS:.1%} of 8 TB/s)")
    out = {
        "metric": "pure-bf16 optimizer-step params/s per GPU + achieved HBM "
                  "GB/s (% of peak)",
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
        "config": {"workload": f"{w.name} rank-0 shard, W={W}, pure bf16",
                   "params_total": sum(w.numels), "shard_params": n,
                   "buckets": nb, "bucket_cap_mb": 25,
                   "bytes_per_param": bpp,
                   "grads_layout": "tiled [tile][W][8192]",
                   "state_layout": "tiled [tile][m|v][8192]",
                   "params": "flat bf16 buffer, in place",
                   "allocation": "one arena: tiled gradients, state, flat"},
        "roofline": {"bound": "hbm", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic_record(f"{args.workload}_bf16")},
        "kernel_ms": {"avg": avg_ms},
    }
    print(json.dumps(out), flush=True)


def checkpoint_main(args, w):
    """Checkpoint and resume of the rank's tiled optimizer state
    (zs_checkpoint_save / zs_checkpoint_load) at the workload's full size:
    each save ends with the file flushed to disk and renamed into place; each
    load restores into a second buffer, which must equal the saved state bit
    for bit.  The file goes to a temporary directory and is removed."""
    import shutil
    import tempfile
    import time

    import torch
    import synth
    import zero_sharded_optimizer_shard_amd as zs
    W = w.world
    lay = zs.zs_layout_build(w.numels, W, w.rank)
    n_tiles = zs.zs_layout_tiles(lay)
    state = torch.empty(n_tiles * 3 * zs.ZS_TILE, dtype=torch.float32,
                        device="cuda")
    synth.dev_normal_f32(state, 0, synth.TAG_MASTER, 0, 0, 0, w.master_sigma)
    back = torch.empty_like(state)
    nbytes = state.numel() * 4
    log(f"checkpoint: {w.name} rank-0 tiled state, {nbytes / 1e9:.2f} GB")
    d = tempfile.mkdtemp(prefix="zsck-")
    path = os.path.join(d, "rank0.zsck")
    saves, loads = [], []
    try:
        for k in range(max(1, min(args.steps, 3))):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            zs.zs_checkpoint_save(lay, path, state, step=k + 1)
            t1 = time.perf_counter()
            back.fill_(float("nan"))
            torch.cuda.synchronize()
            t2 = time.perf_counter()
            t = zs.zs_checkpoint_load(lay, path, back)
            t3 = time.perf_counter()
            if t != k + 1 or not torch.equal(back.view(torch.int32),
                                             state.view(torch.int32)):
                raise SystemExit("checkpoint: restored state differs")
            saves.append(t1 - t0)
            loads.append(t3 - t2)
            log(f"  save {t1 - t0:.2f} s ({nbytes / (t1 - t0) / 1e9:.2f} "
                f"GB/s), load {t3 - t2:.2f} s "
                f"({nbytes / (t3 - t2) / 1e9:.2f} GB/s)")
        fsize = os.path.getsize(path)
    finally:
        shutil.rmtree(d, ignore_errors=True)
    med = lambda x: sorted(x)[len(x) // 2]
    out = {
        "metric": "checkpoint of one rank's optimizer state: save (flushed "
                  "to disk) GB/s, restore GB/s",
        "value": nbytes / med(saves) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": len(saves),
        "warmup": 0,
        "ms_per_step": med(saves) * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name} rank-0 shard, W={W}, tiled "
                               f"[master|m|v] state",
                   "state_bytes": nbytes, "file_bytes": fsize},
        "roofline": None,
        "restore_GBps": nbytes / med(loads) / 1e9,
        "save_s": saves,
        "restore_s": loads,
        "notes": "the restore reads a file the host page cache still holds; "
                 "the save ends with fsync",
    }
    print(json.dumps(out), flush=True)


def accumulate_main(args, w):
    """Gradient accumulation over K micro-batches on the full flat bf16
    gradient buffer of the workload (what backward produces on every rank
    before the bucketed reduce-scatter): the first call starts the fp32
    accumulator, K - 2 calls add, the last adds, divides by K and writes
    the bf16 bucket in place over the last micro-batch's gradient.  Bytes
    per element per cycle: 6 + 10 (K - 2) + 8."""
    import torch
    import synth
    import zero_sharded_optimizer_shard_amd as zs

    K = args.accumulate
    if K < 2:
        raise SystemExit("--accumulate needs K >= 2")
    lay = zs.zs_layout_build(w.numels, w.world, w.rank)
    flat_n = zs.zs_layout_info(lay)[0]
    log(f"workload {w.name} gradient accumulation: {flat_n} elements, "
        f"{K} micro-batches")
    grads = [torch.empty(flat_n, dtype=torch.bfloat16, device="cuda")
             for _ in range(2)]
    for j, g in enumerate(grads):
        synth.dev_normal_bf16(g, 0, synth.TAG_GRAD, j, 0, 0, w.grad_sigma)
    acc = torch.empty(flat_n, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()

    def cycle():
        zs.zs_accumulate(zs.ZS_ACC_FIRST, acc, grads[0], stream=st)
        for j in range(1, K - 1):
            zs.zs_accumulate(zs.ZS_ACC_ADD, acc, grads[j % 2], stream=st)
        zs.zs_accumulate(zs.ZS_ACC_LAST, acc, grads[1], grads[1], k=K,
                         stream=st)

    for _ in range(args.warmup):
        cycle()
    R = max(1, min(args.steps, 10))
    avg_ms, wall_ms = time_steps(cycle, R, st)
    bpe = 6 + 10 * (K - 2) + 8
    gbs = bpe * flat_n / (avg_ms * 1e-3) / 1e9
    log(f"accumulation cycle: {avg_ms:.3f} ms -> {gbs:.0f} GB/s "
        f"({gbs / PEAK_HBM_GBS:.1%} of 8 TB/s)")
    out = {
        "metric": "gradient accumulation, micro-batch gradients per second "
                  "per GPU (elements)",
        "value": K * flat_n / (wall_ms * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": R,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name} flat gradient buffer, {K} "
                               f"micro-batches",
                   "elements": flat_n, "micro_batches": K,
                   "bytes_per_element_per_cycle": bpe},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                     "traffic": (traffic_record(f"{args.workload}_accum")
                                 if K == 2 else None)},
        "kernel_ms": {"avg": avg_ms},
    }
    print(json.dumps(out), flush=True)


def fsdp_units(numels):
    """FSDP wrapping units of a Llama-shaped list (embed, L x [attn_norm, q,
    k, v, o, ffn_norm, gate, up, down], final norm, lm_head): the
    embedding, one unit per block, and final norm + head; as (first tensor,
    last tensor) pairs."""
    L = (len(numels) - 3) // 9
    return ([(0, 0)] + [(1 + 9 * i, 9 + 9 * i) for i in range(L)] +
            [(len(numels) - 2, len(numels) - 1)])


def zero3_main(args, w):
    """ZeRO-3 / FSDP forward: each rank holds only its bf16 shard of the
    parameters (the W ranks' shards are W resident buffers here); before a
    unit runs, zs_gather materialises its full weights into one of two
    buffers, the next unit's gather runs on a second stream while the
    current unit computes, and a buffer is reused only after the unit that
    read it is done (at most two units materialised).  The layer compute is
    a stand-in: one bf16 GEMM per 2-D weight (F.linear, `--tokens` rows;
    the embedding as a lookup), not part of the library.  Reported per
    forward pass: the gathers alone, the compute alone, both pipelined."""
    import torch
    import torch.nn.functional as Fn
    import synth
    import zero_sharded_optimizer_shard_amd as zs

    W = w.world
    # whole tensors: every tensor comes whole from its owner's shard, and
    # the ranks' shards differ in size
    build = (zs.zs_layout_build_tensors if args.whole_tensors
             else zs.zs_layout_build)
    lay = build(w.numels, W, 0)
    flat_n, n, nb, nc = zs.zs_layout_info(lay)
    offs = zs.zs_layout_tensor_offsets(lay, len(w.numels))
    units = fsdp_units(w.numels)
    ranges = [(offs[a], offs[b] + w.numels[b]) for a, b in units]
    biggest = max(hi - lo for lo, hi in ranges)
    log(f"workload {w.name} ZeRO-3: W={W} shard={n} units={len(units)} "
        f"largest unit {biggest} elements"
        f"{' (whole tensors)' if args.whole_tensors else ''}")
    shards = []
    for r in range(W):
        n_r = zs.zs_layout_info(build(w.numels, W, r))[1]
        t = torch.empty(max(n_r, 8), dtype=torch.bfloat16, device="cuda")
        synth.dev_normal_bf16(t, 0, synth.TAG_MASTER, 0, r, 0, 0.02)
        shards.append(t)
    bufs = [torch.empty(biggest, dtype=torch.bfloat16, device="cuda")
            for _ in range(2)]
    d = w.numels[1]                              # hidden size (a norm)
    x = torch.randn(args.tokens, d, dtype=torch.bfloat16, device="cuda")
    ids = torch.randint(0, w.numels[0] // d, (args.tokens,), device="cuda")
    torch.cuda.synchronize()
    log("shards resident")

    def views(u, buf):
        a, b = units[u]
        lo = ranges[u][0]
        out = []
        for t in range(a, b + 1):
            v = buf[offs[t] - lo:offs[t] - lo + w.numels[t]]
            out.append(v.view(-1, d) if w.numels[t] % d == 0 and
                       w.numels[t] > d else None)
        return out

    def compute(u, buf):
        """Stand-in for the unit's forward: the embedding as a lookup, every
        other weight (viewed as [rows, d]) applied once to x with F.linear,
        i.e. 2 * tokens * numel flops per weight; results are dropped."""
        ws = views(u, buf)
        if u == 0:
            Fn.embedding(ids, ws[0])
            return
        for wt in ws:
            if wt is not None:
                Fn.linear(x, wt)

    gs = torch.cuda.Stream()
    st = torch.cuda.current_stream()
    NU = len(units)

    def gathers_alone():
        for u in range(NU):
            zs.zs_gather(lay, shards, ranges[u][0], ranges[u][1],
                         bufs[u % 2], stream=st)

    def compute_alone():
        for u in range(NU):
            compute(u, bufs[u % 2])

    pf = zs.zs_prefetch_create(lay, shards, bufs, gs)

    def pipelined():
        """The library's prefetch object: unit u + 1 is gathered on the
        gather stream while unit u computes; a buffer is reused after the
        compute that read it."""
        gs.wait_stream(st)          # nothing before the timing event
        slots = [zs.zs_prefetch_issue(pf, *ranges[0])]
        for u in range(NU):
            if u + 1 < NU:
                slots.append(zs.zs_prefetch_issue(pf, *ranges[u + 1]))
            buf = zs.zs_prefetch_acquire(pf, slots[u], st)
            compute(u, buf)
            zs.zs_prefetch_release(pf, slots[u], st)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps, (time.perf_counter() - t0) * 1e3 \
            / reps

    K = max(1, min(args.steps, 10))
    g_ms, g_wall = timed(gathers_alone, K)
    elems = sum(hi - lo for lo, hi in ranges)
    g_gbs = 4 * elems / (g_ms * 1e-3) / 1e9
    log(f"gathers alone: {g_ms:.3f} ms per forward ({elems} elements, "
        f"{g_gbs:.0f} GB/s, {g_gbs / PEAK_HBM_GBS:.1%})")
    c_ms, _ = timed(compute_alone, K)
    log(f"stand-in compute alone: {c_ms:.3f} ms per forward")
    p_ms, p_wall = timed(pipelined, K)
    log(f"pipelined: {p_ms:.3f} ms per forward, exposed gather "
        f"{p_ms - c_ms:.3f} ms")
    out = {
        "metric": "ZeRO-3 per-layer parameter gather (FSDP forward with "
                  "prefetch), gathered params/s per GPU",
        "value": elems / (g_ms * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": 1,
        "ms_per_step": g_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name} parameters, W={W} shards, "
                               f"ZeRO-3 gather per FSDP unit"
                               + (", whole tensors from their owners"
                                  if args.whole_tensors else ""),
                   "params_total": sum(w.numels), "fsdp_units": NU,
                   "bytes_per_param": 4, "tokens": args.tokens},
        "roofline": {"bound": "hbm", "achieved": g_gbs,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": g_gbs / PEAK_HBM_GBS,
                     "traffic": traffic_record(
                         f"{args.workload}_zero3"
                         + ("_tensors" if args.whole_tensors else ""))},
        "zero3": {"gathers_alone_ms": g_ms, "compute_alone_ms": c_ms,
                  "pipelined_ms": p_ms, "exposed_gather_ms": p_ms - c_ms,
                  "elements_per_forward": elems},
    }
    print(json.dumps(out), flush=True)


def stream_main(args, w):
    """ZeRO-2 streaming: the W slices of each 25 MiB bucket arrive one bucket
    at a time, last bucket first (the order backward fills them), into a ring
    of 2G staging slots on an upload stream; zs_buckets_step runs on every G
    landed buckets, the groups taking the step streams in turn (so that one
    launch's tail overlaps the next launch), and the upload stream reuses a
    slot only after the step that read it.  Arrival is a
    host-to-device copy from a pinned pool of 4 distinct buckets (bucket b
    uses pool b mod 4), or a device copy from an HBM pool (--arrival d2d).
    Reported per full step (every bucket once): the wall time, the same
    uploads alone, the same bucket steps alone with the staging resident,
    and the exposed step time, measured inside each streamed full step: the
    end of the last launch on any step stream minus the end of the last
    copy on any upload stream (events recorded on every stream after the
    step's last call)."""
    import torch
    import synth
    import zero_sharded_optimizer_shard_amd as zs

    W, T = w.world, zs.ZS_TILE
    lay = zs.zs_layout_build(w.numels, W, w.rank)
    flat_n, n, nb, nc = zs.zs_layout_info(lay)
    n_tiles = zs.zs_layout_tiles(lay)
    B = zs.zs_layout_buckets(lay)
    log(f"workload {w.name} streaming: W={W} shard={n} buckets={nb} "
        f"tiles={n_tiles} arrival={args.arrival} group={args.group}")
    state = torch.empty(n_tiles * 3 * T, dtype=torch.float32, device="cuda")
    master = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.dev_normal_f32(master, 0, synth.TAG_MASTER, 0, 0, 0, w.master_sigma)
    zs.zs_state_pack(lay, master, None, None, state)
    torch.cuda.synchronize()
    del master
    torch.cuda.empty_cache()
    flat = torch.zeros(flat_n, dtype=torch.bfloat16, device="cuda")
    S0 = B[0].slice_numel
    tiles_full = -(-S0 // T)
    slot_elems = tiles_full * W * T
    # the pool: 4 distinct buckets of tiled gradients
    pool_d = []
    tmp = torch.empty((W, S0), dtype=torch.bfloat16, device="cuda")
    for k in range(4):
        for s_ in range(W):
            synth.dev_normal_bf16(tmp[s_], 0, synth.TAG_GRAD, 1, s_,
                                  B[k].shard_off, w.grad_sigma)
        t_ = torch.empty(slot_elems, dtype=torch.bfloat16, device="cuda")
        zs.zs_grads_tile(lay, k, tmp, S0, t_)
        pool_d.append(t_)
    del tmp
    if args.arrival == "h2d":
        pool = [torch.empty(slot_elems, dtype=torch.bfloat16,
                            pin_memory=True) for _ in range(4)]
        for h, d in zip(pool, pool_d):
            h.copy_(d)
        del pool_d
    else:
        pool = pool_d
    G = max(1, min(args.group, zs.ZS_MAX_GROUP))
    slots = 2 * G
    staging = [torch.empty(slot_elems, dtype=torch.bfloat16, device="cuda")
               for _ in range(slots)]
    torch.cuda.synchronize()
    log("inputs resident")
    up = torch.cuda.Stream()
    # groups go to the step streams in turn, so that one group's tail
    # overlaps the next group's start (groups touch disjoint buckets)
    sts = [torch.cuda.Stream() for _ in range(max(1, args.step_streams))]
    st = sts[0]
    order = list(range(nb))[::-1]
    cnt = [-(-B[b].slice_numel // T) * W * T for b in range(nb)]
    t_step = 0

    def full_step(do_upload=True, do_step=True):
        """Every bucket once: arrival k lands in slot k mod 2G; after each G
        arrivals one zs_buckets_step steps them, on the step stream, once
        the last of them has landed (the upload stream is in order)."""
        nonlocal t_step
        t_step += 1
        done = [None] * slots
        for g0 in range(0, nb, G):
            gst = sts[(g0 // G) % len(sts)]
            ids = order[g0:g0 + G]
            sl = [(g0 + i) % slots for i in range(len(ids))]
            landed = None
            if do_upload:
                with torch.cuda.stream(up):
                    waited = set()
                    for b, k in zip(ids, sl):
                        ev = done[k]
                        if ev is not None and id(ev) not in waited:
                            up.wait_event(ev)
                            waited.add(id(ev))
                        staging[k][:cnt[b]].copy_(pool[b % 4][:cnt[b]],
                                                  non_blocking=True)
                    landed = torch.cuda.Event()
                    landed.record(up)
            if do_step:
                if landed is not None:
                    gst.wait_event(landed)
                zs.zs_buckets_step(lay, ids, [staging[k] for k in sl], state,
                                   None, flat, grad_layout="tiled",
                                   step=t_step, stream=gst, **HP)
                ev = torch.cuda.Event()
                ev.record(gst)
                for k in sl:
                    done[k] = ev

    K = w.steps                 # full steps are long here: the config's 2

    def timed(**kw):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            full_step(**kw)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / K

    full_step(do_upload=False)              # warm-up: kernels only
    torch.cuda.synchronize()
    e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
    e0.record(st)
    for s_ in sts[1:]:                      # nothing starts before e0
        s_.wait_event(e0)
    for _ in range(K):
        full_step(do_upload=False)
    for s_ in sts[1:]:                      # e1 after every stream's work
        ev = torch.cuda.Event()
        ev.record(s_)
        st.wait_event(ev)
    e1.record(st)
    torch.cuda.synchronize()
    kern_ev_ms = e0.elapsed_time(e1) / K
    kern_ms = timed(do_upload=False)
    log(f"bucket steps alone: {kern_ms:.2f} ms per full step "
        f"(events {kern_ev_ms:.2f} ms)")
    if args.kernels_only:
        # the group launches alone (for counter runs): no arrival passes
        bpp = 2 * W + 26
        kern_gbs = bpp * n / (kern_ev_ms * 1e-3) / 1e9
        print(json.dumps({
            "metric": "ZeRO-2 bucket-group steps alone, params/s per GPU",
            "value": n / (kern_ev_ms * 1e-3), "unit": "params/s",
            "n_gpus": 1, "steps": K, "warmup": 1, "ms_per_step": kern_ev_ms,
            "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": f"{w.name} rank-0 shard, W={W}, bucket "
                                   f"groups of {G} without arrival",
                       "shard_params": n, "buckets": nb,
                       "bytes_per_param": bpp, "step_streams": len(sts)},
            "roofline": {"bound": "hbm", "achieved": kern_gbs,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": kern_gbs / PEAK_HBM_GBS,
                         "traffic": traffic_record(args.workload)}}))
        return
    up_ms = timed(do_step=False)
    log(f"uploads alone: {up_ms:.2f} ms per full step")
    py_ms = timed()
    log(f"streaming, scheduled from Python: {py_ms:.2f} ms per full step")

    # the streaming step proper: the library's engine schedules the copies
    # into the staging ring and the grouped steps on the step streams
    ups = [up] + [torch.cuda.Stream()
                  for _ in range(max(1, args.upload_streams) - 1)]
    eng = zs.zs_stream_create(lay, G, staging, up if len(ups) == 1 else ups,
                              sts)

    def engine_step():
        nonlocal t_step
        t_step += 1
        zs.zs_stream_step_begin(eng, state, None, flat, step=t_step, **HP)
        for b in order:
            zs.zs_stream_arrive(eng, b, pool[b % 4])
        zs.zs_stream_step_end(eng)

    def stream_ends():
        """Events after the last work queued on every upload and every
        step stream."""
        ends = []
        for group in (ups, sts):
            evs = []
            for s_ in group:
                e = torch.cuda.Event(enable_timing=True)
                e.record(s_)
                evs.append(e)
            ends.append(evs)
        return ends

    engine_step()
    torch.cuda.synchronize()
    marks = [stream_ends()]
    t0 = time.perf_counter()
    for _ in range(K):              # steps queued back to back, no host sync
        engine_step()
        marks.append(stream_ends())
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / K
    ref = marks[0][0][0]
    up_end = [max(ref.elapsed_time(e) for e in eu) for eu, _ in marks]
    step_end = [max(ref.elapsed_time(e) for e in es) for _, es in marks]
    # per full step: the last launch's end after the last copy's end, and
    # the span of the step's copies (from the previous step's last copy:
    # the host queues far ahead of the copies, so they run back to back)
    exposed = [step_end[k] - up_end[k] for k in range(1, K + 1)]
    up_span = [up_end[k] - up_end[k - 1] for k in range(1, K + 1)]
    log(f"streaming (zs_stream engine): {wall_ms:.2f} ms per full step; "
        f"copies {', '.join(f'{x:.1f}' for x in up_span)} ms; last launch "
        f"ends {', '.join(f'{x:.3f}' for x in exposed)} ms after the last "
        f"copy (wall - uploads alone: {wall_ms - up_ms:.2f} ms)")
    bpp = 2 * W + 26
    arrival_bytes = sum(cnt) * 2
    kern_gbs = bpp * n / (kern_ev_ms * 1e-3) / 1e9
    out = {
        "metric": "ZeRO-2 streaming optimizer step, params/s per GPU "
                  "(bucket-by-bucket, overlapped with bucket arrival)",
        "value": n / (wall_ms * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": 1,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name} rank-0 shard, W={W}, ZeRO-2 "
                               f"streaming",
                   "params_total": sum(w.numels), "shard_params": n,
                   "buckets": nb, "bucket_cap_mb": 25,
                   "bytes_per_param": bpp, "arrival": args.arrival,
                   "buckets_per_launch": G, "staging_slots": slots,
                   "step_streams": len(sts), "upload_streams": len(ups),
                   "scheduler": "zs_stream engine (native)",
                   "grads_layout": "tiled [tile][W][8192]"},
        "roofline": {"bound": "hbm", "achieved": kern_gbs,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": kern_gbs / PEAK_HBM_GBS,
                     "traffic": traffic_record(args.workload)},
        "streaming": {"wall_ms_per_step": wall_ms,
                      "uploads_alone_ms_per_step": up_ms,
                      "bucket_steps_alone_ms_per_step": kern_ms,
                      "bucket_steps_alone_event_ms": kern_ev_ms,
                      "exposed_step_ms": sum(exposed) / len(exposed),
                      "exposed_step_ms_each": exposed,
                      "exposed_definition": "per full step: end of the "
                      "last launch on any step stream - end of the last "
                      "copy on any upload stream, events in the same pass",
                      "wall_minus_uploads_alone_ms": wall_ms - up_ms,
                      "copies_in_pass_ms_each": up_span,
                      "python_scheduled_wall_ms": py_ms,
                      "arrival_bytes_per_step": arrival_bytes,
                      "arrival_GBps": arrival_bytes / (up_ms * 1e-3) / 1e9,
                      "per_bucket_kernel_us": kern_ev_ms * 1e3 / nb,
                      "launches_per_step": -(-nb // G)},
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b",
                    choices=["llama8b", "dense7b", "gpt2", "tiny",
                             "llama70b"],
                    help="llama70b runs the ZeRO-2 streaming mode")
    ap.add_argument("--arrival", default="h2d", choices=["h2d", "d2d"],
                    help="streaming mode: buckets arrive from pinned host "
                    "memory (h2d) or from an HBM pool (d2d)")
    ap.add_argument("--pure-bf16", action="store_true",
                    help="pure-bf16 step (no fp32 master, 12 B/param): "
                    "zs_step_bf16 on the flat buffer in place")
    ap.add_argument("--accumulate", type=int, default=0, metavar="K",
                    help="gradient accumulation over K micro-batches "
                    "(zs_accumulate) on the workload's flat gradient buffer")
    ap.add_argument("--checkpoint", action="store_true",
                    help="save and restore the rank's tiled optimizer state "
                    "(zs_checkpoint_save / zs_checkpoint_load) at full size")
    ap.add_argument("--whole-tensors", action="store_true",
                    help="whole-tensor shard assignment "
                    "(zs_layout_build_tensors): every tensor on one rank, "
                    "same step kernel over the rank's owned tensors; with "
                    "--zero3, each tensor gathered whole from its owner")
    ap.add_argument("--zero3", action="store_true",
                    help="ZeRO-3 / FSDP mode: per-layer parameter gather "
                    "(zs_gather) with prefetch, on the workload's layout")
    ap.add_argument("--tokens", type=int, default=2048,
                    help="ZeRO-3 mode: tokens of the stand-in layer compute")
    ap.add_argument("--group", type=int, default=16,
                    help="streaming mode: landed buckets stepped per launch "
                    "(zs_buckets_step); the ring holds 2*group slots")
    ap.add_argument("--upload-streams", type=int, default=1,
                    help="streaming: upload streams the engine copies "
                    "arriving buckets on, in turn (zs_stream_create_multi)")
    ap.add_argument("--step-streams", type=int, default=2,
                    help="streaming mode: step streams the landed groups "
                    "are spread over, in turn")
    ap.add_argument("--placements", type=int, default=3,
                    help="also time the step on this many more arenas "
                    "(each a separate allocation, all alive at once), same "
                    "inputs; reported beside the first draw, which stays "
                    "the headline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", dest="ceiling", action="store_false",
                    help="skip the device ceilings (the step's access "
                    "pattern with XORs for the arithmetic, a read-only "
                    "stream and a plain copy), timed by default")
    ap.add_argument("--ceiling", dest="ceiling", action="store_true",
                    help=argparse.SUPPRESS)
    ap.set_defaults(ceiling=True)
    ap.add_argument("--unfused", action="store_true",
                    help="also time step-to-shard + separate pack")
    ap.add_argument("--kernels-only", action="store_true",
                    help="llama70b: time the bucket-group launches alone "
                    "and skip the arrival passes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="launch one plain 4 GiB device copy before the "
                    "steps (the reference dispatch for rocprofv3 counters)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV",
                                                          "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 --pmc counter CSVs of "
                    "a --copy-calibration run of --workload (and of "
                    "--pure-bf16, --whole-tensors, --zero3 or --accumulate 2 "
                    "for those modes) into profiles/traffic_<key>.json")
    args = ap.parse_args()

    if args.record_traffic:
        import zero_sharded_optimizer_shard_amd as zs
        from synth import workloads as wl
        w = wl.presets()[args.workload]
        n = zs.zs_layout_info(zs.zs_layout_build(w.numels, w.world,
                                                 w.rank))[1]
        per_step = 0
        if w.streaming:
            nb = zs.zs_layout_info(zs.zs_layout_build(w.numels, w.world,
                                                      w.rank))[2]
            per_step = -(-nb // min(args.group, zs.ZS_MAX_GROUP))
        key = args.workload + ("_bf16" if args.pure_bf16 else "")
        if args.whole_tensors:
            key = args.workload + "_tensors"
            n = zs.zs_layout_info(zs.zs_layout_build_tensors(
                w.numels, w.world, w.rank))[1]
        if args.zero3:                      # as zero3_main gathers them
            key = args.workload + "_zero3"
            build = zs.zs_layout_build
            if args.whole_tensors:
                key += "_tensors"
                build = zs.zs_layout_build_tensors
            lay = build(w.numels, w.world, 0)
            offs = zs.zs_layout_tensor_offsets(lay, len(w.numels))
            units = fsdp_units(w.numels)
            n = sum(offs[b] + w.numels[b] - offs[a] for a, b in units)
            per_step = len(units)
        elif args.accumulate:
            key = args.workload + "_accum"
            n = zs.zs_layout_info(zs.zs_layout_build(w.numels, w.world,
                                                     w.rank))[0]
            per_step = 2
        rec = record_traffic(*args.record_traffic, n, w.world, key, per_step)
        print(json.dumps({k: rec[k] for k in
                          ("bytes_per_launch", "ratio_to_algorithmic")}))
        return

    if args.gpus != 1:
        print(f"bench.py: the step is measured on one GPU, with the W "
              f"ranks' gradient slices resident on that device; --gpus "
              f"{args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import zero_sharded_optimizer_shard_amd as zs
    from synth import state as S
    from synth import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    w = wl.presets()[args.workload]
    if args.copy_calibration:
        copy_calibration()
    if args.zero3:
        return zero3_main(args, w)
    if args.pure_bf16:
        return bf16_main(args, w)
    if args.accumulate:
        return accumulate_main(args, w)
    if args.checkpoint:
        return checkpoint_main(args, w)
    if w.streaming:
        return stream_main(args, w)
    W = w.world
    if args.whole_tensors:
        lay = zs.zs_layout_build_tensors(w.numels, W, w.rank)
    else:
        lay = zs.zs_layout_build(w.numels, W, w.rank)
    flat_n, n, nb, nc = zs.zs_layout_info(lay)
    log(f"workload {w.name}: W={W} shard={n} flat={flat_n} buckets={nb} "
        f"chunks={nc}{' (whole tensors)' if args.whole_tensors else ''}")

    n_tiles = zs.zs_layout_tiles(lay)
    T = zs.ZS_TILE
    bpp = 2 * W + 26
    parts = [(n_tiles * W * T, torch.bfloat16),
             (n_tiles * 3 * T, torch.float32), (flat_n, torch.bfloat16)]
    # A working set of a few times the 256 MB Infinity Cache or less would
    # be served partly from it; such shards (the GPT-2-sized one) are
    # stepped over R = 4 independent copies of every operand in turn, so
    # that each launch's bytes come from HBM.
    R = 1 if bpp * n >= (1 << 30) else 4
    # each set's three step buffers from one arena, gradients first (see
    # arena_views); its plain slices, for the slices-layout pass, outside it
    sets = []
    master = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.dev_normal_f32(master, 0, synth.TAG_MASTER, 0, 0, 0,
                         w.master_sigma)
    for _ in range(R):
        Gt, state, flat = arena_views(parts)
        flat.zero_()
        G = torch.empty((W, n), dtype=torch.bfloat16, device="cuda")
        S.dev_grads(G, W, n, 1, w.grad_sigma)
        zs.zs_grads_tile(lay, -1, G, n, Gt)
        zs.zs_state_pack(lay, master, None, None, state)
        sets.append((Gt, state, flat, G))
    del master
    Gt, state, flat, G = sets[0]
    torch.cuda.synchronize()
    log(f"inputs resident ({n_tiles} tiles, {R} set{'s' if R > 1 else ''})")

    st = torch.cuda.current_stream()
    t = 0

    def step_tiled():
        nonlocal t
        t += 1
        Gt_, state_, flat_, _ = sets[t % R]
        zs.zs_step(lay, Gt_, state_, None, flat_, grad_layout="tiled",
                   step=t, stream=st, **HP)

    def step_slices():
        nonlocal t
        t += 1
        _, state_, flat_, G_ = sets[t % R]
        zs.zs_step(lay, G_, state_, None, flat_, grad_layout="slices",
                   grad_stride=n, step=t, stream=st, **HP)

    for _ in range(args.warmup):
        step_tiled()
    torch.cuda.synchronize()
    K = args.steps
    avg_ms, ms_per_step = time_steps(step_tiled, K, st)
    achieved = bpp * n / (avg_ms * 1e-3) / 1e9
    log(f"zs_step (tiled): {avg_ms:.3f} ms per launch, {K} back to back "
        f"-> {achieved:.0f} GB/s ({achieved / PEAK_HBM_GBS:.1%} of 8 TB/s)")
    each = time_each(step_tiled, K, st)
    med = sorted(each)[K // 2] if K % 2 else sum(sorted(each)[K // 2 - 1:
                                                             K // 2 + 1]) / 2
    log(f"  with events around each launch: avg {sum(each) / K:.3f} ms, "
        f"median {med:.3f}, min {min(each):.3f}, max {max(each):.3f}")

    extra = {"per_launch_events_ms": dict(avg=sum(each) / K, median=med,
                                          min=min(each), max=max(each))}
    for _ in range(2):
        step_slices()
    sl_avg, _ = time_steps(step_slices, K, st)
    sl_gbs = bpp * n / (sl_avg * 1e-3) / 1e9
    extra["slices_layout"] = dict(kernel_ms_avg=sl_avg,
                                  params_per_s=n / (sl_avg * 1e-3),
                                  GBps=sl_gbs, frac=sl_gbs / PEAK_HBM_GBS)
    log(f"zs_step (plain slices): {sl_avg:.3f} ms -> {sl_gbs:.0f} GB/s "
        f"({sl_gbs / PEAK_HBM_GBS:.1%})")
    if R == 1:
        # the same step on three plain fp32 arrays (zs_step_plain): the
        # state unpacked from the tiled form, tiled gradients, flat output
        plain = [torch.empty(n, dtype=torch.float32, device="cuda")
                 for _ in range(3)]
        zs.zs_state_unpack(lay, state, *plain)

        def step_plain():
            nonlocal t
            t += 1
            zs.zs_step_plain(lay, Gt, *plain, None, flat,
                             grad_layout="tiled", step=t, stream=st, **HP)

        for _ in range(2):
            step_plain()
        pl_avg, _ = time_steps(step_plain, K, st)
        pl_gbs = bpp * n / (pl_avg * 1e-3) / 1e9
        extra["plain_state"] = dict(kernel_ms_avg=pl_avg, GBps=pl_gbs,
                                    frac=pl_gbs / PEAK_HBM_GBS)
        log(f"zs_step_plain (plain master/m/v): {pl_avg:.3f} ms -> "
            f"{pl_gbs:.0f} GB/s ({pl_gbs / PEAK_HBM_GBS:.1%})")
        del plain
        torch.cuda.empty_cache()
    if args.unfused:
        p = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for _ in range(2):
            zs.zs_step(lay, Gt, state, p, None, grad_layout="tiled", step=t,
                       stream=st, **HP)
            zs.zs_pack(lay, p, flat, stream=st)
        e[0].record(st)
        zs.zs_step(lay, Gt, state, p, None, grad_layout="tiled", step=t,
                   stream=st, **HP)
        e[1].record(st)
        zs.zs_pack(lay, p, flat, stream=st)
        e[2].record(st)
        torch.cuda.synchronize()
        extra["unfused_ms"] = dict(step=e[0].elapsed_time(e[1]),
                                   pack=e[1].elapsed_time(e[2]))
        # the per-tensor pack: this rank's chunks scattered into separate
        # per-tensor buffers through the device chunk table
        import numpy as np
        tensors = [torch.empty(k, dtype=torch.bfloat16, device="cuda")
                   for k in w.numels]
        ptrs = torch.tensor([t_.data_ptr() for t_ in tensors],
                            dtype=torch.int64, device="cuda")
        chunks = zs.zs_layout_chunks(lay)
        dch = torch.from_numpy(np.frombuffer(zs.chunks_bytes(chunks),
                                             np.uint8).copy()).cuda()
        extra["unfused_ms"]["pack"] = _time_launches(
            lambda: zs.zs_pack(lay, p, flat, stream=st), K, st)
        ms = _time_launches(lambda: zs.zs_pack(lay, p, None, dch, len(chunks),
                                               ptrs, stream=st), K, st)
        extra["unfused_ms"]["pack_chunks"] = ms
        extra["pack_GBps"] = dict(
            flat=4 * n / (extra["unfused_ms"]["pack"] * 1e-3) / 1e9,
            chunks=4 * n / (ms * 1e-3) / 1e9)
        log(f"unfused: step {extra['unfused_ms']['step']:.3f} ms, pack to "
            f"flat {extra['unfused_ms']['pack']:.3f} ms "
            f"({extra['pack_GBps']['flat']:.0f} GB/s), pack to "
            f"{len(w.numels)} tensors {ms:.3f} ms "
            f"({extra['pack_GBps']['chunks']:.0f} GB/s)")
        del p, tensors
    if args.placements > 0 and R == 1:
        extra["placements"] = placement_draws(
            args.placements, lambda: arena_views(parts), (Gt, state, flat),
            lay, W, n, K, args.warmup, st, achieved / PEAK_HBM_GBS)
    if args.ceiling and not args.whole_tensors and R == 1:
        c = ceiling(Gt, state, flat, lay, W, n)
        c["step_frac_of_same_mix"] = achieved / c["same_mix"]["GBps"]
        extra["ceilings"] = c
        log(f"ceilings: same mix {c['same_mix']['GBps']:.0f} GB/s "
            f"({c['same_mix']['ms']:.3f} ms), read-only "
            f"{c['read_only']['GBps']:.0f} GB/s, copy "
            f"{c['copy']['GBps']:.0f} GB/s; the step runs at "
            f"{c['step_frac_of_same_mix']:.1%} of the same-mix ceiling")

    traffic = traffic_record(args.workload + ("_tensors" if args.whole_tensors
                                              else ""))
    config = {"workload": f"{w.name} rank-0 shard, W={W}",
              "params_total": sum(w.numels), "shard_params": n,
              "buckets": nb, "bucket_cap_mb": 25,
              "bytes_per_param": bpp,
              # bytes one step touches, against MI355X's 256 MB Infinity
              # Cache: a smaller working set would be served from cache;
              # R independent sets are stepped in turn
              "working_set_bytes": bpp * n,
              "state_sets": R,
              "cache_resident": bpp * n * R < (256 << 20),
              "grads_layout": "tiled [tile][W][8192]",
              "state_layout": "tiled [tile][master|m|v][8192]",
              "allocation": "one arena: tiled gradients, state, flat"}
    if args.whole_tensors:
        config.update(workload=f"{w.name} rank-0 shard, W={W}, whole-tensor "
                      "assignment", assignment="whole tensors, longest "
                      "first to the least-loaded rank", owned_tensors=nb)
        del config["bucket_cap_mb"]
    out = {
        "metric": metric_for(args.workload) if not args.whole_tensors else
        "whole-tensor-assignment optimizer-step params/s per GPU + achieved "
        "HBM GB/s (% of peak)",
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
        "config": config,
        "roofline": {"bound": "hbm", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic},
        "kernel_ms": {"avg": avg_ms},
        "achieved_GBps_per_step": bpp * n / (ms_per_step * 1e-3) / 1e9,
        **extra,
    }
    del G, Gt, state, flat, sets
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(W, args.cpu_seconds)
        nc, mask = host_cores()
        if nc > 1:
            log(f"timing the CPU oracle on {nc} cores (affinity mask: "
                f"{mask}) ...")
            allc = cpu_baseline(W, args.cpu_seconds, nc)
            allc["affinity_mask_cores"] = mask
            allc["thread_share"] = os.environ.get("OMP_NUM_THREADS")
            out["cpu_baseline_all_cores"] = allc
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
