#!/usr/bin/env python3
"""Benchmark one scheduler step of paged-KV attention on one MI355X.

A step is the whole hot path over one synthetic batch: ``paged_kv_append`` of
the step's new K/V rows, then ``paged_attn_step`` (decode partitions, split
reduce, prefill-chunk rows).  Inputs are resident in HBM before the timed
region.  Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_7b]

value = algorithmic KV bytes of the step (each distinct physical token row of
K and V once, fp8 scales included) / wall time of a step, in GB/s (1e9 B/s).
"""
import argparse
import hashlib
import glob
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / f16 matrix rate, vendor figure (no sparsity)
METRIC = "paged decode attention: KV-read GB/s (% of HBM peak), batch-steps/s"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_digest():
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "paged_kv_cache_286_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_counters(workload, kernel):
    """Counter record of `kernel` from committed rocprofv3 runs (HBM bytes per launch,
    L2 hit rate, MFMA busy fraction), if the kernel sources have not changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != source_digest():
        return {}
    return t


def attention_flops(plan):
    """Multiply-adds x 2 of the step's attention: QK^T and PV over every (row, key)
    pair the causal mask keeps, for every query head."""
    D, H = plan.cfg.head_dim, plan.cfg.num_q_heads
    pairs = 0
    for L, Q in zip(plan.context_lens.tolist(), plan.query_lens.tolist()):
        pairs += Q * (L - Q) + Q * (Q + 1) // 2
    return 4 * D * H * pairs


# The oracle as it stands, timed on the host's cores: the workload is generated
# first, then a pool of worker processes is forked from this process before it
# has touched the GPU (the workers inherit the arrays and only read them).
_CPU_WL = None


def _oracle_seqs(seqs):
    """Worker: the oracle's attention for some sequences of the step (one BLAS thread)."""
    import oracle
    from threadpoolctl import threadpool_limits
    wl = _CPU_WL
    p, cfg = wl.plan, wl.cfg
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.paged_attention(wl.q, wl.k, wl.v, p.block_tables, p.context_lens, p.query_lens,
                               wl.scale, cfg.block_size, cfg.kv_dtype, cfg.q_dtype,
                               wl.k_scale, wl.v_scale, seqs=seqs)
        return time.perf_counter() - t0


# At most this many worker processes: a one-GPU job on a shared host is given
# a share of 16 cores, whatever the machine reports.
CPU_POOL_CAP = 16


def cpu_baseline(wl, seconds, single_seconds):
    """Time the float64 oracle on the host: the whole step's attention spread over
    N worker processes (N = usable cores, each with one BLAS thread), repeated
    until about `seconds` of wall time have passed; plus, when single_seconds > 0,
    one thread on a prefix of the step's sequences."""
    import multiprocessing as mp
    import numpy as np
    from paged_kv_cache_286_amd import workloads as W
    global _CPU_WL
    _CPU_WL = wl
    p, cfg = wl.plan, wl.cfg
    per_tok = W.kv_bytes_per_token(cfg)
    host_cores = len(os.sched_getaffinity(0))
    n = max(1, min(host_cores, CPU_POOL_CAP, p.num_seqs))
    # longest-first greedy split of the sequences over n workers, by attention work
    work = p.context_lens.astype(np.int64) * p.query_lens.astype(np.int64)
    groups, load = [[] for _ in range(n)], [0] * n
    for i in np.argsort(-work, kind="stable").tolist():
        k = load.index(min(load))
        groups[k].append(i)
        load[k] += int(work[i])
    groups = [g for g in groups if g]
    step_bytes = W.algorithmic_kv_bytes(p)["unique"]
    ctx = mp.get_context("fork")
    with ctx.Pool(len(groups)) as pool:
        pool.map(_oracle_seqs, [[g[0]] for g in groups])          # workers up, code paged in
        rounds, wall = 0, 0.0
        while rounds == 0 or wall < seconds:
            t0 = time.perf_counter()
            pool.map(_oracle_seqs, groups, chunksize=1)
            wall += time.perf_counter() - t0
            rounds += 1
    gbs = rounds * step_bytes / wall / 1e9
    out = {"value": round(gbs, 4), "unit": "GB/s", "cores": len(groups), "kind": "oracle",
           "sample": f"float64 numpy oracle: attention of the whole step ({p.num_seqs} sequences, "
                     f"{step_bytes} algorithmic KV bytes) {rounds} time(s) in {wall:.1f} s "
                     f"of wall time, sequences split over {len(groups)} worker processes with "
                     f"one BLAS thread each, on {cpu_model()}",
           "steps_per_s": round(rounds / wall, 4),
           "host_cores": host_cores, "cpu_model": cpu_model()}
    if single_seconds > 0:
        done, t_used, toks = 0, 0.0, 0
        for i in range(p.num_seqs):
            t_used += _oracle_seqs([i])
            done += 1
            toks += int(p.context_lens[i])
            if t_used >= single_seconds:
                break
        out["single_core"] = {
            "value": round(toks * per_tok / t_used / 1e9, 4), "unit": "GB/s", "cores": 1,
            "sample": f"the first {done} of {p.num_seqs} sequences ({toks} context tokens) in "
                      f"{t_used:.1f} s on one thread"}
    _CPU_WL = None
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def copy_bandwidth(torch, mib=1024, reps=10):
    """Bytes read + written per second by a plain device copy of `mib` MiB (torch's
    copy kernel): a measured ceiling beside the 8 TB/s specification."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / reps
    del src, dst
    return 2 * n / (ms / 1e3) / 1e9


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_7b")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time of the CPU oracle baseline on its worker pool")
    ap.add_argument("--cpu-single-seconds", type=float, default=5.0,
                    help="CPU time of the one-thread oracle figure (tiny and 7B decode steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="time the steps without per-kernel events")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB --steps times (scales the "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the paged attention step here runs on a single "
              "MI355X (no sharding or collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_kv_cache_286_amd import workloads as W

    # The CPU leg forks worker processes.  torch's CPU thread pool (which the
    # generator's bf16 / fp8 rounding would start) is not safe to fork: a child
    # then blocked forever on a lock one of those threads held.  One intra-op
    # thread keeps the pool from being created.
    torch_threads = torch.get_num_threads()
    torch.set_num_threads(1)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": args.steps}), flush=True)
        return
    log(f"generating workload {args.workload}")
    t0 = time.time()
    wl = W.generate(W.make_plan(args.workload))
    p, cfg = wl.plan, wl.cfg
    alg = W.algorithmic_kv_bytes(p)
    log(f"generated in {time.time() - t0:.1f} s")
    # the CPU leg forks its workers now, before this process initialises the GPU
    cpu = None
    if not args.no_cpu_baseline:
        single = args.cpu_single_seconds if args.workload in ("tiny_decode", "decode_7b") else 0.0
        log(f"CPU oracle baseline (~{args.cpu_seconds:.0f} s on the pool"
            + (f", ~{single:.0f} s on one thread)" if single else ")"))
        cpu = cpu_baseline(wl, args.cpu_seconds, single)
    torch.set_num_threads(torch_threads)

    from paged_kv_cache_286_amd import pagedkv as pk          # raises if the library is not built
    from paged_kv_cache_286_amd.device import DeviceStep
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    log("uploading")
    ds = DeviceStep(wl, "cuda:0")
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        ds.step(stream)
    torch.cuda.synchronize()

    # K steps, each between a pair of events on the launch stream: the median
    # of the K step times is the step time; the mean and the whole region's
    # rate are reported beside it
    log(f"timing {args.steps} steps")
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        starts[i].record(stream)
        ds.step(stream)
        stops[i].record(stream)
    torch.cuda.synchronize()
    step_ms = sorted(a.elapsed_time(b) for a, b in zip(starts, stops))
    ms_per_step = statistics.median(step_ms)
    ms_mean = sum(step_ms) / len(step_ms)
    ms_region = starts[0].elapsed_time(stops[-1]) / args.steps

    # Per-kernel durations: the same number of steps again, every library launch
    # bracketed by a pair of hipEvents on the launch stream.  Kept out of the
    # region above because the markers themselves add ~20 us to a step.
    kernels = {}
    if not args.no_kernel_timing:
        log(f"timing {args.steps} steps per kernel")
        pk.pkv_timing_enable(4 * args.steps + 64)
        for _ in range(args.steps):
            ds.step(stream)
        torch.cuda.synchronize()
        dropped = pk.pkv_timing_collect()
        for kind in range(pk.PKV_KERNEL_KINDS):
            ms, n = pk.pkv_timing_get(kind)
            if n:
                kernels[pk.pkv_kernel_name(kind)] = {"avg_us": round(1000 * ms / n, 3), "launches": n}
        pk.pkv_timing_disable()
        if dropped:
            log(f"warning: {dropped} launches were not timed")

    value = alg["unique"] / (ms_per_step / 1e3) / 1e9
    roofline = None
    # the kernel that reads the step's KV: the decode kernel that ran, or the fused
    # prefill + decode kernel of a mixed step
    timed = [k for k in (pk.pkv_kernel_name(pk.PKV_KERNEL_DECODE),
                         pk.pkv_kernel_name(pk.PKV_KERNEL_DECODE_MFMA),
                         pk.pkv_kernel_name(pk.PKV_KERNEL_STEP_MFMA)) if k in kernels]
    dom = timed[0] if timed else None
    if dom in kernels:
        meas = measured_counters(args.workload, dom)
        secs = kernels[dom]["avg_us"] / 1e6
        if int((p.query_lens == 1).sum()) == 0:
            # prompt rows only: the tile's matrix work bounds it, not its few KV bytes
            flops = attention_flops(p)
            achieved = flops / secs / 1e12
            roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                        "traffic": meas.get("hbm_bytes_per_launch"),
                        "algorithmic_flops_per_launch": flops}
        else:
            achieved = alg["unique"] / secs / 1e9
            roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": meas.get("hbm_bytes_per_launch"),
                        "algorithmic_bytes_per_launch": alg["unique"]}
        roofline["l2_hit_rate"] = meas.get("tcc_hit_rate")
        roofline["mfma_busy"] = meas.get("mfma_busy_frac")
    # a device copy's read + write rate on the same GPU, for reference
    copy_gbs = copy_bandwidth(torch)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_stat": "median of the K steps, each between a pair of HIP events",
        "ms_per_step_mean": round(ms_mean, 5),
        "ms_per_step_p10_p90": [round(step_ms[len(step_ms) // 10], 5),
                                round(step_ms[(9 * len(step_ms)) // 10], 5)],
        "ms_per_step_region": round(ms_region, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f16": "f16", "bf16": "bf16", "fp8_e4m3": "fp8_e4m3"}[cfg.kv_dtype],
        "data": "synthetic (seeded N(0,1) q/K/V, seeded block placement)",
        "config": {
            "workload": args.workload,
            "description": cfg.description,
            "num_seqs": p.num_seqs,
            "query_rows": p.total_q_tokens,
            "num_q_heads": cfg.num_q_heads,
            "num_kv_heads": cfg.num_kv_heads,
            "head_dim": cfg.head_dim,
            "block_size": cfg.block_size,
            "kv_dtype": cfg.kv_dtype,
            "context_tokens": alg["logical_tokens"],
            "algorithmic_kv_bytes": alg["unique"],
            "appended_rows": int(len(wl.slot_mapping)),
        },
        "batch_steps_per_s": round(1000.0 / ms_per_step, 2),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "copy_gbs": round(copy_gbs, 1),
        "pct_of_copy": round(100 * value / copy_gbs, 2),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
