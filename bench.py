"""Benchmark of the MI355X BoB path on the headline workload (one GPU).

One step = one exact BoB call (pass 1 + pass 2) over the resident inputs of
the B=1, H=4, N=65536, d=64 bf16 workload. Prints ONE JSON line on stdout:
throughput (TFLOP/s with the fixed count 34 B H N^2 d), ms per step, the
roofline of the dominant step of the schedule (the method's algorithmic flops
of that step over its average time, from HIP events on the launch stream),
and the fp64 CPU oracle timed on a bounded sample of the same workload.
Everything else goes to stderr.

Work accounting: the method's two passes do 5 and 12 N x N x d products
(34 B H N^2 d flops per call). This implementation runs pass 2 as two
launches that together execute 17 products (9 query-side, 8 key-side; the
5 recompute products are done by both), so pass 2 is timed and credited as
one step over its two launches with the method's 12 products; the executed
counts are reported beside it, not credited.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload IDX]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "BoB TFLOP/s + ms/call at N=65536,d=64 (1 MI355X); % of bf16 MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # MI355X published dense MFMA peaks
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_util.json")
KERNEL_SOURCES = ("exact_second_order_amd/csrc/bob_query.hip", "exact_second_order_amd/csrc/bob_key.hip",
                  "exact_second_order_amd/csrc/bob_device.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the kernel sources' code: `//` comments, trailing blanks and
    empty lines are left out, so the recorded counters survive comment edits."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(stage, causal=False, workload="bob_b1h4n65536d64_bf16"):
    """HBM bytes per launch of `stage` from committed rocprofv3 counters, if
    they were taken on the current kernel sources, the same workload and the
    same mask; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch_causal" if causal else "bytes_per_launch", {}).get(stage)


def measured_mfma(stage, workload="bob_b1h4n65536d64_bf16"):
    """MFMA utilisation and shader clock of `stage` from committed rocprofv3
    counters (unmasked), if taken on the current kernel sources and the same
    workload; else None."""
    try:
        with open(MFMA_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t.get("kernels", {}).get(stage)


# N x N x d products (2 N^2 d flops each). Credited: the method's two passes
# (pass 1: S, G (2), dP, H; pass 2: the recompute plus gradK (2), gradV,
# gradQ (2), graddO (2)); with the first backward also dQ, dK, dV. Executed:
# what each launch runs (pass 2's two sweeps both recompute).
STEP_LAUNCHES = {"pass1": ["pass1"], "pass2": ["pass2_query", "pass2_key"]}


def method_units(first_backward):
    return {"pass1": 5, "pass2": 15 if first_backward else 12}


def executed_units(first_backward):
    return ({"pass1": 5, "pass2_query": 10, "pass2_key": 10} if first_backward
            else {"pass1": 5, "pass2_query": 9, "pass2_key": 8})


def step_accounting(launch_ms, unit_flops, peak, first_backward=False):
    """Per step of the schedule: time (sum of its launches' average times),
    the method's products, TFLOP/s and fraction of `peak` they give."""
    mu = method_units(first_backward)
    out = {}
    for sn, launches in STEP_LAUNCHES.items():
        ms = sum(launch_ms[k] for k in launches)
        tf = mu[sn] * unit_flops / (ms * 1e-3) / 1e12
        out[sn] = {"ms": round(ms, 4), "units": mu[sn], "tflops": round(tf, 2), "frac": round(tf / peak, 4),
                   "launches": launches}
    return out


CEILING_EXE = os.path.join(ROOT, "exact_second_order_amd", "_build", "mfma_ceiling")


def mfma_ceiling():
    """Sustained 32x32x16 (and 16x16x32) bf16 MFMA rate of this GPU under its
    power limit (random-normal operands changing every instruction, and
    zeros), from the standalone program built next to the library; run as a
    child process after the timed region. None if it is missing or fails."""
    import subprocess
    if not os.path.exists(CEILING_EXE):
        log("[bench] mfma ceiling: program not built (run build())")
        return None
    try:
        res = subprocess.run([CEILING_EXE], capture_output=True, text=True, timeout=120)
    except (OSError, subprocess.TimeoutExpired) as e:
        log(f"[bench] mfma ceiling failed: {e}")
        return None
    if res.returncode != 0:
        log(f"[bench] mfma ceiling failed ({res.returncode}): {res.stderr.strip()[-500:]}")
        return None
    try:
        return json.loads(res.stdout.strip().splitlines()[-1])
    except (ValueError, IndexError):
        log(f"[bench] mfma ceiling: unreadable output {res.stdout[-300:]!r}")
        return None


def cpu_baseline(w, rows, block=512, causal=False):
    """fp64 oracle on `rows` query rows against all keys of head 0 (a bounded
    sample of the workload), scaled to TFLOP/s with the same flop convention
    (causal: the sampled rows are the first ones, credited with the key pairs
    they see)."""
    import numpy as np
    import oracle
    from exact_second_order_amd.inputs import workload_inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=os.cpu_count())
    except Exception:  # threadpoolctl missing: report the visible cpus
        cores = len(os.sched_getaffinity(0))
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    ins = workload_inputs(w)
    xs = [ins[k][0, 0].to(dtype=__import__("torch").float64).numpy() for k in
          ("Q", "K", "V", "dO", "gQ", "gK", "gV")]
    # query-side inputs restricted to the sampled rows; causal: the first
    # `rows` queries see only the first `rows` keys, so that prefix is an exact
    # causal problem of its own
    for i in (range(7) if causal else (0, 3, 4)):
        xs[i] = np.ascontiguousarray(xs[i][:rows])
    t0 = time.perf_counter()
    oracle.bob_blocked_head(*xs, w.scale, block=block, causal=causal)
    dt = time.perf_counter() - t0
    pairs = rows * (rows + 1) / 2 if causal else rows * w.N
    flops = 34.0 * pairs * w.d
    what = f"the first {rows} query rows (causal)" if causal else f"{rows} query rows x all {w.N} keys"
    rate = flops / dt
    # the whole call at the sampled rate (an extrapolation, not a run): all
    # B*H heads, all visible (query, key) pairs
    full_pairs = w.B * w.H * (w.N * (w.N + 1) / 2 if causal else float(w.N) * w.N)
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "cpu_model": cpu_model,
            "kind": "oracle",
            "sample": f"{what} of one head (d={w.d}), fp64 row-blocked oracle, {dt:.2f} s; "
                      f"flops counted as 34*d per visible (query, key) pair",
            "extrapolated_full_call_s": round(34.0 * full_pairs * w.d / rate, 1),
            "extrapolation": "the whole workload (all heads and rows) at the sampled rate; not run"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, help="index into the workload table")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="oracle sample size in query rows (default 16384; 32768 with --causal)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--causal", action="store_true",
                    help="causal masking (not the headline); flops credited for the N(N+1)/2 visible pairs")
    ap.add_argument("--first-backward", action="store_true",
                    help="also return the first backward dQ, dK, dV (not the headline); credited with its "
                         "three extra products")
    ap.add_argument("--saved-lse", action="store_true",
                    help="pass 1 starts from a saved log-sum-exp (computed once before timing, as a forward "
                         "would have kept it)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the sustained-MFMA measurement after the timed region")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB first (calibrates HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(heads shard with no exchange; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from exact_second_order_amd import flashbob as fb
    from exact_second_order_amd.inputs import NAMES, WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] workload {w.name}: generating inputs")
    ins = workload_inputs(w)
    x = [ins[k].to(dev) for k in NAMES]
    out = tuple(torch.empty(x[0].shape, dtype=torch.float32, device=dev) for _ in range(4))
    ws = torch.empty(fb.workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    first = (tuple(torch.empty(x[0].shape, dtype=torch.float32, device=dev) for _ in range(3))
             if args.first_backward else None)
    stream = torch.cuda.current_stream(dev)
    lse = fb.rowstats(*x, scale=w.scale, causal=args.causal)[0] if args.saved_lse else None
    if args.copy_mb > 0:
        src = torch.ones(args.copy_mb << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {args.copy_mb} MiB read + {args.copy_mb} MiB written")
        del src, dst

    stages = list(fb.STAGES)
    mu, eu, step_launches = method_units(args.first_backward), executed_units(args.first_backward), STEP_LAUNCHES
    kernel_names = {"pass1": "query_kernel<.., false>",
                    "pass2": "query_kernel<.., true> + key_kernel (pass 2: two launches)"}

    def step(ev=None):
        """One BoB call: the library's single entry point (its three kernels
        launched back to back on the stream)."""
        if ev is not None:
            ev[0].record(stream)
        fb.bob(*x, scale=w.scale, out=out, workspace=ws, causal=args.causal, first_backward=first is not None,
               first_out=first, lse=lse)
        if ev is not None:
            ev[1].record(stream)

    def staged_step(ev):
        """The same call as its three stage calls with events between them
        (the per-kernel breakdown, timed apart from the headline figure)."""
        for i, st in enumerate(stages):
            ev[i].record(stream)
            fb.bob_stage(st, *x, out=out, workspace=ws, scale=w.scale, causal=args.causal, first=first,
                         lse=lse if st == "pass1" else None)
        ev[len(stages)].record(stream)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-kernel breakdown: the same number of steps again, stage by stage
    kevs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        staged_step(kevs[i])
    torch.cuda.synchronize()

    ms_step = wall * 1e3 / args.steps
    # device memory the timed calls added on top of inputs, outputs and
    # workspace (the library allocates nothing: expected 0)
    peak_mem_delta = torch.cuda.max_memory_allocated(dev) - mem0
    step_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    ms_median = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (
        step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])
    frac_pairs = (w.N + 1) / (2.0 * w.N) if args.causal else 1.0  # visible (query, key) pairs
    # credited: the 17 products of the method (not the 22 the kernels execute),
    # plus the first backward's three when it is returned
    flops = (w.flops + (6.0 * w.B * w.H * w.N * w.N * w.d if args.first_backward else 0.0)) * frac_pairs
    tflops = flops / (ms_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype_name]
    unit_flops = 2.0 * w.B * w.H * w.N * w.N * w.d * frac_pairs
    per_kernel = {}
    for i, st in enumerate(stages):
        ms = sum(e[i].elapsed_time(e[i + 1]) for e in kevs) / args.steps
        per_kernel[st] = {"ms": round(ms, 4), "executed_units": eu[st],
                          "executed_tflops": round(eu[st] * unit_flops / (ms * 1e-3) / 1e12, 2)}
    per_step = step_accounting({k: v["ms"] for k, v in per_kernel.items()}, unit_flops, peak, args.first_backward)
    # counter-derived figures (committed profiles of the plain headline run)
    plain = not (args.causal or args.first_backward or args.saved_lse)
    for st in stages:
        traffic = (measured_traffic(st, args.causal, w.name)
                   if not (args.first_backward or args.saved_lse) else None)
        if traffic is not None:
            per_kernel[st]["hbm_bytes"] = int(traffic)
            per_kernel[st]["hbm_GBps"] = round(traffic / (per_kernel[st]["ms"] * 1e-3) / 1e9, 1)
        m = measured_mfma(st, w.name) if plain else None
        if m is not None:
            per_kernel[st]["mfma_util"] = round(m["mfma_util"], 4)
            per_kernel[st]["sclk_ghz"] = round(m["sclk_ghz"], 3)
    # the peak at the shader clock the counters measured under load (the
    # published peak assumes 2.4 GHz; the chip runs slower when power-limited)
    for sn, launches in step_launches.items():
        clk = [per_kernel[k].get("sclk_ghz") for k in launches]
        if all(c is not None for c in clk):
            t = [per_kernel[k]["ms"] for k in launches]
            sclk = sum(c * tt for c, tt in zip(clk, t)) / sum(t)  # time-weighted
            per_step[sn]["sclk_ghz"] = round(sclk, 3)
            per_step[sn]["frac_at_sclk"] = round(per_step[sn]["tflops"] / (peak * sclk / 2.4), 4)
        tr = [per_kernel[k].get("hbm_bytes") for k in launches]
        per_step[sn]["hbm_bytes"] = int(sum(tr)) if all(x is not None for x in tr) else None
    log(f"[bench] ms/step {ms_step:.3f}; {tflops:.1f} TFLOP/s = {100 * tflops / peak:.1f}% of {peak} peak; "
        f"steps {per_step}; launches {per_kernel}")
    dom = max(per_step, key=lambda sn: per_step[sn]["ms"])
    roofline = {"bound": "mfma", "achieved": per_step[dom]["tflops"], "peak": peak, "unit": "TFLOP/s",
                "frac": per_step[dom]["frac"],
                "traffic": (None if (args.first_backward or args.saved_lse) else per_step[dom]["hbm_bytes"]),
                "kernel": kernel_names[dom], "step": dom, "launch_ms": per_step[dom]["ms"],
                "credited_units": mu[dom], "executed_units": sum(eu[k] for k in step_launches[dom])}
    if "frac_at_sclk" in per_step[dom]:
        roofline["sclk_ghz"] = per_step[dom]["sclk_ghz"]
        roofline["frac_at_sclk"] = per_step[dom]["frac_at_sclk"]
    # what the kernels execute (pass 2 recomputes the score tiles in both
    # sweeps), against the MFMA rate this GPU sustains under its power limit
    roofline["executed_tflops"] = round(roofline["executed_units"] * unit_flops
                                        / (per_step[dom]["ms"] * 1e-3) / 1e12, 2)
    if not args.no_ceiling and w.dtype_name == "bf16":
        ceil = mfma_ceiling()
        if ceil is not None:
            log(f"[bench] mfma ceiling {ceil}")
            roofline["mfma_ceiling"] = {"tflops": ceil["random"]["tflops"], "sclk_ghz": ceil["random"]["sclk_ghz"],
                                        "zero_operands_tflops": ceil["zero"]["tflops"],
                                        "instruction": ceil["instruction"]}
            # the 16-row tile instruction under the same limit
            m16 = ceil.get("v_mfma_f32_16x16x32_bf16")
            if m16:
                roofline["mfma_ceiling"]["tflops_16x16x32"] = m16["random"]["tflops"]
            roofline["executed_frac_of_ceiling"] = round(roofline["executed_tflops"] / ceil["random"]["tflops"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        rows = args.cpu_rows or (32768 if args.causal else 16384)
        log(f"[bench] cpu baseline: oracle on {rows} query rows")
        cpu = cpu_baseline(w, min(rows, w.N), causal=args.causal)
        log(f"[bench] cpu baseline {cpu['value']} TFLOP/s on {cpu['cores']} threads")

    res = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype_name,
        "data": "synthetic",
        "config": {"workload": w.name + ("_causal" if args.causal else "") + ("_first" if args.first_backward else "")
                   + ("_savedlse" if args.saved_lse else ""),
                   "B": w.B, "H": w.H, "N": w.N,
                   "d": w.d, "dtype": w.dtype_name, "scale": w.scale, "causal": bool(args.causal),
                   "first_backward": bool(args.first_backward), "saved_lse": bool(args.saved_lse), "seed": WORKLOADS.index(w),
                   "flops_per_step": flops, "frac_of_peak": round(tflops / peak, 4),
                   "ms_median_events": round(ms_median, 4), "ms_min_events": round(step_ms[0], 4),
                   "peak_mem_delta_bytes": int(peak_mem_delta), "steps": per_step, "kernels": per_kernel},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
