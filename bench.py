#!/usr/bin/env python3
"""Benchmark of the NVFP4 block-scaled batched GEMV on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload headline]

A step is one GEMV call (the whole path: A/SFA stream, b' staging, decode,
FMA, reduction, float16 store) over one input set. Input sets are seeded,
synthetic and already resident in HBM; consecutive steps rotate through enough
distinct sets (>= 512 MiB together) that neither the L2s nor the 256 MiB
Infinity Cache hold the next step's operands.

Order of work on the GPU:
  * one call on input set 0, its output copied to the host (checked against
    the oracle after the timing, on the CPU);
  * the streaming-read references (libnvfp4bench.so, four read designs) on
    buffers of the same byte count, each timed like the GEMV; the best one is
    reported as ``attainable``;
  * the GEMV: exactly W untimed warmup steps, then a short spin on the GPU
    while the host enqueues a start event, K steps and an end event behind
    it, so the GPU runs the K steps back to back; between two
    synchronisations. ``ms_per_step`` = GPU time between the events / K, and
    ``value`` = ideal bytes / that. The roofline's ``achieved`` is the same
    quotient: one kernel per step, so the average launch duration over the
    timed region (back-to-back launches, gaps included).
Prints exactly one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

def metric_for(M: int, K: int, L: int) -> str:
    """The headline metric's wording, for the workload's shape (the headline
    7168×16384×1 gives exactly the headline metric)."""
    return f"µs/call and achieved HBM GB/s (% of peak) for NVFP4 GEMV {M}×{K}×{L}"


METRIC = metric_for(7168, 16384, 1)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
ROTATE_BYTES = 512 * 2 ** 20
WORKLOADS = {"headline": synth.HEADLINE, "balanced": synth.BALANCED, "batched": synth.BATCHED,
             "tiny": synth.TINY, "shard": synth.SHARD}
for _w in synth.EDGE:
    WORKLOADS[_w.name] = _w


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """sha256 prefix of the GEMV kernel's sources (the kernel file, then its device header)."""
    h = hashlib.sha256()
    for f in ("nvfp4_gemv.hip", "nvfp4_device.h"):
        h.update(open(os.path.join(ROOT, "block_scaled_fp4_gemv_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload_name: str, layout: str):
    """HBM traffic per launch from a committed counter summary, if it was taken
    on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}_{layout}.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


BOX_CPU_SHARE = 16   # host threads a one-GPU machine allots to a job
SUBMIT_SPIN_CYCLES = 4_000_000   # GPU clock cycles (about 2 ms) of spin ahead of the timed steps
SPIN_CYCLES_PER_STEP = 60_000    # and at least this much per timed step (host enqueue time)


def cpu_baseline(w, layout: str, budget_s: float):
    """The oracle as it stands (never tuned for this) on input set 0: the
    median of 3 timed runs on the one-GPU machine's CPU share (16 threads, fewer if
    the host has fewer), and the median of 3 on one thread, each over a row
    sample (rows repeat past M*L) scaled to one full call; about ``budget_s``
    seconds of CPU work in all."""
    import statistics
    import oracle
    oracle.build(force=False)
    host = os.cpu_count() or 1
    nth = min(host, BOX_CPU_SHARE)
    inp = synth.make_inputs(w, 0)
    rows_total = w.M * w.L

    def sec_per_row(nthreads: int, nrows: int) -> float:
        rows = np.arange(nrows, dtype=np.int64) % rows_total
        t0 = time.perf_counter()
        oracle.gemv_rows(inp, rows, layout, nthreads=nthreads)
        return (time.perf_counter() - t0) / nrows

    share = budget_s / 6.0                               # 3 runs on each setting
    out = {}
    for label, threads in (("multi", nth), ("one", 1)):
        probe = sec_per_row(threads, max(64, 8 * threads))
        nrows = int(max(8 * threads, min(50 * rows_total, share / probe)))
        times = [sec_per_row(threads, nrows) * rows_total for _ in range(3)]
        out[label] = (statistics.median(times), nrows)
    sec, nrows = out["multi"]
    sec1, nrows1 = out["one"]
    return {"value": round(w.ideal_bytes / sec / 1e9, 4), "unit": "GB/s", "cores": nth, "kind": "oracle",
            "sample": (f"median of 3 runs of {nrows} rows ({nth} threads) and of 3 runs of {nrows1} rows "
                       f"(1 thread) of {w.name} input set 0, {layout} scales, each scaled to a full call of "
                       f"{rows_total} rows"),
            "us_per_call": round(sec * 1e6, 1), "host_cpus": host,
            "one_thread": {"value": round(w.ideal_bytes / sec1 / 1e9, 4), "unit": "GB/s",
                           "us_per_call": round(sec1 * 1e6, 1)}}


def timed_steps(step, steps: int, warmup: int):
    """Launch exactly ``warmup`` untimed steps, then a spin on the GPU long
    enough for the host to enqueue the start event, ``steps`` timed steps and
    the end event behind it, so that the GPU runs the timed steps back to back
    (no host launch latency inside the interval). For the headline a HIP
    graph replay measured the same per-step time over 200 steps and carries a
    fixed cost of its own that matters at 20; the batched workload's kernels
    run 1.3-2.7 us faster per call in a graph replay, and the eager time is
    what is reported. Returns (ms per step, warmup)."""
    import torch
    st = torch.cuda.current_stream()
    torch.cuda.synchronize()
    for i in range(warmup):
        step(i, st)
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(max(SUBMIT_SPIN_CYCLES, SPIN_CYCLES_PER_STEP * steps))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        step(i, st)
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps, warmup


def attainable_read(nbytes: int, steps: int, warmup: int, dev):
    """The streaming-read reference in each design on rotating random buffers
    of about ``nbytes`` (rounded down to the design's unit), timed like the
    GEMV. Returns (the design with the highest GB/s, {design: us per call})."""
    import torch
    from block_scaled_fp4_gemv_amd import benchlib
    per_mode = {}
    best = None
    gen = torch.Generator(device=dev)
    gen.manual_seed(12345)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    for mode in sorted(benchlib.STREAM_READ_MODES):
        unit = benchlib.stream_read_unit(mode)
        rd_bytes = nbytes // unit * unit
        if rd_bytes == 0:
            continue
        rd_sets = max(1, min(64, -(-ROTATE_BYTES // rd_bytes)))
        # random bytes, like the GEMV's operands (HBM power, and so clocks, depend on the data)
        bufs = [torch.randint(0, 256, (rd_bytes,), dtype=torch.uint8, device=dev, generator=gen)
                for _ in range(rd_sets)]

        def rd_step(i, stream=None, mode=mode, bufs=bufs, rd_bytes=rd_bytes, rd_sets=rd_sets):
            benchlib.stream_read(bufs[i % rd_sets], rd_bytes, sink, mode, stream)
        ms, _ = timed_steps(rd_step, steps, warmup)
        gbs = rd_bytes / (ms * 1e-3) / 1e9
        per_mode[str(mode)] = {"bytes": rd_bytes, "us_per_call": round(ms * 1e3, 3), "GB/s": round(gbs, 2)}
        log(f"attainable: read design {mode}, {rd_bytes} B: {ms * 1e3:.3f} us per call, {gbs:.0f} GB/s")
        if best is None or gbs > best[1]:
            best = (mode, gbs, rd_bytes, ms)
        del bufs
    if best is None:
        return None, per_mode
    mode, gbs, rd_bytes, ms = best
    return ({"kind": "streaming read of the same byte count (libnvfp4bench.so)",
             "design": benchlib.STREAM_READ_MODES[mode], "bytes": rd_bytes, "us_per_call": round(ms * 1e3, 3),
             "GB/s": round(gbs, 2), "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
             "by_design": per_mode}, per_mode)


def bench_small_n(args, w, dev):
    """N-vector skinny GEMM on the workload's A: HBM bytes = A + SFA + N vectors
    of B and SFB + the N float16 columns of C."""
    import torch
    import block_scaled_fp4_gemv_amd as g
    M, K, L, N, layout = w.M, w.K, w.L, args.small_n, args.layout
    sizes = g.small_n_operand_bytes(M, N, K, L, layout)
    ideal = L * (M * K // 2 + M * K // 16 + N * (K // 2 + K // 16) + 2 * N * M)
    per_set = sizes["a"] + sizes["sfa"]
    nsets = max(1, min(64, -(-ROTATE_BYTES // per_set)))
    log(f"small-N {w.name} N={N}: {nsets} sets of {per_set / 1e6:.1f} MB")
    rng = np.random.default_rng([7, M, N, K, L])
    b_codes = synth.pack_nibbles(rng.integers(0, 16, (L, N, K), dtype=np.uint8))
    sfb_plain = synth.scale_codes(rng, (L, N, K // 16))
    sfb_host = synth.to_blocked(sfb_plain, pad=0) if layout == "blocked" else sfb_plain
    b_dev, sfb_dev = torch.from_numpy(b_codes).to(dev), torch.from_numpy(np.ascontiguousarray(sfb_host)).to(dev)
    sets = []
    for i in range(nsets):
        inp = synth.make_inputs(w, i)
        sets.append((torch.from_numpy(inp.a).to(dev), torch.from_numpy(inp.sfa(layout)).to(dev),
                     torch.empty(L * N * M, dtype=torch.float16, device=dev)))
        if i == 0:
            inp0 = inp

    def step(i, stream=None):
        a, sfa, c = sets[i % nsets]
        g.nvfp4_gemm_small_n(a, b_dev, sfa, sfb_dev, c, M, N, K, L, layout, 1.0, stream)
    step(0)
    torch.cuda.synchronize()
    verified = None
    if not args.no_verify:
        import oracle
        oracle.build(force=False)
        step(0)
        torch.cuda.synchronize()
        got = sets[0][2].cpu().view(torch.int16).numpy().view(np.uint16).reshape(L, N, M)
        ref = oracle.gemm_small_n(inp0.a, b_codes, inp0.sfa_plain, sfb_plain, M, N, K, L,
                                  nthreads=min(os.cpu_count() or 1, 16))
        verified = bool(oracle.check(got, ref).all())
        log(f"small-N parity vs oracle on set 0: {'ok' if verified else 'FAILED'}")
    ms, warm = timed_steps(step, args.steps, args.warmup)
    gbs = ideal / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": f"µs/call and achieved HBM GB/s of the {N}-vector NVFP4 skinny GEMM",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": warm,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"small_n{N}_{w.name}", "M": M, "N": N, "K": K, "L": L, "sf_layout": layout,
                   "ideal_bytes_per_call": ideal, "plan": g.nvfp4_gemm_small_n_plan(M, N, K, L, layout)},
        "us_per_call": round(ms * 1e3, 3), "verified_vs_oracle": verified,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}}), flush=True)


def bench_reblock(args, w, dev):
    """Device reblock of the workload's plain SFA [L][M][K/16] into the 128x4
    blocked layout: HBM bytes = plain read + blocked write."""
    import torch
    import block_scaled_fp4_gemv_amd as g
    M, K, L = w.M, w.K, w.L
    in_bytes = L * M * (K // 16)
    out_bytes = g.nvfp4_blocked_scales_bytes(M, K, L)
    nsets = max(1, min(64, -(-ROTATE_BYTES // (in_bytes + out_bytes))))
    log(f"reblock {w.name}: {nsets} sets of {in_bytes / 1e6:.2f} MB plain -> {out_bytes / 1e6:.2f} MB blocked")
    plains, outs = [], []
    for i in range(nsets):
        plains.append(torch.from_numpy(synth.make_inputs(w, i).sfa_plain).to(dev))
        outs.append(torch.empty(out_bytes, dtype=torch.uint8, device=dev))
    verified = None
    if not args.no_verify:
        import oracle
        oracle.build(force=False)
        g.nvfp4_scales_to_blocked(plains[0], outs[0], M, K, L)
        torch.cuda.synchronize()
        want = oracle.reblock(plains[0].cpu().numpy(), M, K, L).reshape(-1)
        verified = bool(np.array_equal(outs[0].cpu().numpy(), want))
        log(f"reblock parity vs oracle: {'ok' if verified else 'FAILED'}")
    def rstep(i, stream=None):
        g.nvfp4_scales_to_blocked(plains[i % nsets], outs[i % nsets], M, K, L, stream)
    ms, warm = timed_steps(rstep, args.steps, args.warmup)
    gbs = (in_bytes + out_bytes) / (ms * 1e-3) / 1e9
    out = {"metric": "µs/call and achieved HBM GB/s of the plain -> 128x4 blocked SFA reblock",
           "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": warm, "ms_per_step": round(ms, 6), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
           "config": {"workload": f"reblock_sfa_{w.name}", "rows": M, "K": K, "L": L,
                      "plain_bytes": in_bytes, "blocked_bytes": out_bytes, "rotating_sets": nsets},
           "us_per_call": round(ms * 1e3, 3), "verified_vs_oracle": verified,
           "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}}
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        p0 = plains[0].cpu().numpy()
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.reblock(p0, M, K, L)
            reps += 1
            el = time.perf_counter() - t0
            if el >= min(args.cpu_budget, 5.0) or reps >= 50:
                break
        out["cpu_baseline"] = {"value": round((in_bytes + out_bytes) / (el / reps) / 1e9, 4), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{reps} full reblocks of input set 0", "us_per_call": round(el / reps * 1e6, 1)}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps right before the timed steps")
    ap.add_argument("--workload", default="headline", choices=sorted(WORKLOADS))
    ap.add_argument("--layout", default="blocked", choices=["blocked", "plain"])
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--no-attainable", action="store_true", help="skip the streaming-read references")
    ap.add_argument("--small-n", type=int, default=0, metavar="N",
                    help="time the N-vector skinny GEMM (N = 1..8) on the workload's A instead "
                         "(its own JSON line)")
    ap.add_argument("--reblock", action="store_true",
                    help="time the device plain -> blocked reblock of the workload's SFA instead "
                         "(its own JSON line)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run torch's device copy of BYTES bytes --steps times (a plain copy "
                         "kernel of known size, to scale hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this GEMV is built and timed on a single "
              "MI355X (no multi-GPU path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_fp4_gemv_amd as g

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": args.steps}), flush=True)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    if args.reblock:
        bench_reblock(args, w, dev)
        return
    if args.small_n:
        bench_small_n(args, w, dev)
        return
    layout = args.layout
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), {props.multi_processor_count} CUs")

    # ---- rotating input sets, resident in HBM
    per_set = w.ideal_read_bytes
    nsets = max(1, min(64, -(-ROTATE_BYTES // per_set)))
    log(f"workload {w.name}: {nsets} input sets of {per_set / 1e6:.1f} MB")
    sets = []
    for i in range(nsets):
        inp = synth.make_inputs(w, i)
        sets.append(dict(
            a=torch.from_numpy(inp.a).to(dev), b=torch.from_numpy(inp.b).to(dev),
            sfa=torch.from_numpy(inp.sfa(layout)).to(dev), sfb=torch.from_numpy(inp.sfb(layout)).to(dev),
            c=torch.empty(w.L * w.M, dtype=torch.float16, device=dev)))
        if i == 0:
            inp0 = inp
    torch.cuda.synchronize()
    M, K, L = w.M, w.K, w.L
    plan = g.nvfp4_gemv_plan(M, K, L)
    log(f"plan: {plan}")

    def step(i, stream=None):
        s = sets[i % nsets]
        g.nvfp4_gemv(s["a"], s["b"], s["sfa"], s["sfb"], s["c"], M, K, L, layout, stream)

    # ---- one call first (allocates any split-K workspace before timing
    # capture); its output is checked against the oracle after the timing
    step(0)
    torch.cuda.synchronize()
    got0 = sets[0]["c"].cpu().view(torch.int16).numpy().view(np.uint16).reshape(L, M).copy()
    K_steps = args.steps

    # ---- attainable: streaming reads of the same byte count, each design
    # timed like the GEMV
    attainable = None
    if not args.no_attainable:
        attainable, _ = attainable_read(w.ideal_bytes, K_steps, args.warmup, dev)

    # ---- the timed region: exactly W warmup steps, then K back-to-back steps
    t0 = time.perf_counter()
    ms_per_step, warm = timed_steps(step, K_steps, args.warmup)
    wall_s = time.perf_counter() - t0
    log(f"timed: {K_steps} steps after {warm} warmup steps, {ms_per_step * K_steps:.3f} ms GPU "
        f"({wall_s * 1e3:.1f} ms wall incl. warmup)")

    # ---- correctness of the benchmarked configuration (set 0) against the oracle
    verified = None
    if not args.no_verify:
        import oracle
        oracle.build(force=False)
        ref = oracle.gemv(inp0, layout, nthreads=min(os.cpu_count() or 1, BOX_CPU_SHARE))
        verified = bool(oracle.check(got0, ref).all())
        log(f"parity vs oracle on set 0: {'ok' if verified else 'FAILED'}")

    ideal = w.ideal_bytes
    value_gbs = ideal / (ms_per_step * 1e-3) / 1e9
    achieved = ideal / (ms_per_step * 1e-3) / 1e9     # average launch over the timed region
    traffic = traffic_from_profile(w.name, layout)
    out = {
        "metric": metric_for(M, K, L),
        "value": round(value_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": warm,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "M": M, "K": K, "L": L, "N": 1, "sf_layout": layout,
                   "rotating_sets": nsets, "ideal_bytes_per_call": ideal, "plan": plan},
        "us_per_call": round(ms_per_step * 1e3, 3),
        "pct_of_peak": round(100 * value_gbs / PEAK_HBM_GBS, 2),
        "verified_vs_oracle": verified,
        "attainable": attainable,
        # GB/s of the GEMV over GB/s of the streaming read
        "pct_of_attainable": round(100 * value_gbs / attainable["GB/s"], 2) if attainable else None,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic},
        "context": {"b200_target_us_from_pages": {"headline_7168x16384x1": 8.6,
                                                  "batched_4096x7168x8": 17.3,
                                                  "balanced_7168x2048x4": 4.3}},
        "device": props.name,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(w, layout, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
