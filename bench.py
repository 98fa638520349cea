#!/usr/bin/env python3
"""Benchmark of the MoE layer forward pass on one MI355X.

One step = one moe_forward call (router GEMM + gating, permutation and
gather, grouped expert GEMMs, combine) over one batch of seeded synthetic
tokens already resident in HBM.  Prints ONE JSON line on stdout.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME]
                  [--no-cpu-baseline] [--cpu-seconds 15]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/sec + TFLOP/s (% bf16 MFMA peak), Mixtral-shape prefill"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def active_flops(spec, counts):
    """Router GEMM plus the expert GEMMs of the kept assignments (and the shared
    expert); elementwise work, softmax and the combine are not counted."""
    mult = 3 if spec.act == "swiglu" else 2
    router = 2.0 * spec.T * spec.d * spec.E
    experts = 2.0 * float(sum(counts)) * spec.d * spec.F * mult
    shared = 2.0 * spec.T * spec.d * spec.F_shared * 3 * spec.num_shared if spec.F_shared else 0.0
    return router + experts + shared


def kernel_work(spec, counts, name):
    """Algorithmic (flops, HBM bytes) of one step's launches of kernel `name`:
    what the step must compute, read and write once (x once, the weights of
    every expert that received rows once, each intermediate written and read
    once, routing metadata); re-reads caused by tiling are not counted."""
    eb = 2 if spec.dtype == "bf16" else 4
    T, d, E, F, Fs = spec.T, spec.d, spec.E, spec.F, spec.F_shared * spec.num_shared  # shared: S stacked experts
    ec = spec.gating == "expert_choice"
    rows = float(sum(counts))                      # kept (routed) rows
    touched = sum(1 for c in counts if c > 0)      # experts that received rows
    slots = rows if ec else float(T * spec.k)      # gate slots the combine walks
    nw = 2 if spec.act == "swiglu" else 1
    if name == "route":
        return 2.0 * T * d * E, eb * (T * d + E * d) + 4.0 * T * E + (0.0 if ec else 8.0 * T * spec.k)
    if name == "route_gate":  # logits once in and out, selections out (the K-split parts are tiling re-reads)
        return 0.0, 8.0 * T * E + 8.0 * T * spec.k
    if name == "ec_select":
        return 0.0, 4.0 * T * E + 8.0 * rows
    if name == "permute_count":
        return 0.0, 4.0 * slots + 4.0 * E
    if name == "permute_scan":
        return 0.0, 12.0 * E
    if name == "permute_small":
        return 0.0, 8.0 * slots + 4.0 * rows + 8.0 * E
    if name == "permute_scatter":
        return 0.0, 8.0 * slots + 4.0 * rows
    if name == "ec_permute":
        return 0.0, 4.0 * rows + 4.0 * T * E + 4.0 * rows
    if name == "gather_rows":
        return 0.0, 2.0 * eb * rows * d
    if name == "tile_plan":
        return 0.0, 8.0 * E
    if name == "gemm1_act":
        return 2.0 * rows * d * F * nw, eb * (rows * d + touched * nw * F * d + rows * F)
    if name == "gemm2":
        return 2.0 * rows * F * d, eb * (rows * F + touched * d * F + rows * d)
    if name == "gemm1_act_shared":
        return 4.0 * T * d * Fs, eb * (T * d + 2.0 * Fs * d + T * Fs)
    if name == "gemm2_shared":
        return 2.0 * T * Fs * d, eb * (T * Fs + d * Fs + T * d)
    if name == "combine":
        meta = 4.0 * T * E if ec else 8.0 * slots
        return 0.0, eb * (rows * d + T * d + (T * d if Fs else 0.0)) + meta
    return 0.0, 0.0


def kernel_roofline(spec, flops, nbytes, seconds):
    """Bound from the arithmetic intensity against the ridge point (peak
    flops / peak HBM bandwidth); launch-latency for kernels that move under a
    megabyte and do no matrix work.  Returns (bound, achieved, peak, unit)."""
    peak_f = PEAK_BF16_TFLOPS if spec.dtype == "bf16" else PEAK_F32_TFLOPS
    ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops > 0 and flops / max(nbytes, 1.0) >= ridge:
        return "mfma", flops / seconds / 1e12, peak_f, "TFLOP/s"
    bound = "hbm" if (flops > 0 or nbytes >= 1e6) else "latency"
    return bound, nbytes / seconds / 1e9, PEAK_HBM_GBS, "GB/s"


GEMM_SOURCES = ("gemm.hip", "plan.h", "common.h", "kernels.h")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_mixtral_prefill.md")


def gemm_source_sha():
    """Hash of the grouped-GEMM kernel sources (the counters in TRAFFIC_PROFILE
    hold only for the kernel built from these exact files)."""
    import hashlib
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "sparse_mixture_experts_gating_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE
    summary (rocprofv3, calibrated on a 1 GiB copy), or None when that summary is
    for another workload or an older build of the GEMM kernel."""
    if workload != "mixtral_8x7b_prefill_bf16" or not os.path.exists(TRAFFIC_PROFILE):
        return None
    with open(TRAFFIC_PROFILE) as f:
        line = next((l for l in f if l.startswith("traffic-json: ")), None)
    if line is None:
        return None
    rec = json.loads(line[len("traffic-json: "):])
    if rec.get("gemm_source_sha") != gemm_source_sha() or kernel not in rec.get("kernels", {}):
        return None
    k = rec["kernels"][kernel]
    return dict(bytes=k["fetch_bytes"] + k["write_bytes"], read=k["fetch_bytes"], written=k["write_bytes"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral_8x7b_prefill_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer is not sharded "
              "across GPUs by this library", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_mixture_experts_gating_amd as moe
    import workloads

    spec = workloads.BY_NAME[args.workload]
    dev = "cuda:0"
    moe.load()
    log(f"[bench] generating {spec.name} inputs on {dev}")
    inp = workloads.make_inputs(spec, device=dev)
    cfg = moe.config_from_spec(spec)
    w = moe.make_weights(inp)
    routing = moe.alloc_routing(cfg, dev)
    r = moe.make_routing(routing)
    ws = moe.alloc_workspace(cfg, moe.STAGE_FORWARD, dev)
    y = torch.empty((spec.T, spec.d), dtype=spec.torch_dtype, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        moe.moe_forward(cfg, inp["x"], w, y, r, ws)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / max(args.steps, 1)
    counts = routing["counts"].cpu().numpy().tolist()
    flops = active_flops(spec, counts)
    tokens_per_s = spec.T / (ms / 1e3)
    layer_tflops = flops / (ms / 1e3) / 1e12

    # the same step captured once in a HIP graph and replayed: what a caller
    # that replays the layer pays without per-launch host overhead
    graph_ms = None
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(max(args.warmup, 1)):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
        del g
    except RuntimeError as exc:  # capture not available: report the eager number only
        log(f"[bench] graph capture skipped: {exc}")

    # per-step spread: each step between its own pair of events
    per_step = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        per_step.append(e0.elapsed_time(e1))

    # per-kernel durations from HIP events recorded on the launch stream
    log("[bench] per-kernel event timing")
    moe.moe_timing_reset()
    moe.moe_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    names = moe.moe_kernel_names()
    kern = {}
    for i, n in enumerate(names):
        tot, cnt = moe.moe_timing_read(i)
        if cnt:
            kern[n] = dict(avg_us=round(tot * 1e3 / cnt, 3), launches_per_step=cnt / args.steps)
    moe.moe_timing_enable(False)
    # per-kernel rooflines: algorithmic work per step over the kernel's time per step
    for n, v in kern.items():
        fl, nb = kernel_work(spec, counts, n)
        per_step_s = v["avg_us"] * v["launches_per_step"] * 1e-6
        bound, ach, peak, unit = kernel_roofline(spec, fl, nb, per_step_s)
        v.update(gflop=round(fl / 1e9, 3), mbytes=round(nb / 1e6, 3), bound=bound, achieved=round(ach, 2),
                 unit=unit, frac=round(ach / peak, 4))
    dominant = max(kern, key=lambda n: kern[n]["avg_us"] * kern[n]["launches_per_step"])
    dk = kern[dominant]
    traffic = measured_traffic(spec.name, dominant)
    roofline = dict(bound=dk["bound"], kernel=dominant, achieved=dk["achieved"],
                    peak=PEAK_HBM_GBS if dk["unit"] == "GB/s" else
                    (PEAK_BF16_TFLOPS if spec.dtype == "bf16" else PEAK_F32_TFLOPS),
                    unit=dk["unit"], frac=dk["frac"], traffic=None if traffic is None else traffic["bytes"],
                    avg_launch_us=dk["avg_us"])
    if traffic is not None:
        roofline["traffic_detail"] = dict(unit="bytes per launch", read=traffic["read"], written=traffic["written"],
                                          algorithmic=round(dk["mbytes"] * 1e6 / dk["launches_per_step"]),
                                          source="profiles/hbm_traffic_mixtral_prefill.md")

    # cold-cache step: the 256 MB MALL is overwritten by a 512 MiB fill before
    # each step, outside the event pair
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    n_cold = max(3, min(args.steps, 10))
    for _ in range(n_cold):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        cold.append(e0.elapsed_time(e1))
    cold_ms = float(np.median(cold))
    # the same, per kernel (the fill runs outside the library's event pairs)
    moe.moe_timing_reset()
    moe.moe_timing_enable(True)
    for _ in range(n_cold):
        flush.fill_(1)
        step()
    torch.cuda.synchronize()
    kern_cold = {}
    for i, n in enumerate(names):
        tot, cnt = moe.moe_timing_read(i)
        if cnt:
            kern_cold[n] = round(tot * 1e3 / cnt, 3)
    moe.moe_timing_enable(False)
    del flush

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    # measured HBM rates: context for the HBM-bound kernels (the roofline
    # peak stays the published figure)
    with torch.cuda.stream(stream):
        hbm = measured_bandwidth(torch, dev, stream)
    for v in kern.values():
        if v["unit"] == "GB/s":
            v["frac_of_measured_read"] = round(v["achieved"] / hbm["read_gbps"], 4)
            if v["mbytes"] >= 1.0:
                # the same read at this kernel's own size, launch and ramp
                # included (event-timed like the kernel itself)
                with torch.cuda.stream(stream):
                    t_read = size_matched_read_us(torch, dev, stream, int(v["mbytes"] * 1e6))
                v["size_matched_read_us"] = round(t_read, 3)
                v["frac_of_size_matched_read"] = round(t_read / v["avg_us"], 4)

    cpu = parity = None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(spec, inp, args.cpu_seconds, y, routing)
        # active GFLOP/s at the layer's average active work per token
        cpu["gflops_active"] = round(cpu["value"] * flops / spec.T / 1e9, 3)

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded Gaussian tokens, N(0,1/fan_in) weights)",
        "config": {"workload": spec.name, "tokens": spec.T, "d_model": spec.d, "experts": spec.E,
                   "top_k": spec.k, "d_ff": spec.F, "d_ff_shared": spec.F_shared,
                   "num_shared": spec.num_shared if spec.F_shared else 0, "gating": spec.gating,
                   "activation": spec.act, "parallelism": "none (1 GPU)"},
        "layer_tflops_active": round(layer_tflops, 2),
        "layer_frac_bf16_peak": round(layer_tflops / PEAK_BF16_TFLOPS, 4),
        "step_ms_median": round(float(np.median(per_step)), 4),
        "step_ms_min": round(float(np.min(per_step)), 4),
        # the kernels' event times per step, summed: within a few percent of
        # ms_per_step when launch gaps are small
        "stages_sum_ms": round(sum(v["avg_us"] * v["launches_per_step"] for v in kern.values()) / 1e3, 4),
        "cold_ms_per_step": round(cold_ms, 4),
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
        "kernels_us": {n: v["avg_us"] for n, v in kern.items()},
        "kernels_cold_us": kern_cold,
        "kernels": kern,
        "roofline": roofline,
        "hbm_measured": hbm,
        "routing": routing_summary(spec, counts),
        "parity": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def size_matched_read_us(torch, dev, stream, nbytes, reps=20):
    """Event time (us, median of `reps`) of the read `measured_bandwidth`
    times (float32 row sums of a [rows][4096] view), over `nbytes` rounded up
    to whole 16 KiB rows: what a plain read of an HBM-bound kernel's own
    bytes costs at that size, launch and ramp included."""
    import numpy as np
    rows = torch.empty((nbytes + 16383) // 16384, 4096, dtype=torch.float32, device=dev).fill_(1.0)
    rows.sum(dim=1)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rows.sum(dim=1)
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    del rows
    return float(np.median(ts))


def measured_bandwidth(torch, dev, stream, mib=1024, reps=5):
    """HBM rates of plain torch kernels on this GPU, for context next to the
    published 8 TB/s: a device copy of `mib` MiB (bytes read + written per
    second) and a read-only pass over `mib` MiB (float32 row sums of a
    [n / 4096][4096] view; of torch's reductions the fastest reader, a plain
    sum of the flat tensor reads at about two thirds of its rate).
    Event-timed on the launch stream, median of `reps`."""
    import numpy as np
    n = mib << 20
    src = torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)

    def timed(f):
        f()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            f()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        return float(np.median(ts))

    t_copy = timed(lambda: dst.copy_(src))
    rows = src.view(-1, 4096)
    t_read = timed(lambda: rows.sum(dim=1))
    del src, dst
    return {"copy_gbps": round(2 * n / t_copy / 1e9, 1), "read_gbps": round(n / t_read / 1e9, 1), "mib": mib,
            "how": "torch device copy, and float32 row sums of a [n/4096][4096] view, of 1 GiB; "
                   "event-timed, median of 5"}


def routing_summary(spec, counts):
    """Realised expert load of the timed batch: rows per expert, max over
    mean, experts that received no row, and assignments the capacity dropped."""
    import numpy as np
    c = np.asarray(counts, np.int64)
    slots = int(c.sum()) if spec.gating == "expert_choice" else spec.T * spec.k
    return {"rows": int(c.sum()), "rows_per_expert_max": int(c.max()), "rows_per_expert_mean": round(float(c.mean()), 3),
            "load_max_over_mean": round(float(c.max() / max(c.mean(), 1e-30)), 3),
            "empty_experts": int((c == 0).sum()), "dropped_assignments": int(slots - c.sum())}


def cpu_baseline(spec, inp, seconds, y_gpu, routing):
    """The oracle as it stands on the host cores, on a bounded sample of tokens
    of the same workload (host copies of the same inputs).  The same leg then
    checks the timed batch against the oracle: the sampled tokens' outputs
    with the oracle routed by the GPU's own logits (routing-locked) and by its
    own logits (independent, flipped tokens left out), and the routing flips
    over every token.  Returns (cpu_baseline, parity)."""
    import numpy as np
    import torch

    import oracle

    log("[bench] cpu baseline: copying inputs to the host")
    host = {k: (None if v is None else v.detach().cpu().float().numpy()) for k, v in inp.items()}
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(threads))
    oracle._load()
    rng = np.random.default_rng(0)
    n = 8
    while True:
        toks = np.sort(rng.choice(spec.T, size=n, replace=False))
        t0 = time.perf_counter()
        oracle.forward_tokens(spec, host, toks)
        dt = time.perf_counter() - t0
        log(f"[bench] cpu baseline: {n} tokens took {dt:.2f} s")
        if dt >= 0.6 * seconds or n == spec.T:
            break
        n = int(min(spec.T, max(2 * n, n * seconds / max(dt, 1e-3))))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    cpu = {"value": round(n / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "host": {"cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0)), "nproc": os.cpu_count(),
                    "omp_num_threads": os.environ.get("OMP_NUM_THREADS")},
           "sample": f"{n} of {spec.T} tokens of {spec.name}, all layer steps, float64 C loops "
                     f"(OpenMP over the rows of each expert), {dt:.1f} s"}
    return cpu, parity_check(spec, host, toks, y_gpu, routing)


def parity_check(spec, host, toks, y_gpu, routing):
    """Oracle checks of the timed batch (part of the CPU leg)."""
    import numpy as np

    import oracle

    log("[bench] parity: oracle on the GPU's logits and on its own")
    T, E = spec.T, spec.E
    y = y_gpu[__import__("torch").from_numpy(toks).to(y_gpu.device)].float().cpu().numpy().astype(np.float64)
    glg = routing["logits"].cpu().numpy().reshape(T, E)
    gidx = routing["topk_idx"].cpu().numpy()

    def rel(a, b):
        return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)) if len(a) else 0.0

    locked = oracle.forward_tokens(spec, host, toks, lg=glg)
    olg = oracle.logits(host["x"], host["wg"], host["bg"])
    out = {"sampled_tokens": int(len(toks)), "max_rel_err_routing_locked": rel(y, locked["y64"]),
           "max_abs_logit_diff": float(np.abs(glg.astype(np.float64) - olg).max())}
    if spec.gating == "expert_choice":
        C = oracle.capacity(spec.capacity_factor, T, E)
        oidx, _ = oracle.route_expert_choice(olg, C)
        g = gidx.reshape(E, C)
        diff = [set(g[e].tolist()) ^ set(oidx[e].tolist()) for e in range(E)]
        flipped = set().union(*diff)
        out.update(flipped_experts=sum(1 for d_ in diff if d_), flipped_tokens=len(flipped))
        keep = ~np.isin(toks, list(flipped))
    else:
        k = spec.k
        oidx, _ = oracle.route_topk(olg, k, spec.gating)
        g = gidx.reshape(T, k)
        flips = (np.sort(g, 1) != np.sort(oidx, 1)).any(1)
        out.update(flipped_tokens=int(flips.sum()))
        keep = ~flips[toks]
        if spec.gating == "switch" or spec.capacity_factor > 0:
            # a flip moves later tokens of its (group, expert) too: leave out
            # every sampled token whose kept slots differ
            cap = oracle.capacity_topk(spec.capacity_factor, spec.capacity_group or T, k, E, spec.min_capacity)
            grp = spec.capacity_group
            kg = np.where(oracle.permute(g, E, cap, grp)["slot_row"] >= 0, g, -1)
            ko = np.where(oracle.permute(oidx, E, cap, grp)["slot_row"] >= 0, oidx, -1)
            moved = (np.sort(kg, 1) != np.sort(ko, 1)).any(1)
            out.update(flip_affected_tokens=int(moved.sum()))
            keep &= ~moved[toks]
    indep = oracle.forward_tokens(spec, host, toks[keep]) if keep.any() else None
    out["max_rel_err_independent"] = rel(y[keep], indep["y64"]) if indep is not None else None
    out["tolerance"] = 1e-5 if spec.dtype == "f32" else 1e-2
    return out


if __name__ == "__main__":
    main()
