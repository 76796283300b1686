#!/usr/bin/env python3
"""Benchmark of the ring all-reduce over R logical ranks in one MI355X's HBM.

Default run (one JSON line on stdout): ring all-reduce (sum), R = 8 logical
ranks, float32, 16,777,216 elements (64 MiB) per rank, N(0,1) inputs from
seed 2, simple protocol, 512 KiB chunks.  One step = one all-reduce of the
whole [8, 16M] buffer, inputs resident in HBM before the timed region.

  value  = busBW = algBW * 2(R-1)/R,  algBW = per-rank bytes / time
  roofline.achieved = algorithmic HBM bytes 5(R-1) N s / kernel time

Other modes (--mode): config1 (R = 4 int32, 4096 per rank, every form), matrix
(fused, 64 MiB per rank, R = 2..16, every dtype),
sweep (8 B .. 1 GiB per rank, alpha-beta fit), tree-vs-ring (8 B .. 256 KiB),
buckets (R = 16 bf16 reduce-scatter then all-gather, 40 x 25 MiB), stream
(c = a + b and copy reference kernels), counters (a short program for
rocprofv3 --pmc runs), tune (grid sizes), overlap (buckets beside GEMMs on
another stream).  They write a summary line to stdout (and JSON lines to
--out where a mode has several points).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "all-reduce busBW GB/s + HBM GB/s vs peak, R=8 fp32 64 MiB/rank, 1 GPU"
PEAK_HBM_GBPS = 8000.0  # MI355X published HBM3E bandwidth
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# The sources each launch form's kernels are built from: a counter figure in
# the traffic file stays valid while these hash the same.
_CSRC = "collective_communication_ring_amd/csrc/"
KERNEL_SOURCES = {
    "fused": [_CSRC + f for f in ("ar_ring.hip", "ar_slots.h", "ar_elem.h", "ar_internal.h")],
    "step": [_CSRC + f for f in ("ar_ring.hip", "ar_slots.h", "ar_elem.h", "ar_internal.h")],
    "pipelined": [_CSRC + f for f in ("ar_pipe.hip", "ar_elem.h", "ar_internal.h")],
}


def ring_kw(launch, channels=1):
    """Comm keyword arguments for a --launch value ('ll' selects the LL protocol)
    and a number of ring channels."""
    kw = dict(algo="ring", proto="ll") if launch == "ll" else \
        dict(algo="ring", proto="simple", launch=launch)
    if channels > 1:
        kw["channels"] = channels
    return kw


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha(launch):
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[launch]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(key):
    """HBM bytes per launch from the committed counter runs, or None when the
    kernel source changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ent = t.get(key)
    launch = key.rsplit("_", 1)[-1]
    if not ent or launch not in KERNEL_SOURCES or \
            ent.get("kernel_source_sha") != kernel_source_sha(launch):
        return None
    return ent.get("bytes_per_launch")


def time_calls(fn, steps, warmup, torch):
    """Run fn warmup times, then time `steps` back-to-back calls with events
    on the current stream.  Returns (per-call ms list, total ms, wall s)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return per, ev[0].elapsed_time(ev[steps]), wall


def time_graph(fn, calls, torch, reps=3):
    """Capture `calls` back-to-back calls of fn in one HIP graph, replay it
    once untimed, then time `reps` replays with events.  Returns ms per call.
    Removes the host's enqueue pacing from small-message timings."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * calls)
    del g
    return ms


def cpu_baseline_leg(call, target_s=3.0, max_calls=50):
    """The CPU-baseline leg of a mode: runs the oracle on the host, as it is,
    for a bounded sample (at least one call, then until target_s seconds or
    max_calls calls).  `call(oracle)` makes one oracle call.  Returns its last
    result (which the mode also uses to check the GPU's), the average seconds
    per call and the number of calls.  This is the only place bench.py runs
    the oracle."""
    import oracle
    ts = []
    y = None
    t_start = time.perf_counter()
    while not ts or (time.perf_counter() - t_start < target_s and len(ts) < max_calls):
        t0 = time.perf_counter()
        y = call(oracle)
        ts.append(time.perf_counter() - t0)
    return y, sum(ts) / len(ts), len(ts)


def cpu_baseline(x, R, N, s, target_s=12.0, strides=None):
    """The headline's CPU baseline: the full all-reduce on the host until about
    target_s seconds of CPU work; report its busBW.  `strides` are the ring
    channels' strides (one ring of stride 1 by default)."""
    y, t, n = cpu_baseline_leg(lambda o: o.ring_allreduce(x, strides=strides), target_s, 100)
    algbw = N * s / t / 1e9
    return y, dict(value=round(algbw * 2 * (R - 1) / R, 3), unit="GB/s", cores=1, kind="oracle",
                   sample="the full workload (8 ranks x 64 MiB), %d call(s), %.2f s each; "
                          "single-threaded C replay of the same ring order" % (n, t))


def headline(args):
    import numpy as np
    import torch
    from collective_communication_ring_amd import api, inputs, measure

    R, N, s = 8, 16_777_216, 4
    dev = torch.device("cuda:0")
    x = inputs.host_inputs("ring_f32_r8_64MiB")
    send = torch.from_numpy(x).to(dev)
    recv = torch.empty_like(send)
    comm = api.Comm(R, N, "float32", device=dev, chunk_bytes=512 * 1024, grid=args.grid,
                    **ring_kw(args.launch, args.channels))
    _, proto, launch = comm.plan(N)
    launch_name = "ll" if proto == api.AR_LL else {v: k for k, v in api.LAUNCHES.items()}[launch]
    per, total_ms, wall = time_calls(lambda: comm.allreduce(send, recv), args.steps, args.warmup,
                                     torch)
    assert comm.check() == api.AR_SUCCESS
    ms = total_ms / args.steps
    t = ms / 1e3
    algbw = N * s / t / 1e9
    busbw = algbw * measure.busbw_factor("allreduce", R)
    b_alg = measure.allreduce_alg_bytes(R, N, s)
    kernel_ms = sum(per) / len(per)
    achieved = b_alg / (kernel_ms / 1e3) / 1e9
    kernel = {"fused": "k_ring_fused<float32, 16-byte slots, all-reduce>",
              "pipelined": "k_ring_pipelined<float32, 16-byte slots, all-reduce>",
              "ll": "k_ring_ll<float32, all-reduce> (one launch per piece)",
              "step": "k_ring_reduce_step + k_ring_copy_step (2(R-1) launches)"}[launch_name]
    if args.channels > 1:
        kernel += ", one launch per channel x %d channels" % args.channels
    traffic = measured_traffic("ring_allreduce_f32_r8_64MiB_" + launch_name) \
        if args.channels == 1 else None
    line = {
        "metric": METRIC,
        "value": round(busbw, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "ring all-reduce (sum), R=8 logical ranks, fp32, 16,777,216 "
                               "elements (64 MiB) per rank, N(0,1) seed 2, simple protocol, "
                               "512 KiB chunks",
                   "R": R, "count_per_rank": N, "launch": launch_name,
                   "channels": args.channels},
        "algbw_GBps": round(algbw, 3),
        "busbw_GBps": round(busbw, 3),
        "hbm_alg_GBps": round(b_alg / t / 1e9, 3),
        "hbm_alg_frac_of_peak": round(b_alg / t / 1e9 / PEAK_HBM_GBPS, 4),
        # the bytes the counters saw move (roofline.traffic) over the same time:
        # the HBM rate proper, which the algorithmic rate overstates when the
        # L2 serves the hand-off re-reads
        "hbm_measured_GBps": round(traffic / (kernel_ms / 1e3) / 1e9, 3) if traffic else None,
        "hbm_measured_frac_of_peak": round(traffic / (kernel_ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4)
        if traffic else None,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "kernel": kernel, "alg_bytes_per_launch": b_alg
                     if launch_name != "step" else None},
        "wall_s_timed": round(wall, 4),
    }
    y = None
    if not args.no_cpu_baseline:
        y, line["cpu_baseline"] = cpu_baseline(x, R, N, s, strides=comm.channel_strides())
    else:
        line["cpu_baseline"] = None
    if y is not None:
        got = recv.cpu().numpy()
        line["verified_vs_oracle"] = bool(got.tobytes() == y.tobytes())
        if not line["verified_vs_oracle"]:
            log("ERROR: GPU result differs from the oracle")
    print(json.dumps(line), flush=True)
    return 0 if line.get("verified_vs_oracle", True) else 1


def mode_sweep(args):
    """Config 3: ring all-reduce, R = 8, fp32, 8 B .. 1 GiB per rank in powers
    of two, 5 warm-up + 20 timed calls each; alpha-beta fit."""
    import torch
    from collective_communication_ring_amd import api, inputs, measure
    R, s = 8, 4
    dev = torch.device("cuda:0")
    max_bytes = args.max_bytes
    counts = inputs.sweep_counts(8, max_bytes, s)
    Nmax = counts[-1]
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    # flat buffers: the first R*N elements viewed as [R, N] are rank-major
    send_flat = torch.randn(R * Nmax, generator=g, device=dev, dtype=torch.float32)
    recv_flat = torch.empty_like(send_flat)
    comm = api.Comm(R, Nmax, "float32", device=dev, chunk_bytes=512 * 1024, grid=args.grid,
                    **ring_kw(args.launch, args.channels))
    rows = []
    out = open(args.out, "w") if args.out else None
    for N in counts:
        sv = send_flat[:R * N].view(R, N)
        rv = recv_flat[:R * N].view(R, N)
        if args.eager:
            per, total_ms, _ = time_calls(lambda: comm.allreduce(sv, rv), 20, 5, torch)
            t = total_ms / 20 / 1e3
        else:
            t = time_graph(lambda: comm.allreduce(sv, rv), 20, torch) / 1e3
        row = dict(mode="sweep", bytes_per_rank=N * s, count=N, t_us=t * 1e6,
                   algbw_GBps=N * s / t / 1e9,
                   busbw_GBps=N * s / t / 1e9 * measure.busbw_factor("allreduce", R),
                   hbm_alg_GBps=measure.allreduce_alg_bytes(R, N, s) / t / 1e9,
                   launch=args.launch)
        rows.append(row)
        log("sweep %10d B/rank  %10.2f us  busBW %8.2f GB/s" % (N * s, t * 1e6, row["busbw_GBps"]))
        if out:
            out.write(json.dumps(row) + "\n")
            out.flush()
        del sv, rv
    assert comm.check() == api.AR_SUCCESS
    cpu = []
    for N in [n for n in (256, 65536, 1 << 22) if n <= Nmax]:  # 1 KiB, 256 KiB, 16 MiB per rank
        xs = send_flat[:R * N].view(R, N).cpu().numpy()
        _, t_or, n_or = cpu_baseline_leg(lambda o: o.ring_allreduce(xs), 3.0)
        cpu.append(dict(bytes_per_rank=N * s, t_us=t_or * 1e6, calls=n_or))
        log("oracle %10d B/rank  %10.1f us" % (N * s, t_or * 1e6))
    fit = measure.fit_alpha_beta([r["bytes_per_rank"] for r in rows], [r["t_us"] / 1e6 for r in rows])
    small = [r["t_us"] for r in rows if r["bytes_per_rank"] <= 4096]
    large = [r for r in rows if r["bytes_per_rank"] >= 64 << 20]
    cross = {}
    if small:
        cross["alpha_median_small_us"] = sorted(small)[len(small) // 2]
    if len(large) >= 2:
        a, b = large[0], large[-1]
        cross["inv_beta_large_GBps"] = (b["bytes_per_rank"] - a["bytes_per_rank"]) / (
            (b["t_us"] - a["t_us"]) / 1e6) / 1e9
    summary = dict(mode="sweep_fit", R=R, dtype="f32", launch=args.launch, **fit,
                   bus_rate_GBps=fit["inv_beta_GBps"] * measure.busbw_factor("allreduce", R),
                   **cross, cpu_baseline=dict(kind="oracle", cores=1, points=cpu))
    if out:
        out.write(json.dumps(summary) + "\n")
        out.close()
    print(json.dumps(summary), flush=True)
    return 0


def ll_hop_latency_us(torch, iters=20000):
    """One-way latency of an 8-byte LL line between two workgroups, on
    different XCDs and on the same XCD (the tree's per-hop bound)."""
    from collective_communication_ring_amd import api
    dev = torch.device("cuda:0")
    lines = torch.zeros(64, dtype=torch.int64, device=dev)
    result = torch.zeros(1, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    out = {}
    for name, apart in (("xcd_apart", 1), ("same_xcd", 0)):
        api.ar_ll_pingpong(lines.data_ptr(), result.data_ptr(), 100, apart, 2_000_000, st)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        api.ar_ll_pingpong(lines.data_ptr(), result.data_ptr(), iters, apart, 2_000_000, st)
        e1.record()
        torch.cuda.synchronize()
        if int(result.item()) != 0:
            raise RuntimeError("LL ping-pong timed out")
        out[name] = e0.elapsed_time(e1) * 1e3 / (2 * iters)
    return out


def mode_tree_vs_ring(args):
    """Config 4: R = 8, fp32 U[-1,1), 8 B .. 256 KiB per rank; tree + LL
    against ring (fused and step) at the same sizes."""
    import torch
    from collective_communication_ring_amd import api, inputs
    R, s = 8, 4
    dev = torch.device("cuda:0")
    counts = inputs.sweep_counts(8, args.tvr_max_bytes, s)
    Nmax = counts[-1]
    x = inputs.draw("uniform_pm1", R, Nmax, seed=4)
    send_flat = torch.from_numpy(x).to(dev).reshape(-1)
    recv_flat = torch.empty_like(send_flat)
    variants = [("tree-ll", dict(algo="tree", proto="ll")),
                ("ring-ll", dict(algo="ring", proto="ll")),
                ("ring-fused", dict(algo="ring", proto="simple", launch="fused")),
                ("ring-pipelined", dict(algo="ring", proto="simple", launch="pipelined")),
                ("ring-step", dict(algo="ring", proto="simple", launch="step"))]
    comms = {name: api.Comm(R, Nmax, "float32", device=dev, **kw) for name, kw in variants}
    out = open(args.out, "w") if args.out else None
    res = {}
    for N in counts:
        sv = send_flat[:R * N].view(R, N)
        rv = recv_flat[:R * N].view(R, N)
        for name, _ in variants:
            c = comms[name]
            if args.eager:
                _, total_ms, _ = time_calls(lambda: c.allreduce(sv, rv), 20, 5, torch)
                t_us = total_ms / 20 * 1e3
            else:
                t_us = time_graph(lambda: c.allreduce(sv, rv), 20, torch) * 1e3
            res.setdefault(name, []).append(t_us)
            row = dict(mode="tree_vs_ring", variant=name, bytes_per_rank=N * s, t_us=t_us)
            log("%-10s %8d B/rank %9.2f us" % (name, N * s, t_us))
            if out:
                out.write(json.dumps(row) + "\n")
    for c in comms.values():
        assert c.check() == api.AR_SUCCESS
    hop = ll_hop_latency_us(torch)
    log("LL one-way hop latency: %s" % hop)
    # the launch floor: one single-workgroup kernel (a 16-byte copy) per call
    st = lambda: torch.cuda.current_stream().cuda_stream
    launch_floor = time_graph(lambda: api.ar_stream_copy(send_flat.data_ptr(), recv_flat.data_ptr(),
                                                         16, st()), 20, torch) * 1e3
    log("launch floor (16-byte copy kernel, graph-replayed): %.2f us" % launch_floor)
    # latency roofline of the tree: 2 * depth hops (up, then down) per call
    depth = 3 if R == 8 else None
    _, t_or, n_or = cpu_baseline_leg(lambda o: o.tree_allreduce(x), 3.0)
    summary = dict(mode="tree_vs_ring_summary", sizes=[n * s for n in counts], t_us=res,
                   ll_hop_us=hop, tree_depth=depth, launch_floor_us=launch_floor,
                   tree_hop_bound_us=2 * depth * hop["xcd_apart"] if depth else None,
                   cpu_baseline=dict(kind="oracle", cores=1, value_us=t_or * 1e6,
                                     sample="tree all-reduce, %d B/rank, %d calls"
                                            % (Nmax * s, n_or)))
    if out:
        out.write(json.dumps(summary) + "\n")
        out.close()
    print(json.dumps(summary), flush=True)
    return 0


def mode_buckets(args):
    """Config 5: R = 16 bf16 N(0, 0.02), 40 buckets x 13,107,200 elements per
    rank, reduce-scatter then all-gather per bucket (and all-reduce)."""
    import torch
    from collective_communication_ring_amd import api, inputs, measure
    w = inputs.WORKLOADS["buckets_bf16_r16"]
    R, N, B, s = w["R"], w["count"], args.buckets or w["buckets"], 2
    n = N // R
    dev = torch.device("cuda:0")
    xs = [inputs.device_bucket_bf16(R, N, w["seed"], b, dev) for b in range(B)]
    shards = [torch.empty((R, n), dtype=torch.bfloat16, device=dev) for _ in range(B)]
    full = torch.empty((R, N), dtype=torch.bfloat16, device=dev)
    comm = api.Comm(R, N, "bf16", device=dev, grid=args.grid, **ring_kw(args.launch, args.channels))

    def rs_all():
        for b in range(B):
            comm.reduce_scatter(xs[b], shards[b])

    def ag_all():
        for b in range(B):
            comm.all_gather(shards[b], full)

    def ar_all():
        for b in range(B):
            comm.allreduce(xs[b], full)

    rep = {}
    for name, fn, op, alg in (("reduce_scatter", rs_all, "rs", measure.reduce_scatter_alg_bytes(R, N, s)),
                              ("all_gather", ag_all, "ag", measure.all_gather_alg_bytes(R, N, s)),
                              ("allreduce", ar_all, "ar", None)):
        _, total_ms, _ = time_calls(fn, args.steps, 1, torch)
        t = total_ms / args.steps / B / 1e3  # per bucket
        algbw = N * s / t / 1e9
        f = measure.busbw_factor("allreduce" if op == "ar" else op, R)
        rep[name] = dict(t_us_per_bucket=t * 1e6, algbw_GBps=algbw, busbw_GBps=algbw * f,
                         hbm_alg_GBps=(alg / t / 1e9) if alg else None)
        log(name, rep[name])
    assert comm.check() == api.AR_SUCCESS
    import numpy as np
    xh = xs[0].view(torch.int16).cpu().numpy().view(np.uint16)
    sh, t_rs, _ = cpu_baseline_leg(lambda o: o.ring_reduce_scatter(xh, "bf16"), 0.0, 1)
    _, t_ag, _ = cpu_baseline_leg(lambda o: o.ring_all_gather(sh, "bf16"), 0.0, 1)
    rep["cpu_baseline"] = dict(kind="oracle", cores=1, sample="bucket 0, one call each",
                               reduce_scatter_us=t_rs * 1e6, all_gather_us=t_ag * 1e6)
    summary = dict(mode="buckets", R=R, dtype="bf16", buckets=B, count_per_rank=N, **rep)
    print(json.dumps(summary), flush=True)
    return 0


def mode_stream(args):
    """Reference kernels: c = a + b over float32 (the access mix of one reduce
    step) and a plain copy, each on 512 MiB arrays (larger than the 256 MB
    infinity cache)."""
    import torch
    from collective_communication_ring_amd import api
    dev = torch.device("cuda:0")
    n = (512 << 20) // 4
    a = torch.randn(n, device=dev)
    b = torch.randn(n, device=dev)
    c = torch.empty_like(a)
    st = torch.cuda.current_stream().cuda_stream
    _, ms, _ = time_calls(lambda: api.ar_stream_add(a.data_ptr(), b.data_ptr(), c.data_ptr(), n, st),
                          args.steps, args.warmup, torch)
    add_gbps = 3 * n * 4 / (ms / args.steps / 1e3) / 1e9
    _, ms2, _ = time_calls(lambda: api.ar_stream_copy(a.data_ptr(), c.data_ptr(), n * 4, st),
                           args.steps, args.warmup, torch)
    copy_gbps = 2 * n * 4 / (ms2 / args.steps / 1e3) / 1e9
    torch.cuda.synchronize()
    ok = torch.equal(c, a)
    summary = dict(mode="stream", bytes_per_array=n * 4, add_GBps=add_gbps,
                   add_frac=add_gbps / PEAK_HBM_GBPS, copy_GBps=copy_gbps,
                   copy_frac=copy_gbps / PEAK_HBM_GBPS, copy_ok=ok)
    print(json.dumps(summary), flush=True)
    return 0


def mode_overlap(args):
    """DDP-style overlap ("NCCL, NIXL, and Distributed GPU Communication",
    performance checklist: without overlap total = compute + communication,
    with overlap about max(compute, communication) + a tail).  Buckets of a
    ring all-reduce (R = 8 fp32, 25 MiB per rank each) run on a second stream
    while bf16 GEMMs run on the first; reports compute alone, communication
    alone, both serial and both overlapped, and the exposed communication
    time.  Uses a launch form without cross-workgroup waits (fused by
    default), since a concurrent kernel can hold CUs the spin-waiting forms
    would need."""
    import torch
    from collective_communication_ring_amd import api
    dev = torch.device("cuda:0")
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    raw = []
    if args.comm_cus:
        # CU-masked streams need hardware queues of their own (a few per
        # process): create them before anything else takes one.  The first k
        # CU indices (k a multiple of 8, so every XCD gets the same share)
        # go to the collective, the rest to compute.
        k = max(8, args.comm_cus // 8 * 8)
        comm_cus = list(range(k))
        comp_cus = list(range(k, ncu))
        raw = [api.ar_stream_create_cu_masked(comm_cus, ncu),
               api.ar_stream_create_cu_masked(comp_cus, ncu)]
    R, N, B = 8, (25 << 20) // 4, args.buckets or 8
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    xs = [torch.randn((R, N), generator=g, device=dev) for _ in range(B)]
    ys = [torch.empty_like(x) for x in xs]
    launch = args.launch if args.launch in ("fused", "step") else "fused"
    comm = api.Comm(R, N, "float32", device=dev, **ring_kw(launch))
    M = 8192
    a = torch.randn((M, M), generator=g, device=dev).to(torch.bfloat16)
    b = torch.randn((M, M), generator=g, device=dev).to(torch.bfloat16)
    gemms = args.gemms
    if raw:
        s_comm = torch.cuda.ExternalStream(raw[0], device=dev)
        s_comp = torch.cuda.ExternalStream(raw[1], device=dev)
        comm.set_option(api.AR_OPT_GRID, len(comm_cus) * (8 if launch == "step" else 1))
    else:
        s_comp = torch.cuda.current_stream()
        s_comm = torch.cuda.Stream()

    def compute():
        with torch.cuda.stream(s_comp):
            for _ in range(gemms):
                torch.mm(a, b)

    def communicate(stream):
        for x, y in zip(xs, ys):
            comm.allreduce(x, y, stream=stream)

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps * 1e3

    def serial():
        compute()
        s_comm.wait_stream(s_comp)
        communicate(s_comm)

    t_comp = timed(compute)
    t_comm = timed(lambda: communicate(s_comm))
    t_serial = timed(serial)

    def overlapped():
        communicate(s_comm)
        compute()

    t_over = timed(overlapped)
    assert comm.check() == api.AR_SUCCESS
    torch.cuda.synchronize()
    # the comm's workspace is recorded on s_comm: release it while that stream
    # still exists, then destroy the CU-masked streams
    comm.close()
    del comm
    torch.cuda.synchronize()
    for r in raw:
        api.ar_stream_destroy(r)
    out = dict(mode="overlap", launch=launch, comm_cus=args.comm_cus or None, buckets=B,
               bucket_bytes_per_rank=N * 4, R=R,
               gemms=gemms, gemm="bf16 %dx%dx%d" % (M, M, M), compute_ms=t_comp, comm_ms=t_comm,
               serial_ms=t_serial, overlapped_ms=t_over,
               exposed_comm_ms=t_over - t_comp,
               ideal_overlapped_ms=max(t_comp, t_comm))
    print(json.dumps(out), flush=True)
    return 0


def mode_counters(args):
    """A short program for byte-counter runs (rocprofv3 --pmc): a copy of a
    known size (the calibration), then 3 all-reduces of the headline workload
    in each launch form, then a small tree-LL all-reduce."""
    import torch
    from collective_communication_ring_amd import api, inputs
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    n = (512 << 20) // 4
    a = torch.randn(n, device=dev)
    c = torch.empty_like(a)
    for _ in range(3):
        api.ar_stream_copy(a.data_ptr(), c.data_ptr(), n * 4, st)
    torch.cuda.synchronize()
    del a, c
    R, N = 8, 16_777_216
    x = inputs.host_inputs("ring_f32_r8_64MiB")
    send = torch.from_numpy(x).to(dev)
    recv = torch.empty_like(send)
    for launch in ("fused", "step", "pipelined"):
        comm = api.Comm(R, N, "float32", "ring", device=dev, launch=launch, grid=args.grid)
        for _ in range(3):
            comm.allreduce(send, recv)
        torch.cuda.synchronize()
    comm = api.Comm(R, 65536, "float32", "tree", "ll", device=dev)
    small = send[:, :65536].contiguous()
    out = torch.empty_like(small)
    for _ in range(3):
        comm.allreduce(small, out)
    torch.cuda.synchronize()
    print(json.dumps(dict(mode="counters", copy_bytes=n * 4, allreduce_count=N)), flush=True)
    return 0


def mode_config1(args):
    """Config 1: ring all-reduce (sum), R = 4, int32, 4096 elements per rank,
    chunk = count / R; time per call (graph-replayed) in every form, each
    result checked bit for bit against the oracle and the int64 sum."""
    import numpy as np
    import torch
    from collective_communication_ring_amd import api, inputs
    R, N = 4, 4096
    dev = torch.device("cuda:0")
    x = inputs.host_inputs("ring_int32_r4")
    ref, t_or, n_or = cpu_baseline_leg(lambda o: o.ring_allreduce(x), 2.0)
    exact = x.astype(np.int64).sum(axis=0).astype(np.int32)
    send = torch.from_numpy(x).to(dev)
    recv = torch.empty_like(send)
    res = {}
    for name, kw in (("fused", ring_kw("fused")), ("step", ring_kw("step")),
                     ("pipelined", ring_kw("pipelined")), ("ll", ring_kw("ll")),
                     ("tree-ll", dict(algo="tree", proto="ll"))):
        comm = api.Comm(R, N, "int32", device=dev, chunk_bytes=(N // R) * 4, **kw)
        t_us = time_graph(lambda: comm.allreduce(send, recv), 20, torch) * 1e3
        got = recv.cpu().numpy()
        ok = comm.check() == api.AR_SUCCESS and (got == exact[None, :]).all() and (
            name == "tree-ll" or got.tobytes() == ref.tobytes())
        res[name] = dict(t_us=round(t_us, 3), exact=bool(ok))
        log("config 1 %-10s %8.2f us  exact=%s" % (name, t_us, ok))
        comm.close()
    print(json.dumps(dict(mode="config1", R=R, count_per_rank=N, dtype="int32", results=res,
                          cpu_baseline=dict(kind="oracle", cores=1, t_us=t_or * 1e6,
                                            sample="%d calls" % n_or))), flush=True)
    return 0 if all(r["exact"] for r in res.values()) else 1


def mode_matrix(args):
    """Fused ring all-reduce at 64 MiB per rank for R in {2, 4, 8, 16} and
    every dtype: time, busBW and the algorithmic HBM fraction, each result
    checked bit for bit against the oracle."""
    import numpy as np
    import torch
    from collective_communication_ring_amd import api, inputs, measure
    dev = torch.device("cuda:0")
    rows = []
    for dtype, s in (("float32", 4), ("int32", 4), ("bf16", 2)):
        for R in (2, 4, 8, 16):
            N = (64 << 20) // s
            if dtype == "float32":
                x = inputs.draw("normal", R, N, seed=100 + R)
            elif dtype == "int32":
                x = inputs.draw("int_pm1000", R, N, seed=100 + R)
            else:
                x = inputs.to_bf16_bits(inputs.draw("normal_0.02", R, N, seed=100 + R))
            if dtype == "bf16":
                send = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
            else:
                send = torch.from_numpy(x).to(dev)
            recv = torch.empty_like(send)
            comm = api.Comm(R, N, dtype, device=dev, launch="fused")
            _, total_ms, _ = time_calls(lambda: comm.allreduce(send, recv), args.steps,
                                        args.warmup, torch)
            t = total_ms / args.steps / 1e3
            got = recv.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" \
                else recv.cpu().numpy()
            ref, t_or, _ = cpu_baseline_leg(lambda o: o.ring_allreduce(x, dtype), 0.0, 1)
            exact = got.tobytes() == ref.tobytes()
            row = dict(dtype=dtype, R=R, bytes_per_rank=N * s, ms=round(t * 1e3, 4),
                       busbw_GBps=round(N * s / t / 1e9 * measure.busbw_factor("allreduce", R), 1),
                       alg_frac=round(measure.allreduce_alg_bytes(R, N, s) / t / 1e9 /
                                      PEAK_HBM_GBPS, 3),
                       compulsory_TBps=round(2 * R * N * s / t / 1e12, 2), exact=exact,
                       cpu_baseline_s=round(t_or, 3))
            rows.append(row)
            log("matrix %-7s R=%2d %.4f ms busBW %7.1f GB/s alg frac %.3f compulsory %.2f TB/s "
                "exact=%s" % (dtype, R, row["ms"], row["busbw_GBps"], row["alg_frac"],
                              row["compulsory_TBps"], exact))
            comm.close()
            del send, recv, x
            torch.cuda.empty_cache()
    print(json.dumps(dict(mode="matrix", launch="fused", results=rows,
                          cpu_baseline=dict(kind="oracle", cores=1,
                                            sample="one call per row (cpu_baseline_s)"))),
          flush=True)
    return 0 if all(r["exact"] for r in rows) else 1


def mode_tune(args):
    """Time the R = 8 fp32 64 MiB/rank all-reduce for a list of grid sizes
    (workgroups per launch) in one launch form."""
    import torch
    from collective_communication_ring_amd import api, inputs
    R, N, s = 8, 16_777_216, 4
    dev = torch.device("cuda:0")
    x = inputs.host_inputs("ring_f32_r8_64MiB")
    send = torch.from_numpy(x).to(dev)
    recv = torch.empty_like(send)
    ref = None
    t_or = None
    res = []
    for grid in [int(g) for g in args.grids.split(",")]:
        comm = api.Comm(R, N, "float32", device=dev, chunk_bytes=args.chunk_bytes, grid=grid,
                        **ring_kw(args.launch, args.channels))
        if ref is None:
            ref, t_or, _ = cpu_baseline_leg(
                lambda o: o.ring_allreduce(x, strides=comm.channel_strides()), 0.0, 1)
        _, total_ms, _ = time_calls(lambda: comm.allreduce(send, recv), args.steps, args.warmup,
                                    torch)
        ms = total_ms / args.steps
        ok = recv.cpu().numpy().tobytes() == ref.tobytes()
        res.append(dict(grid=grid, ms=ms, busbw=N * s / (ms / 1e3) / 1e9 * 1.75, exact=ok))
        log("grid %6d  %.4f ms  busBW %.1f GB/s  exact=%s" % (grid, ms, res[-1]["busbw"], ok))
        comm.close()
    print(json.dumps(dict(mode="tune", launch=args.launch, results=res,
                          cpu_baseline=dict(kind="oracle", cores=1, seconds=t_or,
                                            sample="one call"))), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--launch", default="auto", choices=["auto", "fused", "step", "pipelined", "ll"],
                    help="ring launch form; 'll' = the ring with the LL protocol")
    ap.add_argument("--grid", type=int, default=0, help="workgroups per launch (0: library default)")
    ap.add_argument("--mode", default="headline",
                    choices=["headline", "config1", "matrix", "sweep", "tree-vs-ring",
                             "buckets", "stream", "counters", "tune", "overlap"])
    ap.add_argument("--max-bytes", type=int, default=1 << 30)
    ap.add_argument("--tvr-max-bytes", type=int, default=256 * 1024,
                    help="tree-vs-ring: largest per-rank size (config 4 stops at 256 KiB)")
    ap.add_argument("--buckets", type=int, default=0)
    ap.add_argument("--out", default=None)
    ap.add_argument("--grids", default="256,512,768,1024,1280,1536,1792,2048")
    ap.add_argument("--gemms", type=int, default=8, help="overlap mode: GEMMs per iteration")
    ap.add_argument("--comm-cus", type=int, default=0,
                    help="overlap mode: CUs reserved for the collective (0: no CU masks)")
    ap.add_argument("--chunk-bytes", type=int, default=512 * 1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--channels", type=int, default=1,
                    help="ring channels (each its own ring stride over a sub-range of "
                         "every segment)")
    ap.add_argument("--eager", action="store_true",
                    help="sweep / tree-vs-ring: time host-enqueued calls instead of graph replays")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the R logical ranks of the ring all live in one "
              "MI355X's HBM, so --gpus must be 1 (got --gpus %d, WORLD_SIZE %d)."
              % (args.gpus, world), file=sys.stderr)
        return 2
    fn = {"headline": headline, "config1": mode_config1, "matrix": mode_matrix,
          "sweep": mode_sweep, "tree-vs-ring": mode_tree_vs_ring,
          "buckets": mode_buckets, "stream": mode_stream, "counters": mode_counters,
          "tune": mode_tune, "overlap": mode_overlap}[args.mode]
    return fn(args)


if __name__ == "__main__":
    sys.exit(main())
