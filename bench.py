#!/usr/bin/env python3
"""Benchmark of the ring all-reduce over R logical ranks in one MI355X's HBM.

Default run (one JSON line on stdout): ring all-reduce (sum), R = 8 logical
ranks, float32, 16,777,216 elements (64 MiB) per rank, N(0,1) inputs from
seed 2, in the library's default launch form (fused: one persistent kernel;
each wave carries a tile of every rank row through all 2(R-1) steps, the
hand-offs stay in the XCD's L2).  One step = one all-reduce of the whole
[8, 16M] buffer, inputs resident in HBM before the timed region.

  value  = busBW = algBW * 2(R-1)/R,  algBW = per-rank bytes / time
  roofline.achieved = HBM bytes per launch / kernel time, where the HBM bytes
           are 2 R N s for the fused form (every input row read once, every
           output row written once: its hops are L2-served) and the hop bytes
           5 (R-1) N s for the forms whose every hop goes through memory;
           roofline.traffic = the bytes rocprofv3's counters saw per launch.
  hop_rate_GBps = 5 (R-1) N s / time: every hop's load and store counted,
           served by L2, or by LDS for the reduce steps of smaller or bf16
           calls, in the fused form (not an HBM rate).

The same line carries, unless --no-extras: the message-size sweep (R = 8
fp32, 8 B .. 1 GiB per rank) with its alpha-beta fit; the trees (fused, and
with LL) against the ring forms (R = 8 fp32, 8 B .. 256 KiB) with the
crossovers and AR_AUTO's choices; a few 25 MiB gradient buckets (R = 16 bf16 reduce-scatter,
all-gather, all-reduce, checked against the oracle); the pipelined ring (simple protocol, 512 KiB chunks)
on the headline workload; and a 512 MiB copy as the streaming ceiling.
cpu_baseline times the oracle on one thread and on all host cores.

Other modes (--mode): r4-int32 (R = 4 int32, 4096 per rank, every form and both
trees), matrix
(fused, 64 MiB per rank, R = 2..16, every dtype),
sweep (8 B .. 1 GiB per rank, alpha-beta fit), tree-vs-ring (8 B .. 256 KiB),
tree-large (both trees beside the fused ring at 4 .. 64 MiB per rank),
buckets (R = 16 bf16 reduce-scatter then all-gather, 40 x 25 MiB), stream
(c = a + b and copy reference kernels), counters (a short program for
rocprofv3 --pmc runs), tune (grid sizes), overlap (buckets beside GEMMs on
another stream).  They write a summary line to stdout (and JSON lines to
--out where a mode has several points).
"""
import argparse
import contextlib
import hashlib
import json
import os
import subprocess
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
    "fused": [_CSRC + f for f in ("ar_fused.hip", "ar_ring.hip", "ar_slots.h", "ar_elem.h",
                                  "ar_internal.h")],
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
    on the current stream (the stream the library launches on).  Returns
    (per-call ms list, total ms, wall s)."""
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


def time_graph(fn, calls, torch, reps=1, warmup=5):
    """`warmup` eager calls, then `calls` back-to-back calls captured in one
    HIP graph; one untimed replay, then `reps` timed replays.  Returns ms per
    call.  Removes the host's enqueue pacing from small-message timings
    (the sweep: 5 warm-up, then 20 timed calls)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(max(1, warmup)):
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


def cpu_info():
    """Host facts for the CPU baseline: logical CPUs (nproc), the CPUs this
    process may run on, the threads the all-cores leg uses (OMP_NUM_THREADS
    when set, else those CPUs) and the CPU model (lscpu)."""
    nproc = os.cpu_count()
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = nproc
    model = None
    try:
        out = subprocess.run(["lscpu"], stdout=subprocess.PIPE, stderr=subprocess.DEVNULL,
                             text=True, timeout=20).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None:
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    env = os.environ.get("OMP_NUM_THREADS", "").strip()
    threads = int(env) if env.isdigit() and int(env) > 0 else usable
    return dict(nproc=nproc, usable_cpus=usable, threads=threads, cpu_model=model)


def cpu_baseline_leg(call, target_s=3.0, max_calls=50, threads=None, warmup=0):
    """The CPU-baseline leg of a mode: runs the oracle on the host, as it is,
    for a bounded sample (`warmup` untimed calls, then at least one timed
    call, then until target_s seconds or max_calls calls).  `call(oracle)`
    makes one oracle call.  With `threads`, the calls run on the oracle's
    OpenMP build with that many threads.  Returns its last result (which the
    mode also uses to check the GPU's), the average seconds per call, the
    number of calls and the threads used.  This and the oracle checks of the
    extras are the only places bench.py runs the oracle."""
    import oracle
    ctx = oracle.parallel(threads) if threads else contextlib.nullcontext(1)
    with ctx as used:
        for _ in range(warmup):
            call(oracle)
        ts = []
        y = None
        t_start = time.perf_counter()
        while not ts or (time.perf_counter() - t_start < target_s and len(ts) < max_calls):
            t0 = time.perf_counter()
            y = call(oracle)
            ts.append(time.perf_counter() - t0)
    return y, sum(ts) / len(ts), len(ts), used


def cpu_baseline(x, R, N, s, strides=None):
    """The headline's CPU baseline: the full all-reduce by the oracle, 5
    warm-up then up to 20 timed calls (at most ~8 s) on one thread, then the
    same on all host cores; both legs must give the same bits.  Reports the
    all-cores busBW as `value` and the one-thread leg beside it."""
    info = cpu_info()
    call = lambda o: o.ring_allreduce(x, strides=strides)
    y1, t1, n1, _ = cpu_baseline_leg(call, 8.0, 20, warmup=1)
    yn, tn, nn, used = cpu_baseline_leg(call, 8.0, 20, threads=info["threads"], warmup=5)
    same = y1.tobytes() == yn.tobytes()
    busbw = lambda t: round(N * s / t / 1e9 * 2 * (R - 1) / R, 3)
    return y1, dict(
        value=busbw(tn), unit="GB/s", cores=used, kind="oracle",
        sample="the full workload (8 ranks x 64 MiB per rank); all cores: %d timed call(s) after 5 "
               "warm-up, %.3f s each, %d OpenMP threads (parallel over the elements of each "
               "step, each element folded in the ring's order); one thread: %d call(s), %.3f s "
               "each" % (nn, tn, used, n1, t1),
        single_thread=dict(value=busbw(t1), unit="GB/s", cores=1, s_per_call=round(t1, 4),
                           calls=n1),
        all_cores=dict(value=busbw(tn), unit="GB/s", cores=used, s_per_call=round(tn, 4),
                       calls=nn),
        legs_bit_identical=same, **info)


def run_extra(extras, name, fn):
    """Run one extra measurement; a failure is reported in its key instead of
    ending the run (its error is also logged)."""
    t0 = time.perf_counter()
    try:
        extras[name] = fn()
    except Exception as e:  # noqa: BLE001 -- reported in the output line
        log("extra %s failed: %r" % (name, e))
        extras[name] = dict(error=repr(e))
    log("extra %s: %.1f s" % (name, time.perf_counter() - t0))


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
    hop_bytes = measure.allreduce_alg_bytes(R, N, s)
    hbm_bytes = measure.allreduce_hbm_bytes(R, N, s)
    # the form's HBM bytes: the fused form's hops are L2-served by design;
    # every other form moves each hop through memory
    alg_bytes = hbm_bytes if launch_name == "fused" else hop_bytes
    kernel_ms = sum(per) / len(per)
    achieved = alg_bytes / (kernel_ms / 1e3) / 1e9
    kernel = {"fused": "k_ring_fused_vec<float32, all-reduce, sum> (one launch)",
              "pipelined": "k_ring_pipelined<float32, 16-byte slots, all-reduce> (one launch)",
              "ll": "k_ring_ll<float32, all-reduce> (one launch per piece)",
              "step": "k_ring_reduce_step + k_ring_copy_step (2(R-1) launches)"}[launch_name]
    if args.channels > 1:
        kernel += ", one launch per channel x %d channels" % args.channels
    traffic = measured_traffic("ring_allreduce_f32_r8_64MiB_" + launch_name) \
        if args.channels == 1 else None
    form = {"fused": "fused launch form: one persistent kernel, each wave64 carries a tile of "
                     "2 KiB of every rank row through all 14 steps; every hop is a store and a "
                     "load of the hand-off slot in the XCD's L2; no flags (tiles are "
                     "independent), so the 512 KiB chunk does not apply",
            "pipelined": "pipelined launch form: simple protocol, 512 KiB chunks handed from rank "
                         "to rank through ready flags",
            "step": "step launch form: one kernel per ring step",
            "ll": "ring with the LL protocol (8-byte lines: 4 B data + 4 B flag)"}[launch_name]
    line = {
        "metric": METRIC,
        "value": round(busbw, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        # per-call event times of the same timed calls (back to back, so each
        # also holds the gap before the next launch)
        "ms_per_call_median": round(sorted(per)[len(per) // 2], 6),
        "ms_per_call_min": round(min(per), 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "ring all-reduce (sum), R=8 logical ranks, fp32, 16,777,216 "
                               "elements (64 MiB) per rank, N(0,1) seed 2; " + form,
                   "R": R, "count_per_rank": N, "launch": launch_name,
                   "channels": args.channels},
        "algbw_GBps": round(algbw, 3),
        "busbw_GBps": round(busbw, 3),
        # HBM: the bytes the form must move over the time of one call
        "hbm_GBps": round(alg_bytes / t / 1e9, 3),
        "hbm_frac_of_peak": round(alg_bytes / t / 1e9 / PEAK_HBM_GBPS, 4),
        # the bytes the counters saw move, over the same time
        "hbm_measured_GBps": round(traffic / t / 1e9, 3) if traffic else None,
        "hbm_measured_frac_of_peak": round(traffic / t / 1e9 / PEAK_HBM_GBPS, 4)
        if traffic else None,
        # every hop's load and store counted (L2-served in the fused form):
        # not an HBM rate
        "hop_rate_GBps": round(hop_bytes / t / 1e9, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "kernel": kernel, "alg_bytes_per_launch": alg_bytes,
                     "alg_bytes_formula": "2 R N s (R input rows read, R output rows written)"
                     if launch_name == "fused" else "5 (R-1) N s (every hop through memory)",
                     "hop_bytes_per_launch": hop_bytes,
                     "kernel_ms": round(kernel_ms, 6)},
        "wall_s_timed": round(wall, 4),
    }
    y = None
    if not args.no_cpu_baseline:
        y, line["cpu_baseline"] = cpu_baseline(x, R, N, s, strides=comm.channel_strides())
    else:
        line["cpu_baseline"] = None
    ok = True
    if y is not None:
        got = recv.cpu().numpy()
        line["verified_vs_oracle"] = bool(got.tobytes() == y.tobytes())
        ok = line["verified_vs_oracle"] and line["cpu_baseline"]["legs_bit_identical"]
        if not line["verified_vs_oracle"]:
            log("ERROR: GPU result differs from the oracle")
    if not args.no_extras:
        extras = {}
        run_extra(extras, "stream_ceiling", lambda: copy_ceiling(torch, api))
        run_extra(extras, "pipelined_ring",
                  lambda: pipelined_headline(torch, api, measure, send, recv, y, R, N, s))
        del send, recv
        torch.cuda.empty_cache()
        run_extra(extras, "sweep", lambda: sweep_fit(torch, api, measure, inputs, np))
        run_extra(extras, "tree_vs_ring", lambda: tree_vs_ring_fit(torch, api, measure, inputs, np))
        run_extra(extras, "buckets", lambda: buckets_few(torch, api, measure, inputs, np,
                                                         args.extra_buckets))
        for k, v in extras.items():
            line[k] = v
            if isinstance(v, dict) and (v.get("error") or v.get("exact") is False):
                ok = False
    print(json.dumps(line), flush=True)
    return 0 if ok else 1


def copy_ceiling(torch, api):
    """A plain 512 MiB device copy (non-temporal loads and stores): the
    streaming ceiling the kernels are compared with."""
    dev = torch.device("cuda:0")
    n = (512 << 20)
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    c = torch.empty_like(a)
    a.fill_(1)
    st = torch.cuda.current_stream().cuda_stream
    _, ms, _ = time_calls(lambda: api.ar_stream_copy(a.data_ptr(), c.data_ptr(), n, st), 20, 5,
                          torch)
    gbps = 2 * n / (ms / 20 / 1e3) / 1e9
    # the headline's row pattern without its hops: 8 rows of 64 MiB read and
    # 8 written back from L2, tile by tile (1 GiB moved, like one all-reduce)
    R, rb = 8, 64 << 20
    c.zero_()
    _, ms2, _ = time_calls(lambda: api.ar_stream_rows(a.data_ptr(), c.data_ptr(), R, rb, st),
                           20, 5, torch)
    rows_gbps = 2 * n / (ms2 / 20 / 1e3) / 1e9
    ok = torch.equal(a, c)
    del a, c
    return dict(bytes=n, copy_GBps=round(gbps, 1), frac_of_peak=round(gbps / PEAK_HBM_GBPS, 4),
                rows_pattern_GBps=round(rows_gbps, 1),
                rows_pattern_frac_of_peak=round(rows_gbps / PEAK_HBM_GBPS, 4),
                rows_pattern="8 rows of 64 MiB, 2 KiB tiles per wave, non-temporal loads, "
                             "plain stores", rows_copy_ok=bool(ok))


def pipelined_headline(torch, api, measure, send, recv, y, R, N, s):
    """The headline workload through the pipelined ring: the simple protocol
    (512 KiB chunks handed on through ready flags, device-scope write-through
    stores), one rank per XCD -- the form that maps onto one rank per GPU."""
    comm = api.Comm(R, N, "float32", device=torch.device("cuda:0"), chunk_bytes=512 * 1024,
                    **ring_kw("pipelined"))
    per, total_ms, _ = time_calls(lambda: comm.allreduce(send, recv), 20, 5, torch)
    ok = comm.check() == api.AR_SUCCESS
    t = total_ms / 20 / 1e3
    exact = bool(ok and (y is None or recv.cpu().numpy().tobytes() == y.tobytes()))
    hop = measure.allreduce_alg_bytes(R, N, s)
    traffic = measured_traffic("ring_allreduce_f32_r8_64MiB_pipelined")
    comm.close()
    return dict(ms=round(t * 1e3, 4), busbw_GBps=round(N * s / t / 1e9 * 1.75, 1),
                hbm_GBps=round(hop / t / 1e9, 1), hbm_frac_of_peak=round(hop / t / 1e9 / 8000, 4),
                traffic=traffic, exact=exact, chunk_bytes=512 * 1024)


def timed_point(fn, torch, eager):
    """ms per call of one sweep point: 5 warm-up then 20 timed calls, as one
    graph replay, or enqueued one by one (eager: one traced dispatch per call,
    for profiler runs)."""
    if eager:
        _, total_ms, _ = time_calls(fn, 20, 5, torch)
        return total_ms / 20
    return time_graph(fn, 20, torch)


def sweep_fit(torch, api, measure, inputs, np, max_bytes=1 << 30, launch="fused", eager=False):
    """The message-size sweep: R = 8 fp32 N(0,1), 8 B .. 1 GiB per rank (28 sizes), 5
    warm-up then 20 timed calls each (one graph replay), fit T = a + b n."""
    R, s = 8, 4
    dev = torch.device("cuda:0")
    counts = inputs.sweep_counts(8, max_bytes, s)
    Nmax = counts[-1]
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    send_flat = torch.randn(R * Nmax, generator=g, device=dev, dtype=torch.float32)
    recv_flat = torch.empty_like(send_flat)
    comm = api.Comm(R, Nmax, "float32", device=dev, chunk_bytes=512 * 1024, **ring_kw(launch))
    pts = []
    exact = True
    for N in counts:
        sv = send_flat[:R * N].view(R, N)
        rv = recv_flat[:R * N].view(R, N)
        t = timed_point(lambda: comm.allreduce(sv, rv), torch, eager) / 1e3
        pts.append([N * s, round(t * 1e6, 3)])
        if N * s <= (1 << 20):  # check the small and mid sizes against the oracle
            xs = sv.cpu().numpy()
            ref, _, _, _ = cpu_baseline_leg(lambda o: o.ring_allreduce(xs), 0.0, 1,
                                            threads=cpu_info()["threads"])
            exact &= rv.cpu().numpy().tobytes() == ref.tobytes()
    exact &= comm.check() == api.AR_SUCCESS
    comm.close()
    del send_flat, recv_flat
    torch.cuda.empty_cache()
    n = [p[0] for p in pts]
    ts = [p[1] / 1e6 for p in pts]
    fit = measure.fit_alpha_beta(n, ts)
    small = sorted(p[1] for p in pts if p[0] <= 4096)
    large = [p for p in pts if p[0] >= 64 << 20]
    out = dict(launch=launch, R=R, dtype="f32", sizes=len(pts), timing="5 warm-up + 20 timed "
               "calls per size, " + ("enqueued one by one" if eager else "one graph replay"),
               exact_up_to_1MiB=bool(exact), exact=bool(exact),
               alpha_us=round(fit["alpha_us"], 3), inv_beta_GBps=round(fit["inv_beta_GBps"], 1),
               bus_rate_GBps=round(fit["inv_beta_GBps"] * measure.busbw_factor("allreduce", R), 1),
               r2=round(fit["r2"], 5), max_rel_residual=round(fit["max_rel_residual"], 4),
               points_bytes_us=pts)
    if small:
        out["alpha_median_le_4KiB_us"] = small[len(small) // 2]
    if len(large) >= 2:
        a, b = large[0], large[-1]
        out["inv_beta_ge_64MiB_GBps"] = round((b[0] - a[0]) / ((b[1] - a[1]) / 1e6) / 1e9, 1)
    return out


TVR_VARIANTS = [("tree-ll", dict(algo="tree", proto="ll")),
                ("tree-fused", dict(algo="tree", proto="simple", launch="fused")),
                ("ring-fused", dict(algo="ring", proto="simple", launch="fused")),
                ("ring-pipelined", dict(algo="ring", proto="simple", launch="pipelined")),
                ("ring-ll", dict(algo="ring", proto="ll")),
                ("ring-step", dict(algo="ring", proto="simple", launch="step"))]


def tree_depth(api, probe_R):
    """Edges on the longest root-to-leaf path of the deeper of the two trees
    (the hops one way), from the library's own tree view."""
    c = api.ar_init(probe_R, 1, api.AR_FLOAT32, api.AR_TREE)
    try:
        depth = 0
        for t in (0, 1):
            for r in range(probe_R):
                d, v = 0, r
                while api.ar_tree_parent(c, t, v) >= 0:
                    v = api.ar_tree_parent(c, t, v)
                    d += 1
                depth = max(depth, d)
        return depth
    finally:
        api.ar_destroy(c)


def tree_vs_ring_fit(torch, api, measure, inputs, np, max_bytes=256 * 1024, eager=False, R=8):
    """Tree against ring: R = 8 (or R) fp32 U[-1,1), 8 B .. 256 KiB per rank (16 sizes): the
    double binary tree (fused, and with LL) against every ring form (5 warm-up
    + 20 timed calls per size, one graph replay); an alpha-beta fit per
    variant, the crossover of each ring form with its tree (the fused tree for
    the fused ring, the LL tree for the others; measured and from the fits),
    and AR_AUTO's choice before and after loading the fitted lines (for the
    hand-off forms also with AR_PROTO_AUTO: tree + LL, ring + LL or the
    simple protocol)."""
    s = 4
    dev = torch.device("cuda:0")
    counts = inputs.sweep_counts(8, max_bytes, s)
    Nmax = counts[-1]
    x = inputs.draw("uniform_pm1", R, Nmax, seed=4)
    send_flat = torch.from_numpy(x).to(dev).reshape(-1)
    recv_flat = torch.empty_like(send_flat)
    comms = {name: api.Comm(R, Nmax, "float32", device=dev, **kw) for name, kw in TVR_VARIANTS}
    res = {name: [] for name, _ in TVR_VARIANTS}
    exact = True
    threads = cpu_info()["threads"]
    for N in counts:
        sv = send_flat[:R * N].view(R, N)
        rv = recv_flat[:R * N].view(R, N)
        xs = sv.cpu().numpy()
        for name, _ in TVR_VARIANTS:
            c = comms[name]
            res[name].append(round(timed_point(lambda: c.allreduce(sv, rv), torch, eager) * 1e3, 3))
            if N in (counts[0], counts[len(counts) // 2], counts[-1]):
                ref, _, _, _ = cpu_baseline_leg(
                    (lambda o: o.tree_allreduce(xs)) if name.startswith("tree")
                    else (lambda o: o.ring_allreduce(xs)), 0.0, 1, threads=threads)
                exact &= rv.cpu().numpy().tobytes() == ref.tobytes()
    for c in comms.values():
        exact &= c.check() == api.AR_SUCCESS
        c.close()
    sizes = [n * s for n in counts]
    fits = {name: measure.fit_alpha_beta(sizes, [t / 1e6 for t in ts]) for name, ts in res.items()}
    # the tree AR_AUTO weighs against each ring form: the fused tree beside
    # the fused ring, the LL tree beside the forms that hand off between ranks
    tree_of = lambda name: "tree-fused" if name == "ring-fused" else "tree-ll"
    crossover = {}
    for name, _ in TVR_VARIANTS:
        if name.startswith("tree"):
            continue
        # the smallest size from which this ring form is faster than its tree
        # at every larger size of the range
        tr = tree_of(name)
        meas = None
        for i in range(len(sizes)):
            if all(res[name][j] < res[tr][j] for j in range(i, len(sizes))):
                meas = sizes[i]
                break
        fitted = measure.crossover_bytes(fits[tr], fits[name])
        crossover[name] = dict(measured_bytes=meas,
                               fit_bytes=round(fitted) if fitted is not None else None)
    # AR_AUTO's choice for each ring form: with the library's default lines,
    # then with the lines fitted here; and how often the choice matches the
    # faster of the two measured times
    probe = api.Comm(R, Nmax, "float32", "auto", device=dev)
    auto = {}
    forms = {"ring-fused": dict(launch=api.AR_LAUNCH_FUSED, proto=api.AR_SIMPLE),
             "ring-pipelined": dict(launch=api.AR_LAUNCH_PIPELINED, proto=api.AR_SIMPLE),
             "ring-step": dict(launch=api.AR_LAUNCH_STEP, proto=api.AR_SIMPLE),
             "ring-ll": dict(launch=api.AR_LAUNCH_FUSED, proto=api.AR_LL)}

    def choices():
        out = {}
        for name, f in forms.items():
            probe.set_option(api.AR_OPT_LAUNCH, f["launch"])
            probe.set_option(api.AR_OPT_PROTO, f["proto"])
            plan = [probe.plan(n)[0] for n in counts]
            faster = [api.AR_TREE if res[tree_of(name)][i] < res[name][i] else api.AR_RING
                      for i in range(len(counts))]
            out[name] = dict(tree_max_bytes=api.ar_auto_tree_max_bytes(probe.handle),
                             matches_measured=sum(p == q for p, q in zip(plan, faster)),
                             of=len(counts))
        return out

    def proto_auto():
        # with AR_PROTO_AUTO a hand-off form's call runs tree + LL, ring + LL
        # or its simple protocol; how often that is the fastest of the three
        out = {}
        for name in ("ring-pipelined", "ring-step"):
            probe.set_option(api.AR_OPT_LAUNCH, forms[name]["launch"])
            probe.set_option(api.AR_OPT_PROTO, api.AR_PROTO_AUTO)
            picks = []
            for n in counts:
                a, p, _ = probe.plan(n)
                picks.append("tree-ll" if a == api.AR_TREE else "ring-ll" if p == api.AR_LL
                             else name)
            best = [min(("tree-ll", "ring-ll", name), key=lambda v: res[v][i])
                    for i in range(len(counts))]
            out[name] = dict(matches_measured=sum(p == b for p, b in zip(picks, best)),
                             of=len(counts),
                             picks={v: picks.count(v) for v in ("tree-ll", "ring-ll", name)})
        probe.set_option(api.AR_OPT_PROTO, api.AR_SIMPLE)
        return out

    auto["default_lines"] = choices()
    auto["default_lines_protocol_auto"] = proto_auto()
    for name, f in fits.items():
        # a line that barely rises over this range fits a huge (or negative)
        # bandwidth: cap it at 1e6 GB/s, which adds < 1 ns at 256 KiB
        bw = f["inv_beta_GBps"]
        bw = 1e6 if not (0 < bw < 1e6) else bw
        api.ar_set_cost(probe.handle, api.COST_FORMS[name], max(0.0, f["alpha_us"]), bw)
    auto["fitted_lines"] = choices()
    auto["fitted_lines_protocol_auto"] = proto_auto()
    probe.close()
    hop = ll_hop_latency_us(torch)
    # the stream is looked up at each call: under capture it is the graph's
    floor = time_graph(lambda: api.ar_stream_copy(send_flat.data_ptr(), recv_flat.data_ptr(), 16,
                                                  torch.cuda.current_stream().cuda_stream),
                       20, torch) * 1e3
    del send_flat, recv_flat
    _, t_or, n_or, used = cpu_baseline_leg(lambda o: o.tree_allreduce(x), 1.0, 5)
    return dict(R=R, dtype="f32", sizes_bytes=sizes, t_us=res, exact=bool(exact),
                fits={k: dict(alpha_us=round(v["alpha_us"], 3),
                              inv_beta_GBps=round(v["inv_beta_GBps"], 2), r2=round(v["r2"], 4))
                      for k, v in fits.items()},
                crossover=crossover, auto=auto, ll_hop_us=hop,
                tree_hops=2 * tree_depth(api, probe_R=R), ring_hops=2 * (R - 1),
                launch_floor_us=round(floor, 3),
                cpu_baseline=dict(kind="oracle", cores=used, us_per_call=round(t_or * 1e6, 1),
                                  sample="tree all-reduce at %d bytes per rank, R = %d, %d call(s)"
                                  % (Nmax * s, R, n_or)))


def buckets_few(torch, api, measure, inputs, np, nb=4):
    """The gradient buckets, the first `nb`: R = 16 bf16 N(0,0.02), 13,107,200
    elements (25 MiB) per rank each; reduce-scatter, then all-gather, then
    all-reduce of every bucket in turn, timed per bucket (5 warm-up passes
    over the buckets, then 20 timed).  Every bucket is checked: the
    reduce-scatter against the oracle's, the all-gather against the oracle's
    all-gather of those shards, and RS then AG equal to the all-reduce bit for
    bit."""
    w = inputs.WORKLOADS["buckets_bf16_r16"]
    R, N, s = w["R"], w["count"], 2
    n = N // R
    dev = torch.device("cuda:0")
    xs = [inputs.device_bucket_bf16(R, N, w["seed"], b, dev) for b in range(nb)]
    shards = [torch.empty((R, n), dtype=torch.bfloat16, device=dev) for _ in range(nb)]
    fulls = [torch.empty((R, N), dtype=torch.bfloat16, device=dev) for _ in range(nb)]
    ars = [torch.empty((R, N), dtype=torch.bfloat16, device=dev) for _ in range(nb)]
    comm = api.Comm(R, N, "bf16", device=dev)

    def each(fn):
        return lambda: [fn(b) for b in range(nb)]

    out, t_of = {}, {}
    for name, fn, hbm, hop in (
            ("reduce_scatter", each(lambda b: comm.reduce_scatter(xs[b], shards[b])),
             measure.reduce_scatter_hbm_bytes(R, N, s), measure.reduce_scatter_alg_bytes(R, N, s)),
            ("all_gather", each(lambda b: comm.all_gather(shards[b], fulls[b])),
             measure.all_gather_hbm_bytes(R, N, s), measure.all_gather_alg_bytes(R, N, s)),
            ("allreduce", each(lambda b: comm.allreduce(xs[b], ars[b])),
             measure.allreduce_hbm_bytes(R, N, s), measure.allreduce_alg_bytes(R, N, s, acc=4))):
        _, total_ms, _ = time_calls(fn, 20, 5, torch)
        t = t_of[name] = total_ms / 20 / nb / 1e3
        algbw = N * s / t / 1e9
        f = measure.busbw_factor("allreduce" if name == "allreduce" else "rs", R)
        # counter bytes of the same kernel (fused form), while its sources match
        meas = measured_traffic("bucket_bf16_r16_25MiB_%s_fused" % name)
        out[name] = dict(us_per_bucket=round(t * 1e6, 2), algbw_GBps=round(algbw, 1),
                         busbw_GBps=round(algbw * f, 1),
                         hbm_GBps=round(hbm / t / 1e9, 1),
                         hbm_frac_of_peak=round(hbm / t / 1e9 / PEAK_HBM_GBPS, 4),
                         hbm_measured_GBps=round(meas / t / 1e9, 1) if meas else None,
                         hbm_measured_frac_of_peak=(round(meas / t / 1e9 / PEAK_HBM_GBPS, 4)
                                                    if meas else None),
                         hop_rate_GBps=round(hop / t / 1e9, 1))
    # the pair the buckets run: reduce-scatter then all-gather, an all-reduce
    t2 = t_of["reduce_scatter"] + t_of["all_gather"]
    out["rs_then_ag"] = dict(us_per_bucket=round(t2 * 1e6, 2), algbw_GBps=round(N * s / t2 / 1e9, 1),
                             busbw_GBps=round(N * s / t2 / 1e9 *
                                              measure.busbw_factor("allreduce", R), 1))
    ok = comm.check() == api.AR_SUCCESS
    threads = cpu_info()["threads"]
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(nb):
        xb = bits(xs[b])
        ref_rs, _, _, _ = cpu_baseline_leg(lambda o: o.ring_reduce_scatter(xb, "bf16"), 0.0, 1,
                                           threads=threads)
        ref_ag, _, _, _ = cpu_baseline_leg(lambda o: o.ring_all_gather(ref_rs, "bf16"), 0.0, 1,
                                           threads=threads)
        ok &= np.array_equal(bits(shards[b]), ref_rs)
        ok &= np.array_equal(bits(fulls[b]), ref_ag)
        ok &= torch.equal(fulls[b].view(torch.int16), ars[b].view(torch.int16))
    comm.close()
    del xs, shards, fulls, ars
    torch.cuda.empty_cache()
    return dict(R=R, dtype="bf16", buckets=nb, count_per_rank=N, exact=bool(ok), **out)


def mode_sweep(args):
    """The message-size sweep alone: ring all-reduce, R = 8, fp32, 8 B .. --max-bytes per
    rank in powers of two, 5 warm-up + 20 timed calls each; alpha-beta fit."""
    import numpy as np
    import torch
    from collective_communication_ring_amd import api, inputs, measure
    out = sweep_fit(torch, api, measure, inputs, np, args.max_bytes, args.launch
                    if args.launch != "auto" else "fused", eager=args.eager)
    print(json.dumps(dict(mode="sweep_fit", **out)), flush=True)
    return 0 if out["exact"] else 1


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
    """Tree against ring alone (up to --tvr-max-bytes per rank): tree + LL against every
    ring form, fits, crossovers and AR_AUTO's choices."""
    import numpy as np
    import torch
    from collective_communication_ring_amd import api, inputs, measure
    out = tree_vs_ring_fit(torch, api, measure, inputs, np, args.tvr_max_bytes, eager=args.eager,
                           R=args.tvr_ranks)
    print(json.dumps(dict(mode="tree_vs_ring", **out)), flush=True)
    return 0 if out["exact"] else 1


def mode_buckets(args):
    """The gradient buckets: R = 16 bf16 N(0, 0.02), 40 buckets x 13,107,200 elements per
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
    for name, fn, op, hbm, hop in (
            ("reduce_scatter", rs_all, "rs", measure.reduce_scatter_hbm_bytes(R, N, s),
             measure.reduce_scatter_alg_bytes(R, N, s)),
            ("all_gather", ag_all, "ag", measure.all_gather_hbm_bytes(R, N, s),
             measure.all_gather_alg_bytes(R, N, s)),
            ("allreduce", ar_all, "ar", measure.allreduce_hbm_bytes(R, N, s), None)):
        _, total_ms, _ = time_calls(fn, args.steps, 1, torch)
        t = total_ms / args.steps / B / 1e3  # per bucket
        algbw = N * s / t / 1e9
        f = measure.busbw_factor("allreduce" if op == "ar" else op, R)
        rep[name] = dict(t_us_per_bucket=t * 1e6, algbw_GBps=algbw, busbw_GBps=algbw * f,
                         hbm_GBps=hbm / t / 1e9, hbm_frac_of_peak=hbm / t / 1e9 / PEAK_HBM_GBPS,
                         hop_rate_GBps=(hop / t / 1e9) if hop else None)
        log(name, rep[name])
    assert comm.check() == api.AR_SUCCESS
    import numpy as np
    xh = xs[0].view(torch.int16).cpu().numpy().view(np.uint16)
    sh, t_rs, _, _ = cpu_baseline_leg(lambda o: o.ring_reduce_scatter(xh, "bf16"), 0.0, 1)
    _, t_ag, _, _ = cpu_baseline_leg(lambda o: o.ring_all_gather(sh, "bf16"), 0.0, 1)
    rep["cpu_baseline"] = dict(kind="oracle", cores=1, sample="bucket 0, one call each",
                               reduce_scatter_us=t_rs * 1e6, all_gather_us=t_ag * 1e6)
    summary = dict(mode="buckets", R=R, dtype="bf16", buckets=B, count_per_rank=N, **rep)
    print(json.dumps(summary), flush=True)
    return 0


def mode_stream(args):
    """Reference kernels: c = a + b over float32 (the access mix of one reduce
    step), a plain copy, and the all-reduce's row pattern without hops (R rows
    read and written back tile by tile, ar_stream_rows), each on 512 MiB
    arrays (larger than the 256 MB infinity cache)."""
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
    rows = {}
    for R in (2, 4, 8, 16):  # the all-reduce's row pattern without hops, R rows
        c.zero_()
        _, ms3, _ = time_calls(lambda: api.ar_stream_rows(a.data_ptr(), c.data_ptr(), R,
                                                          n * 4 // R, st),
                               args.steps, args.warmup, torch)
        torch.cuda.synchronize()
        rows[R] = dict(GBps=round(2 * n * 4 / (ms3 / args.steps / 1e3) / 1e9, 1),
                       ok=bool(torch.equal(c, a)))
    summary = dict(mode="stream", bytes_per_array=n * 4, add_GBps=add_gbps,
                   add_frac=add_gbps / PEAK_HBM_GBPS, copy_GBps=copy_gbps,
                   copy_frac=copy_gbps / PEAK_HBM_GBPS, copy_ok=ok, rows_pattern=rows)
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
    known size (the calibration) and the headline's row pattern without hops
    (ar_stream_rows), then 3 all-reduces of the headline workload in each
    ring launch form and by the fused tree, then 3 small all-reduces by each
    tree form, then 3 reduce-scatters, all-gathers and all-reduces (ring,
    then fused tree) of one 25 MiB gradient bucket."""
    import torch
    from collective_communication_ring_amd import api, inputs
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    n = (512 << 20) // 4
    a = torch.randn(n, device=dev)
    c = torch.empty_like(a)
    for _ in range(3):
        api.ar_stream_copy(a.data_ptr(), c.data_ptr(), n * 4, st)
    # the headline's row pattern without hops: 8 rows of 64 MiB
    for _ in range(3):
        api.ar_stream_rows(a.data_ptr(), c.data_ptr(), 8, n * 4 // 8, st)
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
    # the fused tree on the same workload (16-byte packs)
    comm = api.Comm(R, N, "float32", "tree", "simple", device=dev, launch="fused")
    for _ in range(3):
        comm.allreduce(send, recv)
    torch.cuda.synchronize()
    small = send[:, :65536].contiguous()
    out = torch.empty_like(small)
    for proto, launch in (("ll", None), ("simple", "fused")):
        comm = api.Comm(R, 65536, "float32", "tree", proto, device=dev, launch=launch)
        for _ in range(3):
            comm.allreduce(small, out)
    torch.cuda.synchronize()
    del send, recv, small, out
    # one 25 MiB gradient bucket (R = 16 bf16): reduce-scatter, all-gather, all-reduce
    w = inputs.WORKLOADS["buckets_bf16_r16"]
    Rb, Nb = w["R"], w["count"]
    xb = inputs.device_bucket_bf16(Rb, Nb, w["seed"], 0, dev)
    shard = torch.empty((Rb, Nb // Rb), dtype=torch.bfloat16, device=dev)
    full = torch.empty((Rb, Nb), dtype=torch.bfloat16, device=dev)
    comm = api.Comm(Rb, Nb, "bf16", device=dev)
    for _ in range(3):
        comm.reduce_scatter(xb, shard)
    for _ in range(3):
        comm.all_gather(shard, full)
    for _ in range(3):
        comm.allreduce(xb, full)
    comm = api.Comm(Rb, Nb, "bf16", "tree", "simple", device=dev, launch="fused")
    for _ in range(3):
        comm.allreduce(xb, full)
    torch.cuda.synchronize()
    print(json.dumps(dict(mode="counters", copy_bytes=n * 4, allreduce_count=N,
                          bucket_count=Nb)), flush=True)
    return 0


def mode_r4_int32(args):
    """Ring all-reduce (sum), R = 4, int32, 4096 elements per rank,
    chunk = count / R; time per call (graph-replayed) in every form and both
    tree forms, each result checked bit for bit against the int64 sum (and
    the rings against the oracle's ring)."""
    import numpy as np
    import torch
    from collective_communication_ring_amd import api, inputs
    R, N = 4, 4096
    dev = torch.device("cuda:0")
    x = inputs.host_inputs("ring_int32_r4")
    ref, t_or, n_or, _ = cpu_baseline_leg(lambda o: o.ring_allreduce(x), 2.0)
    exact = x.astype(np.int64).sum(axis=0).astype(np.int32)
    send = torch.from_numpy(x).to(dev)
    recv = torch.empty_like(send)
    res = {}
    for name, kw in (("fused", ring_kw("fused")), ("step", ring_kw("step")),
                     ("pipelined", ring_kw("pipelined")), ("ll", ring_kw("ll")),
                     ("tree-ll", dict(algo="tree", proto="ll")),
                     ("tree-fused", dict(algo="tree", proto="simple", launch="fused"))):
        comm = api.Comm(R, N, "int32", device=dev, chunk_bytes=(N // R) * 4, **kw)
        t_us = time_graph(lambda: comm.allreduce(send, recv), 20, torch) * 1e3
        got = recv.cpu().numpy()
        ok = comm.check() == api.AR_SUCCESS and (got == exact[None, :]).all() and (
            name.startswith("tree") or got.tobytes() == ref.tobytes())
        res[name] = dict(t_us=round(t_us, 3), exact=bool(ok))
        log("r4-int32 %-10s %8.2f us  exact=%s" % (name, t_us, ok))
        comm.close()
    print(json.dumps(dict(mode="r4-int32", R=R, count_per_rank=N, dtype="int32", results=res,
                          cpu_baseline=dict(kind="oracle", cores=1, t_us=t_or * 1e6,
                                            sample="%d calls" % n_or))), flush=True)
    return 0 if all(r["exact"] for r in res.values()) else 1


def mode_tree_large(args):
    """The two tree forms beside the fused ring on the 64 MiB-per-rank inputs
    (R = 8 fp32, N(0,1) seed 2) and on their first 4 and 16 MiB per rank:
    after ~20 ms of untimed calls, event-timed 5 warm-up + 20 calls per
    point (host-enqueued), the 2 R N s
    compulsory bytes' HBM rate, and every 64 MiB result checked bit for bit
    against the oracle's tree or ring; then the fused tree and the fused ring
    on one gradient bucket (R = 16 bf16, 25 MiB per rank), also checked."""
    import torch
    from collective_communication_ring_amd import api, inputs, measure
    dev = torch.device("cuda:0")
    x = inputs.host_inputs("ring_f32_r8_64MiB")
    R, N = x.shape
    s = 4
    send = torch.from_numpy(x).to(dev)
    recv = torch.empty_like(send)
    forms = (("tree-fused", dict(algo="tree", proto="simple", launch="fused")),
             ("tree-ll", dict(algo="tree", proto="ll")),
             ("ring-fused", dict(algo="ring", proto="simple", launch="fused")))
    threads = cpu_info()["threads"]
    res, exact = {}, True
    # ~20 ms of untimed calls first: the first point follows a 512 MiB upload,
    # and 5 warm-up calls of ~20 us each are too short for it otherwise
    comm = api.Comm(R, N, "float32", device=dev, **dict(forms[2][1]))
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.02:
        comm.allreduce(send, recv)
        torch.cuda.synchronize()
    comm.close()
    for n in (N // 16, N // 4, N):
        sv = send.reshape(-1)[:R * n].view(R, n)
        rv = recv.reshape(-1)[:R * n].view(R, n)
        for name, kw in forms:
            comm = api.Comm(R, n, "float32", device=dev, **kw)
            per, total_ms, _ = time_calls(lambda: comm.allreduce(sv, rv), 20, 5, torch)
            us = total_ms / 20 * 1e3
            ok = comm.check() == api.AR_SUCCESS
            if n == N:
                ref, _, _, _ = cpu_baseline_leg(
                    (lambda o: o.tree_allreduce(x)) if name.startswith("tree")
                    else (lambda o: o.ring_allreduce(x)), 0.0, 1, threads=threads)
                ok &= rv.cpu().numpy().tobytes() == ref.tobytes()
            exact &= bool(ok)
            hbm = measure.allreduce_hbm_bytes(R, n, s) / (us / 1e6) / 1e9
            res.setdefault(str(n * s), {})[name] = dict(us=round(us, 2), hbm_GBps=round(hbm, 1),
                                                       hbm_frac=round(hbm / PEAK_HBM_GBPS, 4))
            log("tree-large %9d B/rank %-10s %9.2f us  %7.1f GB/s" % (n * s, name, us, hbm))
            comm.close()
    del send, recv
    torch.cuda.empty_cache()
    # one gradient bucket (R = 16 bf16, 25 MiB per rank): fused tree and fused ring
    w = inputs.WORKLOADS["buckets_bf16_r16"]
    Rb, Nb = w["R"], w["count"]
    xb = inputs.device_bucket_bf16(Rb, Nb, w["seed"], 0, dev)
    full = torch.empty_like(xb)
    xh = xb.view(torch.int16).cpu().numpy().view("uint16")
    bucket = {}
    for name, kw in forms[::2]:
        comm = api.Comm(Rb, Nb, "bf16", device=dev, **kw)
        per, total_ms, _ = time_calls(lambda: comm.allreduce(xb, full), 20, 5, torch)
        us = total_ms / 20 * 1e3
        ref, _, _, _ = cpu_baseline_leg(
            (lambda o: o.tree_allreduce(xh, "bf16")) if name.startswith("tree")
            else (lambda o: o.ring_allreduce(xh, "bf16")), 0.0, 1, threads=threads)
        ok = comm.check() == api.AR_SUCCESS and \
            full.view(torch.int16).cpu().numpy().view("uint16").tobytes() == ref.tobytes()
        exact &= bool(ok)
        hbm = measure.allreduce_hbm_bytes(Rb, Nb, 2) / (us / 1e6) / 1e9
        bucket[name] = dict(us=round(us, 2), hbm_GBps=round(hbm, 1))
        log("tree-large bucket R=16 bf16 %-10s %9.2f us" % (name, us))
        comm.close()
    print(json.dumps(dict(mode="tree_large", R=R, dtype="f32", exact=exact, results=res,
                          bucket_r16_bf16_25MiB=bucket)), flush=True)
    return 0 if exact else 1


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
            ref, t_or, _, _ = cpu_baseline_leg(lambda o: o.ring_allreduce(x, dtype), 0.0, 1)
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
            ref, t_or, _, _ = cpu_baseline_leg(
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
                    choices=["headline", "r4-int32", "matrix", "sweep", "tree-vs-ring",
                             "tree-large", "buckets", "stream", "counters", "tune", "overlap"])
    ap.add_argument("--max-bytes", type=int, default=1 << 30)
    ap.add_argument("--tvr-ranks", type=int, default=8, help="tree-vs-ring: logical ranks R")
    ap.add_argument("--tvr-max-bytes", type=int, default=256 * 1024,
                    help="tree-vs-ring: largest per-rank size (the default stops at 256 KiB)")
    ap.add_argument("--buckets", type=int, default=0)
    ap.add_argument("--out", default=None)
    ap.add_argument("--grids", default="256,512,768,1024,1280,1536,1792,2048")
    ap.add_argument("--gemms", type=int, default=8, help="overlap mode: GEMMs per iteration")
    ap.add_argument("--comm-cus", type=int, default=0,
                    help="overlap mode: CUs reserved for the collective (0: no CU masks)")
    ap.add_argument("--chunk-bytes", type=int, default=512 * 1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline: only the headline workload (no sweep, tree-vs-ring, buckets, "
                         "pipelined ring or copy ceiling)")
    ap.add_argument("--extra-buckets", type=int, default=4,
                    help="headline: 25 MiB gradient buckets timed and checked in the extras")
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
    fn = {"headline": headline, "r4-int32": mode_r4_int32, "matrix": mode_matrix,
          "sweep": mode_sweep, "tree-vs-ring": mode_tree_vs_ring, "tree-large": mode_tree_large,
          "buckets": mode_buckets, "stream": mode_stream, "counters": mode_counters,
          "tune": mode_tune, "overlap": mode_overlap}[args.mode]
    return fn(args)


if __name__ == "__main__":
    sys.exit(main())
