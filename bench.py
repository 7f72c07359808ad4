#!/usr/bin/env python3
"""Benchmark of the fused halo exchange on one MI355X.

One step = one coordinate exchange (halo_exchange_x) + one force exchange
(halo_exchange_f) over the 8x8x8-domain, 22 nm, 1,064,800-atom box (cutoff
1.2 nm, three forwarding pulses, about 2.09 M halo entries per exchange).

Inputs are resident in HBM before the timed region. Each step uses the next of
R replicas (plan metadata, x and f), so that successive steps do not find
their data in the 256 MB Infinity Cache: the timed numbers are HBM numbers.

Prints ONE JSON line (rank 0). `value` is halo atoms/s: halo entries per
exchange divided by the time of one step (coordinates out and forces back).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "halo atoms/s and HBM GB/s (% of peak); µs per coord+force exchange"
# The library's rule for the default exchanges (halo_exchange_x / _f in
# csrc/halo_api.hip): the transposed kernels from these sizes on.
TRANSPOSED_X_MIN_ENTRIES = 1 << 20
TRANSPOSED_F_MIN_ENTRIES = 1 << 20
TRANSPOSED_F_MAX_PULSES = 3
HBM_PEAK_GBS = 8000.0
BYTES_X = 28  # per entry: 4 B index + 12 B gathered source + 12 B store
BYTES_F = 40  # per entry: 4 B index + 12 B region read + 12 B target read + 12 B target write
MALL_BYTES = 256 << 20
MAX_REPLICAS = 128
# The device code of the exchange kernels and the flags it is compiled with
# (the traffic counters in profiles/ are valid while these files are
# unchanged).
KERNEL_SOURCES = ["domain_decomposition_halo_fusedpackx_amd/csrc/exchange_kernels.hpp",
                  "domain_decomposition_halo_fusedpackx_amd/csrc/sync.hpp",
                  "domain_decomposition_halo_fusedpackx_amd/build.py"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload_name: str, kernel: str, sha: str):
    """Measured HBM bytes per launch from the committed PMC summary, if it
    was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"pmc_traffic_{workload_name}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha") != sha:
        return None
    key = f"{kernel}_bytes_per_launch"
    return float(vals[key]) if key in vals else None


def cpu_baseline(w, pos, seconds: float):
    """The serial C oracle on the same workload, single thread, host cores."""
    from oracle import oracle
    from domain_decomposition_halo_fusedpackx_amd import workloads as W

    o = oracle.Oracle(pos, w.box, w.grid, w.cutoff)
    entries = sum(o.pulse(p, d)["send_size"] for p in range(o.n_pulse) for d in range(o.n_dom))
    x = o.home_filled(np.nan)
    base, n_home, n_halo = o.domains()
    f = W.halo_forces(o.total_slots, base, n_home, n_halo, w.seed)

    def timed(fn, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if (el >= budget and reps >= 3) or reps >= 10000:
                return reps, el

    # one thread, pinned to one of the cores this process may use
    allowed = os.sched_getaffinity(0)
    core = max(allowed)  # the last one: core 0 also takes the host's interrupts
    os.sched_setaffinity(0, {core})
    try:
        rx, tx = timed(lambda: o.exchange_x(x), seconds / 2)
        rf, tf = timed(lambda: o.exchange_f(f), seconds / 2)
    finally:
        os.sched_setaffinity(0, allowed)
    us_x, us_f = tx / rx * 1e6, tf / rf * 1e6
    return {"value": entries / ((us_x + us_f) * 1e-6), "unit": "halo atoms/s", "cores": 1,
            "kind": "oracle", "us_per_exchange": {"x": us_x, "f": us_f},
            "sample": f"whole {w.name} workload ({entries} halo entries): {rx} coordinate "
                      f"exchanges in {tx:.2f} s, then {rf} force exchanges in {tf:.2f} s; "
                      f"serial C (gcc -O2), 1 thread pinned to core {core}",
            "host_cpus": os.cpu_count(), "host_cpus_allowed": len(allowed),
            "host_cpu": _cpu_model()}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def replica_count(slots, entries):
    """Copies of plan, x and f the timed loops rotate over: enough to exceed
    twice the 256 MB Infinity Cache, so that every exchange streams its data
    from HBM; at most MAX_REPLICAS (the two smallest workloads then stay in
    the cache)."""
    per_rep_bytes = slots * 12 + entries * 4
    return min(MAX_REPLICAS, max(1, -(-2 * MALL_BYTES // per_rep_bytes)))


def time_loop(torch, fn, n):
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for i in range(n):
        fn(i)
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n  # ms


def time_loops(torch, fn, n, loops):
    """`loops` timed loops of n back-to-back calls (call i of a loop gets i,
    so every loop walks the replicas the same way): the median loop's time
    per call in ms, and every loop's, so that the spread is visible."""
    per = [time_loop(torch, fn, n) for _ in range(loops)]
    return float(np.median(per)), per


def spread(per):
    return {"min": min(per), "median": float(np.median(per)), "max": max(per),
            "loops": len(per)}


def launch_floor_us(torch, n):
    """Back-to-back launches of a one-element kernel on the same stream
    (after a warm-up that loads the kernel)."""
    t = torch.zeros(1, device="cuda")
    for _ in range(20):
        t.add_(1.0)
    return time_loop(torch, lambda i: t.add_(1.0), n) * 1e3


def host_call_us(torch, fn, n, loops=5):
    """Host time to issue one call (no synchronisation inside a loop), median
    over loops of n calls: when it exceeds the GPU time of the call,
    back-to-back timings measure the host, not the kernel."""
    per = []
    for _ in range(loops):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            fn(i)
        el = time.perf_counter() - t0
        torch.cuda.synchronize()
        per.append(el / n * 1e6)
    return float(np.median(per))


def cold_exchange_us(torch, plan, x, f, f_init, suffix, reps, clean=True):
    """Median time of one exchange per direction with cold caches, HIP events
    around the lone exchange. Before each timed exchange a 1 GiB device write
    evicts L2 and the 256 MB cache (the force array is restored before it).
    With clean, a 1 GiB read follows the write, so that the caches hold clean
    lines only; without it the exchange also pays for writing back the dirty
    lines the eviction left behind (about 4 us on workload 5)."""
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, device="cuda")
    s = torch.cuda.current_stream()
    ex_x = getattr(plan, "exchange_x" + suffix)
    ex_f = getattr(plan, "exchange_f" + suffix)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(2 * reps)]

    def evict(v):
        scratch.fill_(v)
        if clean:
            sink.add_(scratch.sum())

    for r in range(reps):
        evict(float(r))
        ev[2 * r][0].record(s)
        ex_x(x)
        ev[2 * r][1].record(s)
        f.copy_(f_init)
        evict(float(r) + 0.5)
        ev[2 * r + 1][0].record(s)
        ex_f(f)
        ev[2 * r + 1][1].record(s)
    torch.cuda.synchronize()
    plan.sync()
    tx = [ev[2 * r][0].elapsed_time(ev[2 * r][1]) * 1e3 for r in range(reps)]
    tf = [ev[2 * r + 1][0].elapsed_time(ev[2 * r + 1][1]) * 1e3 for r in range(reps)]
    del scratch
    return {"us_x": float(np.median(tx)), "us_f": float(np.median(tf))}


def plan_build_ms(torch, HaloPlan, w, pos, reps):
    """Wall time of building the plan on the host (halo_plan_create from host
    positions, then the upload), on the GPU (halo_plan_create_device from
    device positions, with either selection) and of rebuilding a device plan in place
    (halo_plan_rebuild_device), median of reps, after one warm-up each."""
    pos_d = torch.from_numpy(pos).cuda()

    def host():
        p = HaloPlan(pos, w.box, w.grid, w.cutoff)
        p.upload()
        torch.cuda.synchronize()
        return p

    def dev():
        p = HaloPlan.on_device(pos_d, w.box, w.grid, w.cutoff)
        torch.cuda.synchronize()
        return p

    def dev_corner():
        p = HaloPlan.on_device(pos_d, w.box, w.grid, w.cutoff, selection="corner")
        torch.cuda.synchronize()
        return p

    out = {}
    for name, fn in (("host_ms", host), ("device_ms", dev), ("device_corner_ms", dev_corner)):
        fn().close()
        ts = []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            p = fn()
            ts.append((time.perf_counter() - t0) * 1e3)
            p.close()
        out[name] = float(np.median(ts))
    # rebuild in place (a repartitioning step: the plan keeps its device memory)
    p = dev()
    p.rebuild_on_device(pos_d)
    ts = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        p.rebuild_on_device(pos_d)
        torch.cuda.synchronize()
        ts.append((time.perf_counter() - t0) * 1e3)
    p.close()
    out["device_rebuild_ms"] = float(np.median(ts))
    out["speedup"] = out["host_ms"] / out["device_ms"]
    out["reps"] = reps
    out["host_threads"] = min(os.cpu_count() or 1, 16)
    return out


def graph_replays(torch, plans, xs, fs, steps):
    """The default exchanges captured in HIP graphs (one graph of X over all
    replicas, one of F, one of whole steps) and replayed: us per exchange and
    ms per step as a graph-launched MD loop would see them. Capturing switches
    the plans to inferring their epochs on the device, so this runs last."""
    R = len(plans)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            g.capture_begin()
            try:
                fn()
            finally:
                g.capture_end()
        torch.cuda.synchronize()
        return g

    gx = capture(lambda: [plans[r].exchange_x(xs[r], s) for r in range(R)])
    gf = capture(lambda: [plans[r].exchange_f(fs[r], s) for r in range(R)])
    gs = capture(lambda: [(plans[r].exchange_x(xs[r], s), plans[r].exchange_f(fs[r], s))
                          for r in range(R)])
    n = max(2, steps // R)
    out = {}
    for name, g in (("us_x", gx), ("us_f", gf), ("ms_per_step", gs)):
        g.replay()
        ms = time_loop(torch, lambda i: g.replay(), n) / R
        out[name] = ms if name == "ms_per_step" else ms * 1e3
    for p in plans:
        p.sync()
    out["exchanges_per_graph"] = R
    return out


def overlap(torch, plan, x, f, reps):
    """The pages' overlap measurement with a synthetic local workload.

    Local work: a bf16 GEMM (4096 x 4096 by 4096 x 2048) on its own stream,
    standing in for the local non-bonded kernel. Non-local work: the
    coordinate exchange followed by the force exchange on the launch stream.
    Both start together after a common event. Local = start to end of the GEMM;
    non-local = start of the coordinate exchange to end of the force exchange;
    non-overlap = end of the GEMM to end of the force exchange, clamped at 0.
    Medians over reps; the same quantities with each side alone for
    reference."""
    a = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(4096, 2048, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(4096, 2048, device="cuda", dtype=torch.bfloat16)
    main = torch.cuda.current_stream()
    loc = torch.cuda.Stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def run(do_local, do_nonlocal):
        rec = []
        for _ in range(reps):
            go, l0, l1, n0, n1 = ev(), ev(), ev(), ev(), ev()
            go.record(main)
            loc.wait_event(go)
            if do_local:
                l0.record(loc)
                with torch.cuda.stream(loc):
                    torch.mm(a, b, out=c)
                l1.record(loc)
            if do_nonlocal:
                n0.record(main)
                plan.exchange_x(x)
                plan.exchange_f(f)
                n1.record(main)
            main.wait_stream(loc)
            rec.append((l0, l1, n0, n1))
        torch.cuda.synchronize()
        plan.sync()
        out = {}
        if do_local:
            out["local_us"] = float(np.median([l0.elapsed_time(l1) for l0, l1, _, _ in rec])) * 1e3
        if do_nonlocal:
            out["nonlocal_us"] = float(np.median([n0.elapsed_time(n1) for _, _, n0, n1 in rec])) * 1e3
        if do_local and do_nonlocal:
            out["non_overlap_us"] = float(np.median(
                [max(0.0, l1.elapsed_time(n1)) for _, l1, _, n1 in rec])) * 1e3
        return out

    run(True, True)  # warm-up
    alone_l, alone_n, both = run(True, False), run(False, True), run(True, True)
    return {"local_work": "bf16 GEMM 4096x4096 @ 4096x2048 on a second stream",
            "nonlocal_work": "halo_exchange_x + halo_exchange_f",
            "local_alone_us": alone_l["local_us"], "nonlocal_alone_us": alone_n["nonlocal_us"],
            **both, "reps": reps}


STAGE_FIELDS = ("start", "wait_begin", "wait_end", "signal", "end")


def stage_profile(torch, HaloPlan, W, w, pos, launches, reps, replicas=1):
    """Where the time of one exchange goes, per kernel: every work unit's
    clock stamps (halo_plan_debug_timing) from the last of `launches`
    back-to-back launches, grouped by stage of the forwarding chain (pulse and
    whether the unit waits for the index-list and direct forms; zone for the
    transposed form). Per group: median and latest time, in us from the first
    unit's start, of the units' start, first wait begin, last wait end, first
    completion signal and end; medians over `reps` repetitions. The kernel's
    duration per launch from HIP events over the same loop is given with it.
    With replicas > 1 the launches rotate over that many copies of plan and
    buffers (as the bench's timed loops do), so that their data come from
    HBM rather than from the caches."""
    plans = [HaloPlan(pos, w.box, w.grid, w.cutoff) for _ in range(replicas)]
    plan = plans[0]
    for p in plans:
        p.upload()
        p.debug_timing(True)
    xs = [torch.from_numpy(plan.home_filled(pos, 0.0)).cuda() for _ in range(replicas)]
    base, n_home, n_halo = plan.domains()
    f0 = W.halo_forces(plan.total_slots, base, n_home, n_halo, w.seed)
    fs = [torch.from_numpy(f0).cuda() for _ in range(replicas)]
    waits = plan.item_waits()
    pulse_of_item = waits[:, 0] // plan.num_domains
    chunks = plan.chunks()
    # plans built on the host run the index-list exchanges on XCD-local units
    lunits = plan.local_units()
    runs = [("x", "indexmap"), ("x", "indexmap_lds"), ("x", "transposed"), ("x", "direct"),
            ("f", "indexmap"), ("f", "transposed")]
    out = {"workload": w.describe(), "halo_entries": plan.num_entries,
           "items": plan.num_items, "chunks": len(chunks), "local_units": len(lunits),
           "launches": launches, "reps": reps, "replicas": replicas}
    for d, form in runs:
        if (form == "transposed" and len(chunks) == 0) or (form == "indexmap_lds" and
                                                            len(lunits) == 0):
            continue
        name = f"exchange_{d}_{form}"
        bufs = xs if d == "x" else fs
        for r in range(replicas):
            getattr(plans[r], name)(bufs[r])  # first calls (origin maps) untimed
        per_rep, ev_us = [], []
        for _ in range(reps):
            ev_us.append(time_loop(
                torch, lambda i: getattr(plans[i % replicas], name)(bufs[i % replicas]),
                launches) * 1e3)
            st, khz = plans[(launches - 1) % replicas].debug_timing_read()
            tick_us = 1e3 / khz
            local = form.startswith("indexmap") and len(lunits) > 0
            n_units = (len(chunks) if form == "transposed" else
                       len(lunits) if local else plan.num_items)
            st = st[:n_units]
            if local:  # empty positions only record their start and end
                st = st[lunits[:, 2] > 0]
            t0 = st[:, 0].min()
            rel = {k: (st[:, i] - t0) * tick_us for i, k in enumerate(STAGE_FIELDS)}
            reached = {k: st[:, i] != 0 for i, k in enumerate(STAGE_FIELDS)}
            if local:
                lu = lunits[lunits[:, 2] > 0]
                nw = lu[:, 3] if d == "x" else lu[:, 4]
                keys = [f"pulse{sg // plan.num_domains}:"
                        f"{('forwards' if d == 'x' else 'waits') if w else ('home' if d == 'x' else 'no wait')}"
                        for sg, w in zip(lu[:, 0], nw)]
            elif form == "transposed":
                keys = ["home" if z < 0 else f"region{z}" for z in chunks[:, 1]]
            elif d == "x" and form == "indexmap":
                keys = [f"pulse{p}:{'forwards' if wm else 'home'}"
                        for p, wm in zip(pulse_of_item, waits[:, 1])]
            else:
                keys = [f"pulse{p}:{'waits' if wb else 'no wait'}" if form != "direct"
                        else f"pulse{p}" for p, wb in zip(pulse_of_item, reached["wait_begin"])]
            groups = {}
            for k in dict.fromkeys(keys):
                sel = np.array([kk == k for kk in keys])
                g = {"units": int(sel.sum())}
                for fld in STAGE_FIELDS:
                    m = sel & reached[fld]
                    if m.any():
                        g[fld] = (float(np.median(rel[fld][m])), float(rel[fld][m].max()))
                groups[k] = g
            per_rep.append({"span_us": float(rel["end"][reached["end"]].max()),
                            "groups": groups,
                            "xcc_round_robin": float(np.mean(
                                (st[:, 7] - st[:, 5]) % 8 ==
                                np.bincount((st[:, 7] - st[:, 5]) % 8).argmax()))})
        med = {"us_per_launch_events": float(np.median(ev_us)),
               "span_us": float(np.median([r["span_us"] for r in per_rep])),
               "xcc_round_robin": min(r["xcc_round_robin"] for r in per_rep), "groups": {}}
        for k, g in per_rep[0]["groups"].items():
            mg = {"units": g["units"]}
            for fld in STAGE_FIELDS:
                vals = [r["groups"][k][fld] for r in per_rep if fld in r["groups"].get(k, {})]
                if vals:
                    mg[fld] = [round(float(np.median([v[0] for v in vals])), 3),
                               round(float(np.median([v[1] for v in vals])), 3)]
            med["groups"][k] = mg
        out[f"{d}_{form}"] = med
        log(f"stages {d} {form}: {med['us_per_launch_events']:.2f} us per launch (events), "
            f"first start to last end {med['span_us']:.2f} us, workgroups on XCD "
            f"(index + r) mod 8: {100 * med['xcc_round_robin']:.1f} %")
        for k, g in med["groups"].items():
            cols = "  ".join(f"{fld} {g[fld][0]:6.2f}/{g[fld][1]:6.2f}" for fld in STAGE_FIELDS
                             if fld in g)
            log(f"   {k:22s} n={g['units']:5d}  {cols}")
    for p in plans:
        p.sync()
        p.close()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--loops", type=int, default=7,
                    help="timed loops of --steps steps; ms_per_step is the median loop's")
    ap.add_argument("--kernel-launches", type=int, default=240,
                    help="launches per loop of the per-direction timings (at least --steps)")
    ap.add_argument("--config", type=int, default=5, help="workload 1..5 (default 5: 8x8x8)")
    ap.add_argument("--replicas", type=int, default=0,
                    help="rotated copies of plan/x/f (0: enough to exceed 2x the 256 MB cache)")
    ap.add_argument("--impl", choices=["fused", "indexmap", "transposed", "pulsewise"],
                    default="fused", help="fused = the library's defaults (index-list "
                    "coordinates, transposed forces)")
    ap.add_argument("--no-ablation", action="store_true", help="skip the per-pulse baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time budget of the oracle baseline (split over both directions)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-reps", type=int, default=50)
    ap.add_argument("--no-overlap", action="store_true")
    ap.add_argument("--build-reps", type=int, default=5)
    ap.add_argument("--overlap-reps", type=int, default=50)
    ap.add_argument("--stages", action="store_true",
                    help="only the per-stage clock profile of every fused kernel on --config "
                         "(halo_plan_debug_timing; medians over 5 repetitions of 20 launches)")
    ap.add_argument("--stage-replicas", type=int, default=1,
                    help="copies of plan and buffers the --stages launches rotate over "
                         "(1: data stay in the caches; 0: as many as the timed loops use)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device-to-device 3 times (a plain copy kernel of "
                         "known size, for scaling hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the library exchanges halos between virtual domains on one GPU; the "
              "exchange over several GPUs (peer-mapped stores over xGMI) is not implemented. "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from domain_decomposition_halo_fusedpackx_amd import HaloPlan
    from domain_decomposition_halo_fusedpackx_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy << 18  # float32 elements in MIB MiB
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: 3 x {args.calibrate_copy} MiB")
        del src, dst
    w = W.WORKLOADS[args.config]
    pos = W.workload_positions(w)
    log(f"workload {w.describe()}")
    if args.stages:
        reps = args.stage_replicas
        if reps == 0:
            p0 = HaloPlan(pos, w.box, w.grid, w.cutoff)
            reps = replica_count(p0.total_slots, p0.num_entries)
            p0.close()
        print(json.dumps({"stages": stage_profile(torch, HaloPlan, W, w, pos, 20, 5, reps)}),
              flush=True)
        return

    plan0 = HaloPlan(pos, w.box, w.grid, w.cutoff)
    E = plan0.num_entries
    S = plan0.total_slots
    R = args.replicas or replica_count(S, E)
    log(f"entries={E} slots={S} items={plan0.num_items} replicas={R}")
    plans = [plan0] + [HaloPlan(pos, w.box, w.grid, w.cutoff) for _ in range(R - 1)]
    x_home = torch.from_numpy(plan0.home_filled(pos, 0.0)).cuda()
    base, n_home, n_halo = plan0.domains()
    f_init = torch.from_numpy(W.halo_forces(S, base, n_home, n_halo, w.seed)).cuda()
    xs = [x_home.clone() for _ in range(R)]
    fs = [f_init.clone() for _ in range(R)]
    for p in plans:
        p.upload()
    torch.cuda.synchronize()

    fused = args.impl == "fused"
    suffix = "" if fused else "_" + args.impl
    ex_x = lambda p, x: getattr(p, "exchange_x" + suffix)(x)  # noqa: E731
    ex_f = lambda p, f: getattr(p, "exchange_f" + suffix)(f)  # noqa: E731

    def step(i):
        r = i % R
        ex_x(plans[r], xs[r])
        ex_f(plans[r], fs[r])

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    log(f"timed {args.loops} loops of {args.steps} steps")
    ms_step, step_loops = time_loops(torch, step, args.steps, args.loops)
    # Per-kernel launch durations on the launch stream, same replicas: the
    # median of 5 loops of back-to-back launches of one direction.
    nk = max(args.steps, args.kernel_launches)
    ms_x, x_loops = time_loops(torch, lambda i: ex_x(plans[i % R], xs[i % R]), nk, 5)
    ms_f, f_loops = time_loops(torch, lambda i: ex_f(plans[i % R], fs[i % R]), nk, 5)
    for p in plans:
        p.sync()
    log(f"ms/step={ms_step:.4f} (loops {min(step_loops):.4f}..{max(step_loops):.4f}) "
        f"x={ms_x * 1e3:.2f}us f={ms_f * 1e3:.2f}us")

    gbs_x = E * BYTES_X / (ms_x * 1e-3) / 1e9
    gbs_f = E * BYTES_F / (ms_f * 1e-3) / 1e9
    dom = "f" if ms_f >= ms_x else "x"
    sha = kernel_source_sha()
    # the kernels the default exchanges run (halo_exchange_x / _f choose by size)
    # plans built on the host run the index-list form on XCD-local units
    idx_x, idx_f = "pack_local", "unpack_local"
    x_default = "push_x" if E >= TRANSPOSED_X_MIN_ENTRIES else idx_x
    f_default = ("pull_f" if E >= TRANSPOSED_F_MIN_ENTRIES and
                 plan0.num_pulses <= TRANSPOSED_F_MAX_PULSES else idx_f)
    kernel_of = {("fused", "x"): x_default, ("fused", "f"): f_default,
                 ("indexmap", "x"): idx_x, ("indexmap", "f"): idx_f,
                 ("transposed", "x"): "push_x", ("transposed", "f"): "pull_f",
                 ("pulsewise", "x"): "pack_pulse", ("pulsewise", "f"): "unpack_pulse"}
    kname = kernel_of[(args.impl, dom)]
    achieved = gbs_f if dom == "f" else gbs_x
    traffic = read_traffic(w.name, kname, sha)

    out = {
        "metric": METRIC,
        "value": E / (ms_step * 1e-3),
        "unit": "halo atoms/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.describe(), "grid": "x".join(map(str, w.grid)),
                   "n_atoms": w.n_atoms, "cutoff_nm": w.cutoff, "pulses": plan0.num_pulses,
                   "halo_entries": E, "slots": S, "impl": args.impl, "replicas": R,
                   "step": "halo_exchange_x + halo_exchange_f"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kname, "bytes_per_launch": E * (BYTES_F if dom == "f" else BYTES_X),
                     "us_per_launch": (ms_f if dom == "f" else ms_x) * 1e3,
                     "kernel_source_sha": sha},
        "us_per_exchange": {"x": ms_x * 1e3, "f": ms_f * 1e3},
        "gbs": {"x": gbs_x, "f": gbs_f},
        "spread": {"ms_per_step": spread(step_loops),
                   "us_x": spread([t * 1e3 for t in x_loops]),
                   "us_f": spread([t * 1e3 for t in f_loops]),
                   "method": f"ms_per_step: median of {args.loops} loops of {args.steps} steps "
                             f"after {args.warmup} warm-up steps; us_x, us_f: median of 5 loops "
                             f"of {nk} launches; HIP events on the launch stream"},
    }

    if fused and not args.no_ablation:
        # the other forms of the same two exchanges, same replicas
        forms = {}
        for form in ("indexmap", "indexmap_lds", "items", "transposed", "pulsewise", "staged",
                     "atomic", "direct"):
            log(f"form {form}")
            fx = getattr(HaloPlan, "exchange_x_" + form, None)
            ff = getattr(HaloPlan, "exchange_f_" + form, None)
            for r in range(R):  # first calls (staging buffers, origin maps) untimed
                if fx:
                    fx(plans[r], xs[r])
                if ff:
                    ff(plans[r], fs[r])
            torch.cuda.synchronize()
            ux = (time_loops(torch, lambda i: fx(plans[i % R], xs[i % R]), nk, 3)[0] * 1e3
                  if fx else None)
            uf = (time_loops(torch, lambda i: ff(plans[i % R], fs[i % R]), nk, 3)[0] * 1e3
                  if ff else None)
            launches = {"pulsewise": plan0.num_pulses, "staged": 2 * plan0.num_pulses}
            forms[form] = {"us_x": ux, "us_f": uf, "launches_per_exchange": launches.get(form, 1)}
        for p in plans:
            p.sync()
        out["forms"] = forms
        out["pulsewise"] = dict(forms["pulsewise"],
                                speedup_fused_x=forms["pulsewise"]["us_x"] / (ms_x * 1e3),
                                speedup_fused_f=forms["pulsewise"]["us_f"] / (ms_f * 1e3))
        out["launch_floor_us"] = launch_floor_us(torch, args.steps)
        out["host_us_per_call"] = {
            "x": host_call_us(torch, lambda i: ex_x(plans[i % R], xs[i % R]), nk),
            "f": host_call_us(torch, lambda i: ex_f(plans[i % R], fs[i % R]), nk)}
        log("cold exchanges")
        out["cold"] = {form: cold_exchange_us(torch, plans[0], xs[0], fs[0], f_init, suffix,
                                              args.cold_reps)
                       for form, suffix in (("fused", ""), ("pulsewise", "_pulsewise"))}
        out["cold"]["fused_dirty"] = cold_exchange_us(torch, plans[0], xs[0], fs[0], f_init, "",
                                                      args.cold_reps, clean=False)
        out["cold"]["method"] = (
            f"median of {args.cold_reps} single exchanges between HIP events, each after a 1 GiB "
            f"device write and a 1 GiB read that evict L2 and the 256 MB cache and leave them "
            f"clean (fused_dirty: the write only); the events add the dispatch gap of a lone "
            f"kernel (about 5.6 us)")
        # The secondary input: the same atoms in 0.5 nm cell order (spatially
        # sorted, as MD codes keep them), same replica count.
        log("cell-sorted input")
        spos = W.cell_sorted(pos, w.box)
        splans = [HaloPlan(spos, w.box, w.grid, w.cutoff) for _ in range(R)]
        sx = [torch.from_numpy(splans[0].home_filled(spos, 0.0)).cuda() for _ in range(R)]
        sbase, sh, sm = splans[0].domains()
        sf = [torch.from_numpy(W.halo_forces(S, sbase, sh, sm, w.seed)).cuda() for _ in range(R)]
        for p in splans:
            p.upload()
        out["cell_sorted_input"] = {
            "us_x": time_loops(torch, lambda i: splans[i % R].exchange_x(sx[i % R]), nk, 3)[0] * 1e3,
            "us_f": time_loops(torch, lambda i: splans[i % R].exchange_f(sf[i % R]), nk, 3)[0] * 1e3,
            "order": "atoms renumbered by 0.5 nm cell (z, y, x), same positions"}
        for p in splans:
            p.sync()
        del splans, sx, sf
        # The corner selection: the same atoms, edge and corner zones trimmed
        # to the cutoff sphere; fewer entries, same kernels.
        log("corner selection")
        cplans = [HaloPlan(pos, w.box, w.grid, w.cutoff, selection="corner") for _ in range(R)]
        cS = cplans[0].total_slots
        cx = [torch.from_numpy(cplans[0].home_filled(pos, 0.0)).cuda() for _ in range(R)]
        cbase, ch, cm = cplans[0].domains()
        cf = [torch.from_numpy(W.halo_forces(cS, cbase, ch, cm, w.seed)).cuda() for _ in range(R)]
        for p in cplans:
            p.upload()

        def cstep(i):
            cplans[i % R].exchange_x(cx[i % R])
            cplans[i % R].exchange_f(cf[i % R])
        cms = time_loops(torch, cstep, args.steps, args.loops)[0]
        out["corner_selection"] = {
            "halo_entries": cplans[0].num_entries, "slots": cS,
            "ms_per_step": cms,
            "us_x": time_loops(torch, lambda i: cplans[i % R].exchange_x(cx[i % R]),
                               nk, 3)[0] * 1e3,
            "us_f": time_loops(torch, lambda i: cplans[i % R].exchange_f(cf[i % R]),
                               nk, 3)[0] * 1e3,
            "step_speedup_vs_slab": ms_step / cms}
        for p in cplans:
            p.sync()
        del cplans, cx, cf
        log("plan builds")
        out["plan_build"] = plan_build_ms(torch, HaloPlan, w, pos, args.build_reps)
        if not args.no_overlap:
            log("overlap with local work")
            out["overlap"] = overlap(torch, plans[0], xs[0], fs[0], args.overlap_reps)
        log("graph replays")
        out["graph"] = graph_replays(torch, plans, xs, fs, args.steps)

    torch.cuda.synchronize()
    for p in plans:
        p.close()
    log("plans released")

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(w, pos, args.cpu_seconds)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
