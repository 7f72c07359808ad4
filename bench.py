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
HBM_PEAK_GBS = 8000.0
BYTES_X = 28  # per entry: 4 B index + 12 B gathered source + 12 B store
BYTES_F = 40  # per entry: 4 B index + 12 B region read + 12 B target read + 12 B target write
MALL_BYTES = 256 << 20
KERNEL_SOURCES = ["domain_decomposition_halo_fusedpackx_amd/csrc/halo_api.hip",
                  "domain_decomposition_halo_fusedpackx_amd/csrc/sync.hpp"]


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
    reps, t0 = 0, time.perf_counter()
    while True:
        o.exchange_x(x)
        o.exchange_f(f)
        reps += 1
        el = time.perf_counter() - t0
        if (el >= seconds and reps >= 3) or reps >= 10000:
            break
    return {"value": entries * reps / el, "unit": "halo atoms/s", "cores": 1, "kind": "oracle",
            "sample": f"whole {w.name} workload ({entries} halo entries), {reps} steps of one "
                      f"coordinate + one force exchange, serial C (gcc -O2), 1 thread, "
                      f"{el:.2f} s",
            "host_cpus": os.cpu_count(), "host_cpu": platform.processor() or platform.machine()}


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


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5, help="workload 1..5 (default 5: 8x8x8)")
    ap.add_argument("--replicas", type=int, default=0,
                    help="rotated copies of plan/x/f (0: enough to exceed 2x the 256 MB cache)")
    ap.add_argument("--impl", choices=["fused", "indexmap", "transposed", "pulsewise"],
                    default="fused", help="fused = the library's defaults (index-list "
                    "coordinates, transposed forces)")
    ap.add_argument("--no-ablation", action="store_true", help="skip the per-pulse baseline")
    ap.add_argument("--cpu-seconds", type=float, default=3.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device-to-device 3 times (a plain copy kernel of "
                         "known size, for scaling hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only; the exchange over several GPUs is a "
              "design (peer-mapped stores over xGMI), not built. Use --gpus 1.", file=sys.stderr)
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

    plan0 = HaloPlan(pos, w.box, w.grid, w.cutoff)
    E = plan0.num_entries
    S = plan0.total_slots
    per_rep_bytes = S * 12 + E * 4
    R = args.replicas or max(1, -(-2 * MALL_BYTES // per_rep_bytes))
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

    log(f"timed {args.steps} steps")
    ms_step = time_loop(torch, step, args.steps)
    # Per-kernel launch durations on the launch stream, same replicas.
    ms_x = time_loop(torch, lambda i: ex_x(plans[i % R], xs[i % R]), args.steps)
    ms_f = time_loop(torch, lambda i: ex_f(plans[i % R], fs[i % R]), args.steps)
    for p in plans:
        p.sync()
    log(f"ms/step={ms_step:.4f} x={ms_x * 1e3:.2f}us f={ms_f * 1e3:.2f}us")

    gbs_x = E * BYTES_X / (ms_x * 1e-3) / 1e9
    gbs_f = E * BYTES_F / (ms_f * 1e-3) / 1e9
    dom = "f" if ms_f >= ms_x else "x"
    sha = kernel_source_sha()
    f_default = "pull_f" if E >= (1 << 18) else "unpack_fused"
    kernel_of = {("fused", "x"): "pack_fused", ("fused", "f"): f_default,
                 ("indexmap", "x"): "pack_fused", ("indexmap", "f"): "unpack_fused",
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
    }

    if fused and not args.no_ablation:
        # the other forms of the same two exchanges, same replicas
        forms = {}
        for form in ("indexmap", "transposed", "pulsewise"):
            log(f"form {form}")
            fx = getattr(HaloPlan, "exchange_x_" + form)
            ff = getattr(HaloPlan, "exchange_f_" + form)
            ux = time_loop(torch, lambda i: fx(plans[i % R], xs[i % R]), args.steps) * 1e3
            uf = time_loop(torch, lambda i: ff(plans[i % R], fs[i % R]), args.steps) * 1e3
            forms[form] = {"us_x": ux, "us_f": uf,
                           "launches_per_exchange": plan0.num_pulses if form == "pulsewise" else 1}
        for p in plans:
            p.sync()
        out["forms"] = forms
        out["pulsewise"] = dict(forms["pulsewise"],
                                speedup_fused_x=forms["pulsewise"]["us_x"] / (ms_x * 1e3),
                                speedup_fused_f=forms["pulsewise"]["us_f"] / (ms_f * 1e3))

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(w, pos, args.cpu_seconds)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
