"""GPU parity: the HIP exchanges against the serial oracle, bit for bit.

Every test calls the library through the C-ABI (ctypes binding) on device
buffers and compares the whole slot array (home and halo slots) with the
oracle run on the same seeded inputs. Coordinates must match bitwise; fp32
forces too, because both sides add in the same reverse-pulse order. Halo slots
start as NaN, so a slot the kernel fails to write cannot pass.
"""
import os
import sys

import numpy as np
import pytest

from domain_decomposition_halo_fusedpackx_amd import HaloError, HaloPlan
from domain_decomposition_halo_fusedpackx_amd import workloads as W

from .test_oracle_pins import TINY

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU visible")
    return t


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def assert_bitwise(got, want, what):
    g, w = bits(got), bits(want)
    bad = np.flatnonzero((g != w).any(axis=1))
    assert bad.size == 0, (f"{what}: {bad.size} slots differ, first {bad[:5].tolist()}: "
                           f"got {got[bad[:3]].tolist()} want {want[bad[:3]].tolist()}")


def setup_case(oracle_mod, pos, box, grid, rc):
    plan = HaloPlan(pos, box, grid, rc)
    o = oracle_mod.Oracle(pos, box, grid, rc)
    assert plan.total_slots == o.total_slots
    for a, b in zip(plan.domains(), o.domains()):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(plan.home_slots(), o.home_slots())
    return plan, o


IMPLS = ["fused", "indexmap", "transposed", "pulsewise", "staged", "direct", "indexmap_lds",
         "items"]


def exchange(plan, impl, direction, buf, stream=None):
    if impl == "transposed" and plan.num_pulses > 8:
        impl = "indexmap"  # the transposed form refuses plans with more than 8 pulses
    if impl == "direct" and direction == "f":
        impl = "fused"  # the direct form exists for coordinates only
    if impl == "indexmap_lds" and (direction == "f" or len(plan.local_units()) == 0):
        impl = "indexmap"  # coordinates only, on the XCD-local units
    name = {"fused": "exchange_{}", "indexmap": "exchange_{}_indexmap",
            "transposed": "exchange_{}_transposed",
            "pulsewise": "exchange_{}_pulsewise",
            "staged": "exchange_{}_staged",
            "direct": "exchange_{}_direct",
            "indexmap_lds": "exchange_{}_indexmap_lds",
            "items": "exchange_{}_items"}[impl].format(direction)
    getattr(plan, name)(buf, stream)


def run_x(torch, plan, x_host, impl, stream=None):
    x = torch.from_numpy(x_host.copy()).cuda()
    exchange(plan, impl, "x", x, stream)
    torch.cuda.synchronize()
    plan.sync(stream)
    return x.cpu().numpy()


def run_f(torch, plan, f_host, impl, stream=None):
    f = torch.from_numpy(f_host.copy()).cuda()
    exchange(plan, impl, "f", f, stream)
    torch.cuda.synchronize()
    plan.sync(stream)
    return f.cpu().numpy()


def check_both(torch, oracle_mod, plan, o, seed, impl, tag):
    x0 = o.home_filled(np.nan)
    want_x = o.exchange_x(x0.copy())
    say(f"{tag} {impl} exchange_x slots={o.total_slots}")
    assert_bitwise(run_x(torch, plan, x0, impl), want_x, f"{tag} {impl} x")
    base, n_home, n_halo = o.domains()
    f0 = W.halo_forces(o.total_slots, base, n_home, n_halo, seed)
    want_f = o.exchange_f(f0.copy())
    say(f"{tag} {impl} exchange_f")
    assert_bitwise(run_f(torch, plan, f0, impl), want_f, f"{tag} {impl} f")


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_parity_workloads(torch, oracle_mod, wid, impl):
    w = W.WORKLOADS[wid]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    check_both(torch, oracle_mod, plan, o, w.seed, impl, w.name)


@pytest.mark.parametrize("case", TINY, ids=lambda c: "x".join(map(str, c[1])))
def test_parity_tiny_boxes(torch, oracle_mod, case):
    box, grid, rc, n = case
    pos = W.positions(box, n, 7)
    plan, o = setup_case(oracle_mod, pos, box, grid, rc)
    for impl in IMPLS:
        check_both(torch, oracle_mod, plan, o, 7, impl, "tiny" + "x".join(map(str, grid)))


@pytest.mark.parametrize("entries", [64, 200, 256, 2048])
@pytest.mark.parametrize("wid", [3, 4])
def test_parity_item_sizes(torch, oracle_mod, monkeypatch, wid, entries):
    """Items smaller and larger than one workgroup pass, ragged tails."""
    monkeypatch.setenv("HALO_ITEM_ENTRIES", str(entries))
    w = W.WORKLOADS[wid]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    for impl in ("indexmap", "transposed"):
        check_both(torch, oracle_mod, plan, o, w.seed, impl, f"{w.name} items={entries}")


def test_edge_cases(torch, oracle_mod):
    cases = [
        ("empty", np.zeros((0, 3), np.float32), (4.0, 4.0, 4.0), (2, 2, 2), 1.0),
        ("one-domain", W.positions((2.0, 2.0, 2.0), 50, 3), (2.0, 2.0, 2.0), (1, 1, 1), 0.9),
        ("all-in-one-domain", W.positions((1.0, 1.0, 1.0), 64, 4) + np.float32(2.5),
         (4.0, 4.0, 4.0), (2, 2, 2), 1.0),
        ("one-atom", np.array([[0.1, 0.1, 0.1]], np.float32), (4.0, 4.0, 4.0), (2, 2, 2), 1.0),
        # -0 and the largest float below L in every coordinate, and atoms on faces
        ("signed-zero-and-top", np.array(
            [[-0.0, -0.0, -0.0], [np.nextafter(np.float32(4), np.float32(0))] * 3,
             [2.0, -0.0, 2.0], [0.5, 3.5, -0.0]], np.float32), (4.0, 4.0, 4.0), (2, 2, 2), 1.0),
    ]
    for name, pos, box, grid, rc in cases:
        plan, o = setup_case(oracle_mod, pos, box, grid, rc)
        if o.total_slots == 0:
            say(f"{name}: zero slots, exchanges are no-ops")
            x = torch.zeros((0, 3), device="cuda")
            for impl in IMPLS:
                exchange(plan, impl, "x", x)
                exchange(plan, impl, "f", x)
            torch.cuda.synchronize()
            plan.sync()
            continue
        for impl in IMPLS:
            check_both(torch, oracle_mod, plan, o, 9, impl, name)


@pytest.mark.parametrize("wid", [2, 4])
def test_repeats_are_deterministic(torch, oracle_mod, wid):
    """Many exchanges in a row (epochs advance, counters never reset)."""
    w = W.WORKLOADS[wid]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    x0 = o.home_filled(np.nan)
    want_x = o.exchange_x(x0.copy())
    base, n_home, n_halo = o.domains()
    f0 = W.halo_forces(o.total_slots, base, n_home, n_halo, w.seed)
    want_f = o.exchange_f(f0.copy())
    x = torch.from_numpy(x0).cuda()
    f_init = torch.from_numpy(f0).cuda()
    f = torch.empty_like(f_init)
    say(f"{w.name}: 30 rounds, every implementation interleaved")
    for r in range(30):
        for impl in IMPLS:
            exchange(plan, impl, "x", x)
            f.copy_(f_init)
            exchange(plan, impl, "f", f)
            if r % 10 == 9:
                torch.cuda.synchronize()
                assert_bitwise(x.cpu().numpy(), want_x, f"repeat {r} {impl} x")
                assert_bitwise(f.cpu().numpy(), want_f, f"repeat {r} {impl} f")
    torch.cuda.synchronize()
    plan.sync()
    assert_bitwise(f.cpu().numpy(), want_f, "final f")


def test_side_stream(torch, oracle_mod):
    w = W.WORKLOADS[2]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    s = torch.cuda.Stream()
    x0 = o.home_filled(np.nan)
    want = o.exchange_x(x0.copy())
    say("exchange on a side stream")
    with torch.cuda.stream(s):
        x = torch.from_numpy(x0).cuda()
        plan.exchange_x(x)          # current stream = s
        plan.exchange_x(x, s)       # explicit stream
    s.synchronize()
    plan.sync(s)
    assert_bitwise(x.cpu().numpy(), want, "side stream x")


def test_independent_plans_on_concurrent_streams(torch, oracle_mod):
    """Plans share no state: four plans (two workloads, two selections)
    exchange on four streams at once, several times, and stay exact."""
    cases = []
    for wid, sel in ((3, "slab"), (3, "corner"), (4, "slab"), (5, "corner")):
        w = W.WORKLOADS[wid]
        pos = W.workload_positions(w)
        plan = HaloPlan(pos, w.box, w.grid, w.cutoff, selection=sel)
        o = oracle_mod.Oracle(pos, w.box, w.grid, w.cutoff, sel)
        x0 = o.home_filled(np.nan)
        base, n_home, n_halo = o.domains()
        f0 = W.halo_forces(o.total_slots, base, n_home, n_halo, wid)
        plan.upload()
        cases.append((plan, torch.cuda.Stream(), x0, o.exchange_x(x0.copy()), f0,
                      o.exchange_f(f0.copy())))
    torch.cuda.synchronize()
    say("four plans on four streams")
    for r in range(3):
        bufs = []
        for plan, s, x0, _, f0, _ in cases:
            with torch.cuda.stream(s):
                x = torch.from_numpy(x0.copy()).cuda()
                f = torch.from_numpy(f0.copy()).cuda()
                plan.exchange_x(x, s)
                plan.exchange_f(f, s)
            bufs.append((x, f))
        torch.cuda.synchronize()
        for (plan, s, _, want_x, _, want_f), (x, f) in zip(cases, bufs):
            plan.sync(s)
            assert_bitwise(x.cpu().numpy(), want_x, f"round {r} x")
            assert_bitwise(f.cpu().numpy(), want_f, f"round {r} f")


@pytest.mark.parametrize("impl", ["indexmap", "transposed", "items"])
def test_forced_timeout_poisons_and_reset_recovers(torch, oracle_mod, impl):
    """A withheld completion signal makes its dependents hit a tiny spin limit.

    Every wait still ends (the limit is small), the kernel drains, the error
    word surfaces as HALO_ERR_TIMEOUT, the plan refuses work until reset, and
    after the reset results are exact again.
    """
    w = W.WORKLOADS[2]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    x0 = o.home_filled(np.nan)
    want = o.exchange_x(x0.copy())
    x = torch.from_numpy(x0).cuda()
    plan.set_spin_limit(2000)
    plan.debug_withhold(0)  # z0 of domain 0: the forwarding of domain 4's z0 region waits on it
    say(f"forced timeout, coordinate direction, {impl}")
    exchange(plan, impl, "x", x)
    torch.cuda.synchronize()
    with pytest.raises(HaloError) as e:
        plan.sync()
    assert e.value.code == -5
    with pytest.raises(HaloError) as e:
        exchange(plan, impl, "x", x)
    assert e.value.code == -6
    plan.debug_withhold(-1)
    plan.reset()
    plan.set_spin_limit(1 << 20)
    say("after reset")
    x.copy_(torch.from_numpy(x0))
    exchange(plan, impl, "x", x)
    torch.cuda.synchronize()
    plan.sync()
    assert_bitwise(x.cpu().numpy(), want, "x after reset")

    # force direction: withhold pulse y0 of domain 0 (the force sums of its
    # y0 region, or its y0 completion, are waited on by z0)
    base, n_home, n_halo = o.domains()
    f0 = W.halo_forces(o.total_slots, base, n_home, n_halo, 1)
    want_f = o.exchange_f(f0.copy())
    f = torch.from_numpy(f0).cuda()
    plan.set_spin_limit(2000)
    plan.debug_withhold((plan.num_pulses - 2) * plan.num_domains)
    say(f"forced timeout, force direction, {impl}")
    exchange(plan, impl, "f", f)
    torch.cuda.synchronize()
    with pytest.raises(HaloError) as e:
        plan.sync()
    assert e.value.code == -5
    plan.debug_withhold(-1)
    plan.reset()
    plan.set_spin_limit(1 << 20)
    f.copy_(torch.from_numpy(f0))
    exchange(plan, impl, "f", f)
    torch.cuda.synchronize()
    plan.sync()
    assert_bitwise(f.cpu().numpy(), want_f, "f after reset")


@pytest.mark.parametrize("wid", [3, 5])
def test_parity_cell_sorted_input(torch, oracle_mod, wid):
    """The secondary input: the same atoms numbered in 0.5 nm cell order."""
    w = W.WORKLOADS[wid]
    pos = W.cell_sorted(W.workload_positions(w), w.box)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    for impl in ("fused", "transposed"):
        check_both(torch, oracle_mod, plan, o, w.seed, impl, f"{w.name} cell-sorted")


def _capture(torch, fn, stream):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        g.capture_begin()
        try:
            fn()
        finally:
            g.capture_end()
    torch.cuda.synchronize()
    return g


def test_capture_before_upload_is_refused(torch, oracle_mod):
    """The first exchange on a plan uploads it (allocations and a device
    synchronisation): under capture it is refused with HALO_ERR_ARG."""
    w = W.WORKLOADS[2]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    x = torch.from_numpy(o.home_filled(np.nan)).cuda()
    dummy = torch.zeros(4, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    say("capture before upload")

    def body():
        with pytest.raises(HaloError) as e:
            plan.exchange_x(x, s)
        assert e.value.code == -1 and "capture" in str(e.value)
        dummy.add_(1.0)
    _capture(torch, body, s)
    plan.upload()


@pytest.mark.parametrize("form", ["fused", "indexmap", "transposed", "pulsewise", "items"])
@pytest.mark.parametrize("wid", [1, 2, 4, 5])
def test_graph_replays_of_every_form(torch, oracle_mod, wid, form):
    """Both exchanges captured in one HIP graph, replayed three times, with
    eager exchanges of the same plan between the replays: every replay and
    every eager call is bitwise equal to the oracle (the fused kernels infer
    their epoch on the device, so replays and eager calls share the counts)."""
    w = W.WORKLOADS[wid]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    plan.upload()
    x0 = o.home_filled(np.nan)
    want_x = o.exchange_x(x0.copy())
    base, n_home, n_halo = o.domains()
    f0 = W.halo_forces(o.total_slots, base, n_home, n_halo, w.seed)
    want_f = o.exchange_f(f0.copy())
    x0d, f0d = torch.from_numpy(x0).cuda(), torch.from_numpy(f0).cuda()
    x, f = x0d.clone(), f0d.clone()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    say(f"{w.name} {form}: capture X and F")
    g = _capture(torch, lambda: (exchange(plan, form, "x", x, s), exchange(plan, form, "f", f, s)),
                 s)
    for r in range(3):
        x.copy_(x0d)
        f.copy_(f0d)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise(x.cpu().numpy(), want_x, f"{form} replay {r} x")
        assert_bitwise(f.cpu().numpy(), want_f, f"{form} replay {r} f")
        x.copy_(x0d)
        f.copy_(f0d)
        exchange(plan, form, "x", x)
        exchange(plan, form, "f", f)
        torch.cuda.synchronize()
        assert_bitwise(x.cpu().numpy(), want_x, f"{form} eager {r} x")
        assert_bitwise(f.cpu().numpy(), want_f, f"{form} eager {r} f")
    plan.sync()


def test_graph_replays_after_reset(torch, oracle_mod):
    """halo_plan_reset zeroes the counts and the host's epochs: a graph captured
    before it replays exactly afterwards, and so do eager calls."""
    w = W.WORKLOADS[3]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    plan.upload()
    x0 = o.home_filled(np.nan)
    want_x = o.exchange_x(x0.copy())
    base, n_home, n_halo = o.domains()
    f0 = W.halo_forces(o.total_slots, base, n_home, n_halo, w.seed)
    want_f = o.exchange_f(f0.copy())
    x0d, f0d = torch.from_numpy(x0).cuda(), torch.from_numpy(f0).cuda()
    x, f = x0d.clone(), f0d.clone()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = _capture(torch, lambda: (plan.exchange_x(x, s), plan.exchange_f(f, s)), s)
    for r, mode in enumerate(["replay", "reset", "replay", "eager", "reset", "eager", "replay"]):
        say(f"graph and reset: {mode}")
        if mode == "reset":
            plan.reset()
            continue
        x.copy_(x0d)
        f.copy_(f0d)
        torch.cuda.synchronize()
        if mode == "replay":
            g.replay()
        else:
            plan.exchange_x(x)
            plan.exchange_f(f)
        torch.cuda.synchronize()
        assert_bitwise(x.cpu().numpy(), want_x, f"{mode} {r} x")
        assert_bitwise(f.cpu().numpy(), want_f, f"{mode} {r} f")
    plan.sync()


def test_graph_replays_share_counts_with_the_atomic_form(torch, oracle_mod):
    """The ordered and the atomic force kernels share their counters: graphs of
    each, replayed alternately and mixed with eager calls, stay exact (small
    integer forces, so that the atomic sums are exact too)."""
    w = W.WORKLOADS[4]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    plan.upload()
    base, n_home, n_halo = o.domains()
    f0 = W.small_int_forces(o.total_slots, base, n_home, n_halo, 5)
    want = o.exchange_f(f0.copy())
    f0d = torch.from_numpy(f0).cuda()
    f = f0d.clone()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    say("atomic and ordered force graphs")
    g_ord = _capture(torch, lambda: plan.exchange_f_indexmap(f, s), s)
    g_atm = _capture(torch, lambda: plan.exchange_f_atomic(f, s), s)
    for r, g in enumerate([g_ord, g_atm, g_atm, g_ord, None, g_atm, None, g_ord]):
        f.copy_(f0d)
        torch.cuda.synchronize()
        if g is None:
            plan.exchange_f_atomic(f) if r % 2 else plan.exchange_f_indexmap(f)
        else:
            g.replay()
        torch.cuda.synchronize()
        assert_bitwise(f.cpu().numpy(), want, f"step {r}")
    plan.sync()


def test_direct_form_capture(torch, oracle_mod):
    """The direct form's first call derives its origin map and refuses a
    capturing stream; afterwards it is one launch that a graph replays
    exactly, with eager work between the replays."""
    w = W.WORKLOADS[4]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    plan.upload()
    x0 = o.home_filled(np.nan)
    want = o.exchange_x(x0.copy())
    x = torch.from_numpy(x0.copy()).cuda()
    dummy = torch.zeros(4, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    say("direct form: first call under capture is refused")
    g0 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g0.capture_begin()
        try:
            with pytest.raises(HaloError) as e:
                plan.exchange_x_direct(x, s)
            assert e.value.code == -1
            dummy.add_(1.0)
        finally:
            g0.capture_end()
    torch.cuda.synchronize()
    plan.exchange_x_direct(x)
    torch.cuda.synchronize()
    assert_bitwise(x.cpu().numpy(), want, "direct, first call")
    say("direct form: captured and replayed")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g.capture_begin()
        try:
            plan.exchange_x_direct(x, s)
            dummy.add_(1.0)
        finally:
            g.capture_end()
    torch.cuda.synchronize()
    for r in range(3):
        x.copy_(torch.from_numpy(x0))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise(x.cpu().numpy(), want, f"direct replay {r}")
        x.copy_(torch.from_numpy(x0))
        plan.exchange_x(x)  # eager fused exchange between the replays
        torch.cuda.synchronize()
        assert_bitwise(x.cpu().numpy(), want, f"eager after direct replay {r}")
    plan.sync()


def test_exchange_beside_a_gemm(torch, oracle_mod):
    """Fused exchanges while a GEMM occupies the GPU from a second stream:
    every in-kernel wait still ends and the results stay exact."""
    w = W.WORKLOADS[5]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    x0 = o.home_filled(np.nan)
    want_x = o.exchange_x(x0.copy())
    base, n_home, n_halo = o.domains()
    f0 = W.halo_forces(o.total_slots, base, n_home, n_halo, w.seed)
    want_f = o.exchange_f(f0.copy())
    a = torch.randn(4096, 4096, device="cuda")
    b = torch.randn(4096, 4096, device="cuda")
    loc = torch.cuda.Stream()
    x = torch.from_numpy(x0).cuda()
    f_init = torch.from_numpy(f0).cuda()
    f = torch.empty_like(f_init)
    say("exchanges beside a GEMM on another stream")
    for r in range(5):
        with torch.cuda.stream(loc):
            c = a @ b
        f.copy_(f_init)
        plan.exchange_x(x)
        plan.exchange_f(f)
        torch.cuda.synchronize()
        assert_bitwise(x.cpu().numpy(), want_x, f"round {r} x")
        assert_bitwise(f.cpu().numpy(), want_f, f"round {r} f")
    del c
    plan.sync()


@pytest.mark.parametrize("built", ["host", "device"])
def test_scatter_and_gather_home(torch, oracle_mod, built):
    """halo_scatter_home fills exactly the home slots from the atom order;
    after the exchanges, halo_gather_home returns every atom's force."""
    w = W.WORKLOADS[3]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    if built == "device":
        from .test_gpu_plan_device import device_plan
        plan = device_plan(torch, pos, w.box, w.grid, w.cutoff)
    say(f"scatter/gather home ({built} plan)")
    x = torch.full((plan.total_slots, 3), float("nan"), device="cuda")
    plan.scatter_home(torch.from_numpy(pos).cuda(), x)
    plan.exchange_x(x)
    base, n_home, n_halo = o.domains()
    f0 = W.halo_forces(o.total_slots, base, n_home, n_halo, 4)
    f = torch.from_numpy(f0.copy()).cuda()
    plan.exchange_f(f)
    out = torch.empty(len(pos), 3, device="cuda")
    plan.gather_home(f, out)
    torch.cuda.synchronize()
    plan.sync()
    assert_bitwise(x.cpu().numpy(), o.exchange_x(o.home_filled(np.nan)), "x after scatter")
    want_f = o.exchange_f(f0.copy())
    assert_bitwise(out.cpu().numpy(), want_f[o.home_slots()], "gathered forces")
    with pytest.raises(ValueError):
        plan.scatter_home(torch.zeros(3, device="cuda"), x)
