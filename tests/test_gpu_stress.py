"""Race stress: the fused kernels with every group of mutually independent
work units run in reversed order and pseudo-random delays in every unit
(halo_plan_debug_stress). A missing wait or a missing ordering of a store
before its signal shows up as a changed result; the results must stay bitwise
equal to the oracle's (integer-exact for the atomic form)."""
import numpy as np
import pytest

from domain_decomposition_halo_fusedpackx_amd import workloads as W

from .test_gpu_parity import assert_bitwise, exchange, say, setup_case, torch  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wid", [2, 3, 4, 5])
def test_stress_fused_forms(torch, oracle_mod, wid):
    w = W.WORKLOADS[wid]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    x0 = o.home_filled(np.nan)
    want_x = o.exchange_x(x0.copy())
    base, n_home, n_halo = o.domains()
    f0 = W.halo_forces(o.total_slots, base, n_home, n_halo, w.seed)
    want_f = o.exchange_f(f0.copy())
    fi = W.small_int_forces(o.total_slots, base, n_home, n_halo, w.seed)
    want_fi = o.exchange_f(fi.copy())
    for seed in (1, 2, 3):
        plan.debug_stress(seed)
        for impl in ("indexmap", "transposed", "items"):
            say(f"{w.name} stress seed {seed} {impl}")
            x = torch.from_numpy(x0.copy()).cuda()
            exchange(plan, impl, "x", x)
            f = torch.from_numpy(f0.copy()).cuda()
            exchange(plan, impl, "f", f)
            torch.cuda.synchronize()
            plan.sync()
            assert_bitwise(x.cpu().numpy(), want_x, f"stress {seed} {impl} x")
            assert_bitwise(f.cpu().numpy(), want_f, f"stress {seed} {impl} f")
        say(f"{w.name} stress seed {seed} atomic")
        f = torch.from_numpy(fi.copy()).cuda()
        plan.exchange_f_atomic(f)
        torch.cuda.synchronize()
        plan.sync()
        assert_bitwise(f.cpu().numpy(), want_fi, f"stress {seed} atomic f")
    plan.debug_stress(0)
    x = torch.from_numpy(x0.copy()).cuda()
    plan.exchange_x(x)
    torch.cuda.synchronize()
    plan.sync()
    assert_bitwise(x.cpu().numpy(), want_x, "after stress off")


@pytest.mark.parametrize("wid", [3, 4])
def test_stress_in_graph_replays(torch, oracle_mod, wid):
    """The same stress with the epoch inferred on the device: exchanges
    captured in a graph (with the stress orders and delays) and replayed,
    mixed with eager calls; every result stays bitwise equal."""
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
    plan.debug_stress(7)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    graphs = {}
    for impl in ("indexmap", "transposed", "items"):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            g.capture_begin()
            try:
                exchange(plan, impl, "x", x, s)
                exchange(plan, impl, "f", f, s)
            finally:
                g.capture_end()
        torch.cuda.synchronize()
        graphs[impl] = g
    for r, impl in enumerate(["indexmap", "transposed", "transposed", "indexmap"]):
        say(f"{w.name} stressed replay {r} {impl}")
        x.copy_(x0d)
        f.copy_(f0d)
        torch.cuda.synchronize()
        graphs[impl].replay()
        torch.cuda.synchronize()
        plan.sync()
        assert_bitwise(x.cpu().numpy(), want_x, f"stressed replay {r} {impl} x")
        assert_bitwise(f.cpu().numpy(), want_f, f"stressed replay {r} {impl} f")
        x.copy_(x0d)
        f.copy_(f0d)
        exchange(plan, impl, "x", x)
        exchange(plan, impl, "f", f)
        torch.cuda.synchronize()
        plan.sync()
        assert_bitwise(x.cpu().numpy(), want_x, f"stressed eager {r} {impl} x")
        assert_bitwise(f.cpu().numpy(), want_f, f"stressed eager {r} {impl} f")
    plan.debug_stress(0)


def test_rebuild_ends_stress_mode(torch, oracle_mod):
    """A rebuild changes the number of work units; the stress orders of the
    old plan are dropped with it, and the rebuilt plan's exchanges are exact."""
    from .test_gpu_plan_device import device_plan
    w = W.WORKLOADS[3]
    dp = device_plan(torch, W.positions(w.box, 200_000, 41), w.box, w.grid, w.cutoff)
    dp.debug_stress(5)
    pos = W.positions(w.box, 420_000, 42)  # more atoms: more items and chunks
    say("rebuild with stress set")
    dp.rebuild_on_device(torch.from_numpy(pos).cuda())
    o = oracle_mod.Oracle(pos, w.box, w.grid, w.cutoff)
    x0 = o.home_filled(np.nan)
    base, n_home, n_halo = o.domains()
    f0 = W.halo_forces(o.total_slots, base, n_home, n_halo, 42)
    for impl in ("indexmap", "transposed", "items"):
        x = torch.from_numpy(x0.copy()).cuda()
        exchange(dp, impl, "x", x)
        f = torch.from_numpy(f0.copy()).cuda()
        exchange(dp, impl, "f", f)
        torch.cuda.synchronize()
        dp.sync()
        assert_bitwise(x.cpu().numpy(), o.exchange_x(x0.copy()), f"{impl} x")
        assert_bitwise(f.cpu().numpy(), o.exchange_f(f0.copy()), f"{impl} f")
