"""The corner selection on the GPU: plans built on the device equal the
oracle's and the host builder's, and every exchange form on corner plans is
bitwise equal to the oracle (MI355X)."""
import numpy as np
import pytest

from domain_decomposition_halo_fusedpackx_amd import HaloPlan
from domain_decomposition_halo_fusedpackx_amd import workloads as W

from .test_gpu_parity import IMPLS, assert_bitwise, exchange, say, torch  # noqa: F401
from .test_gpu_plan_device import check_same_plan, device_plan
from .test_oracle_pins import TINY
from .test_plan_host import compare_plans, lattice_positions

pytestmark = pytest.mark.gpu

LATTICES = [
    ((4.0, 4.0, 4.0), (2, 2, 2), 1.0, 0.125),
    ((6.0, 6.0, 6.0), (3, 3, 3), 1.25, 0.25),
    ((4.0, 4.0, 8.0), (2, 2, 4), 1.5, 0.25),
]


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_corner_device_plan_equals_oracle_on_workloads(torch, oracle_mod, wid):
    w = W.WORKLOADS[wid]
    check_same_plan(torch, oracle_mod, W.workload_positions(w), w.box, w.grid, w.cutoff,
                    w.name, "corner")


@pytest.mark.parametrize("case", TINY, ids=lambda c: "x".join(map(str, c[1])))
def test_corner_device_plan_equals_oracle_on_tiny_boxes(torch, oracle_mod, case):
    box, grid, rc, n = case
    for seed in (1, 2):
        check_same_plan(torch, oracle_mod, W.positions(box, n, seed), box, grid, rc,
                        "tiny" + "x".join(map(str, grid)), "corner")


@pytest.mark.parametrize("case", LATTICES, ids=lambda c: "x".join(map(str, c[1])))
def test_device_plans_equal_oracle_on_lattices(torch, oracle_mod, case):
    box, grid, rc, step = case
    pos = lattice_positions(box, step)
    for sel in ("slab", "corner"):
        check_same_plan(torch, oracle_mod, pos, box, grid, rc, "lattice", sel)


def _exchanges_match(torch, plan, o, seed, tag):
    x0 = o.home_filled(np.nan)
    want_x = o.exchange_x(x0.copy())
    base, n_home, n_halo = o.domains()
    f0 = W.halo_forces(o.total_slots, base, n_home, n_halo, seed)
    want_f = o.exchange_f(f0.copy())
    for impl in IMPLS:
        say(f"{tag} corner plan, {impl}")
        x = torch.from_numpy(x0.copy()).cuda()
        exchange(plan, impl, "x", x)
        f = torch.from_numpy(f0.copy()).cuda()
        exchange(plan, impl, "f", f)
        torch.cuda.synchronize()
        plan.sync()
        assert_bitwise(x.cpu().numpy(), want_x, f"{tag} {impl} x")
        assert_bitwise(f.cpu().numpy(), want_f, f"{tag} {impl} f")


@pytest.mark.parametrize("built", ["host", "device"])
@pytest.mark.parametrize("wid", [2, 4, 5])
def test_exchanges_on_corner_plans(torch, oracle_mod, wid, built):
    w = W.WORKLOADS[wid]
    pos = W.workload_positions(w)
    if built == "host":
        plan = HaloPlan(pos, w.box, w.grid, w.cutoff, selection="corner")
    else:
        plan = device_plan(torch, pos, w.box, w.grid, w.cutoff, "corner")
    o = oracle_mod.Oracle(pos, w.box, w.grid, w.cutoff, "corner")
    _exchanges_match(torch, plan, o, w.seed, f"{w.name} {built}")


@pytest.mark.parametrize("case", TINY, ids=lambda c: "x".join(map(str, c[1])))
def test_exchanges_on_corner_plans_tiny(torch, oracle_mod, case):
    box, grid, rc, n = case
    pos = W.positions(box, n, 9)
    plan = HaloPlan(pos, box, grid, rc, selection="corner")
    o = oracle_mod.Oracle(pos, box, grid, rc, "corner")
    _exchanges_match(torch, plan, o, 9, "tiny" + "x".join(map(str, grid)))


def test_rebuild_keeps_the_selection(torch, oracle_mod):
    w = W.WORKLOADS[3]
    pos = W.workload_positions(w)
    dp = device_plan(torch, pos, w.box, w.grid, w.cutoff, "corner")
    for seed in (21, 22):
        pos = W.positions(w.box, w.n_atoms, seed)
        say(f"rebuild corner seed {seed}")
        dp.rebuild_on_device(torch.from_numpy(pos).cuda())
        assert dp.selection == "corner"
        o = oracle_mod.Oracle(pos, w.box, w.grid, w.cutoff, "corner")
        compare_plans(dp, o)
    _exchanges_match(torch, dp, o, 22, "rebuilt")
