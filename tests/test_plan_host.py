"""The library's host plan builder against the oracle (CPU only).

The plan is host logic; its layout, home slots and every PulseData field
(sendSize, recvSize, atomOffset, coordShift, indexMap, depOffset split) must
equal the oracle's on every workload and on the tiny multi-pulse boxes.
"""
import numpy as np
import pytest

from domain_decomposition_halo_fusedpackx_amd import HaloError, HaloPlan
from domain_decomposition_halo_fusedpackx_amd import workloads as W

from .test_oracle_pins import TINY


def compare_plans(plan, o):
    assert plan.total_slots == o.total_slots
    assert plan.num_domains == o.n_dom
    assert plan.num_pulses == o.n_pulse
    for a, b in zip(plan.domains(), o.domains()):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(plan.home_slots(), o.home_slots())
    entries = 0
    for p in range(o.n_pulse):
        assert plan.pulse_dim(p) == o.pulse_dims()[p]
        for d in range(o.n_dom):
            a, b = plan.pulse(p, d), o.pulse(p, d)
            for key in ("send_to", "send_size", "recv_from", "recv_size", "atom_offset",
                        "dep_start"):
                assert a[key] == b[key], (p, d, key)
            np.testing.assert_array_equal(a["shift"].view(np.uint32), b["shift"].view(np.uint32))
            np.testing.assert_array_equal(a["index_map"], b["index_map"])
            assert a["items"] >= 1
            entries += a["send_size"]
    assert plan.num_entries == entries


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_plan_equals_oracle_on_workloads(oracle_mod, wid):
    w = W.WORKLOADS[wid]
    pos = W.workload_positions(w)
    plan = HaloPlan(pos, w.box, w.grid, w.cutoff)
    o = oracle_mod.Oracle(pos, w.box, w.grid, w.cutoff)
    compare_plans(plan, o)


@pytest.mark.parametrize("case", TINY, ids=lambda c: "x".join(map(str, c[1])))
def test_plan_equals_oracle_on_tiny_boxes(oracle_mod, case):
    box, grid, rc, n = case
    for seed in (1, 2):
        pos = W.positions(box, n, seed)
        compare_plans(HaloPlan(pos, box, grid, rc), oracle_mod.Oracle(pos, box, grid, rc))


def test_plan_edge_cases(oracle_mod):
    # empty system, one domain, all atoms in one domain
    cases = [
        (np.zeros((0, 3), np.float32), (4.0, 4.0, 4.0), (2, 2, 2), 1.0),
        (W.positions((2.0, 2.0, 2.0), 50, 3), (2.0, 2.0, 2.0), (1, 1, 1), 0.9),
        (W.positions((1.0, 1.0, 1.0), 64, 4) + np.float32(2.5), (4.0, 4.0, 4.0), (2, 2, 2), 1.0),
        (np.array([[-0.0, -0.0, -0.0], [np.nextafter(np.float32(4), np.float32(0))] * 3,
                   [2.0, -0.0, 2.0], [0.5, 3.5, -0.0]], np.float32), (4.0, 4.0, 4.0),
         (2, 2, 2), 1.0),
    ]
    for pos, box, grid, rc in cases:
        compare_plans(HaloPlan(pos, box, grid, rc), oracle_mod.Oracle(pos, box, grid, rc))


def lattice_positions(box, step):
    """Atoms on a regular lattice of spacing `step` (exact in float32): many
    sit exactly on cell faces and at distances that tie with the cutoff."""
    axes = [np.arange(0.0, b, step, dtype=np.float64) for b in box]
    g = np.stack(np.meshgrid(*axes, indexing="ij"), axis=-1).reshape(-1, 3)
    return g.astype(np.float32)


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_corner_plan_equals_oracle_on_workloads(oracle_mod, wid):
    w = W.WORKLOADS[wid]
    pos = W.workload_positions(w)
    plan = HaloPlan(pos, w.box, w.grid, w.cutoff, selection="corner")
    assert plan.selection == "corner"
    o = oracle_mod.Oracle(pos, w.box, w.grid, w.cutoff, "corner")
    compare_plans(plan, o)
    if min(w.grid) > 1:
        assert plan.total_slots < HaloPlan(pos, w.box, w.grid, w.cutoff).total_slots


@pytest.mark.parametrize("case", TINY, ids=lambda c: "x".join(map(str, c[1])))
def test_corner_plan_equals_oracle_on_tiny_boxes(oracle_mod, case):
    box, grid, rc, n = case
    for seed in (1, 2):
        pos = W.positions(box, n, seed)
        compare_plans(HaloPlan(pos, box, grid, rc, selection="corner"),
                      oracle_mod.Oracle(pos, box, grid, rc, "corner"))


@pytest.mark.parametrize("box,grid,rc,step", [
    ((4.0, 4.0, 4.0), (2, 2, 2), 1.0, 0.125),
    ((6.0, 6.0, 6.0), (3, 3, 3), 1.25, 0.25),
    ((4.0, 4.0, 8.0), (2, 2, 4), 1.5, 0.25),
])
def test_plans_equal_oracle_on_lattices(oracle_mod, box, grid, rc, step):
    pos = lattice_positions(box, step)
    for sel in ("slab", "corner"):
        compare_plans(HaloPlan(pos, box, grid, rc, selection=sel),
                      oracle_mod.Oracle(pos, box, grid, rc, sel))


def test_selection_is_checked():
    pos = W.positions((2.0, 2.0, 2.0), 10, 1)
    with pytest.raises(ValueError):
        HaloPlan(pos, (2.0, 2.0, 2.0), (2, 2, 2), 0.5, selection="sphere")
    assert HaloPlan(pos, (2.0, 2.0, 2.0), (2, 2, 2), 0.5).selection == "slab"


@pytest.mark.parametrize("args", [
    ((2.0, 2.0, 2.0), (2, 2, 2), 1.5),
    ((2.0, 2.0, 2.0), (1, 1, 1), 0.0),
    ((2.0, 2.0, 2.0), (1, 1, 1), float("nan")),
    ((2.0, 0.0, 2.0), (1, 1, 1), 0.5),
    ((2.0, 2.0, 2.0), (1, 0, 1), 0.5),
])
def test_error_codes_match_oracle(oracle_mod, args):
    pos = W.positions((2.0, 2.0, 2.0), 10, 1)
    want = oracle_mod.try_build(pos, *args)
    with pytest.raises(HaloError) as e:
        HaloPlan(pos, *args)
    assert e.value.code == want


@pytest.mark.parametrize("bad", [np.nan, np.inf, -0.5, 2.0, 7.0])
def test_position_errors_match_oracle(oracle_mod, bad):
    pos = W.positions((2.0, 2.0, 2.0), 10, 1)
    pos[3, 1] = bad
    want = oracle_mod.try_build(pos, (2.0, 2.0, 2.0), (2, 2, 2), 0.5)
    with pytest.raises(HaloError) as e:
        HaloPlan(pos, (2.0, 2.0, 2.0), (2, 2, 2), 0.5)
    assert e.value.code == want == -3


def _unit_bound(n_entries, item_entries=1024):
    """The work-unit size rule: the largest power of two from 128 to 1024 at
    which the plan keeps 512 units' worth of entries, at most item_entries."""
    size = 1024
    while size > 128 and size * 512 > n_entries:
        size //= 2
    return min(size, item_entries)


def test_item_cutting(monkeypatch):
    """Work items cut the independent and the dependent span of every
    (pulse, domain) separately, with at least one item per (pulse, domain),
    into items of at most the plan-sized bound (256 entries on workload 4,
    or less when HALO_ITEM_ENTRIES says so)."""
    w = W.WORKLOADS[4]
    pos = W.workload_positions(w)
    for env, n in ((64, 64), (200, 200), (300, 256), (1024, 256), (2048, 256)):
        monkeypatch.setenv("HALO_ITEM_ENTRIES", str(env))
        plan = HaloPlan(pos, w.box, w.grid, w.cutoff)
        assert _unit_bound(plan.num_entries, env) == n
        tot = 0
        for p in range(plan.num_pulses):
            for d in range(plan.num_domains):
                q = plan.pulse(p, d)
                dep = q["send_size"] - q["dep_start"]
                assert q["items"] == max(1, -(-q["dep_start"] // n) + -(-dep // n))
                tot += q["items"]
        assert tot == plan.num_items


def _region_of(o, p, d, slot):
    for r in range(p):
        q = o.pulse(r, d)
        if q["atom_offset"] <= slot < q["atom_offset"] + q["recv_size"]:
            return r
    return None


@pytest.mark.parametrize("wid", [2, 4])
def test_item_wait_masks(oracle_mod, wid):
    """Every work item's wait masks follow from the oracle's PulseData: the
    regions its dependent entries read, and the later pulses of the receiver
    that add into the region it reads."""
    w = W.WORKLOADS[wid]
    pos = W.workload_positions(w)
    plan = HaloPlan(pos, w.box, w.grid, w.cutoff)
    o = oracle_mod.Oracle(pos, w.box, w.grid, w.cutoff)
    seen = {}
    waits = plan.item_waits()
    for seg, xm, am in waits:
        p, d = divmod(int(seg), plan.num_domains)
        seen.setdefault((p, d), []).append((xm, am))
    for (p, d), lst in seen.items():
        q = o.pulse(p, d)
        dep = q["index_map"][q["dep_start"]:]
        regions = {_region_of(o, p, d, int(s)) for s in dep}
        assert None not in regions
        union = 0
        for xm, _ in lst:
            union |= int(xm)
        assert union == sum(1 << r for r in regions), (p, d)
        r = q["send_to"]
        rr = o.pulse(p, r)
        lo, hi = rr["atom_offset"], rr["atom_offset"] + rr["recv_size"]
        want_am = 0
        for qq in range(p + 1, o.n_pulse):
            m = o.pulse(qq, r)["index_map"]
            if np.any((m >= lo) & (m < hi)):
                want_am |= 1 << qq
        for _, am in lst:
            assert int(am) == want_am, (p, d)


def test_more_than_32_pulses_is_a_geometry_error(oracle_mod):
    """The library caps a plan at 32 pulses (its work items keep per-pulse wait
    sets as 32-bit masks); the oracle has no such cap. A 12x12x12 grid of 1 nm
    domains with a 10.5 nm cutoff needs 11 pulses per dimension, 33 in all:
    the oracle builds it, the library refuses it with HALO_ERR_GEOMETRY and
    says why. With 1.1 nm domains in z (10 pulses there) the plan has 32
    pulses and builds."""
    pos = np.zeros((0, 3), np.float32)
    grid = (12, 12, 12)
    assert oracle_mod.try_build(pos, (12.0, 12.0, 12.0), grid, 10.5) == 0
    with pytest.raises(HaloError) as e:
        HaloPlan(pos, (12.0, 12.0, 12.0), grid, 10.5)
    assert e.value.code == -2
    assert "33 pulses" in str(e.value) and "at most 32" in str(e.value)
    plan = HaloPlan(pos, (12.0, 12.0, 13.2), grid, 10.5)
    assert plan.num_pulses == 32
    o = oracle_mod.Oracle(pos, (12.0, 12.0, 13.2), grid, 10.5)
    assert o.n_pulse == 32


@pytest.mark.parametrize("wid,bound", [(1, 128), (2, 128), (3, 512), (4, 256), (5, 1024)])
def test_local_unit_size_follows_plan_size(wid, bound):
    """The XCD-local units and the work items are cut at the largest power of
    two from 128 to 1024 entries at which the plan keeps 512 units' worth of
    entries: 128 for the two smallest workloads, 512 / 256 / 1024 for
    workloads 3 / 4 / 5. No unit or item exceeds the bound, and on workloads
    3 and 5 some unit is longer than half of it (the bound is not smaller than
    the rule says)."""
    w = W.WORKLOADS[wid]
    pos = W.workload_positions(w)
    plan = HaloPlan(pos, w.box, w.grid, w.cutoff)
    assert _unit_bound(plan.num_entries) == bound
    lu = plan.local_units()
    n = lu[:, 2][lu[:, 2] > 0]
    assert n.sum() == plan.num_entries
    assert n.max() <= bound
    if wid in (3, 5):
        assert n.max() > bound // 2
    for p in range(plan.num_pulses):
        for d in range(plan.num_domains):
            q = plan.pulse(p, d)
            dep = q["send_size"] - q["dep_start"]
            assert q["items"] == max(1, -(-q["dep_start"] // bound) + -(-dep // bound))
