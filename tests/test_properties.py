"""Property-based pins (hypothesis, CPU only): over random boxes, grids,
cutoffs and atom sets, including positions on cell faces and cutoffs that are
whole multiples of the domain width,
  - the oracle's halos equal the brute-force set definition, each atom once,
    for both selections;
  - the library's host plan equals the oracle's;
  - with small-integer halo forces the force exchange is the exact integer
    adjoint of the coordinate exchange.
"""
import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, event, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

from oracle import bruteforce as BF  # noqa: E402
from domain_decomposition_halo_fusedpackx_amd import HaloPlan  # noqa: E402

from .test_oracle_pins import _dom_of_slot, _halo_slices  # noqa: E402
from .test_plan_host import compare_plans  # noqa: E402

SETTINGS = settings(max_examples=100, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])


@st.composite
def systems(draw):
    """A box, a grid, a cutoff the grid allows, and atoms. Coordinates are
    either multiples of 1/8 (many on faces and at exact distances) or
    arbitrary floats in [0, L)."""
    grid = tuple(draw(st.integers(1, 4)) for _ in range(3))
    box = tuple(float(draw(st.sampled_from([2.0, 3.0, 4.0, 5.0, 6.0, 8.0]))) for _ in range(3))
    widths = [b / g for b, g in zip(box, grid) if g > 1]
    # at most n_d - 1 pulses per decomposed dimension
    cmax = min([w * (g - 1) for w, g in zip((b / g for b, g in zip(box, grid)), grid) if g > 1],
               default=2.0)
    kind = draw(st.sampled_from(["multiple", "any"]))
    if kind == "multiple" and widths:
        w = draw(st.sampled_from(widths))
        k = draw(st.sampled_from([0.25, 0.5, 1.0, 1.5, 2.0]))
        cutoff = w * k
        if cutoff > cmax:
            cutoff = cmax
    else:
        cutoff = draw(st.floats(0.05, float(cmax), allow_nan=False))
    n = draw(st.integers(0, 120))
    grid_pos = draw(st.booleans())
    rng = np.random.default_rng(draw(st.integers(0, 2**31 - 1)))
    if grid_pos:
        pos = np.stack([rng.integers(0, int(b * 8), n) / 8.0 for b in box], axis=1)
    else:
        pos = rng.random((n, 3)) * np.array(box)
    pos = pos.astype(np.float32)
    for d in range(3):
        top = np.nextafter(np.float32(box[d]), np.float32(0))
        pos[:, d] = np.minimum(pos[:, d], top)
    return pos, box, grid, float(np.float32(cutoff))


def _build(oracle_mod, pos, box, grid, rc, selection):
    if oracle_mod.try_build(pos, box, grid, rc, selection) != 0:
        return None
    return oracle_mod.Oracle(pos, box, grid, rc, selection)


@SETTINGS
@given(systems(), st.sampled_from(["slab", "corner"]))
def test_oracle_halos_are_the_definition(oracle_mod, system, selection):
    pos, box, grid, rc = system
    o = _build(oracle_mod, pos, box, grid, rc, selection)
    if o is None:
        return
    event(f"pulses {o.n_pulse}, halo {'empty' if o.total_slots == len(pos) else 'filled'}")
    gids = o.slot_gids()
    want = BF.halo_sets(pos, box, grid, rc, selection)
    for d, (lo, hi) in enumerate(_halo_slices(o)):
        got = np.sort(gids[lo:hi])
        assert len(np.unique(got)) == len(got)
        np.testing.assert_array_equal(got, want[d])


@SETTINGS
@given(systems(), st.sampled_from(["slab", "corner"]))
def test_host_plan_is_the_oracle_plan(oracle_mod, system, selection):
    pos, box, grid, rc = system
    o = _build(oracle_mod, pos, box, grid, rc, selection)
    if o is None:
        return
    compare_plans(HaloPlan(pos, box, grid, rc, selection=selection), o)


@SETTINGS
@given(systems())
def test_force_exchange_is_the_integer_adjoint(oracle_mod, system):
    pos, box, grid, rc = system
    o = _build(oracle_mod, pos, box, grid, rc, "slab")
    if o is None or o.total_slots == 0:
        return
    gids = o.slot_gids()
    halo = np.ones(o.total_slots, bool)
    halo[o.home_slots()] = False
    rng = np.random.default_rng(o.total_slots)
    f = np.zeros((o.total_slots, 3), np.float32)
    f[halo] = rng.integers(-8, 9, (int(halo.sum()), 3)).astype(np.float32)
    f0 = f.copy()
    o.exchange_f(f)
    want = np.zeros((len(pos), 3))
    np.add.at(want, gids[halo], f0[halo].astype(np.float64))
    np.testing.assert_array_equal(f[o.home_slots()].astype(np.float64), want)
    # and the coordinates land as the closed form says
    x = o.home_filled(np.nan)
    o.exchange_x(x)
    dos = _dom_of_slot(o)
    np.testing.assert_array_equal(
        x[halo].view(np.uint32),
        BF.halo_coords(pos, box, grid, gids[halo], dos[halo]).view(np.uint32))
