"""Property-based parity on the GPU (hypothesis): over random systems (the
strategy of tests/test_properties.py) the device-built plan equals the
oracle's, its XCD-local units equal the host build's, and every exchange form
on it is bitwise equal to the oracle."""
import numpy as np
import pytest

pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

from domain_decomposition_halo_fusedpackx_amd import HaloPlan  # noqa: E402
from domain_decomposition_halo_fusedpackx_amd import workloads as W  # noqa: E402

from .test_gpu_parity import IMPLS, assert_bitwise, exchange, say, torch  # noqa: E402,F401
from .test_gpu_plan_device import device_plan  # noqa: E402
from .test_plan_host import compare_plans  # noqa: E402
from .test_properties import systems  # noqa: E402

pytestmark = pytest.mark.gpu


@settings(max_examples=25, deadline=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])
@given(systems(), st.sampled_from(["slab", "corner"]))
def test_random_systems_on_the_gpu(torch, oracle_mod, system, selection):
    pos, box, grid, rc = system
    if oracle_mod.try_build(pos, box, grid, rc, selection) != 0:
        return
    say(f"random system: {len(pos)} atoms, box {box}, grid {grid}, cutoff {rc}, {selection}")
    o = oracle_mod.Oracle(pos, box, grid, rc, selection)
    dp = device_plan(torch, pos, box, grid, rc, selection)
    compare_plans(dp, o)
    hp = HaloPlan(pos, box, grid, rc, selection=selection)
    np.testing.assert_array_equal(dp.local_units(), hp.local_units())
    if o.total_slots == 0:
        return
    x0 = o.home_filled(np.nan)
    want_x = o.exchange_x(x0.copy())
    base, n_home, n_halo = o.domains()
    f0 = W.halo_forces(o.total_slots, base, n_home, n_halo, 3)
    want_f = o.exchange_f(f0.copy())
    for impl in IMPLS:
        x = torch.from_numpy(x0.copy()).cuda()
        exchange(dp, impl, "x", x)
        f = torch.from_numpy(f0.copy()).cuda()
        exchange(dp, impl, "f", f)
        torch.cuda.synchronize()
        dp.sync()
        assert_bitwise(x.cpu().numpy(), want_x, f"{impl} x")
        assert_bitwise(f.cpu().numpy(), want_f, f"{impl} f")
