"""The atomic force exchange (the pages' Algorithm 6 with atomicAdd) against
the oracle.

Its adds onto one slot happen in no fixed order, so it is held to two bars:
- small-integer forces: every partial sum is exact in fp32, so the result
  must equal the oracle's bit for bit whatever the order of the adds;
- N(0,1) forces: per slot, |gpu - oracle| <= 2 (n - 1) u S with u = 2^-24,
  n the number of values summed into the slot and S the sum of their
  magnitudes. Any order of n - 1 fp32 additions lies within (n - 1) u S
  (to first order) of the exact sum, and both sides are such orders. n comes
  from the oracle run on all-ones forces (exact small integers), S from the
  oracle run on |f0| (rounded, hence the small margin).
"""
import numpy as np
import pytest

from domain_decomposition_halo_fusedpackx_amd import HaloError
from domain_decomposition_halo_fusedpackx_amd import workloads as W

from .test_gpu_parity import assert_bitwise, say, setup_case, torch  # noqa: F401
from .test_oracle_pins import TINY

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def run_atomic(torch, plan, f_host):
    f = torch.from_numpy(f_host.copy()).cuda()
    plan.exchange_f_atomic(f)
    torch.cuda.synchronize()
    plan.sync()
    return f.cpu().numpy()


def rounding_bound(o, f0):
    n = o.exchange_f(np.ones_like(f0))
    s = o.exchange_f(np.abs(f0))
    return 2.0 * np.maximum(n - 1.0, 0.0) * U * s.astype(np.float64) * 1.001


def check_atomic(torch, o, plan, seed, tag):
    base, n_home, n_halo = o.domains()
    fi = W.small_int_forces(o.total_slots, base, n_home, n_halo, seed)
    say(f"{tag} atomic f, integer forces")
    assert_bitwise(run_atomic(torch, plan, fi), o.exchange_f(fi.copy()), f"{tag} atomic int f")
    f0 = W.halo_forces(o.total_slots, base, n_home, n_halo, seed)
    want = o.exchange_f(f0.copy())
    say(f"{tag} atomic f, N(0,1) forces")
    got = run_atomic(torch, plan, f0)
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bound = rounding_bound(o, f0)
    bad = np.flatnonzero((err > bound).any(axis=1))
    assert bad.size == 0, (f"{tag}: {bad.size} slots beyond the rounding bound, first "
                           f"{bad[:3].tolist()}: err {err[bad[:3]].tolist()} "
                           f"bound {bound[bad[:3]].tolist()}")
    # slots with a single term take no add: exact
    n = o.exchange_f(np.ones_like(f0))
    one = (n == 1.0).all(axis=1)
    assert_bitwise(got[one], want[one], f"{tag} atomic single-term slots")


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_atomic_force_workloads(torch, oracle_mod, wid):
    w = W.WORKLOADS[wid]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    check_atomic(torch, o, plan, w.seed, w.name)


@pytest.mark.parametrize("case", TINY, ids=lambda c: "x".join(map(str, c[1])))
def test_atomic_force_tiny_boxes(torch, oracle_mod, case):
    box, grid, rc, n = case
    pos = W.positions(box, n, 11)
    plan, o = setup_case(oracle_mod, pos, box, grid, rc)
    check_atomic(torch, o, plan, 11, "tiny" + "x".join(map(str, grid)))


def test_atomic_interleaved_with_ordered(torch, oracle_mod):
    """The atomic and the ordered index-list force kernels share counters:
    interleaved calls must keep both exact (integer forces)."""
    w = W.WORKLOADS[4]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    base, n_home, n_halo = o.domains()
    fi = W.small_int_forces(o.total_slots, base, n_home, n_halo, 5)
    want = o.exchange_f(fi.copy())
    f_init = torch.from_numpy(fi).cuda()
    f = torch.empty_like(f_init)
    say("atomic / ordered force exchanges interleaved, 20 rounds")
    for r in range(20):
        for name in ("exchange_f_atomic", "exchange_f_indexmap", "exchange_f"):
            f.copy_(f_init)
            getattr(plan, name)(f)
            if r % 5 == 4:
                torch.cuda.synchronize()
                assert_bitwise(f.cpu().numpy(), want, f"round {r} {name}")
    torch.cuda.synchronize()
    plan.sync()


def test_atomic_forced_timeout(torch, oracle_mod):
    """A withheld completion signal: the waiting items give up after a tiny
    spin limit, the kernel drains, the timeout surfaces, and after a reset the
    result is exact again."""
    w = W.WORKLOADS[2]
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    base, n_home, n_halo = o.domains()
    fi = W.small_int_forces(o.total_slots, base, n_home, n_halo, 3)
    want = o.exchange_f(fi.copy())
    f = torch.from_numpy(fi).cuda()
    plan.set_spin_limit(2000)
    plan.debug_withhold((plan.num_pulses - 2) * plan.num_domains)
    say("forced timeout, atomic force exchange")
    plan.exchange_f_atomic(f)
    torch.cuda.synchronize()
    with pytest.raises(HaloError) as e:
        plan.sync()
    assert e.value.code == -5
    plan.debug_withhold(-1)
    plan.reset()
    plan.set_spin_limit(1 << 20)
    f.copy_(torch.from_numpy(fi))
    plan.exchange_f_atomic(f)
    torch.cuda.synchronize()
    plan.sync()
    assert_bitwise(f.cpu().numpy(), want, "atomic f after reset")
