"""The staged coordinate exchange that allocates nothing
(halo_exchange_x_staged_noalloc) against the staged exchange that allocates
its staging buffer (halo_exchange_x_staged), through the C ABI: bitwise equal
(and equal to the oracle) on two calls in a row on one GPU, the second with a
smaller plan; refused before the plan is on the device and for plans larger
than the static staging area."""
import numpy as np
import pytest

from domain_decomposition_halo_fusedpackx_amd import HaloError, HaloPlan
from domain_decomposition_halo_fusedpackx_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU visible")
    return t


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def test_noalloc_matches_staged_on_two_calls(torch, oracle_mod):
    for wid in (5, 3):  # the second call with a smaller plan
        w = W.WORKLOADS[wid]
        say(f"no-alloc staged exchange, workload {wid}")
        pos = W.workload_positions(w)
        plan = HaloPlan(pos, w.box, w.grid, w.cutoff)
        o = oracle_mod.Oracle(pos, w.box, w.grid, w.cutoff)
        x0 = o.home_filled(np.nan)
        want = o.exchange_x(x0.copy())
        x_ref = torch.from_numpy(x0.copy()).cuda()
        plan.exchange_x_staged(x_ref)  # uploads the plan, allocates its own staging buffer
        x = torch.from_numpy(x0.copy()).cuda()
        plan.exchange_x_staged_noalloc(x)
        torch.cuda.synchronize()
        plan.sync()
        got, ref = x.cpu().numpy(), x_ref.cpu().numpy()
        assert np.array_equal(bits(got), bits(ref)), f"workload {wid}: differs from the staged form"
        assert np.array_equal(bits(got), bits(want)), f"workload {wid}: differs from the oracle"
        plan.close()


def test_noalloc_refusals(torch):
    w = W.WORKLOADS[2]
    pos = W.workload_positions(w)
    plan = HaloPlan(pos, w.box, w.grid, w.cutoff)
    x = torch.zeros((plan.total_slots, 3), device="cuda")
    with pytest.raises(HaloError) as e:  # not on the device yet
        plan.exchange_x_staged_noalloc(x)
    assert e.value.code == -6 and "halo_plan_upload" in str(e.value)
    plan.close()
    # more entries than the static area holds (12 bytes each, 32 MiB)
    big = W.WORKLOADS[5]
    bpos = W.workload_positions(big)
    bplan = HaloPlan(bpos, big.box, big.grid, 1.6)
    assert bplan.num_entries * 12 > 32 << 20
    bplan.upload()
    bx = torch.zeros((bplan.total_slots, 3), device="cuda")
    with pytest.raises(HaloError) as e:
        bplan.exchange_x_staged_noalloc(bx)
    assert e.value.code == -1 and "static staging area" in str(e.value)
    bplan.close()
