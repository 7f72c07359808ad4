"""The per-unit clock records of halo_plan_debug_timing (GPU).

With the recording on, every exchange form stays bitwise equal to the oracle,
and the records are consistent: every unit the kernel runs has a start and an
end, its waits lie between them, the workgroup indices of one launch are a
permutation, the XCC_ID is one of the chip's XCDs, and a unit that waits for a
region starts its wait no earlier than its own start. Turning the recording
off frees the buffer and reading then fails with HALO_ERR_ARG.
"""
import numpy as np
import pytest

from domain_decomposition_halo_fusedpackx_amd import HaloError
from domain_decomposition_halo_fusedpackx_amd import workloads as W

from .test_gpu_parity import assert_bitwise, say, setup_case, torch  # noqa: F401

pytestmark = pytest.mark.gpu

FORMS = [("x", "exchange_x_indexmap"), ("x", "exchange_x_transposed"),
         ("x", "exchange_x_direct"), ("x", "exchange_x_items"), ("f", "exchange_f_indexmap"),
         ("f", "exchange_f_transposed"), ("f", "exchange_f_atomic"), ("f", "exchange_f_items")]


@pytest.mark.parametrize("wid", [2, 4])
def test_timing_records_and_results(torch, oracle_mod, wid):
    w = W.WORKLOADS[wid]
    say(f"timing records on workload {wid}")
    pos = W.workload_positions(w)
    plan, o = setup_case(oracle_mod, pos, w.box, w.grid, w.cutoff)
    plan.upload()
    plan.debug_timing(True)
    x0 = o.home_filled(np.nan)
    want_x = o.exchange_x(x0.copy())
    base, n_home, n_halo = o.domains()
    # small integers: the atomic form is then exact as well
    rng = np.random.default_rng(wid)
    f0 = rng.integers(-8, 9, size=(o.total_slots, 3)).astype(np.float32)
    for d in range(o.n_dom):
        f0[base[d]:base[d] + n_home[d]] = 0
    want_f = o.exchange_f(f0.copy())
    n_items, n_chunks = plan.num_items, len(plan.chunks())
    lunits = plan.local_units()
    assert len(lunits) > 0  # a host-built plan runs the index-list form on XCD-local units
    for d, name in FORMS:
        buf = torch.from_numpy((x0 if d == "x" else f0).copy()).cuda()
        getattr(plan, name)(buf)
        torch.cuda.synchronize()
        plan.sync()
        assert_bitwise(buf.cpu().numpy(), want_x if d == "x" else want_f, name)
        st, khz = plan.debug_timing_read()
        assert khz > 0
        n = (n_chunks if "transposed" in name else len(lunits) if "indexmap" in name
             else n_items)
        st = st[:n]
        # the workgroups of a launch go to the XCDs round-robin (starting at
        # whichever XCD is next): workgroup b on XCD (b + r) mod 8 for one r.
        # The XCD-local units rely on workgroups b and b + 8 sharing an XCD.
        assert len(np.unique((st[:, 7] - st[:, 5]) % 8)) == 1, name
        start, wb, we, sig, end = (st[:, k] for k in range(5))
        assert (start > 0).all() and (end >= start).all(), name
        waited = wb != 0
        assert (wb[waited] >= start[waited]).all() and (we[waited] >= wb[waited]).all(), name
        assert (end[waited] >= we[waited]).all(), name
        signalled = sig != 0
        assert (sig[signalled] >= start[signalled]).all(), name
        assert (end[signalled] >= sig[signalled]).all(), name
        assert sorted(st[:, 5].tolist()) == list(range(n)), name
        assert ((st[:, 7] >= 0) & (st[:, 7] < 8)).all(), name
        if name == "exchange_x_indexmap":
            # a unit waits exactly when it reads a region
            np.testing.assert_array_equal(waited, lunits[:, 3] > 0)
        if name == "exchange_f_indexmap":
            np.testing.assert_array_equal(waited, lunits[:, 4] > 0)
        if "indexmap" in name:
            # units of one origin on one XCD
            for og in np.unique(lunits[:, 1][lunits[:, 2] > 0]):
                assert len(np.unique(st[:, 7][lunits[:, 1] == og])) == 1
        if name == "exchange_x_direct":
            assert not waited.any()
    plan.debug_timing(False)
    with pytest.raises(HaloError) as e:
        plan.debug_timing_read()
    assert e.value.code == -1
