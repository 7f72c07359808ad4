"""The C-ABI library loads and exports every entry point include/halo.h declares.

No compute call is made here (no GPU): only symbol lookup and the host-only
calls (plan creation, read-out and argument errors).
"""
import ctypes
import os
import re

import numpy as np
import pytest

from domain_decomposition_halo_fusedpackx_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "halo.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(halo_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    for must in ["halo_plan_create", "halo_exchange_x", "halo_exchange_f", "halo_plan_destroy",
                 "halo_last_error", "halo_exchange_x_pulsewise", "halo_exchange_f_pulsewise"]:
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = B.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(B.SIGNATURES) == declared_functions()


def test_library_does_not_link_the_oracle():
    data = open(B.LIB_PATH, "rb").read()
    assert b"oracle_build" not in data and b"oracle_exchange" not in data


def test_create_errors_are_synchronous_and_clean():
    lib = B.load_library()
    box = np.array([2, 2, 2], np.float32)
    grid = np.array([2, 2, 2], np.int32)
    pos = np.full((4, 3), 0.5, np.float32)
    h = ctypes.c_void_p(1)
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert lib.halo_plan_create(P(pos), 4, P(box), P(grid), 0.5, None) == -1
    assert lib.halo_plan_create(None, 4, P(box), P(grid), 0.5, ctypes.byref(h)) == -1
    assert h.value is None
    assert lib.halo_plan_create(P(pos), -1, P(box), P(grid), 0.5, ctypes.byref(h)) == -1
    assert lib.halo_plan_create(P(pos), 4, P(box), P(grid), 1.5, ctypes.byref(h)) == -2
    assert b"pulses" in lib.halo_last_error()
    assert lib.halo_plan_create(P(pos), 4, P(box), P(grid), -1.0, ctypes.byref(h)) == -2
    for bad_sel in (-1, 2):
        assert lib.halo_plan_create_ex(P(pos), 4, P(box), P(grid), 0.5, bad_sel,
                                       ctypes.byref(h)) == -1
        assert b"selection" in lib.halo_last_error()
    assert h.value is None
    assert lib.halo_plan_selection(None) == -1
    pos[2, 0] = 2.0
    assert lib.halo_plan_create(P(pos), 4, P(box), P(grid), 0.5, ctypes.byref(h)) == -3
    assert h.value is None
    # NULL-safe destroy and read-out on NULL
    lib.halo_plan_destroy(None)
    assert lib.halo_plan_total_slots(None) == -1
    assert lib.halo_exchange_x(None, None, None) == -1
    assert lib.halo_exchange_f(None, None, None) == -1
    assert lib.halo_plan_sync(None, None) == -1


def test_binding_rejects_non_device_buffers():
    torch = pytest.importorskip("torch")
    pos = np.full((4, 3), 0.5, np.float32)
    plan = B.HaloPlan(pos, (2.0, 2.0, 2.0), (2, 2, 2), 0.5)
    with pytest.raises(TypeError):
        plan.exchange_x(torch.zeros(plan.total_slots, 3))
    with pytest.raises(TypeError):
        plan.exchange_f(np.zeros((plan.total_slots, 3), np.float32))
