"""Python handle on the serial C oracle (halo_oracle.c).

TEST INFRASTRUCTURE: imported only by tests/, the package smoke check and the
CPU-baseline leg of bench.py. It shares no code with the HIP library.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import subprocess
import weakref

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "halo_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

ERR = {0: "ok", -1: "arg", -2: "geometry", -3: "range", -7: "nomem"}


def build(force: bool = False) -> str:
    """Compile halo_oracle.c into liboracle.so (plain gcc, no fast-math)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None
# Oracles still open are freed by an atexit hook, while the module is intact.
_LIVE = weakref.WeakSet()


@atexit.register
def _close_live():
    for o in list(_LIVE):
        o.close()


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        L = _lib
        vp = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        P = ctypes.POINTER
        L.oracle_build.argtypes = [vp, i64, vp, vp, ctypes.c_float, P(vp)]
        L.oracle_build.restype = ctypes.c_int
        L.oracle_build_ex.argtypes = [vp, i64, vp, vp, ctypes.c_float, i32, P(vp)]
        L.oracle_build_ex.restype = ctypes.c_int
        L.oracle_free.argtypes = [vp]
        L.oracle_free.restype = None
        L.oracle_total_slots.argtypes = [vp]
        L.oracle_total_slots.restype = i64
        L.oracle_num_domains.argtypes = [vp]
        L.oracle_num_domains.restype = i32
        L.oracle_num_pulses.argtypes = [vp]
        L.oracle_num_pulses.restype = i32
        L.oracle_geometry.argtypes = [vp, vp, vp, vp]
        L.oracle_geometry.restype = ctypes.c_int
        L.oracle_pulse_dim.argtypes = [vp, i32, P(i32), P(i32)]
        L.oracle_pulse_dim.restype = ctypes.c_int
        L.oracle_domain.argtypes = [vp, i32, P(i64), P(i32), P(i32)]
        L.oracle_domain.restype = ctypes.c_int
        L.oracle_slot_gids.argtypes = [vp, vp]
        L.oracle_slot_gids.restype = ctypes.c_int
        L.oracle_home_slots.argtypes = [vp, vp]
        L.oracle_home_slots.restype = ctypes.c_int
        L.oracle_pulse.argtypes = [vp, i32, i32, P(i32), P(i32), P(i32), P(i32), P(i32), P(i32),
                                   vp, vp]
        L.oracle_pulse.restype = ctypes.c_int
        L.oracle_exchange_x.argtypes = [vp, vp]
        L.oracle_exchange_x.restype = ctypes.c_int
        L.oracle_exchange_f.argtypes = [vp, vp]
        L.oracle_exchange_f.restype = ctypes.c_int
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle error {code} ({ERR.get(code, '?')})")
        self.code = code


class Oracle:
    """The plan and both exchanges, computed serially on the CPU."""

    CRITERIA = {"slab": 0, "corner": 1}

    def __init__(self, pos, box, grid, cutoff, criterion="slab"):
        L = lib()
        pos = np.ascontiguousarray(pos, dtype=np.float32).reshape(-1, 3)
        self.pos = pos
        self.box = np.ascontiguousarray(box, dtype=np.float32)
        self.grid = np.ascontiguousarray(grid, dtype=np.int32)
        self.cutoff = np.float32(cutoff)
        self.criterion = criterion
        h = ctypes.c_void_p()
        rc = L.oracle_build_ex(_ptr(pos) if pos.size else None, pos.shape[0], _ptr(self.box),
                               _ptr(self.grid), ctypes.c_float(self.cutoff),
                               self.CRITERIA[criterion], ctypes.byref(h))
        if rc != 0:
            raise OracleError(rc)
        self._h = h
        self._free = L.oracle_free
        _LIVE.add(self)
        self.n_atoms = pos.shape[0]
        self.total_slots = L.oracle_total_slots(h)
        self.n_dom = L.oracle_num_domains(h)
        self.n_pulse = L.oracle_num_pulses(h)

    def close(self):
        """Free the C oracle (also done by __del__ and at interpreter exit)."""
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._free(h)
        self._h = None

    def __del__(self):
        self.close()

    # -- plan read-out -------------------------------------------------------
    def geometry(self):
        w = np.zeros(3, np.float64)
        u = np.zeros(3, np.float64)
        npd = np.zeros(3, np.int32)
        lib().oracle_geometry(self._h, _ptr(w), _ptr(u), _ptr(npd))
        return w, u, npd

    def pulse_dims(self):
        out = []
        for p in range(self.n_pulse):
            d, k = ctypes.c_int32(), ctypes.c_int32()
            lib().oracle_pulse_dim(self._h, p, ctypes.byref(d), ctypes.byref(k))
            out.append((d.value, k.value))
        return out

    def domains(self):
        base = np.zeros(self.n_dom, np.int64)
        n_home = np.zeros(self.n_dom, np.int32)
        n_halo = np.zeros(self.n_dom, np.int32)
        for d in range(self.n_dom):
            b, h, m = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
            lib().oracle_domain(self._h, d, ctypes.byref(b), ctypes.byref(h), ctypes.byref(m))
            base[d], n_home[d], n_halo[d] = b.value, h.value, m.value
        return base, n_home, n_halo

    def slot_gids(self):
        g = np.zeros(max(self.total_slots, 1), np.int64)
        lib().oracle_slot_gids(self._h, _ptr(g))
        return g[:self.total_slots]

    def home_slots(self):
        s = np.zeros(max(self.n_atoms, 1), np.int64)
        lib().oracle_home_slots(self._h, _ptr(s))
        return s[:self.n_atoms]

    def pulse(self, p: int, d: int) -> dict:
        i32 = ctypes.c_int32
        st, ss, rf, rs, ao, ds = i32(), i32(), i32(), i32(), i32(), i32()
        shift = np.zeros(3, np.float32)
        L = lib()
        rc = L.oracle_pulse(self._h, p, d, ctypes.byref(st), ctypes.byref(ss), ctypes.byref(rf),
                            ctypes.byref(rs), ctypes.byref(ao), ctypes.byref(ds), _ptr(shift), None)
        if rc != 0:
            raise OracleError(rc)
        im = np.zeros(max(ss.value, 1), np.int32)
        L.oracle_pulse(self._h, p, d, None, None, None, None, None, None, None, _ptr(im))
        return dict(send_to=st.value, send_size=ss.value, recv_from=rf.value, recv_size=rs.value,
                    atom_offset=ao.value, dep_start=ds.value, shift=shift,
                    index_map=im[:ss.value].copy())

    # -- inputs in this layout -------------------------------------------------
    def home_filled(self, fill=np.nan) -> np.ndarray:
        """x in the global layout: home slots hold the positions, halo slots `fill`."""
        x = np.full((self.total_slots, 3), fill, dtype=np.float32)
        x[self.home_slots()] = self.pos
        return x

    # -- the exchanges -------------------------------------------------------
    def exchange_x(self, x: np.ndarray) -> np.ndarray:
        assert x.dtype == np.float32 and x.flags.c_contiguous and x.shape == (self.total_slots, 3)
        rc = lib().oracle_exchange_x(self._h, _ptr(x))
        if rc != 0:
            raise OracleError(rc)
        return x

    def exchange_f(self, f: np.ndarray) -> np.ndarray:
        assert f.dtype == np.float32 and f.flags.c_contiguous and f.shape == (self.total_slots, 3)
        rc = lib().oracle_exchange_f(self._h, _ptr(f))
        if rc != 0:
            raise OracleError(rc)
        return f


def try_build(pos, box, grid, cutoff, criterion="slab") -> int:
    """Return the oracle's status code for these inputs (0 when it builds)."""
    try:
        Oracle(pos, box, grid, cutoff, criterion)
    except OracleError as e:
        return e.code
    return 0
