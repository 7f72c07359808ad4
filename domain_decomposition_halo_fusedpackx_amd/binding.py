"""ctypes binding of libhalo.so (include/halo.h), same names as the C-ABI.

Argument marshalling only: every step of the exchange runs in the HIP library.
PyTorch supplies device memory (torch.cuda tensors) and streams. If the
library has not been built, every call raises: there is no CPU fallback.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import weakref

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhalo.so")

STATUS = {0: "HALO_OK", -1: "HALO_ERR_ARG", -2: "HALO_ERR_GEOMETRY", -3: "HALO_ERR_RANGE",
          -4: "HALO_ERR_HIP", -5: "HALO_ERR_TIMEOUT", -6: "HALO_ERR_STATE", -7: "HALO_ERR_NOMEM", -8: "HALO_ERR_PLACEMENT"}

# Every symbol include/halo.h declares, with (restype, argtypes).
_vp, _i32, _i64, _u32, _f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                               ctypes.c_float)
_P = ctypes.POINTER
_st = ctypes.c_int
SIGNATURES = {
    "halo_plan_create": (_st, [_vp, _i64, _vp, _vp, _f32, _P(_vp)]),
    "halo_plan_create_ex": (_st, [_vp, _i64, _vp, _vp, _f32, _i32, _P(_vp)]),
    "halo_plan_create_device": (_st, [_vp, _i64, _vp, _vp, _f32, _vp, _P(_vp)]),
    "halo_plan_create_device_ex": (_st, [_vp, _i64, _vp, _vp, _f32, _i32, _vp, _P(_vp)]),
    "halo_plan_rebuild_device": (_st, [_vp, _vp, _i64, _vp, _vp]),
    "halo_plan_destroy": (None, [_vp]),
    "halo_last_error": (ctypes.c_char_p, []),
    "halo_plan_total_slots": (_i64, [_vp]),
    "halo_plan_num_domains": (_i32, [_vp]),
    "halo_plan_num_pulses": (_i32, [_vp]),
    "halo_plan_num_entries": (_i64, [_vp]),
    "halo_plan_num_items": (_i32, [_vp]),
    "halo_plan_selection": (_i32, [_vp]),
    "halo_plan_pulse_dim": (_st, [_vp, _i32, _P(_i32), _P(_i32)]),
    "halo_plan_domain": (_st, [_vp, _i32, _P(_i64), _P(_i32), _P(_i32)]),
    "halo_plan_home_slots": (_st, [_vp, _vp]),
    "halo_plan_pulse": (_st, [_vp, _i32, _i32, _P(_i32), _P(_i32), _P(_i32), _P(_i32), _P(_i32),
                              _P(_i32), _P(_i32), _vp, _vp]),
    "halo_plan_item_waits": (_st, [_vp, _i32, _P(_i32), _P(_u32), _P(_u32)]),
    "halo_plan_num_chunks": (_i32, [_vp]),
    "halo_plan_num_local_units": (_i32, [_vp]),
    "halo_plan_local_unit": (_st, [_vp, _i32, _P(_i32), _P(_i32), _P(_i32), _P(_i32), _P(_i32)]),
    "halo_plan_chunk": (_st, [_vp, _i32, _P(_i32), _P(_i32), _P(_i64), _P(_i32), _P(_u32)]),
    "halo_plan_upload": (_st, [_vp]),
    "halo_exchange_x": (_st, [_vp, _vp, _vp]),
    "halo_exchange_f": (_st, [_vp, _vp, _vp]),
    "halo_exchange_x_items": (_st, [_vp, _vp, _vp]),
    "halo_exchange_f_items": (_st, [_vp, _vp, _vp]),
    "halo_exchange_x_indexmap": (_st, [_vp, _vp, _vp]),
    "halo_exchange_f_indexmap": (_st, [_vp, _vp, _vp]),
    "halo_exchange_x_indexmap_lds": (_st, [_vp, _vp, _vp]),
    "halo_exchange_x_transposed": (_st, [_vp, _vp, _vp]),
    "halo_exchange_f_transposed": (_st, [_vp, _vp, _vp]),
    "halo_exchange_x_pulsewise": (_st, [_vp, _vp, _vp]),
    "halo_exchange_f_pulsewise": (_st, [_vp, _vp, _vp]),
    "halo_exchange_f_atomic": (_st, [_vp, _vp, _vp]),
    "halo_exchange_x_staged": (_st, [_vp, _vp, _vp]),
    "halo_exchange_x_direct": (_st, [_vp, _vp, _vp]),
    "halo_scatter_home": (_st, [_vp, _vp, _vp, _vp]),
    "halo_gather_home": (_st, [_vp, _vp, _vp, _vp]),
    "halo_exchange_f_staged": (_st, [_vp, _vp, _vp]),
    "halo_exchange_x_staged_noalloc": (_st, [_vp, _vp, _vp]),
    "halo_plan_sync": (_st, [_vp, _vp]),
    "halo_plan_reset": (_st, [_vp]),
    "halo_plan_set_spin_limit": (_st, [_vp, _u32]),
    "halo_plan_debug_withhold": (_st, [_vp, _i32]),
    "halo_plan_debug_stress": (_st, [_vp, _u32]),
    "halo_plan_debug_timing": (_st, [_vp, _i32]),
    "halo_plan_debug_timing_read": (_st, [_vp, _vp, _i64, _P(_i64), _P(_i32)]),
}

_lib = None
_FUNCS = {}
_TORCH = None
# Plans still open. At interpreter exit they are destroyed by an atexit hook,
# which runs before the process's C-level exit handlers tear down the HIP
# runtime (and any profiler attached to it); a plan left to the garbage
# collector of a finishing interpreter would free its device memory at an
# unspecified point of that teardown.
_LIVE = weakref.WeakSet()


@atexit.register
def _close_live_plans():
    for plan in list(_LIVE):
        plan.close()


def _torch():
    global _TORCH
    if _TORCH is None:
        import torch
        _TORCH = torch
    return _TORCH


class HaloError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def load_library(path: str = LIB_PATH):
    """Load libhalo.so; raise if it is missing (build it with build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the HIP library first "
                           "(python -m domain_decomposition_halo_fusedpackx_amd.build)")
    # PyTorch ships its own HIP runtime under the same soname as the one the
    # library links against; loading torch first makes the library bind to it,
    # so that device pointers and streams from torch are valid for it.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(code: int):
    if code != 0:
        raise HaloError(code, load_library().halo_last_error().decode())


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _stream_handle(stream, device: int = -1):
    """HIP stream handle: the caller's stream object or raw handle, else torch's
    current stream on `device` (the buffer's device)."""
    if stream is None:
        import torch
        if device < 0:
            device = torch.cuda.current_device()
        return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(device))
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


# halo_selection values of include/halo.h
SELECTIONS = {"slab": 0, "corner": 1}


def _selection(name):
    if name not in SELECTIONS:
        raise ValueError(f"selection must be one of {sorted(SELECTIONS)}")
    return SELECTIONS[name]


class HaloPlan:
    """An exchange plan (halo_plan_create_ex) and its two exchanges.
    `selection` is "slab" (the per-dimension test) or "corner" (also the
    Euclidean distance to the receiving domain's box below the cutoff)."""

    def __init__(self, positions, box, grid, cutoff, selection="slab"):
        sel = _selection(selection)
        lib = load_library()
        pos = np.ascontiguousarray(np.asarray(positions, dtype=np.float32).reshape(-1, 3))
        self._box = np.ascontiguousarray(box, dtype=np.float32)
        self._grid = np.ascontiguousarray(grid, dtype=np.int32)
        if self._box.shape != (3,) or self._grid.shape != (3,):
            raise ValueError("box and grid need three entries")
        h = ctypes.c_void_p()
        _check(lib.halo_plan_create_ex(_np_ptr(pos) if pos.size else None, pos.shape[0],
                                       _np_ptr(self._box), _np_ptr(self._grid),
                                       ctypes.c_float(cutoff), sel, ctypes.byref(h)))
        self._finish(h, pos.shape[0])

    @classmethod
    def on_device(cls, positions, box, grid, cutoff, stream=None, selection="slab"):
        """Build the plan on the GPU (halo_plan_create_device_ex) from a
        contiguous float32 torch.cuda tensor of shape (n_atoms, 3)."""
        import torch
        sel = _selection(selection)
        if not isinstance(positions, torch.Tensor) or not positions.is_cuda:
            raise TypeError("positions must be a torch.cuda tensor")
        if positions.dtype != torch.float32 or not positions.is_contiguous():
            raise TypeError("positions must be contiguous float32")
        if positions.numel() % 3:
            raise ValueError("positions must hold 3 floats per atom")
        self = cls.__new__(cls)
        lib = load_library()
        self._box = np.ascontiguousarray(box, dtype=np.float32)
        self._grid = np.ascontiguousarray(grid, dtype=np.int32)
        if self._box.shape != (3,) or self._grid.shape != (3,):
            raise ValueError("box and grid need three entries")
        n = positions.numel() // 3
        h = ctypes.c_void_p()
        _check(lib.halo_plan_create_device_ex(
            ctypes.c_void_p(positions.data_ptr()) if n else None, n, _np_ptr(self._box),
            _np_ptr(self._grid), ctypes.c_float(cutoff), sel,
            _stream_handle(stream, positions.get_device()), ctypes.byref(h)))
        self._finish(h, n)
        return self

    def rebuild_on_device(self, positions, box=None, stream=None):
        """Rebuild this plan on the GPU for new positions (halo_plan_rebuild_device);
        grid, cutoff and selection stay, box may change."""
        import torch
        if not isinstance(positions, torch.Tensor) or not positions.is_cuda:
            raise TypeError("positions must be a torch.cuda tensor")
        if positions.dtype != torch.float32 or not positions.is_contiguous():
            raise TypeError("positions must be contiguous float32")
        if positions.numel() % 3:
            raise ValueError("positions must hold 3 floats per atom")
        if box is not None:
            b = np.ascontiguousarray(box, dtype=np.float32)
            if b.shape != (3,):
                raise ValueError("box needs three entries")
        else:
            b = self._box
        n = positions.numel() // 3
        try:
            _check(load_library().halo_plan_rebuild_device(
                self._h, ctypes.c_void_p(positions.data_ptr()) if n else None, n, _np_ptr(b),
                _stream_handle(stream, positions.get_device())))
        except HaloError as e:
            if e.code not in (-1, -2):  # the plan is now empty
                self.n_atoms = self.total_slots = self.num_entries = self.num_items = 0
            raise
        self._box = b
        self._finish(self._h, n)

    def _finish(self, h, n_atoms):
        lib = load_library()
        self._h = h
        self._destroy = lib.halo_plan_destroy
        _LIVE.add(self)
        self.n_atoms = n_atoms
        self.total_slots = lib.halo_plan_total_slots(h)
        self.num_domains = lib.halo_plan_num_domains(h)
        self.num_pulses = lib.halo_plan_num_pulses(h)
        self.num_entries = lib.halo_plan_num_entries(h)
        self.num_items = lib.halo_plan_num_items(h)
        self.selection = {v: k for k, v in SELECTIONS.items()}[lib.halo_plan_selection(h)]

    def close(self):
        """Destroy the plan (halo_plan_destroy); exchanges on it must have
        finished. Called by __del__ and, for plans still open at interpreter
        exit, by an atexit hook."""
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._destroy(h)
        self._h = None

    def __del__(self):
        self.close()

    # -- read-out -------------------------------------------------------------
    def pulse_dim(self, p: int):
        d, k = ctypes.c_int32(), ctypes.c_int32()
        _check(load_library().halo_plan_pulse_dim(self._h, p, ctypes.byref(d), ctypes.byref(k)))
        return d.value, k.value

    def domains(self):
        lib = load_library()
        n = self.num_domains
        base = np.zeros(n, np.int64)
        n_home = np.zeros(n, np.int32)
        n_halo = np.zeros(n, np.int32)
        for d in range(n):
            b, h, m = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
            _check(lib.halo_plan_domain(self._h, d, ctypes.byref(b), ctypes.byref(h),
                                        ctypes.byref(m)))
            base[d], n_home[d], n_halo[d] = b.value, h.value, m.value
        return base, n_home, n_halo

    def home_slots(self) -> np.ndarray:
        out = np.zeros(max(self.n_atoms, 1), np.int64)
        _check(load_library().halo_plan_home_slots(self._h, _np_ptr(out)))
        return out[:self.n_atoms]

    def pulse(self, p: int, d: int) -> dict:
        lib = load_library()
        v = [ctypes.c_int32() for _ in range(7)]
        shift = np.zeros(3, np.float32)
        _check(lib.halo_plan_pulse(self._h, p, d, *[ctypes.byref(x) for x in v], _np_ptr(shift),
                                   None))
        im = np.zeros(max(v[1].value, 1), np.int32)
        _check(lib.halo_plan_pulse(self._h, p, d, None, None, None, None, None, None, None, None,
                                   _np_ptr(im)))
        return dict(send_to=v[0].value, send_size=v[1].value, recv_from=v[2].value,
                    recv_size=v[3].value, atom_offset=v[4].value, dep_start=v[5].value,
                    items=v[6].value, shift=shift, index_map=im[:v[1].value].copy())

    def item_waits(self):
        """(segment, xwait_mask, await_mask) of every work item, launch order."""
        lib = load_library()
        out = np.zeros((self.num_items, 3), np.int64)
        sg, xm, am = ctypes.c_int32(), ctypes.c_uint32(), ctypes.c_uint32()
        for i in range(self.num_items):
            _check(lib.halo_plan_item_waits(self._h, i, ctypes.byref(sg), ctypes.byref(xm),
                                            ctypes.byref(am)))
            out[i] = (sg.value, xm.value, am.value)
        return out

    def chunks(self):
        """(domain, zone, first, count, mask) of every chunk of the transposed
        form, in its coordinate kernel's launch order."""
        lib = load_library()
        n = lib.halo_plan_num_chunks(self._h)
        out = np.zeros((max(n, 0), 5), np.int64)
        d, z, c, m = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_uint32()
        f = ctypes.c_int64()
        for i in range(n):
            _check(lib.halo_plan_chunk(self._h, i, ctypes.byref(d), ctypes.byref(z),
                                       ctypes.byref(f), ctypes.byref(c), ctypes.byref(m)))
            out[i] = (d.value, z.value, f.value, c.value, m.value)
        return out

    def local_units(self):
        """(segment, origin, entries, x_waits, f_waits) of every XCD-local
        unit position (empty positions: segment and origin -1)."""
        lib = load_library()
        n = lib.halo_plan_num_local_units(self._h)
        out = np.zeros((max(n, 0), 5), np.int64)
        v = [ctypes.c_int32() for _ in range(5)]
        for i in range(n):
            _check(lib.halo_plan_local_unit(self._h, i, *[ctypes.byref(x) for x in v]))
            out[i] = [x.value for x in v]
        return out

    # -- device side ------------------------------------------------------------
    def _buf(self, t):
        """Validate an exchange buffer; returns (pointer, device index)."""
        torch = _torch()
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError("exchange buffers must be torch.cuda tensors")
        if t.dtype is not torch.float32 or not t.is_contiguous():
            raise TypeError("exchange buffers must be contiguous float32")
        if t.numel() != 3 * self.total_slots:
            raise ValueError(f"buffer holds {t.numel()} floats, the plan needs "
                             f"{3 * self.total_slots} (total_slots x 3)")
        ptr = t.data_ptr()
        if ptr & 3:
            raise ValueError("buffer must be 4-byte aligned")
        return ptr, t.get_device()

    def _call(self, name, t, stream):
        # The per-call path stays lean (small exchanges take a few us on the
        # GPU): plain ints for the pointers, the library's function objects
        # looked up once.
        ptr, dev = self._buf(t)
        fn = _FUNCS.get(name)
        if fn is None:
            fn = _FUNCS[name] = getattr(load_library(), name)
        if stream is None:
            s = _torch()._C._cuda_getCurrentRawStream(dev)
        else:
            s = _stream_handle(stream, dev)
        code = fn(self._h, ptr, s)
        if code:
            _check(code)

    def upload(self):
        _check(load_library().halo_plan_upload(self._h))

    def exchange_x(self, x, stream=None):
        self._call("halo_exchange_x", x, stream)

    def exchange_f(self, f, stream=None):
        self._call("halo_exchange_f", f, stream)

    def exchange_x_indexmap(self, x, stream=None):
        self._call("halo_exchange_x_indexmap", x, stream)

    def exchange_f_indexmap(self, f, stream=None):
        self._call("halo_exchange_f_indexmap", f, stream)

    def exchange_x_items(self, x, stream=None):
        self._call("halo_exchange_x_items", x, stream)

    def exchange_f_items(self, f, stream=None):
        self._call("halo_exchange_f_items", f, stream)

    def exchange_x_indexmap_lds(self, x, stream=None):
        self._call("halo_exchange_x_indexmap_lds", x, stream)

    def exchange_x_transposed(self, x, stream=None):
        self._call("halo_exchange_x_transposed", x, stream)

    def exchange_f_transposed(self, f, stream=None):
        self._call("halo_exchange_f_transposed", f, stream)

    def exchange_x_pulsewise(self, x, stream=None):
        self._call("halo_exchange_x_pulsewise", x, stream)

    def exchange_f_pulsewise(self, f, stream=None):
        self._call("halo_exchange_f_pulsewise", f, stream)

    def exchange_f_atomic(self, f, stream=None):
        self._call("halo_exchange_f_atomic", f, stream)

    def exchange_x_staged(self, x, stream=None):
        self._call("halo_exchange_x_staged", x, stream)

    def exchange_f_staged(self, f, stream=None):
        self._call("halo_exchange_f_staged", f, stream)

    def exchange_x_staged_noalloc(self, x, stream=None):
        self._call("halo_exchange_x_staged_noalloc", x, stream)

    def exchange_x_direct(self, x, stream=None):
        self._call("halo_exchange_x_direct", x, stream)

    def _atoms(self, t):
        import torch
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError("per-atom arrays must be torch.cuda tensors")
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError("per-atom arrays must be contiguous float32")
        if t.numel() != 3 * self.n_atoms:
            raise ValueError(f"per-atom array holds {t.numel()} floats, the plan needs "
                             f"{3 * self.n_atoms} (n_atoms x 3)")
        return ctypes.c_void_p(t.data_ptr())

    def scatter_home(self, values, slots, stream=None):
        """slots[home_slot[a]] = values[a] (halo_scatter_home)."""
        v = self._atoms(values)
        ptr, dev = self._buf(slots)
        _check(load_library().halo_scatter_home(self._h, v, ptr, _stream_handle(stream, dev)))

    def gather_home(self, slots, values, stream=None):
        """values[a] = slots[home_slot[a]] (halo_gather_home)."""
        v = self._atoms(values)
        ptr, dev = self._buf(slots)
        _check(load_library().halo_gather_home(self._h, ptr, v, _stream_handle(stream, dev)))

    def sync(self, stream=None):
        _check(load_library().halo_plan_sync(self._h, _stream_handle(stream)))

    def reset(self):
        _check(load_library().halo_plan_reset(self._h))

    def set_spin_limit(self, polls: int):
        _check(load_library().halo_plan_set_spin_limit(self._h, polls))

    def debug_withhold(self, segment: int):
        _check(load_library().halo_plan_debug_withhold(self._h, segment))

    def debug_stress(self, seed: int):
        _check(load_library().halo_plan_debug_stress(self._h, seed))

    def debug_timing(self, enable: bool = True):
        _check(load_library().halo_plan_debug_timing(self._h, 1 if enable else 0))

    def debug_timing_read(self):
        """(stamps, clock_khz): stamps is an int64 array [units, 8] (start,
        first wait begins, last wait ends, first signal, end, workgroup index,
        HW_ID, XCC_ID) as halo_plan_debug_timing_read returns it."""
        lib = load_library()
        n, khz = ctypes.c_int64(), ctypes.c_int32()
        _check(lib.halo_plan_debug_timing_read(self._h, None, 0, ctypes.byref(n),
                                               ctypes.byref(khz)))
        out = np.zeros((max(n.value, 1), 8), np.uint64)
        _check(lib.halo_plan_debug_timing_read(self._h, _np_ptr(out), n.value, None, None))
        return out[:n.value].astype(np.int64), khz.value

    # -- inputs in this layout ----------------------------------------------------
    def home_filled(self, positions, fill=float("nan")) -> np.ndarray:
        """Host array in this plan's slot layout: positions in home slots."""
        x = np.full((self.total_slots, 3), fill, dtype=np.float32)
        x[self.home_slots()] = np.asarray(positions, np.float32).reshape(-1, 3)
        return x
