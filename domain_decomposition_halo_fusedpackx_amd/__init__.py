"""Eighth-shell halo exchange over virtual domains on one MI355X (gfx950).

The exchange itself is the HIP library libhalo.so (include/halo.h); this
package holds its build step, a ctypes binding with the same names, and the
seeded synthetic workloads.
"""
from .binding import HaloError, HaloPlan, load_library, STATUS  # noqa: F401
