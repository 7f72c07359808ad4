"""Seeded synthetic inputs for the halo exchange.

This module only draws random numbers: positions for a box and forces for a
slot layout. It holds none of the exchange's arithmetic, and both the HIP path
and the CPU oracle take their inputs from it.

The five workloads stand in for the water-ethanol systems measured on the
"Redesigning GROMACS Halo Exchange" review (s.6, benchmark systems): a uniform
atom density of 100 atoms/nm^3 (about that of water), periodic rectangular
boxes, domain grids from 1x1x2 to 8x8x8.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

DENSITY = 100.0  # atoms per nm^3


@dataclass(frozen=True)
class Workload:
    name: str
    box: tuple  # (Lx, Ly, Lz) in nm
    grid: tuple  # (nx, ny, nz)
    n_atoms: int
    cutoff: float  # nm
    seed: int

    def describe(self) -> str:
        g = "x".join(str(v) for v in self.grid)
        b = "x".join(f"{v:g}" for v in self.box)
        return (f"{g} virtual domains, periodic {b} nm box, {self.n_atoms:,} atoms, "
                f"cutoff {self.cutoff:g} nm")


WORKLOADS = {
    1: Workload("grid1x1x2", (3.0, 3.0, 6.0), (1, 1, 2), 5_400, 1.0, 1),
    2: Workload("grid2x2x2", (6.0, 6.0, 6.0), (2, 2, 2), 21_600, 1.0, 2),
    3: Workload("grid4x4x4", (15.0, 15.0, 15.0), (4, 4, 4), 337_500, 1.2, 3),
    4: Workload("grid4x4x8", (8.0, 8.0, 8.0), (4, 4, 8), 51_200, 1.2, 4),
    5: Workload("grid8x8x8", (22.0, 22.0, 22.0), (8, 8, 8), 1_064_800, 1.2, 5),
}


def positions(box, n_atoms: int, seed: int) -> np.ndarray:
    """Uniform positions in [0, L) as float32 [n_atoms, 3].

    Drawn in float64 from PCG64(seed), scaled by the box and rounded to
    float32; a value that rounds up to L is moved to the largest float32
    below L.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    u = rng.random((n_atoms, 3))
    box32 = np.asarray(box, dtype=np.float32)
    pos = (u * box32.astype(np.float64)).astype(np.float32)
    for d in range(3):
        top = np.nextafter(box32[d], np.float32(0.0))
        col = pos[:, d]
        col[col >= box32[d]] = top
    return np.ascontiguousarray(pos)


def workload_positions(w: Workload) -> np.ndarray:
    return positions(w.box, w.n_atoms, w.seed)


def cell_sorted(pos: np.ndarray, box, cell: float = 0.5) -> np.ndarray:
    """The same atoms renumbered in the order of a grid of `cell`-sized cubes
    (z slowest, then y, then x; stable within a cube), the spatial order in
    which MD codes keep their atoms. Only the numbering changes."""
    n = np.maximum(1, np.floor(np.asarray(box, np.float64) / cell)).astype(np.int64)
    c = np.minimum((pos.astype(np.float64) / cell).astype(np.int64), n - 1)
    key = (c[:, 2] * n[1] + c[:, 1]) * n[0] + c[:, 0]
    return np.ascontiguousarray(pos[np.argsort(key, kind="stable")])


def halo_forces(total_slots: int, bases, n_home, n_halo, seed: int) -> np.ndarray:
    """Forces for a slot layout: N(0,1) float32 on halo slots, 0 on home slots.

    The layout is given as, per domain, its first slot, its home count and its
    halo count. Halo slots are filled in ascending slot order, three
    components each, from PCG64(seed + 1000).
    """
    f = np.zeros((total_slots, 3), dtype=np.float32)
    bases = np.asarray(bases, dtype=np.int64)
    n_home = np.asarray(n_home, dtype=np.int64)
    n_halo = np.asarray(n_halo, dtype=np.int64)
    mask = np.zeros(total_slots, dtype=bool)
    for b, h, m in zip(bases, n_home, n_halo):
        mask[b + h:b + h + m] = True
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    vals = rng.standard_normal(int(mask.sum()) * 3, dtype=np.float32)
    f[mask] = vals.reshape(-1, 3)
    return f


def small_int_forces(total_slots: int, bases, n_home, n_halo, seed: int, lo=-8, hi=8):
    """Small integer forces (as float32) on halo slots, 0 on home slots."""
    f = np.zeros((total_slots, 3), dtype=np.float32)
    rng = np.random.Generator(np.random.PCG64(seed + 2000))
    for b, h, m in zip(bases, n_home, n_halo):
        f[b + h:b + h + m] = rng.integers(lo, hi + 1, size=(m, 3)).astype(np.float32)
    return f
