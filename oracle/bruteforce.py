"""Brute-force checks that pin the serial oracle to the pages' statement of the
problem, computed without its pulse chain.

TEST INFRASTRUCTURE: imported only by tests/. Nothing here is called by the
product path or by the oracle itself.

What is checked, and where the pages state it ("Redesigning GROMACS Halo
Exchange" review, s.3 "GROMACS domain decomposition halo exchange" and s.4
"Core formulas"; "GPU-Initiated Halo Exchange Cuts CPU Bottlenecks in GROMACS",
"The CPU bottleneck in halo exchange"):

* halo membership: a domain needs the atoms that lie within the cutoff of it
  on its eighth-shell (upper) side; the forwarding chain must deliver each such
  atom exactly once (halo_sets);
* halo coordinates: the periodic image of the original position, i.e. the
  position plus +L in every dimension in which the atom's cell index is below
  the receiving domain's (halo_coords);
* reach: with np(d) pulses per dimension, the chain reaches prod(np(d)+1) - 1
  source domains in sum(np(d)) pulses (source_offsets);
* forces: the force exchange is the transpose of the coordinate gather, so a
  home slot ends with the sum of the forces on all images of its atom
  (force_adjoint);
* counts: the expected number of atoms sent per pulse is density x the volume
  of the slab that pulse covers (expected_send_sizes).
"""
from __future__ import annotations

import numpy as np


def geometry(box, grid, cutoff):
    """Domain width w, cutoff in units of w (u) and pulses per dimension."""
    box = np.asarray(box, np.float32).astype(np.float64)
    grid = np.asarray(grid, np.int64)
    w = box / grid
    u = np.float64(np.float32(cutoff)) / w
    npd = np.where(grid > 1, np.ceil(u), 0).astype(np.int64)
    return w, u, npd


def cells(pos, box, grid):
    """Scaled position t = x / w (clamped below n) and cell index floor(t)."""
    w, _, _ = geometry(box, grid, 1.0)
    grid = np.asarray(grid, np.int64)
    t = np.asarray(pos, np.float32).astype(np.float64) / w
    top = np.nextafter(grid.astype(np.float64), 0.0)
    t = np.minimum(t, top)
    c = np.floor(t).astype(np.int64)
    return t, c


def domain_cells(grid):
    nx, ny, nz = grid
    ids = np.arange(nx * ny * nz)
    return np.stack([ids % nx, (ids // nx) % ny, ids // (nx * ny)], axis=1)


def halo_sets(pos, box, grid, cutoff, criterion="slab"):
    """For every domain, the sorted global ids that its halo must hold.

    An atom belongs to the halo of domain D when it is not a home atom of D and,
    in every decomposed dimension d, it lies either in D's own slab of cells or
    within the cutoff above D's upper face: 0 <= (t_d - (c_d(D) + 1)) mod n_d
    < rc / w_d. With criterion "corner" its Euclidean distance to D's box must
    also be below the cutoff: sum_d (delta_d * w_d)^2 < rc^2 over d = x, y, z,
    delta_d = 0 where it lies in D's slab. This is the set definition,
    evaluated atom by atom.
    """
    grid = np.asarray(grid, np.int64)
    w, u, _ = geometry(box, grid, cutoff)
    t, c = cells(pos, box, grid)
    rc2 = float(np.float32(cutoff)) * float(np.float32(cutoff))
    out = []
    for cd in domain_cells(grid):
        ok = np.ones(len(t), dtype=bool)
        home = np.ones(len(t), dtype=bool)
        dist2 = np.zeros(len(t))
        for d in range(3):
            same = c[:, d] == cd[d]
            home &= same
            delta = t[:, d] - float(cd[d] + 1)
            delta = np.where(delta < 0.0, delta + float(grid[d]), delta)
            dist = np.where(same, 0.0, delta) * w[d]
            dist2 = dist2 + dist * dist
            if grid[d] == 1:
                continue
            ok &= same | (delta < u[d])
        if criterion == "corner":
            ok &= dist2 < rc2
        out.append(np.flatnonzero(ok & ~home))
    return out


def halo_coords(pos, box, grid, gids, dom_of_slot):
    """Closed-form halo coordinates: fp32(x + L) where the image wrapped."""
    grid = np.asarray(grid, np.int64)
    box32 = np.asarray(box, np.float32)
    _, c = cells(pos, box, grid)
    cd = domain_cells(grid)[dom_of_slot]
    ca = c[gids]
    shift = np.where(ca < cd, box32[None, :], np.float32(0.0)).astype(np.float32)
    return (np.asarray(pos, np.float32)[gids] + shift).astype(np.float32)


def source_offsets(pos, box, grid, gids_of_halo, dom):
    """Distinct cell offsets (mod n) from domain `dom` to its halo atoms' homes."""
    grid = np.asarray(grid, np.int64)
    _, c = cells(pos, box, grid)
    cd = domain_cells(grid)[dom]
    off = (c[gids_of_halo] - cd[None, :]) % grid[None, :]
    return {tuple(int(v) for v in row) for row in off}


def force_adjoint(gid_of_slot, home_slot_of_atom, f_init):
    """Home-slot forces after the exchange: the sum over all images of an atom.

    Returns an array shaped like f_init holding, at every home slot, the sum of
    f_init over every slot that holds that atom (its home slot included).
    Computed in float64; exact when the inputs are small integers.
    """
    n_atoms = len(home_slot_of_atom)
    acc = np.zeros((n_atoms, 3), np.float64)
    np.add.at(acc, gid_of_slot, f_init.astype(np.float64))
    out = np.zeros_like(f_init, dtype=np.float64)
    out[home_slot_of_atom] = acc
    return out, acc


def expected_send_sizes(box, grid, cutoff, density):
    """Expected atoms sent per domain in every pulse (z pulses, then y, then x).

    In pulse k of dimension dd a domain sends the atoms of the slab
    [k w_dd, min(rc, (k+1) w_dd)) above its receiver's upper face; across the
    slab the extent is w_d + rc for dimensions already exchanged (their halo is
    forwarded) and w_d for the others.
    """
    box = np.asarray(box, np.float64)
    grid = np.asarray(grid, np.int64)
    rc = float(np.float32(cutoff))
    w = box / grid
    _, _, npd = geometry(box, grid, cutoff)
    sizes = []
    done = set()
    for dd in (2, 1, 0):
        if grid[dd] == 1:
            continue
        for k in range(int(npd[dd])):
            thick = min(rc, (k + 1) * w[dd]) - k * w[dd]
            area = 1.0
            for d in range(3):
                if d == dd:
                    continue
                area *= (w[d] + rc) if d in done else w[d]
            sizes.append((dd, k, density * area * thick))
        done.add(dd)
    return sizes
