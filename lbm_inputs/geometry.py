"""Solid masks (uint8[N], 0 = fluid, 1 = solid), decided in exact integers.

cell = x + nx*(y + ny*z); returned arrays are flat, length nx*ny*nz.
"""
import numpy as np

from .mt64 import MT19937_64, uniform01


def sphere_mask(nx, ny=None, nz=None, radius=16):
    """One sphere at the geometric centre of the box ((n-1)/2 on each axis).
    A cell is solid iff (2i-(nx-1))^2 + (2j-(ny-1))^2 + (2k-(nz-1))^2 <= (2r)^2;
    cells exactly on the sphere count as solid."""
    ny = nx if ny is None else ny
    nz = nx if nz is None else nz
    i = (2 * np.arange(nx, dtype=np.int64) - (nx - 1)) ** 2
    j = (2 * np.arange(ny, dtype=np.int64) - (ny - 1)) ** 2
    k = (2 * np.arange(nz, dtype=np.int64) - (nz - 1)) ** 2
    d2 = k[:, None, None] + j[None, :, None] + i[None, None, :]
    r2 = (2 * int(radius)) ** 2
    return (d2 <= r2).astype(np.uint8).reshape(-1)


def cylinder_mask(nx, ny, nz, cx2, cy2, radius):
    """A cylinder along z through the whole box, axis at (cx2 / 2, cy2 / 2) in
    cell units (half-cell resolution, integers).  A cell is solid iff
    (2i - cx2)^2 + (2j - cy2)^2 <= (2r)^2."""
    i = (2 * np.arange(nx, dtype=np.int64) - int(cx2)) ** 2
    j = (2 * np.arange(ny, dtype=np.int64) - int(cy2)) ** 2
    d2 = j[:, None] + i[None, :]
    plane = (d2 <= (2 * int(radius)) ** 2).astype(np.uint8)
    return np.broadcast_to(plane, (nz, ny, nx)).copy().reshape(-1)


def porous_sphere_count(nx, ny=None, nz=None, per_128cube=300):
    """Sphere count that keeps the porosity of `per_128cube` spheres in a 128^3
    box at any box volume: n = 300 * N / 128^3 (2400 at 256^3, 19200 at 512^3)."""
    ny = nx if ny is None else ny
    nz = nx if nz is None else nz
    return int(round(per_128cube * (nx * ny * nz) / 128.0 ** 3))


_Q = 1024  # sub-cell quantum of the sphere geometry


def porous_mask(nx, ny=None, nz=None, n_spheres=None, seed=5, rmin=6.0, rmax=12.0):
    """Overlapping spheres with uniform centres and radii r ~ U(rmin, rmax) in a
    periodic box.  Per sphere draw c_x, c_y, c_z = n_a U, then r = rmin + (rmax-rmin) U.
    Centres and radii are quantised to 1/1024 cell (floor(v*1024 + 1/2)); a cell
    (i, j, k) is solid iff the squared minimum-image distance between 1024*(i,j,k)
    and the quantised centre is <= the squared quantised radius (int64 exact).
    Returns (mask, n_spheres)."""
    ny = nx if ny is None else ny
    nz = nx if nz is None else nz
    if n_spheres is None:
        n_spheres = porous_sphere_count(nx, ny, nz)
    dims = (nx, ny, nz)
    g = MT19937_64(seed)
    draws = uniform01(g, 4 * n_spheres).reshape(n_spheres, 4)
    mask = np.zeros((nz, ny, nx), np.uint8)
    for s in range(n_spheres):
        cq = [int(np.floor(dims[a] * draws[s, a] * _Q + 0.5)) for a in range(3)]
        r = rmin + (rmax - rmin) * draws[s, 3]
        rq = int(np.floor(r * _Q + 0.5))
        idx, d2 = [], []
        for a in range(3):
            n = dims[a]
            lo = (cq[a] - rq) // _Q
            hi = -((-(cq[a] + rq)) // _Q)
            cells = np.arange(lo, hi + 1, dtype=np.int64)
            if cells.size >= n:
                cells = np.arange(0, n, dtype=np.int64)
            cells = np.mod(cells, n)
            period = n * _Q
            d = np.mod(_Q * cells - cq[a] + period // 2, period) - period // 2
            idx.append(cells)
            d2.append(d * d)
        tot = d2[2][:, None, None] + d2[1][None, :, None] + d2[0][None, None, :]
        hit = tot <= rq * rq
        sub = mask[np.ix_(idx[2], idx[1], idx[0])]
        mask[np.ix_(idx[2], idx[1], idx[0])] = sub | hit.astype(np.uint8)
    return mask.reshape(-1), n_spheres


def random_mask(nx, ny, nz, fraction=0.2, seed=7):
    """Independent solid cells with probability `fraction` (one draw per cell)."""
    n = nx * ny * nz
    g = MT19937_64(seed)
    return (uniform01(g, n) < fraction).astype(np.uint8)
