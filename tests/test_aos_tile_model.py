"""CPU model of the plane-tiled odd in-place step of the AoS layout
(kernels_aos.hpp), restated here: a workgroup per tile of one plane loads
the views of the tile and its ring (three runs of the records of planes
z - 1, z, z + 1), gathers, collides and scatters in its LDS copy, reads and
writes the own slots of bounced links with a z part in memory, and stores
the slots its cells own.  Run for every tile of small boxes (ragged tiles,
rows that wrap inside one tile, walls, solids, one-cell axes, one- and
two-plane boxes) against the plain odd-step slot rule of the fieldcraft
page's in-place pattern (first section): cell x reads f_q from
(opp q, x - c_q) and writes f*_q to (q, x + c_q), its own opposite slot
where the link leaves the fluid.

Checked: every global index is inside the lattice, every LDS position inside
the tile's array; no slot is stored twice; and with a collision that mixes
every input of a cell, the lattice after the step equals the slot rule's
exactly, whichever order the workgroups run in.
"""
import numpy as np
import pytest

import lbm_inputs as li
import oracle

C, _W, OPP = oracle.lattice()
Q = 19


def odd_step_rule(dims, per, mask, lat, collide):
    nx, ny, nz = dims
    out = lat.copy()

    def link(x, y, z, d):
        p = [x + d[0], y + d[1], z + d[2]]
        for a, n in enumerate(dims):
            if not 0 <= p[a] < n:
                if not per[a]:
                    return None
                p[a] %= n
        j = p[0] + nx * (p[1] + ny * p[2])
        return None if mask[j] else j

    for z in range(nz):
        for y in range(ny):
            for x in range(nx):
                i = x + nx * (y + ny * z)
                if mask[i]:
                    continue
                f = np.empty(Q, np.int64)
                slot = {}
                for d in range(Q):
                    j = link(x, y, z, C[d]) if d != 9 else i
                    slot[d] = j * Q + d if j is not None else i * Q + OPP[d]
                    f[OPP[d]] = lat[slot[d]]
                fs = collide(i, f)
                for d in range(Q):
                    out[slot[d]] = fs[d]
    return out


def tiled_odd_step(dims, per, mask, lat, collide, TX, TY, order=1):
    """aos_odd_tile_kernel: one workgroup per tile of TX x TY cells of one
    plane; each runs to completion against one shared memory, in forward or
    reverse order (a slot used by one workgroup and stored by another would
    make the two orders disagree with the slot rule)."""
    nx, ny, nz = dims
    PX, NP = TX + 2, (TX + 2) * (TY + 2)
    nxy, size = nx * ny, lat.size
    mem = lat.copy()
    writer = {}

    def store(k, tile, v):
        assert 0 <= k < size
        assert k not in writer, f"slot {k} written by tiles {writer[k]} and {tile}"
        writer[k] = tile
        mem[k] = v

    ntx, nty = -(-nx // TX), -(-ny // TY)
    tiles = [(tx, ty, z) for ty in range(nty) for tx in range(ntx) for z in range(nz)]
    for tile in (tiles if order > 0 else tiles[::-1]):
        tx, ty, z = tile
        zm, zp = (z - 1) % nz, (z + 1) % nz
        x0, y0 = tx * TX, ty * TY
        nxt, nyt = min(nx - x0, TX), min(ny - y0, TY)

        def pos(P):
            lx, ly = P % PX - 1, P // PX - 1
            if lx > nxt or ly > nyt:
                return None
            gx, gy = x0 + lx, y0 + ly
            if not 0 <= gx < nx:
                if not per[0]:
                    return None
                gx %= nx
            if not 0 <= gy < ny:
                if not per[1]:
                    return None
                gy %= ny
            return lx, ly, gx + nx * gy

        V = np.zeros((Q, NP), np.int64)
        M = np.ones((3, NP), np.uint8)
        planes = (zm, z, zp)
        for P in range(NP):
            r = pos(P)
            if r is None:
                continue
            row = r[2]
            for e in range(Q):
                k = (row + nxy * planes[1 + C[e][2]]) * Q + e
                assert 0 <= k < size
                V[e, P] = mem[k]
            M[0, P] = (not per[2] and z == 0) or mask[row + nxy * zm] != 0
            M[1, P] = mask[row + nxy * z] != 0
            M[2, P] = (not per[2] and z == nz - 1) or mask[row + nxy * zp] != 0
        for ly in range(TY):
            for lx in range(TX):
                if lx >= nxt or ly >= nyt:
                    continue
                P0 = (ly + 1) * PX + lx + 1
                if M[1, P0]:
                    continue
                cell = x0 + lx + nx * (y0 + ly + ny * z)
                f = np.empty(Q, np.int64)
                where = {}
                for d in range(Q):
                    if d == 9:
                        where[d] = ("lds", 9, P0)
                        continue
                    Pn = P0 + C[d][0] + C[d][1] * PX
                    assert 0 <= Pn < NP
                    back = M[1 + C[d][2], Pn] != 0
                    e = OPP[d]
                    if not back:
                        where[d] = ("lds", d, Pn)
                    elif C[d][2] == 0:
                        where[d] = ("lds", e, P0)
                    else:
                        where[d] = ("mem", cell * Q + e)
                for d in range(Q):
                    w = where[d]
                    f[OPP[d]] = V[w[1], w[2]] if w[0] == "lds" else mem[w[1]]
                fs = collide(cell, f)
                for d in range(Q):
                    w = where[d]
                    if w[0] == "lds":
                        V[w[1], w[2]] = fs[d]
                    else:
                        store(w[1], tile, fs[d])
        for P in range(NP):
            r = pos(P)
            if r is None:
                continue
            lx, ly, row = r
            tileP = 0 <= lx < nxt and 0 <= ly < nyt
            for e in range(Q):
                olx, oly = lx - C[e][0], ly - C[e][1]
                otile = 0 <= olx < nxt and 0 <= oly < nyt
                rfluid = M[1 + C[e][2], P] == 0
                ofluid = False
                if otile or tileP:
                    Po = P - C[e][0] - C[e][1] * PX
                    assert 0 <= Po < NP
                    ofluid = M[1, Po] == 0
                if rfluid and ((otile and ofluid) or (C[e][2] == 0 and tileP and not ofluid)):
                    store((row + nxy * planes[1 + C[e][2]]) * Q + e, tile, V[e, P])
    return mem


def mixing_collision(cell, f):
    # every output depends on every input and on the cell and direction
    s = int(np.sum((np.arange(Q) + 3) * f) % 1000003)
    return np.array([(s * 7 + 13 * q + 101 * cell + int(f[q])) % 2147483647 for q in range(Q)], np.int64)


CASES = {
    # dims, periodic, solid fraction, tile (TX, TY)
    "periodic_ragged": ((11, 7, 3), (1, 1, 1), 0.0, (4, 3)),
    "periodic_solids": ((9, 6, 4), (1, 1, 1), 0.25, (4, 2)),
    "walls_solids": ((10, 5, 4), (0, 0, 1), 0.2, (4, 2)),
    "z_walls": ((7, 6, 3), (1, 1, 0), 0.2, (4, 4)),
    "row_wraps_in_tile": ((3, 5, 3), (1, 1, 1), 0.2, (4, 2)),
    "one_cell_x": ((1, 4, 3), (1, 0, 1), 0.1, (4, 2)),
    "one_cell_y_and_z": ((6, 1, 1), (1, 1, 1), 0.0, (4, 2)),
    "one_plane_solids": ((6, 5, 1), (1, 1, 1), 0.2, (4, 2)),
    "two_planes": ((5, 4, 2), (1, 1, 1), 0.2, (2, 2)),
    "z_walls_two_planes": ((5, 4, 2), (1, 1, 0), 0.2, (2, 2)),
    "kernel_tile_ragged": ((70, 10, 2), (1, 0, 1), 0.15, (64, 8)),
}


@pytest.mark.parametrize("order", [1, -1])
@pytest.mark.parametrize("name", sorted(CASES))
def test_tiled_aos_odd_step_matches_slot_rule(name, order):
    dims, per, frac, (TX, TY) = CASES[name]
    n = int(np.prod(dims))
    mask = li.random_mask(*dims, fraction=frac, seed=sum(name.encode())) if frac else np.zeros(n, np.uint8)
    rng = np.random.default_rng(11)
    lat = rng.integers(0, 2 ** 30, size=n * Q, dtype=np.int64)
    want = odd_step_rule(dims, per, mask, lat, mixing_collision)
    got = tiled_odd_step(dims, per, mask, lat, mixing_collision, TX, TY, order)
    np.testing.assert_array_equal(got, want)
