"""Exhaustive CPU check of the in-place address rules on small boxes with
solids, walls and open faces (an independent restatement of the rules, not
the kernels' code; the GPU's collision-free bit-exact runs check the code).

AA (fieldcraft page, first section): even steps read (q, x) and write
(opp q, x); odd steps read (opp q, x - c_q) and write (q, x + c_q), with the
halfway bounce-back substitutions (own slots) where the link leaves the fluid.
Esoteric pull (dense and compact storage) and esoteric twist, as described
in the design notes.
For every scheme and parity: the read slots of all (cell, direction) pairs
are distinct, so are the written slots, each cell writes exactly the slots it
read (no cell can overwrite another's input), and collision-free steps through
the slots reproduce the oracle's streaming bit for bit."""
import numpy as np
import pytest

import lbm_inputs as li
import oracle

C, W, OPP = oracle.lattice()
Q = 19


class Geo:
    def __init__(self, dims, periodic, mask, open_faces):
        self.dims, self.periodic, self.mask = dims, periodic, mask
        self.open = {oracle.FACES.index(k) for k in (open_faces or {})}
        self.n = dims[0] * dims[1] * dims[2]
        self.fluid = [i for i in range(self.n) if mask[i] == 0]

    def coords(self, i):
        nx, ny, _ = self.dims
        return [i % nx, (i // nx) % ny, i // (nx * ny)]

    def link(self, i, d):
        """('fluid' | 'solid' | 'wall' | 'open', wrapped index) of i + d."""
        p, wall, op = self.coords(i), False, False
        for a in range(3):
            p[a] += int(d[a])
            if 0 <= p[a] < self.dims[a]:
                continue
            k = 2 * a + (0 if p[a] < 0 else 1)
            p[a] %= self.dims[a]
            if self.periodic[a]:
                continue
            if k in self.open:
                op = True
            else:
                wall = True
        j = p[0] + self.dims[0] * (p[1] + self.dims[1] * p[2])
        if wall:
            return "wall", j
        if op:
            return "open", j
        return ("solid" if self.mask[j] else "fluid"), j


def aa_slots(g, parity):
    """read[(x, q)], write[(x, q)]: slot read for f_q and written with f*_q."""
    rd, wr = {}, {}
    for x in g.fluid:
        for q in range(Q):
            if parity == 0:
                rd[x, q] = (q, x)
                wr[x, q] = (OPP[q], x)
                continue
            kind, j = g.link(x, -C[q])
            rd[x, q] = (OPP[q], j) if kind == "fluid" else (q, x)
            kind, j = g.link(x, C[q])
            wr[x, q] = (q, j) if kind == "fluid" else (OPP[q], x)
    return rd, wr


def eso_slots(g, parity, compact):
    """Esoteric pull: pair k < 9 has slots S0 = plane k, S1 = plane 18 - k."""
    rd = {}
    bounce = {}
    for x in g.fluid:
        rd[x, 9] = (9, x)
        for k in range(9):
            kind, _ = g.link(x, -C[k])
            rd[x, k] = (k, x) if (kind != "fluid" or parity == 0) else (OPP[k], x)
            kind, j = g.link(x, C[k])
            q = OPP[k]
            if kind == "fluid":
                rd[x, q] = (q if parity == 0 else k, j)
            elif compact:
                rd[x, q] = ("B", bounce.setdefault((x, k), len(bounce)))
            elif kind == "solid":
                rd[x, q] = (k, j)
            else:
                rd[x, q] = (q, j)      # S1 of the wrapped cell beyond a face
    wr = {(x, q): rd[x, OPP[q]] for (x, q) in rd}
    return rd, wr


def twist_slots(g, parity):
    """Esoteric twist: f_q of x at parity P lives at x - c+_q (c+ = max(c, 0)
    per axis) in plane q (P = 0) or opp q (P = 1); below the low face of a
    non-periodic axis the location is a halo slot, keyed by its coordinate -1.
    f*_q goes where f_opp(q) was read, or, bounced back, to the other plane
    at that location: where x finds f_opp(q) at the next step."""
    def loc(x, d):
        p = g.coords(x)
        for a in range(3):
            p[a] += int(d[a])
            if p[a] < 0 and g.periodic[a]:
                p[a] += g.dims[a]
        return tuple(p)

    def plane(par, q):
        return q if par == 0 else OPP[q]

    rd, wr = {}, {}
    for x in g.fluid:
        for q in range(Q):
            rd[x, q] = (plane(parity, q), loc(x, -np.maximum(C[q], 0)))
    for x in g.fluid:
        for q in range(Q):
            kind, _ = g.link(x, C[q])
            o = OPP[q]
            where = loc(x, np.minimum(C[q], 0))
            wr[x, q] = (plane(parity, o) if kind in ("fluid", "open") else plane(1 - parity, o), where)
    return rd, wr


def check_maps(g, rd, wr):
    assert len(set(rd.values())) == len(rd), "two links read one slot"
    assert len(set(wr.values())) == len(wr), "two links write one slot"
    for x in g.fluid:
        assert {rd[x, q] for q in range(Q)} == {wr[x, q] for q in range(Q)}, x


def check_maps_no_cross(g, rd, wr):
    """Reads distinct, writes distinct, and no cell writes a slot that another
    cell reads in the same step (a cell may write a slot no one reads)."""
    assert len(set(rd.values())) == len(rd), "two links read one slot"
    assert len(set(wr.values())) == len(wr), "two links write one slot"
    reader = {s: x for (x, q), s in rd.items()}
    for (x, q), s in wr.items():
        assert reader.get(s, x) == x, (x, q, s, reader.get(s))


def stream_through(g, box, f0, steps, slots):
    """Collision-free steps through the slot maps; returns f after each step."""
    state = {}
    rd0, _ = slots(0)
    for (x, q), s in rd0.items():
        state[s] = f0[q, x]
    f, out = f0.copy(), []
    for t in range(steps):
        rd, wr = slots(t % 2)
        for x in g.fluid:
            for q in range(Q):
                kind, _ = g.link(x, -C[q])
                if kind == "open":
                    continue            # the reservoir's value, not a slot's
                assert state[rd[x, q]] == f[q, x], (t, x, q)
        post = {}
        for (x, q) in rd:
            post[wr[x, q]] = f[q, x]    # omega = 0: f* = f
        state.update(post)
        f = oracle.run(box, f, 1, g.mask)
        out.append(f)
    return out


CASES = {
    "periodic_solids": ((6, 5, 4), (1, 1, 1), 0.2, None),
    "walls": ((5, 4, 6), (0, 1, 0), 0.15, None),
    "open_and_wall_on_one_axis": ((6, 4, 3), (0, 1, 1), 0.1, {"-x": (1.0, (0.02, 0.0, 0.0))}),
    "open_edges": ((5, 5, 4), (0, 0, 1), 0.1, {"-x": (1.0, (0.01, 0.0, 0.0)), "+y": (1.02, (0.0, 0.0, 0.0))}),
    "thin": ((1, 3, 2), (1, 0, 1), 0.0, None),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_in_place_maps_are_race_free_and_stream(name):
    dims, per, frac, faces = CASES[name]
    mask = li.random_mask(*dims, fraction=frac, seed=sum(name.encode())) if frac else np.zeros(int(np.prod(dims)), np.uint8)
    g = Geo(dims, per, mask, faces)
    box = oracle.Box(*dims, periodic=per, tau=float("inf"), open_faces=faces)
    rng = np.random.default_rng(5)
    f0 = oracle.init_equilibrium(box, mask, 1 + 0.01 * rng.standard_normal(g.n),
                                 0.02 * rng.standard_normal((3, g.n)))
    f0 = oracle.apply_open_faces(box, f0 * (1 + 0.01 * rng.standard_normal(f0.shape)), mask)
    f0[:, mask != 0] = 0.0
    for label, slots in (("aa", lambda p: aa_slots(g, p)),
                         ("eso dense", lambda p: eso_slots(g, p, False)),
                         ("eso compact", lambda p: eso_slots(g, p, True))):
        for parity in (0, 1):
            check_maps(g, *slots(parity))
        stream_through(g, box, f0, 4, slots)
    slots = lambda p: twist_slots(g, p)  # noqa: E731
    for parity in (0, 1):
        check_maps_no_cross(g, *slots(parity))
    stream_through(g, box, f0, 4, slots)
