"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: exact
rational identities of the velocity set, the page's printed weights, closed
forms of textbook flows, a brute-force search for streaming, invariants.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import lbm_inputs as li

Q = 19


def _read_table(path):
    rows = []
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _exact_weights(w):
    # every weight is k/36 for an integer k; recover k and insist the double is
    # the correctly rounded k/36.
    out = []
    for x in w:
        k = round(x * 36)
        assert float(Fraction(k, 36)) == x
        out.append(Fraction(k, 36))
    return out


# --------------------------------------------------------------- P1 lattice

def test_velocity_set_and_order():
    c, w, opp = oracle.lattice()
    vecs = [tuple(v) for v in c.tolist()]
    expected = [(cx, cy, cz) for cz in (-1, 0, 1) for cy in (-1, 0, 1) for cx in (-1, 0, 1)
                if cx * cx + cy * cy + cz * cz <= 2]
    assert vecs == expected                 # lexicographic over (c_z, c_y, c_x)
    assert len(set(vecs)) == 19
    assert vecs[9] == (0, 0, 0)
    for q in range(Q):
        assert tuple(-c[q]) == tuple(c[opp[q]])
        assert opp[q] == 18 - q            # a property of this ordering


def test_weights_match_page(golden_dir):
    c, w, _ = oracle.lattice()
    table = {int(r[0]): (int(r[1]), Fraction(int(r[2]), int(r[3])))
             for r in _read_table(os.path.join(golden_dir, "d3q19_weights.txt"))}
    n2 = (c * c).sum(axis=1)
    for cls, (mult, wt) in table.items():
        sel = np.nonzero(n2 == cls)[0]
        assert sel.size == mult
        for q in sel:
            assert w[q] == float(wt)


def test_velocity_set_isotropy_exact():
    c, w, _ = oracle.lattice()
    W = _exact_weights(w)
    C = c.tolist()
    assert sum(W) == 1
    for a in range(3):
        assert sum(W[q] * C[q][a] for q in range(Q)) == 0
    for a, b in itertools.product(range(3), repeat=2):
        s = sum(W[q] * C[q][a] * C[q][b] for q in range(Q))
        assert s == (Fraction(1, 3) if a == b else 0)
    for a, b, d in itertools.product(range(3), repeat=3):
        assert sum(W[q] * C[q][a] * C[q][b] * C[q][d] for q in range(Q)) == 0
    for a, b, d, e in itertools.product(range(3), repeat=4):
        s = sum(W[q] * C[q][a] * C[q][b] * C[q][d] * C[q][e] for q in range(Q))
        iso = Fraction(int(a == b and d == e) + int(a == d and b == e) + int(a == e and b == d), 9)
        assert s == iso


# --------------------------------------------------------- P2 equilibrium

@pytest.mark.parametrize("rho,u", [(1.0, (0.0, 0.0, 0.0)), (1.03, (0.05, -0.02, 0.01)),
                                   (0.97, (-0.1, 0.07, 0.12))])
def test_equilibrium_moments(rho, u):
    c, _, _ = oracle.lattice()
    u = np.array(u)
    feq = oracle.equilibrium(rho, u)
    cf = c.astype(np.float64)
    tol = 1e-15
    assert abs(feq.sum() - rho) <= tol * 4
    np.testing.assert_allclose(cf.T @ feq, rho * u, rtol=0, atol=tol * 4)
    second = np.einsum("qa,qb,q->ab", cf, cf, feq)
    np.testing.assert_allclose(second, rho * np.eye(3) / 3 + rho * np.outer(u, u), rtol=0, atol=tol * 8)
    third = np.einsum("qa,qb,qc,q->abc", cf, cf, cf, feq)
    d = np.eye(3)
    want = rho / 3 * (np.einsum("a,bc->abc", u, d) + np.einsum("b,ac->abc", u, d)
                      + np.einsum("c,ab->abc", u, d))
    np.testing.assert_allclose(third, want, rtol=0, atol=tol * 8)


@pytest.mark.parametrize("tau", [0.51, 0.8, 1.7])
def test_equilibrium_is_fixed_point(tau):
    box = oracle.Box(1, 1, 1, tau=tau)
    for rho, u in [(1.0, (0.02, 0.0, -0.03)), (1.1, (-0.08, 0.05, 0.02))]:
        feq = oracle.equilibrium(rho, np.array(u))
        post = oracle.collide(box, feq)
        assert np.max(np.abs(post - feq)) <= 8 * np.finfo(np.float64).eps * feq.max()


def test_guo_term_moments():
    # zeroth moment 0, first moment (1 - omega/2) F: what makes the momentum
    # gain per step exactly F with u shifted by F/2.
    c, _, _ = oracle.lattice()
    for omega in (0.0, 1.0 / 0.7, 1.0 / 0.55):
        u = np.array([0.03, -0.01, 0.02])
        F = np.array([1e-3, -2e-3, 5e-4])
        g = oracle.guo_term(omega, u, F)
        assert abs(g.sum()) < 1e-18
        np.testing.assert_allclose(c.T.astype(float) @ g, (1 - omega / 2) * F, rtol=1e-13, atol=1e-19)


@pytest.mark.parametrize("omega", [0.0, 1.0 / 0.7, 1.0 / 0.55, 1.9])
@pytest.mark.parametrize("u,F", [((0.03, -0.01, 0.02), (1e-3, -2e-3, 5e-4)),
                                 ((-0.07, 0.11, 0.05), (2e-4, 3e-4, -7e-4)),
                                 ((0.2, 0.15, -0.12), (-1e-2, 4e-3, 6e-3))])
def test_guo_term_higher_moments(omega, u, F):
    # Guo, Zheng and Shi choose the forcing term so that its velocity moments
    # are those of the force acting on the Maxwellian up to second order:
    #   sum_q F_q c_a c_b     = (1 - omega/2) (u_a F_b + u_b F_a),
    #   sum_q F_q c_a c_b c_c = (1 - omega/2) (F_a d_bc + F_b d_ac + F_c d_ab) / 3.
    # The second moment is where the velocity-dependent parts -3 u.F and
    # 9 (c.u)(c.F) act; the simple forcing 3 w c.F, or either velocity part
    # with a wrong sign or factor, fails it.
    c, _, _ = oracle.lattice()
    u, F = np.array(u), np.array(F)
    g = oracle.guo_term(omega, u, F)
    cf = c.astype(np.float64)
    k = 1 - omega / 2
    scale = max(abs(k), 1e-300) * np.max(np.abs(F))
    second = np.einsum("qa,qb,q->ab", cf, cf, g)
    np.testing.assert_allclose(second, k * (np.outer(u, F) + np.outer(F, u)), rtol=0, atol=1e-15 * scale)
    third = np.einsum("qa,qb,qc,q->abc", cf, cf, cf, g)
    d = np.eye(3)
    want = k / 3 * (np.einsum("a,bc->abc", F, d) + np.einsum("b,ac->abc", F, d) + np.einsum("c,ab->abc", F, d))
    np.testing.assert_allclose(third, want, rtol=0, atol=1e-15 * scale)


def test_guo_term_is_second_order_hermite_projection():
    # the term lies in the span of w_q, w_q c_q and w_q c_q c_q (a polynomial
    # of degree two in c times the weight); with its moments up to second
    # order (pinned above) that determines it uniquely.  Solve for the ten
    # coefficients by least squares on exact integer design rows and demand a
    # zero residual.
    c, w, _ = oracle.lattice()
    cf = c.astype(np.float64)
    rows = [np.ones(19)] + [cf[:, a] for a in range(3)]
    rows += [cf[:, a] * cf[:, b] for a in range(3) for b in range(a, 3)]
    A = np.stack(rows, axis=1) * w[:, None]
    rng = np.random.default_rng(17)
    for _ in range(20):
        u = rng.uniform(-0.15, 0.15, 3)
        F = rng.uniform(-1e-3, 1e-3, 3)
        omega = rng.uniform(0.0, 1.95)
        g = oracle.guo_term(omega, u, F)
        coef, *_ = np.linalg.lstsq(A, g, rcond=None)
        assert np.max(np.abs(A @ coef - g)) <= 1e-17
        # and the coefficients are the Hermite ones: 3 F (degree 1),
        # 9/2 (u_a F_b + u_b F_a) on (c_a c_b - d_ab / 3) (degree 2)
        k = 1 - omega / 2
        want = np.zeros(10)
        want[1:4] = 3 * k * F
        i = 4
        for a in range(3):
            for b in range(a, 3):
                s = 9 / 2 * (u[a] * F[b] + u[b] * F[a]) * k
                want[i] = s if a == b else 2 * s
                if a == b:
                    want[0] -= s / 3
                i += 1
        np.testing.assert_allclose(coef, want, rtol=0, atol=1e-15)


# ------------------------------------------------------ P3 conservation

def _random_state(box, seed=3, mask=None):
    rho, u = li.random_fields(box.nx, box.ny, box.nz, seed=seed)
    return oracle.init_equilibrium(box, mask, rho, u)


def test_mass_momentum_conserved_periodic():
    box = oracle.Box(8, 6, 5, tau=0.6)
    f0 = _random_state(box)
    t0 = oracle.totals(box, f0)
    f1 = oracle.run(box, f0, 30)
    t1 = oracle.totals(box, f1)
    assert abs(t1["mass"] - t0["mass"]) / t0["mass"] < 1e-14
    assert np.max(np.abs(t1["momentum"] - t0["momentum"])) / t0["mass"] < 1e-14


def test_momentum_gain_with_force():
    F = (1e-4, -3e-5, 2e-5)
    box = oracle.Box(7, 5, 6, tau=0.75, force=F)
    f0 = _random_state(box, seed=11)
    t0 = oracle.totals(box, f0)
    n = 25
    f1 = oracle.run(box, f0, n)
    t1 = oracle.totals(box, f1)
    assert abs(t1["mass"] - t0["mass"]) / t0["mass"] < 1e-14
    np.testing.assert_allclose(t1["momentum"] - t0["momentum"], n * box.n * np.array(F),
                               rtol=1e-9, atol=1e-12)


def test_mass_conserved_with_walls_and_mask():
    box = oracle.Box(9, 7, 6, periodic=(1, 0, 0), tau=0.65, force=(1e-5, 0, 0))
    mask = li.random_mask(9, 7, 6, fraction=0.25, seed=4)
    f0 = _random_state(box, seed=5, mask=mask)
    m0 = oracle.totals(box, f0, mask)["mass"]
    f1 = oracle.run(box, f0, 20, mask)
    assert abs(oracle.totals(box, f1, mask)["mass"] - m0) / m0 < 1e-14
    solid = mask.astype(bool)
    assert np.all(f1[:, solid] == 0.0)


# ------------------------------------------- momentum exchange with the solids

@pytest.mark.parametrize("periodic,F", [((1, 1, 1), (2e-4, -1e-4, 5e-5)), ((1, 0, 1), (0.0, 0.0, 3e-4)),
                                        ((0, 0, 0), (1e-4, 2e-4, -1e-4))])
def test_momentum_exchange_closes_the_step_budget(periodic, F):
    # each step the collision adds F per fluid cell and every bounce-back link
    # hands 2 f*_q c_q to the solid: P(t+1) - P(t) = N_fluid F - F_exchanged,
    # for any state, exactly up to rounding
    box = oracle.Box(7, 6, 5, periodic=periodic, tau=0.7, force=F)
    mask = li.random_mask(7, 6, 5, fraction=0.2, seed=8)
    nf = int(np.count_nonzero(mask == 0))
    f = _random_state(box, seed=9, mask=mask)
    for _ in range(4):
        fx = oracle.momentum_exchange(box, f, mask)
        p0 = oracle.totals(box, f, mask)
        f = oracle.run(box, f, 1, mask)
        p1 = oracle.totals(box, f, mask)
        want = nf * np.array(F) - fx["solid"] - fx["wall"]
        np.testing.assert_allclose(p1["momentum"] - p0["momentum"], want, rtol=0, atol=1e-14 * p0["mass"])
        if all(periodic):
            assert np.all(fx["wall"] == 0.0)
        assert np.max(np.abs(fx["solid"])) > 1e-6  # the random state pushes on the solids


def test_momentum_exchange_zero_at_rest():
    # fluid at rest, no force: f* = w on every link; in a periodic box every row
    # of a solid body has as many entry links as exit links, and the two walls
    # of a channel mirror each other, so the exchanged force vanishes
    for periodic in ((1, 1, 1), (1, 0, 1), (0, 0, 0)):
        box = oracle.Box(8, 7, 6, periodic=periodic, tau=0.8)
        mask = li.random_mask(8, 7, 6, fraction=0.3, seed=2) if all(periodic) else None
        fx = oracle.momentum_exchange(box, oracle.init_equilibrium(box, mask), mask)
        assert np.max(np.abs(fx["solid"])) < 1e-15 and np.max(np.abs(fx["wall"])) < 1e-15


def test_steady_channel_wall_force_balances_body_force():
    # steady plane Poiseuille flow: the walls carry the whole body force,
    # F_wall = N_fluid g along the flow and nothing across it
    H, g, tau = 16, 1e-5, 0.8
    box = oracle.Box(1, H, 1, periodic=(1, 0, 1), tau=tau, force=(0.0, 0.0, g))
    f = oracle.run(box, oracle.init_equilibrium(box), 6000)
    fx = oracle.momentum_exchange(box, f)
    assert abs(fx["wall"][2] - H * g) < 1e-6 * H * g
    # across the channel the two walls take equal and opposite pressure forces
    # (about 1/3 per wall cell), cancelling to rounding
    assert abs(fx["wall"][0]) < 1e-18 and abs(fx["wall"][1]) < 1e-13
    assert np.all(fx["solid"] == 0.0)


# ----------------------------------------------------------- open faces

def test_open_faces_keep_uniform_flow():
    # a uniform stream whose reservoirs on both open faces hold the same
    # equilibrium is a fixed point of the update: what leaves equals what the
    # reservoir sends in, on every link
    for periodic, faces, u in (((0, 1, 1), ("-x", "+x"), (0.03, -0.01, 0.02)),
                               ((1, 0, 1), ("-y", "+y"), (0.01, 0.025, 0.0)),
                               ((0, 0, 1), ("-x", "+x", "-y", "+y"), (0.02, 0.01, -0.015))):
        box = oracle.Box(7, 6, 5, periodic=periodic, tau=0.8, open_faces={k: (1.02, u) for k in faces})
        n = box.n
        f0 = oracle.init_equilibrium(box, None, np.full(n, 1.02), np.tile(np.array(u)[:, None], (1, n)))
        f1 = oracle.run(box, f0, 40)
        assert np.max(np.abs(f1 - f0)) < 1e-15, periodic


def test_open_faces_close_mass_and_momentum_budget():
    # open x faces, periodic y and z: per step the box gains what the
    # reservoirs send in along the entering links and loses the post-collision
    # populations on the leaving links (collision conserves mass and adds F
    # per fluid cell; bounce-back at solids hands 2 f* c to them)
    F = (1e-4, 2e-5, 0.0)
    faces = {"-x": (1.01, (0.04, 0.0, 0.01)), "+x": (0.99, (0.02, -0.01, 0.0))}
    box = oracle.Box(9, 6, 5, periodic=(0, 1, 1), tau=0.75, force=F, open_faces=faces)
    mask = li.random_mask(9, 6, 5, fraction=0.15, seed=12)
    nf = int(np.count_nonzero(mask == 0))
    c, _, _ = oracle.lattice()
    rho, u = li.random_fields(9, 6, 5, seed=13)
    f = oracle.init_equilibrium(box, mask, rho, u)
    solid = mask.reshape(5, 6, 9).astype(bool)
    feq = {k: oracle.equilibrium(r, v) for k, (r, v) in faces.items()}
    for _ in range(3):
        m0 = oracle.totals(box, f, mask)
        gain_m, gain_p = 0.0, np.zeros(3)
        fz = f.reshape(19, 5, 6, 9)
        for z in range(5):
            for y in range(6):
                for x, face, side in ((0, "-x", 1), (8, "+x", -1)):
                    if solid[z, y, x]:
                        continue
                    post = oracle.collide(box, fz[:, z, y, x])
                    for q in range(19):
                        if c[q][0] == side:      # enters through this face
                            gain_m += feq[face][q]
                            gain_p += feq[face][q] * c[q]
                        elif c[q][0] == -side:   # leaves through it
                            gain_m -= post[q]
                            gain_p -= post[q] * c[q]
        fx = oracle.momentum_exchange(box, f, mask)
        f = oracle.run(box, f, 1, mask)
        m1 = oracle.totals(box, f, mask)
        assert abs(m1["mass"] - m0["mass"] - gain_m) < 1e-13 * m0["mass"]
        want_p = gain_p + nf * np.array(F) - fx["solid"] - fx["wall"]
        np.testing.assert_allclose(m1["momentum"] - m0["momentum"], want_p, rtol=0, atol=1e-13 * m0["mass"])
        assert np.all(fx["wall"] == 0.0)


def test_apply_open_faces_is_what_init_does():
    faces = {"-z": (1.0, (0.0, 0.01, 0.03)), "+y": (1.03, (0.0, 0.0, 0.0))}
    box = oracle.Box(6, 7, 8, periodic=(1, 0, 0), tau=0.9, open_faces=faces)
    rho, u = li.random_fields(6, 7, 8, seed=3)
    f = oracle.init_equilibrium(box, None, rho, u)
    plain = oracle.init_equilibrium(oracle.Box(6, 7, 8, periodic=(1, 0, 0), tau=0.9), None, rho, u)
    np.testing.assert_array_equal(oracle.apply_open_faces(box, plain), f)
    np.testing.assert_array_equal(oracle.apply_open_faces(box, f), f)
    assert np.any(f != plain)


# ------------------------------------------------------ open-face rules
#
# Besides the equilibrium reservoir, an open face may hold a Neumann inlet
# (the equilibrium of the inward cell's density and velocity) or a Zou-He
# condition (prescribed density, or prescribed velocity).  Pins: what each
# rule must make of a uniform stream and of the moments of any state.

def _face_cells(box, face):
    a, side = oracle.FACES.index(face) // 2, oracle.FACES.index(face) % 2
    n = (box.nx, box.ny, box.nz)
    at = 0 if side == 0 else n[a] - 1
    z, y, x = np.meshgrid(np.arange(box.nz), np.arange(box.ny), np.arange(box.nx), indexing="ij")
    sel = (x, y, z)[a].reshape(-1) == at
    return np.nonzero(sel)[0], a, (1 if side == 0 else -1)


def _noisy_state(box, mask, seed):
    # a state far from local equilibrium: equilibrium of random fields plus
    # random positive noise on every population
    rho, u = li.random_fields(box.nx, box.ny, box.nz, seed=seed, drho=0.02, du=0.04)
    plain = oracle.Box(box.nx, box.ny, box.nz, periodic=box.periodic, tau=box.tau, force=box.force)
    f = oracle.init_equilibrium(plain, mask, rho, u)
    rng = np.random.default_rng(seed)
    f = f * (1.0 + 0.05 * rng.standard_normal(f.shape))
    if mask is not None:
        f[:, mask.reshape(-1) != 0] = 0.0
    return f


@pytest.mark.parametrize("rules", [("zou_he_velocity", "zou_he_pressure"), ("neumann", "neumann"),
                                   ("equilibrium", "zou_he_pressure"), ("zou_he_pressure", "zou_he_velocity"),
                                   ("neumann", "zou_he_pressure")])
@pytest.mark.parametrize("axis", [0, 1, 2])
def test_face_rules_keep_uniform_flow(rules, axis):
    # a uniform stream at equilibrium is a fixed point of every rule whose
    # prescribed values agree with it (the pressure rule prescribes only the
    # density and the tangential velocity, so its normal velocity is whatever
    # mass balance gives: the stream's)
    rho0, u0 = 1.02, np.array([0.03, -0.01, 0.02])
    dims = [6, 5, 4]
    dims[axis] = 8
    periodic = [1, 1, 1]
    periodic[axis] = 0
    lo, hi = oracle.FACES[2 * axis], oracle.FACES[2 * axis + 1]
    faces = {lo: (rho0, tuple(u0), rules[0]), hi: (rho0, tuple(u0), rules[1])}
    box = oracle.Box(*dims, periodic=tuple(periodic), tau=0.8, open_faces=faces)
    n = box.n
    f0 = oracle.init_equilibrium(box, None, np.full(n, rho0), np.tile(u0[:, None], (1, n)))
    feq = oracle.equilibrium(rho0, u0)
    assert np.max(np.abs(f0 - feq[:, None])) < 1e-16
    f1 = oracle.run(box, f0, 30)
    assert np.max(np.abs(f1 - f0)) < 1e-14


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("walls", [False, True])
def test_zou_he_prescribes_its_moments(axis, walls):
    # on any state, after the rule: a velocity face's cells carry exactly the
    # prescribed velocity (u = (sum c f + F/2) / rho), a pressure face's cells
    # the prescribed density and tangential velocity -- except at edges with a
    # wall, where the wall's bounce-back supplies some entering populations
    F = (2e-4, -1e-4, 3e-5)
    dims = [7, 6, 5]
    periodic = [1, 1, 1]
    periodic[axis] = 0
    other = 1 - axis
    if walls:
        periodic[other] = 0
    lo, hi = oracle.FACES[2 * axis], oracle.FACES[2 * axis + 1]
    u_in = np.array([0.02, 0.01, -0.015])
    u_t = np.array([0.005, -0.01, 0.02])
    faces = {lo: (1.0, tuple(u_in), "zou_he_velocity"), hi: (0.98, tuple(u_t), "zou_he_pressure")}
    box = oracle.Box(*dims, periodic=tuple(periodic), tau=0.7, force=F, open_faces=faces)
    mask = li.random_mask(*dims, fraction=0.1, seed=21)
    f = oracle.apply_open_faces(box, _noisy_state(box, mask, 22), mask)
    rho, u = oracle.moments(box, f, mask)
    fluid = mask.reshape(-1) == 0
    coords = np.stack(np.meshgrid(np.arange(dims[2]), np.arange(dims[1]), np.arange(dims[0]),
                                  indexing="ij")[::-1]).reshape(3, -1)
    inner = np.ones(box.n, bool)
    if walls:
        inner = (coords[other] > 0) & (coords[other] < dims[other] - 1)
    cells, _, _ = _face_cells(box, lo)
    cells = cells[fluid[cells] & inner[cells]]
    assert cells.size > 5
    np.testing.assert_allclose(u[:, cells], np.tile(u_in[:, None], (1, cells.size)), rtol=0, atol=1e-14)
    cells, _, _ = _face_cells(box, hi)
    cells = cells[fluid[cells] & inner[cells]]
    np.testing.assert_allclose(rho[cells], 0.98, rtol=0, atol=1e-14)
    for t in range(3):
        if t != axis:
            np.testing.assert_allclose(u[t, cells], u_t[t], rtol=0, atol=1e-14)
    # and the prescribed velocity is not what the cells held before
    rho_b, u_b = oracle.moments(box, _noisy_state(box, mask, 22), mask)
    assert np.max(np.abs(rho_b[cells] - 0.98)) > 1e-3


@pytest.mark.parametrize("axis", [0, 2])
def test_zou_he_bounces_back_the_normal_non_equilibrium(axis):
    # Zou and He's closure: the population along the inward normal and its
    # opposite have the same non-equilibrium part (no force here, so the
    # equilibrium is that of the cell's own moments)
    dims = [5, 6, 5]
    periodic = [1, 1, 1]
    periodic[axis] = 0
    lo, hi = oracle.FACES[2 * axis], oracle.FACES[2 * axis + 1]
    faces = {lo: (1.0, (0.01, 0.02, 0.03), "zou_he_velocity"), hi: (1.01, (0.0, 0.0, 0.0), "zou_he_pressure")}
    box = oracle.Box(*dims, periodic=tuple(periodic), tau=0.9, open_faces=faces)
    f = oracle.apply_open_faces(box, _noisy_state(box, None, 31))
    c, _, opp = oracle.lattice()
    for face in (lo, hi):
        cells, a, sigma = _face_cells(box, face)
        qn = [q for q in range(19) if c[q][a] == sigma and np.count_nonzero(c[q]) == 1][0]
        for x in cells:
            r, v = oracle.cell_moments(box, f[:, x])
            feq = oracle.equilibrium(r, v)
            assert abs((f[qn, x] - feq[qn]) - (f[opp[qn], x] - feq[opp[qn]])) < 1e-15


def test_neumann_copies_the_inward_equilibrium():
    # at local equilibrium the Neumann rule hands each entering population the
    # value the inward cell holds in that direction; where the inward cell is
    # solid, the face's own values are used
    box = oracle.Box(7, 5, 4, periodic=(0, 1, 1), tau=0.8,
                     open_faces={"-x": (1.01, (0.02, 0.0, 0.0), "neumann"),
                                 "+x": (0.99, (0.01, 0.01, 0.0), "neumann")})
    mask = np.zeros((4, 5, 7), np.uint8)
    mask[1, 2, 1] = 1   # inward of (0, 2, 1)
    mask[3, 0, 5] = 1   # inward of (6, 0, 3)
    mask = mask.reshape(-1)
    rho, u = li.random_fields(7, 5, 4, seed=41, drho=0.03, du=0.05)
    f = oracle.init_equilibrium(box, mask, rho, u)
    plain = oracle.init_equilibrium(oracle.Box(7, 5, 4, periodic=(0, 1, 1), tau=0.8), mask, rho, u)
    c, _, _ = oracle.lattice()
    fz, pz = f.reshape(19, 4, 5, 7), plain.reshape(19, 4, 5, 7)
    checked = 0
    for x0, x1, side, face in ((0, 1, 1, "-x"), (6, 5, -1, "+x")):
        r, v = box.open_faces[face][:2]
        feq = oracle.equilibrium(r, v)
        for z in range(4):
            for y in range(5):
                for q in range(19):
                    got = fz[q, z, y, x0]
                    if c[q][0] != side:
                        assert got == pz[q, z, y, x0]
                    elif mask.reshape(4, 5, 7)[z, y, x1]:
                        assert got == feq[q]
                    else:
                        assert abs(got - pz[q, z, y, x1]) < 1e-16
                        checked += 1
    assert checked > 100


def test_face_rules_touch_only_entering_populations():
    # applying the rules twice changes nothing (no rule reads what another
    # writes), and init is the plain equilibrium followed by the rules
    faces = {"-y": (1.0, (0.0, 0.03, 0.01), "zou_he_velocity"), "+y": (1.0, (0.0, 0.0, 0.0), "neumann")}
    box = oracle.Box(5, 6, 4, periodic=(1, 0, 1), tau=0.9, force=(0.0, 1e-4, 0.0), open_faces=faces)
    mask = li.random_mask(5, 6, 4, fraction=0.15, seed=5)
    f = oracle.apply_open_faces(box, _noisy_state(box, mask, 51), mask)
    np.testing.assert_array_equal(oracle.apply_open_faces(box, f, mask), f)
    rho, u = li.random_fields(5, 6, 4, seed=52)
    plain = oracle.init_equilibrium(oracle.Box(5, 6, 4, periodic=(1, 0, 1), tau=0.9), mask, rho, u)
    np.testing.assert_array_equal(oracle.init_equilibrium(box, mask, rho, u),
                                  oracle.apply_open_faces(box, plain, mask))


def test_face_rules_need_one_axis():
    with pytest.raises(ValueError):
        oracle.Box(5, 6, 4, periodic=(0, 0, 1), open_faces={"-x": (1.0, (0, 0, 0), "neumann"),
                                                            "+y": (1.0, (0, 0, 0))})
    with pytest.raises(ValueError):
        oracle.Box(2, 6, 4, periodic=(0, 1, 1), open_faces={"-x": (1.0, (0, 0, 0), "zou_he_pressure")})


def test_face_rules_close_mass_and_momentum_budget():
    # per step: the box loses the post-collision populations on links leaving
    # through the open faces and gains the entering populations the rules set
    # (read from the new state); with walls on y and solids inside, the
    # exchanged force is the rest of the momentum change
    F = (1e-4, 0.0, 2e-5)
    faces = {"-x": (1.0, (0.03, 0.0, 0.01), "zou_he_velocity"), "+x": (0.995, (0.0, 0.0, 0.0), "zou_he_pressure")}
    box = oracle.Box(9, 6, 5, periodic=(0, 0, 1), tau=0.75, force=F, open_faces=faces)
    mask = li.random_mask(9, 6, 5, fraction=0.12, seed=61)
    nf = int(np.count_nonzero(mask == 0))
    c, _, _ = oracle.lattice()
    rho, u = li.random_fields(9, 6, 5, seed=62)
    f = oracle.init_equilibrium(box, mask, rho, u)
    solid = mask.reshape(5, 6, 9).astype(bool)
    for _ in range(3):
        m0 = oracle.totals(box, f, mask)
        fx = oracle.momentum_exchange(box, f, mask)
        f1 = oracle.run(box, f, 1, mask)
        gain_m, gain_p = 0.0, np.zeros(3)
        fz, f1z = f.reshape(19, 5, 6, 9), f1.reshape(19, 5, 6, 9)
        for z in range(5):
            for y in range(6):
                for x, side in ((0, 1), (8, -1)):
                    if solid[z, y, x]:
                        continue
                    post = oracle.collide(box, fz[:, z, y, x])
                    for q in range(19):
                        beyond_wall = (y == 0 and c[q][1] == 1) or (y == 5 and c[q][1] == -1)
                        if c[q][0] == side and not beyond_wall:      # enters through the face
                            gain_m += f1z[q, z, y, x]
                            gain_p += f1z[q, z, y, x] * c[q]
                        leaves_wall = (y == 0 and c[q][1] == -1) or (y == 5 and c[q][1] == 1)
                        if c[q][0] == -side and not leaves_wall:     # leaves through it
                            gain_m -= post[q]
                            gain_p -= post[q] * c[q]
        m1 = oracle.totals(box, f1, mask)
        assert abs(m1["mass"] - m0["mass"] - gain_m) < 1e-13 * m0["mass"]
        want_p = gain_p + nf * np.array(F) - fx["solid"] - fx["wall"]
        np.testing.assert_allclose(m1["momentum"] - m0["momentum"], want_p, rtol=0, atol=1e-13 * m0["mass"])
        f = f1


def test_pressure_driven_channel():
    # Zou-He pressure faces at both ends of a walled channel drive Poiseuille
    # flow.  At steady state the density falls linearly by (rho_in - rho_out)
    # over the nx - 1 links between the two face layers, and every column
    # carries the profile that the same force density G = c_s^2 drho/dx gives
    # under halfway bounce-back: the parabola G y'(H - y') / (2 nu rho) plus
    # the constant slip G (16 (tau - 1/2)^2 - 3) / (24 nu rho) (the closed form
    # of the forced channel pin above), up to compressibility, O(drho)
    nx, ny, tau = 32, 10, 0.8
    rin, rout = 1.0015, 0.9985
    faces = {"-x": (rin, (0.0, 0.0, 0.0), "zou_he_pressure"), "+x": (rout, (0.0, 0.0, 0.0), "zou_he_pressure")}
    box = oracle.Box(nx, ny, 1, periodic=(0, 0, 1), tau=tau, open_faces=faces)
    f = oracle.run(box, oracle.init_equilibrium(box), 4000)
    rho, u = oracle.moments(box, f)
    rho, ux = rho.reshape(ny, nx), u[0].reshape(ny, nx)
    nu = (tau - 0.5) / 3.0
    slip = (16.0 * (tau - 0.5) ** 2 - 3.0) / (24.0 * nu)
    yp = np.arange(ny) + 0.5
    for m in (8, 16, 24):
        grad = (rho[:, m - 1].mean() - rho[:, m + 1].mean()) / 2.0
        assert abs(grad / ((rin - rout) / (nx - 1)) - 1.0) < 1e-3
        G, r = grad / 3.0, rho[:, m].mean()
        want = G * yp * (ny - yp) / (2.0 * nu * r) + G * slip / r
        assert np.max(np.abs(ux[:, m] - want)) < 3e-4 * want.max()
    assert np.max(np.abs(u[1].reshape(ny, nx)[:, 8:25])) < 1e-3 * ux.max()  # away from the entrance regions


# ------------------------------------------------ P5 / P6 streaming exactness

def _brute_stream(box, f, mask):
    """Streaming by exhaustive search: the value arriving at x along c_q comes
    from the cell y with y + c_q == x (wrapping only on periodic axes)."""
    c, _, opp = oracle.lattice()
    dims = (box.nx, box.ny, box.nz)
    cells = [(x, y, z) for z in range(box.nz) for y in range(box.ny) for x in range(box.nx)]
    lin = {p: i for i, p in enumerate(cells)}
    out = np.zeros_like(f)
    for xi, xp in enumerate(cells):
        if mask is not None and mask[xi]:
            continue
        for q in range(Q):
            src = None
            for yi, yp in enumerate(cells):
                ok = True
                for a in range(3):
                    t = yp[a] + c[q][a]
                    if box.periodic[a]:
                        t %= dims[a]
                    if t != xp[a]:
                        ok = False
                        break
                if ok:
                    src = yi
                    break
            if src is None or (mask is not None and mask[src]):
                out[q, xi] = f[opp[q], xi]
            else:
                out[q, xi] = f[q, src]
    del lin
    return out


@pytest.mark.parametrize("periodic,with_mask", [((1, 1, 1), False), ((1, 0, 1), False),
                                                ((1, 1, 1), True), ((0, 1, 0), True)])
def test_streaming_matches_brute_force_4cubed(periodic, with_mask):
    box = oracle.Box(4, 4, 4, periodic=periodic, tau=math.inf)   # omega = 0: no collision
    rng = np.random.default_rng(123)
    mask = li.random_mask(4, 4, 4, fraction=0.3, seed=9) if with_mask else None
    f = rng.uniform(0.01, 1.0, size=(Q, box.n))
    if mask is not None:
        f[:, mask.astype(bool)] = 0.0
    got = oracle.run(box, f, 1, mask)
    want = _brute_stream(box, f, mask)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("periodic", [(1, 1, 1), (0, 1, 1), (0, 0, 0)])
def test_streaming_is_permutation(periodic):
    box = oracle.Box(6, 5, 4, periodic=periodic, tau=math.inf)
    mask = li.random_mask(6, 5, 4, fraction=0.2, seed=2)
    rng = np.random.default_rng(5)
    f = rng.uniform(0.0, 1.0, size=(Q, box.n))
    f[:, mask.astype(bool)] = 0.0
    g = oracle.run(box, f, 1, mask)
    fl = ~mask.astype(bool)
    assert np.array_equal(np.sort(f[:, fl].ravel()), np.sort(g[:, fl].ravel()))
    h = oracle.run(box, f, 7, mask)
    assert np.array_equal(np.sort(f[:, fl].ravel()), np.sort(h[:, fl].ravel()))


# --------------------------------------------------------- P8 uniform state

def test_uniform_state_invariant():
    box = oracle.Box(5, 4, 6, tau=0.7, force=(0, 0, 0))
    rho = np.full(box.n, 1.02)
    u = np.tile(np.array([[0.03], [-0.01], [0.02]]), (1, box.n))
    f0 = oracle.init_equilibrium(box, None, rho, u)
    f1 = oracle.run(box, f0, 10)
    assert np.max(np.abs(f1 - f0)) < 1e-15


# ------------------------------------------- P4 Poiseuille: closed form + slip

def _poiseuille(tau, steps, g=1e-6, H=64):
    box = oracle.Box(1, H, 1, periodic=(1, 0, 1), tau=tau, force=(0.0, 0.0, g))
    f = oracle.init_equilibrium(box)
    f = oracle.run(box, f, steps)
    _, u = oracle.moments(box, f)
    nu = (tau - 0.5) / 3.0
    yp = np.arange(H) + 0.5          # distance from the wall plane at y = -1/2
    exact = g * yp * (H - yp) / (2.0 * nu)
    return u[2], exact, u[0], u[1]


def test_poiseuille_gate():
    # the benchmark channel: H = 64, tau = 0.9, g = 1e-6 along z, from rest.
    # After 40000 steps the start-up transient is ~3e-6 of u_max.
    uz, exact, ux, uy = _poiseuille(0.9, 40000, g=1e-6, H=64)
    assert np.max(np.abs(ux)) == 0.0 and np.max(np.abs(uy)) < 1e-11 * exact.max()
    assert np.max(np.abs(uz - exact)) / exact.max() < 1e-3


@pytest.mark.parametrize("tau", [0.9, 0.6, 1.4])
def test_poiseuille_bounce_back_slip(tau):
    # Steady BGK + Guo + halfway bounce-back reproduces the parabola plus a
    # constant slip u_s = g (16 L - 3) / (24 nu), L = (tau - 1/2)^2.  A narrow
    # channel (H = 16) lets the transient die out to rounding level.
    g, H = 1e-6, 16
    nu = (tau - 0.5) / 3.0
    steps = int(40.0 * H * H / (math.pi ** 2 * nu))
    uz, exact, _, _ = _poiseuille(tau, steps, g=g, H=H)
    lam = (tau - 0.5) ** 2
    slip = g * (16 * lam - 3) / (24 * nu)
    np.testing.assert_allclose(uz - exact, np.full_like(uz, slip), rtol=0, atol=1e-9 * exact.max())


def test_poiseuille_exact_at_magic_tau():
    # halfway bounce-back places the wall exactly at the link midpoint when
    # (tau - 1/2)^2 = 3/16, so the steady profile is the parabola itself.
    tau, H = 0.5 + math.sqrt(3.0 / 16.0), 16
    nu = (tau - 0.5) / 3.0
    uz, exact, _, _ = _poiseuille(tau, int(40.0 * H * H / (math.pi ** 2 * nu)), H=H)
    assert np.max(np.abs(uz - exact)) < 1e-9 * exact.max()


# ------------------------------------------------ P9 / P10 decaying flows

def test_shear_wave_decay():
    tau, L, A, t = 0.8, 32, 1e-4, 200
    box = oracle.Box(1, L, 1, tau=tau)
    rho, u = li.shear_wave(1, L, 1, amp=A)
    f = oracle.run(box, oracle.init_equilibrium(box, None, rho, u), t)
    _, uu = oracle.moments(box, f)
    s = np.sin(2 * np.pi * np.arange(L) / L)
    amp = (uu[2] @ s) / (s @ s)
    nu = (tau - 0.5) / 3.0
    k = 2 * np.pi / L
    assert abs(amp / A - math.exp(-nu * k * k * t)) < 0.01 * math.exp(-nu * k * k * t)


def _tgv_rate_error(n, tau=0.6, u0=1e-3):
    """Relative error of the measured kinetic-energy decay exponent against
    the Navier-Stokes law E(t)/E(0) = exp(-6 nu k^2 t), |K|^2 = 3 k^2, over a
    fixed nu k^2 t (100 steps at n = 32)."""
    box = oracle.Box(n, n, n, tau=tau)
    nu = (tau - 0.5) / 3.0
    k = 2 * np.pi / n
    t = int(round(100 * (n / 32) ** 2))
    rho, u = li.taylor_green(n, u0=u0)
    f0 = oracle.init_equilibrium(box, None, rho, u)
    e0 = oracle.totals(box, f0)["ke"]
    e1 = oracle.totals(box, oracle.run(box, f0, t))["ke"]
    return math.log(e1 / e0) / (-6.0 * nu * k * k * t) - 1.0


def test_taylor_green_low_amplitude_decay():
    # Low amplitude (Re = u0/(nu k) ~ 0.15) so the nonlinear term is negligible:
    # the decay exponent must approach 6 nu k^2 at second order in k.
    e16, e32 = _tgv_rate_error(16), _tgv_rate_error(32)
    assert abs(e32) < 0.04
    assert 3.6 < e16 / e32 < 4.4


# ------------------------------------------------- consistency of helpers

_STEP_CELLS_FACES = [
    None,
    {"-y": (1.01, (0.0, 0.02, 0.01)), "+y": (0.99, (0.01, 0.0, -0.02))},
    {"-y": (1.0, (0.0, 0.03, 0.0), "zou_he_velocity"), "+y": (0.995, (0.0, 0.0, 0.0), "zou_he_pressure")},
    {"-y": (1.0, (0.01, 0.02, 0.0), "neumann"), "+y": (1.0, (0.0, 0.0, 0.0), "zou_he_pressure")},
    {"-y": (1.02, (0.0, 0.0, 0.0), "zou_he_pressure"), "+y": (1.0, (0.0, -0.01, 0.01), "zou_he_velocity")},
    {"+y": (1.0, (0.0, 0.0, 0.0), "neumann")},
]


@pytest.mark.parametrize("faces", _STEP_CELLS_FACES)
def test_step_cells_equals_run(faces):
    # one step evaluated cell by cell (the checker of the full-size sampled
    # GPU steps) equals the whole-box step, with walls, solids, a body force
    # and open faces of every kind (reservoirs, Zou-He, Neumann); the face
    # rules read the inward cell's new state, which step_cells recomputes
    box = oracle.Box(6, 5, 7, periodic=(1, 0, 1), tau=0.7, force=(2e-5, 0, -1e-5), open_faces=faces)
    mask = li.random_mask(6, 5, 7, fraction=0.2, seed=8)
    rho, u = li.random_fields(6, 5, 7, seed=6, drho=0.02, du=0.04)
    f0 = oracle.init_equilibrium(box, mask, rho, u)
    rng = np.random.default_rng(6)
    f0 = f0 * (1.0 + 0.05 * rng.standard_normal(f0.shape))
    f0[:, mask.reshape(-1) != 0] = 0.0
    f1 = oracle.run(box, f0, 1, mask)
    cells = np.arange(box.n)
    got = oracle.step_cells(box, f0, cells, mask)
    assert np.array_equal(got.T, f1)
    # a random subset, in random order, gives the same rows
    sub = rng.permutation(box.n)[:57]
    assert np.array_equal(oracle.step_cells(box, f0, sub, mask), f1[:, sub].T)


def test_moments_and_totals_are_plain_sums():
    box = oracle.Box(5, 4, 3, tau=0.9, force=(1e-3, 2e-3, -1e-3))
    mask = li.random_mask(5, 4, 3, fraction=0.3, seed=1)
    f = _random_state(box, seed=2, mask=mask)
    c, _, _ = oracle.lattice()
    rho, u = oracle.moments(box, f, mask)
    fl = ~mask.astype(bool)
    r = f.sum(axis=0)
    j = c.T.astype(float) @ f
    np.testing.assert_allclose(rho[fl], r[fl], rtol=1e-15)
    np.testing.assert_allclose(u[:, fl], (j[:, fl] + 0.5 * np.array(box.force)[:, None]) / r[fl], rtol=1e-13)
    assert np.all(rho[~fl] == 0) and np.all(u[:, ~fl] == 0)
    tot = oracle.totals(box, f, mask)
    assert abs(tot["mass"] - f[:, fl].sum()) < 1e-12
