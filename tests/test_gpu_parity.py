"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: canonical populations within max-abs 1e-5 (fp32) / 1e-12 (fp64) after
100 steps from the same seeded inputs; indexing, masks and streaming bit-exact
(collision-free mode); every layout and scheme bit-identical to one another.
"""
import math

import numpy as np
import pytest

import lbm_inputs as li
import oracle
from gpu_util import LAYOUTS, SCHEMES, TOL, cast, host_f, host_moments, make, need_gpu, say

pytestmark = pytest.mark.gpu
Q = 19
_ORACLE_CACHE = {}


def _oracle_run(key, box, mask, rho, u, n):
    if key not in _ORACLE_CACHE:
        f0 = oracle.init_equilibrium(box, mask, rho, u)
        _ORACLE_CACHE[key] = oracle.run(box, f0, n, mask)
    return _ORACLE_CACHE[key]


# --------------------------------------------------------------- C1 in full

@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("scheme", SCHEMES)
def test_c1_random_periodic_32cubed(layout, scheme):
    """32^3 periodic, tau = 0.8, no force, seeded random rho/u, 100 steps."""
    need_gpu()
    say("c1", layout, scheme)
    rho, u = li.random_fields(32, 32, 32, seed=1)
    rho, u = cast(rho, "f32"), cast(u, "f32")
    box = oracle.Box(32, 32, 32, tau=0.8)
    want = _oracle_run(("c1",), box, None, rho, u, 100)
    lat = make((32, 32, 32), "f32", layout, scheme, tau=0.8, rho=rho, u=u)
    lat.step(100)
    got = host_f(lat)
    err = np.max(np.abs(got - want))
    say("c1 max-abs", err)
    assert err <= TOL["f32"]


# ------------------------------------------- small ragged boxes, all physics

def _case(name):
    if name == "sphere_force":
        shape, per, tau, F = (37, 29, 23), (1, 1, 1), 0.7, (1e-5, 0.0, 0.0)
        mask = li.sphere_mask(37, 29, 23, radius=6)
    elif name == "channel":
        shape, per, tau, F = (24, 20, 33), (1, 0, 1), 0.9, (0.0, 0.0, 1e-5)
        mask = None
    elif name == "porous":
        shape, per, tau, F = (40, 36, 28), (1, 1, 1), 0.65, (1e-5, 0.0, 0.0)
        mask, _ = li.porous_mask(40, 36, 28, n_spheres=12, seed=5, rmin=2.0, rmax=4.0)
    elif name == "closed_box":
        shape, per, tau, F = (19, 17, 13), (0, 0, 0), 0.6, (2e-5, -1e-5, 1e-5)
        mask = li.random_mask(19, 17, 13, fraction=0.15, seed=7)
    else:
        raise KeyError(name)
    return shape, per, tau, F, mask


@pytest.mark.parametrize("precision", ["f32", "f64"])
@pytest.mark.parametrize("name,nsteps", [("sphere_force", 100), ("channel", 101), ("porous", 100),
                                         ("closed_box", 101)])
def test_small_boxes_all_layouts_schemes(name, nsteps, precision):
    need_gpu()
    shape, per, tau, F, mask = _case(name)
    rho, u = li.random_fields(*shape, seed=11)
    rho, u = cast(rho, precision), cast(u, precision)
    box = oracle.Box(*shape, periodic=per, tau=tau, force=F)
    want = _oracle_run((name, precision, nsteps), box, mask, rho, u, nsteps)
    results = {}
    for layout in LAYOUTS:
        for scheme in SCHEMES:
            say(name, precision, layout, scheme, nsteps)
            lat = make(shape, precision, layout, scheme, tau=tau, force=F, mask=mask, periodic=per, rho=rho, u=u)
            lat.step(nsteps)
            assert lat.t == nsteps
            got = host_f(lat)
            err = np.max(np.abs(got - want))
            say("  max-abs", err)
            assert err <= TOL[precision], (layout, scheme, err)
            if mask is not None:
                assert np.all(got[:, mask.astype(bool)] == 0.0)
            results[(layout, scheme)] = got
    ref = results[("stream", "ab")]
    for k, v in results.items():
        assert np.array_equal(v, ref), f"{k} differs from stream/ab"


# ------------------------------------------ streaming bit-exact (omega = 0)

@pytest.mark.parametrize("precision", ["f32", "f64"])
@pytest.mark.parametrize("nsteps", [1, 2, 3])
def test_collision_free_streaming_bit_exact(precision, nsteps):
    """tau = inf makes collision the identity; GPU streaming + bounce-back must
    then move values exactly as the oracle does, from the GPU's own f(0)."""
    need_gpu()
    shape, per = (21, 18, 11), (1, 0, 1)
    mask = li.random_mask(*shape, fraction=0.2, seed=3)
    rho, u = li.random_fields(*shape, seed=4)
    rho, u = cast(rho, precision), cast(u, precision)
    box = oracle.Box(*shape, periodic=per, tau=math.inf)
    f0_oracle = oracle.init_equilibrium(box, mask, rho, u)
    for layout in LAYOUTS:
        for scheme in SCHEMES:
            say("omega0", precision, nsteps, layout, scheme)
            lat = make(shape, precision, layout, scheme, tau=math.inf, mask=mask, periodic=per, rho=rho, u=u)
            f0 = host_f(lat)
            rel = 4e-7 if precision == "f32" else 1e-15
            assert np.max(np.abs(f0 - f0_oracle)) <= rel * np.max(np.abs(f0_oracle))
            lat.step(nsteps)
            got = host_f(lat)
            want = oracle.run(box, f0, nsteps, mask)
            assert np.array_equal(got, want), (layout, scheme)


# --------------------------------------------------- state transfer paths

@pytest.mark.parametrize("precision", ["f32", "f64"])
@pytest.mark.parametrize("shape", [(37, 21, 11), (20, 9, 5), (257, 3, 2), (1, 6, 5)])
def test_collision_free_streaming_periodic_bit_exact(shape, precision):
    """The same on fully periodic boxes without a mask (where the dense AoS
    and SoAoS layouts move three slots per lane and shift values between
    lanes): one to three collision-free steps equal the oracle's streaming
    bit for bit, in every layout and scheme."""
    need_gpu()
    rho, u = li.random_fields(*shape, seed=5)
    rho, u = cast(rho, precision), cast(u, precision)
    box = oracle.Box(*shape, periodic=(1, 1, 1), tau=math.inf)
    for layout in LAYOUTS:
        for scheme in SCHEMES:
            say("omega0 periodic", shape, precision, layout, scheme)
            lat = make(shape, precision, layout, scheme, tau=math.inf, rho=rho, u=u)
            f = host_f(lat)
            for _ in range(3):
                lat.step(1)
                got = host_f(lat)
                want = oracle.run(box, f, 1)
                assert np.array_equal(got, want), (layout, scheme, lat.t)
                f = got


@pytest.mark.parametrize("precision", ["f32", "f64"])
def test_write_read_roundtrip_both_parities(precision):
    """Lattice states (f_q within a factor 2 of w_q) round-trip bit for bit;
    arbitrary values within one unit in the last place of max(|f_q|, w_q)."""
    need_gpu()
    shape, per = (33, 9, 14), (0, 1, 1)
    mask = li.random_mask(*shape, fraction=0.25, seed=9)
    n = int(np.prod(shape))
    rho, u = li.random_fields(*shape, seed=2, drho=0.05, du=0.08)
    box = oracle.Box(*shape, periodic=per, tau=0.7)
    lattice_state = cast(oracle.init_equilibrium(box, mask, rho, u), precision).astype(np.float64)
    rng = np.random.default_rng(2)
    arbitrary = cast(rng.uniform(0.0, 0.5, size=(Q, n)), precision).astype(np.float64)
    arbitrary[:, mask.astype(bool)] = 0.0
    ftype = np.float32 if precision == "f32" else np.float64
    for layout in LAYOUTS:
        for scheme in SCHEMES:
            for pre_steps in (0, 1):
                say("roundtrip", precision, layout, scheme, pre_steps)
                lat = make(shape, precision, layout, scheme, tau=0.7, mask=mask, periodic=per)
                lat.step(pre_steps)
                lat.write_populations(cast(lattice_state, precision))
                assert np.array_equal(host_f(lat), lattice_state), (layout, scheme, pre_steps)
                lat.write_populations(cast(arbitrary, precision))
                got = host_f(lat)
                _, w, _ = oracle.lattice()
                big = np.maximum(np.abs(arbitrary), w[:, None]).astype(ftype)
                ulp = np.spacing(big).astype(np.float64)
                assert np.all(np.abs(got - arbitrary) <= ulp), (layout, scheme, pre_steps)


@pytest.mark.parametrize("precision", ["f32", "f64"])
def test_moments_match_oracle(precision):
    need_gpu()
    shape, per, F = (26, 22, 17), (1, 1, 0), (3e-5, 1e-5, -2e-5)
    mask = li.sphere_mask(*shape, radius=5)
    rho, u = li.random_fields(*shape, seed=12)
    box = oracle.Box(*shape, periodic=per, tau=0.75, force=F)
    for layout in LAYOUTS:
        for scheme in SCHEMES:
            lat = make(shape, precision, layout, scheme, tau=0.75, force=F, mask=mask, periodic=per,
                       rho=cast(rho, precision), u=cast(u, precision))
            lat.step(7)
            f = host_f(lat)
            r_gpu, u_gpu = host_moments(lat)
            r_or, u_or = oracle.moments(box, f, mask)
            tol = 1e-6 if precision == "f32" else 1e-14
            assert np.max(np.abs(r_gpu - r_or)) <= tol
            assert np.max(np.abs(u_gpu - u_or)) <= tol
            solid = mask.astype(bool)
            assert np.all(r_gpu[solid] == 0) and np.all(u_gpu[:, solid] == 0)


def test_checkpoint_resume_bit_exact():
    """n steps, save_state, load into a fresh handle (another layout), n steps
    == 2n steps bit for bit; through canonical populations, within rounding."""
    need_gpu()
    shape, per, F = (30, 20, 10), (1, 1, 1), (1e-5, 0.0, 0.0)
    mask = li.sphere_mask(*shape, radius=4)
    rho, u = li.random_fields(*shape, seed=21)
    rho, u = cast(rho, "f32"), cast(u, "f32")
    for scheme in SCHEMES:
        full = make(shape, "f32", "stream", scheme, tau=0.7, force=F, mask=mask, rho=rho, u=u)
        full.step(10)
        want = host_f(full)
        half = make(shape, "f32", "stream", scheme, tau=0.7, force=F, mask=mask, rho=rho, u=u)
        half.step(5)
        snap = half.save_state().clone()
        pops = half.read_populations().clone()
        for other in ("bundle", "compact"):
            resumed = make(shape, "f32", other, scheme, tau=0.7, force=F, mask=mask)
            resumed.load_state(snap)
            resumed.step(5)
            assert np.array_equal(host_f(resumed), want), other
        approx = make(shape, "f32", "collision", scheme, tau=0.7, force=F, mask=mask)
        approx.write_populations(pops)
        approx.step(5)
        assert np.max(np.abs(host_f(approx) - want)) <= 1e-6


# ----------------------------------- full-size boxes: sampled one-step checks

def _sample_cells(mask, shape, k, seed):
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    cells = rng.choice(n, size=min(k, n), replace=False)
    if mask is not None:
        # add fluid cells with a solid cell at one of the 18 lattice offsets
        # (where bounce-back acts), periodic wrap on the 3-D mask
        nx, ny, nz = shape
        m = mask.astype(bool).reshape(nz, ny, nx)
        hit = np.zeros_like(m)
        for dz, dy, dx in [(dz, dy, dx) for dz in (-1, 0, 1) for dy in (-1, 0, 1) for dx in (-1, 0, 1)
                           if 0 < dx * dx + dy * dy + dz * dz <= 2]:
            hit |= np.roll(m, (dz, dy, dx), axis=(0, 1, 2))
        near = np.nonzero((hit & ~m).reshape(-1))[0]
        if near.size:
            cells = np.concatenate([cells, rng.choice(near, size=min(2048, near.size), replace=False)])
    return np.unique(cells).astype(np.int64)


def _full_size(name):
    if name == "tgv128":
        shape, per, tau, F, mask = (128, 128, 128), (1, 1, 1), 0.6, (0, 0, 0), None
        rho, u = li.taylor_green(128, u0=0.04)
        return shape, per, tau, F, mask, rho, u, "f32"
    if name == "sphere128":
        return (128, 128, 128), (1, 1, 1), 0.7, (1e-6, 0, 0), li.sphere_mask(128, radius=16), None, None, "f32"
    if name == "channel_f64":
        return (64, 64, 256), (1, 0, 1), 0.9, (0, 0, 1e-6), None, None, None, "f64"
    if name == "porous256":
        mask, _ = li.porous_mask(256)
        return (256, 256, 256), (1, 1, 1), 0.65, (1e-6, 0, 0), mask, None, None, "f32"
    raise KeyError(name)


@pytest.mark.parametrize("name,layout,scheme", [
    ("tgv128", "stream", "aa"), ("tgv128", "stream", "ab"),
    ("sphere128", "stream", "aa"), ("sphere128", "bundle", "aa"), ("sphere128", "collision", "aa"),
    ("sphere128", "compact", "aa"), ("channel_f64", "compact", "ab"), ("porous256", "compact", "aa"),
    ("porous256", "compact", "ab"),
    ("channel_f64", "stream", "aa"), ("channel_f64", "stream", "ab"),
    ("porous256", "stream", "aa"), ("porous256", "stream", "ab"),
    ("porous256", "compact", "eso"), ("porous256", "stream", "eso"), ("sphere128", "collision", "eso"),
    ("channel_f64", "bundle", "eso"), ("porous256", "compact", "twist"), ("porous256", "stream", "twist"),
    ("sphere128", "collision", "twist"), ("channel_f64", "bundle", "twist")])
def test_full_size_sampled_steps(name, layout, scheme):
    """At the benchmark sizes: advance a few steps, then check two consecutive
    steps (odd -> even and even -> odd for AA) at sampled cells against the
    oracle evaluated from the GPU's own state."""
    need_gpu()
    shape, per, tau, F, mask, rho, u, prec = _full_size(name)
    say("full-size", name, layout, scheme)
    lat = make(shape, prec, layout, scheme, tau=tau, force=F, mask=mask, periodic=per,
               rho=cast(rho, prec), u=cast(u, prec))
    box = oracle.Box(*shape, periodic=per, tau=tau, force=F)
    n = int(np.prod(shape))
    cells = _sample_cells(mask, shape, 4096, seed=sum(name.encode()))
    lat.step(5)
    prev = host_f(lat)
    for _ in range(2):
        lat.step(1)
        cur = host_f(lat)
        want = oracle.step_cells(box, prev, cells, mask)
        err = np.max(np.abs(cur[:, cells].T - want))
        say("  one-step max-abs", err, "t =", lat.t)
        assert err <= (1e-6 if prec == "f32" else 1e-14)
        prev = cur
    del prev, cur


# --------------------------------------------- compact layout index tables

@pytest.mark.parametrize("periodic", [(1, 1, 1), (0, 1, 0), (1, 0, 1)])
def test_compact_tables_bit_exact(periodic):
    """The device-built tables of the compact layout equal a numpy construction:
    fluid cells ranked in cell order; halo cells hold their periodic image or
    the wall marker beyond a non-periodic face."""
    need_gpu()
    import torch
    shape = (37, 21, 13)
    nx, ny, nz = shape
    mask = li.random_mask(*shape, fraction=0.3, seed=17)
    lat = make(shape, "f32", "compact", "aa", tau=0.7, mask=mask, periodic=periodic)
    torch.cuda.synchronize()
    fluid = mask == 0
    nf = int(fluid.sum())
    assert lat.fluid_cells == nf
    rank = np.full(mask.size, 0xFFFFFFFF, np.uint64)
    rank[fluid] = np.arange(nf)
    px, py, pz = nx + 2, ny + 2, nz + 2
    gz, gy, gx = np.meshgrid(np.arange(pz) - 1, np.arange(py) - 1, np.arange(px) - 1, indexing="ij")
    ok = np.ones(gx.shape, bool)
    coords = []
    for g, n, per in ((gx, nx, periodic[0]), (gy, ny, periodic[1]), (gz, nz, periodic[2])):
        out = (g < 0) | (g >= n)
        if not per:
            ok &= ~out
        coords.append(np.mod(g, n))
    cell = coords[0] + nx * (coords[1] + ny * coords[2])
    # beyond a wall: the wall marker 0xFFFFFFFE (solid cells: 0xFFFFFFFF)
    want_idxp = np.where(ok, rank[cell], 0xFFFFFFFE).astype(np.uint32).reshape(-1)
    ws = lat.workspace.cpu().numpy().view(np.uint32)
    # header (256 B), then the row table, then idxp, then cellp (256-B aligned)
    rows_words = ((4 * ny * nz + 255) // 256 * 256) // 4
    off = 256 // 4 + rows_words
    got_idxp = ws[off:off + want_idxp.size]
    assert np.array_equal(got_idxp, want_idxp)
    cell_off = off + ((4 * want_idxp.size + 255) // 256 * 256) // 4
    pid = np.nonzero(want_idxp.reshape(pz, py, px)[1:-1, 1:-1, 1:-1].reshape(-1) != 0xFFFFFFFF)[0]
    zz, rem = np.divmod(pid, nx * ny)
    yy, xx = np.divmod(rem, nx)
    want_cellp = ((xx + 1) + px * (yy + 1) + px * py * (zz + 1)).astype(np.uint32)
    assert np.array_equal(ws[cell_off:cell_off + nf], want_cellp)


@pytest.mark.parametrize("periodic", [(1, 1, 1), (0, 1, 0), (1, 0, 1), (0, 0, 0)])
def test_twist_ghost_table_bit_exact(periodic):
    """The esoteric twist's stored-index table on the compact layout equals a
    numpy construction: fluid cells keep their rank; a non-fluid location from
    which one of the six offsets (x, y, z, xy, xz, yz) leads to a fluid cell,
    inside the box or below a low face that is not periodic, is a ghost
    numbered nf + (its rank among ghosts in padded-cell order); a periodic
    halo holds its image; anything else is 0xFFFFFFFF."""
    need_gpu()
    import torch
    shape = (23, 17, 11)
    nx, ny, nz = shape
    mask = li.random_mask(*shape, fraction=0.3, seed=29)
    lat = make(shape, "f32", "compact", "twist", tau=0.7, mask=mask, periodic=periodic)
    torch.cuda.synchronize()
    fluid = (mask == 0).reshape(nz, ny, nx)
    nf = int(fluid.sum())
    rank = np.full((nz, ny, nx), 0xFFFFFFFF, np.int64)
    rank[fluid] = np.arange(nf)
    dims = (nx, ny, nz)

    def is_fluid(x, y, z):
        p = [x, y, z]
        for a in range(3):
            if periodic[a]:
                p[a] %= dims[a]
            elif not 0 <= p[a] < dims[a]:
                return False
        return bool(fluid[p[2], p[1], p[0]])

    def candidate(v, a):
        return 0 <= v < dims[a] or (v == -1 and not periodic[a])

    offs = [(1, 0, 0), (0, 1, 0), (0, 0, 1), (1, 1, 0), (1, 0, 1), (0, 1, 1)]
    px, py, pz = nx + 2, ny + 2, nz + 2
    want = np.full((pz, py, px), 0xFFFFFFFF, np.int64)
    ng = 0
    for z in range(-1, nz + 1):
        for y in range(-1, ny + 1):
            for x in range(-1, nx + 1):
                if not (candidate(x, 0) and candidate(y, 1) and candidate(z, 2)):
                    continue
                if 0 <= x < nx and 0 <= y < ny and 0 <= z < nz and fluid[z, y, x]:
                    want[z + 1, y + 1, x + 1] = rank[z, y, x]
                elif not is_fluid(x, y, z) and any(is_fluid(x + a, y + b, z + c) for a, b, c in offs):
                    want[z + 1, y + 1, x + 1] = nf + ng
                    ng += 1
    # periodic halos: the entry of the cell with those coordinates wrapped
    for z in range(pz):
        for y in range(py):
            for x in range(px):
                q = [x, y, z]
                halo = False
                for a, n in enumerate(dims):
                    if periodic[a] and q[a] in (0, n + 1):
                        q[a] = n if q[a] == 0 else 1
                        halo = True
                if halo:
                    want[z, y, x] = want[q[2], q[1], q[0]]
    ws = lat.workspace.cpu().numpy().view(np.uint32)
    up = lambda b: (b + 255) // 256 * 256  # noqa: E731
    npad, n64 = px * py * pz, (nx * ny * nz + 63) // 64 * 64
    off = (256 + up(4 * ny * nz) + up(4 * npad) + 2 * up(4 * n64)) // 4
    got = ws[off:off + npad].astype(np.int64)
    assert np.array_equal(got, want.reshape(-1)), int(np.sum(got != want.reshape(-1)))
    say("twist ghosts", periodic, "fluid", nf, "ghosts", ng)


@pytest.mark.parametrize("layout,scheme", [("compact", "aa"), ("stream", "ab"), ("compact", "eso"),
                                           ("compact", "twist"), ("stream", "twist")])
def test_full_size_open_channel_sampled_steps(layout, scheme):
    """The 768 x 192 x 96 open channel at full size: equilibrium inlet on -x,
    Zou-He pressure outlet on +x, walls in y, periodic z, a cylinder of
    radius 20.  Two consecutive steps at sampled cells -- random ones, cells
    next to the cylinder, and cells of both open faces including their edges
    with the walls -- against the oracle evaluated from the GPU's own state."""
    need_gpu()
    import torch
    from lattice_boltzmann_cfd_d3q19_amd import Lattice
    nx, ny, nz, tau = 768, 192, 96, 0.56
    u_in = (0.05, 0.0, 0.0)
    faces = {"-x": (1.0, u_in), "+x": (1.0, (0.0, 0.0, 0.0), "zou_he_pressure")}
    mask = li.cylinder_mask(nx, ny, nz, 2 * 160, 2 * 96 + 1, 20)
    n = nx * ny * nz
    u = np.tile(np.array(u_in, np.float32)[:, None], (1, n))
    say("full-size open channel", layout, scheme)
    lat = Lattice(nx, ny, nz, precision="f32", layout=layout, scheme=scheme, tau=tau)
    lat.set_geometry(torch.from_numpy(mask), (0, 0, 1))
    lat.set_open_faces(faces)
    lat.init(None, torch.from_numpy(u))
    box = oracle.Box(nx, ny, nz, periodic=(0, 0, 1), tau=tau, open_faces=faces)
    rng = np.random.default_rng(7)
    cells = [_sample_cells(mask, (nx, ny, nz), 4096, seed=11)]
    for x in (0, nx - 1):
        y = np.concatenate([rng.integers(0, ny, 600), [0, ny - 1] * 20])
        z = rng.integers(0, nz, y.size)
        cells.append(x + nx * (y + ny * z))
    cells = np.unique(np.concatenate(cells)).astype(np.int64)
    lat.step(5)
    prev = host_f(lat)
    for _ in range(2):
        lat.step(1)
        cur = host_f(lat)
        want = oracle.step_cells(box, prev, cells, mask)
        err = np.max(np.abs(cur[:, cells].T - want))
        say("  one-step max-abs", err, "t =", lat.t, "cells", cells.size)
        assert err <= 1e-6
        prev = cur
    del prev, cur


def _degenerate(name):
    if name == "one_cell":
        return (1, 1, 1), (1, 1, 1), None                 # every neighbour is the cell itself
    if name == "x_thin":
        return (1, 5, 3), (1, 1, 1), None
    if name == "y_walls_one_cell":
        return (2, 1, 7), (1, 0, 1), None                 # walls on both sides of a 1-cell axis
    if name == "single_fluid":
        m = np.ones((1, 4, 3), np.uint8)
        m[0, 1, 2] = 0
        return (3, 4, 1), (1, 1, 1), m.reshape(-1)
    if name == "all_solid":
        return (5, 4, 3), (1, 0, 1), np.ones(60, np.uint8)
    if name == "ragged_257":
        return (257, 3, 2), (1, 0, 1), li.random_mask(257, 3, 2, fraction=0.2, seed=29)
    # periodic boxes without a mask: the dense layouts' row-bundled path, with
    # rows one cell longer than a 256-wide tile, rows ending inside a 64-wide
    # tile's second wave, and 32-wide tiles (two rows per wave)
    if name == "periodic_257":
        return (257, 3, 2), (1, 1, 1), None
    if name == "periodic_100":
        return (100, 5, 3), (1, 1, 1), None
    if name == "periodic_20":
        return (20, 7, 3), (1, 1, 1), None
    raise KeyError(name)


@pytest.mark.parametrize("precision", ["f32", "f64"])
@pytest.mark.parametrize("name", ["one_cell", "x_thin", "y_walls_one_cell", "single_fluid", "all_solid",
                                  "ragged_257", "periodic_257", "periodic_100", "periodic_20"])
def test_degenerate_boxes(name, precision):
    """Boxes with one-cell axes, a single fluid cell, no fluid at all, and a
    row one cell longer than the widest tile: every layout and scheme against
    the oracle after 7 steps, and all of them bit-identical."""
    need_gpu()
    shape, per, mask = _degenerate(name)
    tau, F = 0.75, (2e-5, -1e-5, 1e-5)
    rho, u = li.random_fields(*shape, seed=37)
    rho, u = cast(rho, precision), cast(u, precision)
    box = oracle.Box(*shape, periodic=per, tau=tau, force=F)
    f0 = oracle.init_equilibrium(box, mask, rho, u)
    want = oracle.run(box, f0, 7, mask)
    results = {}
    for layout in LAYOUTS:
        for scheme in SCHEMES:
            say("degenerate", name, precision, layout, scheme)
            lat = make(shape, precision, layout, scheme, tau=tau, force=F, mask=mask, periodic=per, rho=rho, u=u)
            lat.step(7)
            got = host_f(lat)
            err = np.max(np.abs(got - want))
            assert err <= TOL[precision], (layout, scheme, err)
            r, v = host_moments(lat)
            if mask is not None:
                solid = mask.reshape(-1) != 0
                assert np.all(got[:, solid] == 0.0) and np.all(r[solid] == 0.0) and np.all(v[:, solid] == 0.0)
            results[(layout, scheme)] = got
    ref = results[("stream", "ab")]
    for k, v in results.items():
        assert np.array_equal(v, ref), f"{k} differs from stream/ab"


_MASK512 = {}


def _porous512():
    if "m" not in _MASK512:
        _MASK512["m"] = li.porous_mask(512)[0]
    return _MASK512["m"]


def _neighbourhood(cells, shape):
    """The cells and their 18 neighbours (periodic wrap)."""
    nx, ny, nz = shape
    c, _, _ = oracle.lattice()
    x, y, z = cells % nx, (cells // nx) % ny, cells // (nx * ny)
    out = [cells]
    for q in range(19):
        out.append(((x + c[q][0]) % nx) + nx * (((y + c[q][1]) % ny) + ny * ((z + c[q][2]) % nz)))
    return np.unique(np.concatenate(out))


@pytest.mark.parametrize("layout,scheme", [("compact", "aa"), ("stream", "aa"), ("stream", "ab"),
                                           ("compact", "twist"), ("stream", "twist")])
def test_full_size_512_sampled_steps(layout, scheme):
    """The 512^3 porous medium (19,200 spheres, the large-footprint run): the
    dense layouts address up to 19 x 2^27 elements here, past 2^31, and the
    compact one 83 M fluid cells.  Two consecutive steps at sampled cells
    against the oracle, evaluated from the GPU's own state: the state is
    gathered on the GPU at the cells and their neighbours only, into an
    otherwise untouched (lazily allocated) host array."""
    need_gpu()
    import torch
    shape = (512, 512, 512)
    n = 512 ** 3
    mask = _porous512()
    tau, F = 0.65, (1e-6, 0.0, 0.0)
    say("full-size 512", layout, scheme)
    lat = make(shape, "f32", layout, scheme, tau=tau, force=F, mask=mask)
    box = oracle.Box(*shape, periodic=(1, 1, 1), tau=tau, force=F)
    cells = _sample_cells(mask, shape, 3000, seed=512)
    near = _neighbourhood(cells, shape)
    near_t = torch.from_numpy(near).cuda()
    cells_t = torch.from_numpy(cells).cuda()
    lat.step(5)
    for _ in range(2):
        prev = lat.read_populations()
        f = np.zeros((19, n), np.float64)           # pages are touched only where filled
        f[:, near] = prev.index_select(1, near_t).double().cpu().numpy()
        del prev
        lat.step(1)
        cur = lat.read_populations().index_select(1, cells_t).double().cpu().numpy()
        torch.cuda.synchronize()
        want = oracle.step_cells(box, f, cells, mask)
        err = np.max(np.abs(cur.T - want))
        say("  one-step max-abs", err, "t =", lat.t, "cells", cells.size)
        assert err <= 1e-6
        del f
    del lat
    torch.cuda.empty_cache()
