"""Seeded random configurations against the oracle: box sizes from 1 to 65
cells per axis (ragged, one-cell axes included, x spanning several tiles), random periodic axes, walls,
random solid masks, body forces, relaxation times and open faces of every
kind, run for a random odd or even number of steps on every layout and
scheme.  The canonical populations must match the oracle within 1e-5 (fp32)
or 1e-12 (fp64) and agree bit for bit across layouts and schemes."""
import numpy as np
import pytest

import lbm_inputs as li
import oracle
from gpu_util import LAYOUTS, SCHEMES, TOL, cast, host_f, make, need_gpu, say
from test_gpu_open_faces import _make_open

pytestmark = pytest.mark.gpu

FACE_NAMES = ("-x", "+x", "-y", "+y", "-z", "+z")
RULES = ("equilibrium", "neumann", "zou_he_pressure", "zou_he_velocity")


def random_config(seed):
    rng = np.random.default_rng(seed)
    while True:
        shape = tuple(int(v) for v in rng.choice([1, 2, 3, 5, 8, 13, 17, 20, 33, 47, 65], size=3))
        per = tuple(int(v) for v in rng.integers(0, 2, size=3))
        tau = float(rng.uniform(0.55, 1.3))
        F = tuple(float(v) for v in (rng.uniform(-2e-5, 2e-5, size=3) if rng.random() < 0.6 else (0.0, 0.0, 0.0)))
        mask = None
        if rng.random() < 0.7:
            mask = li.random_mask(*shape, fraction=float(rng.uniform(0.02, 0.3)), seed=int(rng.integers(1, 10_000)))
        faces = {}
        closed = [a for a in range(3) if not per[a]]
        if closed and rng.random() < 0.6:
            if rng.random() < 0.5:
                # reservoirs on any closed faces
                for a in closed:
                    for side in range(2):
                        if rng.random() < 0.5:
                            u = tuple(float(v) for v in rng.uniform(-0.03, 0.03, size=3))
                            faces[FACE_NAMES[2 * a + side]] = (float(rng.uniform(0.99, 1.01)), u)
            else:
                # face rules: all open faces on one axis at least 3 cells long
                a = int(rng.choice(closed))
                if shape[a] >= 3:
                    for side in range(2):
                        if rng.random() < 0.75:
                            u = tuple(float(v) for v in rng.uniform(-0.03, 0.03, size=3))
                            rule = str(rng.choice(RULES))
                            faces[FACE_NAMES[2 * a + side]] = (float(rng.uniform(0.99, 1.01)), u, rule)
        try:
            box = oracle.Box(*shape, periodic=per, tau=tau, force=F, open_faces=faces)
        except ValueError:
            continue
        nsteps = int(rng.integers(1, 13))
        return shape, per, tau, F, mask, faces, box, nsteps


@pytest.mark.parametrize("seed", range(120))
def test_random_config(seed):
    need_gpu()
    precision = "f32" if seed % 2 == 0 else "f64"
    shape, per, tau, F, mask, faces, box, nsteps = random_config(1000 + seed)
    rho, u = li.random_fields(*shape, seed=seed + 7)
    rho, u = cast(rho, precision), cast(0.3 * u, precision)
    f0 = oracle.init_equilibrium(box, mask, rho, u)
    want = oracle.run(box, f0, nsteps, mask)
    ref = None
    for layout in LAYOUTS:
        for scheme in SCHEMES:
            say("random", seed, precision, shape, "periodic", per, "faces", sorted(faces), "steps", nsteps, layout,
                scheme)
            if faces:
                lat = _make_open(shape, precision, layout, scheme, tau, F, faces, mask, per, rho, u)
            else:
                lat = make(shape, precision, layout, scheme, tau=tau, force=F, mask=mask, periodic=per, rho=rho, u=u)
            lat.step(nsteps)
            got = host_f(lat)
            err = np.max(np.abs(got - want))
            say("  max-abs", err)
            assert err <= TOL[precision], (layout, scheme, err)
            if ref is None:
                ref = got
            else:
                assert np.array_equal(got, ref), (layout, scheme, "differs from", LAYOUTS[0], SCHEMES[0])
