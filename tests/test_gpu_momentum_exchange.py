"""Momentum exchange with the solids on the GPU (lbm_momentum_exchange through
the C ABI) against the oracle's orc_momentum_exchange, evaluated on the GPU's
own canonical state, and against the momentum budget of the following step."""
import numpy as np
import pytest
import torch

import lbm_inputs as li
import oracle
from gpu_util import LAYOUTS, SCHEMES, cast, host_moments, make, need_gpu, say
from test_gpu_parity import _case

pytestmark = pytest.mark.gpu


def exact_f(lat, precision, mask):
    """The GPU's state exactly, in float64: stored values s = f - w_T plus the
    weights rounded to the device precision, as the library defines f."""
    s = lat.save_state()
    torch.cuda.synchronize()
    dt = np.float32 if precision == "f32" else np.float64
    c, _, _ = oracle.lattice()
    n2 = (np.asarray(c) ** 2).sum(axis=1)
    w = np.where(n2 == 0, float(dt(1) / dt(3)), np.where(n2 == 1, float(dt(1) / dt(18)), float(dt(1) / dt(36))))
    f = s.double().cpu().numpy() + w[:, None]
    if mask is not None:
        f[:, mask.reshape(-1).astype(bool)] = 0.0
    return f


def _force(lat):
    solid, wall = lat.momentum_exchange()
    torch.cuda.synchronize()
    return solid.cpu().numpy(), wall.cpu().numpy()


@pytest.mark.parametrize("precision", ["f32", "f64"])
@pytest.mark.parametrize("name", ["sphere_force", "channel", "porous", "closed_box"])
def test_force_matches_oracle_all_layouts_schemes(name, precision):
    need_gpu()
    shape, per, tau, F, mask = _case(name)
    rho, u = li.random_fields(*shape, seed=21)
    rho, u = cast(rho, precision), cast(u, precision)
    box = oracle.Box(*shape, periodic=per, tau=tau, force=F)
    n = int(np.prod(shape))
    atol = (4e-9 if precision == "f32" else 1e-15) * n
    results = {}
    for layout in LAYOUTS:
        for scheme in SCHEMES:
            lat = make(shape, precision, layout, scheme, tau=tau, force=F, mask=mask, periodic=per, rho=rho, u=u)
            for steps in (7, 1):  # t = 7 then t = 8: both parities of the in-place scheme
                lat.step(steps)
                say("mex", name, precision, layout, scheme, "t =", lat.t)
                solid, wall = _force(lat)
                want = oracle.momentum_exchange(box, exact_f(lat, precision, mask), mask)
                err = max(np.max(np.abs(solid - want["solid"])), np.max(np.abs(wall - want["wall"])))
                say("  max-abs", err, "force", solid, wall)
                assert err <= atol, (layout, scheme, lat.t, err)
                if mask is None:
                    assert np.all(solid == 0.0)
                if all(per):
                    assert np.all(wall == 0.0)
                results.setdefault(lat.t, {})[(layout, scheme)] = np.concatenate([solid, wall])
    # the dense layouts share the cell-to-workgroup mapping and so the order of
    # the sums: bit-identical; the compact layout sums per fluid cell, in
    # another order: equal to rounding
    for t, r in results.items():
        ref = r[("stream", "ab")]
        for k, v in r.items():
            if k[0] == "compact":
                assert np.max(np.abs(v - ref)) <= 1e-15 * n, f"t={t}: {k} differs from stream/ab"
            else:
                assert np.array_equal(v, ref), f"t={t}: {k} differs from stream/ab"


@pytest.mark.parametrize("layout,scheme", [("compact", "aa"), ("stream", "ab"), ("bundle", "aa"), ("compact", "eso"),
                                           ("collision", "eso"), ("compact", "twist"), ("stream", "twist")])
def test_force_closes_momentum_budget_fp64(layout, scheme):
    # P(t+1) - P(t) = N_fluid F - F_solid - F_wall over the step the force was
    # taken for (P = sum of rho u over fluid cells, u including F/2)
    need_gpu()
    shape, per, tau, F, mask = _case("closed_box")
    rho, u = li.random_fields(*shape, seed=5)
    lat = make(shape, "f64", layout, scheme, tau=tau, force=F, mask=mask, periodic=per, rho=rho, u=u)
    nf = int(np.count_nonzero(mask == 0))
    lat.step(3)
    for _ in range(2):
        say("budget", layout, scheme, "t =", lat.t)
        solid, wall = _force(lat)
        r0, u0 = host_moments(lat)
        lat.step(1)
        r1, u1 = host_moments(lat)
        dp = (r1 * u1).sum(axis=1) - (r0 * u0).sum(axis=1)
        want = nf * np.array(F) - solid - wall
        assert np.max(np.abs(solid)) > 1e-6
        np.testing.assert_allclose(dp, want, rtol=0, atol=1e-12 * r0.sum())


def test_sphere128_force_full_size():
    # the 128^3 sphere benchmark shape after 200 forced steps, in place and
    # compact as timed: GPU force against the oracle on the same state
    need_gpu()
    mask = li.sphere_mask(128, radius=16)
    box = oracle.Box(128, 128, 128, tau=0.7, force=(1e-6, 0.0, 0.0))
    for layout in ("compact", "stream"):
        say("sphere128 mex", layout)
        lat = make((128, 128, 128), "f32", layout, "aa", tau=0.7, force=(1e-6, 0.0, 0.0), mask=mask)
        lat.step(200)
        solid, wall = _force(lat)
        want = oracle.momentum_exchange(box, exact_f(lat, "f32", mask), mask)
        say("  gpu", solid, "oracle", want["solid"])
        assert np.all(wall == 0.0)
        # the drag grows from zero toward the body force on the fluid
        nf = int(np.count_nonzero(mask == 0))
        assert 0.0 < solid[0] < nf * 1e-6
        assert np.max(np.abs(solid - want["solid"])) <= 1e-6 * abs(want["solid"][0]) + 1e-8
