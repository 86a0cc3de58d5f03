"""Fused macroscopic output (lbm_step_moments): the density and velocity the
last step's collision used, written by that step, against lbm_moments taken
before it and against the oracle, for every layout, scheme and precision."""
import numpy as np
import pytest
import torch

import lbm_inputs as li
import oracle
from gpu_util import LAYOUTS, SCHEMES, cast, host_f, make, need_gpu, say
from test_gpu_parity import _case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("precision", ["f32", "f64"])
@pytest.mark.parametrize("name", ["sphere_force", "closed_box"])
def test_step_moments_equal_moments_before_last_step(name, precision):
    need_gpu()
    shape, per, tau, F, mask = _case(name)
    rho, u = li.random_fields(*shape, seed=41)
    rho, u = cast(rho, precision), cast(u, precision)
    box = oracle.Box(*shape, periodic=per, tau=tau, force=F)
    solid = mask.reshape(-1).astype(bool)
    for layout in LAYOUTS:
        for scheme in SCHEMES:
            for k in (5, 6):  # the last step even or odd in the in-place scheme
                say("step_moments", name, precision, layout, scheme, k)
                a = make(shape, precision, layout, scheme, tau=tau, force=F, mask=mask, periodic=per, rho=rho, u=u)
                b = make(shape, precision, layout, scheme, tau=tau, force=F, mask=mask, periodic=per, rho=rho, u=u)
                a.step(k - 1)
                r1, u1 = a.moments()
                f_prev = host_f(a)
                a.step(1)
                r2, u2 = b.step_moments(k)
                torch.cuda.synchronize()
                assert b.t == a.t == k
                r1, u1, r2, u2 = (x.double().cpu().numpy() for x in (r1, u1, r2, u2))
                assert np.array_equal(r2, r1) and np.array_equal(u2, u1)
                assert np.all(r2[solid] == 0.0) and np.all(u2[:, solid] == 0.0)
                assert np.array_equal(host_f(b), host_f(a))
                # and the oracle's moments of the same state f(k - 1)
                wr, wu = oracle.moments(box, f_prev, mask)
                tol = 1e-6 if precision == "f32" else 1e-13
                assert np.max(np.abs(r2 - wr)) <= tol and np.max(np.abs(u2 - wu)) <= tol


def _step_moments_into(lat, k, fill):
    """lbm_step_moments into outputs that start as `fill` everywhere."""
    from lattice_boltzmann_cfd_d3q19_amd import capi
    rho = torch.full((lat.n,), fill, dtype=lat.dtype, device=lat.device)
    u = torch.full((3, lat.n), fill, dtype=lat.dtype, device=lat.device)
    capi.check(capi.lbm_step_moments(lat.handle, k, rho.data_ptr(), u.data_ptr()), "lbm_step_moments", lat.handle)
    torch.cuda.synchronize()
    return rho.double().cpu().numpy(), u.double().cpu().numpy()


@pytest.mark.parametrize("name", ["sphere_force", "closed_box", "porous", "all_solid", "solid_ends"])
def test_step_moments_write_every_cell(name):
    # outputs start as NaN: every cell must be written, the solid ones with 0
    need_gpu()
    if name == "all_solid":
        shape, per, tau, F = (9, 7, 5), (1, 0, 1), 0.8, (0.0, 0.0, 0.0)
        mask = np.ones(9 * 7 * 5, np.uint8)
    elif name == "solid_ends":
        # long solid runs before the first and after the last fluid cell, and
        # a fluid slab narrower than one wave
        shape, per, tau, F = (40, 30, 20), (1, 1, 0), 0.7, (1e-5, 0.0, 0.0)
        m = np.ones((20, 30, 40), np.uint8)
        m[9:11, 3:25, 5:31] = 0
        m[14, 7, 2:4] = 0
        mask = m.reshape(-1)
    else:
        shape, per, tau, F, mask = _case(name)
    rho, u = li.random_fields(*shape, seed=43)
    solid = mask.reshape(-1).astype(bool)
    for layout in LAYOUTS:
        for scheme in SCHEMES:
            for k in (3, 4):
                say("step_moments every cell", name, layout, scheme, k)
                a = make(shape, "f32", layout, scheme, tau=tau, force=F, mask=mask, periodic=per,
                         rho=cast(rho, "f32"), u=cast(u, "f32"))
                a.step(k - 1)
                r1, u1 = a.moments()
                torch.cuda.synchronize()
                b = make(shape, "f32", layout, scheme, tau=tau, force=F, mask=mask, periodic=per,
                         rho=cast(rho, "f32"), u=cast(u, "f32"))
                r2, u2 = _step_moments_into(b, k, float("nan"))
                assert not np.isnan(r2).any() and not np.isnan(u2).any()
                assert np.all(r2[solid] == 0.0) and np.all(u2[:, solid] == 0.0)
                assert np.array_equal(r2, r1.double().cpu().numpy()) and np.array_equal(u2, u1.double().cpu().numpy())


@pytest.mark.parametrize("scheme", SCHEMES)
def test_step_moments_porous256_compact(scheme):
    # the full-size porous box on the compact layout (many waves, chunked
    # workgroup order): every cell written, equal to lbm_moments before the step
    need_gpu()
    mask, _ = li.porous_mask(256)
    shape = (256, 256, 256)
    for k in (1, 2):
        say("step_moments porous256 compact", scheme, k)
        a = make(shape, "f32", "compact", scheme, tau=0.65, force=(1e-6, 0.0, 0.0), mask=mask)
        a.step(k - 1)
        r1, u1 = a.moments()
        torch.cuda.synchronize()
        r1, u1 = r1.cpu().numpy(), u1.cpu().numpy()
        del a
        b = make(shape, "f32", "compact", scheme, tau=0.65, force=(1e-6, 0.0, 0.0), mask=mask)
        r2, u2 = _step_moments_into(b, k, float("nan"))
        del b
        assert not np.isnan(r2).any() and not np.isnan(u2).any()
        assert np.array_equal(r2, r1.astype(np.float64)) and np.array_equal(u2, u1.astype(np.float64))
