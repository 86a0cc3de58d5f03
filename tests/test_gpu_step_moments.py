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
