"""The momentum exchange taken inside the last step (lbm_step_momentum_exchange
through the C ABI): the force equals the separate pass (lbm_momentum_exchange
called just before that step) and the oracle's on the GPU's own state, and the
state after the call equals that of the plain steps bit for bit.  Both step
parities of the in-place schemes, every layout and scheme, walls, solids, open
faces with reservoirs and with face rules, and the boxes without any link."""
import numpy as np
import pytest
import torch

import lbm_inputs as li
import oracle
from gpu_util import LAYOUTS, SCHEMES, cast, make, need_gpu, say
from test_gpu_momentum_exchange import exact_f
from test_gpu_open_faces import _make_open, _open_case
from test_gpu_parity import _case

pytestmark = pytest.mark.gpu


def _vec(pair):
    solid, wall = pair
    torch.cuda.synchronize()
    return np.concatenate([solid.cpu().numpy(), wall.cpu().numpy()])


def _state(lat):
    s = lat.save_state()
    torch.cuda.synchronize()
    return s.cpu().numpy()


def _setup(name, precision):
    if name in ("sphere_force", "porous", "closed_box", "channel"):
        shape, per, tau, F, mask = _case(name)
        faces = None
    else:
        shape, per, tau, F, faces, mask = _open_case(name)
    rho, u = li.random_fields(*shape, seed=41)
    rho, u = cast(rho, precision), cast(0.5 * u, precision)

    def build(layout, scheme):
        if faces is None:
            return make(shape, precision, layout, scheme, tau=tau, force=F, mask=mask, periodic=per, rho=rho, u=u)
        return _make_open(shape, precision, layout, scheme, tau, F, faces, mask, per, rho, u)

    box = oracle.Box(*shape, periodic=per, tau=tau, force=F, open_faces=faces or {})
    return shape, mask, box, build


@pytest.mark.parametrize("precision", ["f32", "f64"])
@pytest.mark.parametrize("name", ["sphere_force", "closed_box", "porous", "zou_he_channel", "inlet_outlet"])
def test_fused_force_equals_separate_pass(name, precision):
    need_gpu()
    shape, mask, box, build = _setup(name, precision)
    n = int(np.prod(shape))
    atol = (4e-9 if precision == "f32" else 1e-15) * n
    for layout in LAYOUTS:
        for scheme in SCHEMES:
            sep = build(layout, scheme)
            fused = build(layout, scheme)
            # 7 steps, then 1: the last step of each call has the other parity
            for steps in (7, 1):
                say("fused force", name, precision, layout, scheme, "steps", steps, "from t =", sep.t)
                sep.step(steps - 1)
                f_before = exact_f(sep, precision, mask)
                want_sep = _vec(sep.momentum_exchange())
                sep.step(1)
                got = _vec(fused.step_momentum_exchange(steps))
                assert fused.t == sep.t
                assert np.array_equal(_state(fused), _state(sep)), (layout, scheme, "state differs")
                want = oracle.momentum_exchange(box, f_before, mask)
                want = np.concatenate([want["solid"], want["wall"]])
                err_o = np.max(np.abs(got - want))
                err_s = np.max(np.abs(got - want_sep))
                say("  vs oracle", err_o, "vs separate pass", err_s, "force", got)
                assert err_o <= atol, (layout, scheme, err_o)
                if layout == "compact":
                    # other workgroup sizes than the separate pass: another
                    # order of summation, equal to rounding
                    assert err_s <= 1e-15 * n * max(1.0, np.max(np.abs(want_sep))), (layout, scheme, err_s)
                else:
                    # the same cells per partial row, summed in the same order
                    assert np.array_equal(got, want_sep), (layout, scheme, got, want_sep)


@pytest.mark.parametrize("precision", ["f32", "f64"])
def test_fused_force_without_links_is_zero(precision):
    need_gpu()
    rho, u = li.random_fields(12, 10, 9, seed=43)
    rho, u = cast(rho, precision), cast(0.5 * u, precision)
    for layout in LAYOUTS:
        for scheme in SCHEMES:
            say("no links", precision, layout, scheme)
            # fully periodic, no mask: no bounce-back link at all
            a = make((12, 10, 9), precision, layout, scheme, tau=0.7, rho=rho, u=u)
            b = make((12, 10, 9), precision, layout, scheme, tau=0.7, rho=rho, u=u)
            got = _vec(a.step_momentum_exchange(3))
            b.step(3)
            assert np.all(got == 0.0)
            assert np.array_equal(_state(a), _state(b))
            # every cell solid: no fluid cell (the compact layout stores none)
            m = np.ones(12 * 10 * 9, np.uint8)
            c = make((12, 10, 9), precision, layout, scheme, tau=0.7, mask=m, periodic=(1, 0, 1))
            assert np.all(_vec(c.step_momentum_exchange(2)) == 0.0)


def test_fused_force_rejects_bad_arguments():
    from lattice_boltzmann_cfd_d3q19_amd import capi
    need_gpu()
    lat = make((8, 8, 8), "f32", "compact", "aa", mask=li.sphere_mask(8, 8, 8, radius=2))
    st, nb = capi.lbm_momentum_exchange_scratch_bytes(lat.desc)
    assert st == capi.LBM_OK
    scratch = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty(6, dtype=torch.float64, device="cuda")
    assert capi.lbm_step_momentum_exchange(lat.handle, 0, out.data_ptr(), scratch.data_ptr(),
                                           nb) == capi.LBM_ERR_INVALID_ARGUMENT
    assert capi.lbm_step_momentum_exchange(lat.handle, 1, out.data_ptr(), scratch.data_ptr(),
                                           nb - 1) == capi.LBM_ERR_INVALID_ARGUMENT
    assert capi.lbm_step_momentum_exchange(lat.handle, 1, out.data_ptr() + 4, scratch.data_ptr(),
                                           nb) == capi.LBM_ERR_MISALIGNED
    assert lat.t == 0
    assert capi.lbm_step_momentum_exchange(lat.handle, 2, out.data_ptr(), scratch.data_ptr(), nb) == capi.LBM_OK
    assert lat.t == 2
