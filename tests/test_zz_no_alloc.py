"""The allocation-free variant of the fused momentum exchange
(lbm_step_momentum_exchange_noalloc), called through the C ABI, against the
entry point that takes a caller's scratch buffer: the same forces and the
same state after the call, bit for bit, on two calls in a row (the second on
a smaller box, whose fewer partial rows land in the array the first call
left filled)."""
import numpy as np
import pytest
import torch

import lbm_inputs as li
from gpu_util import make, need_gpu, say

pytestmark = pytest.mark.gpu


def _pair(shape, layout, scheme, precision, seed):
    mask = li.random_mask(*shape, fraction=0.12, seed=seed)
    rho, u = li.random_fields(*shape, seed=seed + 1)
    dt = np.float32 if precision == "f32" else np.float64
    kw = dict(precision=precision, layout=layout, scheme=scheme, tau=0.7, force=(1e-5, -2e-6, 3e-6),
              mask=mask, periodic=(1, 0, 1), rho=rho.astype(dt), u=u.astype(dt))
    return make(shape, **kw), make(shape, **kw)


@pytest.mark.parametrize("layout,scheme,precision", [("compact", "aa", "f32"), ("stream", "aa", "f32"),
                                                     ("compact", "ab", "f64"), ("collision", "eso", "f32")])
def test_noalloc_equals_scratch_entry_point(layout, scheme, precision):
    need_gpu()
    from lattice_boltzmann_cfd_d3q19_amd import capi
    for shape, nsteps, seed in (((70, 48, 40), 5, 3), ((23, 17, 11), 4, 9)):
        say("no-alloc momentum exchange", layout, scheme, precision, shape, nsteps)
        ref, lat = _pair(shape, layout, scheme, precision, seed)
        lat.step(3)
        ref.step(3)
        want_solid, want_wall = ref.step_momentum_exchange(nsteps)
        out = torch.full((6,), float("nan"), dtype=torch.float64, device="cuda")
        st = capi.lbm_step_momentum_exchange_noalloc(lat.handle, nsteps, out.data_ptr())
        capi.check(st, "lbm_step_momentum_exchange_noalloc", lat.handle)
        torch.cuda.synchronize()
        assert lat.t == ref.t == 3 + nsteps
        want = torch.cat([want_solid, want_wall])
        say("  force", out.tolist())
        assert torch.equal(out, want), (out.tolist(), want.tolist())
        assert float(out[:3].abs().max()) > 0.0     # the solids take a force
        assert torch.equal(lat.read_populations(), ref.read_populations())
        del ref, lat
