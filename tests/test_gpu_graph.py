"""Capture of lbm_step into a HIP graph (through torch's graph capture on the
handle's stream) and repeated replays, with eager work on the same stream
between the replays: every replay equals the same steps launched directly.
The library launches only kernels on the handle's stream (no memsets, no
allocations), so an even number of steps -- which returns the in-place
schemes to the same parity and AB to the same buffer -- can be captured."""
import numpy as np
import pytest
import torch

import lbm_inputs as li
from gpu_util import say, need_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout,scheme", [("stream", "aa"), ("compact", "aa"), ("bundle", "ab"),
                                           ("compact", "eso"), ("compact", "twist"), ("collision", "twist")])
def test_graph_replays_equal_direct_steps(layout, scheme):
    need_gpu()
    from lattice_boltzmann_cfd_d3q19_amd import Lattice
    shape = (24, 20, 18)
    mask = li.sphere_mask(*shape, radius=5)
    rho, u = li.random_fields(*shape, seed=3)
    rho, u = torch.from_numpy(rho.astype(np.float32)), torch.from_numpy(u.astype(np.float32))

    def make(stream):
        lat = Lattice(*shape, precision="f32", layout=layout, scheme=scheme, tau=0.7,
                      force=(1e-5, 0.0, 0.0), stream=stream)
        lat.set_geometry(torch.from_numpy(mask), (1, 0, 1))
        lat.set_open_faces({"-y": (1.0, (0.0, 0.02, 0.0)), "+y": (1.0, (0.0, 0.0, 0.0), "zou_he_pressure")})
        lat.init(rho, u)
        return lat

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        lat = make(s)
        ref = make(s)
        lat.step(3)
        ref.step(3)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        lat.step(2)          # recorded, not run; the handle's time moves on by 2
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for k in range(4):
            say("graph replay", layout, scheme, k)
            g.replay()
            ref.step(2)
            got = lat.read_populations()       # eager work between replays
            want = ref.read_populations()
            r, v = lat.moments()
            torch.cuda.synchronize()
            assert torch.equal(got, want), (layout, scheme, k)
            assert torch.isfinite(r).all() and torch.isfinite(v).all()
