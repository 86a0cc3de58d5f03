"""Two handles on two streams at once: the library keeps no global state, so
interleaved steps of two lattices on separate HIP streams give exactly what
each gives alone."""
import numpy as np
import pytest
import torch

import lbm_inputs as li
from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu


def _lattice(shape, layout, scheme, stream, seed):
    from lattice_boltzmann_cfd_d3q19_amd import Lattice
    mask = li.random_mask(*shape, fraction=0.15, seed=seed)
    rho, u = li.random_fields(*shape, seed=seed)
    lat = Lattice(*shape, precision="f32", layout=layout, scheme=scheme, tau=0.7, force=(1e-5, 0.0, 0.0),
                  stream=stream)
    lat.set_geometry(torch.from_numpy(mask), (1, 0, 1))
    lat.init(torch.from_numpy(rho.astype(np.float32)), torch.from_numpy(u.astype(np.float32)))
    return lat


def test_two_streams_interleaved_equal_alone():
    need_gpu()
    cfg = [((40, 30, 20), "compact", "aa", 41), ((33, 27, 19), "stream", "eso", 43)]
    alone = []
    for shape, layout, scheme, seed in cfg:
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            lat = _lattice(shape, layout, scheme, s, seed)
            lat.step(60)
            alone.append(lat.read_populations())
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    lats = []
    for (shape, layout, scheme, seed), s in zip(cfg, streams):
        with torch.cuda.stream(s):
            lats.append(_lattice(shape, layout, scheme, s, seed))
    for k in range(30):
        for lat in lats:
            lat.step(2)
    outs = []
    for lat, s in zip(lats, streams):
        with torch.cuda.stream(s):
            outs.append(lat.read_populations())
    torch.cuda.synchronize()
    for (shape, layout, scheme, _), a, b in zip(cfg, alone, outs):
        say("two streams", shape, layout, scheme)
        assert torch.equal(a, b), (layout, scheme)
