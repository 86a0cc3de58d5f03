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


def test_handle_stream_differs_from_current_stream():
    """The handle runs on its own stream while the caller stays on the default
    stream: inputs made on the current stream, outputs read on it, and
    temporaries freed right after each call must all be ordered (the binding
    makes each stream wait for the other and records tensor use)."""
    need_gpu()
    shape, layout, scheme, seed = (40, 30, 20), "compact", "aa", 47
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ref = _lattice(shape, layout, scheme, s, seed)
        ref.step(31)
        want_f = ref.read_populations()
        want_r, want_u = ref.moments()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    lat = _lattice(shape, layout, scheme, side, seed)      # called on the default stream
    for _ in range(31):
        lat.step(1)
        junk = torch.empty(1 << 22, device="cuda").fill_(float("nan"))  # reuse freed blocks
        del junk
    f = lat.read_populations()
    r, u = lat.moments()
    f2 = f.clone()          # default-stream work that reads the outputs right away
    r2, u2 = r.clone(), u.clone()
    torch.cuda.synchronize()
    say("handle on a side stream", shape, layout, scheme)
    assert torch.equal(f2, want_f)
    assert torch.equal(r2, want_r) and torch.equal(u2, want_u)
