"""Parity at the full sizes of the five workloads: 100 steps from the seeded
inputs, then the GPU's canonical populations against the CPU oracle's.

Bar (the same as on the small boxes): max-abs 1e-5 over every population of
every cell for fp32, 1e-12 for fp64.
  - 128^3 Taylor-Green vortex (u0 = 0.04, tau = 0.6), fp32: whole box;
  - 128^3 box with a centred sphere of radius 16, force 1e-6 along x,
    tau = 0.7, fp32: whole box, every layout;
  - 64 x 64 x 256 channel, walls beyond y = 0 and y = 63, force 1e-6 along z,
    tau = 0.9, fp64: whole box;
  - 256^3 porous medium (2400 spheres), force 1e-6 along x, tau = 0.65, fp32:
    at the 2048 sampled cells of tests/golden/porous256_f100.txt (the oracle
    needs minutes for this box; make_porous256_f100.py wrote the file from
    the oracle alone).
The three oracle runs of the 128^3 and channel boxes start together in
background threads when the module is first used (ctypes releases the GIL),
so the tests wait for at most the longest of them.
"""
import concurrent.futures
import os

import numpy as np
import pytest
import torch

import lbm_inputs as li
import oracle
from gpu_util import TOL, cast, make, need_gpu, say

pytestmark = pytest.mark.gpu
Q = 19
STEPS = 100


def _config(name):
    """shape, periodic, tau, force, mask, rho, u, precision (inputs as both
    sides consume them: rounded once to the device precision)."""
    if name == "tgv128":
        rho, u = li.taylor_green(128, u0=0.04)
        return (128, 128, 128), (1, 1, 1), 0.6, (0.0, 0.0, 0.0), None, cast(rho, "f32"), cast(u, "f32"), "f32"
    if name == "sphere128":
        return (128, 128, 128), (1, 1, 1), 0.7, (1e-6, 0.0, 0.0), li.sphere_mask(128, radius=16), None, None, "f32"
    if name == "channel_f64":
        return (64, 64, 256), (1, 0, 1), 0.9, (0.0, 0.0, 1e-6), None, None, None, "f64"
    if name == "porous256":
        mask, nsph = li.porous_mask(256)
        assert nsph == 2400
        return (256, 256, 256), (1, 1, 1), 0.65, (1e-6, 0.0, 0.0), mask, None, None, "f32"
    raise KeyError(name)


def _oracle_f(name):
    shape, per, tau, F, mask, rho, u, _ = _config(name)
    box = oracle.Box(*shape, periodic=per, tau=tau, force=F)
    f0 = oracle.init_equilibrium(box, mask, rho, u)
    return oracle.run(box, f0, STEPS, mask)


_POOL = None
_FUT = {}


def _want(name):
    global _POOL
    if _POOL is None:
        _POOL = concurrent.futures.ThreadPoolExecutor(max_workers=3)
        for k in ("tgv128", "sphere128", "channel_f64"):
            _FUT[k] = _POOL.submit(_oracle_f, k)
    return _FUT[name].result()


def _run_gpu(name, layout, scheme):
    shape, per, tau, F, mask, rho, u, prec = _config(name)
    lat = make(shape, prec, layout, scheme, tau=tau, force=F, mask=mask, periodic=per, rho=rho, u=u)
    lat.step(STEPS)
    assert lat.t == STEPS
    return lat, mask, prec


@pytest.mark.parametrize("name,layout,scheme", [
    ("tgv128", "stream", "aa"), ("tgv128", "stream", "ab"), ("tgv128", "compact", "aa"),
    ("tgv128", "collision", "ab"), ("tgv128", "collision", "aa"), ("tgv128", "bundle", "aa"), ("tgv128", "bundle", "ab"),
    ("sphere128", "stream", "aa"), ("sphere128", "bundle", "aa"), ("sphere128", "collision", "aa"),
    ("sphere128", "compact", "aa"), ("sphere128", "stream", "ab"),
    ("channel_f64", "stream", "aa"), ("channel_f64", "stream", "ab"), ("channel_f64", "compact", "aa"),
    ("channel_f64", "compact", "ab"), ("channel_f64", "bundle", "aa")])
def test_full_box_100_steps(name, layout, scheme):
    need_gpu()
    say("full box", name, layout, scheme, "(waiting for the oracle)")
    want = _want(name)
    say("  oracle ready; GPU run")
    lat, mask, prec = _run_gpu(name, layout, scheme)
    got = lat.read_populations()
    torch.cuda.synchronize()
    got = got.double().cpu().numpy()
    del lat
    err = float(np.max(np.abs(got - want)))
    say("  max-abs over the whole box", err)
    assert err <= TOL[prec], (name, layout, scheme, err)
    if mask is not None:
        assert np.all(got[:, mask.astype(bool)] == 0.0)


def _golden_porous(golden_dir):
    rows = np.loadtxt(os.path.join(golden_dir, "porous256_f100.txt"), dtype=np.float64)
    return rows[:, 0].astype(np.int64), rows[:, 1:].T.copy()


@pytest.mark.parametrize("layout,scheme", [("compact", "aa"), ("compact", "ab"), ("stream", "aa"),
                                           ("stream", "ab"), ("compact", "eso"), ("compact", "twist")])
def test_porous256_100_steps_sampled(layout, scheme, golden_dir):
    need_gpu()
    cells, want = _golden_porous(golden_dir)
    assert cells.size > 1900 and want.shape == (Q, cells.size)
    say("porous 256^3, 100 steps", layout, scheme, "cells", cells.size)
    lat, mask, prec = _run_gpu("porous256", layout, scheme)
    assert np.all(mask[cells] == 0)
    f = lat.read_populations()
    idx = torch.from_numpy(cells).to(f.device)
    got = f.index_select(1, idx).double().cpu().numpy()
    solid = torch.from_numpy(mask.astype(bool)).to(f.device)
    solid_max = float(f[:, solid].abs().max()) if bool(solid.any()) else 0.0
    del f, lat
    torch.cuda.synchronize()
    err = float(np.max(np.abs(got - want)))
    say("  max-abs at the sampled cells", err, "| solid cells max", solid_max)
    assert err <= TOL[prec], (layout, scheme, err)
    assert solid_max == 0.0
