"""Helpers shared by the GPU tests: run the HIP path through the C ABI and
bring canonical state back to the host as float64 numpy arrays."""
import sys

import numpy as np
import pytest
import torch

LAYOUTS = ("stream", "bundle", "collision", "compact")
SCHEMES = ("ab", "aa", "eso", "twist")
TOL = {"f32": 1e-5, "f64": 1e-12}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*args):
    print("[gpu-test]", *args, flush=True)
    sys.stdout.flush()


def make(shape, precision="f32", layout="stream", scheme="aa", tau=0.8, force=(0.0, 0.0, 0.0),
         mask=None, periodic=(1, 1, 1), rho=None, u=None):
    from lattice_boltzmann_cfd_d3q19_amd import Lattice
    lat = Lattice(*shape, precision=precision, layout=layout, scheme=scheme, tau=tau, force=force)
    lat.set_geometry(None if mask is None else torch.from_numpy(np.ascontiguousarray(mask)), periodic)
    lat.init(None if rho is None else torch.from_numpy(np.ascontiguousarray(rho)),
             None if u is None else torch.from_numpy(np.ascontiguousarray(u)))
    return lat


def host_f(lat):
    f = lat.read_populations()
    torch.cuda.synchronize()
    return f.double().cpu().numpy()


def host_moments(lat):
    r, u = lat.moments()
    torch.cuda.synchronize()
    return r.double().cpu().numpy(), u.double().cpu().numpy()


def cast(a, precision):
    """Round float64 inputs once to the device precision (both sides then
    consume the same values)."""
    if a is None:
        return None
    return np.asarray(a, np.float64).astype(np.float32 if precision == "f32" else np.float64)
