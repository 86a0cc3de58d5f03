"""Initial density and velocity fields (float64; cast once by the caller).

Arrays are rho[N] and u[3][N] with cell = x + nx*(y + ny*z).
"""
import math

import numpy as np

from .mt64 import MT19937_64, uniform01


def random_fields(nx, ny, nz, seed=1, drho=0.01, du=0.05):
    """Per cell, in linear cell order, draw rho = 1 + drho(2U-1), then
    u_x, u_y, u_z = du(2U-1) each (four draws per cell)."""
    n = nx * ny * nz
    g = MT19937_64(seed)
    r = uniform01(g, 4 * n).reshape(n, 4)
    rho = 1.0 + drho * (2.0 * r[:, 0] - 1.0)
    u = du * (2.0 * r[:, 1:4].T - 1.0)
    return np.ascontiguousarray(rho), np.ascontiguousarray(u)


def _coords(nx, ny, nz):
    z, y, x = np.meshgrid(np.arange(nz), np.arange(ny), np.arange(nx), indexing="ij")
    return x.reshape(-1).astype(np.float64), y.reshape(-1).astype(np.float64), \
        z.reshape(-1).astype(np.float64)


def taylor_green(n, u0=0.04, ny=None, nz=None):
    """3-D Taylor-Green vortex at integer cell coordinates, k = 2 pi / n:
    u = u0 sin kx cos ky cos kz, v = -u0 cos kx sin ky cos kz, w = 0,
    p' = (u0^2/16)(cos 2kx + cos 2ky)(cos 2kz + 2), rho = 1 + 3 p' (c_s^2 = 1/3)."""
    ny = n if ny is None else ny
    nz = n if nz is None else nz
    x, y, z = _coords(n, ny, nz)
    k = 2.0 * math.pi / n
    u = np.empty((3, x.size), np.float64)
    u[0] = u0 * np.sin(k * x) * np.cos(k * y) * np.cos(k * z)
    u[1] = -u0 * np.cos(k * x) * np.sin(k * y) * np.cos(k * z)
    u[2] = 0.0
    p = (u0 * u0 / 16.0) * (np.cos(2 * k * x) + np.cos(2 * k * y)) * (np.cos(2 * k * z) + 2.0)
    rho = 1.0 + 3.0 * p
    return rho, u


def shear_wave(nx, ny, nz, amp=1e-4):
    """u_z = amp sin(2 pi y / ny), rho = 1: an exact incompressible solution
    whose amplitude decays as exp(-nu k^2 t)."""
    x, y, z = _coords(nx, ny, nz)
    u = np.zeros((3, x.size), np.float64)
    u[2] = amp * np.sin(2.0 * math.pi * y / ny)
    return np.ones(x.size, np.float64), u
