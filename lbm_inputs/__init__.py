"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This package holds none of the lattice Boltzmann arithmetic: it only draws
random numbers and builds initial fields and solid masks, so that both sides
of a parity test consume the very same arrays.  Everything is deterministic:

- random numbers come from the 64-bit Mersenne Twister (``MT19937_64``),
  implemented from its published definition (Matsumoto and Nishimura; the
  same engine the C++ standard names ``std::mt19937_64``), turned into
  uniform doubles in [0, 1) as ``(x >> 11) * 2**-53``;
- geometry (sphere and porous masks) is decided in exact integer arithmetic.

Workloads (box sizes and physics of the five benchmark configurations):
  random_fields    -- 32^3 periodic box, rho = 1 + 0.01 U(-1,1), u_a = 0.05 U(-1,1)
  taylor_green     -- 128^3 Taylor-Green vortex, u0 = 0.04
  sphere_mask      -- 128^3 box, sphere of radius 16 at the box centre
  cylinder_mask    -- a cylinder along z (the obstacle of the open-channel workload)
  porous_mask      -- 256^3 (and 512^3) overlapping spheres, r ~ U(6, 12)
"""
from .mt64 import MT19937_64, uniform01
from .fields import random_fields, taylor_green, shear_wave
from .geometry import cylinder_mask, sphere_mask, porous_mask, porous_sphere_count, random_mask

__all__ = ["MT19937_64", "uniform01", "random_fields", "taylor_green", "shear_wave",
           "sphere_mask", "porous_mask", "porous_sphere_count", "random_mask", "cylinder_mask"]
