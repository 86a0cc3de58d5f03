"""Write porous256_f100.txt: the CPU oracle's canonical populations f(100) of
the 256^3 periodic porous medium at sampled cells.

Workload: 2400 overlapping spheres, r ~ U(6, 12), centres uniform, seed 5
(the porous-medium recipe with the sphere count scaled to keep porosity near
0.6 at 256^3); tau = 0.65, body force (1e-6, 0, 0), fluid at rest with
rho = 1 at t = 0, halfway bounce-back on the solids.  The samples are 1024
fluid cells drawn at random and 1024 fluid cells with at least one solid cell
among their 18 lattice neighbours (where bounce-back acts).  Only ``oracle``
and ``lbm_inputs`` are called.

    python tests/golden/make_porous256_f100.py     (about 25 minutes, one core)
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import lbm_inputs as li  # noqa: E402
import oracle  # noqa: E402

N, TAU, FORCE, STEPS, SEED = 256, 0.65, (1e-6, 0.0, 0.0), 100, 5
OUT = os.path.join(HERE, "porous256_f100.txt")


def near_solid(mask3):
    """Fluid cells with a solid cell at one of the 18 offsets c_q != 0
    (periodic wrap), as flat cell indices."""
    solid = mask3.astype(bool)
    hit = np.zeros_like(solid)
    for dz in (-1, 0, 1):
        for dy in (-1, 0, 1):
            for dx in (-1, 0, 1):
                if 0 < dx * dx + dy * dy + dz * dz <= 2:
                    hit |= np.roll(solid, (dz, dy, dx), axis=(0, 1, 2))
    return np.nonzero((hit & ~solid).reshape(-1))[0]


def main():
    mask, nsph = li.porous_mask(N, seed=SEED)
    assert nsph == 2400
    mask3 = mask.reshape(N, N, N)
    rng = np.random.default_rng(100)
    fluid = np.nonzero(mask == 0)[0]
    cells = np.unique(np.concatenate([rng.choice(fluid, 1024, replace=False),
                                      rng.choice(near_solid(mask3), 1024, replace=False)]))
    box = oracle.Box(N, N, N, periodic=(1, 1, 1), tau=TAU, force=FORCE)
    f = oracle.init_equilibrium(box, mask)
    t0 = time.time()
    f = oracle.run(box, f, STEPS, mask)
    print(f"{STEPS} steps in {time.time() - t0:.0f} s", flush=True)
    with open(OUT, "w") as fh:
        fh.write("# 256^3 periodic porous medium (2400 spheres, r ~ U(6,12), seed 5), tau = 0.65,\n")
        fh.write("# force (1e-6, 0, 0), rho = 1 and u = 0 at t = 0: canonical f(100) from the CPU oracle\n")
        fh.write("# (fp64) at sampled fluid cells; written by make_porous256_f100.py.\n")
        fh.write("# columns: cell  f_0 ... f_18  (direction order: lexicographic over (c_z, c_y, c_x))\n")
        for c in cells:
            fh.write(str(int(c)) + " " + " ".join(f"{v:.13e}" for v in f[:, c]) + "\n")


if __name__ == "__main__":
    main()
