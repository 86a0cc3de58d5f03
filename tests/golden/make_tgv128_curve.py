"""Write tgv128_ke_curve.txt: kinetic energy and mass of the 128^3 Taylor-Green
vortex (u0 = 0.04, tau = 0.6, fp32-rounded initial fields) every 50 steps up
to 1000, computed by the CPU oracle only.

    python tests/golden/make_tgv128_curve.py     (about 25 minutes, one core)
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import lbm_inputs as li  # noqa: E402
import oracle  # noqa: E402


def main():
    n, tau, u0 = 128, 0.6, 0.04
    box = oracle.Box(n, n, n, tau=tau)
    rho, u = li.taylor_green(n, u0=u0)
    rho, u = rho.astype(np.float32).astype(np.float64), u.astype(np.float32).astype(np.float64)
    f = oracle.init_equilibrium(box, None, rho, u)
    rows = []
    for t in range(0, 1001, 50):
        if t:
            f = oracle.run(box, f, 50)
        tot = oracle.totals(box, f)
        rows.append((t, float(tot["ke"]), float(tot["mass"])))
        print(t, tot["ke"], tot["mass"], flush=True)
    with open(os.path.join(HERE, "tgv128_ke_curve.txt"), "w") as fh:
        fh.write("# 3-D Taylor-Green vortex, 128^3 periodic, u0 = 0.04, rho = 1 + 3 p', tau = 0.6,\n")
        fh.write("# initial rho and u rounded to fp32; written by make_tgv128_curve.py from the CPU oracle.\n")
        fh.write("# columns: step  kinetic_energy  mass\n")
        for t, ke, m in rows:
            fh.write(f"{t} {ke!r} {m!r}\n")


if __name__ == "__main__":
    main()
