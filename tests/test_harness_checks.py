"""The benchmark's state check flags a run that has gone unstable: the oracle
at tau = 1/2 + 1e-6 with |u| ~ 0.3 (BGK is unstable there) first exceeds the
lattice speed, then overflows to non-finite values; a stable run passes."""
import importlib.util
import os

import numpy as np

import lbm_inputs as li
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def test_state_check_flags_an_unstable_run():
    box = oracle.Box(8, 8, 8, tau=0.5 + 1e-6)
    rho, u = li.random_fields(8, 8, 8, seed=3, du=0.3)
    f = oracle.init_equilibrium(box, None, rho, u)
    finite, bounded = bench.state_check(*oracle.moments(box, f))
    assert finite and bounded
    f = oracle.run(box, f, 50)
    finite, bounded = bench.state_check(*oracle.moments(box, f))
    assert finite and not bounded
    f = oracle.run(box, f, 450)
    finite, bounded = bench.state_check(*oracle.moments(box, f))
    assert not finite and not bounded


def test_state_check_passes_a_stable_run_and_ignores_solids():
    box = oracle.Box(8, 8, 8, tau=0.8, force=(1e-5, 0.0, 0.0))
    mask = li.random_mask(8, 8, 8, fraction=0.2, seed=4)
    rho, u = li.random_fields(8, 8, 8, seed=5)
    f = oracle.run(box, oracle.init_equilibrium(box, mask, rho, u), 100, mask)
    r, v = oracle.moments(box, f, mask)
    assert bench.state_check(r, v, mask) == (True, True)
    # solid cells carry rho = 0, which only the fluid cells may not
    assert bench.state_check(r, v) == (True, False)
