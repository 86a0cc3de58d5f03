"""The benchmark's state check flags a run that has gone unstable: the oracle
at tau = 1/2 + 1e-6 with |u| ~ 0.3 (BGK is unstable there) first exceeds the
lattice speed, then overflows to non-finite values; a stable run passes.  Also
the timed segments, the headline workload's fluid cells and algorithmic
bytes, and the one-GPU guard."""
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


def test_segments_cut_equal_even_parts():
    # the timed region is cut into equal segments of whole step pairs (the
    # in-place scheme alternates two kernels), ten where the count allows
    assert bench.segments(2000) == 10
    for steps in (2, 4, 6, 20, 202, 1000, 2000, 2002):
        r = bench.segments(steps)
        assert 1 <= r <= 10
        assert steps % r == 0 and (steps // r) % 2 == 0


def test_headline_workload_fluid_cells_and_bytes():
    # the seeded 256^3 porous medium: the fluid-cell count and the
    # algorithmic bytes per step (152 B per fluid update in fp32, plus the
    # 1-byte mask of every cell) that the roofline and the profiles use
    wl = bench.workload("porous256")
    mask = wl["mask"]
    assert wl["shape"] == (256, 256, 256) and mask.size == 256 ** 3 and mask.dtype == np.uint8
    nf = int(mask.size - np.count_nonzero(mask))
    assert nf == 10_463_212
    assert 2 * 19 * 4 * nf + mask.size == 1_607_185_440
    assert wl["precision"] == "f32" and wl["tau"] == 0.65


def test_bench_refuses_more_than_one_gpu():
    import json
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
