"""Seeded input generators: pinned to the published engine and to brute force."""
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import lbm_inputs as li


def test_mt19937_64_standard_value():
    # The C++ standard requires the 10000th output of a default-constructed
    # mt19937_64 (seed 5489) to be 9981545732273789042.
    g = li.MT19937_64(5489)
    x = g.next_u64(10000)
    assert int(x[-1]) == 9981545732273789042


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_mt19937_64_matches_libstdcxx():
    src = r"""
#include <cstdio>
#include <random>
int main(int argc, char** argv) {
  unsigned long long seed = std::strtoull(argv[1], nullptr, 10);
  std::mt19937_64 g(seed);
  for (int i = 0; i < 1000; ++i) std::printf("%llu\n", (unsigned long long)g());
}
"""
    with tempfile.TemporaryDirectory() as d:
        cpp = os.path.join(d, "mt.cpp")
        exe = os.path.join(d, "mt")
        with open(cpp, "w") as fh:
            fh.write(src)
        subprocess.run(["g++", "-O1", "-o", exe, cpp], check=True)
        for seed in (1, 5, 123456789):
            out = subprocess.run([exe, str(seed)], check=True, capture_output=True, text=True).stdout
            want = [int(v) for v in out.split()]
            got = [int(v) for v in li.MT19937_64(seed).next_u64(1000)]
            assert got == want


def test_uniform_range_and_resolution():
    u = li.uniform01(li.MT19937_64(9), 100000)
    assert u.min() >= 0.0 and u.max() < 1.0
    assert np.all(np.floor(u * 2.0 ** 53) == u * 2.0 ** 53)
    assert abs(u.mean() - 0.5) < 0.01


def test_random_fields_recipe():
    rho, u = li.random_fields(4, 3, 2, seed=1)
    r = li.uniform01(li.MT19937_64(1), 4 * 24).reshape(24, 4)
    assert np.array_equal(rho, 1 + 0.01 * (2 * r[:, 0] - 1))
    assert np.array_equal(u, 0.05 * (2 * r[:, 1:].T - 1))
    assert np.all(np.abs(rho - 1) <= 0.01) and np.all(np.abs(u) <= 0.05)


def test_sphere_mask_brute_force():
    for n, r in [(10, 3), (9, 4), (16, 5)]:
        m = li.sphere_mask(n, radius=r).reshape(n, n, n)
        c = (n - 1) / 2.0
        for k in range(n):
            for j in range(n):
                for i in range(n):
                    d2 = (i - c) ** 2 + (j - c) ** 2 + (k - c) ** 2
                    assert m[k, j, i] == (1 if d2 <= r * r else 0)


def test_benchmark_sphere_symmetric():
    m = li.sphere_mask(128, radius=16).reshape(128, 128, 128)
    assert np.array_equal(m, m[::-1]) and np.array_equal(m, m[:, ::-1]) and np.array_equal(m, m[:, :, ::-1])
    assert np.array_equal(m, m.transpose(1, 0, 2)) and np.array_equal(m, m.transpose(2, 1, 0))
    n = int(m.sum())
    assert abs(n - 4.0 / 3.0 * math.pi * 16 ** 3) / n < 0.02


def test_porous_mask_brute_force_small():
    nx, ny, nz = 14, 11, 9
    m, ns = li.porous_mask(nx, ny, nz, n_spheres=6, seed=3, rmin=2.0, rmax=4.0)
    m = m.reshape(nz, ny, nx)
    d = li.uniform01(li.MT19937_64(3), 24).reshape(6, 4)
    want = np.zeros_like(m)
    dims = (nx, ny, nz)
    for s in range(6):
        cq = [math.floor(dims[a] * d[s, a] * 1024 + 0.5) for a in range(3)]
        rq = math.floor((2.0 + 2.0 * d[s, 3]) * 1024 + 0.5)
        for k in range(nz):
            for j in range(ny):
                for i in range(nx):
                    tot = 0
                    for a, p in enumerate((i, j, k)):
                        per = dims[a] * 1024
                        dd = (1024 * p - cq[a]) % per
                        dd = min(dd, per - dd)
                        tot += dd * dd
                    if tot <= rq * rq:
                        want[k, j, i] = 1
    assert np.array_equal(m, want)


def test_porous_porosity_128():
    m, ns = li.porous_mask(128, n_spheres=300, seed=5)
    porosity = 1.0 - m.mean()
    # Boolean sphere model: porosity = exp(-n E[V] / L^3), E[r^3] = 810 for U(6, 12)
    expected = math.exp(-300 * 4.0 / 3.0 * math.pi * 810.0 / 128 ** 3)
    assert abs(porosity - expected) < 0.02
    assert li.porous_sphere_count(256) == 2400 and li.porous_sphere_count(512) == 19200
