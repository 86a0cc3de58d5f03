"""The stored populations sit where include/lbm.h says they do.

Distinct canonical populations are written through lbm_write_populations and
the raw device buffer is read back: for every fluid cell and direction, the
element at the address the header gives for the layout holds the stored
(weight-shifted) value f - w, computed in the lattice's precision.  The
address maps are the PortLBM page's layouts (section 3.2, Fig. 2: SoA, SoAoS,
AoS) and the fluid-only layout in 64-cell blocks of 19 planes; the in-place
scheme's even state keeps f_q in slot q of its own cell (fieldcraft page,
first section).
"""
import numpy as np
import pytest
import torch

import lbm_inputs as li
import oracle
from gpu_util import make, need_gpu, say

C, W, _OPP = oracle.lattice()
Q = 19
# storage plane of direction q in the fluid-only layout: opposite directions
# side by side, P(q) = 2q (q < 9), 2(18 - q) + 1 (q > 9), P(9) = 18
PLANE = [2 * q if q < 9 else (2 * (18 - q) + 1 if q > 9 else 18) for q in range(Q)]
# bundles of equal (c_y, c_z) for the SoAoS layout, in direction order
BUNDLES = []
for q in range(Q):
    if BUNDLES and tuple(C[BUNDLES[-1][0]][1:]) == tuple(C[q][1:]):
        BUNDLES[-1].append(q)
    else:
        BUNDLES.append([q])


def address(layout, q, cell, rank, n):
    if layout == "stream":
        return q * n + cell
    if layout == "collision":
        return cell * Q + q
    if layout == "bundle":
        b = next(b for b in BUNDLES if q in b)
        return n * b[0] + cell * len(b) + (q - b[0])
    return (rank // 64) * Q * 64 + PLANE[q] * 64 + rank % 64


@pytest.mark.gpu
@pytest.mark.parametrize("precision", ["f32", "f64"])
@pytest.mark.parametrize("layout", ["stream", "bundle", "collision", "compact"])
def test_stored_populations_at_documented_addresses(layout, precision):
    need_gpu()
    shape = (70, 5, 3)  # rows longer than a 64-cell block, a ragged last block
    n = int(np.prod(shape))
    mask = li.random_mask(*shape, fraction=0.3, seed=41)
    say("raw layout", layout, precision, shape)
    lat = make(shape, precision=precision, layout=layout, scheme="aa", mask=mask)
    rng = np.random.default_rng(5)
    f = (W[:, None] * (1.0 + 0.1 * rng.standard_normal((Q, n)))).astype(np.float64)
    lat.write_populations(torch.from_numpy(f))
    torch.cuda.synchronize()
    raw = lat.buffers[0].cpu().numpy()
    dt = np.float32 if precision == "f32" else np.float64
    wq = np.array([dt(1) / dt(36 // int(round(36 * W[q]))) for q in range(Q)], dtype=dt)
    fluid = np.flatnonzero(mask == 0)
    checked = 0
    for rank, cell in enumerate(fluid):
        for q in range(Q):
            want = dt(f[q, cell]) - wq[q]
            got = raw[address(layout, q, int(cell), rank, n)]
            assert got == want, (layout, precision, int(cell), rank, q, got, want)
            checked += 1
    assert checked == Q * len(fluid)


@pytest.mark.gpu
@pytest.mark.parametrize("precision", ["f32", "f64"])
@pytest.mark.parametrize("scheme", ["aa", "ab"])
@pytest.mark.parametrize("layout", ["stream", "bundle", "collision"])
def test_solid_records_stay_cleared(layout, scheme, precision):
    """Solid cells are never updated: in the in-place and two-lattice schemes
    their slots of a dense layout hold 0 after the initialisation and keep it
    through every step, whatever the kernels around them do with the lines
    they share (the AoS even step copies runs of records through LDS; the
    odd step rewrites views of neighbouring records)."""
    need_gpu()
    shape = (70, 5, 3)  # a ragged last block of 256 records, solids in mixed lines
    n = int(np.prod(shape))
    mask = li.random_mask(*shape, fraction=0.3, seed=43)
    rho, u = li.random_fields(*shape, seed=44)
    say("solid records", layout, scheme, precision, shape)
    lat = make(shape, precision=precision, layout=layout, scheme=scheme, mask=mask, rho=rho, u=u,
               force=(1e-5, 0.0, 0.0))
    solid = np.flatnonzero(mask != 0)
    assert solid.size > 0
    idx = np.array([[address(layout, q, int(c), 0, n) for q in range(Q)] for c in solid]).ravel()
    for steps in (1, 2, 3):
        lat.step(steps)
        torch.cuda.synchronize()
        for buf in lat.buffers:
            raw = buf.cpu().numpy()
            assert np.all(raw[idx] == 0), (layout, scheme, precision, steps)
