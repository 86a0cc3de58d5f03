"""CPU oracle for the fused D3Q19 BGK collide-and-stream update.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``lattice_boltzmann_cfd_d3q19_amd``) never imports it, and this package never
imports the product.  The arithmetic lives in ``lbm_oracle.c`` (plain C, fp64,
single-threaded); this module only marshals numpy arrays through ctypes.

Populations are canonical: ``f[19][N]`` float64, direction-major, cell index
``x + nx*(y + ny*z)``, in the oracle's own direction order (``lattice()``).

Parity status per function (what pins it, from the tests):
  lattice          -- velocity-set identities in exact rationals, page weights
  equilibrium      -- exact moment identities (mass, momentum, momentum flux)
  collide          -- equilibrium fixed point, conservation, Guo momentum input
  run              -- brute-force streaming search, permutation property,
                      Poiseuille closed form, shear-wave and Taylor-Green decay
  step_cells       -- equals ``run`` for one step on every cell
  moments, totals  -- direct sums, checked against numpy on the same f
  momentum_exchange -- the step's momentum budget (P(t+1) - P(t) = N_fluid F
                      minus the exchanged force, any state), zero force at
                      rest, steady channel wall force = N_fluid F
  apply_open_faces -- uniform streams are fixed points of every rule; the
                      moments each Zou-He rule prescribes hold exactly on any
                      state; Neumann copies the inward cell's equilibrium;
                      per-step mass budget through the faces; pressure-driven
                      channel flow
No function is "parity unpinned"; the specific random streams used to build
inputs are unpinned by nature (determinism and statistics only).
"""
import ctypes
import math
import os

import numpy as np

Q = 19
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liblbm_oracle.so")
_lib = None


class _Box(ctypes.Structure):
    _fields_ = [("nx", ctypes.c_int64), ("ny", ctypes.c_int64), ("nz", ctypes.c_int64),
                ("periodic", ctypes.c_int32 * 3), ("tau", ctypes.c_double),
                ("force", ctypes.c_double * 3), ("open", ctypes.c_int32 * 6),
                ("face_rho", ctypes.c_double * 6), ("face_u", (ctypes.c_double * 3) * 6),
                ("face_kind", ctypes.c_int32 * 6)]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER
    dp, u8p, i64p = P(ctypes.c_double), P(ctypes.c_uint8), P(ctypes.c_int64)
    lib.orc_lattice.argtypes = [P(ctypes.c_int32), dp, P(ctypes.c_int32)]
    lib.orc_equilibrium.argtypes = [ctypes.c_double, dp, dp]
    lib.orc_guo_term.argtypes = [ctypes.c_double, dp, dp, dp]
    lib.orc_collide.argtypes = [P(_Box), dp, dp]
    lib.orc_cell_moments.argtypes = [P(_Box), dp, dp, dp]
    lib.orc_init_equilibrium.argtypes = [P(_Box), u8p, dp, dp, dp]
    lib.orc_init_equilibrium.restype = ctypes.c_int
    lib.orc_run.argtypes = [P(_Box), u8p, dp, ctypes.c_int64]
    lib.orc_run.restype = ctypes.c_int
    lib.orc_step_cells.argtypes = [P(_Box), u8p, dp, ctypes.c_int64, i64p, dp]
    lib.orc_step_cells.restype = ctypes.c_int
    lib.orc_moments.argtypes = [P(_Box), u8p, dp, dp, dp]
    lib.orc_totals.argtypes = [P(_Box), u8p, dp, dp]
    lib.orc_momentum_exchange.argtypes = [P(_Box), u8p, dp, dp]
    lib.orc_apply_open_faces.argtypes = [P(_Box), u8p, dp]
    _lib = lib
    return lib


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _mptr(mask):
    if mask is None:
        return None
    return mask.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


FACES = ("-x", "+x", "-y", "+y", "-z", "+z")
# open-face rules, in the C oracle's numbering
FACE_RULES = ("equilibrium", "neumann", "zou_he_pressure", "zou_he_velocity")


class Box:
    """Box description: dims, periodic axes, relaxation time, body force, and
    open faces: ``open_faces`` maps a face name ("-x", "+x", ...) on a
    non-periodic axis to (rho, (ux, uy, uz)) or (rho, (ux, uy, uz), rule),
    rule one of FACE_RULES (default "equilibrium": a reservoir whose
    equilibrium enters the box).  The other rules need every open face on one
    axis and at least 3 cells along it."""

    def __init__(self, nx, ny, nz, periodic=(1, 1, 1), tau=1.0, force=(0.0, 0.0, 0.0), open_faces=None):
        self.nx, self.ny, self.nz = int(nx), int(ny), int(nz)
        self.periodic = tuple(int(p) for p in periodic)
        self.tau = float(tau)
        self.force = tuple(float(v) for v in force)
        self.open_faces = {}
        for k, v in dict(open_faces or {}).items():
            assert k in FACES and not self.periodic[FACES.index(k) // 2], k
            rule = v[2] if len(v) > 2 else "equilibrium"
            assert rule in FACE_RULES, rule
            self.open_faces[k] = (float(v[0]), tuple(float(c) for c in v[1]), rule)
        axes = {FACES.index(k) // 2 for k in self.open_faces}
        for k, (_, _, rule) in self.open_faces.items():
            if rule != "equilibrium":
                a = FACES.index(k) // 2
                if len(axes) > 1 or (self.nx, self.ny, self.nz)[a] < 3:
                    raise ValueError("face rules other than equilibrium need all open faces on one axis, "
                                     "at least 3 cells long")

    @property
    def n(self):
        return self.nx * self.ny * self.nz

    @property
    def omega(self):
        return 0.0 if math.isinf(self.tau) else 1.0 / self.tau

    def _c(self):
        b = _Box()
        b.nx, b.ny, b.nz = self.nx, self.ny, self.nz
        b.periodic[:] = list(self.periodic)
        b.tau = self.tau
        b.force[:] = list(self.force)
        for k, (rho, u, rule) in self.open_faces.items():
            i = FACES.index(k)
            b.open[i] = 1
            b.face_rho[i] = rho
            b.face_u[i][:] = list(u)
            b.face_kind[i] = FACE_RULES.index(rule)
        return b


def _mask(box, mask):
    if mask is None:
        return None
    m = np.ascontiguousarray(mask, dtype=np.uint8).reshape(-1)
    assert m.size == box.n
    return m


def lattice():
    """Return (c[19][3] int32, w[19] float64, opp[19] int32)."""
    lib = _load()
    c = np.zeros((Q, 3), np.int32)
    w = np.zeros(Q, np.float64)
    opp = np.zeros(Q, np.int32)
    lib.orc_lattice(c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _dptr(w),
                    opp.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    return c, w, opp


def equilibrium(rho, u):
    lib = _load()
    uu = np.ascontiguousarray(u, np.float64)
    out = np.zeros(Q, np.float64)
    lib.orc_equilibrium(float(rho), _dptr(uu), _dptr(out))
    return out


def guo_term(omega, u, F):
    lib = _load()
    uu = np.ascontiguousarray(u, np.float64)
    FF = np.ascontiguousarray(F, np.float64)
    out = np.zeros(Q, np.float64)
    lib.orc_guo_term(float(omega), _dptr(uu), _dptr(FF), _dptr(out))
    return out


def collide(box, f_cell):
    lib = _load()
    fin = np.ascontiguousarray(f_cell, np.float64)
    out = np.zeros(Q, np.float64)
    b = box._c()
    lib.orc_collide(ctypes.byref(b), _dptr(fin), _dptr(out))
    return out


def cell_moments(box, f_cell):
    lib = _load()
    fin = np.ascontiguousarray(f_cell, np.float64)
    rho = np.zeros(1, np.float64)
    u = np.zeros(3, np.float64)
    b = box._c()
    lib.orc_cell_moments(ctypes.byref(b), _dptr(fin), _dptr(rho), _dptr(u))
    return float(rho[0]), u


def init_equilibrium(box, mask=None, rho0=None, u0=None):
    """Canonical f(0) = equilibrium(rho0, u0) on fluid cells; [19][N] float64."""
    lib = _load()
    m = _mask(box, mask)
    r = None if rho0 is None else np.ascontiguousarray(rho0, np.float64).reshape(-1)
    u = None if u0 is None else np.ascontiguousarray(u0, np.float64).reshape(3, -1)
    f = np.zeros((Q, box.n), np.float64)
    b = box._c()
    rc = lib.orc_init_equilibrium(ctypes.byref(b), _mptr(m), None if r is None else _dptr(r),
                                  None if u is None else _dptr(u), _dptr(f))
    assert rc == 0
    return f


def run(box, f, nsteps, mask=None):
    """Return f(t + nsteps) from f(t) (a new array; the input is not modified)."""
    lib = _load()
    m = _mask(box, mask)
    out = np.array(f, dtype=np.float64, order="C", copy=True).reshape(Q, box.n)
    b = box._c()
    rc = lib.orc_run(ctypes.byref(b), _mptr(m), _dptr(out), int(nsteps))
    if rc != 0:
        raise MemoryError("oracle run failed")
    return out


def step_cells(box, f, cells, mask=None):
    """f(t+1) at the given cells, shape [len(cells)][19]."""
    lib = _load()
    m = _mask(box, mask)
    fin = np.ascontiguousarray(f, np.float64).reshape(Q, box.n)
    cl = np.ascontiguousarray(cells, np.int64)
    out = np.zeros((cl.size, Q), np.float64)
    b = box._c()
    rc = lib.orc_step_cells(ctypes.byref(b), _mptr(m), _dptr(fin), cl.size,
                            cl.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _dptr(out))
    assert rc == 0
    return out


def moments(box, f, mask=None):
    """(rho[N], u[3][N]) with u including F/2; zeros on solid cells."""
    lib = _load()
    m = _mask(box, mask)
    fin = np.ascontiguousarray(f, np.float64).reshape(Q, box.n)
    rho = np.zeros(box.n, np.float64)
    u = np.zeros((3, box.n), np.float64)
    b = box._c()
    lib.orc_moments(ctypes.byref(b), _mptr(m), _dptr(fin), _dptr(rho), _dptr(u))
    return rho, u


def totals(box, f, mask=None):
    """dict(mass, momentum[3], ke) summed over fluid cells."""
    lib = _load()
    m = _mask(box, mask)
    fin = np.ascontiguousarray(f, np.float64).reshape(Q, box.n)
    out = np.zeros(5, np.float64)
    b = box._c()
    lib.orc_totals(ctypes.byref(b), _mptr(m), _dptr(fin), _dptr(out))
    return {"mass": out[0], "momentum": out[1:4].copy(), "ke": out[4]}


def momentum_exchange(box, f, mask=None):
    """Force on the solids during the step that starts from f: dict(solid[3],
    wall[3]), each the sum of 2 f*_q c_q over the bounce-back links that end
    in a solid cell / leave the box through a non-periodic face."""
    lib = _load()
    m = _mask(box, mask)
    fin = np.ascontiguousarray(f, np.float64).reshape(Q, box.n)
    out = np.zeros(6, np.float64)
    b = box._c()
    lib.orc_momentum_exchange(ctypes.byref(b), _mptr(m), _dptr(fin), _dptr(out))
    return {"solid": out[0:3].copy(), "wall": out[3:6].copy()}


def apply_open_faces(box, f, mask=None):
    """Copy of f with every population entering through an open face set by
    the face's rule."""
    lib = _load()
    m = _mask(box, mask)
    out = np.array(f, np.float64, copy=True).reshape(Q, box.n)
    b = box._c()
    lib.orc_apply_open_faces(ctypes.byref(b), _mptr(m), _dptr(out))
    return out

