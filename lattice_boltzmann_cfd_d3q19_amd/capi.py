"""ctypes binding of liblbm.so: the C ABI of include/lbm.h, same names.

Argument marshalling only -- every step of the update runs in the HIP
kernels of liblbm.so.  Pointers are passed as Python ints (device addresses,
e.g. ``tensor.data_ptr()``); streams as ``torch.cuda.Stream.cuda_stream``.
Importing this module raises if the library has not been built: there is no
CPU fallback.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblbm.so")

LBM_OK = 0
LBM_ERR_INVALID_ARGUMENT = -1
LBM_ERR_UNSUPPORTED = -2
LBM_ERR_BAD_STATE = -3
LBM_ERR_MISALIGNED = -4
LBM_ERR_HIP = -5

LBM_F32, LBM_F64 = 0, 1
LBM_LAYOUT_STREAM, LBM_LAYOUT_BUNDLE, LBM_LAYOUT_COLLISION, LBM_LAYOUT_COMPACT = 0, 1, 2, 3
LBM_SCHEME_AB, LBM_SCHEME_AA, LBM_SCHEME_ESOPULL, LBM_SCHEME_ESOTWIST = 0, 1, 2, 3

EXPORTED = ["lbm_buffer_bytes", "lbm_workspace_bytes", "lbm_create", "lbm_set_workspace", "lbm_set_geometry", "lbm_init_equilibrium", "lbm_step",
            "lbm_moments", "lbm_read_populations", "lbm_write_populations", "lbm_save_state",
            "lbm_load_state", "lbm_destroy", "lbm_time", "lbm_fluid_cells", "lbm_last_hip_error",
            "lbm_status_string", "lbm_momentum_exchange_scratch_bytes", "lbm_momentum_exchange",
            "lbm_set_open_faces", "lbm_step_moments", "lbm_step_momentum_exchange",
            "lbm_step_momentum_exchange_noalloc"]


class lbm_desc(ctypes.Structure):
    _fields_ = [("nx", ctypes.c_int64), ("ny", ctypes.c_int64), ("nz", ctypes.c_int64),
                ("precision", ctypes.c_int32), ("layout", ctypes.c_int32), ("scheme", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("tau", ctypes.c_double), ("force", ctypes.c_double * 3)]


class LbmError(RuntimeError):
    def __init__(self, status, where):
        super().__init__(f"{where}: {lbm_status_string(status)} ({status})")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python lattice_boltzmann_cfd_d3q19_amd/_build.py` (there is no CPU fallback)")

# liblbm.so must share one HIP runtime with the process's torch.  torch ships
# its own libamdhip64 with the same soname (libamdhip64.so.7); loading torch
# first makes the dynamic loader bind liblbm.so to that copy.  Loading ours
# first would map a second HIP runtime, which then sees no device.
try:
    import torch  # noqa: F401
except ImportError:  # no torch: the library binds to the system HIP runtime
    pass

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i64, _i32, _st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32
_Desc_p = ctypes.POINTER(lbm_desc)

_lib.lbm_buffer_bytes.argtypes = [_Desc_p, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(_i32)]
_lib.lbm_buffer_bytes.restype = _st
_lib.lbm_workspace_bytes.argtypes = [_Desc_p, ctypes.POINTER(ctypes.c_size_t)]
_lib.lbm_workspace_bytes.restype = _st
_lib.lbm_set_workspace.argtypes = [_vp, _vp, ctypes.c_size_t]
_lib.lbm_set_workspace.restype = _st
_lib.lbm_fluid_cells.argtypes = [_vp]
_lib.lbm_fluid_cells.restype = _i64
_lib.lbm_create.argtypes = [_Desc_p, _vp, _vp, _vp, ctypes.POINTER(_vp)]
_lib.lbm_create.restype = _st
_lib.lbm_set_geometry.argtypes = [_vp, _vp, ctypes.POINTER(_i32)]
_lib.lbm_set_geometry.restype = _st
_lib.lbm_set_open_faces.argtypes = [_vp, ctypes.POINTER(_i32), ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_double)]
_lib.lbm_set_open_faces.restype = _st
_lib.lbm_init_equilibrium.argtypes = [_vp, _vp, _vp]
_lib.lbm_init_equilibrium.restype = _st
_lib.lbm_step.argtypes = [_vp, _i64]
_lib.lbm_step_moments.argtypes = [_vp, _i64, _vp, _vp]
_lib.lbm_step_moments.restype = _st
_lib.lbm_step.restype = _st
_lib.lbm_moments.argtypes = [_vp, _vp, _vp]
_lib.lbm_moments.restype = _st
_lib.lbm_read_populations.argtypes = [_vp, _vp]
_lib.lbm_read_populations.restype = _st
_lib.lbm_write_populations.argtypes = [_vp, _vp]
_lib.lbm_write_populations.restype = _st
_lib.lbm_save_state.argtypes = [_vp, _vp]
_lib.lbm_save_state.restype = _st
_lib.lbm_load_state.argtypes = [_vp, _vp]
_lib.lbm_load_state.restype = _st
_lib.lbm_momentum_exchange_scratch_bytes.argtypes = [_Desc_p, ctypes.POINTER(ctypes.c_size_t)]
_lib.lbm_momentum_exchange_scratch_bytes.restype = _st
_lib.lbm_momentum_exchange.argtypes = [_vp, _vp, _vp, ctypes.c_size_t]
_lib.lbm_momentum_exchange.restype = _st
_lib.lbm_step_momentum_exchange.argtypes = [_vp, ctypes.c_int64, _vp, _vp, ctypes.c_size_t]
_lib.lbm_step_momentum_exchange.restype = _st
_lib.lbm_step_momentum_exchange_noalloc.argtypes = [_vp, ctypes.c_int64, _vp]
_lib.lbm_step_momentum_exchange_noalloc.restype = _st
_lib.lbm_destroy.argtypes = [_vp]
_lib.lbm_destroy.restype = _st
_lib.lbm_time.argtypes = [_vp]
_lib.lbm_time.restype = _i64
_lib.lbm_last_hip_error.argtypes = [_vp]
_lib.lbm_last_hip_error.restype = ctypes.c_char_p
_lib.lbm_status_string.argtypes = [_st]
_lib.lbm_status_string.restype = ctypes.c_char_p


def library():
    """The loaded ctypes.CDLL (for symbol checks)."""
    return _lib


def make_desc(nx, ny, nz, precision=LBM_F32, layout=LBM_LAYOUT_STREAM, scheme=LBM_SCHEME_AA, tau=1.0,
              force=(0.0, 0.0, 0.0)):
    d = lbm_desc()
    d.nx, d.ny, d.nz = int(nx), int(ny), int(nz)
    d.precision, d.layout, d.scheme, d.reserved = int(precision), int(layout), int(scheme), 0
    d.tau = float(tau)
    d.force[:] = [float(v) for v in force]
    return d


def _ptr(p):
    return None if p is None or p == 0 else ctypes.c_void_p(int(p))


def lbm_status_string(status):
    return _lib.lbm_status_string(int(status)).decode()


def lbm_buffer_bytes(desc):
    """Return (status, bytes_per_buffer, n_buffers)."""
    nb = ctypes.c_size_t(0)
    n = _i32(0)
    st = _lib.lbm_buffer_bytes(ctypes.byref(desc), ctypes.byref(nb), ctypes.byref(n))
    return st, nb.value, n.value


def lbm_workspace_bytes(desc):
    """Return (status, bytes)."""
    nb = ctypes.c_size_t(0)
    st = _lib.lbm_workspace_bytes(ctypes.byref(desc), ctypes.byref(nb))
    return st, nb.value


def lbm_set_workspace(sim, ws, nbytes):
    return _lib.lbm_set_workspace(sim, _ptr(ws), int(nbytes))


def lbm_fluid_cells(sim):
    return _lib.lbm_fluid_cells(sim)


def lbm_create(desc, buf0, buf1=None, stream=None):
    """Return (status, handle)."""
    h = _vp(None)
    st = _lib.lbm_create(ctypes.byref(desc), _ptr(buf0), _ptr(buf1), _ptr(stream), ctypes.byref(h))
    return st, h


def lbm_set_geometry(sim, mask, periodic):
    per = None if periodic is None else (_i32 * 3)(*[int(p) for p in periodic])
    return _lib.lbm_set_geometry(sim, _ptr(mask), per)


FACES = ("-x", "+x", "-y", "+y", "-z", "+z")


# open-face kinds, in the order of lbm_face_kind from LBM_FACE_EQUILIBRIUM (1) on
FACE_KINDS = ("equilibrium", "neumann", "zou_he_pressure", "zou_he_velocity")


def lbm_set_open_faces(sim, faces):
    """faces: {face name: (rho, (ux, uy, uz)) or (rho, (ux, uy, uz), kind)},
    kind one of FACE_KINDS (default "equilibrium"); faces not named are closed."""
    op = (_i32 * 6)()
    rho = (ctypes.c_double * 6)(*([1.0] * 6))
    u = (ctypes.c_double * 18)()
    for k, spec in faces.items():
        r, v = spec[0], spec[1]
        kind = spec[2] if len(spec) > 2 else "equilibrium"
        i = FACES.index(k)
        op[i] = 1 + FACE_KINDS.index(kind)
        rho[i] = float(r)
        for a in range(3):
            u[3 * i + a] = float(v[a])
    return _lib.lbm_set_open_faces(sim, op, rho, u)


def lbm_init_equilibrium(sim, rho=None, u=None):
    return _lib.lbm_init_equilibrium(sim, _ptr(rho), _ptr(u))


def lbm_step(sim, n):
    return _lib.lbm_step(sim, int(n))


def lbm_step_moments(sim, n, rho, u):
    return _lib.lbm_step_moments(sim, int(n), _ptr(rho), _ptr(u))


def lbm_moments(sim, rho, u):
    return _lib.lbm_moments(sim, _ptr(rho), _ptr(u))


def lbm_read_populations(sim, f):
    return _lib.lbm_read_populations(sim, _ptr(f))


def lbm_write_populations(sim, f):
    return _lib.lbm_write_populations(sim, _ptr(f))


def lbm_save_state(sim, s):
    return _lib.lbm_save_state(sim, _ptr(s))


def lbm_load_state(sim, s):
    return _lib.lbm_load_state(sim, _ptr(s))


def lbm_momentum_exchange_scratch_bytes(desc):
    """Return (status, bytes)."""
    nb = ctypes.c_size_t(0)
    st = _lib.lbm_momentum_exchange_scratch_bytes(ctypes.byref(desc), ctypes.byref(nb))
    return st, nb.value


def lbm_momentum_exchange(sim, force, scratch, nbytes):
    return _lib.lbm_momentum_exchange(sim, _ptr(force), _ptr(scratch), int(nbytes))


def lbm_step_momentum_exchange(sim, n, force, scratch, nbytes):
    return _lib.lbm_step_momentum_exchange(sim, int(n), _ptr(force), _ptr(scratch), int(nbytes))


def lbm_step_momentum_exchange_noalloc(sim, n, force):
    return _lib.lbm_step_momentum_exchange_noalloc(sim, int(n), _ptr(force))


LBM_STATIC_SCRATCH_BYTES = 4 << 20


def lbm_destroy(sim):
    return _lib.lbm_destroy(sim)


def lbm_time(sim):
    return _lib.lbm_time(sim)


def lbm_last_hip_error(sim):
    return _lib.lbm_last_hip_error(sim).decode()


def check(status, where="", sim=None):
    if status != LBM_OK:
        if status == LBM_ERR_HIP and sim is not None:
            where = f"{where} [{lbm_last_hip_error(sim)}]"
        raise LbmError(status, where)
    return status
