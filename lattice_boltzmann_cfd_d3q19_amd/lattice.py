"""Thin torch-side convenience wrapper over the C ABI.

Torch provides device memory and the stream only; every operation is one
call into liblbm.so.  Buffers are allocated on the current HIP device.

Streams: the library enqueues its kernels on the handle's stream.  Tensors
passed in or returned are made and used on the caller's current stream, so
when the two differ each call first makes the handle's stream wait for the
current one, then makes the current stream wait for the handle's, and marks
every tensor the call touched as used on the handle's stream (so that the
caching allocator does not hand its memory out again before the kernels that
read or write it have run).
"""
import torch

from . import capi

_PREC = {"f32": (capi.LBM_F32, torch.float32), "f64": (capi.LBM_F64, torch.float64)}
_LAYOUT = {"stream": capi.LBM_LAYOUT_STREAM, "bundle": capi.LBM_LAYOUT_BUNDLE,
           "collision": capi.LBM_LAYOUT_COLLISION, "compact": capi.LBM_LAYOUT_COMPACT}
_SCHEME = {"ab": capi.LBM_SCHEME_AB, "aa": capi.LBM_SCHEME_AA, "eso": capi.LBM_SCHEME_ESOPULL,
           "twist": capi.LBM_SCHEME_ESOTWIST}

Q = 19


class Lattice:
    """One D3Q19 lattice on the GPU.

    precision: "f32" | "f64"; layout: "stream" | "bundle" | "collision" |
    "compact" (SoA over fluid cells only); scheme: "ab" (two lattices, fused
    pull) | "aa" (one lattice, in place) | "eso" (one lattice, in place,
    esoteric pull) | "twist" (one lattice, in place, esoteric twist).
    """

    def __init__(self, nx, ny, nz, precision="f32", layout="stream", scheme="aa", tau=1.0,
                 force=(0.0, 0.0, 0.0), stream=None, device=None):
        if not torch.cuda.is_available():
            raise RuntimeError("no HIP device: the lattice runs only on the GPU")
        self.shape = (int(nx), int(ny), int(nz))
        self.n = self.shape[0] * self.shape[1] * self.shape[2]
        prec, self.dtype = _PREC[precision]
        self.device = torch.device("cuda") if device is None else torch.device(device)
        self.desc = capi.make_desc(nx, ny, nz, prec, _LAYOUT[layout], _SCHEME[scheme], tau, force)
        st, nbytes, nbuf = capi.lbm_buffer_bytes(self.desc)
        capi.check(st, "lbm_buffer_bytes")
        elems = nbytes // torch.empty((), dtype=self.dtype).element_size()
        self.buffers = [torch.empty(elems, dtype=self.dtype, device=self.device) for _ in range(nbuf)]
        self.stream = torch.cuda.current_stream(self.device) if stream is None else stream
        ptrs = [b.data_ptr() for b in self.buffers] + [None]
        st, self.handle = capi.lbm_create(self.desc, ptrs[0], ptrs[1], self.stream.cuda_stream)
        capi.check(st, "lbm_create")
        if torch.cuda.current_stream(self.device).cuda_stream != self.stream.cuda_stream:
            self.stream.wait_stream(torch.cuda.current_stream(self.device))
            for b in self.buffers:
                b.record_stream(self.stream)
        self.mask = None
        st, wbytes = capi.lbm_workspace_bytes(self.desc)
        capi.check(st, "lbm_workspace_bytes")
        self.workspace = None
        if wbytes:
            self.workspace = torch.empty(wbytes, dtype=torch.uint8, device=self.device)
            self._call(lambda: capi.lbm_set_workspace(self.handle, self.workspace.data_ptr(), wbytes),
                       "lbm_set_workspace", self.workspace, handle=False)

    def _call(self, fn, name, *tensors, handle=True):
        """Run one C-ABI call, ordered against the caller's current stream."""
        cur = torch.cuda.current_stream(self.device)
        other = cur.cuda_stream != self.stream.cuda_stream
        if other:
            self.stream.wait_stream(cur)
        st = fn()
        if other:
            for t in tensors:
                if t is not None:
                    t.record_stream(self.stream)
            cur.wait_stream(self.stream)
        capi.check(st, name, self.handle if handle else None)

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value is not None:
            capi.lbm_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- geometry and state -------------------------------------------------
    def set_geometry(self, mask=None, periodic=(1, 1, 1)):
        if mask is not None:
            mask = torch.as_tensor(mask).to(device=self.device, dtype=torch.uint8).contiguous().reshape(-1)
            if mask.numel() != self.n:
                raise ValueError("mask must have nx*ny*nz entries")
        self.mask = mask
        self._call(lambda: capi.lbm_set_geometry(self.handle, None if mask is None else mask.data_ptr(), periodic),
                   "lbm_set_geometry", mask, handle=False)

    def set_open_faces(self, faces):
        """faces: {"-x" | "+x" | "-y" | "+y" | "-z" | "+z": (rho, (ux, uy, uz)[, kind])}
        on non-periodic axes, kind one of capi.FACE_KINDS ("equilibrium" by
        default: a reservoir whose equilibrium enters the box; "neumann",
        "zou_he_pressure", "zou_he_velocity").  Call after set_geometry,
        before init."""
        self._call(lambda: capi.lbm_set_open_faces(self.handle, faces), "lbm_set_open_faces", handle=False)

    def _dev(self, a, shape):
        t = torch.as_tensor(a).to(device=self.device, dtype=self.dtype).contiguous()
        return t.reshape(shape)

    def init(self, rho=None, u=None):
        r = None if rho is None else self._dev(rho, (self.n,))
        v = None if u is None else self._dev(u, (3, self.n))
        self._call(lambda: capi.lbm_init_equilibrium(self.handle, None if r is None else r.data_ptr(),
                                                     None if v is None else v.data_ptr()),
                   "lbm_init_equilibrium", r, v)
        self._keep = (r, v)  # alive until the init kernel has run on the stream

    def step(self, n=1):
        self._call(lambda: capi.lbm_step(self.handle, n), "lbm_step")

    def step_moments(self, n=1):
        """n steps; returns the density and velocity the last step's collision
        used (the moments of the state at t + n - 1), written by that step."""
        rho = torch.empty(self.n, dtype=self.dtype, device=self.device)
        u = torch.empty((3, self.n), dtype=self.dtype, device=self.device)
        self._call(lambda: capi.lbm_step_moments(self.handle, n, rho.data_ptr(), u.data_ptr()),
                   "lbm_step_moments", rho, u)
        return rho, u

    @property
    def t(self):
        return capi.lbm_time(self.handle)

    @property
    def fluid_cells(self):
        """Fluid cells counted by the compact layout (-1 for dense layouts)."""
        return capi.lbm_fluid_cells(self.handle)

    def moments(self):
        rho = torch.empty(self.n, dtype=self.dtype, device=self.device)
        u = torch.empty((3, self.n), dtype=self.dtype, device=self.device)
        self._call(lambda: capi.lbm_moments(self.handle, rho.data_ptr(), u.data_ptr()), "lbm_moments", rho, u)
        return rho, u

    def read_populations(self):
        f = torch.empty((Q, self.n), dtype=self.dtype, device=self.device)
        self._call(lambda: capi.lbm_read_populations(self.handle, f.data_ptr()), "lbm_read_populations", f)
        return f

    def write_populations(self, f):
        ff = self._dev(f, (Q, self.n))
        self._call(lambda: capi.lbm_write_populations(self.handle, ff.data_ptr()), "lbm_write_populations", ff)
        self._keep = (ff,)

    def _mex_buffer(self):
        if getattr(self, "_mex_scratch", None) is None:
            st, nb = capi.lbm_momentum_exchange_scratch_bytes(self.desc)
            capi.check(st, "lbm_momentum_exchange_scratch_bytes")
            self._mex_scratch = torch.empty(nb, dtype=torch.uint8, device=self.device)
        return self._mex_scratch

    def momentum_exchange(self):
        """Force on the solids during the step that starts from the current
        state: (solid, wall), each a float64 tensor of 3 on the device."""
        scratch = self._mex_buffer()
        out = torch.empty(6, dtype=torch.float64, device=self.device)
        self._call(lambda: capi.lbm_momentum_exchange(self.handle, out.data_ptr(), scratch.data_ptr(),
                                                      scratch.numel()), "lbm_momentum_exchange", out, scratch)
        return out[0:3], out[3:6]

    def step_momentum_exchange(self, n=1):
        """n steps; the force on the solids during the last one, taken inside
        that step: (solid, wall) as momentum_exchange() just before it."""
        scratch = self._mex_buffer()
        out = torch.empty(6, dtype=torch.float64, device=self.device)
        self._call(lambda: capi.lbm_step_momentum_exchange(self.handle, n, out.data_ptr(), scratch.data_ptr(),
                                                           scratch.numel()), "lbm_step_momentum_exchange", out, scratch)
        return out[0:3], out[3:6]

    def save_state(self):
        """Exact checkpoint: stored values f - w, canonical order [19][N]."""
        s = torch.empty((Q, self.n), dtype=self.dtype, device=self.device)
        self._call(lambda: capi.lbm_save_state(self.handle, s.data_ptr()), "lbm_save_state", s)
        return s

    def load_state(self, s):
        ss = self._dev(s, (Q, self.n))
        self._call(lambda: capi.lbm_load_state(self.handle, ss.data_ptr()), "lbm_load_state", ss)
        self._keep = (ss,)
