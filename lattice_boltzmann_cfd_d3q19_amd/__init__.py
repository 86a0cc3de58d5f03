"""MI355X-native fused D3Q19 BGK collide-and-stream (HIP kernels for gfx950).

The product is the C-ABI library ``liblbm.so`` (include/lbm.h); ``capi``
binds it with ctypes under the same function names and ``Lattice`` wraps a
handle with torch-allocated device buffers.  There is no CPU path: importing
fails if the library is missing.
"""
from . import capi
from .capi import (lbm_buffer_bytes, lbm_create, lbm_destroy, lbm_init_equilibrium, lbm_load_state,
                   lbm_moments, lbm_read_populations, lbm_save_state, lbm_set_geometry, lbm_status_string,
                   lbm_step, lbm_time, lbm_write_populations, make_desc, LbmError)
from .lattice import Lattice

__all__ = ["capi", "Lattice", "lbm_buffer_bytes", "lbm_create", "lbm_destroy", "lbm_init_equilibrium",
           "lbm_moments", "lbm_read_populations", "lbm_set_geometry", "lbm_status_string", "lbm_step",
           "lbm_time", "lbm_write_populations", "lbm_save_state", "lbm_load_state", "make_desc", "LbmError"]
