"""Host-side checks of the C ABI: exports, sizes and every error path that is
decided before anything reaches the GPU.  No kernel is launched here; the
pointers passed are never dereferenced on these paths."""
import math
import os
import re

import pytest

from lattice_boltzmann_cfd_d3q19_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 256-byte aligned address, never dereferenced here


def _header_functions():
    src = open(os.path.join(ROOT, "include", "lbm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lbm_[a-z_]+)\s*\(", src)))


def test_every_declared_function_is_exported():
    names = _header_functions()
    assert len(names) >= 11
    lib = capi.library()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(capi.EXPORTED) == names


def test_desc_struct_layout_matches_header():
    # int64 x3, int32 x4, double, double[3]
    assert capi.lbm_desc.tau.offset == 40
    assert capi.lbm_desc.force.offset == 48
    assert capi.ctypes.sizeof(capi.lbm_desc) == 72


def _byte_model(golden):
    vals = {}
    for line in open(os.path.join(golden, "byte_model.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            vals[k] = int(v)
    return vals


def test_buffer_bytes_match_page_byte_model(golden_dir):
    bm = _byte_model(golden_dir)
    n = bm["buffer_cells_per_edge"]
    st, nbytes, nbuf = capi.lbm_buffer_bytes(capi.make_desc(n, n, n, capi.LBM_F32, scheme=capi.LBM_SCHEME_AA))
    assert st == capi.LBM_OK and nbuf == 1
    assert nbytes == bm["buffer_mib"] * 2 ** 20
    # per-update traffic of the fused step: 19 reads + 19 writes of fp32
    assert 2 * nbytes // (n ** 3) == bm["inplace_bytes_per_update"]
    assert 2 * bm["inplace_bytes_per_update"] == bm["two_pass_bytes_per_update"]
    st, nbytes64, nbuf = capi.lbm_buffer_bytes(capi.make_desc(n, n, n, capi.LBM_F64, scheme=capi.LBM_SCHEME_AB))
    assert st == capi.LBM_OK and nbuf == 2 and nbytes64 == 2 * nbytes


@pytest.mark.parametrize("field,value", [
    ("nx", 0), ("ny", -3), ("nz", 0), ("precision", 2), ("layout", 4), ("scheme", 5), ("reserved", 1),
    ("tau", 0.5), ("tau", 0.2), ("tau", float("nan")), ("tau", -math.inf)])
def test_invalid_desc_rejected(field, value):
    d = capi.make_desc(8, 8, 8)
    setattr(d, field, value)
    st, h = capi.lbm_create(d, FAKE)
    assert st == capi.LBM_ERR_INVALID_ARGUMENT and not h.value
    assert capi.lbm_buffer_bytes(d)[0] == capi.LBM_ERR_INVALID_ARGUMENT


def test_nonfinite_force_rejected():
    d = capi.make_desc(8, 8, 8, force=(0.0, float("inf"), 0.0))
    assert capi.lbm_create(d, FAKE)[0] == capi.LBM_ERR_INVALID_ARGUMENT


def test_too_many_cells_unsupported():
    d = capi.make_desc(2048, 1024, 1024)
    assert capi.lbm_buffer_bytes(d)[0] == capi.LBM_ERR_UNSUPPORTED


def test_compact_offset_limits():
    # the compact kernels address the populations with 64-bit offsets (a
    # store beyond 4 GB is fine) and the padded neighbour table with 32-bit
    # ones: 4 (nx+2)(ny+2)(nz+2) < 2^32 (and N < 2^31)
    big = dict(layout=capi.LBM_LAYOUT_COMPACT, scheme=capi.LBM_SCHEME_AA)
    assert capi.lbm_buffer_bytes(capi.make_desc(1024, 1024, 256, capi.LBM_F32, **big))[0] == capi.LBM_OK
    st, nbytes, _ = capi.lbm_buffer_bytes(capi.make_desc(1024, 1024, 256, capi.LBM_F64, **big))
    assert st == capi.LBM_OK and nbytes == 19 * 1024 * 1024 * 256 * 8
    assert capi.lbm_buffer_bytes(capi.make_desc(1022, 1022, 1020, capi.LBM_F32, **big))[0] == capi.LBM_OK
    assert capi.lbm_buffer_bytes(capi.make_desc(1022, 1022, 1022, capi.LBM_F32, **big))[0] == capi.LBM_ERR_UNSUPPORTED


def test_esoteric_pull_buffers():
    # one buffer; 19 planes in the dense layouts, 28 in the compact one (the
    # 19 of the blocks, then room for one bounce-back slot per link of the
    # nine pairs)
    for layout, planes in ((capi.LBM_LAYOUT_STREAM, 19), (capi.LBM_LAYOUT_COLLISION, 19),
                           (capi.LBM_LAYOUT_COMPACT, 28)):
        d = capi.make_desc(16, 8, 5, capi.LBM_F32, layout=layout, scheme=capi.LBM_SCHEME_ESOPULL)
        st, nbytes, nbuf = capi.lbm_buffer_bytes(d)
        cells = 640 if layout == capi.LBM_LAYOUT_COMPACT else 640
        assert st == capi.LBM_OK and nbuf == 1 and nbytes == planes * cells * 4
        assert capi.lbm_create(d, FAKE, FAKE + (1 << 20))[0] == capi.LBM_ERR_INVALID_ARGUMENT
        st, h = capi.lbm_create(d, FAKE)
        assert st == capi.LBM_OK
        capi.lbm_destroy(h)
    big = dict(layout=capi.LBM_LAYOUT_COMPACT, scheme=capi.LBM_SCHEME_ESOPULL)
    # 64-bit population offsets here too
    assert capi.lbm_buffer_bytes(capi.make_desc(1024, 1024, 256, capi.LBM_F32, **big))[0] == capi.LBM_OK
    st, nbytes, _ = capi.lbm_buffer_bytes(capi.make_desc(1024, 1024, 256, capi.LBM_F64, **big))
    assert st == capi.LBM_OK and nbytes == 28 * 1024 * 1024 * 256 * 8
    # its workspace holds one more 4-byte table per cell (the bounce-back slots)
    aa = capi.make_desc(16, 8, 5, capi.LBM_F32, layout=capi.LBM_LAYOUT_COMPACT, scheme=capi.LBM_SCHEME_AA)
    eso = capi.make_desc(16, 8, 5, capi.LBM_F32, layout=capi.LBM_LAYOUT_COMPACT, scheme=capi.LBM_SCHEME_ESOPULL)
    assert capi.lbm_workspace_bytes(eso)[1] == capi.lbm_workspace_bytes(aa)[1] + 2560


def test_esoteric_twist_buffers():
    # one buffer, 19 planes; the dense layouts store one halo layer below each
    # low face, (nx+1)(ny+1)(nz+1) cells per plane, and the compact one has
    # room for as many stored cells (fluid and ghost), rounded up to 64
    for layout, cells in ((capi.LBM_LAYOUT_STREAM, 17 * 9 * 6), (capi.LBM_LAYOUT_BUNDLE, 17 * 9 * 6),
                          (capi.LBM_LAYOUT_COLLISION, 17 * 9 * 6), (capi.LBM_LAYOUT_COMPACT, 960)):
        d = capi.make_desc(16, 8, 5, capi.LBM_F32, layout=layout, scheme=capi.LBM_SCHEME_ESOTWIST)
        st, nbytes, nbuf = capi.lbm_buffer_bytes(d)
        assert st == capi.LBM_OK and nbuf == 1 and nbytes == 19 * cells * 4, (layout, nbytes)
        assert capi.lbm_create(d, FAKE, FAKE + (1 << 20))[0] == capi.LBM_ERR_INVALID_ARGUMENT
        st, h = capi.lbm_create(d, FAKE)
        assert st == capi.LBM_OK
        capi.lbm_destroy(h)
    # the padded cells are addressed with 32-bit indices: a box whose cells fit
    # but whose padded cells do not is refused for this scheme only
    thin = dict(nx=1, ny=1, nz=1 << 30)
    assert capi.lbm_buffer_bytes(capi.make_desc(thin["nx"], thin["ny"], thin["nz"], capi.LBM_F32,
                                                scheme=capi.LBM_SCHEME_AA))[0] == capi.LBM_OK
    assert capi.lbm_buffer_bytes(capi.make_desc(thin["nx"], thin["ny"], thin["nz"], capi.LBM_F32,
                                                scheme=capi.LBM_SCHEME_ESOTWIST))[0] == capi.LBM_ERR_UNSUPPORTED
    # its compact workspace also holds the stored index of every padded cell
    # and the ghost count of every padded row
    aa = capi.make_desc(16, 8, 5, capi.LBM_F32, layout=capi.LBM_LAYOUT_COMPACT, scheme=capi.LBM_SCHEME_AA)
    tw = capi.make_desc(16, 8, 5, capi.LBM_F32, layout=capi.LBM_LAYOUT_COMPACT, scheme=capi.LBM_SCHEME_ESOTWIST)
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    assert capi.lbm_workspace_bytes(tw)[1] == capi.lbm_workspace_bytes(aa)[1] + up(4 * 18 * 10 * 7) + up(4 * 10 * 7)


def test_buffer_rules():
    aa = capi.make_desc(8, 8, 8, scheme=capi.LBM_SCHEME_AA)
    ab = capi.make_desc(8, 8, 8, scheme=capi.LBM_SCHEME_AB)
    nbytes = capi.lbm_buffer_bytes(ab)[1]
    assert capi.lbm_create(aa, None)[0] == capi.LBM_ERR_INVALID_ARGUMENT
    assert capi.lbm_create(aa, FAKE, FAKE + 1 << 20)[0] == capi.LBM_ERR_INVALID_ARGUMENT
    assert capi.lbm_create(ab, FAKE, None)[0] == capi.LBM_ERR_INVALID_ARGUMENT
    assert capi.lbm_create(aa, FAKE + 4)[0] == capi.LBM_ERR_MISALIGNED
    assert capi.lbm_create(ab, FAKE, FAKE + 4 * 4096 + 4)[0] == capi.LBM_ERR_MISALIGNED
    # overlapping AB buffers
    assert capi.lbm_create(ab, FAKE, FAKE + 256)[0] == capi.LBM_ERR_INVALID_ARGUMENT
    far = FAKE + ((nbytes + 255) // 256) * 256
    st, h = capi.lbm_create(ab, FAKE, far)
    assert st == capi.LBM_OK and h.value
    capi.lbm_destroy(h)


def test_state_machine_before_any_launch():
    st, h = capi.lbm_create(capi.make_desc(8, 8, 8), FAKE)
    assert st == capi.LBM_OK
    try:
        assert capi.lbm_time(h) == 0
        assert capi.lbm_step(h, 1) == capi.LBM_ERR_BAD_STATE
        assert capi.lbm_step(h, -1) == capi.LBM_ERR_INVALID_ARGUMENT
        assert capi.lbm_moments(h, FAKE, FAKE) == capi.LBM_ERR_BAD_STATE
        assert capi.lbm_read_populations(h, FAKE) == capi.LBM_ERR_BAD_STATE
        assert capi.lbm_write_populations(h, FAKE) == capi.LBM_ERR_BAD_STATE
        assert capi.lbm_moments(h, None, FAKE) == capi.LBM_ERR_INVALID_ARGUMENT
        assert capi.lbm_set_geometry(h, None, (1, 2, 1)) == capi.LBM_ERR_INVALID_ARGUMENT
        assert capi.lbm_set_geometry(h, None, None) == capi.LBM_ERR_INVALID_ARGUMENT
        assert capi.lbm_set_geometry(h, None, (1, 0, 1)) == capi.LBM_OK
        assert capi.lbm_step(h, 0) == capi.LBM_ERR_BAD_STATE
    finally:
        assert capi.lbm_destroy(h) == capi.LBM_OK


def test_momentum_exchange_arguments_before_any_launch():
    d = capi.make_desc(40, 8, 8)
    st, nb = capi.lbm_momentum_exchange_scratch_bytes(d)
    # one row of six doubles per workgroup: tiles of 64 x 4 cells -> 1 x 2 x 8
    assert st == capi.LBM_OK and nb == 6 * 8 * (1 * 2 * 8)
    st, h = capi.lbm_create(d, FAKE)
    assert st == capi.LBM_OK
    try:
        assert capi.lbm_momentum_exchange(h, None, FAKE, nb) == capi.LBM_ERR_INVALID_ARGUMENT
        assert capi.lbm_momentum_exchange(h, FAKE, None, nb) == capi.LBM_ERR_INVALID_ARGUMENT
        assert capi.lbm_momentum_exchange(h, FAKE, FAKE, nb - 1) == capi.LBM_ERR_INVALID_ARGUMENT
        assert capi.lbm_momentum_exchange(h, FAKE, FAKE + 8, nb) == capi.LBM_ERR_MISALIGNED
        assert capi.lbm_momentum_exchange(h, FAKE + 4, FAKE, nb) == capi.LBM_ERR_MISALIGNED
        assert capi.lbm_momentum_exchange(h, FAKE, FAKE, nb) == capi.LBM_ERR_BAD_STATE
        # the same rules for the exchange taken inside the last of n >= 1 steps
        step_mex = capi.lbm_step_momentum_exchange
        assert step_mex(h, 0, FAKE, FAKE, nb) == capi.LBM_ERR_INVALID_ARGUMENT
        assert step_mex(h, 1, None, FAKE, nb) == capi.LBM_ERR_INVALID_ARGUMENT
        assert step_mex(h, 1, FAKE, None, nb) == capi.LBM_ERR_INVALID_ARGUMENT
        assert step_mex(h, 1, FAKE, FAKE, nb - 1) == capi.LBM_ERR_INVALID_ARGUMENT
        assert step_mex(h, 1, FAKE, FAKE + 8, nb) == capi.LBM_ERR_MISALIGNED
        assert step_mex(h, 1, FAKE + 4, FAKE, nb) == capi.LBM_ERR_MISALIGNED
        assert step_mex(h, 1, FAKE, FAKE, nb) == capi.LBM_ERR_BAD_STATE
        assert capi.lbm_time(h) == 0
    finally:
        capi.lbm_destroy(h)
    assert capi.lbm_momentum_exchange(None, FAKE, FAKE, nb) == capi.LBM_ERR_INVALID_ARGUMENT
    assert capi.lbm_step_momentum_exchange(None, 1, FAKE, FAKE, nb) == capi.LBM_ERR_INVALID_ARGUMENT


def test_noalloc_momentum_exchange_arguments_before_any_launch():
    # the variant with the library's fixed scratch: the same argument rules,
    # and boxes whose partial rows exceed the fixed size are refused up front
    noalloc = capi.lbm_step_momentum_exchange_noalloc
    assert noalloc(None, 1, FAKE) == capi.LBM_ERR_INVALID_ARGUMENT
    for shape, fits in (((256, 256, 256), True), ((40, 8, 8), True), ((512, 512, 512), False),
                        ((256, 256, 341), True), ((256, 256, 342), False)):
        d = capi.make_desc(*shape)
        st, nb = capi.lbm_momentum_exchange_scratch_bytes(d)
        assert st == capi.LBM_OK and (nb <= capi.LBM_STATIC_SCRATCH_BYTES) == fits, (shape, nb)
        st, h = capi.lbm_create(d, FAKE)
        assert st == capi.LBM_OK
        try:
            assert noalloc(h, 0, FAKE) == capi.LBM_ERR_INVALID_ARGUMENT
            assert noalloc(h, 1, None) == capi.LBM_ERR_INVALID_ARGUMENT
            assert noalloc(h, 1, FAKE + 4) == capi.LBM_ERR_MISALIGNED
            assert noalloc(h, 1, FAKE) == (capi.LBM_ERR_BAD_STATE if fits else capi.LBM_ERR_UNSUPPORTED)
            assert capi.lbm_time(h) == 0
        finally:
            capi.lbm_destroy(h)


def test_open_faces_arguments():
    st, h = capi.lbm_create(capi.make_desc(8, 8, 8), FAKE)
    assert st == capi.LBM_OK
    try:
        assert capi.lbm_set_geometry(h, None, (0, 1, 1)) == capi.LBM_OK
        assert capi.lbm_set_open_faces(h, {"-x": (1.0, (0.01, 0, 0))}) == capi.LBM_OK
        # faces on the periodic y axis cannot be open
        assert capi.lbm_set_open_faces(h, {"+y": (1.0, (0, 0, 0))}) == capi.LBM_ERR_INVALID_ARGUMENT
        assert capi.lbm_set_open_faces(h, {"+x": (0.0, (0, 0, 0))}) == capi.LBM_ERR_INVALID_ARGUMENT
        assert capi.lbm_set_open_faces(h, {"+x": (1.0, (float("nan"), 0, 0))}) == capi.LBM_ERR_INVALID_ARGUMENT
        assert capi.lbm_set_open_faces(h, {}) == capi.LBM_OK
        assert capi.lbm_step(h, 1) == capi.LBM_ERR_BAD_STATE
    finally:
        capi.lbm_destroy(h)
    assert capi.lbm_set_open_faces(None, {}) == capi.LBM_ERR_INVALID_ARGUMENT


def _raw_open_faces(h, kinds, rho=1.0, u=(0.0, 0.0, 0.0)):
    import ctypes
    op = (ctypes.c_int32 * 6)(*kinds)
    r = (ctypes.c_double * 6)(*([rho] * 6))
    v = (ctypes.c_double * 18)(*(list(u) * 6))
    return capi._lib.lbm_set_open_faces(h, op, r, v)


def test_face_kinds_arguments():
    st, h = capi.lbm_create(capi.make_desc(8, 8, 8), FAKE)
    assert st == capi.LBM_OK
    try:
        assert capi.lbm_set_geometry(h, None, (0, 0, 1)) == capi.LBM_OK
        for kind in capi.FACE_KINDS:
            assert capi.lbm_set_open_faces(h, {"-x": (1.0, (0.02, 0, 0), kind),
                                                "+x": (1.0, (0.0, 0, 0), "zou_he_pressure")}) == capi.LBM_OK
        # kinds beyond the enum
        assert _raw_open_faces(h, (5, 0, 0, 0, 0, 0)) == capi.LBM_ERR_INVALID_ARGUMENT
        assert _raw_open_faces(h, (-1, 0, 0, 0, 0, 0)) == capi.LBM_ERR_INVALID_ARGUMENT
        # a rule face needs every open face on its axis
        assert capi.lbm_set_open_faces(h, {"-x": (1.0, (0, 0, 0), "neumann"),
                                           "+y": (1.0, (0, 0, 0))}) == capi.LBM_ERR_UNSUPPORTED
        assert capi.lbm_set_open_faces(h, {"-x": (1.0, (0, 0, 0)), "+y": (1.0, (0, 0, 0))}) == capi.LBM_OK
        # the velocity rule's density needs 1 - sigma u_a > 0 (inward speed below 1)
        assert capi.lbm_set_open_faces(h, {"-x": (1.0, (1.0, 0, 0), "zou_he_velocity")}) == \
            capi.LBM_ERR_INVALID_ARGUMENT
        assert capi.lbm_set_open_faces(h, {"+x": (1.0, (-1.0, 0, 0), "zou_he_velocity")}) == \
            capi.LBM_ERR_INVALID_ARGUMENT
        assert capi.lbm_set_open_faces(h, {"+x": (1.0, (1.0, 0, 0), "zou_he_velocity")}) == capi.LBM_OK
    finally:
        capi.lbm_destroy(h)
    # at least 3 cells along the rule face's axis
    st, h = capi.lbm_create(capi.make_desc(2, 8, 8), FAKE)
    assert st == capi.LBM_OK
    try:
        assert capi.lbm_set_geometry(h, None, (0, 1, 1)) == capi.LBM_OK
        assert capi.lbm_set_open_faces(h, {"-x": (1.0, (0, 0, 0), "zou_he_pressure")}) == capi.LBM_ERR_UNSUPPORTED
        assert capi.lbm_set_open_faces(h, {"-x": (1.0, (0, 0, 0))}) == capi.LBM_OK
    finally:
        capi.lbm_destroy(h)


def test_null_handle_and_status_strings():
    assert capi.lbm_destroy(None) == capi.LBM_OK
    assert capi.lbm_time(None) == -1
    assert capi.lbm_step(None, 1) == capi.LBM_ERR_INVALID_ARGUMENT
    for code in (0, -1, -2, -3, -4, -5):
        assert capi.lbm_status_string(code) and capi.lbm_status_string(code) != "unknown status"
    assert capi.lbm_status_string(42) == "unknown status"


def test_single_hip_runtime_in_process():
    # torch bundles its own libamdhip64 (same soname); the library must bind to
    # it rather than map a second HIP runtime (which would see no device).
    maps = open("/proc/self/maps").read()
    libs = {os.path.realpath(p) for p in re.findall(r"(/\S*libamdhip64\S*)", maps)}
    assert len(libs) == 1, libs


def test_workspace_rules():
    dense = capi.make_desc(10, 8, 6, layout=capi.LBM_LAYOUT_STREAM)
    comp = capi.make_desc(10, 8, 6, layout=capi.LBM_LAYOUT_COMPACT)
    st, wd = capi.lbm_workspace_bytes(dense)
    assert st == capi.LBM_OK and wd == 0
    st, wc = capi.lbm_workspace_bytes(comp)
    # index table over the halo-padded box + one index per cell + row table
    assert st == capi.LBM_OK and wc >= 4 * (12 * 10 * 8) + 4 * 480 + 4 * 48
    st, nb, _ = capi.lbm_buffer_bytes(comp)
    assert nb == 19 * 512 * 4          # room for an all-fluid box, rounded to 64 cells
    st, h = capi.lbm_create(comp, FAKE)
    assert st == capi.LBM_OK
    try:
        assert capi.lbm_fluid_cells(h) == -1
        assert capi.lbm_init_equilibrium(h) == capi.LBM_ERR_BAD_STATE     # no workspace yet
        assert capi.lbm_set_workspace(h, FAKE + 4, wc) == capi.LBM_ERR_MISALIGNED
        assert capi.lbm_set_workspace(h, FAKE, wc - 1) == capi.LBM_ERR_INVALID_ARGUMENT
        assert capi.lbm_set_workspace(h, FAKE, wc) == capi.LBM_OK
        assert capi.lbm_set_workspace(h, None, 0) == capi.LBM_OK
        assert capi.lbm_init_equilibrium(h) == capi.LBM_ERR_BAD_STATE
    finally:
        capi.lbm_destroy(h)
