// capi.cpp -- the C ABI of liblbm.so (declared in include/lbm.h).
//
// Validation and the state machine live here, on the host; every GPU action
// is a kernel launch through launch.hpp on the handle's stream.
//
// Stored state per scheme (what "canonical f(t)" is read from):
//   AB: buffer `cur` holds h(t), the post-collision values of step t-1 (for
//       t = 0: the streaming pre-image of f(0)), so that f(t) = stream(h(t))
//       and one fused pull-collide step maps h(t) to h(t+1) in the other
//       buffer.
//   AA: the single buffer holds f(t) in natural slots when t is even, and the
//       post-collision values of step t-1 in the swapped slots of the
//       in-place pattern when t is odd (fieldcraft page, first section).
//   ESOPULL: the single buffer holds f(t) in the slots of the esoteric pull
//       of parity t % 2 (each pair's own-cell and neighbour slots swap roles
//       every step).
//   ESOTWIST: the single buffer holds f(t) in the slots of the esoteric twist
//       of parity t % 2: f_q(x) at the location x - max(c_q, 0), in plane q
//       when t is even and plane opposite(q) when t is odd (dense layouts: a
//       halo layer below each low face; compact layout: ghost cells after the
//       fluid ones).
// In every scheme the values are stored shifted by the lattice weights
// (f - w).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <new>

#include "../../include/lbm.h"
#include "d3q19.hpp"
#include "kernels.hpp"
#include "kernels_faces.hpp"
#include "launch.hpp"

static_assert(lbm::kRuleNeumann == LBM_FACE_NEUMANN && lbm::kRuleZouHePressure == LBM_FACE_ZOU_HE_PRESSURE &&
                  lbm::kRuleZouHeVelocity == LBM_FACE_ZOU_HE_VELOCITY,
              "face kinds of the kernels and of the C ABI");

struct lbm_sim {
    lbm_desc d;
    void* buf[2];
    hipStream_t stream;
    const uint8_t* mask;
    int32_t periodic[3];
    void* ws;  // caller-owned workspace (compact layout tables)
    size_t ws_bytes;
    lbm::CompactTables tables;
    bool initialized;
    int64_t t;
    int cur;  // AB: index of the buffer holding h(t)
    double omega;
    hipError_t last_hip;  // status of the last failed launch (hipSuccess if none)
    uint32_t open;        // open faces (bit k: -x, +x, -y, +y, -z, +z)
    int32_t face_kind[6]; // 0 closed, 1 reservoir, 2 Neumann, 3 Zou-He pressure, 4 Zou-He velocity
    double face_rho[6];
    double face_u[6][3];
    int xcd8;  // the device has 8 XCDs: -1 not asked yet, then 0 or 1
};

// Device scratch of lbm_step_momentum_exchange_noalloc: the per-workgroup
// partial rows of the momentum-exchange sums (6 doubles per row), for callers
// that cannot allocate.  Every GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not the device memory: its device address comes from hipGetSymbolAddress,
// once per device (static_scratch below), and only that address is used.
constexpr size_t kStaticScratchBytes = size_t(4) << 20;  // 4 MiB: 87,381 rows
static __device__ __align__(256) double scratch[kStaticScratchBytes / sizeof(double)];
static_assert(kStaticScratchBytes == LBM_STATIC_SCRATCH_BYTES, "the header states the scratch size");

namespace {

constexpr uintptr_t kAlign = 256;

bool compact(const lbm_desc& d) { return d.layout == LBM_LAYOUT_COMPACT; }

uint64_t ncells(const lbm_desc& d) { return (uint64_t)d.nx * (uint64_t)d.ny * (uint64_t)d.nz; }

// Stored cells a compact buffer has room for: every cell of the box, and for
// the esoteric twist also the halo below the low faces (its ghost cells lie
// among the box's solid cells and in that halo); rounded up to 64.
uint64_t compact_capacity(const lbm_desc& d)
{
    const uint64_t cells = d.scheme == LBM_SCHEME_ESOTWIST
                               ? (uint64_t)(d.nx + 1) * (uint64_t)(d.ny + 1) * (uint64_t)(d.nz + 1)
                               : ncells(d);
    return (cells + 63) / 64 * 64;
}

lbm_status validate_desc(const lbm_desc* d)
{
    if (d == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    if (d->nx < 1 || d->ny < 1 || d->nz < 1) return LBM_ERR_INVALID_ARGUMENT;
    if (d->precision != LBM_F32 && d->precision != LBM_F64) return LBM_ERR_INVALID_ARGUMENT;
    if (d->layout != LBM_LAYOUT_STREAM && d->layout != LBM_LAYOUT_BUNDLE && d->layout != LBM_LAYOUT_COLLISION &&
        d->layout != LBM_LAYOUT_COMPACT)
        return LBM_ERR_INVALID_ARGUMENT;
    if (d->scheme != LBM_SCHEME_AB && d->scheme != LBM_SCHEME_AA && d->scheme != LBM_SCHEME_ESOPULL &&
        d->scheme != LBM_SCHEME_ESOTWIST)
        return LBM_ERR_INVALID_ARGUMENT;
    if (d->reserved != 0) return LBM_ERR_INVALID_ARGUMENT;
    if (std::isnan(d->tau) || !(d->tau > 0.5)) return LBM_ERR_INVALID_ARGUMENT;
    for (int a = 0; a < 3; ++a)
        if (!std::isfinite(d->force[a])) return LBM_ERR_INVALID_ARGUMENT;
    // cell indices are 32-bit inside the kernels; so is the padded index of
    // the compact layout's neighbour table
    const double n = (double)d->nx * (double)d->ny * (double)d->nz;
    if (d->nx > INT32_MAX || d->ny > INT32_MAX || d->nz > INT32_MAX || n >= 2147483648.0)
        return LBM_ERR_UNSUPPORTED;
    // the dense esoteric twist stores a halo layer below each low face and
    // addresses its (nx+1)(ny+1)(nz+1) cells with 32-bit indices
    if (!compact(*d) && d->scheme == LBM_SCHEME_ESOTWIST &&
        (double)(d->nx + 1) * (double)(d->ny + 1) * (double)(d->nz + 1) >= 2147483648.0)
        return LBM_ERR_UNSUPPORTED;
    // the compact kernels address the padded index table with 32-bit byte
    // offsets (the populations with 64-bit ones)
    if (compact(*d) && 4.0 * (double)(d->nx + 2) * (double)(d->ny + 2) * (double)(d->nz + 2) >= 4294967296.0)
        return LBM_ERR_UNSUPPORTED;
    return LBM_OK;
}

size_t elem_size(const lbm_desc& d) { return d.precision == LBM_F64 ? 8 : 4; }

// Population buffer size; the compact layout reserves room for an all-fluid
// box, and its esoteric pull nine more planes' worth of bounce-back slots.
size_t buffer_bytes(const lbm_desc& d)
{
    uint64_t cells = compact(d) ? compact_capacity(d) : ncells(d);
    if (!compact(d) && d.scheme == LBM_SCHEME_ESOTWIST)
        cells = (uint64_t)(d.nx + 1) * (uint64_t)(d.ny + 1) * (uint64_t)(d.nz + 1);
    const uint64_t planes = compact(d) && d.scheme == LBM_SCHEME_ESOPULL ? lbm::kEsoPlanes : lbm::kQ;
    return (size_t)planes * cells * elem_size(d);
}

// open faces that are equilibrium reservoirs (applied inside the steps)
uint32_t reservoir_bits(const lbm_sim* s)
{
    uint32_t b = 0;
    for (int k = 0; k < 6; ++k)
        if (((s->open >> k) & 1u) && s->face_kind[k] == LBM_FACE_EQUILIBRIUM) b |= 1u << k;
    return b;
}

lbm::LaunchGeom geom_of(const lbm_sim* s)
{
    lbm::LaunchGeom g{};
    g.nx = s->d.nx;
    g.ny = s->d.ny;
    g.nz = s->d.nz;
    for (int a = 0; a < 3; ++a) g.periodic[a] = s->periodic[a];
    g.open = s->open;
    g.res = reservoir_bits(s);
    g.mask = s->mask;
    g.xcd8 = s->xcd8 == 1;
    return g;
}

// Whether the current device has the 8 XCDs the chunked workgroup orders are
// laid out for (asked once, at the first initialisation); 0 if the runtime
// cannot tell.
void ask_xcd8(lbm_sim* s)
{
    if (s->xcd8 >= 0) return;
    int dev = 0, n = 0;
    s->xcd8 = hipGetDevice(&dev) == hipSuccess &&
                      hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && n == 8
                  ? 1
                  : 0;
}

lbm::LaunchPhys phys_of(const lbm_sim* s)
{
    lbm::LaunchPhys p{};
    p.omega = s->omega;
    p.has_force = false;
    for (int a = 0; a < 3; ++a) {
        p.force[a] = s->d.force[a];
        if (s->d.force[a] != 0.0) p.has_force = true;
    }
    for (int k = 0; k < 6; ++k) {
        p.face_rho[k] = s->face_rho[k];
        for (int a = 0; a < 3; ++a) p.face_u[k][a] = s->face_u[k][a];
        p.face_kind[k] = s->face_kind[k];
    }
    p.res = reservoir_bits(s);
    return p;
}

// Kind of the stored state at the current time.
int state_kind(const lbm_sim* s)
{
    if (s->d.scheme == LBM_SCHEME_AB) return lbm::kAB;
    if (s->d.scheme == LBM_SCHEME_ESOPULL) return (s->t % 2 == 0) ? lbm::kEsoEven : lbm::kEsoOdd;
    if (s->d.scheme == LBM_SCHEME_ESOTWIST) return (s->t % 2 == 0) ? lbm::kTwEven : lbm::kTwOdd;
    return (s->t % 2 == 0) ? lbm::kAAEven : lbm::kAAOdd;
}

lbm_status hip_status(lbm_sim* s, hipError_t e)
{
    if (e == hipSuccess) return LBM_OK;
    s->last_hip = e;
    return LBM_ERR_HIP;
}

lbm_status io(lbm_sim* s, int op, void* out0, void* out1, const void* in0, const void* in1)
{
    const lbm::LaunchGeom g = geom_of(s);
    const lbm::LaunchPhys p = phys_of(s);
    const int st = state_kind(s);
    void* a = s->d.scheme == LBM_SCHEME_AB ? s->buf[s->cur] : s->buf[0];
    hipError_t e;
    if (compact(s->d)) {
        if (s->d.precision == LBM_F32)
            e = lbm::launch_io_compact<float>(st, op, (float*)a, g, s->tables, p, (float*)out0, (float*)out1,
                                              (const float*)in0, (const float*)in1, s->stream);
        else
            e = lbm::launch_io_compact<double>(st, op, (double*)a, g, s->tables, p, (double*)out0, (double*)out1,
                                               (const double*)in0, (const double*)in1, s->stream);
        return hip_status(s, e);
    }
    void* b = (s->d.scheme == LBM_SCHEME_AB && op == lbm::kWriteEq) ? s->buf[1 - s->cur] : nullptr;
    if (s->d.precision == LBM_F32)
        e = lbm::launch_io<float>(s->d.layout, st, op, (float*)a, (float*)b, g, p, (float*)out0, (float*)out1,
                                  (const float*)in0, (const float*)in1, s->stream);
    else
        e = lbm::launch_io<double>(s->d.layout, st, op, (double*)a, (double*)b, g, p, (double*)out0,
                                   (double*)out1, (const double*)in0, (const double*)in1, s->stream);
    return hip_status(s, e);
}

// The face rules of the open faces that are not reservoirs, on the stored
// state (after an initialisation, a write of populations, or a step).
lbm_status apply_face_rules(lbm_sim* s)
{
    if ((s->open & ~reservoir_bits(s)) == 0) return LBM_OK;
    const lbm::LaunchGeom g = geom_of(s);
    const lbm::LaunchPhys p = phys_of(s);
    const int st = state_kind(s);
    void* a = s->d.scheme == LBM_SCHEME_AB ? s->buf[s->cur] : s->buf[0];
    const lbm::CompactTables* t = compact(s->d) ? &s->tables : nullptr;
    hipError_t e;
    if (s->d.precision == LBM_F32)
        e = lbm::launch_face_rules<float>(s->d.layout, st, (float*)a, g, t, p, s->stream);
    else
        e = lbm::launch_face_rules<double>(s->d.layout, st, (double*)a, g, t, p, s->stream);
    return hip_status(s, e);
}

// Compact layout: build the tables, then learn the fluid count (one wait).
lbm_status build_compact(lbm_sim* s)
{
    if (s->ws == nullptr) return LBM_ERR_BAD_STATE;
    const bool eso = s->d.scheme == LBM_SCHEME_ESOPULL, twist = s->d.scheme == LBM_SCHEME_ESOTWIST;
    const lbm::CompactLayoutBytes lay = lbm::compact_workspace_layout(s->d.nx, s->d.ny, s->d.nz, eso, twist);
    char* base = (char*)s->ws;
    lbm::CompactTables& t = s->tables;
    t.header = (uint32_t*)(base + lay.header);
    t.rows = (uint32_t*)(base + lay.rows);
    t.idxp = (uint32_t*)(base + lay.idxp);
    t.cellp = (uint32_t*)(base + lay.cellp);
    t.cellid = (uint32_t*)(base + lay.cellid);
    t.bbase = eso ? (uint32_t*)(base + lay.bbase) : nullptr;
    t.tidx = twist ? (uint32_t*)(base + lay.tidx) : nullptr;
    t.grows = twist ? (uint32_t*)(base + lay.grows) : nullptr;
    t.nf = 0;
    t.stride = 0;
    hipError_t e = lbm::launch_compact_build(geom_of(s), t, s->stream);
    if (e != hipSuccess) return hip_status(s, e);
    uint32_t nf = 0;
    e = hipMemcpyAsync(&nf, t.header, sizeof(nf), hipMemcpyDeviceToHost, s->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(s->stream);
    if (e != hipSuccess) return hip_status(s, e);
    t.nf = nf;
    t.stride = ((uint64_t)nf + 63) / 64 * 64;
    if (twist) {
        // ghost cells after the fluid ones: the stride covers both
        e = lbm::launch_compact_twist(geom_of(s), t, s->stream);
        uint32_t ng = 0;
        if (e == hipSuccess) e = hipMemcpyAsync(&ng, t.header + 2, sizeof(ng), hipMemcpyDeviceToHost, s->stream);
        if (e == hipSuccess) e = hipStreamSynchronize(s->stream);
        if (e != hipSuccess) return hip_status(s, e);
        t.stride = ((uint64_t)nf + ng + 63) / 64 * 64;
    }
    return hip_status(s, lbm::launch_compact_bounce(geom_of(s), t, s->stream));
}

}  // namespace

extern "C" {

lbm_status lbm_buffer_bytes(const lbm_desc* desc, size_t* bytes_per_buffer, int32_t* n_buffers)
{
    const lbm_status v = validate_desc(desc);
    if (v != LBM_OK) return v;
    if (bytes_per_buffer == nullptr && n_buffers == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    if (bytes_per_buffer) *bytes_per_buffer = buffer_bytes(*desc);
    if (n_buffers) *n_buffers = desc->scheme == LBM_SCHEME_AB ? 2 : 1;
    return LBM_OK;
}

lbm_status lbm_workspace_bytes(const lbm_desc* desc, size_t* bytes)
{
    const lbm_status v = validate_desc(desc);
    if (v != LBM_OK) return v;
    if (bytes == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    *bytes = compact(*desc) ? lbm::compact_workspace_layout(desc->nx, desc->ny, desc->nz,
                                                             desc->scheme == LBM_SCHEME_ESOPULL,
                                                             desc->scheme == LBM_SCHEME_ESOTWIST)
                                  .total
                            : 0;
    return LBM_OK;
}

lbm_status lbm_create(const lbm_desc* desc, void* buf0, void* buf1, void* hip_stream, lbm_sim** out)
{
    if (out == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    const lbm_status v = validate_desc(desc);
    if (v != LBM_OK) return v;
    if (buf0 == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    if (desc->scheme != LBM_SCHEME_AB && buf1 != nullptr) return LBM_ERR_INVALID_ARGUMENT;
    if (desc->scheme == LBM_SCHEME_AB && buf1 == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    if ((uintptr_t)buf0 % kAlign != 0 || (buf1 && (uintptr_t)buf1 % kAlign != 0)) return LBM_ERR_MISALIGNED;
    if (buf1 != nullptr) {
        const uintptr_t bytes = (uintptr_t)buffer_bytes(*desc);
        const uintptr_t p0 = (uintptr_t)buf0, p1 = (uintptr_t)buf1;
        if (p0 < p1 + bytes && p1 < p0 + bytes) return LBM_ERR_INVALID_ARGUMENT;  // overlap
    }
    lbm_sim* s = new (std::nothrow) lbm_sim{};
    if (s == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    s->d = *desc;
    s->buf[0] = buf0;
    s->buf[1] = buf1;
    s->stream = (hipStream_t)hip_stream;
    s->mask = nullptr;
    s->periodic[0] = s->periodic[1] = s->periodic[2] = 1;
    s->ws = nullptr;
    s->ws_bytes = 0;
    s->initialized = false;
    s->t = 0;
    s->cur = 0;
    s->xcd8 = -1;
    s->omega = std::isinf(desc->tau) ? 0.0 : 1.0 / desc->tau;
    s->last_hip = hipSuccess;
    *out = s;
    return LBM_OK;
}

lbm_status lbm_set_workspace(lbm_sim* sim, void* ws, size_t bytes)
{
    if (sim == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    if (ws != nullptr && (uintptr_t)ws % kAlign != 0) return LBM_ERR_MISALIGNED;
    size_t need = 0;
    lbm_workspace_bytes(&sim->d, &need);
    if (ws != nullptr && bytes < need) return LBM_ERR_INVALID_ARGUMENT;
    sim->ws = ws;
    sim->ws_bytes = ws == nullptr ? 0 : bytes;
    sim->initialized = false;
    sim->t = 0;
    sim->cur = 0;
    return LBM_OK;
}

lbm_status lbm_set_geometry(lbm_sim* sim, const uint8_t* mask, const int32_t periodic[3])
{
    if (sim == nullptr || periodic == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    for (int a = 0; a < 3; ++a)
        if (periodic[a] != 0 && periodic[a] != 1) return LBM_ERR_INVALID_ARGUMENT;
    sim->mask = mask;
    for (int a = 0; a < 3; ++a) sim->periodic[a] = periodic[a];
    sim->open = 0;
    for (int k = 0; k < 6; ++k) sim->face_kind[k] = 0;
    sim->initialized = false;
    sim->t = 0;
    sim->cur = 0;
    return LBM_OK;
}

lbm_status lbm_set_open_faces(lbm_sim* sim, const int32_t open[6], const double rho[6], const double u[18])
{
    if (sim == nullptr || open == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    uint32_t bits = 0, axes = 0;
    bool rules = false;
    for (int k = 0; k < 6; ++k) {
        if (open[k] < 0 || open[k] > LBM_FACE_ZOU_HE_VELOCITY) return LBM_ERR_INVALID_ARGUMENT;
        if (!open[k]) continue;
        if (sim->periodic[k / 2] || rho == nullptr || u == nullptr) return LBM_ERR_INVALID_ARGUMENT;
        if (!std::isfinite(rho[k]) || !(rho[k] > 0.0)) return LBM_ERR_INVALID_ARGUMENT;
        for (int a = 0; a < 3; ++a)
            if (!std::isfinite(u[3 * k + a])) return LBM_ERR_INVALID_ARGUMENT;
        // the velocity rule's density is (par + 2 out) / (1 - sigma u_a)
        const double sg = (k % 2 == 0) ? 1.0 : -1.0;
        if (open[k] == LBM_FACE_ZOU_HE_VELOCITY && !(sg * u[3 * k + k / 2] < 1.0)) return LBM_ERR_INVALID_ARGUMENT;
        bits |= 1u << k;
        axes |= 1u << (k / 2);
        rules = rules || open[k] != LBM_FACE_EQUILIBRIUM;
    }
    if (rules) {
        // every open face on one axis, at least 3 cells along it: the rules'
        // cells are then independent (none reads what another writes)
        const int64_t n[3] = {sim->d.nx, sim->d.ny, sim->d.nz};
        if (axes != 1u && axes != 2u && axes != 4u) return LBM_ERR_UNSUPPORTED;
        const int a = axes == 1u ? 0 : axes == 2u ? 1 : 2;
        if (n[a] < 3) return LBM_ERR_UNSUPPORTED;
    }
    sim->open = bits;
    for (int k = 0; k < 6; ++k) {
        const bool o = (bits >> k) & 1u;
        sim->face_kind[k] = o ? open[k] : 0;
        sim->face_rho[k] = o ? rho[k] : 1.0;
        for (int a = 0; a < 3; ++a) sim->face_u[k][a] = o ? u[3 * k + a] : 0.0;
    }
    sim->initialized = false;
    sim->t = 0;
    sim->cur = 0;
    return LBM_OK;
}

lbm_status lbm_init_equilibrium(lbm_sim* sim, const void* rho, const void* u)
{
    if (sim == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    if (compact(sim->d) && sim->ws == nullptr) return LBM_ERR_BAD_STATE;
    sim->t = 0;
    sim->cur = 0;
    sim->initialized = false;
    ask_xcd8(sim);
    if (compact(sim->d)) {
        const lbm_status b = build_compact(sim);
        if (b != LBM_OK) return b;
    }
    lbm_status r = io(sim, lbm::kWriteEq, nullptr, nullptr, rho, u);
    if (r == LBM_OK) r = apply_face_rules(sim);
    if (r == LBM_OK) sim->initialized = true;
    return r;
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device dev: looked up on the first call for
// that device, with that device current, and kept.  nullptr (and the HIP
// error in *err) if the lookup fails.
void* static_scratch(int dev, hipError_t* err)
{
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] != nullptr) return g_scratch_ptr[dev];
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e == hipSuccess && prev != dev) e = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (prev >= 0 && prev != dev) {
        const hipError_t back = hipSetDevice(prev);
        if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess || ptr == nullptr) {
        *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
        return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
    return ptr;
}

// n steps; the last one also writes the density and velocity its collision
// used into rho / u when they are given, or sums its momentum exchange into
// force (partial: the scratch rows) when that is given.
lbm_status run_steps(lbm_sim* sim, int64_t n, void* rho, void* u, double* force = nullptr,
                     double* partial = nullptr)
{
    const lbm::LaunchGeom g = geom_of(sim);
    const lbm::LaunchPhys p = phys_of(sim);
    for (int64_t i = 0; i < n; ++i) {
        int kind;
        void *a, *b = nullptr;
        if (sim->d.scheme == LBM_SCHEME_AB) {
            kind = lbm::kAB;
            a = sim->buf[sim->cur];
            b = sim->buf[1 - sim->cur];
        } else {
            kind = state_kind(sim);
            a = sim->buf[0];
        }
        void* ro = i + 1 == n ? rho : nullptr;
        void* uo = i + 1 == n ? u : nullptr;
        hipError_t e;
        const lbm::CompactTables* t = compact(sim->d) ? &sim->tables : nullptr;
        if (force != nullptr && i + 1 == n) {
            if (sim->d.precision == LBM_F32)
                e = lbm::launch_step_mex<float>(sim->d.layout, kind, (float*)a, (float*)b, g, t, p, partial, force,
                                                sim->stream);
            else
                e = lbm::launch_step_mex<double>(sim->d.layout, kind, (double*)a, (double*)b, g, t, p, partial,
                                                 force, sim->stream);
        } else if (t != nullptr) {
            if (sim->d.precision == LBM_F32)
                e = lbm::launch_step_compact<float>(kind, (float*)a, (float*)b, g, sim->tables, p, (float*)ro,
                                                    (float*)uo, sim->stream);
            else
                e = lbm::launch_step_compact<double>(kind, (double*)a, (double*)b, g, sim->tables, p, (double*)ro,
                                                     (double*)uo, sim->stream);
        } else if (sim->d.precision == LBM_F32) {
            e = lbm::launch_step<float>(sim->d.layout, kind, (float*)a, (float*)b, g, p, (float*)ro, (float*)uo,
                                        sim->stream);
        } else {
            e = lbm::launch_step<double>(sim->d.layout, kind, (double*)a, (double*)b, g, p, (double*)ro,
                                         (double*)uo, sim->stream);
        }
        if (e != hipSuccess) return hip_status(sim, e);
        if (sim->d.scheme == LBM_SCHEME_AB) sim->cur = 1 - sim->cur;
        sim->t += 1;
        const lbm_status r = apply_face_rules(sim);
        if (r != LBM_OK) return r;
    }
    return LBM_OK;
}

}  // namespace

extern "C" {

lbm_status lbm_step(lbm_sim* sim, int64_t n)
{
    if (sim == nullptr || n < 0) return LBM_ERR_INVALID_ARGUMENT;
    if (!sim->initialized) return LBM_ERR_BAD_STATE;
    return run_steps(sim, n, nullptr, nullptr);
}

lbm_status lbm_step_moments(lbm_sim* sim, int64_t n, void* rho, void* u)
{
    if (sim == nullptr || n < 1 || rho == nullptr || u == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    if (!sim->initialized) return LBM_ERR_BAD_STATE;
    return run_steps(sim, n, rho, u);
}

lbm_status lbm_step_momentum_exchange(lbm_sim* sim, int64_t n, void* force, void* scratch, size_t scratch_bytes)
{
    if (sim == nullptr || n < 1 || force == nullptr || scratch == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    size_t need = 0;
    lbm_momentum_exchange_scratch_bytes(&sim->d, &need);
    if (scratch_bytes < need) return LBM_ERR_INVALID_ARGUMENT;
    if ((uintptr_t)scratch % kAlign != 0 || (uintptr_t)force % sizeof(double) != 0) return LBM_ERR_MISALIGNED;
    if (!sim->initialized) return LBM_ERR_BAD_STATE;
    return run_steps(sim, n, nullptr, nullptr, (double*)force, (double*)scratch);
}

lbm_status lbm_step_momentum_exchange_noalloc(lbm_sim* sim, int64_t n, void* force)
{
    if (sim == nullptr || n < 1 || force == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    if ((uintptr_t)force % sizeof(double) != 0) return LBM_ERR_MISALIGNED;
    size_t need = 0;
    lbm_momentum_exchange_scratch_bytes(&sim->d, &need);
    if (need > kStaticScratchBytes) return LBM_ERR_UNSUPPORTED;
    if (!sim->initialized) return LBM_ERR_BAD_STATE;
    int dev = 0;
    hipError_t e = sim->stream != nullptr ? hipStreamGetDevice(sim->stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(sim, e);
    if (dev < 0 || dev >= kMaxDevices) return LBM_ERR_UNSUPPORTED;
    void* ptr = static_scratch(dev, &e);
    if (ptr == nullptr) return hip_status(sim, e);
    return run_steps(sim, n, nullptr, nullptr, (double*)force, (double*)ptr);
}

lbm_status lbm_moments(lbm_sim* sim, void* rho, void* u)
{
    if (sim == nullptr || rho == nullptr || u == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    if (!sim->initialized) return LBM_ERR_BAD_STATE;
    return io(sim, lbm::kReadMoments, rho, u, nullptr, nullptr);
}

lbm_status lbm_read_populations(lbm_sim* sim, void* f)
{
    if (sim == nullptr || f == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    if (!sim->initialized) return LBM_ERR_BAD_STATE;
    return io(sim, lbm::kReadF, f, nullptr, nullptr, nullptr);
}

lbm_status lbm_write_populations(lbm_sim* sim, const void* f)
{
    if (sim == nullptr || f == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    if (!sim->initialized) return LBM_ERR_BAD_STATE;
    const lbm_status r = io(sim, lbm::kWriteF, nullptr, nullptr, f, nullptr);
    return r == LBM_OK ? apply_face_rules(sim) : r;
}

lbm_status lbm_save_state(lbm_sim* sim, void* s)
{
    if (sim == nullptr || s == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    if (!sim->initialized) return LBM_ERR_BAD_STATE;
    return io(sim, lbm::kReadS, s, nullptr, nullptr, nullptr);
}

lbm_status lbm_load_state(lbm_sim* sim, const void* s)
{
    if (sim == nullptr || s == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    if (!sim->initialized) return LBM_ERR_BAD_STATE;
    return io(sim, lbm::kWriteS, nullptr, nullptr, s, nullptr);
}

lbm_status lbm_momentum_exchange_scratch_bytes(const lbm_desc* desc, size_t* bytes)
{
    const lbm_status v = validate_desc(desc);
    if (v != LBM_OK) return v;
    if (bytes == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    lbm::LaunchGeom g{};
    g.nx = desc->nx;
    g.ny = desc->ny;
    g.nz = desc->nz;
    *bytes = 6 * sizeof(double) * lbm::mex_partial_rows(g);
    return LBM_OK;
}

lbm_status lbm_momentum_exchange(lbm_sim* sim, void* force, void* scratch, size_t scratch_bytes)
{
    if (sim == nullptr || force == nullptr || scratch == nullptr) return LBM_ERR_INVALID_ARGUMENT;
    size_t need = 0;
    lbm_momentum_exchange_scratch_bytes(&sim->d, &need);
    if (scratch_bytes < need) return LBM_ERR_INVALID_ARGUMENT;
    if ((uintptr_t)scratch % kAlign != 0 || (uintptr_t)force % sizeof(double) != 0) return LBM_ERR_MISALIGNED;
    if (!sim->initialized) return LBM_ERR_BAD_STATE;
    const lbm::LaunchGeom g = geom_of(sim);
    const lbm::LaunchPhys p = phys_of(sim);
    const int st = state_kind(sim);
    void* a = sim->d.scheme == LBM_SCHEME_AB ? sim->buf[sim->cur] : sim->buf[0];
    const lbm::CompactTables* t = compact(sim->d) ? &sim->tables : nullptr;
    hipError_t e;
    if (sim->d.precision == LBM_F32)
        e = lbm::launch_momentum_exchange<float>(sim->d.layout, st, (float*)a, g, t, p, (double*)scratch,
                                                 (double*)force, sim->stream);
    else
        e = lbm::launch_momentum_exchange<double>(sim->d.layout, st, (double*)a, g, t, p, (double*)scratch,
                                                  (double*)force, sim->stream);
    return hip_status(sim, e);
}

lbm_status lbm_destroy(lbm_sim* sim)
{
    delete sim;
    return LBM_OK;
}

int64_t lbm_time(const lbm_sim* sim) { return sim == nullptr ? -1 : sim->t; }

int64_t lbm_fluid_cells(const lbm_sim* sim)
{
    if (sim == nullptr || !sim->initialized || !compact(sim->d)) return -1;
    return (int64_t)sim->tables.nf;
}

const char* lbm_last_hip_error(const lbm_sim* sim)
{
    if (sim == nullptr) return "no handle";
    return hipGetErrorName(sim->last_hip);
}

const char* lbm_status_string(lbm_status status)
{
    switch (status) {
    case LBM_OK: return "ok";
    case LBM_ERR_INVALID_ARGUMENT: return "invalid argument";
    case LBM_ERR_UNSUPPORTED: return "unsupported size or option";
    case LBM_ERR_BAD_STATE: return "call out of order (create, [set_workspace, set_geometry], init, then step)";
    case LBM_ERR_MISALIGNED: return "device buffer not 256-byte aligned";
    case LBM_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
    }
}

}  // extern "C"
