// launch.hpp -- host-side launchers between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lbm {

struct LaunchGeom {
    int64_t nx, ny, nz;
    int32_t periodic[3];
    uint32_t open;  // bit k: face k (-x, +x, -y, +y, -z, +z) is open (its axis is not periodic)
    uint32_t res;   // bit k: open face k is an equilibrium reservoir (the others have face rules)
    const uint8_t* mask;
    // the device has 8 XCDs, over which the dispatcher deals workgroups
    // round robin: the XCD-chunked workgroup orders assume that layout and
    // are used only then (otherwise the hardware order)
    bool xcd8;
};

struct LaunchPhys {
    double omega;
    double force[3];
    bool has_force;
    double face_rho[6];     // prescribed values of each open face
    double face_u[6][3];
    int32_t face_kind[6];   // 0 closed, 1 reservoir, kRuleNeumann, kRuleZouHePressure, kRuleZouHeVelocity
    uint32_t res;           // bit k: face_kind[k] == 1
};

// One fused step of kind `kind` (kAB: a = source, b = destination; kAAEven /
// kAAOdd: a = the lattice, b unused) over the whole box.
// rho_out / u_out: device T[N] / T[3][N] for the density and velocity the
// step's collision uses (0 on solid cells), or null.
template <typename T>
hipError_t launch_step(int layout, int kind, T* a, T* b, const LaunchGeom& g, const LaunchPhys& p, T* rho_out,
                       T* u_out, hipStream_t s);

// Canonical-state transfer `op` (an IoOp) for a stored state of kind `state`.
template <typename T>
hipError_t launch_io(int layout, int state, int op, T* a, T* b, const LaunchGeom& g, const LaunchPhys& p,
                     T* out0, T* out1, const T* in0, const T* in1, hipStream_t s);

// Tables of the fluid-compacted layout, carved out of the caller's workspace.
struct CompactTables {
    uint32_t* header;  // [0] = fluid cell count, written by the build
    uint32_t* rows;    // per x-row fluid counts, then their exclusive scan
    uint32_t* idxp;    // halo-padded cell -> compact index (kInvalid: solid / wall)
    uint32_t* cellp;   // compact index -> padded cell
    uint32_t* cellid;  // compact index -> cell index
    uint32_t* bbase;   // esoteric pull: first bounce-back slot of each fluid cell (else null)
    uint32_t* tidx;    // esoteric twist: stored index of each padded cell (else null)
    uint32_t* grows;   // esoteric twist: ghost cells per padded row, then their exclusive scan
    uint32_t nf;       // fluid cells (known on the host after the build)
    uint64_t stride;   // population stride, nf rounded up to 64
};

// Byte offsets of the tables inside a workspace, and its size.
struct CompactLayoutBytes {
    size_t header, rows, idxp, cellp, cellid, bbase, tidx, grows, total;
};
// bounce: also the esoteric pull's bounce-back slot table (4 bytes per cell);
// twist: also the esoteric twist's stored-index table and ghost row counts
CompactLayoutBytes compact_workspace_layout(int64_t nx, int64_t ny, int64_t nz, bool bounce, bool twist);

// Build the compact tables from the mask and the periodic flags.
hipError_t launch_compact_build(const LaunchGeom& g, const CompactTables& t, hipStream_t s);

// Esoteric pull: bbase[i] = number of bounce-back links (x + c_k not fluid,
// k < 9) of the fluid cells before i (an exclusive scan); needs t.nf.
hipError_t launch_compact_bounce(const LaunchGeom& g, const CompactTables& t, hipStream_t s);

// Esoteric twist: ghost cells and the stored-index table tidx (fluid cells
// keep their indices, ghosts follow from nf in cell order); header[2] = the
// ghost count.  Needs t.nf; no-op if t.tidx is null.
hipError_t launch_compact_twist(const LaunchGeom& g, const CompactTables& t, hipStream_t s);

template <typename T>
hipError_t launch_step_compact(int kind, T* a, T* b, const LaunchGeom& g, const CompactTables& t,
                               const LaunchPhys& p, T* rho_out, T* u_out, hipStream_t s);

template <typename T>
hipError_t launch_io_compact(int state, int op, T* a, const LaunchGeom& g, const CompactTables& t,
                             const LaunchPhys& p, T* out0, T* out1, const T* in0, const T* in1, hipStream_t s);

// Face rules of the open faces that are not reservoirs, applied to the state
// of kind `state` that a step (or an initialisation) just left in `a`; one
// launch per such face.  t: the compact tables, or null for a dense layout.
template <typename T>
hipError_t launch_face_rules(int layout, int state, T* a, const LaunchGeom& g, const CompactTables* t,
                             const LaunchPhys& p, hipStream_t s);

// Momentum exchange with the solids for the step that starts from the stored
// state: force[0..2] on the mask's solid cells, force[3..5] on the walls
// (device double[6]).  partial: device double[6 * mex_partial_rows(g)].
size_t mex_partial_rows(const LaunchGeom& g);

template <typename T>
hipError_t launch_momentum_exchange(int layout, int state, T* a, const LaunchGeom& g, const CompactTables* t,
                                    const LaunchPhys& p, double* partial, double* force, hipStream_t s);

// One step of kind `kind` (as launch_step / launch_step_compact; t null for a
// dense layout) that also sums the momentum exchange of its own bounce-back
// links into force[0..5] (as launch_momentum_exchange for the state the step
// starts from).  partial: device double[6 * mex_partial_rows(g)].
template <typename T>
hipError_t launch_step_mex(int layout, int kind, T* a, T* b, const LaunchGeom& g, const CompactTables* t,
                           const LaunchPhys& p, double* partial, double* force, hipStream_t s);

}  // namespace lbm
