// launch.hpp -- host-side launchers between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lbm {

struct LaunchGeom {
    int64_t nx, ny, nz;
    int32_t periodic[3];
    const uint8_t* mask;
    int32_t xcd_remap;
};

struct LaunchPhys {
    double omega;
    double force[3];
    bool has_force;
};

// One fused step of kind `kind` (kAB: a = source, b = destination; kAAEven /
// kAAOdd: a = the lattice, b unused) over the whole box.
template <typename T>
hipError_t launch_step(int layout, int kind, T* a, T* b, const LaunchGeom& g, const LaunchPhys& p,
                       hipStream_t s);

// Canonical-state transfer `op` (an IoOp) for a stored state of kind `state`.
template <typename T>
hipError_t launch_io(int layout, int state, int op, T* a, T* b, const LaunchGeom& g, const LaunchPhys& p,
                     T* out0, T* out1, const T* in0, const T* in1, hipStream_t s);

}  // namespace lbm
