// kernels_compact.hpp -- the fluid-compacted SoA layout ("compact").
//
// Only fluid cells are stored: population q of the i-th fluid cell (fluid
// cells ranked in cell order) lives at q * S + i, S = the fluid count rounded
// up to 64.  In a porous medium a dense layout moves whole cache lines that
// are mostly solid (in the 256^3, 62%-porous benchmark medium 98.6% of
// 128-byte lines hold some fluid, so a dense step moves ~1.6x the fluid
// bytes); here every population line is fully used.
//
// Geometry tables (caller-owned workspace, built on the device at init):
//   idxp[p]   for every cell of the box padded by one halo layer on each side,
//             p = (x+1) + px ((y+1) + py (z+1)), px = nx+2, py = ny+2: the
//             compact index of the cell, kInvalid for solid cells; halo cells
//             hold the index of their periodic image, or kInvalid beyond a
//             non-periodic face (halfway bounce-back walls).
//   cellp[i]  padded id p of the i-th fluid cell.
// A neighbour along c_d is then idxp[cellp[i] + off_d] with
// off_d = c_x + px (c_y + py c_z): no coordinates, no wrap logic.
#pragma once

#include "kernels.hpp"

namespace lbm {

constexpr uint32_t kInvalid = 0xFFFFFFFFu;

struct CompactGeom {
    const uint32_t* idxp;
    const uint32_t* cellp;
    uint32_t nf;   // fluid cells
    uint32_t px;   // nx + 2
    uint32_t pxy;  // (nx + 2)(ny + 2)
    uint64_t s;    // population stride
};

// Compact indices of the 18 neighbours x + c_d (kInvalid = solid or wall).
__device__ __forceinline__ void neighbours(const CompactGeom& g, uint32_t p, uint32_t (&nb)[kQ])
{
#pragma unroll
    for (int d = 0; d < kQ; ++d) {
        if (d == 9) {
            nb[d] = kInvalid;
            continue;
        }
        const int32_t off = kCx[d] + (int32_t)g.px * kCy[d] + (int32_t)g.pxy * kCz[d];
        nb[d] = g.idxp[(uint32_t)((int32_t)p + off)];
    }
}

// Where canonical f_q(x, t) of fluid cell i lives for stored state kind S
// (same maps as the dense layouts; x - c_q = x + c_opp(q)).
template <int S, typename T>
__device__ __forceinline__ T* compact_state_slot(T* buf, uint64_t s, uint32_t i, const uint32_t (&nb)[kQ], int q)
{
    const uint32_t up = nb[opp(q)];
    if constexpr (S == kAB) {
        return up == kInvalid ? buf + (uint64_t)opp(q) * s + i : buf + (uint64_t)q * s + up;
    } else if constexpr (S == kAAEven) {
        return buf + (uint64_t)q * s + i;
    } else {
        return up == kInvalid ? buf + (uint64_t)q * s + i : buf + (uint64_t)opp(q) * s + up;
    }
}

// One fused time step over the fluid cells, one work-item per fluid cell.
template <typename T, int K, bool FORCE>
__global__ void __launch_bounds__(kBlockThreads) step_compact_kernel(T* __restrict__ a, T* __restrict__ b,
                                                                     CompactGeom g, Phys<T> p)
{
    const uint32_t i = blockIdx.x * kBlockThreads + threadIdx.x;
    if (i >= g.nf) return;
    const uint64_t s = g.s;
    T f[kQ];
    if constexpr (K == kAAEven) {
        // purely local: read (q, i), write (opp q, i)
#pragma unroll
        for (int q = 0; q < kQ; ++q) f[q] = ld_pop(a + (uint64_t)q * s + i);
        collide<T, FORCE>(f, p);
#pragma unroll
        for (int q = 0; q < kQ; ++q) st_pop(a + (uint64_t)opp(q) * s + i, f[q]);
        return;
    }
    uint32_t nb[kQ];
    neighbours(g, g.cellp[i], nb);
#pragma unroll
    for (int q = 0; q < kQ; ++q) f[q] = ld_pop(compact_state_slot<K == kAB ? kAB : kAAOdd>(a, s, i, nb, q));
    collide<T, FORCE>(f, p);
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        if constexpr (K == kAB) {
            st_pop(b + (uint64_t)q * s + i, f[q]);
        } else {
            const uint32_t dn = nb[q];  // x + c_q
            T* dst = dn == kInvalid ? a + (uint64_t)opp(q) * s + i : a + (uint64_t)q * s + dn;
            st_pop(dst, f[q]);
        }
    }
}

// State transfers between canonical dense arrays ([19][N], [N], [3][N]) and
// the compact store; one work-item per cell of the box (tile mapping of the
// dense kernels).  Solid cells read as 0 and own no storage.
template <typename T, int S, int OP>
__global__ void __launch_bounds__(kBlockThreads) io_compact_kernel(T* __restrict__ a, CompactGeom cg, Geom g,
                                                                   Phys<T> p, T* __restrict__ out0,
                                                                   T* __restrict__ out1,
                                                                   const T* __restrict__ in0,
                                                                   const T* __restrict__ in1)
{
    Cell c;
    if (!locate(g, c)) return;
    const uint64_t n = g.n;
    const uint32_t i = cg.idxp[(c.x + 1) + cg.px * (c.y + 1) + cg.pxy * (c.z + 1)];
    if (i == kInvalid) {
        if constexpr (OP == kReadF || OP == kReadS) {
#pragma unroll
            for (int q = 0; q < kQ; ++q) out0[(uint64_t)q * n + c.id] = T(0);
        } else if constexpr (OP == kReadMoments) {
            out0[c.id] = T(0);
#pragma unroll
            for (int d = 0; d < 3; ++d) out1[(uint64_t)d * n + c.id] = T(0);
        }
        return;
    }
    uint32_t nb[kQ];
    neighbours(cg, cg.cellp[i], nb);
    const uint64_t s = cg.s;
    T f[kQ];
    if constexpr (OP == kReadF || OP == kReadMoments || OP == kReadS) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) f[q] = *compact_state_slot<S>(a, s, i, nb, q);
        if constexpr (OP == kReadF) {
#pragma unroll
            for (int q = 0; q < kQ; ++q) out0[(uint64_t)q * n + c.id] = f[q] + wq<T>(q);
        } else if constexpr (OP == kReadS) {
#pragma unroll
            for (int q = 0; q < kQ; ++q) out0[(uint64_t)q * n + c.id] = f[q];
        } else {
            T drho, rho, ux, uy, uz;
            moments<T, true>(f, p, drho, rho, ux, uy, uz);
            out0[c.id] = rho;
            out1[c.id] = ux;
            out1[n + c.id] = uy;
            out1[2 * n + c.id] = uz;
        }
    } else {
        if constexpr (OP == kWriteF) {
#pragma unroll
            for (int q = 0; q < kQ; ++q) f[q] = in0[(uint64_t)q * n + c.id] - wq<T>(q);
        } else if constexpr (OP == kWriteS) {
#pragma unroll
            for (int q = 0; q < kQ; ++q) f[q] = in0[(uint64_t)q * n + c.id];
        } else {
            const T rho = in0 != nullptr ? in0[c.id] : T(1);
            T ux = T(0), uy = T(0), uz = T(0);
            if (in1 != nullptr) {
                ux = in1[c.id];
                uy = in1[n + c.id];
                uz = in1[2 * n + c.id];
            }
            shifted_equilibrium(rho, ux, uy, uz, f);
        }
#pragma unroll
        for (int q = 0; q < kQ; ++q) *compact_state_slot<S>(a, s, i, nb, q) = f[q];
    }
}

}  // namespace lbm
