// kernels_force.hpp -- momentum exchange with the solids.
//
// During a step, every population f*_q that leaves a fluid cell x toward a
// solid cell or through a wall is reflected at the link midpoint (halfway
// bounce-back) and comes back along -c_q, so the solid takes 2 f*_q c_q
// (fieldcraft page "GPU lattice Boltzmann: streaming layout and performance",
// first section: the momentum exchange is taken over the wall links of the
// step whose forces are read back).  These kernels evaluate it for the step
// that starts from the stored state: gather the cell's 19 populations through
// the state map, collide (the same function as the step kernels), and sum
// 2 f*_q c_q over the bounce-back links, separately for links that end in a
// solid cell of the mask and for links that leave the box through a wall
// (open faces carry flux, not force).  Sums are in double: per workgroup in a fixed order,
// then over the workgroups in a fixed order, so the result is deterministic.
#pragma once

#include "kernels.hpp"
#include "kernels_compact.hpp"

namespace lbm {

// Dense layouts: one work-item per cell (tile mapping of the step kernels),
// one partial row of six doubles per workgroup.
template <typename T, int L, int S>
__global__ void __launch_bounds__(kBlockThreads) mex_kernel(T* __restrict__ a, Geom g, Phys<T> p,
                                                            double* __restrict__ partial)
{
    double acc[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    Cell c;
    if (locate(g, c) && !(g.mask != nullptr && g.mask[c.id] != 0)) {
        const uint32_t bits = link_bits<true>(g, c);
        const uint32_t obits = open_bits(g, c);
        T s[kQ];
#pragma unroll
        for (int q = 0; q < kQ; ++q) s[q] = *state_slot<S, L>(a, g, c, bits, q, obits);
        if constexpr (S != kAAEven) apply_open(s, obits, p, c);
        collide<T, true>(s, p);
        // x + c_q is solid or beyond a wall iff the upstream bit of opp(q) is
        // set; a face with a face rule sets it too, but its links carry flux
        add_links(acc, s, c, [&](int q) {
            return ((bits >> opp(q)) & 1u) != 0 && !beyond_rule_face(g, c, kCx[q], kCy[q], kCz[q]);
        });
    }
    block_sum6<kBlockThreads>(acc, partial + 6 * (size_t)blockIdx.x);
}


// Compact layout: one work-item per fluid cell, the gathers of the step
// kernels (row-wise neighbour reads, the same slot maps), one partial row per
// workgroup.  The index table marks wall links (kWall) apart from solid ones
// (kInvalid) and from open faces (kOpen + k, which carry no force).
template <typename T, int S>
__global__ void __launch_bounds__(kBlockThreads) mex_compact_kernel(T* __restrict__ a, CompactGeom g, Phys<T> p,
                                                                    double* __restrict__ partial)
{
    double acc[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    const uint32_t i = blockIdx.x * kBlockThreads + threadIdx.x;
    if (i < g.nf) {
        const coff_t sb = cplane<T>();
        const coff_t own0 = cbytes<T>(i);
        const coff_t own1 = own0 + sb;
        char* const A = (char*)a;
        uint32_t nb[kQ];
        neighbours_rows(g, g.cellp[i], nb);
        T f[kQ];
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            if constexpr (solid_slots_live(S)) {
                f[q] = a[compact_state_off<S>(g, i, nb, q)];
                continue;
            }
            coff_t off;
            if constexpr (S == kAAEven) {
                off = sub_of(q) ? own1 : own0;
            } else if constexpr (S == kAB) {
                off = q == 9 ? own0 : link_off<T>(nb[opp(q)], sub_of(q) ? sb : (coff_t)0, sub_of(opp(q)) ? own1 : own0);
            } else {
                off = q == 9 ? own0 : link_off<T>(nb[opp(q)], sub_of(opp(q)) ? sb : (coff_t)0, sub_of(q) ? own1 : own0);
            }
            f[q] = ld_at<T>(pair_block(A, pair_of(q), sb), off);
        }
        if constexpr (S != kAAEven)
            if (g.open) apply_open_nb(f, nb, p);
        collide<T, true>(f, p);
        add_links_nb(acc, f, nb);
    }
    block_sum6<kBlockThreads>(acc, partial + 6 * (size_t)blockIdx.x);
}

// out[0..5] = sum of the n partial rows, in row order per work-item, then the
// workgroup sum.
static __global__ void __launch_bounds__(kBlockThreads) mex_sum_kernel(const double* __restrict__ partial, uint32_t n,
                                                                double* __restrict__ out)
{
    double acc[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (uint32_t r = threadIdx.x; r < n; r += kBlockThreads)
#pragma unroll
        for (int k = 0; k < 6; ++k) acc[k] += partial[6 * (size_t)r + k];
    block_sum6<kBlockThreads>(acc, out);
}

}  // namespace lbm
