// kernels_faces.hpp -- open faces with a face rule.
//
// The PortLBM paper ("PortLBM: A Portable Lattice Boltzmann Tool Leveraging
// SYCL on AMD, NVIDIA, and Intel GPUs", section 3.1, boundary paragraph) sets
// the inlet to the equilibrium of Dirichlet or Neumann values and the outlet
// by an adapted Zou-He condition.  The Dirichlet reservoir is applied inside
// the step kernels (a constant per entering population).  The other rules
// depend on the state, so they run as a pass after each step over the cells
// of their face:
//   Neumann          the entering populations take the equilibrium of the
//                    density and velocity of the cell one layer inward
//                    (zero normal gradient), read from the new state;
//   Zou-He pressure  prescribed density and tangential velocity;
//   Zou-He velocity  prescribed velocity;
// the Zou-He rules (Zou and He, Phys. Fluids 9, 1591, 1997) take each
// entering population from its opposite by non-equilibrium bounce-back, with
// the transverse momentum correction of the 3-D lattice (Hecht and Harting,
// J. Stat. Mech. 2010, P01018); the momentum there is the bare sum of c f,
// rho u - F/2 under Guo forcing.
//
// To the step kernels such a face is a wall: the links through it are
// bounced into the own slots, and this pass overwrites those slots (the
// entering populations of the stored state) with the rule's values.  The
// pass writes only entering populations of cells on its face and reads none
// of them: a Zou-He cell reads its own parallel and leaving populations, a
// Neumann cell the cell one layer inward, which lies on no open face (every
// open face of the box is on the rule face's axis, at least 3 cells long).
// So the cells of a face are independent, and the pass is race-free in place.
#pragma once

#include "kernels.hpp"
#include "kernels_compact.hpp"

namespace lbm {

// Face kinds (the values of the open-face argument of the C ABI).
constexpr uint32_t kRuleNeumann = 2;
constexpr uint32_t kRuleZouHePressure = 3;
constexpr uint32_t kRuleZouHeVelocity = 4;

// Constants of one face rule, computed on the host in double and rounded to T.
template <typename T>
struct FaceRule {
    uint32_t k;            // face: 2 axis + side (-x, +x, -y, +y, -z, +z)
    uint32_t kind;         // kRule*
    uint32_t nx, ny, nz;   // box
    uint32_t n0;           // cells along the face's first tangential axis
    uint32_t ncell;        // cells on the face
    T drho;                // pressure rule: rho - 1
    T jt[3];               // pressure rule: rho u_t - F_t / 2 (the normal entry unused)
    T u[3];                // velocity rule: u
    T ua_s;                // velocity rule: sigma u_a (sigma = +1 on a low face, -1 on a high face)
    T inv_den;             // velocity rule: 1 / (1 - sigma u_a)
    T hfa_s;               // sigma F_a / 2
    T seq[kQ];             // Neumann rule where the inward cell is solid: feq(rho, u) - w
};

// Coordinates of the t-th cell of the face (first tangential axis fastest).
template <typename T>
__device__ __forceinline__ void face_cell(const FaceRule<T>& r, uint32_t t, uint32_t& x, uint32_t& y, uint32_t& z)
{
    const uint32_t ax = r.k >> 1;
    const bool hi = (r.k & 1u) != 0;
    const uint32_t t0 = t % r.n0, t1 = t / r.n0;
    if (ax == 0) {
        x = hi ? r.nx - 1 : 0;
        y = t0;
        z = t1;
    } else if (ax == 1) {
        x = t0;
        y = hi ? r.ny - 1 : 0;
        z = t1;
    } else {
        x = t0;
        y = t1;
        z = hi ? r.nz - 1 : 0;
    }
}

// Zou-He on the stored (weight-shifted) populations s of a cell of face r.k:
// the entries with bit q of `ent` set are replaced.  With s = f - w the
// parallel group's weights sum to 2/3 and the leaving group's to 1/6, so
// rho - par - 2 out = (rho - 1) - par_s - 2 out_s; the antisymmetric sums
// (tangential momentum, f_q - f_opp) do not see the weights.
template <typename T>
__device__ __forceinline__ void zou_he(T (&s)[kQ], uint32_t ent, const FaceRule<T>& r, const Phys<T>& p)
{
    const uint32_t ax = r.k >> 1;
    const int sg = (r.k & 1u) ? -1 : 1;
    T par = T(0), out = T(0), tx = T(0), ty = T(0), tz = T(0);
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        const int ca = ax == 0 ? kCx[q] : ax == 1 ? kCy[q] : kCz[q];
        if (ca == 0) {
            par += s[q];
            if (kCx[q] != 0) tx += T(kCx[q]) * s[q];
            if (kCy[q] != 0) ty += T(kCy[q]) * s[q];
            if (kCz[q] != 0) tz += T(kCz[q]) * s[q];
        } else if (ca == -sg) {
            out += s[q];
        }
    }
    // bare momentum j: sigma j_a = rho - par - 2 out by mass
    T jx, jy, jz;
    if (r.kind == kRuleZouHePressure) {
        const T jn = r.drho - par - T(2) * out;
        const T ja = sg > 0 ? jn : -jn;
        jx = ax == 0 ? ja : r.jt[0];
        jy = ax == 1 ? ja : r.jt[1];
        jz = ax == 2 ? ja : r.jt[2];
    } else {
        // rho (1 - sigma u_a) = par + 2 out - sigma F_a / 2
        const T rho = T(1) + (par + T(2) * out - r.hfa_s + r.ua_s) * r.inv_den;
        jx = rho * r.u[0] - p.hfx;
        jy = rho * r.u[1] - p.hfy;
        jz = rho * r.u[2] - p.hfz;
    }
    // transverse correction N_t = tpar_t / 2 - j_t / 3 (none along the normal)
    const T nx = ax == 0 ? T(0) : T(0.5) * tx - jx / T(3);
    const T ny = ax == 1 ? T(0) : T(0.5) * ty - jy / T(3);
    const T nz = ax == 2 ? T(0) : T(0.5) * tz - jz / T(3);
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        if (q == 9) continue;
        // feq_q - feq_opp(q) = 6 w_q c_q . j: 1/3 on an axis link, 1/6 on a diagonal
        const int n2 = kCx[q] * kCx[q] + kCy[q] * kCy[q] + kCz[q] * kCz[q];
        const T cj = T(kCx[q]) * jx + T(kCy[q]) * jy + T(kCz[q]) * jz;
        const T corr = T(kCx[q]) * nx + T(kCy[q]) * ny + T(kCz[q]) * nz;
        const T v = s[opp(q)] + (n2 == 1 ? cj / T(3) : cj / T(6)) - corr;
        s[q] = ((ent >> q) & 1u) ? v : s[q];
    }
}

// Neumann: e := shifted equilibrium of the inward cell's moments (s1), or the
// face's own values when that cell is solid (s1 is then all zeros, so the
// unused equilibrium stays finite).  Both are formed and one is selected: a
// branch here leaves part of e in private memory.
template <typename T>
__device__ __forceinline__ void neumann_values(T (&e)[kQ], const T (&s1)[kQ], bool solid1, const FaceRule<T>& r,
                                               const Phys<T>& p)
{
    T drho, rho, ux, uy, uz;
    moments<T, true>(s1, p, drho, rho, ux, uy, uz);
    shifted_equilibrium(rho, ux, uy, uz, e);
#pragma unroll
    for (int q = 0; q < kQ; ++q) e[q] = solid1 ? r.seq[q] : e[q];
}

// Dense layouts: one work-item per cell of the face, the state maps of the
// state transfers (kind S of the state the step just left).
template <typename T, int L, int S>
__global__ void __launch_bounds__(kBlockThreads) face_kernel(T* __restrict__ a, Geom g, Phys<T> p, FaceRule<T> r)
{
    const uint32_t t = blockIdx.x * kBlockThreads + threadIdx.x;
    if (t >= r.ncell) return;
    Cell c;
    face_cell(r, t, c.x, c.y, c.z);
    fill_cell(g, c);
    if (g.mask != nullptr && g.mask[c.id] != 0) return;
    const uint32_t ax = r.k >> 1;
    const int sg = (r.k & 1u) ? -1 : 1;
    const uint32_t bits = link_bits<true>(g, c);
    const uint32_t obits = open_bits(g, c);
    T s[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) s[q] = *state_slot<S, L>(a, g, c, bits, q, obits);
    // entering through this face: c_q[ax] = sigma, unless the upstream cell
    // also lies beyond a wall of another axis (an edge: the wall wins)
    uint32_t ent = 0;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        if (q == 9) continue;
        const int ca = ax == 0 ? kCx[q] : ax == 1 ? kCy[q] : kCz[q];
        const bool wall = beyond_wall(c, ax == 0 ? 0 : -kCx[q], ax == 1 ? 0 : -kCy[q], ax == 2 ? 0 : -kCz[q]);
        ent |= (uint32_t)(ca == sg && !wall) << q;
    }
    if (r.kind == kRuleNeumann) {
        Cell c1 = c;
        if (ax == 0) c1.x += sg;
        if (ax == 1) c1.y += sg;
        if (ax == 2) c1.z += sg;
        fill_cell(g, c1);
        const bool solid1 = g.mask != nullptr && g.mask[c1.id] != 0;
        T s1[kQ], e[kQ];
        if (!solid1) {
            const uint32_t bits1 = link_bits<true>(g, c1), obits1 = open_bits(g, c1);
#pragma unroll
            for (int q = 0; q < kQ; ++q) s1[q] = *state_slot<S, L>(a, g, c1, bits1, q, obits1);
        } else {
#pragma unroll
            for (int q = 0; q < kQ; ++q) s1[q] = T(0);
        }
        neumann_values(e, s1, solid1, r, p);
#pragma unroll
        for (int q = 0; q < kQ; ++q) s[q] = ((ent >> q) & 1u) ? e[q] : s[q];
    } else {
        zou_he(s, ent, r, p);
    }
    // the entering populations' slots: their upstream bit is set (the face is
    // a wall to the steps), so these are the own bounce slots
#pragma unroll
    for (int q = 0; q < kQ; ++q)
        if ((ent >> q) & 1u) *state_slot<S, L>(a, g, c, bits, q, obits) = s[q];
}

// Compact layout: the same on the fluid-compacted store; the index table
// marks the halo beyond face k as kOpen + k.
template <typename T, int S>
__global__ void __launch_bounds__(kBlockThreads) face_compact_kernel(T* __restrict__ a, CompactGeom cg, Phys<T> p,
                                                                     FaceRule<T> r)
{
    const uint32_t t = blockIdx.x * kBlockThreads + threadIdx.x;
    if (t >= r.ncell) return;
    uint32_t x, y, z;
    face_cell(r, t, x, y, z);
    const uint32_t pp = (x + 1) + cg.px * (y + 1) + cg.pxy * (z + 1);
    const uint32_t i = cg.idxp[pp];
    if (i == kInvalid) return;
    uint32_t nb[kQ];
    neighbours(cg, pp, nb);
    T f[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) f[q] = *compact_state_slot<S>(a, cg, i, nb, q);
    uint32_t ent = 0;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
        if (q != 9) ent |= (uint32_t)(nb[opp(q)] == kOpen + r.k) << q;
    if (r.kind == kRuleNeumann) {
        const uint32_t ax = r.k >> 1;
        const uint32_t stride = ax == 0 ? 1u : ax == 1 ? cg.px : cg.pxy;
        const uint32_t pp1 = (r.k & 1u) ? pp - stride : pp + stride;
        const uint32_t i1 = cg.idxp[pp1];
        const bool solid1 = i1 == kInvalid;
        T f1[kQ], e[kQ];
        if (!solid1) {
            uint32_t nb1[kQ];
            neighbours(cg, pp1, nb1);
#pragma unroll
            for (int q = 0; q < kQ; ++q) f1[q] = *compact_state_slot<S>(a, cg, i1, nb1, q);
        } else {
#pragma unroll
            for (int q = 0; q < kQ; ++q) f1[q] = T(0);
        }
        neumann_values(e, f1, solid1, r, p);
#pragma unroll
        for (int q = 0; q < kQ; ++q) f[q] = ((ent >> q) & 1u) ? e[q] : f[q];
    } else {
        zou_he(f, ent, r, p);
    }
#pragma unroll
    for (int q = 0; q < kQ; ++q)
        if ((ent >> q) & 1u) *compact_state_slot<S>(a, cg, i, nb, q) = f[q];
}

}  // namespace lbm
