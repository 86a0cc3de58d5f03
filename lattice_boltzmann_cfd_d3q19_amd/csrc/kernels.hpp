// kernels.hpp -- fused D3Q19 BGK collide-and-stream kernels for gfx950.
//
// One work-item updates one cell.  A step kernel gathers the cell's 19
// populations into registers, forms density and velocity, relaxes toward the
// second-order equilibrium with the optional Guo forcing term, and scatters
// the 19 results: the whole lattice Boltzmann update of the PortLBM page
// ("PortLBM: A Portable Lattice Boltzmann Tool ...", section 3.1, Eq. 1,
// split as in section 3.3, Eq. 3) in one pass over HBM, 2 x 19 x sizeof(T)
// bytes per fluid cell.  All 19 loads are issued before any store, which is
// what makes the one-lattice AA pattern race-free (fieldcraft page "GPU
// lattice Boltzmann: streaming layout and performance", first section: a
// cell writes exactly the slots it read, gathered before scattered).
//
// Work decomposition: the box is cut into tiles of BX x BY cells (BX along
// x, the fastest index, so each wave64 covers consecutive cells of one row
// or of a few short rows); one workgroup per tile, tiles numbered x-, then
// y-, then z-fastest.  Optionally the hardware's round-robin placement of
// workgroups over the 8 XCDs is undone so that each XCD sweeps a contiguous
// range of tiles (neighbouring rows share an L2).
//
// The collision arithmetic is one inlined function used by every layout and
// scheme, compiled with floating-point contraction off, so the result of a
// step does not depend on layout or scheme: all of them agree bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "d3q19.hpp"

namespace lbm {

struct Geom {
    uint32_t nx, ny, nz, nxy;
    uint32_t per_x, per_y, per_z;  // 1 = periodic, 0 = bounce-back wall beyond both faces
    uint32_t ntx, nty, ntiles;     // tiles per x-row of tiles, per y-column, total
    uint32_t xcd_remap;            // 1 = give each XCD a contiguous tile range
    uint64_t n;                    // cells
    const uint8_t* mask;           // uint8[n], nonzero = solid; may be null
};

template <typename T>
struct Phys {
    T omega;  // 1 / tau (0 for tau = inf)
    T guo;    // 1 - omega / 2
    T fx, fy, fz;
    T hfx, hfy, hfz;  // F / 2
};

enum IoOp : int { kReadF = 0, kReadMoments = 1, kWriteF = 2, kWriteEq = 3 };

// ---------------------------------------------------------------- layout

// Address of population q of `cell` in a buffer of the given layout.
template <int L, typename T>
__device__ __forceinline__ T* slot(T* base, uint64_t n, int q, uint32_t cell)
{
    if constexpr (L == kStream) {
        return base + (uint64_t)q * n + cell;
    } else if constexpr (L == kBundle) {
        return base + (uint64_t)kBundleFirst[q] * n + (uint64_t)cell * (uint32_t)kBundleSize[q] +
               (uint32_t)(q - kBundleFirst[q]);
    } else {
        return base + (uint64_t)cell * (uint32_t)kQ + (uint32_t)q;
    }
}

// ----------------------------------------------------------- tile mapping

// Workgroup i is placed on XCD i % 8.  Renumber so that XCD k owns the k-th
// contiguous slice of the tile range (slices differ in size by at most one).
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t pid, uint32_t ntiles)
{
    const uint32_t q = ntiles / 8u, r = ntiles % 8u;
    const uint32_t xcd = pid % 8u, local = pid / 8u;
    return xcd < r ? xcd * (q + 1u) + local : r * (q + 1u) + (xcd - r) * q + local;
}

struct Cell {
    uint32_t x, y, z, id;
    uint32_t ox[3], oy[3], oz[3];  // wrapped neighbour coordinates as index offsets
    bool wall[3][2];               // beyond the low / high face on a non-periodic axis
};

// Decode this work-item's cell; false if it lies outside the box.
__device__ __forceinline__ bool locate(const Geom& g, Cell& c)
{
    uint32_t tile = blockIdx.x;
    if (g.xcd_remap) tile = xcd_contiguous(tile, g.ntiles);
    const uint32_t tx = tile % g.ntx;
    const uint32_t rest = tile / g.ntx;
    const uint32_t ty = rest % g.nty;
    c.z = rest / g.nty;
    c.x = tx * blockDim.x + threadIdx.x;
    c.y = ty * blockDim.y + threadIdx.y;
    if (c.x >= g.nx || c.y >= g.ny) return false;
    c.id = c.x + g.nx * (c.y + g.ny * c.z);
    const uint32_t xm = c.x == 0 ? g.nx - 1 : c.x - 1, xp = c.x + 1 == g.nx ? 0 : c.x + 1;
    const uint32_t ym = c.y == 0 ? g.ny - 1 : c.y - 1, yp = c.y + 1 == g.ny ? 0 : c.y + 1;
    const uint32_t zm = c.z == 0 ? g.nz - 1 : c.z - 1, zp = c.z + 1 == g.nz ? 0 : c.z + 1;
    c.ox[0] = xm;
    c.ox[1] = c.x;
    c.ox[2] = xp;
    c.oy[0] = ym * g.nx;
    c.oy[1] = c.y * g.nx;
    c.oy[2] = yp * g.nx;
    c.oz[0] = zm * g.nxy;
    c.oz[1] = c.z * g.nxy;
    c.oz[2] = zp * g.nxy;
    c.wall[0][0] = !g.per_x && c.x == 0;
    c.wall[0][1] = !g.per_x && c.x + 1 == g.nx;
    c.wall[1][0] = !g.per_y && c.y == 0;
    c.wall[1][1] = !g.per_y && c.y + 1 == g.ny;
    c.wall[2][0] = !g.per_z && c.z == 0;
    c.wall[2][1] = !g.per_z && c.z + 1 == g.nz;
    return true;
}

// Cell index of (x + dx, y + dy, z + dz), wrapped periodically.
__device__ __forceinline__ uint32_t nbr(const Cell& c, int dx, int dy, int dz)
{
    return c.ox[dx + 1] + c.oy[dy + 1] + c.oz[dz + 1];
}

__device__ __forceinline__ bool beyond_wall(const Cell& c, int dx, int dy, int dz)
{
    return (dx < 0 && c.wall[0][0]) || (dx > 0 && c.wall[0][1]) || (dy < 0 && c.wall[1][0]) ||
           (dy > 0 && c.wall[1][1]) || (dz < 0 && c.wall[2][0]) || (dz > 0 && c.wall[2][1]);
}

// Bit q set iff the upstream cell x - c_q is solid or beyond a wall, i.e. the
// population arriving along c_q is the bounced-back one.
template <bool BND>
__device__ __forceinline__ uint32_t link_bits(const Geom& g, const Cell& c)
{
    uint32_t bits = 0;
    if constexpr (BND) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            if (q == 9) continue;
            const int dx = -kCx[q], dy = -kCy[q], dz = -kCz[q];
            bool solid = beyond_wall(c, dx, dy, dz);
            if (!solid && g.mask != nullptr) solid = g.mask[nbr(c, dx, dy, dz)] != 0;
            bits |= (uint32_t)solid << q;
        }
    }
    return bits;
}

// ------------------------------------------------------------- collision

template <typename T>
__device__ __forceinline__ T wq(int q)
{
    return T(kW36[q]) / T(36);
}

// rho = sum_q f_q (q order), j = sum_q c_q f_q, u = (j + F/2) / rho.
template <typename T, bool FORCE>
__device__ __forceinline__ void moments(const T (&f)[kQ], const Phys<T>& p, T& rho, T& ux, T& uy, T& uz)
{
    rho = f[0];
#pragma unroll
    for (int q = 1; q < kQ; ++q) rho = rho + f[q];
    T xp = T(0), xm = T(0), yp = T(0), ym = T(0), zp = T(0), zm = T(0);
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        if (kCx[q] > 0) xp = xp + f[q];
        if (kCx[q] < 0) xm = xm + f[q];
        if (kCy[q] > 0) yp = yp + f[q];
        if (kCy[q] < 0) ym = ym + f[q];
        if (kCz[q] > 0) zp = zp + f[q];
        if (kCz[q] < 0) zm = zm + f[q];
    }
    T jx = xp - xm, jy = yp - ym, jz = zp - zm;
    if constexpr (FORCE) {
        jx = jx + p.hfx;
        jy = jy + p.hfy;
        jz = jz + p.hfz;
    }
    const T inv = T(1) / rho;
    ux = jx * inv;
    uy = jy * inv;
    uz = jz * inv;
}

template <int q, typename T>
__device__ __forceinline__ T cdot(T ax, T ay, T az)
{
    T s = T(0);
    if constexpr (kCx[q] > 0) s = s + ax;
    if constexpr (kCx[q] < 0) s = s - ax;
    if constexpr (kCy[q] > 0) s = s + ay;
    if constexpr (kCy[q] < 0) s = s - ay;
    if constexpr (kCz[q] > 0) s = s + az;
    if constexpr (kCz[q] < 0) s = s - az;
    return s;
}

// Equilibrium of directions q and opposite(q) from the even and odd parts:
// feq = w rho (1 - 3/2 u^2 + 9/2 (c.u)^2) +- w rho 3 (c.u).
template <int q, typename T>
__device__ __forceinline__ void feq_pair(T rho, T ux, T uy, T uz, T base, T& fq, T& fo)
{
    const T cu = cdot<q>(ux, uy, uz);
    const T wr = wq<T>(q) * rho;
    const T even = wr * (base + T(4.5) * cu * cu);
    const T odd = wr * (T(3) * cu);
    fq = even + odd;
    fo = even - odd;
}

template <typename T>
__device__ __forceinline__ T eq_base(T ux, T uy, T uz)
{
    const T usq = ux * ux + uy * uy + uz * uz;
    return T(1) - T(1.5) * usq;
}

template <int q, typename T, bool FORCE>
__device__ __forceinline__ void relax_pair(T (&f)[kQ], const Phys<T>& p, T rho, T ux, T uy, T uz, T base, T uF)
{
    constexpr int o = opp(q);
    T eq, eo;
    feq_pair<q>(rho, ux, uy, uz, base, eq, eo);
    T nq = fma(p.omega, eq - f[q], f[q]);
    T no = fma(p.omega, eo - f[o], f[o]);
    if constexpr (FORCE) {
        // Guo term: (1 - omega/2) w [3 (c - u) + 9 (c.u) c] . F, split into the
        // parts even and odd under c -> -c.
        const T cu = cdot<q>(ux, uy, uz);
        const T cF = cdot<q>(p.fx, p.fy, p.fz);
        const T gw = p.guo * wq<T>(q);
        const T even = gw * (T(9) * cu * cF - T(3) * uF);
        const T odd = gw * (T(3) * cF);
        nq = nq + (even + odd);
        no = no + (even - odd);
    }
    f[q] = nq;
    f[o] = no;
}

template <typename T, bool FORCE>
__device__ __forceinline__ void collide(T (&f)[kQ], const Phys<T>& p)
{
    T rho, ux, uy, uz;
    moments<T, FORCE>(f, p, rho, ux, uy, uz);
    const T base = eq_base(ux, uy, uz);
    T uF = T(0);
    if constexpr (FORCE) uF = ux * p.fx + uy * p.fy + uz * p.fz;
    relax_pair<0, T, FORCE>(f, p, rho, ux, uy, uz, base, uF);
    relax_pair<1, T, FORCE>(f, p, rho, ux, uy, uz, base, uF);
    relax_pair<2, T, FORCE>(f, p, rho, ux, uy, uz, base, uF);
    relax_pair<3, T, FORCE>(f, p, rho, ux, uy, uz, base, uF);
    relax_pair<4, T, FORCE>(f, p, rho, ux, uy, uz, base, uF);
    relax_pair<5, T, FORCE>(f, p, rho, ux, uy, uz, base, uF);
    relax_pair<6, T, FORCE>(f, p, rho, ux, uy, uz, base, uF);
    relax_pair<7, T, FORCE>(f, p, rho, ux, uy, uz, base, uF);
    relax_pair<8, T, FORCE>(f, p, rho, ux, uy, uz, base, uF);
    // rest population
    const T e9 = wq<T>(9) * rho * base;
    T n9 = fma(p.omega, e9 - f[9], f[9]);
    if constexpr (FORCE) n9 = n9 + p.guo * wq<T>(9) * (T(-3) * uF);
    f[9] = n9;
}

template <typename T>
__device__ __forceinline__ void equilibrium(T rho, T ux, T uy, T uz, T (&f)[kQ])
{
    const T base = eq_base(ux, uy, uz);
    feq_pair<0>(rho, ux, uy, uz, base, f[0], f[18]);
    feq_pair<1>(rho, ux, uy, uz, base, f[1], f[17]);
    feq_pair<2>(rho, ux, uy, uz, base, f[2], f[16]);
    feq_pair<3>(rho, ux, uy, uz, base, f[3], f[15]);
    feq_pair<4>(rho, ux, uy, uz, base, f[4], f[14]);
    feq_pair<5>(rho, ux, uy, uz, base, f[5], f[13]);
    feq_pair<6>(rho, ux, uy, uz, base, f[6], f[12]);
    feq_pair<7>(rho, ux, uy, uz, base, f[7], f[11]);
    feq_pair<8>(rho, ux, uy, uz, base, f[8], f[10]);
    f[9] = wq<T>(9) * rho * base;
}

// ------------------------------------------------------ stored-state maps

// Where the canonical population f_q(x, t) lives for a stored state of kind S
// (kAB: the source lattice holds h(t) with f(t) = stream(h(t)); kAAEven: the
// lattice holds f(t) in natural slots; kAAOdd: it holds the post-collision
// values of step t-1 in swapped slots).  This is the gather half of a step.
template <int S, int L, typename T>
__device__ __forceinline__ T* state_slot(T* buf, uint64_t n, const Cell& c, uint32_t bits, int q)
{
    const bool bb = (bits >> q) & 1u;
    const uint32_t up = nbr(c, -kCx[q], -kCy[q], -kCz[q]);
    if constexpr (S == kAB) {
        return bb ? slot<L>(buf, n, opp(q), c.id) : slot<L>(buf, n, q, up);
    } else if constexpr (S == kAAEven) {
        return slot<L>(buf, n, q, c.id);
    } else {
        return bb ? slot<L>(buf, n, q, c.id) : slot<L>(buf, n, opp(q), up);
    }
}

// ----------------------------------------------------------------- kernels

constexpr int kBlockThreads = 256;

// One fused time step.  K: kAB (a = source, b = destination), kAAEven or
// kAAOdd (a = the single lattice).  BND: a mask or a wall exists.
template <typename T, int L, int K, bool BND, bool FORCE>
__global__ void __launch_bounds__(kBlockThreads) step_kernel(T* __restrict__ a, T* __restrict__ b,
                                                             Geom g, Phys<T> p)
{
    Cell c;
    if (!locate(g, c)) return;
    if constexpr (BND) {
        if (g.mask != nullptr && g.mask[c.id] != 0) return;  // solid cells are never updated
    }
    const uint32_t bits = link_bits<BND>(g, c);
    const uint64_t n = g.n;

    T f[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        if constexpr (K == kAB) {
            f[q] = *state_slot<kAB, L>(a, n, c, bits, q);
        } else if constexpr (K == kAAEven) {
            f[q] = *slot<L>(a, n, q, c.id);
        } else {
            f[q] = *state_slot<kAAOdd, L>(a, n, c, bits, q);
        }
    }

    collide<T, FORCE>(f, p);

#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        if constexpr (K == kAB) {
            *slot<L>(b, n, q, c.id) = f[q];
        } else if constexpr (K == kAAEven) {
            *slot<L>(a, n, opp(q), c.id) = f[q];
        } else {
            // toward x + c_q, or straight back into (opp q, x) if that cell is
            // solid or beyond a wall (its upstream bit for opp q is set)
            const bool bb = (bits >> opp(q)) & 1u;
            T* dst = bb ? slot<L>(a, n, opp(q), c.id)
                        : slot<L>(a, n, q, nbr(c, kCx[q], kCy[q], kCz[q]));
            *dst = f[q];
        }
    }
}

// State input/output: canonical populations or moments in and out of a
// stored state of kind S (see state_slot).  b is the second AB lattice (only
// cleared on solid cells by kWriteEq) or null.
template <typename T, int L, int S, int OP>
__global__ void __launch_bounds__(kBlockThreads) io_kernel(T* __restrict__ a, T* __restrict__ b, Geom g,
                                                           Phys<T> p, T* __restrict__ out0,
                                                           T* __restrict__ out1,
                                                           const T* __restrict__ in0,
                                                           const T* __restrict__ in1)
{
    Cell c;
    if (!locate(g, c)) return;
    const uint64_t n = g.n;
    const bool solid = g.mask != nullptr && g.mask[c.id] != 0;
    if (solid) {
        if constexpr (OP == kReadF) {
#pragma unroll
            for (int q = 0; q < kQ; ++q) out0[(uint64_t)q * n + c.id] = T(0);
        } else if constexpr (OP == kReadMoments) {
            out0[c.id] = T(0);
#pragma unroll
            for (int d = 0; d < 3; ++d) out1[(uint64_t)d * n + c.id] = T(0);
        } else {
#pragma unroll
            for (int q = 0; q < kQ; ++q) {
                *slot<L>(a, n, q, c.id) = T(0);
                if (b != nullptr) *slot<L>(b, n, q, c.id) = T(0);
            }
        }
        return;
    }
    const uint32_t bits = link_bits<true>(g, c);
    T f[kQ];
    if constexpr (OP == kReadF || OP == kReadMoments) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) f[q] = *state_slot<S, L>(a, n, c, bits, q);
        if constexpr (OP == kReadF) {
#pragma unroll
            for (int q = 0; q < kQ; ++q) out0[(uint64_t)q * n + c.id] = f[q];
        } else {
            T rho, ux, uy, uz;
            moments<T, true>(f, p, rho, ux, uy, uz);
            out0[c.id] = rho;
            out1[c.id] = ux;
            out1[n + c.id] = uy;
            out1[2 * n + c.id] = uz;
        }
    } else {
        if constexpr (OP == kWriteF) {
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
            equilibrium(rho, ux, uy, uz, f);
        }
#pragma unroll
        for (int q = 0; q < kQ; ++q) *state_slot<S, L>(a, n, c, bits, q) = f[q];
    }
}

}  // namespace lbm
