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
// y-, then z-fastest.  The SoA layouts keep the hardware's round-robin
// placement of consecutive workgroups over the 8 XCDs (every cache line is
// touched by one workgroup only; a contiguous slab of tiles per XCD measured
// 8% slower and chunked orders up to 8% slower on the 256^3 porous box).  The
// AoS layout, whose neighbour records share lines across rows, uses chunked
// orders (xcd_chunked).
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
    uint32_t xk;                   // workgroup chunk per XCD turn (1 = hardware order)
    uint32_t open;                 // bit k: face k (-x, +x, -y, +y, -z, +z) is an open reservoir
    uint32_t fix;                  // bit k: face k is open with a face rule (a wall to the steps)
    uint64_t n;                    // cells
    const uint8_t* mask;           // uint8[n], nonzero = solid; may be null
};

// Relaxation and forcing constants, computed once on the host in double and
// rounded to T.  The Guo term (1 - omega/2) w_q [3 (c_q - u) + 9 (c_q.u) c_q].F
// of a pair (q, opp q), q < 9, splits into an even part
// gev[q] (c_q.u) - gu[class] (u.F) and an odd part god[q] (+ for q, - for
// opp q), with gev[q] = 9 (1 - omega/2) w_q (c_q.F), god[q] = 3 (1 - omega/2)
// w_q (c_q.F) and gu = 3 (1 - omega/2) w for the rest / axis / diagonal class.
template <typename T>
struct Phys {
    T omega;  // 1 / tau (0 for tau = inf)
    T fx, fy, fz;
    T hfx, hfy, hfz;  // F / 2
    T gev[9], god[9];
    T gu[3];  // [0] rest, [1] axis (w = 1/18), [2] diagonal (w = 1/36)
    // Open faces: the shifted equilibrium feq_q(rho_k, u_k) - w_q of face k's
    // reservoir, the value of every population entering through face k.
    T seq[6][kQ];
    uint32_t res;  // bit k: face k is a reservoir (the others' entering values are stored)
};

// State transfers: canonical populations f out / in, moments out, equilibrium
// in, and the stored (weight-shifted) values f - w out / in (exact checkpoint).
enum IoOp : int { kReadF = 0, kReadMoments = 1, kWriteF = 2, kWriteEq = 3, kReadS = 4, kWriteS = 5 };

// ---------------------------------------------------------------- layout

// Element offset of population q of `cell` in a buffer of the given layout.
// q is a compile-time constant at every call, so the direction's part is
// uniform (scalar) and the per-lane part is one 64-bit add.
template <int L>
__device__ __forceinline__ uint64_t slot_off(uint64_t n, int q, uint32_t cell)
{
    if constexpr (L == kStream) {
        return (uint64_t)q * n + cell;
    } else if constexpr (L == kBundle) {
        return (uint64_t)kBundleFirst[q] * n + (uint64_t)cell * (uint32_t)kBundleSize[q] +
               (uint32_t)(q - kBundleFirst[q]);
    } else {
        return (uint64_t)cell * (uint32_t)kQ + (uint32_t)q;
    }
}

// Address of population q of `cell` in a buffer of the given layout.
template <int L, typename T>
__device__ __forceinline__ T* slot(T* base, uint64_t n, int q, uint32_t cell)
{
    return base + slot_off<L>(n, q, cell);
}

// ------------------------------------------------------- memory access

// Population stores of the step kernels are nontemporal: every slot is written
// once per step and not read again before the next step, so the stores should
// not displace lines that neighbouring cells are still reading (measured on
// MI355X: +6% for the fused pull on a periodic 256^3 box, +27% on the porous
// one; neutral for the in-place pattern).  Nontemporal loads lose the reuse of
// partially consumed lines between neighbouring waves and are off.
#ifndef LBM_NT_LOAD
#define LBM_NT_LOAD 0
#endif
#ifndef LBM_NT_STORE
#define LBM_NT_STORE 1
#endif

template <typename T>
__device__ __forceinline__ T ld_pop(const T* p)
{
#if LBM_NT_LOAD
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

// The even step of the in-place pattern reads only its own cells' slots.
// Nontemporal loads there (NT) measured faster on periodic boxes without a
// mask in the SoA and bundle layouts (256^3: stream even + odd 0.471 + 0.491
// -> 0.436 + 0.450 ms, bundle 0.475 + 0.546 -> 0.459 + 0.515 ms) and slower
// with a mask (porous 256^3 stream: 0.555 + 0.583 -> 0.699 + 0.528 ms; the
// 128^3 sphere also lost) and in the AoS layout (even step 0.550 -> 1.253 ms:
// the 19 loads of a record share its lines), so the step kernel uses them
// only in the no-mask instance of those two layouts.
template <bool NT, typename T>
__device__ __forceinline__ T ld_pop_own(const T* p)
{
    if constexpr (NT) {
        return __builtin_nontemporal_load(p);
    } else {
        return ld_pop(p);
    }
}

// The AoS layout stores plain: each cache line of its records is written in
// pieces by the cells of several rows, which the L2 merges only if the pieces
// stay there (nontemporal stores measured 1.93 vs 1.71 ms for the odd
// in-place step and 1.32 vs 0.93 ms for the pull on a periodic 256^3 box,
// 0.84 vs 0.74 ms for the pull on the porous one; the other layouts lose
// 3-25% with plain stores).
template <int L>
constexpr bool nt_store()
{
    return LBM_NT_STORE && L != kCollision;
}

template <int L, typename V>
__device__ __forceinline__ void st_pop(V* p, V v)
{
    if constexpr (nt_store<L>()) {
        __builtin_nontemporal_store(v, p);
    } else {
        *p = v;
    }
}

// ----------------------------------------------------------- tile mapping

struct Cell {
    uint32_t x, y, z, id;
    uint32_t ox[3], oy[3], oz[3];  // wrapped neighbour coordinates as index offsets
    bool wall[3][2];               // at the low / high face of a non-periodic axis, beyond it a wall
    bool open[3][2];               // ... beyond it an open face
};

// Workgroup w runs on XCD w % 8 (the dispatcher deals workgroups out round
// robin).  Renumbered in chunks of k consecutive workgroups, XCD x takes
// chunks x, x + 8, x + 16, ...: neighbouring rows of tiles then share an L2.
// k = 1 is the hardware order; the grid is rounded up to 8 k workgroups.
__device__ __forceinline__ uint32_t xcd_chunked(uint32_t hw, uint32_t k)
{
    const uint32_t x = hw & 7u, l = hw >> 3;
    return ((l / k) * 8u + x) * k + l % k;
}

// Index, wrapped neighbour offsets and face flags of the cell (c.x, c.y, c.z).
// A face with a face rule is a wall here: the steps bounce its links back
// into the own slots, whose entering values the rule then replaces.
__device__ __forceinline__ void fill_cell(const Geom& g, Cell& c)
{
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
    const bool at[3][2] = {{!g.per_x && c.x == 0, !g.per_x && c.x + 1 == g.nx},
                           {!g.per_y && c.y == 0, !g.per_y && c.y + 1 == g.ny},
                           {!g.per_z && c.z == 0, !g.per_z && c.z + 1 == g.nz}};
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int sd = 0; sd < 2; ++sd) {
            const bool open = (g.open >> (2 * a + sd)) & 1u;
            c.wall[a][sd] = at[a][sd] && !open;
            c.open[a][sd] = at[a][sd] && open;
        }
}

// Decode this work-item's cell; false if it lies outside the box.
__device__ __forceinline__ bool locate(const Geom& g, Cell& c)
{
    const uint32_t tile = g.xk > 1 ? xcd_chunked(blockIdx.x, g.xk) : blockIdx.x;
    if (tile >= g.ntiles) return false;
    const uint32_t tx = tile % g.ntx;
    const uint32_t rest = tile / g.ntx;
    const uint32_t ty = rest % g.nty;
    c.z = rest / g.nty;
    c.x = tx * blockDim.x + threadIdx.x;
    c.y = ty * blockDim.y + threadIdx.y;
    if (c.x >= g.nx || c.y >= g.ny) return false;
    fill_cell(g, c);
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

// x + (dx, dy, dz) lies beyond a face with a face rule and beyond no wall
// (such links carry flux, not force on a wall).
__device__ __forceinline__ bool beyond_rule_face(const Geom& g, const Cell& c, int dx, int dy, int dz)
{
    const int d[3] = {dx, dy, dz};
    bool rule = false, wall = false;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        if (d[a] == 0) continue;
        const int sd = d[a] < 0 ? 0 : 1;
        if (!c.wall[a][sd]) continue;
        if ((g.fix >> (2 * a + sd)) & 1u) {
            rule = true;
        } else {
            wall = true;
        }
    }
    return rule && !wall;
}

__device__ __forceinline__ bool beyond_open(const Cell& c, int dx, int dy, int dz)
{
    return (dx < 0 && c.open[0][0]) || (dx > 0 && c.open[0][1]) || (dy < 0 && c.open[1][0]) ||
           (dy > 0 && c.open[1][1]) || (dz < 0 && c.open[2][0]) || (dz > 0 && c.open[2][1]);
}

// Bit q set iff the upstream cell x - c_q is solid or beyond a wall, i.e. the
// population arriving along c_q is the bounced-back one.  A link that leaves
// through an open face (and no wall) is not bounced back, whatever the
// wrapped cell on the far side holds.
// The wrapped neighbour index is inside the box even where a face cuts the
// link, so its mask byte is read unconditionally (one uniform test for the
// mask pointer, no per-lane branch around the 18 loads).
template <bool BND>
__device__ __forceinline__ uint32_t link_bits(const Geom& g, const Cell& c)
{
    uint32_t bits = 0;
    if constexpr (BND) {
        if (g.mask != nullptr) {
            uint8_t m[kQ];
#pragma unroll
            for (int q = 0; q < kQ; ++q)
                if (q != 9) m[q] = g.mask[nbr(c, -kCx[q], -kCy[q], -kCz[q])];
#pragma unroll
            for (int q = 0; q < kQ; ++q)
                if (q != 9)
                    bits |= (uint32_t)(m[q] != 0 && !beyond_open(c, -kCx[q], -kCy[q], -kCz[q])) << q;
        }
#pragma unroll
        for (int q = 0; q < kQ; ++q)
            if (q != 9) bits |= (uint32_t)beyond_wall(c, -kCx[q], -kCy[q], -kCz[q]) << q;
    }
    return bits;
}

// Bit q set iff the population arriving along c_q enters through an open face
// (x - c_q beyond an open face and beyond no wall).
__device__ __forceinline__ uint32_t open_bits(const Geom& g, const Cell& c)
{
    uint32_t bits = 0;
    if (g.open != 0) {
#pragma unroll
        for (int q = 0; q < kQ; ++q)
            if (q != 9)
                bits |= (uint32_t)(beyond_open(c, -kCx[q], -kCy[q], -kCz[q]) &&
                                   !beyond_wall(c, -kCx[q], -kCy[q], -kCz[q]))
                        << q;
    }
    return bits;
}

// The faces through which population q can enter a cell: x - c_q lies beyond
// the low face of axis a when c_q[a] > 0, beyond the high face when c_q[a] <
// 0.  f0 is on the first axis with c_q[a] != 0 (x, y, z order), f1 on the
// second (-1 if c_q has one nonzero component).  Where both are open, f0 is
// used.
template <int q>
struct Entering {
    static constexpr int a0 = kCx[q] != 0 ? 0 : kCy[q] != 0 ? 1 : 2;
    static constexpr int a1 = (a0 < 1 && kCy[q] != 0) ? 1 : (a0 < 2 && kCz[q] != 0) ? 2 : -1;
    static constexpr int c0 = a0 == 0 ? kCx[q] : a0 == 1 ? kCy[q] : kCz[q];
    static constexpr int c1 = a1 == 1 ? kCy[q] : a1 == 2 ? kCz[q] : 0;
    static constexpr int side0 = c0 > 0 ? 0 : 1;
    static constexpr int f0 = 2 * a0 + side0;
    static constexpr int f1 = a1 < 0 ? -1 : 2 * a1 + (c1 > 0 ? 0 : 1);
};

// v, pinned in a register.  "Loaded value or reservoir constant" is
// otherwise turned into one load through a selected pointer (a flat load,
// and the constant copied to private memory for it to point at).
template <typename T>
__device__ __forceinline__ T in_register(T v)
{
    asm("" : "+v"(v));
    return v;
}

// The reservoir value of population q entering c (stored, shifted form).
template <int q, typename T>
__device__ __forceinline__ T entering_value(const Phys<T>& p, const Cell& c)
{
    using E = Entering<q>;
    if constexpr (E::f1 < 0) {
        return p.seq[E::f0][q];
    } else {
        return c.open[E::a0][E::side0] ? p.seq[E::f0][q] : p.seq[E::f1][q];
    }
}

// Odd in-place step: where x + c_q lies beyond an open face, f*_q leaves the
// box and the slot it would have taken, the own slot (opp q, x), receives the
// reservoir's population entering along -c_q: f[q] := that value.
template <int q = 0, typename T>
__device__ __forceinline__ void open_outflow(T (&f)[kQ], uint32_t obits, const Phys<T>& p, const Cell& c)
{
    if constexpr (q < kQ) {
        if constexpr (q != 9) f[q] = ((obits >> opp(q)) & 1u) ? entering_value<opp(q)>(p, c) : f[q];
        open_outflow<q + 1>(f, obits, p, c);
    }
}

// f[q] := the reservoir value where population q enters through an open face.
template <int q = 0, typename T>
__device__ __forceinline__ void apply_open(T (&f)[kQ], uint32_t obits, const Phys<T>& p, const Cell& c)
{
    if constexpr (q < kQ) {
        if constexpr (q != 9) f[q] = ((obits >> q) & 1u) ? entering_value<q>(p, c) : in_register(f[q]);
        apply_open<q + 1>(f, obits, p, c);
    }
}

// ------------------------------------------------------------- collision

// Lattice weights, each correctly rounded to T.  No set of fp32 weights can
// make both sum_q w_q = 1 and 3 sum_q w_q c_q c_q = 1 exact, so conservation is
// secured another way: storage is shifted (s = f - w, below), which turns the
// mass error of the weight sum into drho * (sum w - 1), and the equilibrium's
// odd part is built so that its first moment is rho u exactly (odd_parts).
// An earlier choice, weights nudged to sum exactly to 1, left 36 w36 = 1 -
// 6e-8 and so removed omega * 6e-8 of the momentum in every collision (the
// 128^3 Taylor-Green energy then fell 2e-5 below the fp64 result per 100
// steps).
template <typename T>
struct Weights {
    static constexpr T w36 = T(1) / T(36);
    static constexpr T w18 = T(1) / T(18);
    static constexpr T w0 = T(1) / T(3);
};

template <typename T>
__device__ __forceinline__ T wq(int q)
{
    return kW36[q] == 12 ? Weights<T>::w0 : kW36[q] == 2 ? Weights<T>::w18 : Weights<T>::w36;
}

// Stored populations are shifted by their weights, s_q = f_q - w_q (the
// populations of the fluid at rest with rho = 1 are subtracted).  Collision
// then works on deviations of order 1e-3 instead of values of order 0.3, so
// fp32 rounding errors shrink by two to three orders of magnitude; near rest
// (where every cell rounds alike) unshifted fp32 drifts in mass by ~1e-9 per
// cell and step.  In exact arithmetic the update is unchanged: sum_q w_q = 1,
// sum_q w_q c_q = 0, so rho = 1 + sum_q s_q and j = sum_q c_q s_q, and
// s*_q = s_q + omega (feq_q - w_q - s_q) + F_q.  Streaming moves s exactly as
// it would move f (w_q = w_opposite(q)).

// 1 / b for fp32: the hardware reciprocal (within 1 ulp) refined by one
// Newton step, r + r (1 - b r), which leaves it within about half an ulp.
__device__ __forceinline__ float recip_nr(float b)
{
    const float r = __builtin_amdgcn_rcpf(b);
    return fmaf(fmaf(-b, r, 1.0f), r, r);
}

// a / b from r ~ 1 / b: q0 = a r is within an ulp or so, the residual
// a - b q0 is exact in one fma, and q0 + r (a - b q0) rounds to the
// correctly rounded quotient except when 1/b itself sits almost exactly
// between two floats (Markstein's correction; b is the density, of order 1,
// so no scaling is needed).
__device__ __forceinline__ float quotient_rn(float a, float b, float r)
{
    const float q0 = a * r;
    return fmaf(fmaf(-b, q0, a), r, q0);
}

// drho = sum_q s_q (q order), rho = 1 + drho, j = sum_q c_q s_q,
// u = (j + F/2) / rho.
template <typename T, bool FORCE>
__device__ __forceinline__ void moments(const T (&s)[kQ], const Phys<T>& p, T& drho, T& rho, T& ux, T& uy,
                                        T& uz)
{
    drho = s[0];
#pragma unroll
    for (int q = 1; q < kQ; ++q) drho = drho + s[q];
    rho = T(1) + drho;
    T xp = T(0), xm = T(0), yp = T(0), ym = T(0), zp = T(0), zm = T(0);
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        if (kCx[q] > 0) xp = xp + s[q];
        if (kCx[q] < 0) xm = xm + s[q];
        if (kCy[q] > 0) yp = yp + s[q];
        if (kCy[q] < 0) ym = ym + s[q];
        if (kCz[q] > 0) zp = zp + s[q];
        if (kCz[q] < 0) zm = zm + s[q];
    }
    T jx = xp - xm, jy = yp - ym, jz = zp - zm;
    if constexpr (FORCE) {
        jx = jx + p.hfx;
        jy = jy + p.hfy;
        jz = jz + p.hfz;
    }
    // u = j / rho.  j * (1 / rho) rounds twice and, in fp32, biases the
    // velocity enough to lift the 128^3 Taylor-Green energy by 1e-8 per step
    // against the fp64 result; the quotient must be (nearly) correctly
    // rounded.  fp64 divides; fp32 takes one reciprocal per cell and corrects
    // each quotient with its exact residual (quotient_rn below).
    if constexpr (sizeof(T) == 4) {
        const T r = recip_nr(rho);
        ux = quotient_rn(jx, rho, r);
        uy = quotient_rn(jy, rho, r);
        uz = quotient_rn(jz, rho, r);
    } else {
        ux = jx / rho;
        uy = jy / rho;
        uz = jz / rho;
    }
}

template <int q, typename T>
__device__ __forceinline__ T cdot(T ax, T ay, T az)
{
    T r = T(0);
    if constexpr (kCx[q] > 0) r = r + ax;
    if constexpr (kCx[q] < 0) r = r - ax;
    if constexpr (kCy[q] > 0) r = r + ay;
    if constexpr (kCy[q] < 0) r = r - ay;
    if constexpr (kCz[q] > 0) r = r + az;
    if constexpr (kCz[q] < 0) r = r - az;
    return r;
}

constexpr bool is_diagonal(int q) { return sq(kCx[q]) + sq(kCy[q]) + sq(kCz[q]) == 2; }

// Odd parts o_q (s_q gets +o_q, s_opp(q) gets -o_q) of the shifted equilibrium
// for the nine pairs q < 9.  Diagonal pairs: w rho 3 (c.u).  Axis pairs (q = 8,
// 6, 2, along -x, -y, -z): whatever makes sum_q c_q feq_q = rho u hold in T up
// to unbiased rounding, rho u_a / 2 minus the diagonal pairs' share; with exact
// weights this equals w18 rho 3 (c.u), the textbook value.
template <typename T>
__device__ __forceinline__ void odd_parts(T rho, T ux, T uy, T uz, T (&o)[9])
{
    T sx = T(0), sy = T(0), sz = T(0);
#pragma unroll
    for (int q = 0; q < 9; ++q) {
        if (!is_diagonal(q)) continue;
        T cu = T(0);
        if (kCx[q] > 0) cu = cu + ux;
        if (kCx[q] < 0) cu = cu - ux;
        if (kCy[q] > 0) cu = cu + uy;
        if (kCy[q] < 0) cu = cu - uy;
        if (kCz[q] > 0) cu = cu + uz;
        if (kCz[q] < 0) cu = cu - uz;
        o[q] = Weights<T>::w36 * (rho * (T(3) * cu));
        if (kCx[q] > 0) sx = sx + o[q];
        if (kCx[q] < 0) sx = sx - o[q];
        if (kCy[q] > 0) sy = sy + o[q];
        if (kCy[q] < 0) sy = sy - o[q];
        if (kCz[q] > 0) sz = sz + o[q];
        if (kCz[q] < 0) sz = sz - o[q];
    }
    static_assert(kCx[8] == -1 && kCy[6] == -1 && kCz[2] == -1, "axis pairs are q = 8, 6, 2");
    o[8] = -(T(0.5) * rho * ux - sx);
    o[6] = -(T(0.5) * rho * uy - sy);
    o[2] = -(T(0.5) * rho * uz - sz);
}

// Even part of the shifted equilibrium of pair q: w (drho + rho (9/2 (c.u)^2 - 3/2 u^2)).
template <int q, typename T>
__device__ __forceinline__ T even_part(T drho, T rho, T ux, T uy, T uz, T k15)
{
    const T cu = cdot<q>(ux, uy, uz);
    return wq<T>(q) * (drho + rho * (T(4.5) * cu * cu - k15));
}

template <typename T>
__device__ __forceinline__ T k15_of(T ux, T uy, T uz)
{
    return T(1.5) * (ux * ux + uy * uy + uz * uz);
}

template <int q, typename T, bool FORCE>
__device__ __forceinline__ void relax_pair(T (&s)[kQ], const Phys<T>& p, T drho, T rho, T ux, T uy, T uz, T k15,
                                           T guF, T odd)
{
    constexpr int o = opp(q);
    const T even = even_part<q>(drho, rho, ux, uy, uz, k15);
    T nq = fma(p.omega, (even + odd) - s[q], s[q]);
    T no = fma(p.omega, (even - odd) - s[o], s[o]);
    if constexpr (FORCE) {
        // Guo term of the pair, even part then odd part (constants in Phys)
        const T geven = p.gev[q] * cdot<q>(ux, uy, uz) - guF;
        nq = nq + (geven + p.god[q]);
        no = no + (geven - p.god[q]);
    }
    s[q] = nq;
    s[o] = no;
}

// BGK collision of one cell, in place on the shifted populations; also hands
// back the density and velocity it relaxed toward (u includes F/2).
template <typename T, bool FORCE>
__device__ __forceinline__ void collide(T (&s)[kQ], const Phys<T>& p, T& rho, T& ux, T& uy, T& uz)
{
    T drho;
    moments<T, FORCE>(s, p, drho, rho, ux, uy, uz);
    const T k15 = k15_of(ux, uy, uz);
    T uF = T(0), guF0 = T(0), guF18 = T(0), guF36 = T(0);
    if constexpr (FORCE) {
        uF = ux * p.fx + uy * p.fy + uz * p.fz;
        guF0 = p.gu[0] * uF;
        guF18 = p.gu[1] * uF;
        guF36 = p.gu[2] * uF;
    }
    T od[9];
    odd_parts(rho, ux, uy, uz, od);
#define LBM_RELAX(q) relax_pair<q, T, FORCE>(s, p, drho, rho, ux, uy, uz, k15, is_diagonal(q) ? guF36 : guF18, od[q])
    LBM_RELAX(0);
    LBM_RELAX(1);
    LBM_RELAX(2);
    LBM_RELAX(3);
    LBM_RELAX(4);
    LBM_RELAX(5);
    LBM_RELAX(6);
    LBM_RELAX(7);
    LBM_RELAX(8);
#undef LBM_RELAX
    // rest population: shifted equilibrium w0 (drho - rho 3/2 u^2)
    const T e9 = wq<T>(9) * (drho - rho * k15);
    T n9 = fma(p.omega, e9 - s[9], s[9]);
    if constexpr (FORCE) n9 = n9 - guF0;
    s[9] = n9;
}

template <typename T, bool FORCE>
__device__ __forceinline__ void collide(T (&s)[kQ], const Phys<T>& p)
{
    T rho, ux, uy, uz;
    collide<T, FORCE>(s, p, rho, ux, uy, uz);
}

// Destination of the macroscopic fields a step can write as it goes (the
// density and velocity its collision used): rho[N], u[3][N] in cell order.
template <typename T>
struct MomOut {
    T* rho;
    T* u;
    uint64_t n;
    double* partial;      // fused momentum exchange: six sums per workgroup (MEX instances)
    const uint8_t* mask;  // compact layout with output: the solid cells the waves zero (null: none)
};

template <typename T>
__device__ __forceinline__ void write_moments(const MomOut<T>& o, uint64_t id, T rho, T ux, T uy, T uz)
{
    o.rho[id] = rho;
    o.u[id] = ux;
    o.u[o.n + id] = uy;
    o.u[2 * o.n + id] = uz;
}

// Shifted equilibrium populations of (rho, u): s_q = feq_q(rho, u) - w_q, built
// exactly as in the collision.
template <typename T>
__device__ __forceinline__ void shifted_equilibrium(T rho, T ux, T uy, T uz, T (&s)[kQ])
{
    const T drho = rho - T(1);
    const T k15 = k15_of(ux, uy, uz);
    T od[9];
    odd_parts(rho, ux, uy, uz, od);
#define LBM_SEQ_PAIR(q)                                                      \
    {                                                                        \
        const T e = even_part<q>(drho, rho, ux, uy, uz, k15);                \
        s[q] = e + od[q];                                                    \
        s[opp(q)] = e - od[q];                                               \
    }
    LBM_SEQ_PAIR(0)
    LBM_SEQ_PAIR(1)
    LBM_SEQ_PAIR(2)
    LBM_SEQ_PAIR(3)
    LBM_SEQ_PAIR(4)
    LBM_SEQ_PAIR(5)
    LBM_SEQ_PAIR(6)
    LBM_SEQ_PAIR(7)
    LBM_SEQ_PAIR(8)
#undef LBM_SEQ_PAIR
    s[9] = wq<T>(9) * (drho - rho * k15);
}

// ------------------------------------------------- momentum exchange sums
//
// During a step every population f*_q that leaves a fluid cell toward a solid
// cell or through a wall comes back along -c_q (halfway bounce-back), so the
// solid takes 2 f*_q c_q (fieldcraft page, first section: the momentum
// exchange over the wall links of a step).  Sums are in double, per
// workgroup in a fixed order, then over the workgroups in a fixed order.

// v[0..5] summed over the workgroup (at most NT work-items, 2-D blocks
// flattened x-fastest, which is how the hardware forms its waves); thread 0
// writes the six sums to out.  Every work-item of the workgroup must call it.
template <int NT>
__device__ __forceinline__ void block_sum6(double (&v)[6], double* __restrict__ out)
{
    __shared__ double part[NT / 64][6];
    const uint32_t tid = threadIdx.x + blockDim.x * threadIdx.y;
#pragma unroll
    for (int k = 0; k < 6; ++k)
        for (int o = 32; o > 0; o >>= 1) v[k] += __shfl_down(v[k], o, 64);
    if ((tid & 63u) == 0)
#pragma unroll
        for (int k = 0; k < 6; ++k) part[tid / 64][k] = v[k];
    __syncthreads();
    if (tid == 0) {
#pragma unroll
        for (int k = 0; k < 6; ++k) {
            double s = part[0][k];
            for (uint32_t w = 1; w < (blockDim.x * blockDim.y + 63) / 64; ++w) s += part[w][k];
            out[k] = s;
        }
    }
}

// Add 2 f*_q c_q of the outgoing link q (stored value s*_q = f*_q - w_q, w_q
// rounded to T as in storage) to the solid (acc[0..2]) or wall (acc[3..5])
// sums; f* is formed in double, so no rounding of s* + w to T.
template <int q, typename T>
__device__ __forceinline__ void add_link(double (&acc)[6], T spost, bool bounced, bool wall)
{
    const double v = bounced ? 2.0 * ((double)spost + (double)wq<T>(q)) : 0.0;
    const double vs = wall ? 0.0 : v, vw = wall ? v : 0.0;
    if constexpr (kCx[q] != 0) {
        acc[0] += kCx[q] * vs;
        acc[3] += kCx[q] * vw;
    }
    if constexpr (kCy[q] != 0) {
        acc[1] += kCy[q] * vs;
        acc[4] += kCy[q] * vw;
    }
    if constexpr (kCz[q] != 0) {
        acc[2] += kCz[q] * vs;
        acc[5] += kCz[q] * vw;
    }
}

template <int q = 0, typename T, typename Pred>
__device__ __forceinline__ void add_links(double (&acc)[6], const T (&s)[kQ], const Cell& c, Pred bounced)
{
    if constexpr (q < kQ) {
        if constexpr (q != 9) add_link<q>(acc, s[q], bounced(q), beyond_wall(c, kCx[q], kCy[q], kCz[q]));
        add_links<q + 1>(acc, s, c, bounced);
    }
}

// ------------------------------------------------------ stored-state maps

// Where the canonical population f_q(x, t) lives for a stored state of kind S
// (kAB: the source lattice holds h(t) with f(t) = stream(h(t)); kAAEven: the
// lattice holds f(t) in natural slots; kAAOdd: it holds the post-collision
// values of step t-1 in swapped slots).  This is the gather half of a step.
// Both candidate offsets are formed and one is selected (v_cndmask): the
// arms are a uniform plane offset plus a per-lane add, cheap enough that the
// select is not turned into a divergent branch around the load.
//
// Esoteric pull (kEsoEven / kEsoOdd, parity P): the pair p < 9, c = c_p,
// keeps two slots per cell, S0 = plane p and S1 = plane opp(p).  A step of
// parity P reads f_p from the own slot (x, S_P) -- where the cell x - c put
// f*_p -- and f_opp(p) from (x + c, S_{1-P}) -- where x + c put f*_opp(p) --
// and writes f*_opp(p) into the first and f*_p into the second: the next step
// finds them as the populations that reached x - c and x + c.  A link that
// ends outside the fluid keeps its value in a slot no other cell touches: the
// own side (x - c solid or beyond a face) in the own S0; the neighbour side in
// the S0 of x + c if that is a solid cell, and in the S1 of the wrapped cell
// if x + c lies beyond a face (that cell's own side then lies beyond the
// opposite face and uses its S0).  obits: the reservoir links (open_bits).
template <int S, int L>
__device__ __forceinline__ uint64_t eso_off(uint64_t n, const Cell& c, uint32_t bits, uint32_t obits, int q)
{
    constexpr bool odd = S == kEsoOdd;
    if (q == 9) return slot_off<L>(n, 9, c.id);
    const bool out = ((bits | obits) >> q) & 1u;  // the upstream cell x - c_q is not fluid
    if (q < 9) {
        const uint64_t s0 = slot_off<L>(n, q, c.id);
        if constexpr (!odd) {
            return s0;
        } else {
            const uint64_t s1 = slot_off<L>(n, opp(q), c.id);
            return out ? s0 : s1;
        }
    } else {
        const int p = opp(q);  // x + c_p = x - c_q
        const uint32_t up = nbr(c, kCx[p], kCy[p], kCz[p]);
        const uint64_t s1 = slot_off<L>(n, q, up), s0 = slot_off<L>(n, p, up);
        const bool face = beyond_wall(c, kCx[p], kCy[p], kCz[p]) || beyond_open(c, kCx[p], kCy[p], kCz[p]);
        // normal: S_{1-P} of the neighbour; solid: its S0; beyond a face: S1
        const uint64_t normal = odd ? s0 : s1;
        return !out ? normal : face ? s1 : s0;
    }
}

// Esoteric twist (kTwEven / kTwOdd, parity P).  With c+ = max(c_q, 0) per
// axis, f_q(x) lives at the location x - c+ (the cell itself or one of the
// six cells behind it along -x, -y, -z and the face diagonals between them)
// in plane q (P = 0) or opp(q) (P = 1).  A step reads every f_q there and
// writes f*_q where it read f_opp(q), i.e. at x + c- (c- = min(c_q, 0)) in
// plane opp(q) (P = 0) or q (P = 1): the next step finds it there as the
// population that reached x + c_q.  A bounced-back f*_q goes to the other
// plane of that location instead, where x itself finds f_opp(q) next.
// Behind a low face that is not periodic the location lies below the box
// (it holds a bounced or reservoir value of the cell next to it); on a
// periodic axis it wraps.  The dense storage of this scheme keeps the cells
// of the box at their cell index (rows stay line-aligned) and the cells of
// the layer below the low faces after them: first those with x = -1
// ((ny+1)(nz+1), y and z from -1), then y = -1 (nx (nz+1)), then z = -1
// (nx ny), (nx+1)(ny+1)(nz+1) cells per plane in all.
__device__ __forceinline__ uint64_t twist_cells(const Geom& g)
{
    return (uint64_t)(g.nx + 1) * (uint64_t)(g.ny + 1) * (uint64_t)(g.nz + 1);
}

// storage index of x - (ox, oy, oz), o in {0, 1}^3
__device__ __forceinline__ uint32_t twist_loc(const Geom& g, const Cell& c, int ox, int oy, int oz)
{
    // coordinate of v - o: v - o, or behind the low face -1 if that face is
    // not periodic (then `below`), else the wrapped cell n - 1
    auto back = [](uint32_t v, int o, bool face, uint32_t n, bool& below) -> uint32_t {
        if (o == 0 || v > 0u) return v - (uint32_t)o;
        below = face;
        return face ? 0u : n - 1u;
    };
    bool bx = false, by = false, bz = false;
    const uint32_t x = back(c.x, ox, c.wall[0][0] || c.open[0][0], g.nx, bx);
    const uint32_t y = back(c.y, oy, c.wall[1][0] || c.open[1][0], g.ny, by);
    const uint32_t z = back(c.z, oz, c.wall[2][0] || c.open[2][0], g.nz, bz);
    const uint32_t n = (uint32_t)g.n;
    const uint32_t h1 = (g.ny + 1u) * (g.nz + 1u), h2 = g.nx * (g.nz + 1u);
    // (a coordinate flagged below is -1: y + 1 and z + 1 are then 0)
    const uint32_t yb = by ? 0u : y + 1u, zb = bz ? 0u : z + 1u;
    if (bx) return n + yb + (g.ny + 1u) * zb;
    if (by) return n + h1 + x + g.nx * zb;
    if (bz) return n + h1 + h2 + x + g.nx * y;
    return x + g.nx * (y + g.ny * z);
}

// element offset of f_q(x) in a twist state of parity P
template <int P, int L>
__device__ __forceinline__ uint64_t twist_off(const Geom& g, const Cell& c, int q)
{
    const int pl = P == 0 ? q : opp(q);
    return slot_off<L>(twist_cells(g), pl, twist_loc(g, c, kCx[q] > 0, kCy[q] > 0, kCz[q] > 0));
}

template <int S, int L, typename T>
__device__ __forceinline__ T* state_slot(T* buf, const Geom& g, const Cell& c, uint32_t bits, int q,
                                         uint32_t obits = 0u)
{
    const uint64_t n = g.n;
    if constexpr (is_twist(S)) return buf + twist_off<S == kTwOdd ? 1 : 0, L>(g, c, q);
    if constexpr (is_eso(S)) return buf + eso_off<S, L>(n, c, bits, obits, q);
    const bool bb = (bits >> q) & 1u;
    const uint32_t up = nbr(c, -kCx[q], -kCy[q], -kCz[q]);
    if constexpr (S == kAB) {
        const uint64_t own = slot_off<L>(n, opp(q), c.id), far = slot_off<L>(n, q, up);
        return buf + (bb ? own : far);
    } else if constexpr (S == kAAEven) {
        return slot<L>(buf, n, q, c.id);
    } else {
        const uint64_t own = slot_off<L>(n, q, c.id), far = slot_off<L>(n, opp(q), up);
        return buf + (bb ? own : far);
    }
}

// ----------------------------------------------------------------- kernels

constexpr int kBlockThreads = 256;

// The update of one fluid cell by step_kernel.
template <typename T, int L, int K, int BND, bool FORCE, bool OUT, bool MEX>
__device__ __forceinline__ void step_cell(T* __restrict__ a, T* __restrict__ b, const Geom& g, const Phys<T>& p,
                                          const MomOut<T>& mo, const Cell& c, double (&acc)[6])
{
    const uint32_t bits = link_bits<BND != 0>(g, c);
    const uint32_t obits = BND == 2 ? open_bits(g, c) : 0u;  // populations entering through open faces
    const uint64_t n = g.n;

    T f[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        if constexpr (K == kAB) {
            f[q] = ld_pop(state_slot<kAB, L>(a, g, c, bits, q));
        } else if constexpr (K == kAAEven) {
            f[q] = ld_pop_own<BND == 0 && L != kCollision>(slot<L>(a, n, q, c.id));
        } else if constexpr (K == kAAOdd) {
            f[q] = ld_pop(state_slot<kAAOdd, L>(a, g, c, bits, q));
        } else if constexpr (is_twist(K)) {
            f[q] = ld_pop(a + twist_off<K == kTwOdd ? 1 : 0, L>(g, c, q));
        } else {
            f[q] = ld_pop(a + eso_off<K, L>(n, c, bits, obits, q));
        }
    }
    // the even step's natural slots already hold the reservoir values (the odd
    // step and the initialisation put them there); the gathers take them here
    if constexpr (BND == 2 && K != kAAEven) apply_open(f, obits, p, c);

    T rho, ux, uy, uz;
    collide<T, FORCE>(f, p, rho, ux, uy, uz);
    if constexpr (OUT) write_moments(mo, c.id, rho, ux, uy, uz);
    // MEX: x + c_q is solid or beyond a wall iff the upstream bit of opp(q)
    // is set; a face with a face rule sets it too, but its links carry flux.
    // Summed after the stores (f is still f*), unless open_outflow changes f.
    constexpr bool kMexEarly = BND == 2 && K == kAAOdd;
    const auto link_bounced = [&](int q) {
        return ((bits >> opp(q)) & 1u) != 0 && !beyond_rule_face(g, c, kCx[q], kCy[q], kCz[q]);
    };
    if constexpr (MEX && kMexEarly) add_links(acc, f, c, link_bounced);
    if constexpr (BND == 2 && K == kAAOdd) open_outflow(f, obits, p, c);

#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        if constexpr (K == kAB) {
            st_pop<L>(slot<L>(b, n, q, c.id), f[q]);
        } else if constexpr (K == kAAEven) {
            st_pop<L>(slot<L>(a, n, opp(q), c.id), f[q]);
        } else if constexpr (is_eso(K)) {
            // into the slot f_opp(q) was read from
            st_pop<L>(a + eso_off<K, L>(n, c, bits, obits, opp(q)), f[q]);
        } else if constexpr (is_twist(K)) {
            // where f_opp(q) was read from; bounced back (x + c_q solid or
            // beyond a wall: the upstream bit of opp q), the other plane there
            constexpr int P = K == kTwOdd ? 1 : 0;
            const uint64_t normal = twist_off<P, L>(g, c, opp(q)), back = twist_off<1 - P, L>(g, c, opp(q));
            st_pop<L>(a + (((bits >> opp(q)) & 1u) ? back : normal), f[q]);
        } else {
            // toward x + c_q, or straight back into (opp q, x) if that cell is
            // solid or beyond a wall (its upstream bit for opp q is set); if
            // x + c_q lies beyond an open face, f*_q leaves the box and (opp q,
            // x) receives the reservoir's population entering along -c_q
            // (the reservoir values were put into f by open_outflow above)
            const bool own_slot = ((bits | obits) >> opp(q)) & 1u;
            const uint64_t own = slot_off<L>(n, opp(q), c.id);
            const uint64_t far = slot_off<L>(n, q, nbr(c, kCx[q], kCy[q], kCz[q]));
            st_pop<L>(a + (own_slot ? own : far), f[q]);
        }
    }
    if constexpr (MEX && !kMexEarly) add_links(acc, f, c, link_bounced);
}

// ------------------------------------- row-bundled access (AoS and SoAoS)
//
// In the collision (AoS) and bundle (SoAoS) layouts the three directions of a
// stencil row -- equal (c_y, c_z), c_x = -1, 0, +1, the runs {1,2,3} {5,6,7}
// {8,9,10} {11,12,13} {15,16,17} of the canonical order -- are adjacent slots
// of a cell, and a step's gather for them reads three adjacent slots from
// the cells x - 1, x, x + 1 of one neighbour row.  Lanes of a wave hold
// consecutive x of one row (tiles are at least 32 cells wide: a wave is one
// 64-cell row segment or two 32-cell ones), so every lane loads the three
// slots of its own x in one 12-byte access and the x - 1 / x + 1 values move
// between neighbouring lanes by a cross-lane shift; a lane at either end of
// its segment loads the one value from outside directly.  The odd in-place
// step's scatter is assembled the same way: a lane stores the three slots of
// the cell at its own x in the target row, the values coming from the lanes
// that computed them, and a segment's end lane stores the one value whose
// target cell lies beyond the segment.  Every slot keeps the writer the
// generic kernel gives it (its upstream cell, in the same wave), and a wave
// only uses values of slots it writes itself (loads meant for a lane beyond
// the segment are discarded), so the in-place step stays race-free.
//
// Used where it measured faster: boxes without solid cells or walls (the
// no-mask periodic instance), for the odd in-place step of both layouts and
// the pull of the bundle layout (periodic 256^3, fp32, per launch: AoS odd
// 2.114 -> 1.948 ms, SoAoS odd 0.515 -> 0.471 ms, SoAoS pull 0.458 -> 0.450
// ms).  The AoS pull is left out: with plain stores it went 0.930 -> 0.910
// ms on the 256^3 box but 0.109 -> 0.117 ms at 128^3.  With solid cells every lane
// must still load for its neighbours and the bounced links add own-record
// accesses and per-slot stores: on the 256^3 porous box the AoS odd step
// took 1.43 ms against 1.19 ms, the SoAoS one 0.80 against 0.59 ms.
#ifndef LBM_ROW_BUNDLED
#define LBM_ROW_BUNDLED 1
#endif
template <int L, int K, int BND>
constexpr bool bundled_path()
{
    return LBM_ROW_BUNDLED && BND == 0 &&
           ((K == kAAOdd && (L == kCollision || L == kBundle)) || (K == kAB && L == kBundle));
}

// Three consecutive slots of one lane.  fp32: one 12-byte access
// (dwordx3).  fp64: a 16-byte and an 8-byte access; a three-element double
// vector would be widened to 32 bytes, and its store would overwrite the
// slot after the triple.
template <typename T>
struct Vec3 {
    T x, y, z;
};

typedef float f32x3_a4 __attribute__((ext_vector_type(3), aligned(4)));
typedef double f64x2_a8 __attribute__((ext_vector_type(2), aligned(8)));

template <typename T>
__device__ __forceinline__ Vec3<T> ld3(const T* p)
{
    Vec3<T> r;
    if constexpr (sizeof(T) == 4) {
        const f32x3_a4 v = *(const f32x3_a4*)p;
        r.x = v.x;
        r.y = v.y;
        r.z = v.z;
    } else {
        const f64x2_a8 v = *(const f64x2_a8*)p;
        r.x = v.x;
        r.y = v.y;
        r.z = p[2];
    }
    return r;
}

template <int L, typename T>
__device__ __forceinline__ void st3(T* p, Vec3<T> v)
{
    if constexpr (sizeof(T) == 4) {
        f32x3_a4 w;
        w.x = v.x;
        w.y = v.y;
        w.z = v.z;
        st_pop<L>((f32x3_a4*)p, w);
    } else {
        f64x2_a8 w;
        w.x = v.x;
        w.y = v.y;
        st_pop<L>((f64x2_a8*)p, w);
        st_pop<L>(p + 2, v.z);
    }
}

// two consecutive slots
template <int L, typename T>
__device__ __forceinline__ void st2(T* p, T a, T b)
{
    typedef T v2 __attribute__((ext_vector_type(2), aligned(sizeof(T))));
    v2 w;
    w.x = a;
    w.y = b;
    st_pop<L>((v2*)p, w);
}

// A row of three directions q0 = B, q1 = B + 1, q2 = B + 2 (c_x = -1, 0, +1);
// the opposite row is opp(q2), opp(q1), opp(q0) in slot order.
template <int B>
struct Row3 {
    static constexpr int q0 = B, q1 = B + 1, q2 = B + 2;
    static constexpr int cy = kCy[B], cz = kCz[B];
    static_assert(kBundleSize[B] == 3 && kBundleFirst[B] == B && kCx[q0] == -1 && kCx[q2] == 1, "stencil row");
};

// Gather of one three-direction row: f_q = (opp q, x - c_q) for the odd
// in-place step (K = kAAOdd), src (q, x - c_q) for the pull (K = kAB).
// first / last: this lane ends its segment on the left / right.
template <int B, int L, int K, typename T>
__device__ __forceinline__ void gather_row3(const T* __restrict__ a, const Geom& g, const Cell& c, bool first,
                                            bool last, T (&f)[kQ])
{
    using R = Row3<B>;
    const uint64_t n = g.n;
    constexpr int lo = K == kAAOdd ? opp(R::q2) : R::q0;  // first slot of the triple read at x
    const Vec3<T> v = ld3(a + slot_off<L>(n, lo, nbr(c, 0, -R::cy, -R::cz)));
    // f_q0 (c_x = -1) comes from x + 1, f_q2 (c_x = +1) from x - 1
    constexpr int s0 = K == kAAOdd ? opp(R::q0) : R::q0;
    constexpr int s2 = K == kAAOdd ? opp(R::q2) : R::q2;
    T from_next = __shfl_down(K == kAAOdd ? v.z : v.x, 1, 64);
    T from_prev = __shfl_up(K == kAAOdd ? v.x : v.z, 1, 64);
    if (last) from_next = a[slot_off<L>(n, s0, nbr(c, 1, -R::cy, -R::cz))];
    if (first) from_prev = a[slot_off<L>(n, s2, nbr(c, -1, -R::cy, -R::cz))];
    f[R::q0] = from_next;
    f[R::q1] = v.y;
    f[R::q2] = from_prev;
}

// Scatter of one three-direction row for the odd in-place step: f*_q to
// (q, x + c_q).  This lane stores the row's slots of the target cell at its
// own x, (x, y + c_y, z + c_z), written by the cells x + 1, x, x - 1.
template <int B, int L, typename T>
__device__ __forceinline__ void scatter_row3_odd(T* __restrict__ a, const Geom& g, const Cell& c, bool first,
                                                 bool last, const T (&f)[kQ])
{
    using R = Row3<B>;
    const uint64_t n = g.n;
    const T w0 = __shfl_down(f[R::q0], 1, 64);  // f*_q0 of x + 1
    const T w2 = __shfl_up(f[R::q2], 1, 64);    // f*_q2 of x - 1
    T* const t = a + slot_off<L>(n, R::q0, nbr(c, 0, R::cy, R::cz));
    if (!first && !last) {
        Vec3<T> w;
        w.x = w0;
        w.y = f[R::q1];
        w.z = w2;
        st3<L>(t, w);
    } else {
        // a segment end: the slot whose writer lies beyond the segment is
        // that writer's, and this lane's value bound beyond the segment is
        // stored here
        if (!first) {
            st2<L>(t + 1, f[R::q1], w2);
        } else if (!last) {
            st2<L>(t, w0, f[R::q1]);
        } else {
            st_pop<L>(t + 1, f[R::q1]);
        }
        if (first) st_pop<L>(a + slot_off<L>(n, R::q0, nbr(c, -1, R::cy, R::cz)), f[R::q0]);
        if (last) st_pop<L>(a + slot_off<L>(n, R::q2, nbr(c, 1, R::cy, R::cz)), f[R::q2]);
    }
}

// The update of one cell by step_kernel on the row-bundled path (every cell
// of the box is fluid and every link stays inside the box).
template <typename T, int L, int K, bool FORCE, bool OUT>
__device__ __forceinline__ void step_cell_bundled(T* __restrict__ a, T* __restrict__ b, const Geom& g,
                                                  const Phys<T>& p, const MomOut<T>& mo, const Cell& c)
{
    static_assert(bundled_path<L, K, 0>(), "row-bundled access");
    const uint64_t n = g.n;
    // segment ends: the wave's lanes cover min(tile width, 64) consecutive x
    const uint32_t seg = blockDim.x < 64u ? blockDim.x : 64u;
    const uint32_t lx = threadIdx.x & (seg - 1u);
    const bool first = lx == 0u || c.x == 0u;
    const bool last = lx == seg - 1u || c.x + 1u == g.nx;
    T f[kQ];
    gather_row3<1, L, K>(a, g, c, first, last, f);
    gather_row3<5, L, K>(a, g, c, first, last, f);
    gather_row3<8, L, K>(a, g, c, first, last, f);
    gather_row3<11, L, K>(a, g, c, first, last, f);
    gather_row3<15, L, K>(a, g, c, first, last, f);
    // the four diagonal rows hold one direction each (c_x = 0)
    constexpr int kS = K == kAAOdd ? kAAOdd : kAB;
    f[0] = ld_pop(state_slot<kS, L>(a, g, c, 0u, 0));
    f[4] = ld_pop(state_slot<kS, L>(a, g, c, 0u, 4));
    f[14] = ld_pop(state_slot<kS, L>(a, g, c, 0u, 14));
    f[18] = ld_pop(state_slot<kS, L>(a, g, c, 0u, 18));
    T rho, ux, uy, uz;
    collide<T, FORCE>(f, p, rho, ux, uy, uz);
    if constexpr (OUT) write_moments(mo, c.id, rho, ux, uy, uz);
    if constexpr (K == kAB) {
#define LBM_AB_STORE3(B)                                    \
    {                                                       \
        Vec3<T> w;                                          \
        w.x = f[B];                                         \
        w.y = f[B + 1];                                     \
        w.z = f[B + 2];                                     \
        st3<L>(b + slot_off<L>(n, B, c.id), w);                \
    }
        LBM_AB_STORE3(1)
        LBM_AB_STORE3(5)
        LBM_AB_STORE3(8)
        LBM_AB_STORE3(11)
        LBM_AB_STORE3(15)
#undef LBM_AB_STORE3
        st_pop<L>(b + slot_off<L>(n, 0, c.id), f[0]);
        st_pop<L>(b + slot_off<L>(n, 4, c.id), f[4]);
        st_pop<L>(b + slot_off<L>(n, 14, c.id), f[14]);
        st_pop<L>(b + slot_off<L>(n, 18, c.id), f[18]);
    } else {
        scatter_row3_odd<1, L>(a, g, c, first, last, f);
        scatter_row3_odd<5, L>(a, g, c, first, last, f);
        scatter_row3_odd<8, L>(a, g, c, first, last, f);
        scatter_row3_odd<11, L>(a, g, c, first, last, f);
        scatter_row3_odd<15, L>(a, g, c, first, last, f);
        st_pop<L>(a + slot_off<L>(n, 0, nbr(c, kCx[0], kCy[0], kCz[0])), f[0]);
        st_pop<L>(a + slot_off<L>(n, 4, nbr(c, kCx[4], kCy[4], kCz[4])), f[4]);
        st_pop<L>(a + slot_off<L>(n, 14, nbr(c, kCx[14], kCy[14], kCz[14])), f[14]);
        st_pop<L>(a + slot_off<L>(n, 18, nbr(c, kCx[18], kCy[18], kCz[18])), f[18]);
    }
}

// One fused time step.  K: kAB (a = source, b = destination), kAAEven,
// kAAOdd, kEsoEven or kEsoOdd (a = the single lattice).  BND: 0 = fully
// periodic, no mask; 1 = a mask or a wall exists; 2 = also open faces (a
// separate instance, so the reservoir selects cost the other kernels no
// registers).  OUT: also write the density and velocity the collision used
// (0 on solid cells).  MEX: also sum the momentum exchange of the step over
// the workgroup into mo.partial (row = the workgroup's tile).
template <typename T, int L, int K, int BND, bool FORCE, bool OUT, bool MEX = false>
__global__ void __launch_bounds__(kBlockThreads) step_kernel(T* __restrict__ a, T* __restrict__ b,
                                                             Geom g, Phys<T> p, MomOut<T> mo)
{
    static_assert(!MEX || BND != 0, "a periodic box without mask has no bounce-back links");
    Cell c;
    if constexpr (bundled_path<L, K, BND>()) {
        // every cell is fluid; lanes beyond the box's rows leave
        if (!locate(g, c)) return;
        step_cell_bundled<T, L, K, FORCE, OUT>(a, b, g, p, mo, c);
        return;
    }
    bool active = locate(g, c);
    if constexpr (BND) {
        if (active && g.mask != nullptr && g.mask[c.id] != 0) {  // solid cells are never updated
            if constexpr (OUT) write_moments(mo, c.id, T(0), T(0), T(0), T(0));
            active = false;
        }
    }
    if constexpr (!MEX) {
        if (!active) return;
    }
    // MEX: also the momentum exchange of this step (the workgroup's sums go
    // to mo.partial; every work-item reaches the reduction)
    double acc[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    if (active) step_cell<T, L, K, BND, FORCE, OUT, MEX>(a, b, g, p, mo, c, acc);
    if constexpr (MEX) {
        const uint32_t tile = g.xk > 1 ? xcd_chunked(blockIdx.x, g.xk) : blockIdx.x;
        if (tile < g.ntiles) block_sum6<kBlockThreads>(acc, mo.partial + 6 * (size_t)tile);
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
        if constexpr (OP == kReadF || OP == kReadS) {
#pragma unroll
            for (int q = 0; q < kQ; ++q) out0[(uint64_t)q * n + c.id] = T(0);
        } else if constexpr (OP == kReadMoments) {
            out0[c.id] = T(0);
#pragma unroll
            for (int d = 0; d < 3; ++d) out1[(uint64_t)d * n + c.id] = T(0);
        } else if constexpr (!solid_slots_live(S)) {
            // (in the esoteric schemes a solid cell's slots hold the
            // bounce-back values of its fluid neighbours' links: not cleared)
#pragma unroll
            for (int q = 0; q < kQ; ++q) {
                *slot<L>(a, n, q, c.id) = T(0);
                if (b != nullptr) *slot<L>(b, n, q, c.id) = T(0);
            }
        }
        return;
    }
    const uint32_t bits = link_bits<true>(g, c);
    const uint32_t obits = open_bits(g, c);
    T f[kQ];
    if constexpr (OP == kReadF || OP == kReadMoments || OP == kReadS) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) f[q] = *state_slot<S, L>(a, g, c, bits, q, obits);
        if constexpr (S != kAAEven) apply_open(f, obits, p, c);
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
        // populations entering through an open face are the reservoir's: the
        // even state stores them in their natural slots, the others have no
        // slot for them (their map would point across the box)
        if constexpr (S == kAAEven) apply_open(f, obits, p, c);
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            if (S != kAAEven && ((obits >> q) & 1u)) continue;
            *state_slot<S, L>(a, g, c, bits, q, obits) = f[q];
        }
    }
}

}  // namespace lbm
