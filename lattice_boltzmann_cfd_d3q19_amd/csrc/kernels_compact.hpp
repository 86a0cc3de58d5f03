// kernels_compact.hpp -- the fluid-compacted layout ("compact").
//
// Only fluid cells are stored, ranked in cell order, in blocks of 64: block b
// holds the 19 storage planes of fluid cells 64 b .. 64 b + 63 one after the
// other, so population q of the i-th fluid cell lives at element
// (i / 64) * 19 * 64 + P(q) * 64 + i % 64, P(q) the storage plane of q
// (opposite directions side by side, below).  In a porous medium a dense
// layout moves whole cache lines that are mostly solid (in the 256^3,
// 62%-porous benchmark medium 98.6% of 128-byte lines hold some fluid, so a
// dense step moves ~1.6x the fluid bytes); here every population line is
// fully used.  A wave's 64 cells are one block: its 19 slots of a direction
// are one 256-byte run and its whole state one contiguous 4864-byte region
// (fp32), so a step streams one region per wave instead of 19 planes that
// lie S elements apart.  Measured on MI355X, 256^3 porous box, fp32, against
// 19 planes of S cells: even in-place step 0.256 -> 0.243 ms, odd step 0.367
// -> 0.342 ms, fused pull 0.331 -> 0.307 ms (an in-place swap probe with the
// even step's pattern: 6.0 -> 6.8 TB/s); the all-fluid periodic 256^3 box
// tied (0.903 -> 0.904 ms per step pair).
//
// Geometry tables (caller-owned workspace, built on the device at init):
//   idxp[p]   for every cell of the box padded by one halo layer on each side,
//             p = (x+1) + px ((y+1) + py (z+1)), px = nx+2, py = ny+2: the
//             compact index of the cell, kInvalid for solid cells; halo cells
//             hold the index of their periodic image, kWall beyond a wall
//             face (halfway bounce-back) or kOpen + k beyond open face k.
//   cellp[i]  padded id p of the i-th fluid cell.
//   cellid[i] cell index x + nx (y + ny z) of the i-th fluid cell (for the
//             macroscopic fields a step writes as it goes).
// A neighbour along c_d is then idxp[cellp[i] + off_d] with
// off_d = c_x + px (c_y + py c_z): no coordinates, no wrap logic.
#pragma once

#include "kernels.hpp"

namespace lbm {

// Index-table markers: a solid cell, and a halo cell beyond a non-periodic
// face (a wall).  Both are "no fluid neighbour" (>= kWall) to the step
// kernels; the momentum exchange tells them apart.
constexpr uint32_t kInvalid = 0xFFFFFFFFu;
constexpr uint32_t kWall = 0xFFFFFFFEu;
// halo beyond open face k (-x, +x, -y, +y, -z, +z): kOpen + k
constexpr uint32_t kOpen = 0xFFFFFFF0u;

__device__ __forceinline__ bool no_fluid(uint32_t nbv) { return nbv >= kOpen; }
__device__ __forceinline__ bool bounced(uint32_t nbv) { return nbv >= kWall; }
__device__ __forceinline__ bool is_open(uint32_t nbv) { return nbv >= kOpen && nbv < kWall; }
// beyond an open face that is a reservoir (res: bit k for face k); the other
// open faces have face rules, and their entering values are stored like
// bounced ones
__device__ __forceinline__ bool is_res(uint32_t nbv, uint32_t res)
{
    return is_open(nbv) && ((res >> ((nbv - kOpen) & 7u)) & 1u);
}

// Reservoir value of population q entering through the open face that the
// table entry nbv (of the upstream cell x - c_q) names.
template <int q, typename T>
__device__ __forceinline__ T entering_value_nb(const Phys<T>& p, uint32_t nbv)
{
    using E = Entering<q>;
    if constexpr (E::f1 < 0) {
        return p.seq[E::f0][q];
    } else {
        return nbv == kOpen + (uint32_t)E::f0 ? p.seq[E::f0][q] : p.seq[E::f1][q];
    }
}

// f[q] := the reservoir value where the upstream entry nb[opp q] is open.
template <int q = 0, typename T>
__device__ __forceinline__ void apply_open_nb(T (&f)[kQ], const uint32_t (&nb)[kQ], const Phys<T>& p)
{
    if constexpr (q < kQ) {
        if constexpr (q != 9) f[q] = is_res(nb[opp(q)], p.res) ? entering_value_nb<q>(p, nb[opp(q)]) : in_register(f[q]);
        apply_open_nb<q + 1>(f, nb, p);
    }
}

// Workgroup sizes of the compact step kernels.  Measured on the porous
// boxes: 512-thread gathers 0.5% (256^3) and 1.2% (512^3) faster than 256,
// 128 slower; the even step is fastest at 256 (128: +5%, 1024: +4% at 512^3).
#ifndef LBM_GATHER_THREADS
#define LBM_GATHER_THREADS 512
#endif
#ifndef LBM_EVEN_THREADS
#define LBM_EVEN_THREADS 256
#endif
constexpr int kGatherThreads = LBM_GATHER_THREADS;
constexpr int kEvenThreads = LBM_EVEN_THREADS;

struct CompactGeom {
    const uint32_t* idxp;
    const uint32_t* cellp;
    const uint32_t* cellid;  // cell index x + nx (y + ny z) of the i-th fluid cell
    const uint32_t* bbase;   // esoteric pull: first bounce-back slot of the i-th fluid cell
    const uint32_t* tidx;    // esoteric twist: stored index of every padded cell (fluid, ghost) or kInvalid
    uint32_t nf;   // fluid cells
    uint32_t px;   // nx + 2
    uint32_t pxy;  // (nx + 2)(ny + 2)
    uint32_t s;    // stored cells (fluid, and the esoteric twist's ghosts) rounded up to 64
    uint32_t xk;   // workgroup chunk per XCD turn of the gather kernels (1 = hardware order)
    uint32_t open; // bit k: face k is an open reservoir (table entries kOpen + k mark
                   // every open face; the rule faces act as walls to the steps)
    uint32_t full; // every cell of the box is fluid (host-side launch choices only)
    uint32_t nx, ny, nz, nxy;  // the box (the direct-neighbour instances)
    uint32_t direct;           // every cell fluid and every axis periodic (host-side)
};

// Compact indices of the 18 neighbours x + c_d (kInvalid: solid, kWall: wall),
// used by the state transfers: one table read per direction.
__device__ __forceinline__ void neighbours(const CompactGeom& g, uint32_t p, uint32_t (&nb)[kQ])
{
#pragma unroll
    for (int d = 0; d < kQ; ++d) {
        if (d == 9) {
            nb[d] = kInvalid;
            continue;
        }
        const int32_t off = kCx[d] + (int32_t)g.px * kCy[d] + (int32_t)g.pxy * kCz[d];
        // 4 x (padded cells) < 2^32 is checked on the host: a 32-bit byte offset
        nb[d] = *(const uint32_t*)((const char*)g.idxp + (uint32_t)((int32_t)p + off) * 4u);
    }
}

// The same 18 indices for the step kernels, read row by row.  The D3Q19
// neighbours lie in nine x-rows of the padded table, (c_y, c_z) in {-1,0,1}^2;
// the own row and the four rows sharing one offset with it hold three
// neighbours each, at x - 1, x, x + 1, which are consecutive entries and
// come in one three-dword load (dword-aligned; legal for global memory on
// this target), and the four (c_y, c_z) diagonal rows hold one each.  Nine
// vector-memory instructions instead of eighteen: the address unit, not HBM,
// limits these kernels, and it is paid per instruction.
typedef uint32_t u32x3_a4 __attribute__((ext_vector_type(3), aligned(4)));

__device__ __forceinline__ void neighbours_rows(const CompactGeom& g, uint32_t p, uint32_t (&nb)[kQ])
{
    const char* t = (const char*)g.idxp;
    u32x3_a4 r[3][3];  // [c_z + 1][c_y + 1]: entries at x - 1, x, x + 1
    uint32_t diag[3][3];
#pragma unroll
    for (int cz = -1; cz <= 1; ++cz) {
#pragma unroll
        for (int cy = -1; cy <= 1; ++cy) {
            const uint32_t row = (uint32_t)((int32_t)p + (int32_t)g.px * cy + (int32_t)g.pxy * cz);
            if (cy != 0 && cz != 0) {
                diag[cz + 1][cy + 1] = *(const uint32_t*)(t + row * 4u);
            } else {
                r[cz + 1][cy + 1] = *(const u32x3_a4*)(t + (row - 1u) * 4u);
            }
        }
    }
#pragma unroll
    for (int d = 0; d < kQ; ++d) {
        if (d == 9) {
            nb[d] = kInvalid;
        } else if (kCy[d] != 0 && kCz[d] != 0) {
            nb[d] = diag[kCz[d] + 1][kCy[d] + 1];
        } else {
            const u32x3_a4& v = r[kCz[d] + 1][kCy[d] + 1];
            nb[d] = kCx[d] < 0 ? v.x : kCx[d] == 0 ? v.y : v.z;
        }
    }
}

// The same 18 indices on a box whose every cell is fluid and whose every axis
// is periodic: the compact index of a cell is then its cell index, and the
// neighbours follow from its coordinates with periodic wrap, with no table
// reads (the gather kernels' DIRECT instances).
__device__ __forceinline__ void neighbours_direct(const CompactGeom& g, uint32_t i, uint32_t (&nb)[kQ])
{
    const uint32_t nx = g.nx, ny = g.ny, nz = g.nz, nxy = g.nxy;
    const uint32_t z = i / nxy, r = i - z * nxy, y = r / nx, x = r - y * nx;
    const uint32_t X[3] = {x == 0 ? nx - 1 : x - 1, x, x + 1 == nx ? 0 : x + 1};
    const uint32_t Y[3] = {(y == 0 ? ny - 1 : y - 1) * nx, y * nx, (y + 1 == ny ? 0 : y + 1) * nx};
    const uint32_t Z[3] = {(z == 0 ? nz - 1 : z - 1) * nxy, z * nxy, (z + 1 == nz ? 0 : z + 1) * nxy};
#pragma unroll
    for (int d = 0; d < kQ; ++d) nb[d] = d == 9 ? kInvalid : X[kCx[d] + 1] + Y[kCy[d] + 1] + Z[kCz[d] + 1];
}

// Bit q of bm: link q is bounced back (x + c_q solid or beyond a wall); of
// wm: it leaves through a wall.  Taken right after the table reads, so the
// fused momentum exchange does not keep the 18 indices alive.
__device__ __forceinline__ void link_masks(const uint32_t (&nb)[kQ], uint32_t& bm, uint32_t& wm)
{
    bm = 0u;
    wm = 0u;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        if (q == 9) continue;
        bm |= (bounced(nb[q]) ? 1u : 0u) << q;
        wm |= (nb[q] == kWall ? 1u : 0u) << q;
    }
}

template <int q = 0, typename T>
__device__ __forceinline__ void add_links_mask(double (&acc)[6], const T (&s)[kQ], uint32_t bm, uint32_t wm)
{
    if constexpr (q < kQ) {
        if constexpr (q != 9) add_link<q>(acc, s[q], ((bm >> q) & 1u) != 0, ((wm >> q) & 1u) != 0);
        add_links_mask<q + 1>(acc, s, bm, wm);
    }
}

// Momentum exchange on the compact store: the index table marks wall links
// (kWall) apart from solid ones (kInvalid) and from open faces (kOpen + k,
// which carry no force).
template <int q = 0, typename T>
__device__ __forceinline__ void add_links_nb(double (&acc)[6], const T (&s)[kQ], const uint32_t (&nb)[kQ])
{
    if constexpr (q < kQ) {
        if constexpr (q != 9) add_link<q>(acc, s[q], bounced(nb[q]), nb[q] == kWall);
        add_links_nb<q + 1>(acc, s, nb);
    }
}

// Storage order of the populations: opposite directions side by side.  Pair
// k = 0..8 holds directions k and 18 - k in planes 2k and 2k + 1 (sub-planes
// 0 and 1); the rest population is plane 18.  Every access of a step kernel
// then lies in the two planes of its pair, so it is one uniform base (the
// pair's first plane, a scalar register) plus a byte offset per lane, and a
// bounce-back select only chooses between two offsets inside that pair.
constexpr int pair_of(int q) { return q < 9 ? q : q > 9 ? kQ - 1 - q : 9; }
constexpr int sub_of(int q) { return q > 9 ? 1 : 0; }
constexpr int plane_of(int q) { return 2 * pair_of(q) + sub_of(q); }

// Element (plane pl, compact index j) of the population store: blocks of 64
// cells, each holding its 19 planes side by side.  The esoteric pull's
// bounce-back region follows the 19 S elements of the blocks.  Offsets are 64
// bits wide (a store of more than 4 GB is addressed like a small one).
constexpr uint32_t kCBlock = 64;
typedef uint64_t coff_t;
__device__ __forceinline__ uint64_t celem(int pl, uint32_t j)
{
    return (uint64_t)(j >> 6) * (uint64_t)(kQ * kCBlock) + (uint64_t)pl * kCBlock + (j & (kCBlock - 1u));
}
// byte offset of cell j in plane 0, and the bytes from one plane to the next
template <typename T>
__device__ __forceinline__ coff_t cbytes(uint32_t j)
{
    return celem(0, j) * sizeof(T);
}
template <typename T>
__device__ __forceinline__ constexpr coff_t cplane()
{
    return kCBlock * sizeof(T);
}

// Esoteric pull on the compact store: pair k < 9 keeps its two slots in the
// planes of the other schemes, S0 = P(k) and S1 = P(18 - k), and the rest
// population is in plane P(9) = 18.  At a step of parity P the own side of
// pair k is (S_P, i), or (S0, i) if x - c_k is not fluid; the neighbour side
// is (S_{1-P}, nb[k]) for a fluid neighbour.  Solid cells and the halo have
// no storage here, so a neighbour-side bounce-back link keeps its value in a
// region after the blocks, at element 19 S + bbase[i] + (the cell's
// bounce-back links of the pairs before k): one slot per such link, packed in
// cell order, so that a wave's bounced links share one or two lines.
constexpr int kEsoPlanes = 28;     // 19 planes and up to 9 S bounce-back slots
constexpr int kEsoBouncePlane = 19;

// Bit k (k < 9): the neighbour side x + c_k of pair k is not fluid.
__device__ __forceinline__ uint32_t eso_bounce_mask(const uint32_t (&nb)[kQ])
{
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 9; ++k) m |= (no_fluid(nb[k]) ? 1u : 0u) << k;
    return m;
}

// Bounce-back slot of pair k of fluid cell i (relative to plane 19).
__device__ __forceinline__ uint32_t eso_bounce_slot(uint32_t base, uint32_t mask, int k)
{
    return base + (uint32_t)__popc(mask & ((1u << k) - 1u));
}

// Element offset (from the start of the buffer) of canonical f_q(x, t) of
// fluid cell i for stored state kind S (same maps as the dense layouts;
// x - c_q = x + c_opp(q)); used by the state transfers.
// Esoteric twist on the compact store (the map of the dense layouts, see
// twist_off): the fluid cells keep their indices 0 .. nf - 1; a location
// x - o (o one of the six offsets c+ of the directions with a positive
// component) that is not a fluid cell has a ghost cell of its own, numbered
// after the fluid cells in cell order (a solid cell behind a fluid one, or
// the halo below a low face that is not periodic).  tidx gives the stored
// index of every padded cell, the periodic image in a periodic halo.
// Every location x - o of a fluid cell is fluid or a ghost; the clamp keeps
// the index inside the buffer all the same (a table error then shows as a
// wrong value, not as an access beyond the allocation).
__device__ __forceinline__ uint32_t twist_ghost_index(const CompactGeom& g, uint32_t v)
{
    return min(v, g.s - 1u);
}

__device__ __forceinline__ uint32_t twist_compact_loc(const CompactGeom& g, uint32_t i, int ox, int oy, int oz)
{
    if (ox == 0 && oy == 0 && oz == 0) return i;
    const uint32_t off = (uint32_t)ox + (uint32_t)oy * g.px + (uint32_t)oz * g.pxy;
    return twist_ghost_index(g, g.tidx[g.cellp[i] - off]);
}

template <int S>
__device__ __forceinline__ uint64_t compact_state_off(const CompactGeom& g, uint32_t i, const uint32_t (&nb)[kQ],
                                                      int q)
{
    const uint64_t s = g.s;  // the bounce-back region follows 19 s elements
    const uint32_t up = nb[opp(q)];
    if constexpr (is_twist(S)) {
        const int pl = S == kTwOdd ? opp(q) : q;
        return celem(plane_of(pl), twist_compact_loc(g, i, kCx[q] > 0, kCy[q] > 0, kCz[q] > 0));
    } else if constexpr (is_eso(S)) {
        constexpr bool odd = S == kEsoOdd;
        if (q == 9) return celem(plane_of(9), i);
        if (q < 9) return celem(plane_of((no_fluid(up) || !odd) ? q : opp(q)), i);
        const int k = opp(q);  // neighbour side: x + c_k = x - c_q
        if (!no_fluid(up)) return celem(plane_of(odd ? k : q), up);
        return (uint64_t)kEsoBouncePlane * s + eso_bounce_slot(g.bbase[i], eso_bounce_mask(nb), k);
    } else if constexpr (S == kAB) {
        return no_fluid(up) ? celem(plane_of(opp(q)), i) : celem(plane_of(q), up);
    } else if constexpr (S == kAAEven) {
        return celem(plane_of(q), i);
    } else {
        return no_fluid(up) ? celem(plane_of(q), i) : celem(plane_of(opp(q)), up);
    }
}

template <int S, typename T>
__device__ __forceinline__ T* compact_state_slot(T* buf, const CompactGeom& g, uint32_t i, const uint32_t (&nb)[kQ],
                                                 int q)
{
    return buf + compact_state_off<S>(g, i, nb, q);
}

// Loads and stores of the compact step kernels.  Measured on MI355X, 256^3
// porous box:
//   - even step (purely local, every line read and rewritten once): nontemporal
//     loads and stores, 9% faster than plain ones (and the odd step after it
//     gains 4%, its lines no longer competing with the even step's);
//   - odd step (gathers and scatters, lines shared between neighbouring
//     workgroups): plain loads and stores; nontemporal stores cost 1%,
//     nontemporal loads 50%;
//   - fused pull: plain loads, nontemporal stores (the destination lattice is
//     not read in the same step), 3% faster than plain stores.
template <typename T>
__device__ __forceinline__ T ld_at(const char* blk, coff_t off)
{
    return *(const T*)(blk + off);
}

template <bool NT, typename T>
__device__ __forceinline__ void st_at(char* blk, coff_t off, T v)
{
    if constexpr (NT) {
        __builtin_nontemporal_store(v, (T*)(blk + off));
    } else {
        *(T*)(blk + off) = v;
    }
}

// Odd step: for each direction d whose neighbour entry is an open face, the
// value written to d's slot (the own slot (opp d, x)) is the reservoir's
// population entering along -c_d instead of f*_d.
template <int d = 0, typename T>
__device__ __forceinline__ void open_outflow(T (&f)[kQ], const uint32_t (&nb)[kQ], const Phys<T>& p)
{
    if constexpr (d < kQ) {
        if constexpr (d != 9) f[d] = is_res(nb[d], p.res) ? entering_value_nb<opp(d)>(p, nb[d]) : f[d];
        open_outflow<d + 1>(f, nb, p);
    }
}

// Byte offset, inside the block of pair(d), of the slot that direction d
// of fluid cell i owns in the in-place odd step and in the pull's gather:
// sub-plane `sv` at the neighbour's index `nbv` if that neighbour is fluid,
// else the own cell's slot in the other sub-plane (halfway bounce-back).
// Written as a select of two cheap values so it compiles to v_cndmask, not
// to a divergent branch.
template <typename T>
__device__ __forceinline__ coff_t link_off(uint32_t nbv, coff_t nb_sub_bytes, coff_t own_bytes)
{
    const coff_t via_nb = cbytes<T>(nbv) + nb_sub_bytes;
    return no_fluid(nbv) ? own_bytes : via_nb;
}

// Workgroup w runs on XCD w % 8 (the dispatcher deals workgroups out round
// robin).  The gather kernels renumber them in chunks of K consecutive
// workgroups: XCD x takes chunks x, x + 8, x + 16, ... so that a chunk's
// neighbour rows (y +- 1 within the chunk, z +- 1 one plane = 8 chunks
// later when K is an eighth of a plane's workgroups) are gathered through one
// L2, while all XCDs still sweep the lattice together.  K = 1 is the
// hardware order.  The grid is rounded up to 8 K workgroups; the extra ones
// find no cells and exit.


// planes 2k, 2k + 1 of pair k in the first block (a uniform 64-bit base; a
// cell's block comes with its per-lane offset)
__device__ __forceinline__ char* pair_block(char* base, int k, coff_t plane_bytes)
{
    return base + (uint64_t)(2 * k) * plane_bytes;
}

// Fields output of a compact step, written by waves in cell order.  The wave
// of fluid cells i0 .. i0 + 63 covers the cell range [r0, r1): r0 = its
// first cell (0 for the first wave), r1 = the next wave's first cell (N
// after the last fluid cell); the cells of the range that are not the
// wave's own are solid and get zeros.  The wave writes the range in chunks
// of 64 consecutive cells: each lane takes one cell and the values of a
// fluid one come from the lane that computed them (the k-th fluid cell of
// the range is the wave's k-th), so every store covers whole lines instead
// of scattering the fluid cells and patching the solid ones around them.
// fo: the lane's own density and velocity.  Called by every work-item of a
// wave with i0 < nf, blocks one-dimensional.
template <typename T>
__device__ __forceinline__ void write_fields_range(const MomOut<T>& mo, const uint32_t* __restrict__ cellid,
                                                   uint32_t nf, uint32_t i0, const T (&fo)[4])
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t r0 = i0 == 0 ? 0 : cellid[i0];
    const uint64_t r1 = i0 + 64u < nf ? cellid[i0 + 64u] : mo.n;
    uint32_t before = 0;  // the wave's fluid cells ahead of this chunk
    for (uint64_t c0 = r0; c0 < r1; c0 += 64) {
        const uint64_t c = c0 + lane;
        const bool in = c < r1;
        const bool fluid = in && (mo.mask == nullptr || mo.mask[c] == 0);
        const uint64_t bal = __ballot(fluid);
        const int src = (int)((before + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull))) & 63u);
        const T rho = __shfl(fo[0], src, 64), ux = __shfl(fo[1], src, 64);
        const T uy = __shfl(fo[2], src, 64), uz = __shfl(fo[3], src, 64);
        if (in) write_moments(mo, c, fluid ? rho : T(0), fluid ? ux : T(0), fluid ? uy : T(0), fluid ? uz : T(0));
        before += (uint32_t)__popcll(bal);
    }
}

// Gather step over the fluid cells, one work-item per fluid cell: the
// two-lattice fused pull (K = kAB, a = source, b = destination) or the odd
// step of the in-place pattern (K = kAAOdd, a = the lattice).  OPEN: some
// faces are open (a separate instance: the reservoir selects would cost the
// other cases registers).
template <typename T, int K, bool FORCE, bool OPEN, bool OUT, bool MEX, bool DIRECT>
__device__ __forceinline__ void step_compact_cell(T* __restrict__ a, T* __restrict__ b, const CompactGeom& g,
                                                  const Phys<T>& p, uint32_t i, double (&acc)[6], T (&fo)[4])
{
    const coff_t sb = cplane<T>();  // bytes from one plane of a block to the next
    const coff_t own0 = cbytes<T>(i);  // own slot in sub-plane 0 / 1 of a block
    const coff_t own1 = own0 + sb;
    char* const A = (char*)a;
    char* const B = (char*)b;
    uint32_t nb[kQ];
    if constexpr (DIRECT) {
        neighbours_direct(g, i, nb);
    } else {
        neighbours_rows(g, g.cellp[i], nb);
    }
    uint32_t bm = 0u, wm = 0u;
    if constexpr (MEX) link_masks(nb, bm, wm);
    T f[kQ];
    if constexpr (K == kAB) {
        // f_q = src[q][x - c_q], or src[opp q][x] if x - c_q is solid, or the
        // reservoir's value if x - c_q lies beyond an open face
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            const coff_t off = q == 9 ? own0
                                      : link_off<T>(nb[opp(q)], sub_of(q) ? sb : (coff_t)0, sub_of(opp(q)) ? own1 : own0);
            f[q] = ld_at<T>(pair_block(A, pair_of(q), sb), off);
        }
        if constexpr (OPEN) apply_open_nb(f, nb, p);
        T rho, ux, uy, uz;
        collide<T, FORCE>(f, p, rho, ux, uy, uz);
#pragma unroll
        for (int q = 0; q < kQ; ++q) st_at<true>(pair_block(B, pair_of(q), sb), sub_of(q) ? own1 : own0, f[q]);
        if constexpr (MEX) add_links_mask(acc, f, bm, wm);
        if constexpr (OUT) {
            fo[0] = rho;
            fo[1] = ux;
            fo[2] = uy;
            fo[3] = uz;
        }
    } else {
        // slot of direction d: (d, x + c_d), or (opp d, x) if x + c_d is solid.
        // The odd step reads f_{opp d} from it and writes f*_d into it.
        coff_t off[kQ];
#pragma unroll
        for (int d = 0; d < kQ; ++d)
            off[d] = d == 9 ? own0 : link_off<T>(nb[d], sub_of(d) ? sb : (coff_t)0, sub_of(opp(d)) ? own1 : own0);
#pragma unroll
        for (int q = 0; q < kQ; ++q) f[q] = ld_at<T>(pair_block(A, pair_of(q), sb), off[opp(q)]);
        if constexpr (OPEN) apply_open_nb(f, nb, p);
        T rho, ux, uy, uz;
        collide<T, FORCE>(f, p, rho, ux, uy, uz);
        if constexpr (OUT) {
            fo[0] = rho;
            fo[1] = ux;
            fo[2] = uy;
            fo[3] = uz;
        }
        // (with open faces f changes before the stores: sum the links first)
        if constexpr (MEX && OPEN) add_links_mask(acc, f, bm, wm);
        // beyond an open face, f*_d leaves the box and the own slot (opp d, x)
        // takes the reservoir's population entering along -c_d
        if constexpr (OPEN) open_outflow(f, nb, p);
#pragma unroll
        for (int q = 0; q < kQ; ++q) st_at<false>(pair_block(A, pair_of(q), sb), off[q], f[q]);
        if constexpr (MEX && !OPEN) add_links_mask(acc, f, bm, wm);
    }
}

// Gather step over the fluid cells, one work-item per fluid cell (see
// step_compact_cell).  MEX: also sum the momentum exchange of the step over
// the workgroup into mo.partial (row = the logical workgroup).  DIRECT: an
// all-fluid, fully periodic box (neighbours from coordinates).
template <typename T, int K, bool FORCE, bool OPEN, bool OUT, bool MEX = false, bool DIRECT = false>
__global__ void __launch_bounds__(kGatherThreads) step_compact_kernel(T* __restrict__ a, T* __restrict__ b,
                                                                     CompactGeom g, Phys<T> p, MomOut<T> mo)
{
    static_assert(K == kAB || K == kAAOdd, "the even step has its own kernel");
    const uint32_t wg = g.xk > 1 ? xcd_chunked(blockIdx.x, g.xk) : blockIdx.x;
    const uint32_t i = wg * kGatherThreads + threadIdx.x;
    double acc[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    T fo[4];  // the fields of the OUT instances
    if constexpr (OUT) {
        static_assert(!MEX, "no fields output in a momentum-exchange step");
        fo[0] = fo[1] = fo[2] = fo[3] = T(0);
        if (i < g.nf) step_compact_cell<T, K, FORCE, OPEN, true, false, DIRECT>(a, b, g, p, i, acc, fo);
        const uint32_t i0 = i - (threadIdx.x & 63u);
        if (i0 < g.nf) write_fields_range(mo, g.cellid, g.nf, i0, fo);
    } else if constexpr (!MEX) {
        if (i >= g.nf) return;
        step_compact_cell<T, K, FORCE, OPEN, OUT, false, DIRECT>(a, b, g, p, i, acc, fo);
    } else {
        if (i < g.nf) step_compact_cell<T, K, FORCE, OPEN, OUT, true, DIRECT>(a, b, g, p, i, acc, fo);
        if (wg < (g.nf + kGatherThreads - 1) / kGatherThreads)
            block_sum6<kGatherThreads>(acc, mo.partial + 6 * (size_t)wg);
    }
}

// Esoteric-pull step on the compact store (K = kEsoEven / kEsoOdd; the
// slot map is described at compact_state_off).  The own side of pair k and
// a fluid neighbour side lie in the pair's two planes of the blocks (a
// uniform base plus a per-lane byte offset, as in the other compact
// kernels); a bounced
// neighbour side goes to the packed bounce-back region instead.
template <typename T, int K, bool FORCE, bool OPEN, bool OUT, bool MEX, bool DIRECT>
__device__ __forceinline__ void eso_compact_cell(T* __restrict__ a, const CompactGeom& g, const Phys<T>& p,
                                                 uint32_t i, double (&acc)[6], T (&fo)[4])
{
    constexpr uint32_t P = K == kEsoOdd ? 1u : 0u;
    const coff_t sb = cplane<T>();
    const coff_t own = cbytes<T>(i);
    char* const A = (char*)a;
    uint32_t nb[kQ];
    if constexpr (DIRECT) {
        neighbours_direct(g, i, nb);
    } else {
        neighbours_rows(g, g.cellp[i], nb);
    }
    uint32_t bm = 0u, wm = 0u;
    if constexpr (MEX) link_masks(nb, bm, wm);
    const uint32_t bmask = eso_bounce_mask(nb);
    const uint32_t bbase = bmask != 0u ? g.bbase[i] : 0u;
    T* const B = a + (uint64_t)kEsoBouncePlane * g.s;  // after the blocks
    coff_t own_off[9];
    T* nb_ptr[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        own_off[k] = (P == 0u || no_fluid(nb[opp(k)])) ? own : own + sb;
        char* const blk = pair_block(A, k, sb);
        T* const via_nb = (T*)(blk + (1u - P) * sb + cbytes<T>(nb[k]));
        nb_ptr[k] = ((bmask >> k) & 1u) ? B + eso_bounce_slot(bbase, bmask, k) : via_nb;
    }
    char* const rest = pair_block(A, 9, sb);
    T f[kQ];
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        f[k] = ld_at<T>(pair_block(A, k, sb), own_off[k]);
        f[opp(k)] = *nb_ptr[k];
    }
    f[9] = ld_at<T>(rest, own);
    if constexpr (OPEN) apply_open_nb(f, nb, p);
    T rho, ux, uy, uz;
    collide<T, FORCE>(f, p, rho, ux, uy, uz);
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        *nb_ptr[k] = f[k];                                          // f*_k streams to x + c_k
        st_at<false>(pair_block(A, k, sb), own_off[k], f[opp(k)]);  // f*_opp(k) streams to x - c_k
    }
    st_at<false>(rest, own, f[9]);
    if constexpr (OUT) {
            fo[0] = rho;
            fo[1] = ux;
            fo[2] = uy;
            fo[3] = uz;
        }
    if constexpr (MEX) add_links_mask(acc, f, bm, wm);
}

template <typename T, int K, bool FORCE, bool OPEN, bool OUT, bool MEX = false, bool DIRECT = false>
__global__ void __launch_bounds__(kGatherThreads) eso_compact_kernel(T* __restrict__ a, CompactGeom g, Phys<T> p,
                                                                    MomOut<T> mo)
{
    static_assert(is_eso(K), "esoteric-pull step");
    const uint32_t wg = g.xk > 1 ? xcd_chunked(blockIdx.x, g.xk) : blockIdx.x;
    const uint32_t i = wg * kGatherThreads + threadIdx.x;
    double acc[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    T fo[4];  // the fields of the OUT instances
    if constexpr (OUT) {
        static_assert(!MEX, "no fields output in a momentum-exchange step");
        fo[0] = fo[1] = fo[2] = fo[3] = T(0);
        if (i < g.nf) eso_compact_cell<T, K, FORCE, OPEN, true, false, DIRECT>(a, g, p, i, acc, fo);
        const uint32_t i0 = i - (threadIdx.x & 63u);
        if (i0 < g.nf) write_fields_range(mo, g.cellid, g.nf, i0, fo);
    } else if constexpr (!MEX) {
        if (i >= g.nf) return;
        eso_compact_cell<T, K, FORCE, OPEN, OUT, false, DIRECT>(a, g, p, i, acc, fo);
    } else {
        if (i < g.nf) eso_compact_cell<T, K, FORCE, OPEN, OUT, true, DIRECT>(a, g, p, i, acc, fo);
        if (wg < (g.nf + kGatherThreads - 1) / kGatherThreads)
            block_sum6<kGatherThreads>(acc, mo.partial + 6 * (size_t)wg);
    }
}

// Esoteric-twist step on the compact store (K = kTwEven / kTwOdd; the map is
// described at twist_compact_loc and twist_off).  Every population of the
// pair (q, opp q) stays in the pair's two planes of the blocks: reads and
// both candidate writes are a uniform base plus a per-lane offset, and a bounced
// link only selects the other sub-plane at the same location.
template <typename T, int K, bool FORCE, bool OPEN, bool OUT, bool MEX, bool DIRECT>
__device__ __forceinline__ void twist_compact_cell(T* __restrict__ a, const CompactGeom& g, const Phys<T>& p,
                                                   uint32_t i, double (&acc)[6], T (&fo)[4])
{
    constexpr int P = K == kTwOdd ? 1 : 0;
    const coff_t sb = cplane<T>();
    char* const A = (char*)a;
    uint32_t nb[kQ];
    // stored indices of x - o, o = (ox, oy, oz) in {0, 1}^3, at [ox + 2 oy + 4 oz]
    uint32_t loc[7];
    loc[0] = i;
    if constexpr (DIRECT) {
        // no ghosts: x - o is the neighbour along -o, a direction of the stencil
        neighbours_direct(g, i, nb);
        loc[1] = nb[dir_of(-1, 0, 0)];
        loc[2] = nb[dir_of(0, -1, 0)];
        loc[3] = nb[dir_of(-1, -1, 0)];
        loc[4] = nb[dir_of(0, 0, -1)];
        loc[5] = nb[dir_of(-1, 0, -1)];
        loc[6] = nb[dir_of(0, -1, -1)];
    } else {
        const uint32_t pc = g.cellp[i];
        neighbours_rows(g, pc, nb);
        loc[1] = twist_ghost_index(g, g.tidx[pc - 1u]);
        loc[2] = twist_ghost_index(g, g.tidx[pc - g.px]);
        loc[3] = twist_ghost_index(g, g.tidx[pc - 1u - g.px]);
        loc[4] = twist_ghost_index(g, g.tidx[pc - g.pxy]);
        loc[5] = twist_ghost_index(g, g.tidx[pc - 1u - g.pxy]);
        loc[6] = twist_ghost_index(g, g.tidx[pc - g.px - g.pxy]);
    }
    uint32_t bm = 0u, wm = 0u;
    if constexpr (MEX) link_masks(nb, bm, wm);
    T f[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        const int o = (kCx[q] > 0 ? 1 : 0) + (kCy[q] > 0 ? 2 : 0) + (kCz[q] > 0 ? 4 : 0);
        const int pl = P == 0 ? q : opp(q);
        f[q] = ld_at<T>(pair_block(A, pair_of(q), sb), (sub_of(pl) ? sb : (coff_t)0) + cbytes<T>(loc[o]));
    }
    if constexpr (OPEN) apply_open_nb(f, nb, p);
    T rho, ux, uy, uz;
    collide<T, FORCE>(f, p, rho, ux, uy, uz);
    if constexpr (OUT) {
            fo[0] = rho;
            fo[1] = ux;
            fo[2] = uy;
            fo[3] = uz;
        }
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        // where f_opp(q) was read (x + c-_q, plane opp q at P = 0, q at P = 1),
        // or the other plane there if the link bounces back (x + c_q solid,
        // beyond a wall or a face with a face rule; a reservoir's link leaves)
        const int o = (kCx[q] < 0 ? 1 : 0) + (kCy[q] < 0 ? 2 : 0) + (kCz[q] < 0 ? 4 : 0);
        const bool back = no_fluid(nb[q]) && !is_res(nb[q], g.open);
        const int pn = P == 0 ? opp(q) : q, pb = P == 0 ? q : opp(q);
        const coff_t sub = back ? (sub_of(pb) ? sb : (coff_t)0) : (sub_of(pn) ? sb : (coff_t)0);
        st_at<false>(pair_block(A, pair_of(q), sb), sub + cbytes<T>(loc[o]), f[q]);
    }
    if constexpr (MEX) add_links_mask(acc, f, bm, wm);
}

template <typename T, int K, bool FORCE, bool OPEN, bool OUT, bool MEX = false, bool DIRECT = false>
__global__ void __launch_bounds__(kGatherThreads) twist_compact_kernel(T* __restrict__ a, CompactGeom g, Phys<T> p,
                                                                      MomOut<T> mo)
{
    static_assert(is_twist(K), "esoteric-twist step");
    const uint32_t wg = g.xk > 1 ? xcd_chunked(blockIdx.x, g.xk) : blockIdx.x;
    const uint32_t i = wg * kGatherThreads + threadIdx.x;
    double acc[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    T fo[4];  // the fields of the OUT instances
    if constexpr (OUT) {
        static_assert(!MEX, "no fields output in a momentum-exchange step");
        fo[0] = fo[1] = fo[2] = fo[3] = T(0);
        if (i < g.nf) twist_compact_cell<T, K, FORCE, OPEN, true, false, DIRECT>(a, g, p, i, acc, fo);
        const uint32_t i0 = i - (threadIdx.x & 63u);
        if (i0 < g.nf) write_fields_range(mo, g.cellid, g.nf, i0, fo);
    } else if constexpr (!MEX) {
        if (i >= g.nf) return;
        twist_compact_cell<T, K, FORCE, OPEN, OUT, false, DIRECT>(a, g, p, i, acc, fo);
    } else {
        if (i < g.nf) twist_compact_cell<T, K, FORCE, OPEN, OUT, true, DIRECT>(a, g, p, i, acc, fo);
        if (wg < (g.nf + kGatherThreads - 1) / kGatherThreads)
            block_sum6<kGatherThreads>(acc, mo.partial + 6 * (size_t)wg);
    }
}

// Even step of the in-place pattern: purely local, read (q, i), write
// (opp q, i).  The cells [nf, s) are padding: they are updated like the
// others but never read as state.  Wider accesses (2 or 4 cells per
// work-item, 8- or 16-byte vectors) measured no faster: this step moves
// every line once and runs at the HBM rate of the in-place pattern.
template <typename T, bool FORCE, bool OUT>
__global__ void __launch_bounds__(kEvenThreads) even_compact_kernel(T* __restrict__ a, uint32_t s, Phys<T> p,
                                                                    MomOut<T> mo, const uint32_t* __restrict__ cellid,
                                                                    uint32_t nf)
{
    const uint32_t i = blockIdx.x * kEvenThreads + threadIdx.x;
    if (i >= s) return;
    const coff_t sb = cplane<T>();
    const coff_t own0 = cbytes<T>(i);
    const coff_t own1 = own0 + sb;
    char* const A = (char*)a;
    T f[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q)
        f[q] = __builtin_nontemporal_load((const T*)(pair_block(A, pair_of(q), sb) + (sub_of(q) ? own1 : own0)));
    T rho, ux, uy, uz;
    collide<T, FORCE>(f, p, rho, ux, uy, uz);
#pragma unroll
    for (int q = 0; q < kQ; ++q) st_at<true>(pair_block(A, pair_of(q), sb), sub_of(opp(q)) ? own1 : own0, f[q]);
    if constexpr (OUT) {
        // s is a multiple of 64: the whole wave is still here
        const T fo[4] = {rho, ux, uy, uz};
        const uint32_t i0 = i - (threadIdx.x & 63u);
        if (i0 < nf) write_fields_range(mo, cellid, nf, i0, fo);
    }
}

// The even step with the momentum exchange of that step: the same purely
// local update (fluid cells only), plus the neighbour table to know which
// links are bounced back; the workgroup's sums go to mo.partial.
template <typename T, bool FORCE>
__global__ void __launch_bounds__(kEvenThreads) even_compact_mex_kernel(T* __restrict__ a, CompactGeom g,
                                                                        Phys<T> p, MomOut<T> mo)
{
    const uint32_t i = blockIdx.x * kEvenThreads + threadIdx.x;
    double acc[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    if (i < g.nf) {
        const coff_t sb = cplane<T>();
        const coff_t own0 = cbytes<T>(i);
        const coff_t own1 = own0 + sb;
        char* const A = (char*)a;
        uint32_t nb[kQ];
        neighbours_rows(g, g.cellp[i], nb);
        uint32_t bm, wm;
        link_masks(nb, bm, wm);
        T f[kQ];
#pragma unroll
        for (int q = 0; q < kQ; ++q)
            f[q] = __builtin_nontemporal_load((const T*)(pair_block(A, pair_of(q), sb) + (sub_of(q) ? own1 : own0)));
        collide<T, FORCE>(f, p);
#pragma unroll
        for (int q = 0; q < kQ; ++q) st_at<true>(pair_block(A, pair_of(q), sb), sub_of(opp(q)) ? own1 : own0, f[q]);
        add_links_mask(acc, f, bm, wm);
    }
    block_sum6<kEvenThreads>(acc, mo.partial + 6 * (size_t)blockIdx.x);
}

// rho and u := 0 on every cell: the fields of a step on a box without fluid
// cells (no step kernel runs there).
template <typename T>
__global__ void __launch_bounds__(kBlockThreads) zero_fields_kernel(MomOut<T> mo)
{
    const uint64_t id = (uint64_t)blockIdx.x * kBlockThreads + threadIdx.x;
    if (id < mo.n) write_moments(mo, id, T(0), T(0), T(0), T(0));
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
    T f[kQ];
    if constexpr (OP == kReadF || OP == kReadMoments || OP == kReadS) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) f[q] = *compact_state_slot<S>(a, cg, i, nb, q);
        if constexpr (S != kAAEven)
            if (cg.open) apply_open_nb(f, nb, p);
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
        // even state keeps them in their natural slots, the others have none
        if constexpr (S == kAAEven)
            if (cg.open) apply_open_nb(f, nb, p);
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            if (S != kAAEven && is_res(nb[opp(q)], p.res)) continue;
            *compact_state_slot<S>(a, cg, i, nb, q) = f[q];
        }
    }
}

}  // namespace lbm
