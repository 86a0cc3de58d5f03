// kernels_aos.hpp -- steps of the AoS (collision) layout staged through LDS:
// the odd in-place step on boxes with solid cells or walls, one plane tile at
// a time; the even in-place step, one run of consecutive records at a time;
// and the two-lattice pull, whose writes are staged the same way (the last
// two at the end of this file).
//
// In the AoS layout (PortLBM page, section 3.2, Fig. 2: the 19 populations of
// a cell side by side, a 76-byte record in fp32) the odd step of the in-place
// pattern makes cell x read and rewrite slot d of the record at x + c_d for
// every d (fieldcraft page "GPU lattice Boltzmann: streaming layout and
// performance", first section).  Straight from memory, one lane per cell, a
// wave touches one to three slots of each of 64 records in nine neighbour
// rows: every wave instruction spreads over ~38 cache lines for 256 useful
// bytes, and the step is bound by that L1/L2 traffic (the PortLBM page finds
// the collision layout L1-bound too, section 5.2, Table 2).
//
// Views.  The slots that the cells of plane z access are slot d of the
// record at x + c_d: the slots with c_z = -1 (directions 0..4 in the
// lexicographic (c_z, c_y, c_x) order) of records in plane z - 1, those with
// c_z = 0 (5..13) of records in plane z, and those with c_z = +1 (14..18) of
// records in plane z + 1, each at the xy positions of the cells and of the
// one-cell ring around them.  Call those 19 slots the view of an xy position
// at plane z.  Two planes' views never share a slot, so tiles of different
// planes are independent and there is no halo in z.
//
// A workgroup takes a tile of TX x TY cells of one plane: it loads the view
// of every position of the tile and its ring as three contiguous runs of
// its three records (20, 36 and 20 bytes in fp32) into LDS, every fluid cell
// gathers, collides and scatters in LDS, and the workgroup writes back the
// slots its own cells own (whole runs where it owns all of them).  Tiles are
// numbered z-fastest, so the tiles of planes z - 1, z, z + 1 over one xy
// range, which read and write the three runs of the same records, run
// together and meet in one L2.
//
// Ownership.  In the odd step every slot is read and rewritten by exactly one
// fluid cell: slot e of a fluid record R belongs to o = R - c_e if o is fluid
// (its link e is not bounced), else to R itself (its link opp(e) is bounced
// back into its own slot e).  Slots of solid records belong to nobody.  A
// workgroup writes a view slot back iff its owner is one of its cells:
//   - o = P - c_e (xy) in plane z is a fluid cell of the tile and R is a
//     fluid cell inside the box, or
//   - c_e has no z part, P is a cell of the tile, R = (P, z) is fluid and o is
//     not (solid, or beyond a wall): R's own bounce-back slot.
// A bounced link whose own slot lies in another plane's view (c_z != 0)
// reads and writes that one slot in memory directly; the view that holds it
// never writes it back (its o is solid).  The same record may appear twice in
// one tile's LDS (a row that wraps around inside the tile); the rule still
// gives each slot one writer, because a slot's owner determines the LDS copy
// it uses.  Loading a slot that another workgroup owns is harmless: its value
// is never used here, and it is never written back here.
#pragma once

#include "kernels.hpp"

namespace lbm {

template <typename T>
struct AosTile {
    static constexpr int TX = 64;                     // one wave per tile row
    static constexpr int TY = sizeof(T) == 4 ? 8 : 4;  // LDS: 52 KB fp32, 61 KB fp64
    static constexpr int PX = TX + 2;                 // positions per LDS row (ring included)
    static constexpr int NP = PX * (TY + 2);          // positions of tile and ring
    static constexpr int kThreads = TX * TY;
};

// n consecutive values at p (p aligned to sizeof(T)): 16-byte vector accesses,
// then the remainder
template <int N, typename T>
__device__ __forceinline__ void load_run(const T* p, T* v)
{
    constexpr int W = 16 / (int)sizeof(T);
    typedef T vec __attribute__((ext_vector_type(W), aligned(sizeof(T))));
#pragma unroll
    for (int i = 0; i + W <= N; i += W) {
        const vec x = *(const vec*)(p + i);
#pragma unroll
        for (int j = 0; j < W; ++j) v[i + j] = x[j];
    }
#pragma unroll
    for (int i = N / W * W; i < N; ++i) v[i] = p[i];
}

template <int N, typename T>
__device__ __forceinline__ void store_run(T* p, const T* v)
{
    constexpr int W = 16 / (int)sizeof(T);
    typedef T vec __attribute__((ext_vector_type(W), aligned(sizeof(T))));
#pragma unroll
    for (int i = 0; i + W <= N; i += W) {
        vec x;
#pragma unroll
        for (int j = 0; j < W; ++j) x[j] = v[i + j];
        *(vec*)(p + i) = x;
    }
#pragma unroll
    for (int i = N / W * W; i < N; ++i) p[i] = v[i];
}

// Run [E0, E0 + N) of a view: one vector run if this workgroup owns all of
// its slots, else the owned slots one by one.
template <int E0, int N, typename T>
__device__ __forceinline__ void store_owned(T* rec, const T (&v)[kQ], uint32_t own)
{
    constexpr uint32_t all = ((1u << N) - 1u) << E0;
    if ((own & all) == all) {
        store_run<N>(rec + E0, v + E0);
    } else {
#pragma unroll
        for (int e = E0; e < E0 + N; ++e)
            if ((own >> e) & 1u) rec[e] = v[e];
    }
}

struct TileFrame {
    uint32_t x0, y0, z, zm, zp;
    int nxt, nyt;  // cells of the tile along x, y (fewer at the box's far faces)
};

// Tile position P (ring included) -> its cell's wrapped (x, y); false if the
// position is unused (beyond a ragged tile's ring) or lies beyond a wall.
template <int PX>
__device__ __forceinline__ bool tile_pos(const Geom& g, const TileFrame& t, int P, int& lx, int& ly, uint32_t& x,
                                         uint32_t& y)
{
    lx = P % PX - 1;
    ly = P / PX - 1;
    if (lx > t.nxt || ly > t.nyt) return false;
    int gx = (int)t.x0 + lx, gy = (int)t.y0 + ly;
    if (gx < 0 || gx >= (int)g.nx) {
        if (!g.per_x) return false;
        gx = gx < 0 ? gx + (int)g.nx : gx - (int)g.nx;
    }
    if (gy < 0 || gy >= (int)g.ny) {
        if (!g.per_y) return false;
        gy = gy < 0 ? gy + (int)g.ny : gy - (int)g.ny;
    }
    x = (uint32_t)gx;
    y = (uint32_t)gy;
    return true;
}

// Odd in-place step of the AoS layout over one plane tile per workgroup, for
// boxes with a mask or a wall (without open faces or the fused momentum
// exchange, which take step_kernel).  OUT: also write the density and
// velocity (0 on solid cells).
template <typename T, bool FORCE, bool OUT>
__global__ void __launch_bounds__(AosTile<T>::kThreads) aos_odd_tile_kernel(T* __restrict__ a, Geom g, Phys<T> p,
                                                                           MomOut<T> mo)
{
    using Tl = AosTile<T>;
    constexpr int TX = Tl::TX, PX = Tl::PX, NP = Tl::NP, NT = Tl::kThreads;
    __shared__ T V[kQ][NP];
    // not-fluid flags (solid, beyond a wall, or an unused position) of the
    // records of planes z - 1, z, z + 1 at each position
    __shared__ uint8_t M[3][NP];

    const uint32_t tile = g.xk > 1 ? xcd_chunked(blockIdx.x, g.xk) : blockIdx.x;
    if (tile >= g.ntiles) return;  // whole workgroups only: before any barrier
    TileFrame t;
    {
        t.z = tile % g.nz;
        const uint32_t rest = tile / g.nz;
        t.x0 = (rest % g.ntx) * (uint32_t)TX;
        t.y0 = (rest / g.ntx) * (uint32_t)Tl::TY;
        t.zm = t.z == 0 ? g.nz - 1 : t.z - 1;
        t.zp = t.z + 1 == g.nz ? 0 : t.z + 1;
        t.nxt = min((int)(g.nx - t.x0), TX);
        t.nyt = min((int)(g.ny - t.y0), Tl::TY);
    }
    const uint64_t zm_off = (uint64_t)g.nxy * t.zm, z_off = (uint64_t)g.nxy * t.z, zp_off = (uint64_t)g.nxy * t.zp;

    // 1. views of the tile and its ring into LDS (a position beyond a wall
    //    or beyond the ring of a ragged tile is left alone: no cell reads it)
    for (int P = (int)threadIdx.x; P < NP; P += NT) {
        int lx, ly;
        uint32_t x, y;
        if (tile_pos<PX>(g, t, P, lx, ly, x, y)) {
            const uint64_t row = (uint64_t)x + (uint64_t)g.nx * y;
            T v[kQ];
            load_run<5>(a + (row + zm_off) * kQ, v);
            load_run<9>(a + (row + z_off) * kQ + 5, v + 5);
            load_run<5>(a + (row + zp_off) * kQ + 14, v + 14);
#pragma unroll
            for (int e = 0; e < kQ; ++e) V[e][P] = v[e];
            const bool m = g.mask != nullptr;
            M[0][P] = (!g.per_z && t.z == 0) || (m && g.mask[row + zm_off] != 0);
            M[1][P] = m && g.mask[row + z_off] != 0;
            M[2][P] = (!g.per_z && t.z + 1 == g.nz) || (m && g.mask[row + zp_off] != 0);
        } else {
            M[0][P] = M[1][P] = M[2][P] = 1;
        }
    }
    __syncthreads();

    // 2. one cell per work-item: gather, collide, scatter, all in LDS
    {
        const int lx = (int)threadIdx.x % TX, ly = (int)threadIdx.x / TX;
        const bool in_box = lx < t.nxt && ly < t.nyt;
        const int P0 = (ly + 1) * PX + lx + 1;
        const bool fluid = in_box && M[1][P0] == 0;
        const uint64_t cell = (uint64_t)(t.x0 + (uint32_t)lx) + (uint64_t)g.nx * (t.y0 + (uint32_t)ly) + z_off;
        if constexpr (OUT) {
            if (in_box && !fluid) write_moments(mo, cell, T(0), T(0), T(0), T(0));
        }
        if (fluid) {
            // bit d: x + c_d is solid or beyond a wall (link d bounced back)
            uint32_t bb = 0;
#pragma unroll
            for (int d = 0; d < kQ; ++d)
                if (d != 9) bb |= (uint32_t)(M[1 + kCz[d]][P0 + kCx[d] + kCy[d] * PX] != 0) << d;
            T* const rec = a + cell * kQ;
            T f[kQ];
            // f_opp(d) from slot (d, x + c_d), or from the own slot (opp d, x)
            // if bounced: in LDS for in-plane links, in memory for links with
            // a z part
#pragma unroll
            for (int d = 0; d < kQ; ++d) {
                if (d == 9) continue;
                const int e = opp(d);
                const int Pn = P0 + kCx[d] + kCy[d] * PX;
                const bool back = (bb >> d) & 1u;
                if (kCz[d] == 0) {
                    f[e] = back ? V[e][P0] : V[d][Pn];
                } else {
                    T v = V[d][Pn];
                    if (back) v = rec[e];
                    f[e] = v;
                }
            }
            f[9] = V[9][P0];
            T rho, ux, uy, uz;
            collide<T, FORCE>(f, p, rho, ux, uy, uz);
            if constexpr (OUT) write_moments(mo, cell, rho, ux, uy, uz);
            // f*_d into the same slot
#pragma unroll
            for (int d = 0; d < kQ; ++d) {
                if (d == 9) continue;
                const int e = opp(d);
                const int Pn = P0 + kCx[d] + kCy[d] * PX;
                const bool back = (bb >> d) & 1u;
                if (kCz[d] == 0) {
                    if (back) {
                        V[e][P0] = f[d];
                    } else {
                        V[d][Pn] = f[d];
                    }
                } else if (back) {
                    rec[e] = f[d];
                } else {
                    V[d][Pn] = f[d];
                }
            }
            V[9][P0] = f[9];
        }
    }
    __syncthreads();

    // 3. write back the owned slots of every view
    for (int P = (int)threadIdx.x; P < NP; P += NT) {
        int lx, ly;
        uint32_t x, y;
        if (!tile_pos<PX>(g, t, P, lx, ly, x, y)) continue;
        const bool tileP = lx >= 0 && lx < t.nxt && ly >= 0 && ly < t.nyt;
        uint32_t own = 0;
#pragma unroll
        for (int e = 0; e < kQ; ++e) {
            const int olx = lx - kCx[e], oly = ly - kCy[e];
            const bool otile = olx >= 0 && olx < t.nxt && oly >= 0 && oly < t.nyt;
            const bool rfluid = M[1 + kCz[e]][P] == 0;
            bool ofluid = false;
            if (otile || tileP) ofluid = M[1][P - kCx[e] - kCy[e] * PX] == 0;
            own |= (uint32_t)(rfluid && ((otile && ofluid) || (kCz[e] == 0 && tileP && !ofluid))) << e;
        }
        if (own == 0) continue;
        T v[kQ];
#pragma unroll
        for (int e = 0; e < kQ; ++e) v[e] = V[e][P];
        const uint64_t row = (uint64_t)x + (uint64_t)g.nx * y;
        store_owned<0, 5>(a + (row + zm_off) * kQ, v, own);
        store_owned<5, 9>(a + (row + z_off) * kQ, v, own);
        store_owned<14, 5>(a + (row + zp_off) * kQ, v, own);
    }
}

// Even in-place step of the AoS layout, staged through LDS.  The even step is
// purely local: a fluid cell reads slot q of its own record and writes f*_q
// to slot opp q of the same record.  One lane per cell straight from memory
// reads and writes 76-byte records at a 76-byte stride, so every wave
// instruction spreads over ~38 cache lines.  Here a workgroup takes the
// records of kCells consecutive cells, one contiguous run of memory (its
// start is 16-byte aligned: kCells * 19 * sizeof(T) is a multiple of 16),
// copies it into LDS with consecutive 16-byte accesses (8 lines per
// instruction), updates the fluid cells' records in LDS, and copies the run
// back.  A 16-byte piece that lies in solid records only is neither read nor
// written (nobody touches solid records in this step, and a porous medium's
// solid lines then stay out of the traffic).  NT: nontemporal accesses (for
// lattices beyond the last-level cache; a cache-resident lattice keeps its
// lines for the odd step that follows).  OUT: also the density and velocity
// (0 on solid cells).

template <typename T>
struct AosEven {
    static constexpr int kCells = 256;                // one per work-item
    static constexpr int kVec = 16 / (int)sizeof(T);  // elements per 16-byte access
    static constexpr int kElems = kCells * kQ;
    static constexpr int kChunks = kElems / kVec;
    static_assert(kElems % kVec == 0, "whole 16-byte accesses per workgroup");
};

template <typename T, bool NT, bool FORCE, bool OUT>
__global__ void __launch_bounds__(AosEven<T>::kCells) aos_even_staged_kernel(T* __restrict__ a, Geom g, Phys<T> p,
                                                                            MomOut<T> mo)
{
    using E = AosEven<T>;
    typedef T vec __attribute__((ext_vector_type(E::kVec)));
    __shared__ vec S[E::kChunks];
    __shared__ uint8_t solid[E::kCells];
    T* const R = (T*)S;
    const uint64_t c0 = (uint64_t)blockIdx.x * E::kCells;
    const uint32_t nc = (uint32_t)min((uint64_t)E::kCells, g.n - c0);  // cells of this workgroup
    const uint32_t ne = nc * (uint32_t)kQ, nch = ne / (uint32_t)E::kVec;
    const bool masked = g.mask != nullptr;
    if (masked) {
        if (threadIdx.x < nc) solid[threadIdx.x] = g.mask[c0 + threadIdx.x] != 0;
        __syncthreads();
    }
    // the elements e0 .. e1 of this workgroup's run (one or two records)
    // touch a fluid record
    const auto live = [&](uint32_t e0, uint32_t e1) {
        return !masked || !solid[e0 / kQ] || !solid[e1 / kQ];
    };
    T* const base = a + c0 * kQ;
    const vec* const src = (const vec*)base;
    for (uint32_t k = threadIdx.x; k < nch; k += E::kCells) {
        if (live(k * E::kVec, k * E::kVec + E::kVec - 1)) {
            if constexpr (NT) {
                S[k] = __builtin_nontemporal_load(src + k);
            } else {
                S[k] = src[k];
            }
        }
    }
    for (uint32_t e = nch * E::kVec + threadIdx.x; e < ne; e += E::kCells)
        if (live(e, e)) R[e] = base[e];
    __syncthreads();
    if (threadIdx.x < nc) {
        const uint64_t cell = c0 + threadIdx.x;
        T* const rec = R + threadIdx.x * kQ;
        if (!masked || !solid[threadIdx.x]) {
            T f[kQ];
#pragma unroll
            for (int q = 0; q < kQ; ++q) f[q] = rec[q];
            T rho, ux, uy, uz;
            collide<T, FORCE>(f, p, rho, ux, uy, uz);
            if constexpr (OUT) write_moments(mo, cell, rho, ux, uy, uz);
#pragma unroll
            for (int q = 0; q < kQ; ++q) rec[opp(q)] = f[q];
        } else if constexpr (OUT) {
            write_moments(mo, cell, T(0), T(0), T(0), T(0));
        }
    }
    __syncthreads();
    vec* const dst = (vec*)base;
    for (uint32_t k = threadIdx.x; k < nch; k += E::kCells) {
        if (live(k * E::kVec, k * E::kVec + E::kVec - 1)) {
            if constexpr (NT) {
                __builtin_nontemporal_store(S[k], dst + k);
            } else {
                dst[k] = S[k];
            }
        }
    }
    for (uint32_t e = nch * E::kVec + threadIdx.x; e < ne; e += E::kCells)
        if (live(e, e)) base[e] = R[e];
}

// Two-lattice pull of the AoS layout with its writes staged through LDS: a
// cell gathers f_q from slot q of the record at x - c_q of the source (or
// from its own opposite slot if that cell is solid or beyond a wall), as in
// step_kernel, and writes its 19 post-collision values into its own record of
// the destination.  The records of kCells consecutive cells are one
// contiguous run there, so the workgroup assembles them in LDS and writes
// the run with consecutive 16-byte accesses instead of 76-byte-strided ones.
// A solid cell's record gets 0, the value every solid record of a dense
// layout holds in the in-place and two-lattice schemes (the initialisation
// and the state transfers write it, no step changes it); a piece that lies
// in solid records only is not written at all.  BND: 1 if the box has a
// mask or a wall (no open faces here).  Workgroups are renumbered in XCD
// chunks (g.xk) so that the rows a chunk gathers from share an L2.
template <typename T, int BND, bool NT, bool FORCE, bool OUT>
__global__ void __launch_bounds__(AosEven<T>::kCells) aos_pull_staged_kernel(const T* __restrict__ a,
                                                                            T* __restrict__ b, Geom g, Phys<T> p,
                                                                            MomOut<T> mo)
{
    using E = AosEven<T>;
    typedef T vec __attribute__((ext_vector_type(E::kVec)));
    __shared__ vec S[E::kChunks];
    __shared__ uint8_t solid[E::kCells];
    T* const R = (T*)S;
    const uint32_t wg = g.xk > 1 ? xcd_chunked(blockIdx.x, g.xk) : blockIdx.x;
    const uint64_t c0 = (uint64_t)wg * E::kCells;
    if (c0 >= g.n) return;  // whole workgroups only: before any barrier
    const uint32_t nc = (uint32_t)min((uint64_t)E::kCells, g.n - c0);  // cells of this workgroup
    const uint32_t ne = nc * (uint32_t)kQ, nch = ne / (uint32_t)E::kVec;
    const bool masked = BND != 0 && g.mask != nullptr;
    if (threadIdx.x < nc) {
        Cell c;
        const uint32_t id = (uint32_t)(c0 + threadIdx.x);
        c.z = id / g.nxy;
        const uint32_t r = id - c.z * g.nxy;
        c.y = r / g.nx;
        c.x = r - c.y * g.nx;
        fill_cell(g, c);
        T* const rec = R + threadIdx.x * kQ;
        const bool is_solid = masked && g.mask[c.id] != 0;
        solid[threadIdx.x] = is_solid;
        if (!is_solid) {
            const uint32_t bits = link_bits<BND != 0>(g, c);
            T f[kQ];
#pragma unroll
            for (int q = 0; q < kQ; ++q) f[q] = ld_pop(state_slot<kAB, kCollision>(a, g, c, bits, q));
            T rho, ux, uy, uz;
            collide<T, FORCE>(f, p, rho, ux, uy, uz);
            if constexpr (OUT) write_moments(mo, c.id, rho, ux, uy, uz);
#pragma unroll
            for (int q = 0; q < kQ; ++q) rec[q] = f[q];
        } else {
            if constexpr (OUT) write_moments(mo, c.id, T(0), T(0), T(0), T(0));
#pragma unroll
            for (int q = 0; q < kQ; ++q) rec[q] = T(0);
        }
    }
    __syncthreads();
    // the elements e0 .. e1 of this workgroup's run touch a fluid record
    const auto live = [&](uint32_t e0, uint32_t e1) {
        return !masked || !solid[e0 / kQ] || !solid[e1 / kQ];
    };
    T* const base = b + c0 * kQ;
    vec* const dst = (vec*)base;
    for (uint32_t k = threadIdx.x; k < nch; k += E::kCells) {
        if (live(k * E::kVec, k * E::kVec + E::kVec - 1)) {
            if constexpr (NT) {
                __builtin_nontemporal_store(S[k], dst + k);
            } else {
                dst[k] = S[k];
            }
        }
    }
    for (uint32_t e = nch * E::kVec + threadIdx.x; e < ne; e += E::kCells)
        if (live(e, e)) base[e] = R[e];
}

}  // namespace lbm
