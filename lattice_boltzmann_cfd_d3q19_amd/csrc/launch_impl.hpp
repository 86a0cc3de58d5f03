// launch_impl.hpp -- launcher templates; instantiated once per precision.
#pragma once

#include <cmath>
#include <cstdlib>

#include "kernels.hpp"
#include "kernels_aos.hpp"
#include "kernels_compact.hpp"
#include "kernels_faces.hpp"
#include "kernels_force.hpp"
#include "launch.hpp"

namespace lbm {

struct Shape {
    dim3 grid, block;
    Geom g;
};

// Tile shape: BX = smallest power of two >= nx, clamped to [32, 256], so a
// wave64 covers one row segment (or two rows of 32); BY fills 256 threads.
inline Shape make_shape(const LaunchGeom& lg, bool xcd_chunks = false)
{
    Shape s{};
    uint32_t bx = 32;
    while (bx < 256 && (int64_t)bx < lg.nx) bx *= 2;
    const uint32_t by = (uint32_t)kBlockThreads / bx;
    Geom& g = s.g;
    g.nx = (uint32_t)lg.nx;
    g.ny = (uint32_t)lg.ny;
    g.nz = (uint32_t)lg.nz;
    g.nxy = g.nx * g.ny;
    g.per_x = lg.periodic[0] != 0;
    g.per_y = lg.periodic[1] != 0;
    g.per_z = lg.periodic[2] != 0;
    g.open = lg.res;
    g.fix = lg.open & ~lg.res;
    g.ntx = (g.nx + bx - 1) / bx;
    g.nty = (g.ny + by - 1) / by;
    g.ntiles = g.ntx * g.nty * g.nz;
    g.n = (uint64_t)lg.nx * (uint64_t)lg.ny * (uint64_t)lg.nz;
    g.mask = lg.mask;
    g.xk = 1;
    if (xcd_chunks && lg.xcd8) {
        // an eighth of a z-plane's tiles per chunk: the tiles of rows y +- 1
        // and of the planes z +- 1 then run on the same XCD
        g.xk = (g.ntx * g.nty + 7) / 8;
        if (g.xk < 1) g.xk = 1;
    }
    s.block = dim3(bx, by, 1);
    const uint32_t chunk = 8 * g.xk;
    s.grid = dim3(g.xk > 1 ? (g.ntiles + chunk - 1) / chunk * chunk : g.ntiles, 1, 1);
    return s;
}

// Resident workgroups per CU of the step kernels.  A step kernel's CU holds
// as many workgroups as registers allow (the compact gathers: four of 512
// work-items); together with the XCD-chunked order that puts about a dozen
// z-planes of an XCD's slab of the box in flight at once, more than its 4 MB
// L2 keeps, so the lines that neighbouring rows and planes share (read by
// one cell, written by another) are fetched and written back more than
// once.  Fewer resident workgroups narrow that front.  The cap is applied by
// reserving LDS the kernels do not use (160 KiB per CU on gfx950):
// floor(160 KiB / (w + 1/2)) bytes per workgroup leaves room for w of them.
// Targets per kernel class, measured on the 256^3 porous and periodic boxes
// (fp32, mean launch time, reserved LDS 0 / 27 / 33 / 41 / 54 / 82 KB):
//   compact odd in-place step: 2 (porous 0.389 -> 0.367 ms, periodic 0.494
//     -> 0.491); compact even step: 3 (0.270 -> 0.255, 0.450 -> 0.410);
//     compact esoteric twist: 2 (0.428 -> 0.408, 0.554 -> 0.550); compact
//     esoteric pull: no cap (no gain); re-measured with the blocked compact
//     store (porous, no cap / 2 / 3 / 4): odd 0.348 / 0.342 / 0.348 / 0.348,
//     even 0.264 / 0.247 / 0.242 / 0.253, pull 0.312 / 0.302 / 0.307 / 0.313
//     (the pull's target is 2 since);
//   even in-place steps of the dense layouts: SoA 2 without solids (0.438 ->
//     0.405), 3 with (0.555 -> 0.535); SoAoS 2 without (0.478 -> 0.432), 3
//     with (0.476 -> 0.456); AoS 3 without (0.554 -> 0.541), none with
//     (measured on step_kernel, which the AoS even step now takes only in a
//     fused momentum-exchange step: otherwise it is staged through LDS,
//     aos_even_staged_kernel, eight workgroups per CU);
//   the dense gathers of boxes with open faces: no cap (see below);
//   SoA odd step: 2 without solids (0.449 -> 0.418), 4 with (0.586 ->
//     0.574); SoA pull: 2 without (0.450 -> 0.420), 3 with (0.651 -> 0.566);
//   SoAoS pull with solids: 5 (0.519 -> 0.497); SoAoS odd step: no cap;
//   AoS odd step without solids: 2 (1.709 -> 1.044); AoS pull: 2 without
//     (0.929 -> 0.824), 3 with (0.743 -> 0.718) (step_kernel; the AoS pull
//     now runs with staged writes, aos_pull_staged_kernel, except on boxes
//     with open faces and in fused momentum-exchange steps); AoS odd step with solids:
//     no cap (1.18 -> 1.27 at 2; it now runs on the plane tiles, whose own
//     LDS leaves room for three workgroups per CU).
// The caps apply only to lattices larger than the 256 MB last-level cache:
// at 128^3 (159 MB, cache-resident) the kernels are latency-bound and lost
// up to 12% with them (Taylor-Green stream odd step 0.059 -> 0.066 ms),
// while every 256^3 and 512^3 box (fp32 and fp64) gained or tied (512^3
// porous: compact even 2.26 -> 2.14 ms, odd 3.24 -> 3.06, SoA pull 5.80 ->
// 4.61).
// An experiment build (LBM_LDS_FROM_ENV) takes the bytes from the
// environment instead (LBM_LDS for the gathers, LBM_LDS_EVEN for the even
// in-place steps), and scales the compact gathers' XCD chunk by
// LBM_XK_NUM / LBM_XK_DEN, to measure other settings without rebuilding.
// Measured with it on the 256^3 and 512^3 porous boxes: 256-work-item
// workgroups for the compact gathers (best 0.373 ms at four per CU) and
// chunks of 1/16, 1/4 or 1/2 plane were slower than 512 work-items, two per
// CU, an eighth of a plane per chunk (0.367 ms); chunked orders for the SoA
// and SoAoS layouts stayed slower under the caps too (256^3 porous SoA
// pull 0.567 -> 0.681 ms).
constexpr size_t kLdsPerCu = 160 * 1024;
constexpr uint64_t kLastLevelCache = 256ull << 20;

// a lattice of `cells` stored cells does not fit in the last-level cache
template <typename T>
constexpr bool beyond_llc(uint64_t cells)
{
    return cells * (uint64_t)kQ * sizeof(T) > kLastLevelCache;
}

constexpr size_t lds_for_workgroups(int w)
{
    return w <= 0 ? 0 : (size_t)(2 * kLdsPerCu / (size_t)(2 * w + 1));
}

// target for a dense step kernel of layout L, kind K, boundary instance bnd
// (0: no solids or walls); 0 = no cap
template <int L, int K>
constexpr int dense_step_workgroups(int bnd)
{
    // the open-face instance's gathers: no cap (768 x 192 x 96 open channel,
    // SoA pull 0.419 -> 0.481 ms at three workgroups per CU, 0.440 at four)
    if (bnd == 2 && K != kAAEven) return 0;
    if constexpr (K == kAAEven) {
        if constexpr (L == kCollision) return bnd == 0 ? 3 : 0;
        return bnd == 0 ? 2 : 3;
    } else if constexpr (K == kAAOdd) {
        if constexpr (L == kStream) return bnd == 0 ? 2 : 4;
        if constexpr (L == kCollision) return bnd == 0 ? 2 : 0;
        return 0;
    } else if constexpr (K == kAB) {
        if constexpr (L == kStream) return bnd == 0 ? 2 : 3;
        if constexpr (L == kCollision) return bnd == 0 ? 2 : 3;
        return bnd == 0 ? 0 : 5;
    } else {
        return 0;
    }
}

template <int K>
constexpr int compact_step_workgroups()
{
    return K == kAAOdd ? 2 : K == kAAEven ? 3 : K == kAB ? 2 : is_twist(K) ? 2 : 0;
}

#ifdef LBM_LDS_FROM_ENV
inline size_t lds_env(const char* name, size_t dflt)
{
    const char* v = getenv(name);
    return v ? (size_t)strtoul(v, nullptr, 10) : dflt;
}
#endif

// reserved LDS of a launch: even = an even in-place step (AA even or the
// esoteric schemes' even steps are gathers too; only the AA even step is
// purely local), w = the class's target
inline size_t step_lds(bool even, int w, bool big)
{
    const size_t dflt = big ? lds_for_workgroups(w) : 0;
#ifdef LBM_LDS_FROM_ENV
    return lds_env(even ? "LBM_LDS_EVEN" : "LBM_LDS", dflt);
#else
    (void)even;
    return dflt;
#endif
}

template <typename T>
inline Phys<T> make_phys(const LaunchPhys& lp)
{
    Phys<T> p{};
    p.omega = (T)lp.omega;
    p.fx = (T)lp.force[0];
    p.fy = (T)lp.force[1];
    p.fz = (T)lp.force[2];
    p.hfx = (T)(0.5 * lp.force[0]);
    p.hfy = (T)(0.5 * lp.force[1]);
    p.hfz = (T)(0.5 * lp.force[2]);
    const double guo = 1.0 - 0.5 * lp.omega;
    for (int q = 0; q < 9; ++q) {
        const double w = kW36[q] / 36.0;
        const double cF = kCx[q] * lp.force[0] + kCy[q] * lp.force[1] + kCz[q] * lp.force[2];
        p.gev[q] = (T)(9.0 * guo * w * cF);
        p.god[q] = (T)(3.0 * guo * w * cF);
    }
    p.gu[0] = (T)(3.0 * guo / 3.0);
    p.gu[1] = (T)(3.0 * guo / 18.0);
    p.gu[2] = (T)(3.0 * guo / 36.0);
    // open-face reservoirs: feq(rho_k, u_k) in double, minus the weight as
    // stored (rounded to T), then rounded once to T
    for (int k = 0; k < 6; ++k) {
        const double rho = lp.face_rho[k], *u = lp.face_u[k];
        const double usq = u[0] * u[0] + u[1] * u[1] + u[2] * u[2];
        for (int q = 0; q < kQ; ++q) {
            const double w = kW36[q] / 36.0;
            const double cu = kCx[q] * u[0] + kCy[q] * u[1] + kCz[q] * u[2];
            const double feq = w * rho * (1.0 + 3.0 * cu + 4.5 * cu * cu - 1.5 * usq);
            const T wt = kW36[q] == 12 ? T(1) / T(3) : kW36[q] == 2 ? T(1) / T(18) : T(1) / T(36);
            p.seq[k][q] = (T)(feq - (double)wt);
        }
    }
    p.res = lp.res;
    return p;
}

template <typename T, int L, int K, int BND, bool FORCE>
hipError_t launch_step_t(T* a, T* b, const Shape& s, const Phys<T>& p, const MomOut<T>& mo, hipStream_t st)
{
    Geom g = s.g;
    Phys<T> ph = p;
    MomOut<T> m = mo;
    void* args[] = {&a, &b, &g, &ph, &m};
    // hipLaunchKernel reports the status of this launch only (no stale errors)
    const void* k;
    if constexpr (BND != 0) {
        // the fused momentum exchange (no field output in the same step)
        if (mo.partial != nullptr) {
            if (mo.rho != nullptr) return hipErrorInvalidValue;
            return hipLaunchKernel((const void*)&step_kernel<T, L, K, BND, FORCE, false, true>, s.grid, s.block, args,
                                   0, st);
        }
    }
    k = mo.rho != nullptr ? (const void*)&step_kernel<T, L, K, BND, FORCE, true>
                          : (const void*)&step_kernel<T, L, K, BND, FORCE, false>;
    const size_t lds = step_lds(K == kAAEven, dense_step_workgroups<L, K>(BND), beyond_llc<T>(g.n));
    return hipLaunchKernel(k, s.grid, s.block, args, lds, st);
}

template <typename T, int L, int K>
hipError_t launch_step_k(T* a, T* b, const Shape& s, const Phys<T>& p, const MomOut<T>& mo, int bnd, bool force,
                         hipStream_t st)
{
    if (bnd == 2)
        return force ? launch_step_t<T, L, K, 2, true>(a, b, s, p, mo, st)
                     : launch_step_t<T, L, K, 2, false>(a, b, s, p, mo, st);
    if (bnd == 1)
        return force ? launch_step_t<T, L, K, 1, true>(a, b, s, p, mo, st)
                     : launch_step_t<T, L, K, 1, false>(a, b, s, p, mo, st);
    return force ? launch_step_t<T, L, K, 0, true>(a, b, s, p, mo, st)
                 : launch_step_t<T, L, K, 0, false>(a, b, s, p, mo, st);
}

template <typename T, int L>
hipError_t launch_step_l(int kind, T* a, T* b, const Shape& s, const Phys<T>& p, const MomOut<T>& mo, int bnd,
                         bool force, hipStream_t st)
{
    switch (kind) {
    case kAB: return launch_step_k<T, L, kAB>(a, b, s, p, mo, bnd, force, st);
    case kAAEven: return launch_step_k<T, L, kAAEven>(a, b, s, p, mo, bnd, force, st);
    case kAAOdd: return launch_step_k<T, L, kAAOdd>(a, b, s, p, mo, bnd, force, st);
    case kEsoEven: return launch_step_k<T, L, kEsoEven>(a, b, s, p, mo, bnd, force, st);
    case kEsoOdd: return launch_step_k<T, L, kEsoOdd>(a, b, s, p, mo, bnd, force, st);
    case kTwEven: return launch_step_k<T, L, kTwEven>(a, b, s, p, mo, bnd, force, st);
    case kTwOdd: return launch_step_k<T, L, kTwOdd>(a, b, s, p, mo, bnd, force, st);
    default: return hipErrorInvalidValue;
    }
}

inline int boundary_instance(const LaunchGeom& lg)
{
    return lg.res != 0 ? 2 : (lg.mask != nullptr || !lg.periodic[0] || !lg.periodic[1] || !lg.periodic[2]);
}

// The odd in-place step of the AoS layout on boxes with solid cells or walls:
// plane tiles staged through LDS (kernels_aos.hpp).  Boxes with open faces and
// the fused momentum exchange take step_kernel, and so do periodic boxes
// without a mask, where its row-bundled path is faster (256^3: 1.045 against
// 1.17 ms).  An experiment build can turn the tiles off (LBM_AOS_TILED=0).
#ifndef LBM_AOS_TILED
#define LBM_AOS_TILED 1
#endif
// XCD chunk: consecutive tiles (the planes of one xy range) on one XCD
#ifndef LBM_AOS_XK
#define LBM_AOS_XK 32
#endif

// Tiles of AosTile<T> cells, numbered z-, then x-, then y-fastest.
template <typename T>
inline Shape make_aos_tile_shape(const LaunchGeom& lg)
{
    using Tl = AosTile<T>;
    Shape s = make_shape(lg, false);
    Geom& g = s.g;
    g.ntx = (g.nx + Tl::TX - 1) / Tl::TX;
    g.nty = (g.ny + Tl::TY - 1) / Tl::TY;
    g.ntiles = g.ntx * g.nty * g.nz;
    g.xk = lg.xcd8 ? LBM_AOS_XK : 1;
    const uint32_t chunk = 8 * g.xk;
    s.block = dim3(Tl::kThreads, 1, 1);
    s.grid = dim3(g.xk > 1 ? (g.ntiles + chunk - 1) / chunk * chunk : g.ntiles, 1, 1);
    return s;
}

template <typename T, bool FORCE>
hipError_t launch_aos_odd_t(T* a, const Shape& s, const Phys<T>& p, const MomOut<T>& mo, hipStream_t st)
{
    Geom g = s.g;
    Phys<T> ph = p;
    MomOut<T> m = mo;
    void* args[] = {&a, &g, &ph, &m};
    const void* k = mo.rho != nullptr ? (const void*)&aos_odd_tile_kernel<T, FORCE, true>
                                      : (const void*)&aos_odd_tile_kernel<T, FORCE, false>;
    return hipLaunchKernel(k, s.grid, s.block, args, 0, st);
}

template <typename T>
hipError_t launch_aos_odd(T* a, const LaunchGeom& lg, const Phys<T>& p, const MomOut<T>& mo, bool force,
                          hipStream_t st)
{
    const Shape s = make_aos_tile_shape<T>(lg);
    return force ? launch_aos_odd_t<T, true>(a, s, p, mo, st) : launch_aos_odd_t<T, false>(a, s, p, mo, st);
}

// The even in-place step of the AoS layout staged through LDS
// (kernels_aos.hpp); the fused momentum exchange takes step_kernel.  An
// experiment build can turn it off (LBM_AOS_EVEN_STAGED=0).
#ifndef LBM_AOS_EVEN_STAGED
#define LBM_AOS_EVEN_STAGED 1
#endif

template <typename T>
hipError_t launch_aos_even(T* a, const LaunchGeom& lg, const Phys<T>& p, const MomOut<T>& mo, bool force,
                           hipStream_t st)
{
    using E = AosEven<T>;
    Geom g = make_shape(lg, false).g;
    Phys<T> ph = p;
    MomOut<T> m = mo;
    void* args[] = {&a, &g, &ph, &m};
    const bool out = mo.rho != nullptr;
    // nontemporal beyond the last-level cache (measured: 256^3 porous 0.327
    // -> 0.289 ms; a cache-resident 128^3 box keeps plain accesses, its odd
    // step then reads the even step's lines from the cache: 0.175 -> 0.158)
    const void* k;
    if (beyond_llc<T>(g.n)) {
        k = force ? (out ? (const void*)&aos_even_staged_kernel<T, true, true, true>
                         : (const void*)&aos_even_staged_kernel<T, true, true, false>)
                  : (out ? (const void*)&aos_even_staged_kernel<T, true, false, true>
                         : (const void*)&aos_even_staged_kernel<T, true, false, false>);
    } else {
        k = force ? (out ? (const void*)&aos_even_staged_kernel<T, false, true, true>
                         : (const void*)&aos_even_staged_kernel<T, false, true, false>)
                  : (out ? (const void*)&aos_even_staged_kernel<T, false, false, true>
                         : (const void*)&aos_even_staged_kernel<T, false, false, false>);
    }
    const dim3 grid((uint32_t)((g.n + E::kCells - 1) / E::kCells)), block(E::kCells);
    return hipLaunchKernel(k, grid, block, args, 0, st);
}

// The AoS two-lattice pull with its writes staged through LDS
// (kernels_aos.hpp); boxes with open faces and the fused momentum exchange
// take step_kernel.  An experiment build can turn it off
// (LBM_AOS_PULL_STAGED=0).
#ifndef LBM_AOS_PULL_STAGED
#define LBM_AOS_PULL_STAGED 1
#endif
#ifndef LBM_AOS_PULL_NT
#define LBM_AOS_PULL_NT 1
#endif

template <typename T, int BND, bool NT>
const void* aos_pull_kernel(bool force, bool out)
{
    return force ? (out ? (const void*)&aos_pull_staged_kernel<T, BND, NT, true, true>
                        : (const void*)&aos_pull_staged_kernel<T, BND, NT, true, false>)
                 : (out ? (const void*)&aos_pull_staged_kernel<T, BND, NT, false, true>
                        : (const void*)&aos_pull_staged_kernel<T, BND, NT, false, false>);
}

template <typename T>
hipError_t launch_aos_pull(const T* a, T* b, const LaunchGeom& lg, const Phys<T>& p, const MomOut<T>& mo,
                           int bnd, bool force, hipStream_t st)
{
    using E = AosEven<T>;
    Geom g = make_shape(lg, false).g;
    // an eighth of a z-plane's workgroups per XCD chunk, as for the tiles
    const uint64_t nwg = (g.n + E::kCells - 1) / E::kCells;
    const uint64_t wg_plane = ((uint64_t)g.nxy + E::kCells - 1) / E::kCells;
    g.xk = lg.xcd8 ? (uint32_t)((wg_plane + 7) / 8) : 1;
    if (g.xk < 1) g.xk = 1;
    const uint64_t chunk = 8ull * g.xk;
    const dim3 grid((uint32_t)(g.xk > 1 ? (nwg + chunk - 1) / chunk * chunk : nwg)), block(E::kCells);
    Phys<T> ph = p;
    MomOut<T> m = mo;
    void* args[] = {&a, &b, &g, &ph, &m};
    const bool out = mo.rho != nullptr, nt = LBM_AOS_PULL_NT && beyond_llc<T>(g.n);
    const void* k = bnd == 0 ? (nt ? aos_pull_kernel<T, 0, true>(force, out) : aos_pull_kernel<T, 0, false>(force, out))
                             : (nt ? aos_pull_kernel<T, 1, true>(force, out) : aos_pull_kernel<T, 1, false>(force, out));
    return hipLaunchKernel(k, grid, block, args, 0, st);
}

template <typename T>
hipError_t launch_step_mo(int layout, int kind, T* a, T* b, const LaunchGeom& lg, const LaunchPhys& lp,
                          const MomOut<T>& mo, hipStream_t st)
{
    // XCD-chunked tile order for the AoS layout only.  Measured, 256^3 porous
    // box, hardware order -> chunked: collision AA odd 2.06 -> 1.22 ms, AB
    // 0.92 -> 0.78 ms; stream AA +8% / +2% and AB +7%, bundle within 2%.
    const Shape s = make_shape(lg, layout == kCollision);
    const Phys<T> p = make_phys<T>(lp);
    const int bnd = boundary_instance(lg);
    if (LBM_AOS_EVEN_STAGED && layout == kCollision && kind == kAAEven && mo.partial == nullptr)
        return launch_aos_even<T>(a, lg, p, mo, lp.has_force, st);
    if (LBM_AOS_PULL_STAGED && layout == kCollision && kind == kAB && bnd != 2 && mo.partial == nullptr)
        return launch_aos_pull<T>(a, b, lg, p, mo, bnd, lp.has_force, st);
    if (LBM_AOS_TILED && layout == kCollision && kind == kAAOdd && bnd == 1 && mo.partial == nullptr)
        return launch_aos_odd<T>(a, lg, p, mo, lp.has_force, st);
    switch (layout) {
    case kStream: return launch_step_l<T, kStream>(kind, a, b, s, p, mo, bnd, lp.has_force, st);
    case kBundle: return launch_step_l<T, kBundle>(kind, a, b, s, p, mo, bnd, lp.has_force, st);
    case kCollision: return launch_step_l<T, kCollision>(kind, a, b, s, p, mo, bnd, lp.has_force, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_step(int layout, int kind, T* a, T* b, const LaunchGeom& lg, const LaunchPhys& lp, T* rho_out,
                       T* u_out, hipStream_t st)
{
    const MomOut<T> mo{rho_out, u_out, (uint64_t)lg.nx * (uint64_t)lg.ny * (uint64_t)lg.nz, nullptr, nullptr};
    return launch_step_mo<T>(layout, kind, a, b, lg, lp, mo, st);
}

template <typename T, int L, int S, int OP>
hipError_t launch_io_t(T* a, T* b, const Shape& s, const Phys<T>& p, T* o0, T* o1, const T* i0, const T* i1,
                       hipStream_t st)
{
    Geom g = s.g;
    Phys<T> ph = p;
    void* args[] = {&a, &b, &g, &ph, &o0, &o1, &i0, &i1};
    return hipLaunchKernel((const void*)&io_kernel<T, L, S, OP>, s.grid, s.block, args, 0, st);
}

template <typename T, int L, int S>
hipError_t launch_io_s(int op, T* a, T* b, const Shape& s, const Phys<T>& p, T* o0, T* o1, const T* i0,
                       const T* i1, hipStream_t st)
{
    switch (op) {
    case kReadF: return launch_io_t<T, L, S, kReadF>(a, b, s, p, o0, o1, i0, i1, st);
    case kReadMoments: return launch_io_t<T, L, S, kReadMoments>(a, b, s, p, o0, o1, i0, i1, st);
    case kWriteF: return launch_io_t<T, L, S, kWriteF>(a, b, s, p, o0, o1, i0, i1, st);
    case kWriteEq: return launch_io_t<T, L, S, kWriteEq>(a, b, s, p, o0, o1, i0, i1, st);
    case kReadS: return launch_io_t<T, L, S, kReadS>(a, b, s, p, o0, o1, i0, i1, st);
    case kWriteS: return launch_io_t<T, L, S, kWriteS>(a, b, s, p, o0, o1, i0, i1, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int L>
hipError_t launch_io_l(int state, int op, T* a, T* b, const Shape& s, const Phys<T>& p, T* o0, T* o1,
                       const T* i0, const T* i1, hipStream_t st)
{
    switch (state) {
    case kAB: return launch_io_s<T, L, kAB>(op, a, b, s, p, o0, o1, i0, i1, st);
    case kAAEven: return launch_io_s<T, L, kAAEven>(op, a, b, s, p, o0, o1, i0, i1, st);
    case kAAOdd: return launch_io_s<T, L, kAAOdd>(op, a, b, s, p, o0, o1, i0, i1, st);
    case kEsoEven: return launch_io_s<T, L, kEsoEven>(op, a, b, s, p, o0, o1, i0, i1, st);
    case kEsoOdd: return launch_io_s<T, L, kEsoOdd>(op, a, b, s, p, o0, o1, i0, i1, st);
    case kTwEven: return launch_io_s<T, L, kTwEven>(op, a, b, s, p, o0, o1, i0, i1, st);
    case kTwOdd: return launch_io_s<T, L, kTwOdd>(op, a, b, s, p, o0, o1, i0, i1, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_io(int layout, int state, int op, T* a, T* b, const LaunchGeom& lg, const LaunchPhys& lp,
                     T* o0, T* o1, const T* i0, const T* i1, hipStream_t st)
{
    const Shape s = make_shape(lg);
    const Phys<T> p = make_phys<T>(lp);
    switch (layout) {
    case kStream: return launch_io_l<T, kStream>(state, op, a, b, s, p, o0, o1, i0, i1, st);
    case kBundle: return launch_io_l<T, kBundle>(state, op, a, b, s, p, o0, o1, i0, i1, st);
    case kCollision: return launch_io_l<T, kCollision>(state, op, a, b, s, p, o0, o1, i0, i1, st);
    default: return hipErrorInvalidValue;
    }
}

// ------------------------------------------------------------ compact

// The gathers of an all-fluid, fully periodic box compute their neighbours
// from coordinates instead of reading the index tables (an experiment build
// can turn this off).
#ifndef LBM_COMPACT_DIRECT
#define LBM_COMPACT_DIRECT 1
#endif

inline CompactGeom compact_geom(const LaunchGeom& lg, const CompactTables& t)
{
    CompactGeom g{};
    g.idxp = t.idxp;
    g.cellp = t.cellp;
    g.cellid = t.cellid;
    g.bbase = t.bbase;
    g.tidx = t.tidx;
    g.nf = t.nf;
    g.px = (uint32_t)lg.nx + 2;
    g.pxy = (uint32_t)((lg.nx + 2) * (lg.ny + 2));
    g.s = (uint32_t)t.stride;
    g.open = lg.res;
    g.full = (uint64_t)t.nf == (uint64_t)lg.nx * (uint64_t)lg.ny * (uint64_t)lg.nz;
    g.nx = (uint32_t)lg.nx;
    g.ny = (uint32_t)lg.ny;
    g.nz = (uint32_t)lg.nz;
    g.nxy = (uint32_t)(lg.nx * lg.ny);
    // (open faces and face rules sit on non-periodic faces only: such a box has none)
    g.direct = LBM_COMPACT_DIRECT && g.full && lg.periodic[0] && lg.periodic[1] && lg.periodic[2];
    // XCD chunk of the gather kernels: an eighth of the workgroups of an
    // average z-plane, so the rows at z +- 1 fall on the same XCD as the
    // rows they are gathered by.  Measured (odd in-place step): 256^3 porous
    // 0.430 -> 0.382 ms, 512^3 porous 3.59 -> 3.20 ms, 128^3 sphere 0.066 ->
    // 0.064 ms, periodic 256^3 unchanged; fixed chunks of 4 to 80
    // workgroups were no better on any of them.
    const uint64_t wg_plane = ((uint64_t)t.nf / (uint64_t)lg.nz + kGatherThreads - 1) / kGatherThreads;
    g.xk = (uint32_t)((wg_plane + 7) / 8);
#ifdef LBM_LDS_FROM_ENV
    g.xk = (uint32_t)(g.xk * lds_env("LBM_XK_NUM", 8) / lds_env("LBM_XK_DEN", 8));
#endif
    if (g.xk < 1 || !lg.xcd8) g.xk = 1;
    return g;
}

template <typename T, int K, bool FORCE>
hipError_t launch_step_compact_t(T* a, T* b, CompactGeom g, Phys<T> p, MomOut<T> mo, hipStream_t st)
{
    if (g.nf == 0) return hipSuccess;
    void* args[] = {&a, &b, &g, &p, &mo};
    uint32_t nwg = (g.nf + kGatherThreads - 1) / kGatherThreads;
    if (g.xk > 1) nwg = (nwg + 8 * g.xk - 1) / (8 * g.xk) * (8 * g.xk);
    const dim3 grid(nwg), block(kGatherThreads);
    const bool out = mo.rho != nullptr;
    if (mo.partial != nullptr) {
        if (out) return hipErrorInvalidValue;
        const void* k = g.open ? (const void*)&step_compact_kernel<T, K, FORCE, true, false, true>
                               : (const void*)&step_compact_kernel<T, K, FORCE, false, false, true>;
        return hipLaunchKernel(k, grid, block, args, 0, st);
    }
    // an all-fluid, fully periodic box: neighbours from coordinates
    const void* k = g.open ? (out ? (const void*)&step_compact_kernel<T, K, FORCE, true, true>
                                  : (const void*)&step_compact_kernel<T, K, FORCE, true, false>)
                    : g.direct ? (out ? (const void*)&step_compact_kernel<T, K, FORCE, false, true, false, true>
                                    : (const void*)&step_compact_kernel<T, K, FORCE, false, false, false, true>)
                           : (out ? (const void*)&step_compact_kernel<T, K, FORCE, false, true>
                                  : (const void*)&step_compact_kernel<T, K, FORCE, false, false>);
    const size_t lds = step_lds(false, compact_step_workgroups<K>(), beyond_llc<T>(g.nf));
    return hipLaunchKernel(k, grid, block, args, lds, st);
}

template <typename T, bool FORCE>
hipError_t launch_even_compact_t(T* a, CompactGeom g, Phys<T> p, MomOut<T> mo, hipStream_t st)
{
    if (g.nf == 0) return hipSuccess;
    if (mo.partial != nullptr) {
        if (mo.rho != nullptr) return hipErrorInvalidValue;
        void* args[] = {&a, &g, &p, &mo};
        const dim3 grid((g.s + kEvenThreads - 1) / kEvenThreads), block(kEvenThreads);
        return hipLaunchKernel((const void*)&even_compact_mex_kernel<T, FORCE>, grid, block, args, 0, st);
    }
    uint32_t s = g.s, nf = g.nf;
    const uint32_t* cellid = g.cellid;
    void* args[] = {&a, &s, &p, &mo, &cellid, &nf};
    const dim3 grid((s + kEvenThreads - 1) / kEvenThreads), block(kEvenThreads);
    const void* k = mo.rho != nullptr ? (const void*)&even_compact_kernel<T, FORCE, true>
                                      : (const void*)&even_compact_kernel<T, FORCE, false>;
    // the even step's target: 3 with solid cells, 2 on an all-fluid box
    // (periodic 256^3: 0.428 -> 0.407 ms; the porous box keeps 3, 0.242
    // against 0.247 ms at 2)
    const size_t lds = step_lds(true, g.full ? 2 : compact_step_workgroups<kAAEven>(), beyond_llc<T>(g.nf));
    return hipLaunchKernel(k, grid, block, args, lds, st);
}

template <typename T, int K, bool FORCE>
hipError_t launch_eso_compact_t(T* a, CompactGeom g, Phys<T> p, MomOut<T> mo, hipStream_t st)
{
    if (g.nf == 0) return hipSuccess;
    void* args[] = {&a, &g, &p, &mo};
    uint32_t nwg = (g.nf + kGatherThreads - 1) / kGatherThreads;
    if (g.xk > 1) nwg = (nwg + 8 * g.xk - 1) / (8 * g.xk) * (8 * g.xk);
    const dim3 grid(nwg), block(kGatherThreads);
    const bool out = mo.rho != nullptr;
    if (mo.partial != nullptr) {
        if (out) return hipErrorInvalidValue;
        const void* k = g.open ? (const void*)&eso_compact_kernel<T, K, FORCE, true, false, true>
                               : (const void*)&eso_compact_kernel<T, K, FORCE, false, false, true>;
        return hipLaunchKernel(k, grid, block, args, 0, st);
    }
    const void* k = g.open ? (out ? (const void*)&eso_compact_kernel<T, K, FORCE, true, true>
                                  : (const void*)&eso_compact_kernel<T, K, FORCE, true, false>)
                    : g.direct ? (out ? (const void*)&eso_compact_kernel<T, K, FORCE, false, true, false, true>
                                      : (const void*)&eso_compact_kernel<T, K, FORCE, false, false, false, true>)
                           : (out ? (const void*)&eso_compact_kernel<T, K, FORCE, false, true>
                                  : (const void*)&eso_compact_kernel<T, K, FORCE, false, false>);
    const size_t lds = step_lds(false, compact_step_workgroups<K>(), beyond_llc<T>(g.nf));
    return hipLaunchKernel(k, grid, block, args, lds, st);
}

template <typename T, int K, bool FORCE>
hipError_t launch_twist_compact_t(T* a, CompactGeom g, Phys<T> p, MomOut<T> mo, hipStream_t st)
{
    if (g.nf == 0) return hipSuccess;
    void* args[] = {&a, &g, &p, &mo};
    uint32_t nwg = (g.nf + kGatherThreads - 1) / kGatherThreads;
    if (g.xk > 1) nwg = (nwg + 8 * g.xk - 1) / (8 * g.xk) * (8 * g.xk);
    const dim3 grid(nwg), block(kGatherThreads);
    const bool out = mo.rho != nullptr;
    if (mo.partial != nullptr) {
        if (out) return hipErrorInvalidValue;
        const void* k = g.open ? (const void*)&twist_compact_kernel<T, K, FORCE, true, false, true>
                               : (const void*)&twist_compact_kernel<T, K, FORCE, false, false, true>;
        return hipLaunchKernel(k, grid, block, args, 0, st);
    }
    const void* k = g.open ? (out ? (const void*)&twist_compact_kernel<T, K, FORCE, true, true>
                                  : (const void*)&twist_compact_kernel<T, K, FORCE, true, false>)
                    : g.direct ? (out ? (const void*)&twist_compact_kernel<T, K, FORCE, false, true, false, true>
                                      : (const void*)&twist_compact_kernel<T, K, FORCE, false, false, false, true>)
                           : (out ? (const void*)&twist_compact_kernel<T, K, FORCE, false, true>
                                  : (const void*)&twist_compact_kernel<T, K, FORCE, false, false>);
    const size_t lds = step_lds(false, compact_step_workgroups<K>(), beyond_llc<T>(g.nf));
    return hipLaunchKernel(k, grid, block, args, lds, st);
}

template <typename T, int K>
hipError_t launch_step_compact_k(T* a, T* b, CompactGeom g, Phys<T> p, MomOut<T> mo, bool force, hipStream_t st)
{
    if constexpr (is_eso(K)) {
        return force ? launch_eso_compact_t<T, K, true>(a, g, p, mo, st) : launch_eso_compact_t<T, K, false>(a, g, p, mo, st);
    } else if constexpr (is_twist(K)) {
        return force ? launch_twist_compact_t<T, K, true>(a, g, p, mo, st)
                     : launch_twist_compact_t<T, K, false>(a, g, p, mo, st);
    } else if constexpr (K == kAAEven) {
        return force ? launch_even_compact_t<T, true>(a, g, p, mo, st) : launch_even_compact_t<T, false>(a, g, p, mo, st);
    } else {
        return force ? launch_step_compact_t<T, K, true>(a, b, g, p, mo, st)
                     : launch_step_compact_t<T, K, false>(a, b, g, p, mo, st);
    }
}

template <typename T>
hipError_t launch_step_compact_mo(int kind, T* a, T* b, const LaunchGeom& lg, const CompactTables& t,
                                  const LaunchPhys& lp, const MomOut<T>& mo, hipStream_t st)
{
    const CompactGeom g = compact_geom(lg, t);
    const Phys<T> p = make_phys<T>(lp);
    MomOut<T> m = mo;
    if (m.rho != nullptr) {
        // the step's waves write the solid cells between their fluid cells;
        // a box without fluid cells runs no step, only this fill
        m.mask = lg.mask;
        if (g.nf == 0) {
            const uint64_t blocks = (m.n + kBlockThreads - 1) / kBlockThreads;
            void* args[] = {&m};
            return hipLaunchKernel((const void*)&zero_fields_kernel<T>, dim3((uint32_t)blocks), dim3(kBlockThreads),
                                   args, 0, st);
        }
    }
    switch (kind) {
    case kAB: return launch_step_compact_k<T, kAB>(a, b, g, p, m, lp.has_force, st);
    case kAAEven: return launch_step_compact_k<T, kAAEven>(a, b, g, p, m, lp.has_force, st);
    case kAAOdd: return launch_step_compact_k<T, kAAOdd>(a, b, g, p, m, lp.has_force, st);
    case kEsoEven: return launch_step_compact_k<T, kEsoEven>(a, b, g, p, m, lp.has_force, st);
    case kEsoOdd: return launch_step_compact_k<T, kEsoOdd>(a, b, g, p, m, lp.has_force, st);
    case kTwEven: return launch_step_compact_k<T, kTwEven>(a, b, g, p, m, lp.has_force, st);
    case kTwOdd: return launch_step_compact_k<T, kTwOdd>(a, b, g, p, m, lp.has_force, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_step_compact(int kind, T* a, T* b, const LaunchGeom& lg, const CompactTables& t,
                               const LaunchPhys& lp, T* rho_out, T* u_out, hipStream_t st)
{
    const MomOut<T> mo{rho_out, u_out, (uint64_t)lg.nx * (uint64_t)lg.ny * (uint64_t)lg.nz, nullptr, nullptr};
    return launch_step_compact_mo<T>(kind, a, b, lg, t, lp, mo, st);
}

template <typename T, int S, int OP>
hipError_t launch_io_compact_t(T* a, CompactGeom cg, const Shape& s, Phys<T> p, T* o0, T* o1, const T* i0,
                               const T* i1, hipStream_t st)
{
    Geom g = s.g;
    void* args[] = {&a, &cg, &g, &p, &o0, &o1, &i0, &i1};
    return hipLaunchKernel((const void*)&io_compact_kernel<T, S, OP>, s.grid, s.block, args, 0, st);
}

template <typename T, int S>
hipError_t launch_io_compact_s(int op, T* a, CompactGeom cg, const Shape& s, Phys<T> p, T* o0, T* o1,
                               const T* i0, const T* i1, hipStream_t st)
{
    switch (op) {
    case kReadF: return launch_io_compact_t<T, S, kReadF>(a, cg, s, p, o0, o1, i0, i1, st);
    case kReadMoments: return launch_io_compact_t<T, S, kReadMoments>(a, cg, s, p, o0, o1, i0, i1, st);
    case kWriteF: return launch_io_compact_t<T, S, kWriteF>(a, cg, s, p, o0, o1, i0, i1, st);
    case kWriteEq: return launch_io_compact_t<T, S, kWriteEq>(a, cg, s, p, o0, o1, i0, i1, st);
    case kReadS: return launch_io_compact_t<T, S, kReadS>(a, cg, s, p, o0, o1, i0, i1, st);
    case kWriteS: return launch_io_compact_t<T, S, kWriteS>(a, cg, s, p, o0, o1, i0, i1, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_io_compact(int state, int op, T* a, const LaunchGeom& lg, const CompactTables& t,
                             const LaunchPhys& lp, T* o0, T* o1, const T* i0, const T* i1, hipStream_t st)
{
    const Shape s = make_shape(lg);
    const CompactGeom cg = compact_geom(lg, t);
    const Phys<T> p = make_phys<T>(lp);
    switch (state) {
    case kAB: return launch_io_compact_s<T, kAB>(op, a, cg, s, p, o0, o1, i0, i1, st);
    case kAAEven: return launch_io_compact_s<T, kAAEven>(op, a, cg, s, p, o0, o1, i0, i1, st);
    case kAAOdd: return launch_io_compact_s<T, kAAOdd>(op, a, cg, s, p, o0, o1, i0, i1, st);
    case kEsoEven: return launch_io_compact_s<T, kEsoEven>(op, a, cg, s, p, o0, o1, i0, i1, st);
    case kEsoOdd: return launch_io_compact_s<T, kEsoOdd>(op, a, cg, s, p, o0, o1, i0, i1, st);
    case kTwEven: return launch_io_compact_s<T, kTwEven>(op, a, cg, s, p, o0, o1, i0, i1, st);
    case kTwOdd: return launch_io_compact_s<T, kTwOdd>(op, a, cg, s, p, o0, o1, i0, i1, st);
    default: return hipErrorInvalidValue;
    }
}

// ------------------------------------------------------------ face rules

template <typename T>
inline FaceRule<T> make_face_rule(const LaunchGeom& lg, const LaunchPhys& lp, const Phys<T>& p, int k)
{
    FaceRule<T> r{};
    const int ax = k / 2;
    const double sg = (k % 2 == 0) ? 1.0 : -1.0;
    const double rho = lp.face_rho[k], *u = lp.face_u[k];
    r.k = (uint32_t)k;
    r.kind = (uint32_t)lp.face_kind[k];
    r.nx = (uint32_t)lg.nx;
    r.ny = (uint32_t)lg.ny;
    r.nz = (uint32_t)lg.nz;
    r.n0 = ax == 0 ? r.ny : r.nx;
    r.ncell = ax == 0 ? r.ny * r.nz : ax == 1 ? r.nx * r.nz : r.nx * r.ny;
    r.drho = (T)(rho - 1.0);
    for (int t = 0; t < 3; ++t) {
        r.jt[t] = (T)(rho * u[t] - 0.5 * lp.force[t]);
        r.u[t] = (T)u[t];
    }
    r.ua_s = (T)(sg * u[ax]);
    r.inv_den = (T)(1.0 / (1.0 - sg * u[ax]));
    r.hfa_s = (T)(0.5 * sg * lp.force[ax]);
    for (int q = 0; q < kQ; ++q) r.seq[q] = p.seq[k][q];
    return r;
}

template <typename T, int L>
hipError_t launch_face_l(int state, T* a, const Geom& g, const Phys<T>& p, const FaceRule<T>& r, hipStream_t st)
{
    Geom gg = g;
    Phys<T> pp = p;
    FaceRule<T> rr = r;
    void* args[] = {&a, &gg, &pp, &rr};
    const dim3 grid((r.ncell + kBlockThreads - 1) / kBlockThreads), block(kBlockThreads);
    switch (state) {
    case kAB: return hipLaunchKernel((const void*)&face_kernel<T, L, kAB>, grid, block, args, 0, st);
    case kAAEven: return hipLaunchKernel((const void*)&face_kernel<T, L, kAAEven>, grid, block, args, 0, st);
    case kAAOdd: return hipLaunchKernel((const void*)&face_kernel<T, L, kAAOdd>, grid, block, args, 0, st);
    case kEsoEven: return hipLaunchKernel((const void*)&face_kernel<T, L, kEsoEven>, grid, block, args, 0, st);
    case kEsoOdd: return hipLaunchKernel((const void*)&face_kernel<T, L, kEsoOdd>, grid, block, args, 0, st);
    case kTwEven: return hipLaunchKernel((const void*)&face_kernel<T, L, kTwEven>, grid, block, args, 0, st);
    case kTwOdd: return hipLaunchKernel((const void*)&face_kernel<T, L, kTwOdd>, grid, block, args, 0, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_face_compact(int state, T* a, const CompactGeom& cg, const Phys<T>& p, const FaceRule<T>& r,
                               hipStream_t st)
{
    CompactGeom gg = cg;
    Phys<T> pp = p;
    FaceRule<T> rr = r;
    void* args[] = {&a, &gg, &pp, &rr};
    const dim3 grid((r.ncell + kBlockThreads - 1) / kBlockThreads), block(kBlockThreads);
    switch (state) {
    case kAB: return hipLaunchKernel((const void*)&face_compact_kernel<T, kAB>, grid, block, args, 0, st);
    case kAAEven: return hipLaunchKernel((const void*)&face_compact_kernel<T, kAAEven>, grid, block, args, 0, st);
    case kAAOdd: return hipLaunchKernel((const void*)&face_compact_kernel<T, kAAOdd>, grid, block, args, 0, st);
    case kEsoEven: return hipLaunchKernel((const void*)&face_compact_kernel<T, kEsoEven>, grid, block, args, 0, st);
    case kEsoOdd: return hipLaunchKernel((const void*)&face_compact_kernel<T, kEsoOdd>, grid, block, args, 0, st);
    case kTwEven: return hipLaunchKernel((const void*)&face_compact_kernel<T, kTwEven>, grid, block, args, 0, st);
    case kTwOdd: return hipLaunchKernel((const void*)&face_compact_kernel<T, kTwOdd>, grid, block, args, 0, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_face_rules(int layout, int state, T* a, const LaunchGeom& lg, const CompactTables* t,
                             const LaunchPhys& lp, hipStream_t st)
{
    const uint32_t rules = lg.open & ~lg.res;
    if (rules == 0) return hipSuccess;
    const Shape sh = make_shape(lg);
    const Phys<T> p = make_phys<T>(lp);
    for (int k = 0; k < 6; ++k) {
        if (!((rules >> k) & 1u)) continue;
        const FaceRule<T> r = make_face_rule<T>(lg, lp, p, k);
        if (r.ncell == 0) continue;
        hipError_t e;
        if (t != nullptr) {
            e = launch_face_compact<T>(state, a, compact_geom(lg, *t), p, r, st);
        } else {
            switch (layout) {
            case kStream: e = launch_face_l<T, kStream>(state, a, sh.g, p, r, st); break;
            case kBundle: e = launch_face_l<T, kBundle>(state, a, sh.g, p, r, st); break;
            case kCollision: e = launch_face_l<T, kCollision>(state, a, sh.g, p, r, st); break;
            default: return hipErrorInvalidValue;
            }
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ------------------------------------------------------ momentum exchange

// force[0..5] = the sum of partial rows 0 .. rows - 1 (zeros if rows = 0)
inline hipError_t launch_mex_sum(double* partial, uint32_t rows, double* force, hipStream_t st)
{
    const double* part = partial;
    void* args[] = {&part, &rows, &force};
    return hipLaunchKernel((const void*)&mex_sum_kernel, dim3(1), dim3(kBlockThreads), args, 0, st);
}

template <typename T, int L, int S>
hipError_t launch_mex_t(T* a, const Shape& sh, const Phys<T>& p, double* partial, hipStream_t st)
{
    Geom g = sh.g;
    Phys<T> ph = p;
    void* args[] = {&a, &g, &ph, &partial};
    return hipLaunchKernel((const void*)&mex_kernel<T, L, S>, sh.grid, sh.block, args, 0, st);
}

template <typename T, int S>
hipError_t launch_mex_compact_t(T* a, CompactGeom cg, const Phys<T>& p, double* partial, hipStream_t st)
{
    Phys<T> ph = p;
    void* args[] = {&a, &cg, &ph, &partial};
    const dim3 grid((cg.nf + kBlockThreads - 1) / kBlockThreads), block(kBlockThreads);
    return hipLaunchKernel((const void*)&mex_compact_kernel<T, S>, grid, block, args, 0, st);
}

template <typename T, int L>
hipError_t launch_mex_l(int state, T* a, const Shape& sh, const Phys<T>& p, double* partial, hipStream_t st)
{
    switch (state) {
    case kAB: return launch_mex_t<T, L, kAB>(a, sh, p, partial, st);
    case kAAEven: return launch_mex_t<T, L, kAAEven>(a, sh, p, partial, st);
    case kAAOdd: return launch_mex_t<T, L, kAAOdd>(a, sh, p, partial, st);
    case kEsoEven: return launch_mex_t<T, L, kEsoEven>(a, sh, p, partial, st);
    case kEsoOdd: return launch_mex_t<T, L, kEsoOdd>(a, sh, p, partial, st);
    case kTwEven: return launch_mex_t<T, L, kTwEven>(a, sh, p, partial, st);
    case kTwOdd: return launch_mex_t<T, L, kTwOdd>(a, sh, p, partial, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_momentum_exchange(int layout, int state, T* a, const LaunchGeom& lg, const CompactTables* t,
                                    const LaunchPhys& lp, double* partial, double* force, hipStream_t st)
{
    // partial rows: one per workgroup; fewer than mex_partial_rows() in the
    // compact case (fluid cells / 256 <= cells / 256 <= tiles)
    const Shape sh = make_shape(lg);
    const Phys<T> p = make_phys<T>(lp);
    hipError_t e = hipSuccess;
    uint32_t rows = sh.grid.x;
    if (t != nullptr) {
        const CompactGeom cg = compact_geom(lg, *t);
        rows = (cg.nf + kBlockThreads - 1) / kBlockThreads;
        if (rows > 0) {
            switch (state) {
            case kAB: e = launch_mex_compact_t<T, kAB>(a, cg, p, partial, st); break;
            case kAAEven: e = launch_mex_compact_t<T, kAAEven>(a, cg, p, partial, st); break;
            case kAAOdd: e = launch_mex_compact_t<T, kAAOdd>(a, cg, p, partial, st); break;
            case kEsoEven: e = launch_mex_compact_t<T, kEsoEven>(a, cg, p, partial, st); break;
            case kEsoOdd: e = launch_mex_compact_t<T, kEsoOdd>(a, cg, p, partial, st); break;
            case kTwEven: e = launch_mex_compact_t<T, kTwEven>(a, cg, p, partial, st); break;
            case kTwOdd: e = launch_mex_compact_t<T, kTwOdd>(a, cg, p, partial, st); break;
            default: return hipErrorInvalidValue;
            }
        }
    } else {
        switch (layout) {
        case kStream: e = launch_mex_l<T, kStream>(state, a, sh, p, partial, st); break;
        case kBundle: e = launch_mex_l<T, kBundle>(state, a, sh, p, partial, st); break;
        case kCollision: e = launch_mex_l<T, kCollision>(state, a, sh, p, partial, st); break;
        default: return hipErrorInvalidValue;
        }
    }
    if (e != hipSuccess) return e;
    return launch_mex_sum(partial, rows, force, st);
}

// Fused variant: the step's own gathers and collision give the exchanged
// momentum, so the separate pass (a second read of the lattice) is not needed.
// Partial rows: the dense tiles (the fully periodic box without mask has no
// bounce-back link and writes none), the compact step's workgroups (fewer:
// at least 256 work-items each).
static_assert(kGatherThreads >= kBlockThreads && kEvenThreads >= kBlockThreads,
              "the compact steps' partial rows must fit in the dense layouts' scratch");

template <typename T>
hipError_t launch_step_mex(int layout, int kind, T* a, T* b, const LaunchGeom& lg, const CompactTables* t,
                           const LaunchPhys& lp, double* partial, double* force, hipStream_t st)
{
    const MomOut<T> mo{nullptr, nullptr, (uint64_t)lg.nx * (uint64_t)lg.ny * (uint64_t)lg.nz, partial, nullptr};
    uint32_t rows;
    hipError_t e;
    if (t != nullptr) {
        const uint32_t nf = t->nf;
        const uint32_t s = (uint32_t)t->stride;
        rows = nf == 0 ? 0u
               : kind == kAAEven ? (s + kEvenThreads - 1) / kEvenThreads
                                 : (nf + kGatherThreads - 1) / kGatherThreads;
        e = launch_step_compact_mo<T>(kind, a, b, lg, *t, lp, mo, st);
    } else if (boundary_instance(lg) == 0) {
        rows = 0;
        e = launch_step<T>(layout, kind, a, b, lg, lp, nullptr, nullptr, st);
    } else {
        rows = make_shape(lg).g.ntiles;
        e = launch_step_mo<T>(layout, kind, a, b, lg, lp, mo, st);
    }
    if (e != hipSuccess) return e;
    return launch_mex_sum(partial, rows, force, st);
}

}  // namespace lbm
