// compact_build.hip -- device construction of the compact layout's tables
// (row counts, their exclusive scan, per-row compact indices, periodic halo).
#include "kernels_compact.hpp"
#include "launch.hpp"

namespace lbm {

// ------------------------------------------------------- table building

// Fluid cells per x-row; one workgroup per row r = y + ny z.
__global__ void __launch_bounds__(kBlockThreads) compact_count_rows(const uint8_t* __restrict__ mask, uint32_t nx,
                                                                    uint32_t* __restrict__ row_count)
{
    __shared__ uint32_t part[kBlockThreads / 64];
    const uint32_t r = blockIdx.x;
    uint32_t cnt = 0;
    for (uint32_t x = threadIdx.x; x < nx; x += kBlockThreads)
        cnt += (mask == nullptr || mask[(uint64_t)r * nx + x] == 0) ? 1u : 0u;
    // wave64 reduction, then across the four waves
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_down(cnt, o, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x / 64] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kBlockThreads / 64; ++w) t += part[w];
        row_count[r] = t;
    }
}

// Exclusive scan of the row counts in place (one workgroup of 1024), total in
// *total.  Each thread owns a contiguous chunk of rows.
__global__ void __launch_bounds__(1024) compact_scan_rows(uint32_t* __restrict__ rows, uint32_t nrows,
                                                          uint32_t* __restrict__ total)
{
    __shared__ uint32_t sums[1024];
    const uint32_t t = threadIdx.x;
    const uint32_t chunk = (nrows + 1023u) / 1024u;
    const uint32_t lo = min(nrows, t * chunk), hi = min(nrows, lo + chunk);
    uint32_t s = 0;
    for (uint32_t r = lo; r < hi; ++r) s += rows[r];
    sums[t] = s;
    __syncthreads();
    // Hillis-Steele inclusive scan over the 1024 chunk sums
    for (uint32_t o = 1; o < 1024; o <<= 1) {
        const uint32_t v = t >= o ? sums[t - o] : 0u;
        __syncthreads();
        sums[t] += v;
        __syncthreads();
    }
    uint32_t run = sums[t] - s;  // exclusive prefix of this chunk
    for (uint32_t r = lo; r < hi; ++r) {
        const uint32_t v = rows[r];
        rows[r] = run;
        run += v;
    }
    if (t == 1023) *total = sums[1023];
}

// Compact indices of the cells of row r (one workgroup per row), in x order.
__global__ void __launch_bounds__(kBlockThreads) compact_fill_rows(const uint8_t* __restrict__ mask, uint32_t nx,
                                                                   uint32_t ny, uint32_t px, uint32_t pxy,
                                                                   const uint32_t* __restrict__ row_start,
                                                                   uint32_t* __restrict__ idxp,
                                                                   uint32_t* __restrict__ cellp,
                                                                   uint32_t* __restrict__ cellid)
{
    __shared__ uint32_t wave_tot[kBlockThreads / 64];
    const uint32_t r = blockIdx.x;
    const uint32_t y = r % ny, z = r / ny;
    uint32_t base = row_start[r];
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x / 64;
    for (uint32_t x0 = 0; x0 < nx; x0 += kBlockThreads) {
        const uint32_t x = x0 + threadIdx.x;
        const bool inside = x < nx;
        const bool fluid = inside && (mask == nullptr || mask[(uint64_t)r * nx + x] == 0);
        const uint64_t bal = __ballot(fluid);
        const uint32_t below = __popcll(bal & ((1ull << lane) - 1ull));  // fluid lanes before this one
        if (lane == 0) wave_tot[wave] = __popcll(bal);
        __syncthreads();
        uint32_t before = 0, all = 0;
        for (uint32_t w = 0; w < kBlockThreads / 64; ++w) {
            before += w < wave ? wave_tot[w] : 0u;
            all += wave_tot[w];
        }
        if (inside) {
            const uint32_t p = (x + 1) + px * (y + 1) + pxy * (z + 1);
            if (fluid) {
                const uint32_t i = base + before + below;
                idxp[p] = i;
                cellp[i] = p;
                cellid[i] = r * nx + x;
            } else {
                idxp[p] = kInvalid;
            }
        }
        base += all;
        __syncthreads();
    }
}

// Halo of idxp: periodic image, kWall beyond a wall face, kOpen + k beyond open face k.
__global__ void __launch_bounds__(kBlockThreads) compact_fill_halo(uint32_t nx, uint32_t ny, uint32_t nz,
                                                                   uint32_t per_x, uint32_t per_y, uint32_t per_z,
                                                                   uint32_t open, uint32_t px, uint32_t pxy,
                                                                   uint64_t npad, uint32_t* __restrict__ idxp)
{
    const uint64_t p = (uint64_t)blockIdx.x * kBlockThreads + threadIdx.x;
    if (p >= npad) return;
    const uint32_t pp = (uint32_t)p;
    const int32_t gx = (int32_t)(pp % px) - 1;
    const int32_t gy = (int32_t)((pp / px) % (ny + 2)) - 1;
    const int32_t gz = (int32_t)(pp / pxy) - 1;
    const bool ox = gx < 0 || gx >= (int32_t)nx, oy = gy < 0 || gy >= (int32_t)ny, oz = gz < 0 || gz >= (int32_t)nz;
    if (!ox && !oy && !oz) return;  // interior: filled per row
    // beyond a non-periodic face: a wall wins over an open face; of two open
    // faces, the one on the first axis in x, y, z order
    const bool out[3] = {ox && !per_x, oy && !per_y, oz && !per_z};
    const int32_t gc[3] = {gx, gy, gz};
    bool wall = false;
    int face = -1;
    for (int a = 0; a < 3; ++a) {
        if (!out[a]) continue;
        const int k = 2 * a + (gc[a] < 0 ? 0 : 1);
        if ((open >> k) & 1u) {
            if (face < 0) face = k;
        } else {
            wall = true;
        }
    }
    if (wall || face >= 0) {
        idxp[pp] = wall ? kWall : kOpen + (uint32_t)face;
        return;
    }
    const uint32_t ix = (uint32_t)((gx + (int32_t)nx) % (int32_t)nx);
    const uint32_t iy = (uint32_t)((gy + (int32_t)ny) % (int32_t)ny);
    const uint32_t iz = (uint32_t)((gz + (int32_t)nz) % (int32_t)nz);
    idxp[pp] = idxp[(ix + 1) + px * (iy + 1) + pxy * (iz + 1)];
}


// Bounce-back links of each fluid cell on the neighbour side of the
// esoteric pull: x + c_k, k < 9, not fluid.
__global__ void __launch_bounds__(kBlockThreads) compact_bounce_counts(const uint32_t* __restrict__ idxp,
                                                                       const uint32_t* __restrict__ cellp,
                                                                       uint32_t nf, uint32_t px, uint32_t pxy,
                                                                       uint32_t* __restrict__ count)
{
    const uint32_t i = blockIdx.x * kBlockThreads + threadIdx.x;
    if (i >= nf) return;
    const uint32_t p = cellp[i];
    uint32_t n = 0;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const int32_t off = kCx[k] + (int32_t)px * kCy[k] + (int32_t)pxy * kCz[k];
        n += no_fluid(idxp[(uint32_t)((int32_t)p + off)]) ? 1u : 0u;
    }
    count[i] = n;
}

// ---------------------------------------------- esoteric-twist ghosts
//
// The twist reads and writes x - o for the six offsets o of the directions
// with a positive component (x, y, z, and the face diagonals xy, xz, yz).
// A padded cell that is not fluid gets storage ("ghost") if one of those
// offsets leads from it to a fluid cell; candidates are the interior cells
// and the halo below a low face that is not periodic (a periodic low halo is
// the image of a cell on the other side, which is a candidate itself).

// padded coordinate v of an axis with n cells is a candidate location
__device__ __forceinline__ bool twist_candidate(uint32_t v, uint32_t n, uint32_t per)
{
    return (v >= 1u && v <= n) || (v == 0u && per == 0u);
}

__device__ __forceinline__ bool twist_ghost(const uint32_t* __restrict__ idxp, uint32_t p, uint32_t px, uint32_t pxy)
{
    if (!no_fluid(idxp[p])) return false;
    const uint32_t offs[6] = {1u, px, pxy, 1u + px, 1u + pxy, px + pxy};
    bool g = false;
#pragma unroll
    for (int k = 0; k < 6; ++k) g = g || !no_fluid(idxp[p + offs[k]]);
    return g;
}

// Ghost cells per padded row r = py + (ny + 2) pz; one workgroup per row.
__global__ void __launch_bounds__(kBlockThreads) twist_count_rows(const uint32_t* __restrict__ idxp, uint32_t nx,
                                                                  uint32_t ny, uint32_t nz, uint32_t per_x,
                                                                  uint32_t per_y, uint32_t per_z,
                                                                  uint32_t* __restrict__ row_count)
{
    __shared__ uint32_t part[kBlockThreads / 64];
    const uint32_t r = blockIdx.x;
    const uint32_t py = r % (ny + 2u), pz = r / (ny + 2u);
    const uint32_t px = nx + 2u, pxy = px * (ny + 2u);
    const bool row_ok = twist_candidate(py, ny, per_y) && twist_candidate(pz, nz, per_z);
    uint32_t cnt = 0;
    if (row_ok)
        for (uint32_t x = threadIdx.x; x < px; x += kBlockThreads)
            cnt += (twist_candidate(x, nx, per_x) && twist_ghost(idxp, x + px * py + pxy * pz, px, pxy)) ? 1u : 0u;
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_down(cnt, o, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x / 64] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kBlockThreads / 64; ++w) t += part[w];
        row_count[r] = t;
    }
}

// tidx of every cell of padded row r: the fluid index, nf + the ghost's rank
// (in cell order), or kInvalid.  Periodic halos are filled afterwards.
__global__ void __launch_bounds__(kBlockThreads) twist_fill_rows(const uint32_t* __restrict__ idxp, uint32_t nx,
                                                                 uint32_t ny, uint32_t nz, uint32_t per_x,
                                                                 uint32_t per_y, uint32_t per_z, uint32_t nf,
                                                                 const uint32_t* __restrict__ row_start,
                                                                 uint32_t* __restrict__ tidx)
{
    __shared__ uint32_t wave_tot[kBlockThreads / 64];
    const uint32_t r = blockIdx.x;
    const uint32_t py = r % (ny + 2u), pz = r / (ny + 2u);
    const uint32_t px = nx + 2u, pxy = px * (ny + 2u);
    const bool row_ok = twist_candidate(py, ny, per_y) && twist_candidate(pz, nz, per_z);
    const bool row_in = py >= 1u && py <= ny && pz >= 1u && pz <= nz;
    uint32_t base = nf + row_start[r];
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x / 64;
    for (uint32_t x0 = 0; x0 < px; x0 += kBlockThreads) {
        const uint32_t x = x0 + threadIdx.x;
        const bool inside = x < px;
        const uint32_t p = x + px * py + pxy * pz;
        const bool ghost = inside && row_ok && twist_candidate(x, nx, per_x) && twist_ghost(idxp, p, px, pxy);
        const uint64_t bal = __ballot(ghost);
        const uint32_t below = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) wave_tot[wave] = __popcll(bal);
        __syncthreads();
        uint32_t before = 0, all = 0;
        for (uint32_t w = 0; w < kBlockThreads / 64; ++w) {
            before += w < wave ? wave_tot[w] : 0u;
            all += wave_tot[w];
        }
        if (inside) {
            const bool fluid = row_in && x >= 1u && x <= nx && !no_fluid(idxp[p]);
            tidx[p] = ghost ? base + before + below : fluid ? idxp[p] : kInvalid;
        }
        base += all;
        __syncthreads();
    }
}

// Periodic halos of tidx: the entry of the cell with every periodic halo
// coordinate wrapped (the others kept), which is never such a halo itself.
__global__ void __launch_bounds__(kBlockThreads) twist_fill_halo(uint32_t nx, uint32_t ny, uint32_t nz, uint32_t per_x,
                                                                 uint32_t per_y, uint32_t per_z, uint64_t npad,
                                                                 uint32_t* __restrict__ tidx)
{
    const uint64_t pp = (uint64_t)blockIdx.x * kBlockThreads + threadIdx.x;
    if (pp >= npad) return;
    const uint32_t px = nx + 2u, pxy = px * (ny + 2u);
    const uint32_t p = (uint32_t)pp;
    uint32_t x = p % px, y = (p / px) % (ny + 2u), z = p / pxy;
    const bool hx = per_x && (x == 0u || x == nx + 1u), hy = per_y && (y == 0u || y == ny + 1u),
               hz = per_z && (z == 0u || z == nz + 1u);
    if (!hx && !hy && !hz) return;
    if (hx) x = x == 0u ? nx : 1u;
    if (hy) y = y == 0u ? ny : 1u;
    if (hz) z = z == 0u ? nz : 1u;
    tidx[p] = tidx[x + px * y + pxy * z];
}

CompactLayoutBytes compact_workspace_layout(int64_t nx, int64_t ny, int64_t nz, bool bounce, bool twist)
{
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    CompactLayoutBytes b{};
    const size_t nrows = (size_t)ny * (size_t)nz;
    const size_t npad = (size_t)(nx + 2) * (size_t)(ny + 2) * (size_t)(nz + 2);
    const size_t n64 = ((size_t)nx * (size_t)ny * (size_t)nz + 63) / 64 * 64;
    b.header = 0;
    b.rows = 256;
    b.idxp = b.rows + up(4 * nrows);
    b.cellp = b.idxp + up(4 * npad);
    b.cellid = b.cellp + up(4 * n64);
    b.bbase = b.cellid + up(4 * n64);
    b.tidx = b.bbase + (bounce ? up(4 * n64) : 0);
    b.grows = b.tidx + (twist ? up(4 * npad) : 0);
    b.total = b.grows + (twist ? up(4 * (size_t)(ny + 2) * (size_t)(nz + 2)) : 0);
    return b;
}

hipError_t launch_compact_build(const LaunchGeom& lg, const CompactTables& t, hipStream_t st)
{
    const uint32_t nx = (uint32_t)lg.nx, ny = (uint32_t)lg.ny, nz = (uint32_t)lg.nz;
    const uint32_t nrows = ny * nz;
    const uint32_t px = nx + 2, pxy = (nx + 2) * (ny + 2);
    const uint64_t npad = (uint64_t)pxy * (nz + 2);
    hipLaunchKernelGGL(compact_count_rows, dim3(nrows), dim3(kBlockThreads), 0, st, lg.mask, nx, t.rows);
    hipLaunchKernelGGL(compact_scan_rows, dim3(1), dim3(1024), 0, st, t.rows, nrows, t.header);
    hipLaunchKernelGGL(compact_fill_rows, dim3(nrows), dim3(kBlockThreads), 0, st, lg.mask, nx, ny, px, pxy,
                       (const uint32_t*)t.rows, t.idxp, t.cellp, t.cellid);
    hipLaunchKernelGGL(compact_fill_halo, dim3((uint32_t)((npad + kBlockThreads - 1) / kBlockThreads)),
                       dim3(kBlockThreads), 0, st, nx, ny, nz, (uint32_t)(lg.periodic[0] != 0),
                       (uint32_t)(lg.periodic[1] != 0), (uint32_t)(lg.periodic[2] != 0), lg.open, px, pxy, npad,
                       t.idxp);
    return hipGetLastError();
}

hipError_t launch_compact_twist(const LaunchGeom& lg, const CompactTables& t, hipStream_t st)
{
    if (t.tidx == nullptr) return hipSuccess;
    const uint32_t nx = (uint32_t)lg.nx, ny = (uint32_t)lg.ny, nz = (uint32_t)lg.nz;
    const uint32_t prow = (ny + 2) * (nz + 2);
    const uint64_t npad = (uint64_t)(nx + 2) * (ny + 2) * (nz + 2);
    const uint32_t per_x = lg.periodic[0] != 0, per_y = lg.periodic[1] != 0, per_z = lg.periodic[2] != 0;
    hipLaunchKernelGGL(twist_count_rows, dim3(prow), dim3(kBlockThreads), 0, st, (const uint32_t*)t.idxp, nx, ny, nz,
                       per_x, per_y, per_z, t.grows);
    // ghost count into header[2]
    hipLaunchKernelGGL(compact_scan_rows, dim3(1), dim3(1024), 0, st, t.grows, prow, t.header + 2);
    hipLaunchKernelGGL(twist_fill_rows, dim3(prow), dim3(kBlockThreads), 0, st, (const uint32_t*)t.idxp, nx, ny, nz,
                       per_x, per_y, per_z, t.nf, (const uint32_t*)t.grows, t.tidx);
    hipLaunchKernelGGL(twist_fill_halo, dim3((uint32_t)((npad + kBlockThreads - 1) / kBlockThreads)),
                       dim3(kBlockThreads), 0, st, nx, ny, nz, per_x, per_y, per_z, npad, t.tidx);
    return hipGetLastError();
}

hipError_t launch_compact_bounce(const LaunchGeom& lg, const CompactTables& t, hipStream_t st)
{
    if (t.bbase == nullptr || t.nf == 0) return hipSuccess;
    const uint32_t px = (uint32_t)lg.nx + 2, pxy = (uint32_t)((lg.nx + 2) * (lg.ny + 2));
    hipLaunchKernelGGL(compact_bounce_counts, dim3((t.nf + kBlockThreads - 1) / kBlockThreads), dim3(kBlockThreads),
                       0, st, (const uint32_t*)t.idxp, (const uint32_t*)t.cellp, t.nf, px, pxy, t.bbase);
    // total bounce-back links into header[1]
    hipLaunchKernelGGL(compact_scan_rows, dim3(1), dim3(1024), 0, st, t.bbase, t.nf, t.header + 1);
    return hipGetLastError();
}

}  // namespace lbm
