// d3q19.hpp -- D3Q19 lattice constants for the gfx950 kernels.
//
// Velocity set inside {-1,0,1}^3 with |c|^2 <= 2 and weights 1/3 (rest),
// 1/18 (axis), 1/36 (diagonal): codechina page "GPU加速LBM流体仿真",
// sections 2.1-2.2.  Direction order: lexicographic over (c_z, c_y, c_x)
// (the PortLBM page's 2-D raster of Fig. 2 extended to 3-D), so q = 9 is rest
// and opposite(q) = 18 - q.
//
// Bundles for the SoAoS layout (PortLBM page, section 3.2, Fig. 2c: one
// bundle per stencil row): directions with equal (c_y, c_z).  In this order
// they are the contiguous runs {0} {1,2,3} {4} {5,6,7} {8,9,10} {11,12,13}
// {14} {15,16,17} {18}.
#pragma once

namespace lbm {

constexpr int kQ = 19;

constexpr int kCx[kQ] = {0, -1, 0, 1, 0, -1, 0, 1, -1, 0, 1, -1, 0, 1, 0, -1, 0, 1, 0};
constexpr int kCy[kQ] = {-1, 0, 0, 0, 1, -1, -1, -1, 0, 0, 0, 1, 1, 1, -1, 0, 0, 0, 1};
constexpr int kCz[kQ] = {-1, -1, -1, -1, -1, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 1, 1, 1, 1};

constexpr int opp(int q) { return kQ - 1 - q; }

// the direction with velocity (cx, cy, cz); -1 if it is not in the set
constexpr int dir_of(int cx, int cy, int cz)
{
    for (int q = 0; q < kQ; ++q)
        if (kCx[q] == cx && kCy[q] == cy && kCz[q] == cz) return q;
    return -1;
}

// |c|^2 class -> weight numerator over 36.
constexpr int kW36[kQ] = {1, 1, 2, 1, 1, 1, 2, 1, 2, 12, 2, 1, 2, 1, 1, 1, 2, 1, 1};

// Bundle of each direction, the bundle's first direction and its size.
constexpr int kBundleFirst[kQ] = {0, 1, 1, 1, 4, 5, 5, 5, 8, 8, 8, 11, 11, 11, 14, 15, 15, 15, 18};
constexpr int kBundleSize[kQ] = {1, 3, 3, 3, 1, 3, 3, 3, 3, 3, 3, 3, 3, 3, 1, 3, 3, 3, 1};

constexpr int sq(int v) { return v * v; }

constexpr bool table_is_consistent()
{
    for (int q = 0; q < kQ; ++q) {
        if (kCx[opp(q)] != -kCx[q] || kCy[opp(q)] != -kCy[q] || kCz[opp(q)] != -kCz[q]) return false;
        int n2 = sq(kCx[q]) + sq(kCy[q]) + sq(kCz[q]);
        int w = n2 == 0 ? 12 : n2 == 1 ? 2 : 1;
        if (kW36[q] != w) return false;
        int b = kBundleFirst[q];
        if (kCy[b] != kCy[q] || kCz[b] != kCz[q] || q - b >= kBundleSize[q]) return false;
        if (q > 0) {
            int prev = (kCz[q - 1] + 1) * 9 + (kCy[q - 1] + 1) * 3 + (kCx[q - 1] + 1);
            int cur = (kCz[q] + 1) * 9 + (kCy[q] + 1) * 3 + (kCx[q] + 1);
            if (cur <= prev) return false;
        }
    }
    return true;
}
static_assert(table_is_consistent(), "D3Q19 table inconsistent");
static_assert(dir_of(0, 0, 0) == 9 && dir_of(-1, 0, -1) == 1 && dir_of(0, -1, -1) == 0 && dir_of(1, 1, 1) == -1,
              "dir_of");

enum Layout : int { kStream = 0, kBundle = 1, kCollision = 2 };
// What a kernel does with the stored populations:
//   kAB      two-lattice fused pull (reads src, writes dst);
//   kAAEven  one lattice, even step: read (q,x), write (opp q, x);
//   kAAOdd   one lattice, odd step: read (opp q, x - c_q), write (q, x + c_q);
//   kEsoEven, kEsoOdd  one lattice, esoteric pull: each pair of opposite
//            directions is read from the own cell and from the neighbour along
//            one of them and written back to the same two slots, whose roles
//            swap from one step to the next (even / odd step).
//   kTwEven, kTwOdd  one lattice, esoteric twist: each population is read
//            from the cell itself or one of the six cells behind it along
//            -x, -y, -z and the face diagonals between them, and written to
//            the slot its opposite was read from, with the planes of a pair
//            swapping roles from one step to the next.
enum Kind : int { kAB = 0, kAAEven = 1, kAAOdd = 2, kEsoEven = 3, kEsoOdd = 4, kTwEven = 5, kTwOdd = 6 };

constexpr bool is_eso(int k) { return k == kEsoEven || k == kEsoOdd; }
constexpr bool is_twist(int k) { return k == kTwEven || k == kTwOdd; }
// the stored state uses slots of solid (and, for the twist, halo) cells
constexpr bool solid_slots_live(int k) { return is_eso(k) || is_twist(k); }

}  // namespace lbm
