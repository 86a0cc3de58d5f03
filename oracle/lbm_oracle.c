/*
 * lbm_oracle.c -- plain, slow, obviously correct CPU oracle for the D3Q19 BGK
 * lattice Boltzmann update with halfway bounce-back and Guo body forcing.
 *
 * TEST INFRASTRUCTURE ONLY: called by the tests, by the smoke check and by
 * the benchmark's CPU-baseline leg.  The product (GPU) path never loads it.
 *
 * Single-threaded, fp64 throughout (long double for the global sums), built
 * with -O2 -ffp-contract=off.  Each time step is written exactly as the
 * lattice Boltzmann equation splits it -- a collision pass over every cell
 * into a separate post-collision array, then a streaming pass that pulls
 * from it -- with no fusion, blocking or reordering.
 *
 * What the pages fix, and where:
 *  - BGK lattice Boltzmann equation, dt = 1:  PortLBM page ("PortLBM: A
 *    Portable Lattice Boltzmann Tool Leveraging SYCL on AMD, NVIDIA, and
 *    Intel GPUs"), section 3.1, Eq. (1); its split into a collision and a
 *    streaming step, section 3.3, Eq. (3).
 *  - Second-order polynomial equilibrium with coefficients 1, 3, 9/2, -3/2:
 *    PortLBM page, section 3.1, Eq. (2).
 *  - D3Q19 weights 1/3 (rest), 1/18 (6 axis), 1/36 (12 diagonal) and the
 *    velocity set inside {-1,0,1}^3: codechina page ("GPU加速LBM流体仿真"),
 *    sections 2.1 and 2.2.
 *  - Halfway bounce-back at fluid-solid links: PortLBM page, section 3.1,
 *    last paragraph; the same per-link rule in every streaming scheme:
 *    fieldcraft page ("GPU lattice Boltzmann: streaming layout and
 *    performance"), first section.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - Direction order: lexicographic over (c_z, c_y, c_x) of the vectors in
 *    {-1,0,1}^3 with |c|^2 <= 2 (PortLBM's 2-D raster, Fig. 2, extended to 3-D).
 *  - Equilibrium: the compressible form w rho (1 + 3 c.u + 9/2 (c.u)^2 - 3/2 u^2)
 *    with u = (sum c f + F/2) / rho.
 *  - Forcing: Guo, Zheng and Shi (Phys. Rev. E 65, 046308, 2002),
 *    F_q = (1 - omega/2) w_q [3 (c_q - u) + 9 (c_q.u) c_q] . F, with F a
 *    constant force density.
 *  - tau = +inf means omega = 0: collision is the identity (streaming only).
 *  - Cells outside a non-periodic face count as solid, unless that face is
 *    open: then the populations leaving through it are dropped and those
 *    entering through it are set by the face's rule after streaming
 *    (PortLBM page, section 3.1, boundary paragraph: an inlet takes the
 *    equilibrium distribution of Dirichlet or Neumann values, the outlet an
 *    adapted Zou-He condition).  Readings: Dirichlet = a reservoir at
 *    feq(face rho, face u); Neumann = feq of the density and velocity of the
 *    cell one layer inward (zero normal gradient, same state); Zou-He = the
 *    non-equilibrium bounce-back of Zou and He (Phys. Fluids 9, 1591, 1997)
 *    on the entering populations, with the transverse momentum correction
 *    that the 3-D lattice needs (Hecht and Harting, J. Stat. Mech. 2010,
 *    P01018), for a prescribed density (pressure) or velocity; the momentum
 *    in it is the bare sum of c f, i.e. rho u - F/2 under Guo forcing.
 */
#include "lbm_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int32_t C[ORC_Q][3];
static double W[ORC_Q];
static int32_t OPP[ORC_Q];
static int tables_ready = 0;

/* Build the velocity set by enumeration rather than from a typed table. */
static void build_tables(void)
{
    if (tables_ready) return;
    int q = 0;
    for (int cz = -1; cz <= 1; ++cz)
        for (int cy = -1; cy <= 1; ++cy)
            for (int cx = -1; cx <= 1; ++cx) {
                int n2 = cx * cx + cy * cy + cz * cz;
                if (n2 > 2) continue;
                C[q][0] = cx;
                C[q][1] = cy;
                C[q][2] = cz;
                W[q] = (n2 == 0) ? 1.0 / 3.0 : (n2 == 1) ? 1.0 / 18.0 : 1.0 / 36.0;
                ++q;
            }
    for (int a = 0; a < ORC_Q; ++a)
        for (int p = 0; p < ORC_Q; ++p)
            if (C[p][0] == -C[a][0] && C[p][1] == -C[a][1] && C[p][2] == -C[a][2]) OPP[a] = p;
    tables_ready = 1;
}

void orc_lattice(int32_t c[ORC_Q][3], double w[ORC_Q], int32_t opp[ORC_Q])
{
    build_tables();
    for (int q = 0; q < ORC_Q; ++q) {
        for (int a = 0; a < 3; ++a) c[q][a] = C[q][a];
        w[q] = W[q];
        opp[q] = OPP[q];
    }
}

static double omega_of(const orc_box *b)
{
    return isinf(b->tau) ? 0.0 : 1.0 / b->tau;
}

void orc_equilibrium(double rho, const double u[3], double feq[ORC_Q])
{
    build_tables();
    double usq = u[0] * u[0] + u[1] * u[1] + u[2] * u[2];
    for (int q = 0; q < ORC_Q; ++q) {
        double cu = C[q][0] * u[0] + C[q][1] * u[1] + C[q][2] * u[2];
        feq[q] = W[q] * rho * (1.0 + 3.0 * cu + 4.5 * cu * cu - 1.5 * usq);
    }
}

void orc_guo_term(double omega, const double u[3], const double F[3], double out[ORC_Q])
{
    build_tables();
    for (int q = 0; q < ORC_Q; ++q) {
        double cu = C[q][0] * u[0] + C[q][1] * u[1] + C[q][2] * u[2];
        double s = 0.0;
        for (int a = 0; a < 3; ++a) s += (3.0 * (C[q][a] - u[a]) + 9.0 * cu * C[q][a]) * F[a];
        out[q] = (1.0 - 0.5 * omega) * W[q] * s;
    }
}

void orc_cell_moments(const orc_box *b, const double f[ORC_Q], double *rho, double u[3])
{
    build_tables();
    double r = 0.0, j[3] = {0.0, 0.0, 0.0};
    for (int q = 0; q < ORC_Q; ++q) {
        r += f[q];
        for (int a = 0; a < 3; ++a) j[a] += C[q][a] * f[q];
    }
    *rho = r;
    for (int a = 0; a < 3; ++a) u[a] = (j[a] + 0.5 * b->force[a]) / r;
}

void orc_collide(const orc_box *b, const double f[ORC_Q], double post[ORC_Q])
{
    double rho, u[3], feq[ORC_Q], fq[ORC_Q];
    double omega = omega_of(b);
    orc_cell_moments(b, f, &rho, u);
    orc_equilibrium(rho, u, feq);
    orc_guo_term(omega, u, b->force, fq);
    for (int q = 0; q < ORC_Q; ++q) post[q] = f[q] - omega * (f[q] - feq[q]) + fq[q];
}

static int64_t ncells(const orc_box *b)
{
    return b->nx * b->ny * b->nz;
}

static int is_solid(const uint8_t *mask, int64_t cell)
{
    return mask != NULL && mask[cell] != 0;
}

/* What lies at (x + dx, y + dy, z + dz): a fluid cell (its index in *cell),
 * a solid cell or a wall (bounce-back), or the reservoir of an open face
 * (its number in *face).  Periodic axes wrap.  Beyond two faces at once (an
 * edge of the box), a wall wins over an open face, and of two open faces the
 * one on the first axis in x, y, z order is used. */
enum { LINK_FLUID = 0, LINK_SOLID = 1, LINK_WALL = 2, LINK_OPEN = 3 };

static int classify(const orc_box *b, const uint8_t *mask, int64_t x, int64_t y, int64_t z, int dx, int dy,
                    int dz, int64_t *cell, int *face)
{
    int64_t p[3] = {x + dx, y + dy, z + dz};
    int64_t n[3] = {b->nx, b->ny, b->nz};
    int wall = 0, open_face = -1;
    for (int a = 0; a < 3; ++a) {
        if (p[a] >= 0 && p[a] < n[a]) continue;
        if (b->periodic[a]) {
            p[a] = (p[a] + n[a]) % n[a];
            continue;
        }
        int k = 2 * a + (p[a] < 0 ? 0 : 1);
        if (b->open[k]) {
            if (open_face < 0) open_face = k;
        } else {
            wall = 1;
        }
    }
    if (wall) return LINK_WALL;
    if (open_face >= 0) {
        *face = open_face;
        return LINK_OPEN;
    }
    *cell = p[0] + b->nx * (p[1] + b->ny * p[2]);
    return is_solid(mask, *cell) ? LINK_SOLID : LINK_FLUID;
}

static void face_equilibrium(const orc_box *b, int face, double feq[ORC_Q])
{
    orc_equilibrium(b->face_rho[face], b->face_u[face], feq);
}

static int is_reservoir(const orc_box *b, int face)
{
    return b->face_kind[face] == ORC_FACE_EQUILIBRIUM;
}

/* The rule of face k (not a reservoir) at one cell on that face.  fx: the
 * cell's 19 populations after streaming; the entries with ent[q] set (the
 * populations entering through face k) are replaced.  f1: the 19 populations
 * of the cell one layer inward along the face normal (NULL if solid), read by
 * the Neumann rule only. */
static void face_rule(const orc_box *b, int k, double fx[ORC_Q], const int ent[ORC_Q], const double *f1)
{
    const int a = k / 2;
    const int sigma = (k % 2 == 0) ? 1 : -1; /* inward normal is sigma e_a */
    if (b->face_kind[k] == ORC_FACE_NEUMANN) {
        double rho, u[3], feq[ORC_Q];
        if (f1 != NULL) {
            orc_cell_moments(b, f1, &rho, u);
        } else {
            rho = b->face_rho[k];
            for (int t = 0; t < 3; ++t) u[t] = b->face_u[k][t];
        }
        orc_equilibrium(rho, u, feq);
        for (int q = 0; q < ORC_Q; ++q)
            if (ent[q]) fx[q] = feq[q];
        return;
    }
    /* Zou-He: mass of the populations parallel to the face (c_a = 0) and of
     * those leaving through it (c_a = -sigma); tangential momentum of the
     * parallel ones */
    double par = 0.0, out = 0.0, tpar[3] = {0.0, 0.0, 0.0};
    for (int q = 0; q < ORC_Q; ++q) {
        if (C[q][a] == 0) {
            par += fx[q];
            for (int t = 0; t < 3; ++t) tpar[t] += C[q][t] * fx[q];
        } else if (C[q][a] == -sigma) {
            out += fx[q];
        }
    }
    /* bare momentum j = sum c f = rho u - F/2.  Mass: rho = par + in + out and
     * sigma j_a = in - out, so sigma j_a = rho - par - 2 out. */
    double rho, j[3];
    if (b->face_kind[k] == ORC_FACE_ZOU_HE_PRESSURE) {
        rho = b->face_rho[k];
        for (int t = 0; t < 3; ++t) j[t] = rho * b->face_u[k][t] - 0.5 * b->force[t];
        j[a] = sigma * (rho - par - 2.0 * out);
    } else {
        rho = (par + 2.0 * out - 0.5 * sigma * b->force[a]) / (1.0 - sigma * b->face_u[k][a]);
        for (int t = 0; t < 3; ++t) j[t] = rho * b->face_u[k][t] - 0.5 * b->force[t];
    }
    /* transverse correction: the parallel populations carry tangential
     * momentum tpar; the entering ones must bring j_t - tpar - (leaving ones'
     * share), which the bounce-back of the opposites gives up to 2 N_t */
    double nt[3] = {0.0, 0.0, 0.0};
    for (int t = 0; t < 3; ++t)
        if (t != a) nt[t] = 0.5 * tpar[t] - j[t] / 3.0;
    for (int q = 0; q < ORC_Q; ++q) {
        if (!ent[q]) continue;
        double cj = 0.0, corr = 0.0;
        for (int t = 0; t < 3; ++t) {
            cj += C[q][t] * j[t];
            corr += C[q][t] * nt[t];
        }
        /* feq_q - feq_opp(q) = 6 w_q c_q . j (the odd part of the equilibrium) */
        fx[q] = fx[OPP[q]] + 6.0 * W[q] * cj - corr;
    }
}

/* Which populations of cell (xx, y, z) enter through face k; 0 if none. */
static int entering_through(const orc_box *b, const uint8_t *mask, int64_t xx, int64_t y, int64_t z, int k,
                            int ent[ORC_Q])
{
    int any = 0;
    for (int q = 0; q < ORC_Q; ++q) {
        int64_t src;
        int face = -1;
        ent[q] = classify(b, mask, xx, y, z, -C[q][0], -C[q][1], -C[q][2], &src, &face) == LINK_OPEN && face == k;
        any |= ent[q];
    }
    return any;
}

/* Apply the rule of face k to every fluid cell on it, in place in f. */
static void face_cells_apply(const orc_box *b, const uint8_t *mask, double *f, int k)
{
    int64_t N = ncells(b);
    const int a = k / 2;
    const int sigma = (k % 2 == 0) ? 1 : -1;
    int64_t n[3] = {b->nx, b->ny, b->nz};
    for (int64_t z = 0; z < b->nz; ++z)
        for (int64_t y = 0; y < b->ny; ++y)
            for (int64_t xx = 0; xx < b->nx; ++xx) {
                int64_t p[3] = {xx, y, z};
                if (p[a] != (sigma > 0 ? 0 : n[a] - 1)) continue;
                int64_t x = xx + b->nx * (y + b->ny * z);
                if (is_solid(mask, x)) continue;
                int ent[ORC_Q];
                if (!entering_through(b, mask, xx, y, z, k, ent)) continue;
                p[a] += sigma;
                int64_t x1 = p[0] + b->nx * (p[1] + b->ny * p[2]);
                double fx[ORC_Q], f1[ORC_Q];
                for (int q = 0; q < ORC_Q; ++q) {
                    fx[q] = f[q * N + x];
                    f1[q] = f[q * N + x1];
                }
                face_rule(b, k, fx, ent, is_solid(mask, x1) ? NULL : f1);
                for (int q = 0; q < ORC_Q; ++q)
                    if (ent[q]) f[q * N + x] = fx[q];
            }
}

/* Apply the rules of the open faces that are not reservoirs.  A rule writes
 * only the entering populations of cells on its face and reads none of them
 * (a Zou-He cell reads its parallel and leaving populations, a Neumann cell
 * the cell one layer inward, which is on no open face), so the order of the
 * cells does not matter. */
static void apply_rule_faces(const orc_box *b, const uint8_t *mask, double *f)
{
    for (int k = 0; k < 6; ++k)
        if (b->open[k] && !is_reservoir(b, k)) face_cells_apply(b, mask, f, k);
}

void orc_apply_open_faces(const orc_box *b, const uint8_t *mask, double *f)
{
    build_tables();
    int64_t N = ncells(b);
    for (int64_t z = 0; z < b->nz; ++z)
        for (int64_t y = 0; y < b->ny; ++y)
            for (int64_t xx = 0; xx < b->nx; ++xx) {
                int64_t x = xx + b->nx * (y + b->ny * z);
                if (is_solid(mask, x)) continue;
                for (int q = 0; q < ORC_Q; ++q) {
                    int64_t src;
                    int face;
                    if (classify(b, mask, xx, y, z, -C[q][0], -C[q][1], -C[q][2], &src, &face) != LINK_OPEN)
                        continue;
                    if (!is_reservoir(b, face)) continue;
                    double feq[ORC_Q];
                    face_equilibrium(b, face, feq);
                    f[q * N + x] = feq[q];
                }
            }
    apply_rule_faces(b, mask, f);
}

int orc_init_equilibrium(const orc_box *b, const uint8_t *mask, const double *rho0,
                         const double *u0, double *f)
{
    build_tables();
    int64_t N = ncells(b);
    for (int64_t x = 0; x < N; ++x) {
        double feq[ORC_Q];
        if (is_solid(mask, x)) {
            for (int q = 0; q < ORC_Q; ++q) f[q * N + x] = 0.0;
            continue;
        }
        double rho = rho0 ? rho0[x] : 1.0;
        double u[3] = {0.0, 0.0, 0.0};
        if (u0)
            for (int a = 0; a < 3; ++a) u[a] = u0[a * N + x];
        orc_equilibrium(rho, u, feq);
        for (int q = 0; q < ORC_Q; ++q) f[q * N + x] = feq[q];
    }
    orc_apply_open_faces(b, mask, f);
    return 0;
}

/* Collision pass: post[q][x] for every cell (0 on solid cells). */
static void collide_all(const orc_box *b, const uint8_t *mask, const double *f, double *post)
{
    int64_t N = ncells(b);
    for (int64_t x = 0; x < N; ++x) {
        double in[ORC_Q], out[ORC_Q];
        if (is_solid(mask, x)) {
            for (int q = 0; q < ORC_Q; ++q) post[q * N + x] = 0.0;
            continue;
        }
        for (int q = 0; q < ORC_Q; ++q) in[q] = f[q * N + x];
        orc_collide(b, in, out);
        for (int q = 0; q < ORC_Q; ++q) post[q * N + x] = out[q];
    }
}

/* Streaming pass (pull): the value arriving at x along c_q left x - c_q, unless
 * that cell is solid or beyond a wall, in which case the population that left
 * x along -c_q is reflected back at the link midpoint, or lies beyond an open
 * face, in which case it is the face reservoir's equilibrium population (for
 * the other face rules, a placeholder that the rule replaces). */
static void stream_all(const orc_box *b, const uint8_t *mask, const double *post, double *fnew)
{
    int64_t N = ncells(b);
    for (int64_t z = 0; z < b->nz; ++z)
        for (int64_t y = 0; y < b->ny; ++y)
            for (int64_t xx = 0; xx < b->nx; ++xx) {
                int64_t x = xx + b->nx * (y + b->ny * z);
                for (int q = 0; q < ORC_Q; ++q) {
                    if (is_solid(mask, x)) {
                        fnew[q * N + x] = 0.0;
                        continue;
                    }
                    int64_t src = -1;
                    int face = -1;
                    int kind = classify(b, mask, xx, y, z, -C[q][0], -C[q][1], -C[q][2], &src, &face);
                    if (kind == LINK_FLUID) {
                        fnew[q * N + x] = post[q * N + src];
                    } else if (kind == LINK_OPEN && is_reservoir(b, face)) {
                        double feq[ORC_Q];
                        face_equilibrium(b, face, feq);
                        fnew[q * N + x] = feq[q];
                    } else {
                        /* solid, wall, or an open face with a rule: the rule
                         * replaces this placeholder after the pass */
                        fnew[q * N + x] = post[OPP[q] * N + x];
                    }
                }
            }
}

int orc_run(const orc_box *b, const uint8_t *mask, double *f, int64_t nsteps)
{
    build_tables();
    int64_t N = ncells(b);
    if (nsteps <= 0) return 0;
    double *post = (double *)malloc(sizeof(double) * ORC_Q * (size_t)N);
    if (!post) return -1;
    for (int64_t t = 0; t < nsteps; ++t) {
        collide_all(b, mask, f, post);
        stream_all(b, mask, post, f); /* f is overwritten only after post is complete */
        apply_rule_faces(b, mask, f);
    }
    free(post);
    return 0;
}

/* f(t+1) at one fluid cell before the rules of open faces (pull over the
 * post-collision values of the source cells, computed here one by one). */
static void step_one_cell(const orc_box *b, const uint8_t *mask, const double *f, int64_t x, double o[ORC_Q])
{
    int64_t N = ncells(b);
    int64_t xx = x % b->nx, y = (x / b->nx) % b->ny, z = x / (b->nx * b->ny);
    for (int q = 0; q < ORC_Q; ++q) {
        int64_t src = -1;
        int face = -1;
        int kind = classify(b, mask, xx, y, z, -C[q][0], -C[q][1], -C[q][2], &src, &face);
        if (kind == LINK_OPEN && is_reservoir(b, face)) {
            double feq[ORC_Q];
            face_equilibrium(b, face, feq);
            o[q] = feq[q];
            continue;
        }
        int use_bb = kind != LINK_FLUID;
        int64_t from = use_bb ? x : src;
        double in[ORC_Q], post[ORC_Q];
        for (int p = 0; p < ORC_Q; ++p) in[p] = f[p * N + from];
        orc_collide(b, in, post);
        o[q] = use_bb ? post[OPP[q]] : post[q];
    }
}

int orc_step_cells(const orc_box *b, const uint8_t *mask, const double *f, int64_t ncell,
                   const int64_t *cells, double *out)
{
    build_tables();
    int64_t N = ncells(b);
    for (int64_t k = 0; k < ncell; ++k) {
        int64_t x = cells[k];
        double *o = out + k * ORC_Q;
        if (x < 0 || x >= N) return -1;
        if (is_solid(mask, x)) {
            for (int q = 0; q < ORC_Q; ++q) o[q] = 0.0;
            continue;
        }
        step_one_cell(b, mask, f, x, o);
        int64_t p[3] = {x % b->nx, (x / b->nx) % b->ny, x / (b->nx * b->ny)};
        for (int face = 0; face < 6; ++face) {
            int ent[ORC_Q];
            if (!b->open[face] || is_reservoir(b, face)) continue;
            if (!entering_through(b, mask, p[0], p[1], p[2], face, ent)) continue;
            int64_t p1[3] = {p[0], p[1], p[2]};
            p1[face / 2] += (face % 2 == 0) ? 1 : -1;
            int64_t x1 = p1[0] + b->nx * (p1[1] + b->ny * p1[2]);
            double f1[ORC_Q];
            if (!is_solid(mask, x1)) step_one_cell(b, mask, f, x1, f1);
            face_rule(b, face, o, ent, is_solid(mask, x1) ? NULL : f1);
        }
    }
    return 0;
}

void orc_moments(const orc_box *b, const uint8_t *mask, const double *f, double *rho, double *u)
{
    build_tables();
    int64_t N = ncells(b);
    for (int64_t x = 0; x < N; ++x) {
        if (is_solid(mask, x)) {
            rho[x] = 0.0;
            for (int a = 0; a < 3; ++a) u[a * N + x] = 0.0;
            continue;
        }
        double in[ORC_Q], r, v[3];
        for (int q = 0; q < ORC_Q; ++q) in[q] = f[q * N + x];
        orc_cell_moments(b, in, &r, v);
        rho[x] = r;
        for (int a = 0; a < 3; ++a) u[a * N + x] = v[a];
    }
}

void orc_totals(const orc_box *b, const uint8_t *mask, const double *f, double out[5])
{
    build_tables();
    int64_t N = ncells(b);
    long double m = 0.0L, p[3] = {0.0L, 0.0L, 0.0L}, ke = 0.0L;
    for (int64_t x = 0; x < N; ++x) {
        if (is_solid(mask, x)) continue;
        double in[ORC_Q], r, v[3];
        for (int q = 0; q < ORC_Q; ++q) {
            in[q] = f[q * N + x];
            m += (long double)in[q];
        }
        orc_cell_moments(b, in, &r, v);
        for (int a = 0; a < 3; ++a) p[a] += (long double)r * (long double)v[a];
        ke += 0.5L * (long double)r * ((long double)v[0] * v[0] + (long double)v[1] * v[1] +
                                        (long double)v[2] * v[2]);
    }
    out[0] = (double)m;
    for (int a = 0; a < 3; ++a) out[1 + a] = (double)p[a];
    out[4] = (double)ke;
}

/* Momentum exchange of the halfway bounce-back links during the step that
 * starts from f (fieldcraft page, first section: the momentum exchange is
 * taken over the wall links of a step).  A population f*_q that leaves fluid
 * cell x toward a solid cell or a wall is reflected at the link midpoint and
 * comes back as f*_q along -c_q, so the solid receives 2 f*_q c_q.  out[0..2]
 * sums the links that end in a solid cell of the mask, out[3..5] the links
 * that leave the box through a wall (a non-periodic face that is not open;
 * links through open faces carry flux, not force on a solid). */
void orc_momentum_exchange(const orc_box *b, const uint8_t *mask, const double *f, double out[6])
{
    build_tables();
    int64_t N = ncells(b);
    long double solid[3] = {0.0L, 0.0L, 0.0L}, wall[3] = {0.0L, 0.0L, 0.0L};
    for (int64_t z = 0; z < b->nz; ++z)
        for (int64_t y = 0; y < b->ny; ++y)
            for (int64_t xx = 0; xx < b->nx; ++xx) {
                int64_t x = xx + b->nx * (y + b->ny * z);
                if (is_solid(mask, x)) continue;
                double in[ORC_Q], post[ORC_Q];
                for (int q = 0; q < ORC_Q; ++q) in[q] = f[q * N + x];
                orc_collide(b, in, post);
                for (int q = 0; q < ORC_Q; ++q) {
                    int64_t dst = -1;
                    int face = -1;
                    int kind = classify(b, mask, xx, y, z, C[q][0], C[q][1], C[q][2], &dst, &face);
                    if (kind == LINK_FLUID || kind == LINK_OPEN) continue;
                    long double *acc = kind == LINK_WALL ? wall : solid;
                    for (int a = 0; a < 3; ++a) acc[a] += 2.0L * (long double)post[q] * (long double)C[q][a];
                }
            }
    for (int a = 0; a < 3; ++a) {
        out[a] = (double)solid[a];
        out[3 + a] = (double)wall[a];
    }
}
