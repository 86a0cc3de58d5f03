/*
 * lbm_oracle.h -- C interface of the CPU oracle for the fused D3Q19 BGK
 * collide-and-stream update.
 *
 * TEST INFRASTRUCTURE ONLY.  The oracle exists to check the GPU path; only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header, table or helper with the GPU library.
 *
 * Every array of populations is "canonical": double f[19][N], direction-major,
 * cell = x + nx*(y + ny*z), directions in the oracle's own order (see
 * orc_lattice).  f holds the pre-collision populations f(t) of the lattice
 * Boltzmann equation (PortLBM page, section 3.1, Eq. 1).  Solid cells hold 0.
 */
#ifndef LBM_ORACLE_H
#define LBM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_Q 19

typedef struct {
    int64_t nx, ny, nz;
    int32_t periodic[3]; /* 1: periodic axis; 0: halfway bounce-back wall beyond both faces */
    double tau;          /* BGK relaxation time; +inf gives omega = 0 (no collision) */
    double force[3];     /* constant body-force density, Guo forcing; zeros = off */
    /* Open faces, in the order -x, +x, -y, +y, -z, +z (only on non-periodic
     * axes): open[k] = 1 replaces the wall beyond face k by an open boundary
     * whose rule face_kind[k] sets every population entering through it;
     * face_rho[k] and face_u[k] are its prescribed values. */
    int32_t open[6];
    double face_rho[6];
    double face_u[6][3];
    /* Rule of each open face (ORC_FACE_*).  The rules other than the
     * equilibrium reservoir need every open face of the box on one axis and
     * at least 3 cells along it. */
    int32_t face_kind[6];
} orc_box;

/* Open-face rules (PortLBM page, section 3.1: equilibrium distribution from
 * Dirichlet or Neumann values at the inlet, an adapted Zou-He condition at
 * the outlet).  Each sets the populations entering through the face, after
 * every streaming pass:
 *  EQUILIBRIUM     feq(face_rho, face_u) (a reservoir; Dirichlet values)
 *  NEUMANN         feq(rho, u) of the cell one layer inward along the face
 *                  normal, in the same state (zero normal gradient); the
 *                  reservoir's values if that cell is solid
 *  ZOU_HE_PRESSURE density face_rho and tangential velocity from face_u;
 *                  the normal velocity follows from mass
 *  ZOU_HE_VELOCITY velocity face_u; the density follows from mass
 * The Zou-He rules take each entering population from its opposite by
 * non-equilibrium bounce-back, with the transverse momentum correction of
 * the 3-D lattice, so that the cell's density (pressure rule) or velocity
 * (velocity rule) and its tangential momentum are the prescribed ones. */
enum { ORC_FACE_EQUILIBRIUM = 0, ORC_FACE_NEUMANN = 1, ORC_FACE_ZOU_HE_PRESSURE = 2, ORC_FACE_ZOU_HE_VELOCITY = 3 };

/* Velocity set, weights and opposite-direction table. */
void orc_lattice(int32_t c[ORC_Q][3], double w[ORC_Q], int32_t opp[ORC_Q]);

/* Second-order equilibrium of one cell. */
void orc_equilibrium(double rho, const double u[3], double feq[ORC_Q]);

/* Guo forcing term of one cell (u includes the F/2 shift). */
void orc_guo_term(double omega, const double u[3], const double F[3], double out[ORC_Q]);

/* BGK collision of one cell: post = f - omega (f - feq) + F_q. */
void orc_collide(const orc_box *b, const double f[ORC_Q], double post[ORC_Q]);

/* Density and velocity (u includes F/2) of one cell. */
void orc_cell_moments(const orc_box *b, const double f[ORC_Q], double *rho, double u[3]);

/* f := equilibrium(rho0, u0) on fluid cells, 0 on solid cells.  rho0 == NULL
 * means 1 everywhere, u0 == NULL means 0; u0 is [3][N]. mask may be NULL. */
int orc_init_equilibrium(const orc_box *b, const uint8_t *mask, const double *rho0,
                         const double *u0, double *f);

/* Advance f by nsteps (collide, then stream with halfway bounce-back). */
int orc_run(const orc_box *b, const uint8_t *mask, double *f, int64_t nsteps);

/* One step evaluated only at the listed cells: out[k][19] = f(t+1) at cells[k]. */
int orc_step_cells(const orc_box *b, const uint8_t *mask, const double *f, int64_t ncells,
                   const int64_t *cells, double *out);

/* rho[N], u[3][N] from f; zeros on solid cells. */
void orc_moments(const orc_box *b, const uint8_t *mask, const double *f, double *rho, double *u);

/* out = {mass, Px, Py, Pz, kinetic energy} summed over fluid cells in long double. */
void orc_totals(const orc_box *b, const uint8_t *mask, const double *f, double out[5]);

/* Set every population entering the box through an open face by that face's
 * rule (the state invariant of open faces; init and every step apply it). */
void orc_apply_open_faces(const orc_box *b, const uint8_t *mask, double *f);

/* Momentum-exchange force of the step that starts from f: sum over the
 * bounce-back links (fluid x, x + c_q solid or beyond a wall) of 2 f*_q c_q,
 * f* = collision of f(x).  out = {solid x, y, z, wall x, y, z}. */
void orc_momentum_exchange(const orc_box *b, const uint8_t *mask, const double *f, double out[6]);

#ifdef __cplusplus
}
#endif
#endif
