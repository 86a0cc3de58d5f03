/* Drives every entry point of the CPU oracle on small boxes (solids, walls,
 * open faces of every kind, degenerate axes) for an AddressSanitizer /
 * UndefinedBehaviorSanitizer build: any out-of-bounds access or undefined
 * operation aborts the process.  Test infrastructure only. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/lbm_oracle.h"

static unsigned long long rng = 88172645463325252ULL;
static double urand(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) * (1.0 / 9007199254740992.0);
}

static int exercise(orc_box *b, double solid_fraction)
{
    const int64_t n = b->nx * b->ny * b->nz;
    uint8_t *mask = (uint8_t *)malloc((size_t)n);
    double *rho = (double *)malloc(sizeof(double) * (size_t)n);
    double *u = (double *)malloc(sizeof(double) * 3 * (size_t)n);
    double *f = (double *)malloc(sizeof(double) * ORC_Q * (size_t)n);
    double *r = (double *)malloc(sizeof(double) * (size_t)n);
    double *v = (double *)malloc(sizeof(double) * 3 * (size_t)n);
    int64_t cells[8];
    double out[8 * ORC_Q], tot[5], mex[6];
    if (!mask || !rho || !u || !f || !r || !v) return 1;
    for (int64_t i = 0; i < n; ++i) {
        mask[i] = urand() < solid_fraction;
        rho[i] = 1.0 + 0.01 * (2.0 * urand() - 1.0);
        for (int a = 0; a < 3; ++a) u[a * n + i] = 0.03 * (2.0 * urand() - 1.0);
    }
    if (orc_init_equilibrium(b, mask, rho, u, f) != 0) return 2;
    if (orc_run(b, mask, f, 5) != 0) return 3;
    for (int k = 0; k < 8; ++k) cells[k] = (int64_t)(urand() * (double)n) % n;
    cells[0] = 0;
    cells[1] = n - 1;
    if (orc_step_cells(b, mask, f, 8, cells, out) != 0) return 4;
    orc_moments(b, mask, f, r, v);
    orc_totals(b, mask, f, tot);
    orc_momentum_exchange(b, mask, f, mex);
    orc_apply_open_faces(b, mask, f);
    for (int64_t i = 0; i < ORC_Q * n; ++i)
        if (!isfinite(f[i])) return 5;
    free(mask);
    free(rho);
    free(u);
    free(f);
    free(r);
    free(v);
    return 0;
}

static orc_box make(int64_t nx, int64_t ny, int64_t nz, int px, int py, int pz)
{
    orc_box b;
    memset(&b, 0, sizeof b);
    b.nx = nx;
    b.ny = ny;
    b.nz = nz;
    b.periodic[0] = px;
    b.periodic[1] = py;
    b.periodic[2] = pz;
    b.tau = 0.8;
    b.force[0] = 1e-5;
    b.force[2] = -2e-5;
    for (int k = 0; k < 6; ++k) b.face_rho[k] = 1.0;
    return b;
}

int main(void)
{
    int32_t c[ORC_Q][3], opp[ORC_Q];
    double w[ORC_Q];
    orc_lattice(c, w, opp);
    orc_box boxes[8];
    boxes[0] = make(6, 5, 4, 1, 1, 1);
    boxes[1] = make(5, 4, 6, 0, 1, 0);
    boxes[2] = make(1, 1, 1, 1, 1, 1);
    boxes[3] = make(2, 1, 7, 1, 0, 1);
    /* equilibrium reservoirs on two axes, walls on the third */
    boxes[4] = make(5, 5, 4, 0, 0, 0);
    boxes[4].open[0] = boxes[4].open[3] = 1;
    boxes[4].face_u[0][0] = 0.02;
    /* each face rule on an x axis with y walls */
    for (int kind = 1; kind <= 3; ++kind) {
        boxes[4 + kind] = make(6, 4, 3, 0, 0, 1);
        boxes[4 + kind].open[0] = boxes[4 + kind].open[1] = 1;
        boxes[4 + kind].face_kind[0] = kind;
        boxes[4 + kind].face_kind[1] = kind == 3 ? 2 : kind;
        boxes[4 + kind].face_u[0][0] = 0.03;
    }
    for (int i = 0; i < 8; ++i) {
        const int rc = exercise(&boxes[i], i == 2 ? 0.0 : 0.15);
        if (rc != 0) {
            printf("box %d failed: %d\n", i, rc);
            return 1;
        }
    }
    printf("ok\n");
    return 0;
}
