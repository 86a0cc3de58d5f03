/*
 * lbm.h -- C ABI of the MI355X (gfx950) D3Q19 BGK collide-and-stream library
 * (liblbm.so).
 *
 * The library advances the lattice Boltzmann equation with BGK relaxation
 * (PortLBM page, "PortLBM: A Portable Lattice Boltzmann Tool Leveraging SYCL
 * on AMD, NVIDIA, and Intel GPUs", section 3.1, Eq. 1) on a D3Q19 lattice
 * (weights 1/3, 1/18, 1/36: codechina page "GPU加速LBM流体仿真", section 2.2),
 * relaxing toward the second-order equilibrium (PortLBM section 3.1, Eq. 2,
 * compressible form w rho (1 + 3 c.u + 9/2 (c.u)^2 - 3/2 u^2)), with halfway
 * bounce-back on a solid mask (PortLBM section 3.1, last paragraph) and an
 * optional constant body force (Guo, Zheng and Shi 2002 forcing term).
 * Every step is one fused kernel: gather 19 populations, moments,
 * equilibrium, forcing, relaxation, scatter 19 populations.
 *
 * Propagation schemes (PortLBM section 3.3; fieldcraft page "GPU lattice
 * Boltzmann: streaming layout and performance", first section):
 *   LBM_SCHEME_AB  two lattices; each cell pulls from the source lattice and
 *                  writes post-collision values into the destination one.
 *   LBM_SCHEME_AA  one lattice, in place.  Even steps read slot (q, x) and
 *                  write (opposite(q), x); odd steps read (opposite(q), x - c_q)
 *                  and write (q, x + c_q).  Each cell writes exactly the slots
 *                  it read.
 *   LBM_SCHEME_ESOPULL  one lattice, in place, the esoteric pull that PortLBM
 *                  (section 3.3) names among the in-place schemes (Lehmann,
 *                  Computation 10, 92, 2022): each pair of opposite directions
 *                  (q, 18 - q), q < 9, has two slots per cell; a step reads f_q
 *                  from the own cell and f_(18-q) from the neighbour x + c_q,
 *                  and writes the collided f_(18-q) and f_q back into those two
 *                  slots, whose roles swap every step.  Bounce-back links keep
 *                  their value in slots no other link uses (a solid
 *                  neighbour's, the wrapped cell's beyond a face; in the
 *                  compact layout a packed region after the blocks).
 *   LBM_SCHEME_ESOTWIST  one lattice, in place, the esoteric twist that
 *                  PortLBM (section 3.3) names with AA and the esoteric pull
 *                  (Geier and Schoenherr, Computation 5, 19, 2017): with
 *                  c+ = max(c_q, 0) per axis, f_q(x) lives at x - c+ (the cell
 *                  or one of the six behind it along -x, -y, -z and their face
 *                  diagonals) in plane q at even t, opposite(q) at odd t; a step
 *                  writes the collided f_q where it read f_opposite(q), or into
 *                  the other plane there when the link bounces back.  Dense
 *                  layouts keep one halo layer below each low face for the
 *                  values behind a wall: their buffers hold (nx+1)(ny+1)(nz+1)
 *                  cells per plane (lbm_buffer_bytes).  The compact layout
 *                  gives each solid or halo cell behind a fluid cell a ghost
 *                  slot after the fluid cells (its buffer has room for the
 *                  same (nx+1)(ny+1)(nz+1) cells; its workspace also holds
 *                  the stored index of every padded cell).
 * Population layouts (PortLBM section 3.2, Fig. 2):
 *   LBM_LAYOUT_STREAM     SoA: all cells of direction 0, then direction 1, ...
 *   LBM_LAYOUT_BUNDLE     SoAoS: directions grouped in bundles of equal
 *                         (c_y, c_z) (one stencil row each); cell-major
 *                         inside a bundle.
 *   LBM_LAYOUT_COLLISION  AoS: the 19 populations of a cell are contiguous.
 *   LBM_LAYOUT_COMPACT    fluid cells only, in cell order, in blocks of 64
 *                         cells that each hold the cells' 19 planes side by
 *                         side (AoSoA): population q of the i-th fluid cell
 *                         at element (i / 64) * 19 * 64 + P(q) * 64 + i % 64,
 *                         with the planes of opposite directions adjacent:
 *                         P(q) = 2q for q < 9, 2(18 - q) + 1 for q > 9,
 *                         P(9) = 18.  The blocks fill 19 * S elements, S = the
 *                         fluid count rounded up to 64.  Needs a workspace
 *                         (lbm_set_workspace) for its neighbour tables; in
 *                         porous media it moves only fluid bytes.  Limit
 *                         (else LBM_ERR_UNSUPPORTED): 4 (nx+2)(ny+2)(nz+2) <
 *                         2^32 (32-bit offsets into the neighbour table).
 *                         ESOPULL keeps the bounce-back values of its
 *                         neighbour-side links after the 19 S elements, one slot
 *                         per link packed in cell order (9 more planes of
 *                         room, 4 workspace bytes more per cell).
 *
 * Conventions shared by every entry point:
 *  - Cell index: cell = x + nx * (y + ny * z), N = nx * ny * nz.
 *  - Canonical direction order q = 0..18: the vectors of {-1,0,1}^3 with
 *    |c|^2 <= 2 in lexicographic order over (c_z, c_y, c_x); q = 9 is rest
 *    and opposite(q) = 18 - q.
 *  - "Canonical populations" f[19][N] (direction-major) are the
 *    pre-collision populations f(t) of Eq. 1 at the current time t, whatever
 *    the scheme stores internally.
 *  - T is float for LBM_F32 and double for LBM_F64.
 *  - Every pointer handed to the library is a device pointer on the current
 *    HIP device; the caller allocates and owns all device memory and keeps it
 *    alive while a handle refers to it.  The library never allocates or frees
 *    device memory.
 *  - All GPU work is enqueued on the handle's stream; no call blocks the host.
 *    Launch failures are reported as LBM_ERR_HIP; faults inside a kernel
 *    surface at the caller's next synchronisation of that stream.
 *  - Argument and state errors are detected on the host before anything is
 *    enqueued; on error nothing is enqueued and the handle is unchanged.
 *  - Nothing is printed.  One handle must not be used from two threads at once.
 */
#ifndef LBM_H
#define LBM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t lbm_status;
#define LBM_OK 0
#define LBM_ERR_INVALID_ARGUMENT (-1) /* bad pointer, size, enum, tau, force, n */
#define LBM_ERR_UNSUPPORTED (-2)      /* valid request outside what is built (e.g. N >= 2^31) */
#define LBM_ERR_BAD_STATE (-3)        /* call out of order (step before init, ...) */
#define LBM_ERR_MISALIGNED (-4)       /* population buffer not 256-byte aligned */
#define LBM_ERR_HIP (-5)              /* the HIP runtime refused a launch */

#define LBM_F32 0
#define LBM_F64 1

#define LBM_LAYOUT_STREAM 0
#define LBM_LAYOUT_BUNDLE 1
#define LBM_LAYOUT_COLLISION 2
#define LBM_LAYOUT_COMPACT 3

#define LBM_SCHEME_AB 0
#define LBM_SCHEME_AA 1
#define LBM_SCHEME_ESOPULL 2
#define LBM_SCHEME_ESOTWIST 3

typedef struct lbm_desc {
    int64_t nx, ny, nz;  /* box size in cells, each >= 1 */
    int32_t precision;   /* LBM_F32 or LBM_F64 */
    int32_t layout;      /* LBM_LAYOUT_* */
    int32_t scheme;      /* LBM_SCHEME_* */
    int32_t reserved;    /* must be 0 */
    double tau;          /* BGK relaxation time, > 1/2; +INFINITY means omega = 0
                            (collision-free: steps only stream and bounce back) */
    double force[3];     /* constant body-force density (Guo forcing); zeros = off */
} lbm_desc;

typedef struct lbm_sim lbm_sim; /* opaque handle (host memory only) */

/* Size of one population buffer, 19 * N * sizeof(T) bytes (compact layout:
 * 19 * roundup(N, 64) * sizeof(T), room for an all-fluid box; 28 planes
 * instead of 19 for the compact esoteric pull; for the esoteric twist
 * (nx+1)(ny+1)(nz+1) cells per plane instead of N, rounded up to 64 on the
 * compact layout), and how many the scheme needs (2 for AB; 1 for AA,
 * ESOPULL and ESOTWIST, the in-place schemes of PortLBM section 3.3).  Host
 * only; never touches the GPU. */
lbm_status lbm_buffer_bytes(const lbm_desc *desc, size_t *bytes_per_buffer, int32_t *n_buffers);

/* Device workspace the layout needs for geometry tables: 0 for the dense
 * layouts; for LBM_LAYOUT_COMPACT about 4 bytes per cell of the box padded by
 * one halo layer plus 8 bytes per cell (index tables).  Host only. */
lbm_status lbm_workspace_bytes(const lbm_desc *desc, size_t *bytes);

/* Create a handle over caller-owned population memory: one lattice of 19
 * populations per cell for the in-place schemes, two for the two-lattice
 * pull (PortLBM section 3.3, Eq. 3, and its four algorithms; fieldcraft
 * page, first section: one buffer in place against two buffers).
 *   buf0, buf1   device buffers of lbm_buffer_bytes() bytes each, 256-byte
 *                aligned.  AB needs both (distinct, not overlapping); AA
 *                takes buf0 and requires buf1 == NULL.
 *   hip_stream   hipStream_t to enqueue on; NULL = the null stream.
 * The new handle has no geometry (all fluid, fully periodic) and is not
 * initialised.  Host only. */
lbm_status lbm_create(const lbm_desc *desc, void *buf0, void *buf1, void *hip_stream,
                      lbm_sim **out);

/* Attach caller-owned device workspace (256-byte aligned, at least
 * lbm_workspace_bytes() bytes; NULL detaches).  The library writes its
 * geometry tables there at lbm_init_equilibrium and reads them every step;
 * it must stay alive and untouched.  Invalidates the state (re-init).
 * Host only. */
lbm_status lbm_set_workspace(lbm_sim *sim, void *ws, size_t bytes);

/* Solid mask and boundary kind per axis (PortLBM section 3.1, halfway bounce-back).
 *   mask       device uint8[N], 0 = fluid, nonzero = solid; NULL = no solids.
 *              Read by every later step; must stay alive and unchanged.
 *   periodic   host int32[3] for x, y, z: 1 = periodic, 0 = halfway
 *              bounce-back wall half a cell beyond both faces of that axis.
 * Invalidates the state: lbm_init_equilibrium must be called again.  Host only. */
lbm_status lbm_set_geometry(lbm_sim *sim, const uint8_t *mask, const int32_t periodic[3]);

/* Kinds of open face (the values of lbm_set_open_faces' open[k]).  PortLBM
 * page, section 3.1, boundary paragraph: the inlet takes the equilibrium
 * distribution of Dirichlet or Neumann values, the outlet an adapted Zou-He
 * condition.  Each sets the populations entering the box through the face:
 *   LBM_FACE_EQUILIBRIUM      feq(rho[k], u[k]): a reservoir (Dirichlet);
 *   LBM_FACE_NEUMANN          feq of the density and velocity of the cell one
 *                             layer inward along the face normal, at the same
 *                             time (zero normal gradient); feq(rho[k], u[k])
 *                             where that cell is solid;
 *   LBM_FACE_ZOU_HE_PRESSURE  Zou and He (Phys. Fluids 9, 1591, 1997):
 *                             density rho[k] and the tangential components of
 *                             u[k]; the normal velocity follows from mass;
 *   LBM_FACE_ZOU_HE_VELOCITY  Zou-He with velocity u[k]; the density follows
 *                             from mass (rho[k] unused).
 * The Zou-He kinds take each entering population from its opposite by
 * non-equilibrium bounce-back with the transverse momentum correction of the
 * 3-D lattice (Hecht and Harting, J. Stat. Mech. 2010, P01018), the momentum
 * being rho u - F/2 under a body force, so that a face cell's density
 * (pressure) or velocity (velocity) and its tangential momentum are exactly the
 * prescribed ones. */
typedef enum {
    LBM_FACE_CLOSED = 0,
    LBM_FACE_EQUILIBRIUM = 1,
    LBM_FACE_NEUMANN = 2,
    LBM_FACE_ZOU_HE_PRESSURE = 3,
    LBM_FACE_ZOU_HE_VELOCITY = 4
} lbm_face_kind;

/* Open faces.  Faces are numbered -x, +x, -y, +y, -z, +z.  open[k] != 0
 * replaces the wall beyond face k, whose axis must be non-periodic, by an
 * open boundary of kind open[k] (lbm_face_kind): populations leaving through
 * it are dropped, and those entering through it are set by its kind.  Where a
 * link crosses two faces (an edge of the box), a wall wins over an open face,
 * and of two open faces the one on the first axis in x, y, z order is used.
 * The entering populations of the state always obey the faces' kinds:
 * lbm_init_equilibrium and lbm_write_populations apply them to what they
 * store (lbm_load_state stores its input as it is), and every step applies
 * them to the state it leaves (the kinds other than EQUILIBRIUM by a pass over
 * the face's cells after the step).  Bounce-back links to solid cells and
 * walls are unchanged; links through open faces carry no momentum-exchange
 * force.
 *   open   host int32[6], lbm_face_kind values.
 *   rho    host double[6] (> 0 where open), u host double[18]; read only
 *          where open[k] != 0 (may be NULL when no face is open).
 * lbm_set_geometry resets all faces to closed.  Invalidates the state.
 * LBM_ERR_INVALID_ARGUMENT for an open face on a periodic axis, an unknown
 * kind, a non-finite or non-positive rho or non-finite u, or a
 * ZOU_HE_VELOCITY face whose inward velocity component is >= 1;
 * LBM_ERR_UNSUPPORTED if a kind other than EQUILIBRIUM is used while open
 * faces lie on more than one axis or the box is less than 3 cells long on
 * their axis.  Host only. */
lbm_status lbm_set_open_faces(lbm_sim *sim, const int32_t open[6], const double rho[6], const double u[18]);

/* f(0) = equilibrium(rho, u) on fluid cells, 0 on solid cells; t := 0.  The
 * equilibrium is PortLBM section 3.1, Eq. 2 in its compressible form
 * w_q rho (1 + 3 c_q.u + 9/2 (c_q.u)^2 - 3/2 u^2) with the D3Q19 weights.
 *   rho   device T[N] or NULL (rho = 1).
 *   u     device T[3][N] (component-major) or NULL (u = 0).
 * AB stores the streaming pre-image of f(0) in buf0, so that the first fused
 * pull-collide step acts on f(0) itself.  LBM_LAYOUT_COMPACT first builds its
 * neighbour tables from the mask and the periodic flags in the workspace
 * (LBM_ERR_BAD_STATE without one) and then waits once on the stream to learn
 * the fluid-cell count: the only call that blocks the host. */
lbm_status lbm_init_equilibrium(lbm_sim *sim, const void *rho, const void *u);

/* Advance n >= 0 time steps (one fused kernel launch each, plus one small
 * launch per open face of a NEUMANN or ZOU_HE kind); t += n.  Each step is
 * f(t+1) = S(C(f(t))): C is the BGK collision of PortLBM section 3.1, Eq. 1
 * (relaxation with omega = 1/tau toward Eq. 2's equilibrium, plus the Guo
 * forcing term (1 - omega/2) w_q [3 (c_q - u) + 9 (c_q.u) c_q] . F when a
 * force is set), S the streaming of section 3.3, Eq. 3, with halfway
 * bounce-back (section 3.1, last paragraph); gather and scatter follow the
 * scheme's address rule (fieldcraft page, first section, for AA).
 * LBM_ERR_INVALID_ARGUMENT for n < 0; LBM_ERR_BAD_STATE before init. */
lbm_status lbm_step(lbm_sim *sim, int64_t n);

/* Advance n >= 1 time steps like lbm_step; the last step also writes the
 * density and velocity its collision uses, i.e. the moments of f(t + n - 1),
 * t the time before the call (the fused macroscopic output of the PortLBM
 * page, section 5.2: its combined kernel writes four macroscopic values per
 * update besides the populations; here 4 sizeof(T) bytes more per cell on
 * the last step instead of a separate pass over the state).
 *   rho   device T[N], u device T[3][N] (component-major, u includes F/2);
 *         0 on solid cells.  The values equal what lbm_moments returns
 *         before the last step, bit for bit.
 * On the compact layout each wave of the last step writes its whole range of
 * box cells (from its first fluid cell to the next wave's) in chunks of 64
 * consecutive cells: the fluid cells' values, moved by a cross-lane shuffle
 * from the lanes that computed them, and zeros at the solid cells between
 * them; the step's first and last waves also cover the solid cells before
 * the first and after the last fluid cell.  Only a box without any fluid
 * cell gets a separate pass that writes zeros.  LBM_ERR_INVALID_ARGUMENT for
 * n < 1 or NULL outputs. */
lbm_status lbm_step_moments(lbm_sim *sim, int64_t n, void *rho, void *u);

/* Density and velocity of the canonical state f(t) (PortLBM section 3.1: the
 * macroscopic velocity is the first moment of the populations; with Guo
 * forcing it includes half the force):
 * rho = sum_q f_q, u = (sum_q c_q f_q + F/2) / rho; 0 on solid cells.
 *   rho   device T[N];   u   device T[3][N] (component-major). */
lbm_status lbm_moments(lbm_sim *sim, void *rho, void *u);

/* Copy the canonical populations f(t) into device T[19][N]; 0 on solid cells. */
lbm_status lbm_read_populations(lbm_sim *sim, void *f);

/* Replace the state by canonical populations f (device T[19][N]) at the
 * current t (checkpoint restore).  Values on solid cells are ignored.
 * Internally populations are stored shifted by their lattice weights
 * (f_q - w_q); a write/read round trip returns f bit for bit when every f_q
 * lies within a factor of two of w_q (any state with |u| below ~0.15), and
 * otherwise within one unit in the last place of max(|f_q|, w_q). */
lbm_status lbm_write_populations(lbm_sim *sim, const void *f);

/* Exact checkpoint: copy out (save) or replace (load) the stored state,
 * device T[19][N] in canonical order holding f_q - w_q (the populations minus
 * their lattice weights, the form the kernels keep); 0 on solid cells for
 * save, ignored there for load.  save followed by load restores the state bit
 * for bit, so n steps, save, load into a fresh handle, n more steps equals 2n
 * steps exactly. */
lbm_status lbm_save_state(lbm_sim *sim, void *s);
lbm_status lbm_load_state(lbm_sim *sim, const void *s);

/* Momentum exchange with the solids (fieldcraft page, first section: the
 * momentum exchange is taken over the wall links of a step).  For the step
 * that starts from the current state f(t), every population f*_q that leaves
 * a fluid cell x toward a solid cell or through a wall is bounced back at the
 * link midpoint, so the solid receives 2 f*_q c_q; f* is the post-collision
 * state of x (collision and forcing exactly as in lbm_step).  Writes
 *   force   device double[6]: the sum over links that end in a solid cell of
 *           the mask (x, y, z), then over links that leave the box through a
 *           wall, i.e. a non-periodic face that is not open (x, y, z).
 *           8-byte aligned.
 *   scratch device, 256-byte aligned, at least
 *           lbm_momentum_exchange_scratch_bytes() bytes (per-workgroup
 *           partial sums); reused by the caller freely once the call's work
 *           on the stream has completed.
 * The state and time are unchanged.  Sums are in double and in a fixed order,
 * so the result is deterministic.  With F the body force and N_f the fluid
 * cells, the fluid's momentum changes over that step by N_f F minus the two
 * forces.  LBM_ERR_BAD_STATE before init; LBM_ERR_INVALID_ARGUMENT for NULL
 * pointers or a short scratch; LBM_ERR_MISALIGNED for a misaligned buffer. */
lbm_status lbm_momentum_exchange_scratch_bytes(const lbm_desc *desc, size_t *bytes);
lbm_status lbm_momentum_exchange(lbm_sim *sim, void *force, void *scratch, size_t scratch_bytes);

/* n >= 1 steps as lbm_step, the last of which also sums its own momentum
 * exchange into force (device double[6], as lbm_momentum_exchange): the same
 * links, values and order of summation as lbm_momentum_exchange called just
 * before that last step, taken from that step's own gathers and collision
 * instead of a separate pass over the lattice (fieldcraft page, first
 * section: the force is read back from the step that bounces the
 * populations).  The state after the call equals that of lbm_step(sim, n)
 * bit for bit.  scratch as for lbm_momentum_exchange (the same size).
 * Errors as lbm_momentum_exchange, and LBM_ERR_INVALID_ARGUMENT for n < 1. */
lbm_status lbm_step_momentum_exchange(lbm_sim *sim, int64_t n, void *force, void *scratch, size_t scratch_bytes);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * lbm_step_momentum_exchange without a scratch argument.  The partial rows
 * live in a fixed array inside the library, LBM_STATIC_SCRATCH_BYTES per GPU,
 * held by every GPU the library runs on until the process ends; the call
 * allocates nothing.  Results and state equal those of
 * lbm_step_momentum_exchange bit for bit.
 *   force  device double[6], 8-byte aligned.
 * LBM_ERR_UNSUPPORTED when lbm_momentum_exchange_scratch_bytes() of the
 * handle's box exceeds LBM_STATIC_SCRATCH_BYTES (48 bytes per 256-cell tile
 * of the box: a 256^3 box needs 3 MiB and fits, a 512^3 box does not);
 * other errors as lbm_step_momentum_exchange.  Every call on one
 * GPU uses that GPU's one array: calls that overlap in time on one GPU (two
 * handles on two streams, or two host threads) race and give wrong forces;
 * serialise them.  The first call on a device looks up the array's device
 * address (hipGetSymbolAddress) with that device current. */
#define LBM_STATIC_SCRATCH_BYTES ((size_t)4 << 20)
lbm_status lbm_step_momentum_exchange_noalloc(lbm_sim *sim, int64_t n, void *force);

/* Release the handle (host memory only); NULL is a no-op.  The caller's
 * population buffers, workspace and mask are not freed (the caller owns all
 * device memory, as lbm_create states); no GPU work is enqueued, so the
 * caller may free them once the stream's enqueued steps have completed. */
lbm_status lbm_destroy(lbm_sim *sim);

/* Current time step t, or -1 for a NULL handle. */
int64_t lbm_time(const lbm_sim *sim);

/* Fluid cells counted by the compact layout's table build; -1 before init or
 * for a dense layout. */
int64_t lbm_fluid_cells(const lbm_sim *sim);

/* Name of the HIP error behind the handle's last LBM_ERR_HIP ("hipSuccess" if
 * none; "no handle" for NULL).  Static string; host only. */
const char *lbm_last_hip_error(const lbm_sim *sim);

/* Static description of a status code. */
const char *lbm_status_string(lbm_status status);

#ifdef __cplusplus
}
#endif
#endif
