/*
 * dadj.h - C ABI of the MI355X record-and-replay discrete-adjoint library
 * (libdadj.so, HIP kernels for gfx950).
 *
 * The problem (DiffEqGPU page "Using GPU-accelerated Ensembles with Automatic
 * Differentiation", ensemble examples): an ensemble of n independent initial
 * value problems y' = f(y, p_i), y(t0) = u0_i, each trajectory with its own
 * parameters p_i and initial state u0_i, one trajectory per GPU lane (gist.science
 * page "Differentiable astrophysics at scale", Methodology: per-thread
 * integration).
 *
 * The path ("GRADSOLVE: fast exact gradients for ODE ensembles on GPUs",
 * gptget.net summary, Methodology, and the evolve.pub review, Summary):
 *   1. da_record      - one adaptive solve per trajectory; the accepted step
 *                       sizes form a zero-padded fixed-length mesh.
 *   2. da_replay_grad - fixed-step replay of that mesh and its reverse sweep:
 *                       the exact discrete adjoint with the mesh held fixed
 *                       (review, Strengths: paper section 3.1; FAQ on
 *                       exactness), repeated for many passes against one record.
 *   3. da_solve_fwd   - the forward-only adaptive solve (summary, Key results).
 * plus da_replay_fwd (forward replay only) and da_mesh_sort (a replay order of
 * the trajectories by step count so that each wavefront's lanes carry similar
 * work).
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers unless marked "host"; all memory is
 *    owned by the caller.  The library allocates no device memory (except the
 *    1 KiB scratch that da_mesh_max_steps allocates and frees within the
 *    call) and keeps no state apart from a thread-local error message, the
 *    code objects of right-hand sides registered at run time
 *    (da_rhs_register) and the static device scratch of
 *    da_replay_grad_noalloc (one per GPU, with its looked-up address).
 *  - Per-trajectory arrays are component-major: element (c, i) of an array
 *    with C components lives at index c * n + i (trajectory index fastest), so
 *    a wavefront reads and writes contiguous memory.
 *  - Floating-point buffers use the problem's dtype (double or float);
 *    t0, t1, save times and tolerances are host doubles.
 *  - Argument checks run synchronously before any launch; on failure the call
 *    returns a negative da_err, launches nothing and leaves outputs untouched.
 *    Everything else is asynchronous on `stream` (a hipStream_t; NULL is the
 *    default stream).  A failed launch returns DA_EHIP.
 *  - A trajectory that fails (see da_lane_status) never fails the call; its
 *    status says why and its gradients and loss are NaN.
 *  - Outputs are overwritten, not accumulated.  Results are deterministic:
 *    the same inputs give bitwise identical outputs on the same device.
 */
#ifndef DADJ_H
#define DADJ_H

#ifndef __HIPCC_RTC__
#include <stddef.h>
#include <stdint.h>
#else  /* run-time compilation of the kernels: the runtime's own integer types */
typedef __hip_internal::int32_t int32_t;
typedef __hip_internal::int64_t int64_t;
typedef __hip_internal::uint32_t uint32_t;
typedef __hip_internal::uint64_t uint64_t;
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DA_F64 = 0, DA_F32 = 1 } da_dtype;

/* Integrators: explicit Tsitouras 5(4) and Dormand-Prince 5(4) (both 7
 * stages, first-same-as-last, 5th-order solution propagated), the
 * second-order Rosenbrock method ROS2 with gamma = 1 + 1/sqrt(2) (summary,
 * Abstract: explicit and Rosenbrock integrators), and Rodas3, a third-order,
 * stiffly accurate, L-stable Rosenbrock method (four stages, embedded
 * second-order estimate, gamma = 1/2; Sandu et al. 1997) for stiff problems
 * at tight tolerances.  The Rosenbrock methods take systems of dimension
 * <= 3 and the eight-species kinetics system, and no dense output
 * (DA_EUNSUPPORTED).  DA_RKF78 is Fehlberg's 7(8) pair (13 stages, the
 * 7th-order solution propagated, its difference to the 8th-order one the
 * error estimate; Fehlberg 1968), the higher-order explicit method for
 * tight tolerances: linear, Lorenz-63 and Robertson, no dense output.
 * DA_ROS4 is a fourth-order Rosenbrock method with an embedded third-order
 * solution (four stages, gamma = 1/2, A-stable, stability function 1/3 at
 * infinity; Shampine 1982, ACM TOMS 8:93): the same systems and limits as
 * Rodas3, and one order more for stiff problems at tight tolerances. */
typedef enum {
  DA_TSIT5 = 0,
  DA_DOPRI5 = 1,
  DA_ROS2 = 2,
  DA_RODAS3 = 3,
  DA_RKF78 = 4,
  DA_ROS4 = 5
} da_method;

/* Built-in right-hand sides (dimension d, parameter count P):
 *  DA_RHS_LINEAR    d=1, P=1: y' = p0 y
 *  DA_RHS_LORENZ63  d=3, P=3: (s (y2-y1), y1 (r-y3) - y2, y1 y2 - b y3),
 *                   p = (s, r, b) (DiffEqGPU page, forward-mode example)
 *  DA_RHS_ROBERTSON d=3, P=3: (-k1 y1 + k3 y2 y3, k1 y1 - k2 y2^2 - k3 y2 y3,
 *                   k2 y2^2), p = (k1, k2, k3)
 *  DA_RHS_LORENZ96  4<=d<=64, P=1: x_i' = (x_{i+1} - x_{i-2}) x_{i-1} - x_i + F,
 *                   indices cyclic, p = (F).  Explicit methods only.
 *  DA_RHS_KINETICS8 d=8, P=4: an eight-species mass-action reaction cycle,
 *                   a synthetic stiff system of the size of the HIRES test
 *                   problem; nine reactions, each moving one unit of mass
 *                   (sum y_i is conserved), with rates
 *                   p0 y0 (y0->y1), p1 y1^2 (y1->y2), p2 y1 y2 (y1->y0),
 *                   p3 y2 (y2->y3), 10 p3 y3 (y3->y4), 1e-3 p1 y4^2 (y4->y5),
 *                   25 p0 y5 (y5->y6), 0.1 p2 y6 y2 (y6->y7), 0.01 p3 y7
 *                   (y7->y0).  Rosenbrock methods only.                   */
typedef enum {
  DA_RHS_LINEAR = 0,
  DA_RHS_LORENZ63 = 1,
  DA_RHS_ROBERTSON = 2,
  DA_RHS_LORENZ96 = 3,
  DA_RHS_KINETICS8 = 4
} da_rhs;

/* Identifiers of right-hand sides registered at run time (da_rhs_register)
 * start here. */
#define DA_RHS_USER_BASE 1024

typedef enum {
  DA_OK = 0,
  DA_EINVAL = -1,       /* invalid argument                                 */
  DA_EUNSUPPORTED = -2, /* valid but not implemented (e.g. ROS2 on LORENZ96) */
  DA_EHIP = -3,         /* a HIP call or kernel launch failed               */
  DA_EWORKSPACE = -4    /* workspace too small                              */
} da_err;

/* Per-trajectory outcome of a record (or forward solve). */
typedef enum {
  DA_LANE_OK = 0,
  DA_LANE_MAX_STEPS = 1,    /* max_steps accepted steps did not reach t1     */
  DA_LANE_DT_UNDERFLOW = 2, /* the step no longer advances t                 */
  DA_LANE_NONFINITE = 3,    /* u0 or p holds a NaN or infinity               */
  DA_LANE_MAX_ATTEMPTS = 4  /* max_attempts step attempts did not reach t1   */
} da_lane_status;

#define DA_MAX_SAVES 128

/* Problem and solver options.  Zero for dt0, max_attempts, safety, fac_min,
 * fac_max selects the default: Hairer-Norsett-Wanner starting step,
 * 4*max_steps attempts, 0.9, 0.2, 10.
 * Adaptive control (record and forward solve): error norm = RMS over
 * components of err / (atol + rtol max(|y_n|, |y_{n+1}|)); accept iff it is
 * <= 1; next step = used step * clamp(safety E^(-1/(q+1)), fac_min, fac_max)
 * with q the embedded order (4 for the 5(4) pairs, 1 for ROS2, 2 for
 * Rodas3, 3 for DA_ROS4, 7 for Fehlberg 7(8)), no growth
 * on the step after a rejection.  Steps are shortened to land exactly on each
 * save time and on t1, or, with dense = 1, on t1 only, each save time then
 * being read from the interpolant of the accepted step that contains it
 * (see da_mesh.save_theta). */
typedef struct {
  int32_t rhs;         /* da_rhs                                              */
  int32_t dim;         /* state dimension d                                   */
  int32_t n_params;    /* parameter count P                                   */
  int32_t method;      /* da_method                                           */
  int32_t dtype;       /* da_dtype of every floating buffer                   */
  double t0, t1;       /* integration interval, t1 > t0                       */
  double rtol, atol;   /* >= 0, rtol + atol > 0                               */
  double dt0;          /* > 0: first trial step; <= 0: automatic              */
  int32_t max_steps;   /* mesh length = largest number of accepted steps      */
  int32_t max_attempts;
  int32_t n_save;      /* 0..DA_MAX_SAVES; 0 = the final state is the only save */
  const double *save_times; /* host, n_save values strictly increasing in (t0, t1] */
  double safety, fac_min, fac_max;
  int32_t checkpoint;  /* reverse sweep of da_replay_grad: the forward replay
                          keeps every checkpoint-th state in the workspace and
                          the sweep recomputes the states in between in
                          registers; 1 = keep every state; 0 = the library's
                          choice: on built-in systems of up to four
                          components (not Lorenz-96) without dense output,
                          when n_save = 0: in FP64 4 for ROS2 and 2 for
                          Tsit5, Dopri5, Rodas3 and DA_ROS4, in FP32 4 for
                          all five; when n_save > 0, 2 for ROS2 in FP64;
                          else 1.
                          1, 2, 4 or 8 (or 0).  The result does not depend
                          on it.                                             */
  int32_t dense;       /* 0: steps land on the save times.  1: dense output
                          ("Differentiable astrophysics at scale",
                          Methodology: the solution is interpolated at the
                          observation times instead of ending steps there).
                          The page names no interpolant; this library uses
                          the cubic Hermite interpolant of the accepted step
                          [t_k, t_k + h] through y_k, y_{k+1} and the slopes
                          f(y_k), f(y_{k+1}) (the step's first and last stage
                          derivatives):
                            y(t_k + th h) = H00 y_k + H01 y_{k+1}
                                          + h (H10 f(y_k) + H11 f(y_{k+1})),
                            H00 = (1-th)^2 (1+2th), H01 = th^2 (3-2th),
                            H10 = th (1-th)^2,      H11 = -th^2 (1-th).
                          Save time t_s belongs to the step with
                          t_k < t_s <= t_k + h; th = (t_s - t_k) / h in double,
                          capped at 1, exactly 1 at the step's end.  th is part
                          of the mesh and, like h, carries no derivative.
                          Explicit methods only (DA_EUNSUPPORTED with ROS2,
                          Rodas3 and DA_ROS4).  */
} da_problem;

/* The record: one zero-padded step mesh per trajectory, reused by every
 * replay until the next record.  S = max(1, n_save) save slots.  Every array
 * is in trajectory order.
 *
 * The step log is tiled so that each trajectory owns 128-byte chunks of B
 * consecutive steps, B = 16 (F64) or 32 (F32), and a wavefront's chunks are
 * adjacent: step k of trajectory i is element ((k / B) * n + i) * B + k % B,
 * for k < T * B with T = ceil(max_steps / B) chunks.  Steps at and after
 * n_steps[i] are zero (a zero step leaves the state unchanged).  h must be
 * 128-byte aligned; da_mesh_h_elems gives its length.
 *
 * perm is a replay order: NULL replays trajectory j on lane j; otherwise lane
 * j replays trajectory perm[j] (da_mesh_sort makes one).  It only schedules
 * work: inputs and outputs stay in trajectory order and results do not
 * depend on it.  da_record neither reads nor writes it.
 *
 * h_rows is an optional replay table, the same step sizes laid out for the
 * replay: row k holds step k of the trajectory of every lane,
 * h_rows[k * n + j] = step k of trajectory perm[j] (of j without perm), zero
 * at and after its n_steps, for k < rows.  A wavefront then reads one
 * contiguous row segment per step.  da_mesh_sort fills it; the replays read
 * it instead of h when it is not NULL, and report a trajectory with more than
 * `rows` steps as failed (NaN outputs). */
typedef struct {
  void *h;           /* [T][n][B] accepted step sizes, zero padded            */
  int32_t *n_steps;  /* [n] accepted steps                                    */
  int32_t *save_idx; /* [S][n] mesh index k at which save time s is reached
                        (the state after k steps; with dense output, the end
                        of the step that contains it); -1 if never reached   */
  int32_t *status;   /* [n] da_lane_status                                    */
  int32_t *perm;     /* [n] lane -> trajectory replay order, or NULL          */
  void *h_rows;      /* [rows][n] replay table, or NULL                       */
  int32_t rows;      /* rows of h_rows (1..max_steps when h_rows is set)      */
  void *save_theta;  /* [S][n] (problem dtype) step fraction of each save:
                        with dense output save s is read from step
                        save_idx[s] - 1 at fraction save_theta[s]; without it
                        every reached save has fraction 1.  Written by
                        da_record when not NULL; required by da_record and by
                        the replays of a problem with dense = 1 (a replay
                        gradient with the final-state loss reads no save and
                        does not need it).                                   */
  int32_t defer_pad; /* 1: da_record writes each trajectory's chunks only up to
                        the one holding its last step (zero after that step)
                        and leaves the later chunks as they are;
                        da_mesh_pad then writes their zeros, on any stream,
                        after the record.  The replays, the sensitivities and
                        da_mesh_sort read no chunk past a trajectory's last
                        step, so they need not wait for it.  0: da_record
                        writes the zeros itself.                             */
  int32_t *n_attempts; /* [n] trial steps of the record (accepted + rejected:
                        rejections = n_attempts - n_steps), written by
                        da_record when not NULL; the replays do not read
                        it.  The record statistics the review's Strengths
                        quote (Table 5: step counts across the ensemble)
                        come from n_steps and this.                          */
} da_mesh;

/* Elements (of the problem's dtype) of the step log of n trajectories:
 * T * n * B.  0 for a NULL problem or n <= 0. */
int64_t da_mesh_h_elems(const da_problem *prob, int64_t n);

/* Scalar loss of the replayed states; the gradient is of the sum over
 * trajectories, i.e. per trajectory of its own term:
 *  DA_LOSS_SUMSQ_FINAL: L_i = scale * sum_c y_{N_i}[c]^2 (final state)
 *  DA_LOSS_MSE_SAVE:    L_i = scale * sum_s sum_c (y_{idx_s}[c] - aux[s][c][i])^2
 *  DA_LOSS_COTANGENT:   L_i = scale * sum_s sum_c aux[s][c][i] * y_{idx_s}[c]
 * aux is [S][d][n] in trajectory order (NULL for SUMSQ_FINAL).  y_{idx_s} is
 * the save s (with dense output the interpolated state).  The MSE of the
 * calibration workload uses scale = 1 / (n S d). */
typedef enum {
  DA_LOSS_SUMSQ_FINAL = 0,
  DA_LOSS_MSE_SAVE = 1,
  DA_LOSS_COTANGENT = 2
} da_loss_kind;

typedef struct {
  int32_t kind;      /* da_loss_kind */
  const void *aux;   /* device [S][d][n] or NULL */
  double scale;
} da_loss;

/* Record: one adaptive solve per trajectory (summary, Methodology: record the
 * accepted steps; review, Summary: zero-padded fixed-length mesh).
 * u0 [d][n], p [P][n]; fills mesh->h (every chunk, padding included),
 * n_steps, save_idx, status and save_theta (when not NULL; required with
 * dense output), and, if y_save is not NULL, y_save [S][d][n] with the state
 * at each save time (NaN where not reached). */
int da_record(const da_problem *prob, int64_t n, const void *u0, const void *p,
              da_mesh *mesh, void *y_save, void *stream);

/* Forward-only adaptive solve (summary, Key results: the forward kernel):
 * the same integration as da_record without the mesh.  y_save [S][d][n],
 * n_steps [n] and status [n] (either may be NULL). */
int da_solve_fwd(const da_problem *prob, int64_t n, const void *u0, const void *p,
                 void *y_save, int32_t *n_steps, int32_t *status, void *stream);

/* Lane ordering: fills mesh->perm (required, [n]) with the trajectories in
 * order of decreasing n_steps; equal counts keep their index order, so the
 * order is deterministic.  Replaying in this order gives each wavefront
 * lanes of nearly equal step counts (the GRADSOLVE review, Strengths, quotes
 * the paper's Table 5: max/mean step count 1.33-1.34 across an ensemble).
 * When mesh->h_rows is not NULL it also writes the replay table in that
 * order (mesh->rows rows; da_mesh_max_steps gives the smallest that holds
 * every trajectory).  Reads n_steps and h.  Work space of
 * da_mesh_sort_workspace bytes is required. */
size_t da_mesh_sort_workspace(const da_problem *prob, int64_t n);
int da_mesh_sort(const da_problem *prob, int64_t n, da_mesh *mesh, void *workspace,
                 size_t ws_bytes, void *stream);

/* Zero padding of a record taken with mesh->defer_pad = 1: writes zeros to
 * every chunk after the one that holds each trajectory's last step (reads
 * n_steps, writes h).  Asynchronous on stream, which must be ordered after
 * the record. */
int da_mesh_pad(const da_problem *prob, int64_t n, const da_mesh *mesh, void *stream);

/* Largest n_steps over the mesh, returned to the host (synchronises the
 * stream; allocates and frees a 1 KiB device scratch buffer).  Used to size
 * the replay workspace. */
int da_mesh_max_steps(int64_t n, const da_mesh *mesh, int32_t *host_max, void *stream);

/* Fixed-step replay of the mesh (review, Summary: branch-free fixed-length
 * chain): y_save [S][d][n] at each save index (with dense output, the
 * interpolant at the save's fraction); reproduces the record's saves bit for
 * bit. */
int da_replay_fwd(const da_problem *prob, int64_t n, const void *u0, const void *p,
                  const da_mesh *mesh, void *y_save, void *stream);

/* Replay plus reverse sweep through the replayed stages, mesh held fixed:
 * exact gradient of the loss with respect to every trajectory's u0 and p
 * (review, Strengths and FAQ).  Outputs (each may be NULL): loss_out [n],
 * grad_u0 [d][n], grad_p [P][n].  Checkpoint states of the forward replay
 * (see da_problem.checkpoint) are kept in the workspace;
 * da_replay_grad_workspace gives the size for all n trajectories at once
 * given max_n_steps, an upper bound of n_steps over the trajectories (the
 * trajectories above it are reported as failed, NaN).  A smaller workspace
 * (at least enough for 256 trajectories) makes the call process the
 * ensemble in consecutive chunks; less returns DA_EWORKSPACE. */
size_t da_replay_grad_workspace(const da_problem *prob, int64_t n, int32_t max_n_steps);
/* The checkpoint interval da_replay_grad uses for this problem: its
 * checkpoint field, or the library's choice when that is 0; 0 for a NULL
 * problem or an interval other than 0, 1, 2, 4, 8. */
int32_t da_checkpoint_interval(const da_problem *prob);
int da_replay_grad(const da_problem *prob, int64_t n, const void *u0, const void *p,
                   const da_mesh *mesh, const da_loss *loss, void *loss_out,
                   void *grad_u0, void *grad_p, int32_t max_n_steps, void *workspace,
                   size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory at call time (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * da_replay_grad with its workspace taken from a static device scratch of
 * DA_NOALLOC_SCRATCH_BYTES bytes instead of a caller buffer.  Same arguments,
 * kernels and results as da_replay_grad (bit for bit); the call allocates
 * nothing.  The ensemble is processed in consecutive chunks of as many
 * trajectories as the scratch holds (a multiple of 256); when it holds fewer
 * than 256 trajectories of max_n_steps steps (about 10900 steps of a
 * three-component FP64 system at checkpoint interval 1) the call returns
 * DA_EWORKSPACE before any launch.  The caller still owns and passes every
 * input and output.
 * Each GPU holds one copy of the scratch from the first call on it until the
 * process ends; the first call on a device looks up its address, with that
 * device current (make that first call outside graph capture).  All calls on
 * one GPU share that copy: calls that overlap in time on one GPU (two
 * streams, two threads) race and must be ordered by the caller.  Nothing in
 * the scratch needs to start at zero. */
#define DA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int da_replay_grad_noalloc(const da_problem *prob, int64_t n, const void *u0, const void *p,
                           const da_mesh *mesh, const da_loss *loss, void *loss_out,
                           void *grad_u0, void *grad_p, int32_t max_n_steps, void *stream);

/* Forward-mode sensitivities of the replay, mesh held fixed: the d + P unit
 * directions (u0 components first, then parameters) are carried as tangents
 * through the same fixed-step replay as da_replay_grad ("Differentiable
 * astrophysics at scale", Methodology: forward sensitivities integrated
 * alongside the state in the per-trajectory kernel; "GRADSOLVE" review, FAQ:
 * no derivative of the step sizes).  Outputs (each may be NULL):
 * sens [S][d][d+P][n] with d y(save s)[c] / d theta_q (NaN where the save is
 * not reached); with loss not NULL, loss_out [n], grad_u0 [d][n] and
 * grad_p [P][n], the gradient of that loss by the chain rule through the
 * tangents (the same quantity as da_replay_grad computes in reverse).
 * Needs no workspace.  Every method (for the Rosenbrock methods the tangents
 * run through the Jacobian, the LU factors with the pivots of the values,
 * and every solve)
 * and every right-hand side (Lorenz-96: one wavefront per trajectory, four
 * directions per lane).  Trajectories whose record failed get NaN. */
int da_replay_sens(const da_problem *prob, int64_t n, const void *u0, const void *p,
                   const da_mesh *mesh, const da_loss *loss, void *loss_out, void *grad_u0,
                   void *grad_p, void *sens, void *stream);

/* da_replay_sens restricted to the unit directions q_begin .. q_begin +
 * q_count - 1 of the d + P (u0 components first, then parameters).  Forward
 * mode costs one replay per group of directions, which is why it pays when
 * few directions are wanted ("Differentiable astrophysics at scale",
 * Methodology: forward sensitivities with respect to the parameters suit
 * problems with few parameters and many outputs): the P parameter directions
 * of a system with many state components are q_begin = d, q_count = P.
 * Outputs (each may be NULL): sens [S][d][q_count][n] with
 * d y(save s)[c] / d theta_q at q - q_begin; with loss not NULL, loss_out [n]
 * and grad [q_count][n], dL / d theta_q at q - q_begin.  Each direction's
 * values are those da_replay_sens gives for it (the directions do not
 * interact).  DA_EINVAL when the range is empty or outside [0, d + P). */
int da_replay_sens_dirs(const da_problem *prob, int64_t n, const void *u0, const void *p,
                        const da_mesh *mesh, int32_t q_begin, int32_t q_count,
                        const da_loss *loss, void *loss_out, void *grad, void *sens,
                        void *stream);

/* Right-hand side compiled at run time ("GRADSOLVE", evolve.pub review, FAQ:
 * registered right-hand sides of small dimension run in the fused kernels,
 * hand-written or translated from the caller's function).  The caller gives
 * f as C++ statements, the body of
 *     template <class T, class TY, class TP>
 *     void f(const TY *y, const TP *p, T *dy)
 * that set dy[0..dim) from y[0..dim) and p[0..n_params).  T is the number
 * type to compute in (a real or a tangent number); y and p hold numbers
 * that convert to T (for the derivatives, one of them holds plain reals), so
 * declare intermediate values as T (or auto) and do not assume y[i] or p[q]
 * is a T.  Use + - * /, constants (preferably written T(c)) and sqrt, exp,
 * log, sin, cos, tanh, pow(x, c) with a real constant c.  The library compiles the
 * record, forward solve, replay, replay-gradient and sensitivity kernels for
 * it with hipRTC, for one dtype and one explicit method (DA_TSIT5 or
 * DA_DOPRI5), and loads them on the current device.  The vector-Jacobian
 * products of the reverse sweep come from forward-mode tangent numbers run
 * through f (J_y^T v from the dim Jacobian columns, J_p^T v from the n_params
 * columns).  Registration blocks for the compilation (seconds); a source that
 * does not compile returns DA_EINVAL with the compiler's log in
 * da_last_error().  On success *rhs_id (>= DA_RHS_USER_BASE) is the da_rhs
 * value to put in da_problem.rhs, with the same dim, n_params, dtype and
 * method, on the same device (DA_EINVAL / DA_EUNSUPPORTED otherwise).  Unlike
 * the rest of the library, a registration is global state: its code object
 * stays loaded until da_rhs_release.  Registration and release must not race
 * with launches that use the same identifier.  A body heavy enough to fill
 * the gradient kernel's registers (the test source that calls every allowed
 * function, at dimension 3, is near that point) has been seen to give wrong
 * gradients at checkpoint interval 1 in trajectory order once a build of the
 * kernels made it spill more; the cause was not found.  For such a body,
 * compare the gradient with another interval or the replay order before
 * relying on it. */
typedef struct {
  int32_t dim;         /* 1..16 */
  int32_t n_params;    /* 1..16 */
  int32_t dtype;       /* da_dtype */
  int32_t method;      /* DA_TSIT5 or DA_DOPRI5 */
  const char *f_body;  /* host string, NUL-terminated */
} da_rhs_def;

int da_rhs_register(const da_rhs_def *def, int32_t *rhs_id);

/* A right-hand side compiled at run time for systems of dimension up to 64
 * ("GRADSOLVE", evolve.pub review, FAQ: registered right-hand sides up to
 * state dimension 64 run in the fused kernels) whose component i depends on
 * the components i + o (mod dim) for a few fixed offsets o: a cyclic
 * stencil, such as Lorenz-96 (offsets -2, -1, 0, 1).  They run on the
 * wavefront-per-trajectory kernels (lane i of a wavefront holds component i;
 * the neighbours move between lanes).  The caller gives component i of f as
 * C++ statements, the body of
 *     template <class T, class Y> T f(const Y &y, const T *p)
 * returning dy_i, where y(o) is the component i + o (mod dim) for a declared
 * offset o (NaN for any other), y.i is i and y.d is dim, and p holds the
 * n_params parameters; T is a real or a tangent number, with the operations
 * and functions listed for da_rhs_register.  The vector-Jacobian products
 * come from one forward pass on tangent numbers with a direction per offset
 * and per parameter: (J^T v)_i adds, in the declared offset order, the
 * products v_j df_j/dy(o) of the components j = i - o; J_p^T v sums each
 * component's terms over the wavefront.  Methods DA_TSIT5 and DA_DOPRI5,
 * FP64 and FP32, dense output, every kernel (record, forward solve, replay,
 * replay-gradient with the Lorenz-96 workspace of 64 values per stored
 * state, sensitivities).  Registration, errors, identifiers and release as
 * for da_rhs_register; DA_EINVAL for a dim outside 2..64, n_params outside
 * 1..16, or offsets that are not distinct values in [-3, 3]. */
typedef struct {
  int32_t dim;             /* 2..64 */
  int32_t n_params;        /* 1..16 */
  int32_t dtype;           /* da_dtype */
  int32_t method;          /* DA_TSIT5 or DA_DOPRI5 */
  int32_t n_offsets;       /* 1..7 */
  const int32_t *offsets;  /* host [n_offsets]: distinct, each in [-3, 3] */
  const char *f_body;      /* host string, NUL-terminated */
} da_rhs_stencil_def;

int da_rhs_register_stencil(const da_rhs_stencil_def *def, int32_t *rhs_id);
int da_rhs_release(int32_t rhs_id);

/* Message of the last non-zero return on this thread ("" if none). */
const char *da_last_error(void);

/* Library version (major*10000 + minor*100 + patch). */
int da_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DADJ_H */
