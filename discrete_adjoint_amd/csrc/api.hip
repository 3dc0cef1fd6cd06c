// C ABI of libdadj: argument checks, defaults, dispatch and error reporting.
// The operations and their sources are described in include/dadj.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "dadj.h"
#include "dadj_internal.hpp"

// Device scratch of da_replay_grad_noalloc, for callers that cannot allocate
// device memory: DA_NOALLOC_SCRATCH_BYTES bytes that every GPU the library
// runs on holds from its first use until the process ends.  Host code never
// uses this name as an address (here it is a host-side stand-in); the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[DA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[4096] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return DA_OK;
}

int hip_fail(hipError_t e, const char *what) {
  const std::string rtc = dadj::rtc_take_error();  // a registered rhs that failed to compile
  if (!rtc.empty()) return fail(DA_EHIP, "%s: %s", what, rtc.c_str());
  return fail(DA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool shape_ok(int rhs, int d, int P) {
  switch (rhs) {
    case DA_RHS_LINEAR: return d == 1 && P == 1;
    case DA_RHS_LORENZ63: return d == 3 && P == 3;
    case DA_RHS_ROBERTSON: return d == 3 && P == 3;
    case DA_RHS_LORENZ96: return d >= 4 && d <= 64 && P == 1;
    case DA_RHS_KINETICS8: return d == 8 && P == 4;
  }
  return false;
}

size_t dsize(int dtype) { return dtype == DA_F64 ? 8 : 4; }

// Values per stored state in the replay-gradient workspace: a full
// wavefront row for the wavefront kernels (Lorenz-96 and registered
// stencils), else the dimension.
int ws_row_of(int rhs, int dim) {
  if (rhs >= DA_RHS_USER_BASE) return dadj::rtc_is_stencil(rhs) ? 64 : dim;
  return dadj::ws_row(rhs, dim);
}

// Checkpoint interval of the reverse sweep when the caller leaves it to the
// library.  Every kernel family stores states and recomputes the stages from
// them (storing the stages would move 2 s d values per step through HBM
// against about s right-hand sides of recomputation, far slower for every
// built-in system); the interval trades stored states against recomputed
// steps.  The lane kernels replay the steps that every trajectory of a
// wavefront still has without per-lane guards (built-in systems of up to
// four components, intervals 1, 2 and 4, final-state loss, no dense
// output), and a segment of several steps is one block of independent work
// for the scheduler there.  Measured on MI355X, gradient pass in ms at
// intervals 1 / 2 / 4 / 8, final-state loss:
//   ROS2, Robertson (d = 3), FP64, 65536 trajectories:  13.55 / 11.43 / 10.60 / 15.69
//   Dopri5, Lorenz-63 (d = 3), FP64, 2^20:              10.56 / 9.75 / 10.10 / 11.95
//   Tsit5, Lorenz-63, FP64, 1024:                       0.0438 / 0.0419 / 0.0427 / 0.0581
//   Rodas3, Robertson:                                  0.574 / 0.509 / 0.520
//   fourth-order Rosenbrock method, Robertson:          0.526 / 0.470 / 0.496
//   Fehlberg 7(8), Lorenz-63, FP64, 2^20:               4.92 / 5.01 / 5.15 / 6.19
// and with the guarded replay (losses at save times, registered or larger
// systems):
//   ROS2, Robertson, FP64:                              16.6 / 15.4 / 15.9 / 15.8
//   Tsit5, Lorenz-63, FP32, 65536, MSE at 10 saves:     0.189 (two wavefronts) / 0.208
//   Rodas3, kinetics (d = 8), FP64, 65536:              4.04 / 5.40 / 7.44 (spills)
//   Tsit5, Lorenz-96 (d = 64, wavefront kernel), 16384: 1.23 / 1.32 / 1.37 / 1.41
// In FP32, final-state loss, intervals 1 / 2 / 4:
//   Tsit5, Lorenz-63, 65536:                            0.1066 (two wavefronts) / 0.1042 / 0.1002
//   Dopri5, Lorenz-63, 2^20:                            5.39 / 4.84 / 4.68
//   ROS2 / Rodas3 / fourth-order method, Robertson:     9.90 / 8.08 / 7.63, 0.490 / 0.420 / 0.397,
//                                                       0.448 / 0.400 / 0.386
// A problem with save times is taken to be replayed with losses at them.
// So, on built-in systems of up to four components (not the wavefront
// kernels' Lorenz-96), without dense output, with no save times: in FP64 4
// for ROS2 and 2 for Tsit5, Dopri5, Rodas3 and the fourth-order method, in
// FP32 4 for all five; with save times, 2 for ROS2 in FP64.  Everywhere else
// 1 (every state stored).
int default_checkpoint(const da_problem &pb) {
  const bool lane_builtin = pb.rhs < DA_RHS_USER_BASE && pb.rhs != DA_RHS_LORENZ96 &&
                            pb.dim <= 4 && pb.dense == 0;
  if (!lane_builtin) return 1;
  const bool f64 = pb.dtype == DA_F64;
  const bool branch_free = pb.method == DA_ROS2 || pb.method == DA_TSIT5 ||
                           pb.method == DA_DOPRI5 || pb.method == DA_RODAS3 ||
                           pb.method == DA_ROS4;
  if (pb.n_save == 0 && branch_free) return (!f64 || pb.method == DA_ROS2) ? 4 : 2;
  if (pb.method == DA_ROS2 && f64) return 2;
  return 1;
}

int resolved_checkpoint(const da_problem &pb) {
  return pb.checkpoint > 0 ? pb.checkpoint : default_checkpoint(pb);
}

// Validates the problem and resolves defaults.
int check_problem(const da_problem *pb, int64_t n, dadj::ProbArgs &pr, dadj::SaveTimes *st) {
  if (!pb) return fail(DA_EINVAL, "problem is NULL");
  if (n < 0 || n > (int64_t)0x7fffffff) return fail(DA_EINVAL, "n = %lld out of range", (long long)n);
  if (pb->dtype != DA_F64 && pb->dtype != DA_F32) return fail(DA_EINVAL, "bad dtype %d", pb->dtype);
  if (pb->method < DA_TSIT5 || pb->method > DA_ROS4)
    return fail(DA_EINVAL, "bad method %d", pb->method);
  const bool rosenbrock =
      pb->method == DA_ROS2 || pb->method == DA_RODAS3 || pb->method == DA_ROS4;
  if (pb->rhs >= DA_RHS_USER_BASE) {
    std::string msg;
    const int rc = dadj::rtc_check(*pb, msg);
    if (rc) return fail(rc, "%s", msg.c_str());
  } else {
    if (pb->rhs < DA_RHS_LINEAR || pb->rhs > DA_RHS_KINETICS8)
      return fail(DA_EINVAL, "bad rhs %d", pb->rhs);
    if (!shape_ok(pb->rhs, pb->dim, pb->n_params))
      return fail(DA_EINVAL, "rhs %d does not take dim=%d, n_params=%d", pb->rhs, pb->dim,
                  pb->n_params);
    if (pb->rhs == DA_RHS_LORENZ96 && rosenbrock)
      return fail(DA_EUNSUPPORTED,
                  "the Rosenbrock methods do not take Lorenz-96");
    if (pb->rhs == DA_RHS_KINETICS8 && !rosenbrock)
      return fail(DA_EUNSUPPORTED, "the kinetics system takes the Rosenbrock methods only");
    if (pb->rhs == DA_RHS_LORENZ96 && pb->method == DA_RKF78)
      return fail(DA_EUNSUPPORTED, "Lorenz-96 takes Tsit5 and Dopri5 only");
  }
  if (!(isfinite(pb->t0) && isfinite(pb->t1) && pb->t1 > pb->t0))
    return fail(DA_EINVAL, "need finite t0 < t1");
  if (!(pb->rtol >= 0) || !(pb->atol >= 0) || !(pb->rtol + pb->atol > 0) || !isfinite(pb->rtol) ||
      !isfinite(pb->atol))
    return fail(DA_EINVAL, "tolerances must be finite, >= 0 and not both 0");
  if (pb->max_steps < 1) return fail(DA_EINVAL, "max_steps must be >= 1");
  if (pb->max_steps > (1 << 24)) return fail(DA_EINVAL, "max_steps above 2^24");
  if (pb->n_save < 0 || pb->n_save > DA_MAX_SAVES)
    return fail(DA_EINVAL, "n_save must be in [0, %d]", DA_MAX_SAVES);
  if (pb->n_save > 0 && !pb->save_times) return fail(DA_EINVAL, "save_times is NULL");
  double prev = pb->t0;
  for (int s = 0; s < pb->n_save; ++s) {
    const double ts = pb->save_times[s];
    if (!(ts > prev) || ts > pb->t1)
      return fail(DA_EINVAL, "save_times must increase strictly within (t0, t1]");
    prev = ts;
  }
  if (!(pb->safety >= 0 && pb->fac_min >= 0 && pb->fac_max >= 0) || pb->max_attempts < 0)
    return fail(DA_EINVAL, "negative controller option");
  if (pb->checkpoint != 0 && pb->checkpoint != 1 && pb->checkpoint != 2 && pb->checkpoint != 4 &&
      pb->checkpoint != 8)
    return fail(DA_EINVAL, "checkpoint must be 0, 1, 2, 4 or 8");
  if (pb->dense != 0 && pb->dense != 1) return fail(DA_EINVAL, "dense must be 0 or 1");
  if (pb->dense && (rosenbrock || pb->method == DA_RKF78))
    return fail(DA_EUNSUPPORTED, "dense output is available for Tsit5 and Dopri5");
  pr.rhs = pb->rhs;
  pr.dim = pb->dim;
  pr.n_params = pb->n_params;
  pr.method = pb->method;
  pr.dtype = pb->dtype;
  pr.max_steps = pb->max_steps;
  pr.max_attempts = pb->max_attempts > 0 ? pb->max_attempts : 4 * pb->max_steps;
  pr.n_save = pb->n_save;
  pr.S = pb->n_save > 0 ? pb->n_save : 1;
  pr.t0 = pb->t0;
  pr.t1 = pb->t1;
  pr.rtol = pb->rtol;
  pr.atol = pb->atol;
  pr.dt0 = pb->dt0;
  pr.safety = pb->safety > 0 ? pb->safety : 0.9;
  pr.fac_min = pb->fac_min > 0 ? pb->fac_min : 0.2;
  pr.fac_max = pb->fac_max > 0 ? pb->fac_max : 10.0;
  const int B = dadj::chunk_steps(pb->dtype);
  pr.n_chunks = (pb->max_steps + B - 1) / B;
  pr.checkpoint = pb->checkpoint > 0 ? pb->checkpoint : default_checkpoint(*pb);
  pr.dense = pb->dense;
  if (st) {
    memset(st, 0, sizeof *st);
    for (int s = 0; s < pb->n_save; ++s) st->t[s] = pb->save_times[s];
  }
  return DA_OK;
}

int check_mesh(const da_mesh *m, bool need_status, int32_t max_steps) {
  if (!m) return fail(DA_EINVAL, "mesh is NULL");
  if (!m->h || !m->n_steps || !m->save_idx || (need_status && !m->status))
    return fail(DA_EINVAL, "mesh arrays must not be NULL");
  if ((uintptr_t)m->h % dadj::CHUNK_BYTES != 0)
    return fail(DA_EINVAL, "mesh->h must be %d-byte aligned", dadj::CHUNK_BYTES);
  if (m->h_rows && (m->rows < 1 || m->rows > max_steps))
    return fail(DA_EINVAL, "mesh->rows = %d must be in [1, max_steps] with h_rows", m->rows);
  return DA_OK;
}

void fill_replay_args(dadj::ReplayArgs &a, const dadj::ProbArgs &pr, int64_t n, const void *u0,
                      const void *p, const da_mesh *mesh) {
  memset(&a, 0, sizeof a);
  a.pr = pr;
  a.n = n;
  a.u0 = u0;
  a.p = p;
  a.h = mesh->h;
  a.h_rows = mesh->h_rows;
  a.rows = mesh->h_rows ? mesh->rows : 0;
  a.nsteps = mesh->n_steps;
  a.sidx = mesh->save_idx;
  a.status = mesh->status;
  a.perm = mesh->perm;
  a.theta = mesh->save_theta;
}

bool user_rhs(const dadj::ProbArgs &pr) { return pr.rhs >= DA_RHS_USER_BASE; }

hipError_t launch_record(const dadj::RecordArgs &a, const dadj::SaveTimes &st, hipStream_t s) {
  if (user_rhs(a.pr)) return dadj::launch_rtc_record(a, st, s);
  if (a.pr.rhs == DA_RHS_LORENZ96) return dadj::launch_l96_record(a, st, s);
  if (a.pr.method == DA_ROS2) return dadj::launch_ros2_record(a, st, s);
  if (a.pr.method == DA_RODAS3) return dadj::launch_rodas3_record(a, st, s);
  if (a.pr.method == DA_ROS4) return dadj::launch_ros4_record(a, st, s);
  if (a.pr.method == DA_RKF78) return dadj::launch_rkf78_record(a, st, s);
  return dadj::launch_erk_record(a, st, s);
}

hipError_t launch_replay_fwd(const dadj::ReplayArgs &a, hipStream_t s) {
  if (user_rhs(a.pr)) return dadj::launch_rtc_replay_fwd(a, s);
  if (a.pr.rhs == DA_RHS_LORENZ96) return dadj::launch_l96_replay_fwd(a, s);
  if (a.pr.method == DA_ROS2) return dadj::launch_ros2_replay_fwd(a, s);
  if (a.pr.method == DA_RODAS3) return dadj::launch_rodas3_replay_fwd(a, s);
  if (a.pr.method == DA_ROS4) return dadj::launch_ros4_replay_fwd(a, s);
  if (a.pr.method == DA_RKF78) return dadj::launch_rkf78_replay_fwd(a, s);
  return dadj::launch_erk_replay_fwd(a, s);
}

hipError_t launch_replay_grad(const dadj::ReplayArgs &a, hipStream_t s) {
  if (user_rhs(a.pr)) return dadj::launch_rtc_replay_grad(a, s);
  if (a.pr.rhs == DA_RHS_LORENZ96) return dadj::launch_l96_replay_grad(a, s);
  if (a.pr.method == DA_ROS2) return dadj::launch_ros2_replay_grad(a, s);
  if (a.pr.method == DA_RODAS3) return dadj::launch_rodas3_replay_grad(a, s);
  if (a.pr.method == DA_ROS4) return dadj::launch_ros4_replay_grad(a, s);
  if (a.pr.method == DA_RKF78) return dadj::launch_rkf78_replay_grad(a, s);
  return dadj::launch_erk_replay_grad(a, s);
}

}  // namespace

extern "C" {

int da_version(void) { return 100; }

int da_rhs_register(const da_rhs_def *def, int32_t *rhs_id) {
  if (!def || !rhs_id) return fail(DA_EINVAL, "def and rhs_id must not be NULL");
  if (def->dim < 1 || def->dim > 16) return fail(DA_EINVAL, "dim must be in [1, 16]");
  if (def->n_params < 1 || def->n_params > 16)
    return fail(DA_EINVAL, "n_params must be in [1, 16]");
  if (def->dtype != DA_F64 && def->dtype != DA_F32) return fail(DA_EINVAL, "bad dtype %d", def->dtype);
  if (def->method != DA_TSIT5 && def->method != DA_DOPRI5)
    return fail(DA_EUNSUPPORTED, "registered right-hand sides run the explicit methods");
  if (!def->f_body) return fail(DA_EINVAL, "f_body is NULL");
  std::string msg;
  const int rc = dadj::rtc_register(*def, rhs_id, msg);
  if (rc) return fail(rc, "%s", msg.c_str());
  return ok();
}

int da_rhs_register_stencil(const da_rhs_stencil_def *def, int32_t *rhs_id) {
  if (!def || !rhs_id) return fail(DA_EINVAL, "def and rhs_id must not be NULL");
  if (def->dim < 2 || def->dim > 64) return fail(DA_EINVAL, "dim must be in [2, 64]");
  if (def->n_params < 1 || def->n_params > 16)
    return fail(DA_EINVAL, "n_params must be in [1, 16]");
  if (def->dtype != DA_F64 && def->dtype != DA_F32) return fail(DA_EINVAL, "bad dtype %d", def->dtype);
  if (def->method != DA_TSIT5 && def->method != DA_DOPRI5)
    return fail(DA_EUNSUPPORTED, "registered right-hand sides run the explicit methods");
  if (def->n_offsets < 1 || def->n_offsets > 7 || !def->offsets)
    return fail(DA_EINVAL, "need 1 to 7 offsets");
  for (int i = 0; i < def->n_offsets; ++i) {
    const int o = def->offsets[i];
    if (o < -3 || o > 3) return fail(DA_EINVAL, "offset %d outside [-3, 3]", o);
    for (int j = 0; j < i; ++j)
      if (def->offsets[j] == o) return fail(DA_EINVAL, "offset %d given twice", o);
  }
  if (!def->f_body) return fail(DA_EINVAL, "f_body is NULL");
  std::string msg;
  const int rc = dadj::rtc_register_stencil(*def, rhs_id, msg);
  if (rc) return fail(rc, "%s", msg.c_str());
  return ok();
}

int da_rhs_release(int32_t rhs_id) {
  std::string msg;
  const int rc = dadj::rtc_release(rhs_id, msg);
  if (rc) return fail(rc, "%s", msg.c_str());
  return ok();
}

const char *da_last_error(void) { return g_err; }

int da_record(const da_problem *prob, int64_t n, const void *u0, const void *p, da_mesh *mesh,
              void *y_save, void *stream) {
  dadj::ProbArgs pr;
  dadj::SaveTimes st;
  int rc = check_problem(prob, n, pr, &st);
  if (rc) return rc;
  if (n == 0) return ok();
  if ((rc = check_mesh(mesh, true, pr.max_steps))) return rc;
  if (pr.dense && !mesh->save_theta)
    return fail(DA_EINVAL, "dense output needs mesh->save_theta");
  if (n > 0 && (!u0 || !p)) return fail(DA_EINVAL, "u0 and p must not be NULL");
  if (n == 0) return ok();
  dadj::RecordArgs a;
  a.pr = pr;
  a.n = n;
  a.u0 = u0;
  a.p = p;
  a.h = mesh->h;
  a.nsteps = mesh->n_steps;
  a.sidx = mesh->save_idx;
  a.theta = mesh->save_theta;
  a.status = mesh->status;
  a.y_save = y_save;
  a.defer_pad = mesh->defer_pad != 0;
  a.natt = mesh->n_attempts;
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = launch_record(a, st, s);
  if (e != hipSuccess) return hip_fail(e, "record launch");
  return ok();
}

int da_solve_fwd(const da_problem *prob, int64_t n, const void *u0, const void *p, void *y_save,
                 int32_t *n_steps, int32_t *status, void *stream) {
  dadj::ProbArgs pr;
  dadj::SaveTimes st;
  int rc = check_problem(prob, n, pr, &st);
  if (rc) return rc;
  if (n > 0 && (!u0 || !p)) return fail(DA_EINVAL, "u0 and p must not be NULL");
  if (n == 0) return ok();
  dadj::RecordArgs a;
  a.pr = pr;
  a.n = n;
  a.u0 = u0;
  a.p = p;
  a.h = nullptr;
  a.nsteps = n_steps;
  a.sidx = nullptr;
  a.theta = nullptr;
  a.status = status;
  a.defer_pad = 0;
  a.natt = nullptr;
  a.y_save = y_save;
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = launch_record(a, st, s);
  if (e != hipSuccess) return hip_fail(e, "solve_fwd launch");
  return ok();
}

int64_t da_mesh_h_elems(const da_problem *prob, int64_t n) {
  if (!prob || n <= 0 || prob->max_steps < 1 || (prob->dtype != DA_F64 && prob->dtype != DA_F32))
    return 0;
  const int B = dadj::chunk_steps(prob->dtype);
  return (int64_t)((prob->max_steps + B - 1) / B) * n * B;
}

size_t da_mesh_sort_workspace(const da_problem *prob, int64_t n) {
  if (!prob || n <= 0) return 0;
  return dadj::sort_workspace_bytes(n);
}

int da_mesh_sort(const da_problem *prob, int64_t n, da_mesh *mesh, void *workspace,
                 size_t ws_bytes, void *stream) {
  dadj::ProbArgs pr;
  int rc = check_problem(prob, n, pr, nullptr);
  if (rc) return rc;
  if (n == 0) return ok();
  if ((rc = check_mesh(mesh, false, pr.max_steps))) return rc;
  if (!mesh->perm) return fail(DA_EINVAL, "mesh->perm must not be NULL");
  const size_t need = dadj::sort_workspace_bytes(n);
  if (!workspace || ws_bytes < need)
    return fail(DA_EWORKSPACE, "mesh sort needs %zu bytes of workspace, got %zu", need, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dadj::launch_mesh_sort(pr, n, mesh->n_steps, mesh->perm, workspace, ws_bytes, s);
  if (e == hipSuccess && mesh->h_rows)
    e = dadj::launch_replay_table(pr, n, mesh->h, mesh->n_steps, mesh->perm, mesh->h_rows,
                                  mesh->rows, s);
  if (e != hipSuccess) return hip_fail(e, "mesh sort launch");
  return ok();
}

int da_mesh_pad(const da_problem *prob, int64_t n, const da_mesh *mesh, void *stream) {
  dadj::ProbArgs pr;
  int rc = check_problem(prob, n, pr, nullptr);
  if (rc) return rc;
  if (n == 0) return ok();
  if ((rc = check_mesh(mesh, false, pr.max_steps))) return rc;
  const hipError_t e =
      dadj::launch_mesh_pad(pr, n, mesh->n_steps, mesh->h, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mesh pad launch");
  return ok();
}

int da_mesh_max_steps(int64_t n, const da_mesh *mesh, int32_t *host_max, void *stream) {
  if (!host_max) return fail(DA_EINVAL, "host_max is NULL");
  if (n < 0) return fail(DA_EINVAL, "n < 0");
  if (n == 0) {
    *host_max = 0;
    return ok();
  }
  if (!mesh || !mesh->n_steps) return fail(DA_EINVAL, "mesh is NULL");
  hipStream_t s = (hipStream_t)stream;
  int32_t *d = nullptr;
  hipError_t e = hipMalloc((void **)&d, dadj::max_steps_scratch_ints() * sizeof(int32_t));
  if (e != hipSuccess) return hip_fail(e, "hipMalloc");
  e = dadj::launch_max_steps(n, mesh->n_steps, d, s);
  if (e == hipSuccess) e = hipMemcpyAsync(host_max, d, sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  const hipError_t e2 = hipFree(d);
  if (e != hipSuccess) return hip_fail(e, "max steps");
  if (e2 != hipSuccess) return hip_fail(e2, "hipFree");
  return ok();
}

int da_replay_fwd(const da_problem *prob, int64_t n, const void *u0, const void *p,
                  const da_mesh *mesh, void *y_save, void *stream) {
  dadj::ProbArgs pr;
  int rc = check_problem(prob, n, pr, nullptr);
  if (rc) return rc;
  if (n == 0) return ok();
  if ((rc = check_mesh(mesh, false, pr.max_steps))) return rc;
  if (n > 0 && (!u0 || !p || !y_save)) return fail(DA_EINVAL, "u0, p and y_save must not be NULL");
  if (pr.dense && !mesh->save_theta)
    return fail(DA_EINVAL, "dense output needs mesh->save_theta");
  if (n == 0) return ok();
  dadj::ReplayArgs a;
  fill_replay_args(a, pr, n, u0, p, mesh);
  a.y_save = y_save;
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = launch_replay_fwd(a, s);
  if (e != hipSuccess) return hip_fail(e, "replay_fwd launch");
  return ok();
}

int32_t da_checkpoint_interval(const da_problem *prob) {
  if (!prob || prob->checkpoint < 0 || prob->checkpoint > 8) return 0;
  const int ck = resolved_checkpoint(*prob);
  return (ck == 1 || ck == 2 || ck == 4 || ck == 8) ? ck : 0;
}

size_t da_replay_grad_workspace(const da_problem *prob, int64_t n, int32_t max_n_steps) {
  if (!prob || n <= 0 || max_n_steps <= 0 || prob->dim <= 0) return 0;
  const int ck = resolved_checkpoint(*prob);
  if (ck <= 0 || ck > 8) return 0;
  return (size_t)n * (size_t)((max_n_steps + ck - 1) / ck) *
         (size_t)ws_row_of(prob->rhs, prob->dim) * dsize(prob->dtype);
}

}  // extern "C"

namespace {

// Device address of `scratch` on each device, looked up on the device's first
// da_replay_grad_noalloc call with that device current.
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices] = {};

int noalloc_scratch(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(DA_EUNSUPPORTED, "device %d is beyond the %d devices of the scratch table", dev,
                kScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(DA_EHIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DA_OK;
}

// The replay gradient of da_replay_grad and da_replay_grad_noalloc.  With
// noalloc the workspace is the static scratch, looked up after the argument
// checks (so that they need no device), and the error raised when it holds
// fewer than one block of trajectories names the scratch.
int replay_grad(const da_problem *prob, int64_t n, const void *u0, const void *p,
                const da_mesh *mesh, const da_loss *loss, void *loss_out, void *grad_u0,
                void *grad_p, int32_t max_n_steps, void *workspace, size_t ws_bytes,
                bool noalloc, void *stream) {
  dadj::ProbArgs pr;
  int rc = check_problem(prob, n, pr, nullptr);
  if (rc) return rc;
  if (n == 0) return ok();
  if ((rc = check_mesh(mesh, true, pr.max_steps))) return rc;
  if (!loss) return fail(DA_EINVAL, "loss is NULL");
  if (loss->kind < DA_LOSS_SUMSQ_FINAL || loss->kind > DA_LOSS_COTANGENT)
    return fail(DA_EINVAL, "bad loss kind %d", loss->kind);
  if (loss->kind != DA_LOSS_SUMSQ_FINAL && !loss->aux)
    return fail(DA_EINVAL, "loss kind %d needs aux", loss->kind);
  if (!isfinite(loss->scale)) return fail(DA_EINVAL, "loss scale must be finite");
  if (pr.dense && loss->kind != DA_LOSS_SUMSQ_FINAL && !mesh->save_theta)
    return fail(DA_EINVAL, "dense output needs mesh->save_theta");
  if (max_n_steps < 0 || max_n_steps > pr.max_steps)
    return fail(DA_EINVAL, "max_n_steps must be in [0, max_steps]");
  if (n > 0 && (!u0 || !p)) return fail(DA_EINVAL, "u0 and p must not be NULL");
  if (n == 0) return ok();
  const size_t per_lane = (size_t)((max_n_steps + pr.checkpoint - 1) / pr.checkpoint) *
                          ws_row_of(pr.rhs, pr.dim) * dsize(pr.dtype);
  int64_t C = n;
  if (per_lane > 0) {
    if (noalloc) {
      const int rs = noalloc_scratch(&workspace);
      if (rs) return rs;
      ws_bytes = DA_NOALLOC_SCRATCH_BYTES;
    }
    if (!workspace) return fail(DA_EWORKSPACE, "workspace is NULL");
    const size_t fit = ws_bytes / per_lane;
    if (fit < (size_t)n) {
      C = (int64_t)(fit / dadj::BLOCK) * dadj::BLOCK;
      if (C < dadj::BLOCK && noalloc)
        return fail(DA_EWORKSPACE,
                    "da_replay_grad_noalloc: %zu bytes per trajectory (max_n_steps %d, checkpoint "
                    "interval %d) times %d trajectories exceed the %zu-byte static scratch; call "
                    "da_replay_grad with a workspace",
                    per_lane, max_n_steps, pr.checkpoint, dadj::BLOCK, ws_bytes);
      if (C < dadj::BLOCK)
        return fail(DA_EWORKSPACE, "workspace %zu bytes holds fewer than %d trajectories", ws_bytes,
                    dadj::BLOCK);
    }
  }
  dadj::ReplayArgs a;
  fill_replay_args(a, pr, n, u0, p, mesh);
  a.loss_kind = loss->kind;
  a.aux = loss->aux;
  a.scale = loss->scale;
  a.loss_out = loss_out;
  a.gu0 = grad_u0;
  a.gp = grad_p;
  a.ws = workspace;
  a.ws_lanes = C;
  a.max_n_steps = max_n_steps;
  hipStream_t s = (hipStream_t)stream;
  for (int64_t slot0 = 0; slot0 < n; slot0 += C) {
    a.slot0 = slot0;
    a.nslots = (n - slot0) < C ? (n - slot0) : C;
    const hipError_t e = launch_replay_grad(a, s);
    if (e != hipSuccess) return hip_fail(e, "replay_grad launch");
  }
  return ok();
}

}  // namespace

extern "C" {

int da_replay_grad(const da_problem *prob, int64_t n, const void *u0, const void *p,
                   const da_mesh *mesh, const da_loss *loss, void *loss_out, void *grad_u0,
                   void *grad_p, int32_t max_n_steps, void *workspace, size_t ws_bytes,
                   void *stream) {
  return replay_grad(prob, n, u0, p, mesh, loss, loss_out, grad_u0, grad_p, max_n_steps,
                     workspace, ws_bytes, false, stream);
}

int da_replay_grad_noalloc(const da_problem *prob, int64_t n, const void *u0, const void *p,
                           const da_mesh *mesh, const da_loss *loss, void *loss_out,
                           void *grad_u0, void *grad_p, int32_t max_n_steps, void *stream) {
  return replay_grad(prob, n, u0, p, mesh, loss, loss_out, grad_u0, grad_p, max_n_steps, nullptr,
                     0, true, stream);
}

// Forward-mode sensitivities along directions q_begin .. q_begin + q_count - 1
// (q_count < 0: all d + P); gq, when not null, takes the gradient of the range.
static int replay_sens(const da_problem *prob, int64_t n, const void *u0, const void *p,
                       const da_mesh *mesh, int32_t q_begin, int32_t q_count, const da_loss *loss,
                       void *loss_out, void *grad_u0, void *grad_p, void *gq, void *sens,
                       void *stream) {
  dadj::ProbArgs pr;
  int rc = check_problem(prob, n, pr, nullptr);
  if (rc) return rc;
  const int Q = pr.dim + pr.n_params;
  if (q_count < 0) {
    q_begin = 0;
    q_count = Q;
  }
  if (q_begin < 0 || q_count < 1 || q_begin > Q - q_count)
    return fail(DA_EINVAL, "direction range [%d, %d + %d) outside the %d directions", q_begin,
                q_begin, q_count, Q);
  if (n == 0) return ok();
  if ((rc = check_mesh(mesh, true, pr.max_steps))) return rc;
  if (pr.dense && (sens || (loss && loss->kind != DA_LOSS_SUMSQ_FINAL)) && !mesh->save_theta)
    return fail(DA_EINVAL, "dense output needs mesh->save_theta");
  if (loss) {
    if (loss->kind < DA_LOSS_SUMSQ_FINAL || loss->kind > DA_LOSS_COTANGENT)
      return fail(DA_EINVAL, "bad loss kind %d", loss->kind);
    if (loss->kind != DA_LOSS_SUMSQ_FINAL && !loss->aux)
      return fail(DA_EINVAL, "loss kind %d needs aux", loss->kind);
    if (!isfinite(loss->scale)) return fail(DA_EINVAL, "loss scale must be finite");
  }
  if (!u0 || !p) return fail(DA_EINVAL, "u0 and p must not be NULL");
  dadj::ReplayArgs a;
  fill_replay_args(a, pr, n, u0, p, mesh);
  a.sens = sens;
  a.q_begin = q_begin;
  a.q_count = q_count;
  a.has_loss = loss != nullptr;
  if (loss) {
    a.loss_kind = loss->kind;
    a.aux = loss->aux;
    a.scale = loss->scale;
    a.loss_out = loss_out;
    a.gu0 = grad_u0;
    a.gp = grad_p;
    a.gq = gq;
  }
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = user_rhs(pr)                   ? dadj::launch_rtc_replay_sens(a, s)
                       : pr.rhs == DA_RHS_LORENZ96   ? dadj::launch_l96_replay_sens(a, s)
                       : pr.method == DA_ROS2        ? dadj::launch_ros2_replay_sens(a, s)
                       : pr.method == DA_RODAS3      ? dadj::launch_rodas3_replay_sens(a, s)
                       : pr.method == DA_ROS4        ? dadj::launch_ros4_replay_sens(a, s)
                       : pr.method == DA_RKF78       ? dadj::launch_rkf78_replay_sens(a, s)
                                                     : dadj::launch_erk_replay_sens(a, s);
  if (e != hipSuccess) return hip_fail(e, "replay_sens launch");
  return ok();
}

int da_replay_sens(const da_problem *prob, int64_t n, const void *u0, const void *p,
                   const da_mesh *mesh, const da_loss *loss, void *loss_out, void *grad_u0,
                   void *grad_p, void *sens, void *stream) {
  return replay_sens(prob, n, u0, p, mesh, 0, -1, loss, loss_out, grad_u0, grad_p, nullptr, sens,
                     stream);
}

int da_replay_sens_dirs(const da_problem *prob, int64_t n, const void *u0, const void *p,
                        const da_mesh *mesh, int32_t q_begin, int32_t q_count,
                        const da_loss *loss, void *loss_out, void *grad, void *sens,
                        void *stream) {
  if (q_count < 1) return fail(DA_EINVAL, "q_count must be at least 1");
  return replay_sens(prob, n, u0, p, mesh, q_begin, q_count, loss, loss_out, nullptr, nullptr,
                     grad, sens, stream);
}

}  // extern "C"
