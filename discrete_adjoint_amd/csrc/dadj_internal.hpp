// Host/device interface between the C ABI (api.hip) and the kernel files.
#pragma once

#ifndef __HIPCC_RTC__
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#endif

#include "dadj.h"

namespace dadj {

constexpr int BLOCK = 256;  // threads per workgroup of the lane-per-trajectory kernels
// Step-log chunk owned by one trajectory: one 128-byte line, so that a
// lane reading its trajectory's chunk in any lane order fetches no other
// trajectory's steps.
constexpr int CHUNK_BYTES = 128;

// Steps per chunk of the tiled step log.
constexpr int chunk_steps(int dtype) { return dtype == DA_F64 ? 16 : 32; }

// Values per trajectory and checkpoint in the replay-gradient workspace: the
// state, padded to a whole wavefront for the wavefront-per-trajectory
// systems.
constexpr int ws_row(int rhs, int dim) { return rhs == DA_RHS_LORENZ96 ? 64 : dim; }

enum { LANE_OK = 0, LANE_MAX_STEPS = 1, LANE_DT_UNDERFLOW = 2, LANE_NONFINITE = 3,
       LANE_MAX_ATTEMPTS = 4 };

// Problem, flattened, defaults resolved.
struct ProbArgs {
  int32_t rhs, dim, n_params, method, dtype;
  int32_t max_steps, max_attempts, n_save, S;  // S = max(1, n_save)
  int32_t n_chunks;                             // T = ceil(max_steps / B)
  int32_t checkpoint;                           // resolved: 1, 2, 4 or 8
  int32_t dense;                                // saves from the step interpolant
  double t0, t1, rtol, atol, dt0, safety, fac_min, fac_max;
};

// Save times by value (kernel argument); t[n_save - 1] <= t1.
struct SaveTimes {
  double t[DA_MAX_SAVES];
};

struct RecordArgs {
  ProbArgs pr;
  int64_t n;
  const void *u0, *p;
  void *h;              // [T][n][B] or null (forward solve)
  int32_t *nsteps;      // [n] or null
  int32_t *sidx;        // [S][n] or null
  void *theta;          // [S][n] step fraction of each save, or null
  int32_t *status;      // [n] or null
  void *y_save;         // [S][d][n] or null
  int32_t defer_pad;    // leave the chunks after each trajectory's last one
  int32_t *natt;        // [n] trial steps (accepted + rejected), or null
};

struct ReplayArgs {
  ProbArgs pr;
  int64_t n;
  const void *u0, *p;
  const void *h;               // tiled step log [T][n][B]
  const void *h_rows;          // replay table [rows][n] in lane order, or null
  int32_t rows;
  const int32_t *nsteps, *sidx, *status, *perm;
  const void *theta;           // [S][n] step fraction of each save (dense output)
  void *y_save;                // replay_fwd output [S][d][n]
  int32_t loss_kind;
  const void *aux;             // [S][d][n]
  double scale;
  void *loss_out, *gu0, *gp;   // [n], [d][n], [P][n]
  void *ws;                    // [ceil(max_n_steps / checkpoint)][d][ws_lanes]
  void *sens;                  // sensitivity output [S][d][q_count][n] or null
  int32_t has_loss;            // sensitivity call: loss outputs requested
  int32_t q_begin, q_count;    // sensitivity call: unit directions q_begin .. + q_count - 1
  void *gq;                    // sensitivity call: gradient [q_count][n] (else gu0 / gp)
  int64_t slot0, nslots, ws_lanes;
  int32_t max_n_steps;
};

#ifndef __HIPCC_RTC__  // host side: launchers of the built-in kernels
hipError_t launch_erk_record(const RecordArgs &a, const SaveTimes &st, hipStream_t s);
hipError_t launch_erk_replay_fwd(const ReplayArgs &a, hipStream_t s);
hipError_t launch_erk_replay_grad(const ReplayArgs &a, hipStream_t s);
hipError_t launch_l96_record(const RecordArgs &a, const SaveTimes &st, hipStream_t s);
hipError_t launch_l96_replay_fwd(const ReplayArgs &a, hipStream_t s);
hipError_t launch_l96_replay_grad(const ReplayArgs &a, hipStream_t s);
hipError_t launch_l96_replay_sens(const ReplayArgs &a, hipStream_t s);
hipError_t launch_erk_replay_sens(const ReplayArgs &a, hipStream_t s);
hipError_t launch_ros2_record(const RecordArgs &a, const SaveTimes &st, hipStream_t s);
hipError_t launch_ros2_replay_fwd(const ReplayArgs &a, hipStream_t s);
hipError_t launch_ros2_replay_grad(const ReplayArgs &a, hipStream_t s);
hipError_t launch_ros2_replay_sens(const ReplayArgs &a, hipStream_t s);
hipError_t launch_rodas3_record(const RecordArgs &a, const SaveTimes &st, hipStream_t s);
hipError_t launch_rodas3_replay_fwd(const ReplayArgs &a, hipStream_t s);
hipError_t launch_rodas3_replay_grad(const ReplayArgs &a, hipStream_t s);
hipError_t launch_rodas3_replay_sens(const ReplayArgs &a, hipStream_t s);
hipError_t launch_ros4_record(const RecordArgs &a, const SaveTimes &st, hipStream_t s);
hipError_t launch_ros4_replay_fwd(const ReplayArgs &a, hipStream_t s);
hipError_t launch_ros4_replay_grad(const ReplayArgs &a, hipStream_t s);
hipError_t launch_ros4_replay_sens(const ReplayArgs &a, hipStream_t s);
hipError_t launch_rkf78_record(const RecordArgs &a, const SaveTimes &st, hipStream_t s);
hipError_t launch_rkf78_replay_fwd(const ReplayArgs &a, hipStream_t s);
hipError_t launch_rkf78_replay_grad(const ReplayArgs &a, hipStream_t s);
hipError_t launch_rkf78_replay_sens(const ReplayArgs &a, hipStream_t s);

// Mesh utilities
size_t sort_workspace_bytes(int64_t n);
hipError_t launch_mesh_sort(const ProbArgs &pr, int64_t n, const int32_t *nsteps, int32_t *perm,
                            void *ws, size_t ws_bytes, hipStream_t s);
hipError_t launch_replay_table(const ProbArgs &pr, int64_t n, const void *h,
                               const int32_t *nsteps, const int32_t *perm, void *h_rows,
                               int32_t rows, hipStream_t s);
hipError_t launch_mesh_pad(const ProbArgs &pr, int64_t n, const int32_t *nsteps, void *h,
                           hipStream_t s);
size_t max_steps_scratch_ints();  // size of dev_out below
hipError_t launch_max_steps(int64_t n, const int32_t *nsteps, int32_t *dev_out, hipStream_t s);

// Right-hand sides compiled at run time (rtc.hip)
int rtc_register(const da_rhs_def &def, int32_t *id, std::string &err);
int rtc_register_stencil(const da_rhs_stencil_def &def, int32_t *id, std::string &err);
bool rtc_is_stencil(int32_t rhs);  // a registered stencil (wavefront kernels)
int rtc_release(int32_t id, std::string &err);
int rtc_check(const da_problem &pb, std::string &err);
std::string rtc_take_error();  // message of the last failed lazy compilation on this thread
hipError_t launch_rtc_record(const RecordArgs &a, const SaveTimes &st, hipStream_t s);
hipError_t launch_rtc_replay_fwd(const ReplayArgs &a, hipStream_t s);
hipError_t launch_rtc_replay_grad(const ReplayArgs &a, hipStream_t s);
hipError_t launch_rtc_replay_sens(const ReplayArgs &a, hipStream_t s);

#endif

}  // namespace dadj
