// Launchers of the explicit Runge-Kutta methods on the lane-per-trajectory
// kernels (the method itself is in erk_method.hpp).  The replay-gradient
// kernels are built in erk_grad_<dtype>_<method>.hip, one file per pair, so
// that their many instantiations compile in parallel.
#include "erk_method.hpp"

namespace dadj {

hipError_t launch_erk_grad_f64_tsit5(const ReplayArgs &a, hipStream_t s);
hipError_t launch_erk_grad_f64_dopri5(const ReplayArgs &a, hipStream_t s);
hipError_t launch_erk_grad_f32_tsit5(const ReplayArgs &a, hipStream_t s);
hipError_t launch_erk_grad_f32_dopri5(const ReplayArgs &a, hipStream_t s);

hipError_t launch_erk_record(const RecordArgs &a, const SaveTimes &st, hipStream_t s) {
  DADJ_ERK_DISPATCH(record_t, (a, st, s));
}
hipError_t launch_erk_replay_fwd(const ReplayArgs &a, hipStream_t s) {
  DADJ_ERK_DISPATCH(replay_fwd_t, (a, s));
}
hipError_t launch_erk_replay_grad(const ReplayArgs &a, hipStream_t s) {
  const bool ts = a.pr.method == DA_TSIT5;
  if (a.pr.dtype == DA_F64) return ts ? launch_erk_grad_f64_tsit5(a, s) : launch_erk_grad_f64_dopri5(a, s);
  return ts ? launch_erk_grad_f32_tsit5(a, s) : launch_erk_grad_f32_dopri5(a, s);
}

}  // namespace dadj
