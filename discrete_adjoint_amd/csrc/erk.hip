// Launchers of the explicit Runge-Kutta methods on the lane-per-trajectory
// kernels (the method itself is in erk_method.hpp).
#include "erk_method.hpp"

namespace dadj {

hipError_t launch_erk_record(const RecordArgs &a, const SaveTimes &st, hipStream_t s) {
  DADJ_ERK_DISPATCH(record_t, (a, st, s));
}
hipError_t launch_erk_replay_fwd(const ReplayArgs &a, hipStream_t s) {
  DADJ_ERK_DISPATCH(replay_fwd_t, (a, s));
}
hipError_t launch_erk_replay_grad(const ReplayArgs &a, hipStream_t s) {
  DADJ_ERK_DISPATCH(replay_grad_t, (a, s));
}

}  // namespace dadj
