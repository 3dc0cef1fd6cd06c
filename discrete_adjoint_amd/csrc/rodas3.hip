// Rodas3 (Sandu, Verwer, Blom, Spee, Carmichael and Potra 1997, the
// Rosenbrock solvers of atmospheric chemistry) for the lane-per-trajectory
// kernels: a third-order, stiffly accurate, L-stable Rosenbrock method with
// four stages and an embedded second-order solution (err = u_4), the
// higher-order stiff integrator beside ROS2 on the record-and-replay path.
#include "rosenbrock4.hpp"

namespace dadj {
namespace {

struct Rodas3Tab {
  static constexpr double GAMMA = 0.5;
  static constexpr double A[4][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {2, 0, 0, 0}, {2, 0, 1, 0}};
  static constexpr double C[4][4] = {
      {0, 0, 0, 0}, {4, 0, 0, 0}, {1, -1, 0, 0}, {1, -1, -8.0 / 3.0, 0}};
  static constexpr double M[4] = {2, 0, 1, 1};
  static constexpr double E[4] = {0, 0, 0, 1};
  static constexpr int order = 3, err_order = 2;
  // gamma c_ij, the coefficient of u_j in the right-hand side of stage i
  __device__ static __forceinline__ constexpr double gc(int i, int j) { return GAMMA * C[i][j]; }
};

template <class R> struct Rodas3 : Rosenbrock4<Rodas3Tab, R> {};

}  // namespace

hipError_t launch_rodas3_record(const RecordArgs &a, const SaveTimes &st, hipStream_t s) {
  DADJ_ROS4S_DISPATCH(Rodas3, record_t, (a, st, s));
}
hipError_t launch_rodas3_replay_fwd(const ReplayArgs &a, hipStream_t s) {
  DADJ_ROS4S_DISPATCH(Rodas3, replay_fwd_t, (a, s));
}
hipError_t launch_rodas3_replay_grad(const ReplayArgs &a, hipStream_t s) {
  DADJ_ROS4S_DISPATCH(Rodas3, replay_grad_t, (a, s));
}
hipError_t launch_rodas3_replay_sens(const ReplayArgs &a, hipStream_t s) {
  DADJ_ROS4S_DISPATCH(Rodas3, replay_sens_t, (a, s));
}

}  // namespace dadj
