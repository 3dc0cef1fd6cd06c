// A fourth-order Rosenbrock method with an embedded third-order solution
// (Shampine 1982, "Implementation of Rosenbrock methods", ACM TOMS 8:93, its
// four-stage parameter set; A-stable, stability function tending to 1/3 at
// infinity) for the lane-per-trajectory kernels, the fourth-order stiff
// integrator beside ROS2 and Rodas3.  The fourth stage is evaluated at the
// third stage's point (a_4j = a_3j); err = sum e_i u_i is the difference of
// the fourth- and third-order solutions.
#include "rosenbrock4.hpp"

namespace dadj {
namespace {

struct Ros4Tab {
  static constexpr double GAMMA = 0.5;
  static constexpr double A[4][4] = {{0, 0, 0, 0},
                                     {2, 0, 0, 0},
                                     {48.0 / 25.0, 6.0 / 25.0, 0, 0},
                                     {48.0 / 25.0, 6.0 / 25.0, 0, 0}};
  static constexpr double C[4][4] = {{0, 0, 0, 0},
                                     {-8, 0, 0, 0},
                                     {372.0 / 25.0, 12.0 / 5.0, 0, 0},
                                     {-112.0 / 125.0, -54.0 / 125.0, -2.0 / 5.0, 0}};
  static constexpr double M[4] = {19.0 / 9.0, 0.5, 25.0 / 108.0, 125.0 / 108.0};
  static constexpr double E[4] = {17.0 / 54.0, 7.0 / 36.0, 0, 125.0 / 108.0};
  static constexpr int order = 4, err_order = 3;
  // gamma c_ij, the coefficient of u_j in the right-hand side of stage i
  __device__ static __forceinline__ constexpr double gc(int i, int j) { return GAMMA * C[i][j]; }
};

template <class R> struct Ros4 : Rosenbrock4<Ros4Tab, R> {};

}  // namespace

hipError_t launch_ros4_record(const RecordArgs &a, const SaveTimes &st, hipStream_t s) {
  DADJ_ROS4S_DISPATCH(Ros4, record_t, (a, st, s));
}
hipError_t launch_ros4_replay_fwd(const ReplayArgs &a, hipStream_t s) {
  DADJ_ROS4S_DISPATCH(Ros4, replay_fwd_t, (a, s));
}
hipError_t launch_ros4_replay_grad(const ReplayArgs &a, hipStream_t s) {
  DADJ_ROS4S_DISPATCH(Ros4, replay_grad_t, (a, s));
}
hipError_t launch_ros4_replay_sens(const ReplayArgs &a, hipStream_t s) {
  DADJ_ROS4S_DISPATCH(Ros4, replay_sens_t, (a, s));
}

}  // namespace dadj
