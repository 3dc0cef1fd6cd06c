// Replay-gradient kernels of the explicit methods for double and Dopri5
// (one file per dtype and method, see erk.hip).
#include "erk_method.hpp"

namespace dadj {

hipError_t launch_erk_grad_f64_dopri5(const ReplayArgs &a, hipStream_t s) {
  DADJ_ERK_RHS_DISPATCH(replay_grad_t, double, Dopri5Tab, (a, s));
}

}  // namespace dadj
