// Forward-mode sensitivities of the replay: the state of every lane carries
// G tangent directions (unit vectors in u0, then in p) through the fixed-step
// replay, with the mesh held fixed as in the reverse sweep ("Differentiable
// astrophysics at scale", Methodology: forward sensitivities integrated in the
// same per-trajectory kernel; "GRADSOLVE" review, FAQ on exactness: no
// derivative of the step sizes).  The d + P directions are split into groups
// of G, one group per grid row, so a group costs one replay of the state plus
// G tangents.  Outputs: the sensitivity matrices at the save times and the
// loss gradient by the chain rule through the tangents.
#include "sens_kernel.hpp"

namespace dadj {

hipError_t launch_erk_replay_sens(const ReplayArgs &a, hipStream_t s) {
  DADJ_ERK_DISPATCH(replay_sens_t, (a, s));
}

}  // namespace dadj
