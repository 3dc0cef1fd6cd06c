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
namespace {

template <class T, class M, bool DENSE>
hipError_t replay_sens_d(const ReplayArgs &a, hipStream_t s) {
  constexpr int Q = M::Rhs::D + M::Rhs::P;
  const dim3 grid((unsigned)((a.n + BLOCK - 1) / BLOCK), (unsigned)((Q + SENS_G - 1) / SENS_G));
  if (a.h_rows)
    hipLaunchKernelGGL((k_replay_sens<T, M, SENS_G, true, DENSE>), grid, BLOCK, 0, s, a);
  else
    hipLaunchKernelGGL((k_replay_sens<T, M, SENS_G, false, DENSE>), grid, BLOCK, 0, s, a);
  return hipGetLastError();
}

// Dense output changes only the saves: without loss terms at the saves and
// without sensitivity output the plain kernel computes the same.
template <class T, class M>
hipError_t replay_sens_t(const ReplayArgs &a, hipStream_t s) {
  const bool at_saves = a.sens || (a.has_loss && a.loss_kind != DA_LOSS_SUMSQ_FINAL);
  if (a.pr.dense && at_saves) return replay_sens_d<T, M, true>(a, s);
  return replay_sens_d<T, M, false>(a, s);
}

}  // namespace

hipError_t launch_erk_replay_sens(const ReplayArgs &a, hipStream_t s) {
  DADJ_ERK_DISPATCH(replay_sens_t, (a, s));
}

}  // namespace dadj
