// Lorenz-96 ensembles (state dimension 4..64) on the wavefront-per-trajectory
// kernels: explicit Tsit5 and Dopri5 in FP64 and FP32; record, replay,
// reverse sweep and forward-mode sensitivities.
#include "wave_kernels.hpp"

namespace dadj {
namespace {

using wave::WAVES;

// FULL: the dimension fills the wavefront (neighbours by DPP rotations).
template <class T, class M, bool FULL, bool DENSE>
hipError_t wrecord_f(const RecordArgs &a, const SaveTimes &st, hipStream_t s) {
  const unsigned grid = (unsigned)((a.n + WAVES - 1) / WAVES);
  if (a.h)
    hipLaunchKernelGGL((wave::k_wrecord<T, M, true, FULL, DENSE>), grid, 64 * WAVES, 0, s, a, st);
  else
    hipLaunchKernelGGL((wave::k_wrecord<T, M, false, FULL, DENSE>), grid, 64 * WAVES, 0, s, a, st);
  return hipGetLastError();
}
template <class T, class M, bool DENSE>
hipError_t wrecord_d(const RecordArgs &a, const SaveTimes &st, hipStream_t s) {
  return a.pr.dim == 64 ? wrecord_f<T, M, true, DENSE>(a, st, s)
                        : wrecord_f<T, M, false, DENSE>(a, st, s);
}
template <class T, class M>
hipError_t wrecord_t(const RecordArgs &a, const SaveTimes &st, hipStream_t s) {
  return a.pr.dense ? wrecord_d<T, M, true>(a, st, s) : wrecord_d<T, M, false>(a, st, s);
}

template <class T, class M, bool FULL, bool DENSE>
hipError_t wreplay_fwd_f(const ReplayArgs &a, hipStream_t s) {
  const unsigned grid = (unsigned)((a.n + WAVES - 1) / WAVES);
  hipLaunchKernelGGL((wave::k_wreplay_fwd<T, M, FULL, DENSE>), grid, 64 * WAVES, 0, s, a);
  return hipGetLastError();
}
template <class T, class M, bool DENSE>
hipError_t wreplay_fwd_d(const ReplayArgs &a, hipStream_t s) {
  return a.pr.dim == 64 ? wreplay_fwd_f<T, M, true, DENSE>(a, s)
                        : wreplay_fwd_f<T, M, false, DENSE>(a, s);
}
template <class T, class M>
hipError_t wreplay_fwd_t(const ReplayArgs &a, hipStream_t s) {
  return a.pr.dense ? wreplay_fwd_d<T, M, true>(a, s) : wreplay_fwd_d<T, M, false>(a, s);
}

template <class T, class M, bool FULL, bool DENSE>
hipError_t wreplay_grad_f(const ReplayArgs &a, hipStream_t s) {
  const unsigned grid = (unsigned)((a.nslots + WAVES - 1) / WAVES);
  switch (a.pr.checkpoint) {
    case 1: hipLaunchKernelGGL((wave::k_wreplay_grad<T, M, 1, FULL, DENSE>), grid, 64 * WAVES, 0, s, a); break;
    case 2: hipLaunchKernelGGL((wave::k_wreplay_grad<T, M, 2, FULL, DENSE>), grid, 64 * WAVES, 0, s, a); break;
    case 4: hipLaunchKernelGGL((wave::k_wreplay_grad<T, M, 4, FULL, DENSE>), grid, 64 * WAVES, 0, s, a); break;
    case 8: hipLaunchKernelGGL((wave::k_wreplay_grad<T, M, 8, FULL, DENSE>), grid, 64 * WAVES, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template <class T, class M, bool DENSE>
hipError_t wreplay_grad_d(const ReplayArgs &a, hipStream_t s) {
  return a.pr.dim == 64 ? wreplay_grad_f<T, M, true, DENSE>(a, s)
                        : wreplay_grad_f<T, M, false, DENSE>(a, s);
}
// The final-state loss reads no save: a dense problem runs the plain kernel.
template <class T, class M>
hipError_t wreplay_grad_t(const ReplayArgs &a, hipStream_t s) {
  const bool dense = a.pr.dense && a.loss_kind != DA_LOSS_SUMSQ_FINAL;
  return dense ? wreplay_grad_d<T, M, true>(a, s) : wreplay_grad_d<T, M, false>(a, s);
}

// Sensitivities: WSENS_G tangent directions per lane, ceil(q_count /
// WSENS_G) direction groups on the second grid dimension; a single direction
// (such as F alone) takes one per lane.
using wave::WSENS_G;
template <class T, class M, bool FULL, bool DENSE>
hipError_t wreplay_sens_f(const ReplayArgs &a, hipStream_t s) {
  if (a.q_count == 1) {
    const dim3 grid((unsigned)((a.n + WAVES - 1) / WAVES), 1);
    hipLaunchKernelGGL((wave::k_wreplay_sens<T, M, 1, FULL, DENSE>), grid, 64 * WAVES, 0, s, a);
  } else {
    const dim3 grid((unsigned)((a.n + WAVES - 1) / WAVES),
                    (unsigned)((a.q_count + WSENS_G - 1) / WSENS_G));
    hipLaunchKernelGGL((wave::k_wreplay_sens<T, M, WSENS_G, FULL, DENSE>), grid, 64 * WAVES, 0,
                       s, a);
  }
  return hipGetLastError();
}
template <class T, class M, bool DENSE>
hipError_t wreplay_sens_d(const ReplayArgs &a, hipStream_t s) {
  return a.pr.dim == 64 ? wreplay_sens_f<T, M, true, DENSE>(a, s)
                        : wreplay_sens_f<T, M, false, DENSE>(a, s);
}
// Without loss terms at the saves and without sensitivity output, a dense
// problem runs the plain kernel.
template <class T, class M>
hipError_t wreplay_sens_t(const ReplayArgs &a, hipStream_t s) {
  const bool at_saves = a.sens || (a.has_loss && a.loss_kind != DA_LOSS_SUMSQ_FINAL);
  return (a.pr.dense && at_saves) ? wreplay_sens_d<T, M, true>(a, s)
                                  : wreplay_sens_d<T, M, false>(a, s);
}

#define DADJ_L96_DISPATCH(FN, ARGS)                                                    \
  do {                                                                                 \
    const bool f64 = a.pr.dtype == DA_F64;                                             \
    if (a.pr.method == DA_TSIT5)                                                       \
      return f64 ? FN<double, wave::WErk<Tsit5Tab, wave::L96>> ARGS                    \
                 : FN<float, wave::WErk<Tsit5Tab, wave::L96>> ARGS;                    \
    if (a.pr.method == DA_DOPRI5)                                                      \
      return f64 ? FN<double, wave::WErk<Dopri5Tab, wave::L96>> ARGS                   \
                 : FN<float, wave::WErk<Dopri5Tab, wave::L96>> ARGS;                   \
    return hipErrorInvalidValue;                                                       \
  } while (0)

}  // namespace

hipError_t launch_l96_record(const RecordArgs &a, const SaveTimes &st, hipStream_t s) {
  DADJ_L96_DISPATCH(wrecord_t, (a, st, s));
}
hipError_t launch_l96_replay_fwd(const ReplayArgs &a, hipStream_t s) {
  DADJ_L96_DISPATCH(wreplay_fwd_t, (a, s));
}
hipError_t launch_l96_replay_grad(const ReplayArgs &a, hipStream_t s) {
  DADJ_L96_DISPATCH(wreplay_grad_t, (a, s));
}
hipError_t launch_l96_replay_sens(const ReplayArgs &a, hipStream_t s) {
  DADJ_L96_DISPATCH(wreplay_sens_t, (a, s));
}

}  // namespace dadj
