// Second-order Rosenbrock method ROS2 (Verwer, Spee, Blom, Hundsdorfer 1999,
// gamma = 1 + 1/sqrt(2)) for the lane-per-trajectory kernels, the stiff
// integrator of the record-and-replay path ("GRADSOLVE: fast exact gradients
// for ODE ensembles on GPUs", gptget.net summary, Abstract: Rosenbrock
// integrators; evolve.pub review, Summary: default second-order Rosenbrock).
// Per lane: the d x d Jacobian (d <= 3), W = I - gamma h J, its LU factors
// with partial pivoting (ties keep the lower row), two solves per step; the
// reverse sweep uses transposed solves with the same factors and contracts
// Jbar = -gamma h Wbar with the derivative of J.  The forward step is written
// once for values and for the tangent numbers of the sensitivity kernel (V is
// either; the step size and gamma carry no tangent).
#include "rosenbrock.hpp"

namespace dadj {
namespace {

template <int D, class V> struct Ros2Step {
  V J[D * D], LU[D * D], rinv[D];  // rinv[k] = 1 / U_kk
  int perm[D];
  bool swapped;  // some row exchange happened (perm is not the identity)
  V f1[D], k1[D], Y2[D], f2[D], r2[D], k2[D], ynew[D], err[D];
};

// One ROS2 step from y with size h:
//   k1 = W^-1 f(y);  Y2 = y + h k1;  k2 = W^-1 (f(Y2) - 2 k1);
//   y+ = y + h (3/2 k1 + 1/2 k2);  err = h (1/2 k1 + 1/2 k2).
// X = false: factors without row exchanges (lu_factor<D, false>); `need`
// is set where that differs from partial pivoting.
template <class Rhs, bool X = true, class V, class H>
__device__ __forceinline__ void ros2_forward(const V (&y)[Rhs::D], const V *p, H h,
                                             Ros2Step<Rhs::D, V> &s, bool &need) {
  constexpr int D = Rhs::D;
  Rhs::jac(y, p, s.J);
  const H gh = H(ROS2_GAMMA) * h;
#pragma unroll
  for (int a = 0; a < D; ++a)
#pragma unroll
    for (int b = 0; b < D; ++b)
      s.LU[a * D + b] = (a == b) ? smac(-gh, s.J[a * D + b], V(1)) : smul(-gh, s.J[a * D + b]);
  lu_factor<D, X>(s.LU, s.perm, s.rinv, s.swapped, need);
  Rhs::f(y, p, s.f1);
  lu_solve<D, X>(s.LU, s.rinv, s.perm, s.swapped, s.f1, s.k1);
#pragma unroll
  for (int c = 0; c < D; ++c) s.Y2[c] = smac(h, s.k1[c], y[c]);
  Rhs::f(s.Y2, p, s.f2);
#pragma unroll
  for (int c = 0; c < D; ++c) s.r2[c] = cmac(-2.0, s.k1[c], s.f2[c]);
  lu_solve<D, X>(s.LU, s.rinv, s.perm, s.swapped, s.r2, s.k2);
#pragma unroll
  for (int c = 0; c < D; ++c) {
    const V acc = cmac(0.5, s.k2[c], cmul(1.5, s.k1[c]));
    s.ynew[c] = smac(h, acc, y[c]);
    const V e = cmac(0.5, s.k2[c], cmul(0.5, s.k1[c]));
    s.err[c] = smul(h, e);
  }
}

template <class R>
struct Ros2 {
  using Rhs = R;
  static constexpr int D = R::D;
  static constexpr int order = 2, err_order = 1;
  static constexpr bool dense_output = false;
  // The record zeroes the log's rows after the integration only: a
  // second-order method fills much of its log (9915 of 16384 steps on the
  // Robertson workload), and most rows zeroed while it integrates would be
  // overwritten by its later steps.  65536 trajectories: 10.8 -> 9.7 ms.
  static constexpr int pad_every = 0;
  template <class T> struct Cache {};

  template <class T>
  __device__ static __forceinline__ void begin(const T (&)[D], const T *, const T (&)[D],
                                               Cache<T> &) {}

  template <class T>
  __device__ static __forceinline__ void attempt(const T (&y)[D], const T *p, T h, Cache<T> &,
                                                 T (&ynew)[D], T (&err)[D]) {
    Ros2Step<D, T> s;
    bool need = false;
    ros2_forward<Rhs>(y, p, h, s, need);
#pragma unroll
    for (int c = 0; c < D; ++c) {
      ynew[c] = s.ynew[c];
      err[c] = s.err[c];
    }
  }

  template <class T> __device__ static __forceinline__ void accepted(Cache<T> &) {}

  // V: values, or the tangent numbers of the sensitivity kernel
  template <class V, class H>
  __device__ static __forceinline__ void fwd(V (&y)[D], const V *p, H h) {
    Ros2Step<D, V> s;
    bool need = false;
    ros2_forward<Rhs>(y, p, h, s, need);
#pragma unroll
    for (int c = 0; c < D; ++c) y[c] = s.ynew[c];
  }

  // attempt, fwd and adj without row exchanges (the record's trial steps and
  // the gradient kernel's branch-free path): the results are those of
  // attempt, fwd and adj wherever `need` stays false (partial pivoting would
  // keep every row in place, every pivot in the range of recip_nx); where it
  // is set, the caller repeats the step with attempt, fwd or adj.
  static constexpr bool row_exchanges = true;
  template <class T>
  __device__ static __forceinline__ void attempt_nx(const T (&y)[D], const T *p, T h, Cache<T> &,
                                                    T (&ynew)[D], T (&err)[D], bool &need) {
    Ros2Step<D, T> s;
    ros2_forward<Rhs, false>(y, p, h, s, need);
#pragma unroll
    for (int c = 0; c < D; ++c) {
      ynew[c] = s.ynew[c];
      err[c] = s.err[c];
    }
  }
  template <class V, class H>
  __device__ static __forceinline__ void fwd_nx(V (&y)[D], const V *p, H h, bool &need) {
    Ros2Step<D, V> s;
    ros2_forward<Rhs, false>(y, p, h, s, need);
#pragma unroll
    for (int c = 0; c < D; ++c) y[c] = s.ynew[c];
  }
  template <class T>
  __device__ static __forceinline__ void adj_nx(const T (&y)[D], const T *p, T h, T (&lam)[D],
                                                T *g, bool &need) {
    adj_x<false>(y, p, h, lam, g, need);
  }
  template <class T>
  __device__ static __forceinline__ void adj(const T (&y)[D], const T *p, T h, T (&lam)[D], T *g) {
    bool need = false;
    adj_x<true>(y, p, h, lam, g, need);
  }

  // Reverse with the mesh fixed:
  //   kbar1 = 3/2 h lam, kbar2 = 1/2 h lam, ybar = lam
  //   rbar2 = W^-T kbar2, Wbar = -rbar2 k2^T
  //   Y2bar = J(Y2)^T rbar2, g += J_p(Y2)^T rbar2
  //   kbar1 += -2 rbar2 + h Y2bar, ybar += Y2bar
  //   rbar1 = W^-T kbar1, Wbar += -rbar1 k1^T
  //   ybar += J(y)^T rbar1, g += J_p(y)^T rbar1
  //   Jbar = -gamma h Wbar; ybar, g += contraction of Jbar with dJ
  template <bool X, class T>
  __device__ static __forceinline__ void adj_x(const T (&y)[D], const T *p, T h, T (&lam)[D],
                                               T *g, bool &need) {
    Ros2Step<D, T> s;
    ros2_forward<Rhs, X>(y, p, h, s, need);
    T yb[D], kb1[D], kb2[D], rb1[D], rb2[D], Y2b[D], w[D], Wb[D * D], Jb[D * D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
      const T ab = h * lam[c];
      kb1[c] = T(1.5) * ab;
      kb2[c] = T(0.5) * ab;
      yb[c] = lam[c];
    }
    lu_solve_t<D, X>(s.LU, s.rinv, s.perm, s.swapped, kb2, rb2);
#pragma unroll
    for (int a = 0; a < D; ++a)
#pragma unroll
      for (int b = 0; b < D; ++b) Wb[a * D + b] = (-rb2[a]) * s.k2[b];
    Rhs::vjp_y(s.Y2, p, rb2, Y2b);
    Rhs::vjp_p_acc(s.Y2, p, rb2, g);
#pragma unroll
    for (int c = 0; c < D; ++c) {
      kb1[c] = mac(T(-2), rb2[c], kb1[c]);
      kb1[c] = mac(h, Y2b[c], kb1[c]);
      yb[c] = yb[c] + Y2b[c];
    }
    lu_solve_t<D, X>(s.LU, s.rinv, s.perm, s.swapped, kb1, rb1);
#pragma unroll
    for (int a = 0; a < D; ++a)
#pragma unroll
      for (int b = 0; b < D; ++b) Wb[a * D + b] = mac(-rb1[a], s.k1[b], Wb[a * D + b]);
    Rhs::vjp_y(y, p, rb1, w);
    Rhs::vjp_p_acc(y, p, rb1, g);
#pragma unroll
    for (int c = 0; c < D; ++c) yb[c] = yb[c] + w[c];
    const T gh = T(ROS2_GAMMA) * h;
#pragma unroll
    for (int q = 0; q < D * D; ++q) Jb[q] = (-gh) * Wb[q];
    Rhs::jac_contract_acc(y, p, Jb, yb, g);
#pragma unroll
    for (int c = 0; c < D; ++c) lam[c] = yb[c];
  }
};

#define DADJ_ROS2_DISPATCH(FN, ARGS)                                                  \
  do {                                                                                \
    const bool f64 = a.pr.dtype == DA_F64;                                            \
    switch (a.pr.rhs) {                                                               \
      case DA_RHS_LINEAR:                                                             \
        return f64 ? FN<double, Ros2<Linear>> ARGS : FN<float, Ros2<Linear>> ARGS;    \
      case DA_RHS_LORENZ63:                                                           \
        return f64 ? FN<double, Ros2<Lorenz63>> ARGS : FN<float, Ros2<Lorenz63>> ARGS; \
      case DA_RHS_ROBERTSON:                                                          \
        return f64 ? FN<double, Ros2<Robertson>> ARGS : FN<float, Ros2<Robertson>> ARGS; \
      case DA_RHS_KINETICS8:                                                          \
        return f64 ? FN<double, Ros2<Kinetics8>> ARGS : FN<float, Ros2<Kinetics8>> ARGS; \
      default:                                                                        \
        return hipErrorInvalidValue;                                                  \
    }                                                                                 \
  } while (0)

}  // namespace

hipError_t launch_ros2_record(const RecordArgs &a, const SaveTimes &st, hipStream_t s) {
  DADJ_ROS2_DISPATCH(record_t, (a, st, s));
}
hipError_t launch_ros2_replay_fwd(const ReplayArgs &a, hipStream_t s) {
  DADJ_ROS2_DISPATCH(replay_fwd_t, (a, s));
}
hipError_t launch_ros2_replay_grad(const ReplayArgs &a, hipStream_t s) {
  DADJ_ROS2_DISPATCH(replay_grad_t, (a, s));
}
hipError_t launch_ros2_replay_sens(const ReplayArgs &a, hipStream_t s) {
  DADJ_ROS2_DISPATCH(replay_sens_t, (a, s));
}

}  // namespace dadj
