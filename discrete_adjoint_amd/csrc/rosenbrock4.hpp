// The four-stage Rosenbrock methods (Rodas3, and a fourth-order method with
// a third-order companion) in the lane-per-trajectory kernels, written once
// for a coefficient table in the transformed form.  Per lane: the d x d
// Jacobian, W = I - gamma h J, its LU factors with partial pivoting, and per
// stage
//   Y_i = y + sum_{j<i} a_ij u_j,
//   u_i = W^-1 (gamma h f(Y_i) + sum_{j<i} gamma c_ij u_j),
// then y+ = y + sum m_i u_i and err = sum e_i u_i.  The published forms
// solve (I / (gamma h) - J) u_i = f(Y_i) + sum_j (c_ij / h) u_j, the same
// system multiplied by gamma h.  The reverse sweep runs the stages backwards
// with transposed solves on the same factors and contracts
// Jbar = -gamma h Wbar with the derivative of J, as for ROS2.
//
// A table Tab provides GAMMA, A[4][4], C[4][4], M[4], E[4], order and
// err_order as constexpr members; a zero coefficient costs nothing.
#pragma once

#include "rosenbrock.hpp"

namespace dadj {
namespace {

template <int D, class V> struct Ros4sStep {
  V J[D * D], LU[D * D], rinv[D];
  int perm[D];
  bool swapped;
  V Y[4][D], u[4][D], ynew[D], err[D];
};

// One step from y with size h.  Stage sums: Y_i from y adding a_ij u_j
// for j = 0, 1, ...; the stage right-hand side is the sum of gamma c_ij u_j
// (a product, then multiply-adds) with gamma h f(Y_i) added last; y+ from y
// adding m_i u_i in stage order.  V: a real or a tangent number.
// X = false: factors without row exchanges (lu_factor<D, false>); `need` is
// set where that differs from partial pivoting.
template <class Tab, class Rhs, bool X = true, class V, class H>
__device__ __forceinline__ void ros4s_forward(const V (&y)[Rhs::D], const V *p, H h,
                                               Ros4sStep<Rhs::D, V> &s, bool &need) {
  constexpr int D = Rhs::D;
  Rhs::jac(y, p, s.J);
  const H gh = H(Tab::GAMMA) * h;
#pragma unroll
  for (int a = 0; a < D; ++a)
#pragma unroll
    for (int b = 0; b < D; ++b)
      s.LU[a * D + b] = (a == b) ? smac(-gh, s.J[a * D + b], V(1)) : smul(-gh, s.J[a * D + b]);
  lu_factor<D, X>(s.LU, s.perm, s.rinv, s.swapped, need);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int c = 0; c < D; ++c) {
      V acc = y[c];
#pragma unroll
      for (int j = 0; j < i; ++j)
        if (Tab::A[i][j] != 0.0) acc = cmac(Tab::A[i][j], s.u[j][c], acc);
      s.Y[i][c] = acc;
    }
    V f[D], r[D];
    Rhs::f(s.Y[i], p, f);
#pragma unroll
    for (int c = 0; c < D; ++c) {
      V acc = V(0);
      bool first = true;
#pragma unroll
      for (int j = 0; j < i; ++j)
        if (Tab::gc(i, j) != 0.0) {
          acc = first ? cmul(Tab::gc(i, j), s.u[j][c]) : cmac(Tab::gc(i, j), s.u[j][c], acc);
          first = false;
        }
      r[c] = first ? smul(gh, f[c]) : smac(gh, f[c], acc);
    }
    lu_solve<D, X>(s.LU, s.rinv, s.perm, s.swapped, r, s.u[i]);
  }
#pragma unroll
  for (int c = 0; c < D; ++c) {
    V acc = y[c];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (Tab::M[i] != 0.0) acc = cmac(Tab::M[i], s.u[i][c], acc);
    s.ynew[c] = acc;
    V e = V(0);
    bool first = true;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (Tab::E[i] != 0.0) {
        e = first ? cmul(Tab::E[i], s.u[i][c]) : cmac(Tab::E[i], s.u[i][c], e);
        first = false;
      }
    s.err[c] = e;
  }
}

template <class Tab, class R>
struct Rosenbrock4 {
  using Rhs = R;
  static constexpr int D = R::D;
  static constexpr int order = Tab::order, err_order = Tab::err_order;
  static constexpr bool dense_output = false;
  template <class T> struct Cache {};

  template <class T>
  __device__ static __forceinline__ void begin(const T (&)[D], const T *, const T (&)[D],
                                               Cache<T> &) {}

  template <class T>
  __device__ static __forceinline__ void attempt(const T (&y)[D], const T *p, T h, Cache<T> &,
                                                 T (&ynew)[D], T (&err)[D]) {
    Ros4sStep<D, T> s;
    bool need = false;
    ros4s_forward<Tab, Rhs>(y, p, h, s, need);
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
    Ros4sStep<D, V> s;
    bool need = false;
    ros4s_forward<Tab, Rhs>(y, p, h, s, need);
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
    Ros4sStep<D, T> s;
    ros4s_forward<Tab, Rhs, false>(y, p, h, s, need);
#pragma unroll
    for (int c = 0; c < D; ++c) {
      ynew[c] = s.ynew[c];
      err[c] = s.err[c];
    }
  }
  template <class V, class H>
  __device__ static __forceinline__ void fwd_nx(V (&y)[D], const V *p, H h, bool &need) {
    Ros4sStep<D, V> s;
    ros4s_forward<Tab, Rhs, false>(y, p, h, s, need);
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

  // Reverse with the mesh fixed, stages from the last to the first:
  //   ubar_i = m_i lam + sum_{l>i} (a_li Ybar_l + gamma c_li rbar_l)
  //            (the m term, then l = i+1, ... with its a term before its c
  //            term; a product, then multiply-adds)
  //   rbar_i = W^-T ubar_i, Wbar -= rbar_i u_i^T, fbar_i = gamma h rbar_i,
  //   Ybar_i = J(Y_i)^T fbar_i, g += J_p(Y_i)^T fbar_i, ybar += Ybar_i;
  // then Jbar = -gamma h Wbar contracted with the derivative of J at y.
  template <bool X, class T>
  __device__ static __forceinline__ void adj_x(const T (&y)[D], const T *p, T h, T (&lam)[D],
                                               T *g, bool &need) {
    Ros4sStep<D, T> s;
    ros4s_forward<Tab, Rhs, X>(y, p, h, s, need);
    const T gh = T(Tab::GAMMA) * h;
    T yb[D], rb[4][D], Yb[4][D], Wb[D * D], Jb[D * D];
#pragma unroll
    for (int c = 0; c < D; ++c) yb[c] = lam[c];
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      T ub[D], fb[D];
#pragma unroll
      for (int c = 0; c < D; ++c) {
        T acc = T(0);
        bool first = true;
        if (Tab::M[i] != 0.0) {
          acc = cmul(Tab::M[i], lam[c]);
          first = false;
        }
#pragma unroll
        for (int l = i + 1; l < 4; ++l) {
          if (Tab::A[l][i] != 0.0) {
            acc = first ? cmul(Tab::A[l][i], Yb[l][c]) : cmac(Tab::A[l][i], Yb[l][c], acc);
            first = false;
          }
          if (Tab::gc(l, i) != 0.0) {
            acc = first ? cmul(Tab::gc(l, i), rb[l][c]) : cmac(Tab::gc(l, i), rb[l][c], acc);
            first = false;
          }
        }
        ub[c] = acc;
      }
      lu_solve_t<D, X>(s.LU, s.rinv, s.perm, s.swapped, ub, rb[i]);
#pragma unroll
      for (int a = 0; a < D; ++a)
#pragma unroll
        for (int b = 0; b < D; ++b)
          Wb[a * D + b] = (i == 3) ? (-rb[i][a]) * s.u[i][b] : mac(-rb[i][a], s.u[i][b], Wb[a * D + b]);
#pragma unroll
      for (int c = 0; c < D; ++c) fb[c] = gh * rb[i][c];
      Rhs::vjp_y(s.Y[i], p, fb, Yb[i]);
      Rhs::vjp_p_acc(s.Y[i], p, fb, g);
#pragma unroll
      for (int c = 0; c < D; ++c) yb[c] = yb[c] + Yb[i][c];
    }
#pragma unroll
    for (int q = 0; q < D * D; ++q) Jb[q] = (-gh) * Wb[q];
    Rhs::jac_contract_acc(y, p, Jb, yb, g);
#pragma unroll
    for (int c = 0; c < D; ++c) lam[c] = yb[c];
  }
};

}  // namespace
}  // namespace dadj

// Launcher body for a four-stage method template M on the systems that have
// an explicit Jacobian.
#define DADJ_ROS4S_DISPATCH(M, FN, ARGS)                                                    \
  do {                                                                                      \
    const bool f64 = a.pr.dtype == DA_F64;                                                  \
    switch (a.pr.rhs) {                                                                     \
      case DA_RHS_LINEAR:                                                                   \
        return f64 ? FN<double, M<Linear>> ARGS : FN<float, M<Linear>> ARGS;                \
      case DA_RHS_LORENZ63:                                                                 \
        return f64 ? FN<double, M<Lorenz63>> ARGS : FN<float, M<Lorenz63>> ARGS;            \
      case DA_RHS_ROBERTSON:                                                                \
        return f64 ? FN<double, M<Robertson>> ARGS : FN<float, M<Robertson>> ARGS;          \
      case DA_RHS_KINETICS8:                                                                \
        return f64 ? FN<double, M<Kinetics8>> ARGS : FN<float, M<Kinetics8>> ARGS;          \
      default:                                                                              \
        return hipErrorInvalidValue;                                                        \
    }                                                                                       \
  } while (0)
