// Explicit Runge-Kutta methods (Tsit5, Dopri5) for the lane-per-trajectory
// kernels: one trial step for the record, one replay step, and its reverse.
// Stage states and stage derivatives stay in registers.
#pragma once

#include "lane_kernels.hpp"

namespace dadj {

template <class Tab, class R>
struct Erk {
  using Rhs = R;
  static constexpr int D = R::D;
  static constexpr int order = Tab::order, err_order = Tab::err_order;
  static constexpr bool dense_output = true;
  template <class T> struct Cache {
    T Y[7][D], K[7][D];
  };

  // K[0] = f(y) is carried between steps (first same as last).
  template <class T>
  __device__ static __forceinline__ void begin(const T (&)[D], const T *, const T (&f0)[D],
                                               Cache<T> &c) {
#pragma unroll
    for (int i = 0; i < D; ++i) c.K[0][i] = f0[i];
  }

  // Trial step: ynew = Y[6] (5th order), err = h sum_j e_j K_j with e = b - bhat.
  template <class T>
  __device__ static __forceinline__ void attempt(const T (&y)[D], const T *p, T h, Cache<T> &c,
                                                 T (&ynew)[D], T (&err)[D]) {
    erk_stages<Tab, Rhs, 6, true>(y, p, h, c.Y, c.K);
#pragma unroll
    for (int i = 0; i < D; ++i) {
      ynew[i] = c.Y[6][i];
      T acc = T(0);
      bool first = true;
#pragma unroll
      for (int j = 0; j < 7; ++j) {
        if (Tab::e[j] != 0.0) {
          if (first) { acc = T(Tab::e[j]) * c.K[j][i]; first = false; }
          else acc = mac(T(Tab::e[j]), c.K[j][i], acc);
        }
      }
      err[i] = h * acc;
    }
  }

  template <class T> __device__ static __forceinline__ void accepted(Cache<T> &c) {
#pragma unroll
    for (int i = 0; i < D; ++i) c.K[0][i] = c.K[6][i];
  }

  // Replay step: y <- Y[6] = y + h sum_j b_j K_j (six right-hand sides).  T
  // may be a tangent type (the sensitivity kernels), H is the step type.
  template <class T, class H>
  __device__ static __forceinline__ void fwd(T (&y)[D], const T *p, H h) {
    T Y[7][D], K[7][D];
    Rhs::f(y, p, K[0]);
    erk_stages<Tab, Rhs, 6, false>(y, p, h, Y, K);
#pragma unroll
    for (int i = 0; i < D; ++i) y[i] = Y[6][i];
  }

  // The reverse sweep runs on two wavefronts for small ensembles
  // (k_replay_grad2): one recomputes the stages (pre), one runs the adjoint
  // (adj_pre).
  static constexpr bool two_wave_reverse = true;

  // What the reverse of one step needs from its forward recomputation: the
  // state y_k and the stage states Y_1..Y_5, in v = (y, Y_1, ..., Y_5).
  template <class T> struct Pre {
    static constexpr int NV = 6 * D;
    T v[NV];
    int bits;
  };
  template <class T>
  __device__ static __forceinline__ void pre(const T (&y)[D], const T *p, T h, Pre<T> &q) {
    T Y[7][D], K[7][D];
    Rhs::f(y, p, K[0]);
    erk_stages<Tab, Rhs, 5, false>(y, p, h, Y, K);
#pragma unroll
    for (int c = 0; c < D; ++c) q.v[c] = y[c];
#pragma unroll
    for (int i = 1; i <= 5; ++i)
#pragma unroll
      for (int c = 0; c < D; ++c) q.v[i * D + c] = Y[i][c];
    q.bits = 0;
  }

  // Reverse of fwd at y = y_k: lam (dL/dy_{k+1} -> dL/dy_k), g += dL/dp.
  //   kbar_i = h (b_i lam + sum_{l>i} a[l][i] w_l),  w_i = J(Y_i)^T kbar_i,
  //   g += J_p(Y_i)^T kbar_i,  lam <- lam + w_5 + w_4 + ... + w_0.
  // Stage states Y_1..Y_5 are recomputed from y_k (pre); the stage slopes
  // are dead once the states are formed, and the w_i are summed into lam at
  // the end in the order of the formula.
  template <class T>
  __device__ static __forceinline__ void adj(const T (&y)[D], const T *p, T h, T (&lam)[D], T *g) {
    Pre<T> q;
    pre(y, p, h, q);
    adj_pre(q, p, h, lam, g);
  }

  template <class T>
  __device__ static __forceinline__ void adj_pre(const Pre<T> &q, const T *p, T h, T (&lam)[D],
                                                 T *g) {
    T Y[6][D], Wv[7][D], kb[D];
#pragma unroll
    for (int i = 0; i <= 5; ++i)
#pragma unroll
      for (int c = 0; c < D; ++c) Y[i][c] = q.v[i * D + c];
#pragma unroll
    for (int i = 5; i >= 0; --i) {
#pragma unroll
      for (int c = 0; c < D; ++c) {
        T acc = T(0);
        bool first = true;
        if (Tab::a[6][i] != 0.0) {
          acc = T(Tab::a[6][i]) * lam[c];
          first = false;
        }
#pragma unroll
        for (int l = i + 1; l <= 5; ++l) {
          if (Tab::a[l][i] != 0.0) {
            if (first) { acc = T(Tab::a[l][i]) * Wv[l][c]; first = false; }
            else acc = mac(T(Tab::a[l][i]), Wv[l][c], acc);
          }
        }
        kb[c] = h * acc;
      }
      Rhs::vjp_y(Y[i], p, kb, Wv[i]);
      Rhs::vjp_p_acc(Y[i], p, kb, g);
    }
#pragma unroll
    for (int c = 0; c < D; ++c) {
      T s = lam[c];
#pragma unroll
      for (int i = 5; i >= 0; --i) s = s + Wv[i][c];
      lam[c] = s;
    }
  }
};

// FN<T, Erk<TAB, rhs>> ARGS for the problem's right-hand side.
#define DADJ_ERK_RHS_DISPATCH(FN, T, TAB, ARGS)                                           \
  do {                                                                                     \
    switch (a.pr.rhs) {                                                                    \
      case DA_RHS_LINEAR: return FN<T, Erk<TAB, Linear>> ARGS;                             \
      case DA_RHS_LORENZ63: return FN<T, Erk<TAB, Lorenz63>> ARGS;                         \
      case DA_RHS_ROBERTSON: return FN<T, Erk<TAB, Robertson>> ARGS;                       \
      default: return hipErrorInvalidValue;                                                \
    }                                                                                      \
  } while (0)

// FN<T, Erk<tableau, rhs>> ARGS for the problem's dtype, method and
// right-hand side.
#define DADJ_ERK_DISPATCH(FN, ARGS)                                                        \
  do {                                                                                     \
    const bool ts = a.pr.method == DA_TSIT5;                                               \
    if (a.pr.dtype == DA_F64) {                                                            \
      if (ts) DADJ_ERK_RHS_DISPATCH(FN, double, Tsit5Tab, ARGS);                           \
      DADJ_ERK_RHS_DISPATCH(FN, double, Dopri5Tab, ARGS);                                  \
    }                                                                                      \
    if (ts) DADJ_ERK_RHS_DISPATCH(FN, float, Tsit5Tab, ARGS);                              \
    DADJ_ERK_RHS_DISPATCH(FN, float, Dopri5Tab, ARGS);                                     \
  } while (0)

}  // namespace dadj
