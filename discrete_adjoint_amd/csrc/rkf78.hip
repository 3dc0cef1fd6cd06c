// Fehlberg 7(8) (Fehlberg 1968, NASA TR R-287) for the lane-per-trajectory
// kernels: the higher-order explicit pair beside Tsit5 and Dopri5.  13 stages
// with rational coefficients; the 7th-order solution y + h sum b_j K_j (which
// needs K_1..K_11) is propagated, and its difference to the 8th-order
// companion, (41/840) h (K_1 + K_11 - K_12 - K_13), is the error estimate.
// Not first same as last: a trial step evaluates all 13 stages, a replay step
// the first 11.  The reverse sweep recomputes the 11 stages from the stored
// state and runs the transposed tableau, as for the 5(4) pairs.
#include "lane_kernels.hpp"
#include "sens_kernel.hpp"

namespace dadj {
namespace {

constexpr double RK78_A[13][13] = {
    {},
    {2.0 / 27.0},
    {1.0 / 36.0, 1.0 / 12.0},
    {1.0 / 24.0, 0, 1.0 / 8.0},
    {5.0 / 12.0, 0, -25.0 / 16.0, 25.0 / 16.0},
    {1.0 / 20.0, 0, 0, 1.0 / 4.0, 1.0 / 5.0},
    {-25.0 / 108.0, 0, 0, 125.0 / 108.0, -65.0 / 27.0, 125.0 / 54.0},
    {31.0 / 300.0, 0, 0, 0, 61.0 / 225.0, -2.0 / 9.0, 13.0 / 900.0},
    {2.0, 0, 0, -53.0 / 6.0, 704.0 / 45.0, -107.0 / 9.0, 67.0 / 90.0, 3.0},
    {-91.0 / 108.0, 0, 0, 23.0 / 108.0, -976.0 / 135.0, 311.0 / 54.0, -19.0 / 60.0, 17.0 / 6.0,
     -1.0 / 12.0},
    {2383.0 / 4100.0, 0, 0, -341.0 / 164.0, 4496.0 / 1025.0, -301.0 / 82.0, 2133.0 / 4100.0,
     45.0 / 82.0, 45.0 / 164.0, 18.0 / 41.0},
    {3.0 / 205.0, 0, 0, 0, 0, -6.0 / 41.0, -3.0 / 205.0, -3.0 / 41.0, 3.0 / 41.0, 6.0 / 41.0},
    {-1777.0 / 4100.0, 0, 0, -341.0 / 164.0, 4496.0 / 1025.0, -289.0 / 82.0, 2193.0 / 4100.0,
     51.0 / 82.0, 33.0 / 164.0, 12.0 / 41.0, 0, 1.0},
};
// 7th-order weights and the 8th-order companion's
constexpr double RK78_B[13] = {41.0 / 840.0, 0, 0, 0, 0, 34.0 / 105.0, 9.0 / 35.0,
                               9.0 / 35.0, 9.0 / 280.0, 9.0 / 280.0, 41.0 / 840.0, 0, 0};
constexpr double RK78_B8[13] = {0, 0, 0, 0, 0, 34.0 / 105.0, 9.0 / 35.0,
                                9.0 / 35.0, 9.0 / 280.0, 9.0 / 280.0, 0, 41.0 / 840.0,
                                41.0 / 840.0};
// error weights e = b7 - b8
struct Rk78Weights {
  double v[13];
};
constexpr Rk78Weights make_rk78_e() {
  Rk78Weights r{};
  for (int j = 0; j < 13; ++j) r.v[j] = RK78_B[j] - RK78_B8[j];
  return r;
}
constexpr Rk78Weights RK78_E = make_rk78_e();

// Stages 0..LAST from y: Y_i = fma(h, sum_{j<i} a_ij K_j, y) (a product, then
// multiply-adds), K_i = f(Y_i).  V: a real or a tangent number.  The stages
// are unrolled by template recursion, so that every stage index is a
// compile-time constant and the stage arrays stay in registers.
template <class Rhs, int I, int LAST>
struct Rk78Stage {
  template <class V, class H>
  __device__ static __forceinline__ void run(const V (&y)[Rhs::D], const V *p, H h,
                                             V (&Y)[LAST + 1][Rhs::D], V (&K)[LAST + 1][Rhs::D]) {
    constexpr int D = Rhs::D;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      V acc = V(0);
      bool first = true;
#pragma unroll
      for (int j = 0; j < I; ++j)
        if (RK78_A[I][j] != 0.0) {
          acc = first ? cmul(RK78_A[I][j], K[j][c]) : cmac(RK78_A[I][j], K[j][c], acc);
          first = false;
        }
      Y[I][c] = smac(h, acc, y[c]);
    }
    Rhs::f(Y[I], p, K[I]);
    Rk78Stage<Rhs, I + 1, LAST>::run(y, p, h, Y, K);
  }
};
template <class Rhs, int LAST>
struct Rk78Stage<Rhs, LAST + 1, LAST> {
  template <class V, class H>
  __device__ static __forceinline__ void run(const V (&)[Rhs::D], const V *, H,
                                             V (&)[LAST + 1][Rhs::D], V (&)[LAST + 1][Rhs::D]) {}
};

template <class Rhs, int LAST, class V, class H>
__device__ __forceinline__ void rk78_stages(const V (&y)[Rhs::D], const V *p, H h,
                                            V (&Y)[LAST + 1][Rhs::D], V (&K)[LAST + 1][Rhs::D]) {
#pragma unroll
  for (int c = 0; c < Rhs::D; ++c) Y[0][c] = y[c];
  Rhs::f(y, p, K[0]);
  Rk78Stage<Rhs, 1, LAST>::run(y, p, h, Y, K);
}

// Reverse of stage I (then I - 1, ..., 0): kbar_I = h (b_I lam +
// sum_{l>I} a_lI w_l), w_I = J(Y_I)^T kbar_I, g += J_p(Y_I)^T kbar_I, and w_I
// added into s.
template <class Rhs, int I>
struct Rk78Rev {
  template <class T>
  __device__ static __forceinline__ void run(const T (&Y)[11][Rhs::D], const T *p, T h,
                                             const T (&lam)[Rhs::D], T (&Wv)[11][Rhs::D],
                                             T (&s)[Rhs::D], T *g) {
    constexpr int D = Rhs::D;
    T kb[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
      T acc = T(0);
      bool first = true;
      if (RK78_B[I] != 0.0) {
        acc = cmul(RK78_B[I], lam[c]);
        first = false;
      }
#pragma unroll
      for (int l = I + 1; l <= 10; ++l)
        if (RK78_A[l][I] != 0.0) {
          acc = first ? cmul(RK78_A[l][I], Wv[l][c]) : cmac(RK78_A[l][I], Wv[l][c], acc);
          first = false;
        }
      kb[c] = h * acc;
    }
    Rhs::vjp_y(Y[I], p, kb, Wv[I]);
    Rhs::vjp_p_acc(Y[I], p, kb, g);
#pragma unroll
    for (int c = 0; c < D; ++c) s[c] = s[c] + Wv[I][c];
    Rk78Rev<Rhs, I - 1>::run(Y, p, h, lam, Wv, s, g);
  }
};
template <class Rhs>
struct Rk78Rev<Rhs, -1> {
  template <class T>
  __device__ static __forceinline__ void run(const T (&)[11][Rhs::D], const T *, T,
                                             const T (&)[Rhs::D], T (&)[11][Rhs::D],
                                             T (&)[Rhs::D], T *) {}
};

// sum_j w_j K_j[c] over the nonzero weights (a product, then multiply-adds)
template <int S, class V, int D>
__device__ __forceinline__ V rk78_combine(const double (&w)[13], const V (&K)[S][D], int c) {
  V acc = V(0);
  bool first = true;
#pragma unroll
  for (int j = 0; j < S; ++j)
    if (w[j] != 0.0) {
      acc = first ? cmul(w[j], K[j][c]) : cmac(w[j], K[j][c], acc);
      first = false;
    }
  return acc;
}

template <class R>
struct Rkf78 {
  using Rhs = R;
  static constexpr int D = R::D;
  static constexpr int order = 7, err_order = 7;  // the error of the 7th-order solution: h^8
  static constexpr bool dense_output = false;
  // The gradient kernel keeps its guarded replay: the thirteen stages fill
  // the registers, and the branch-free path measured slower (Lorenz-63,
  // 2^20 trajectories: 4.92 ms guarded at interval 1, 5.01 branch-free at 2).
  static constexpr bool branch_free_replay = false;
  // The record zeroes the log's rows after the integration only: on
  // Lorenz-63 with 2^20 trajectories 8.1 ms, against 9.1 with a zero row
  // every second attempt during it and 9.7 with one every attempt.
  static constexpr int pad_every = 0;
  template <class T> struct Cache {};

  template <class T>
  __device__ static __forceinline__ void begin(const T (&)[D], const T *, const T (&)[D],
                                               Cache<T> &) {}

  // Trial step: all 13 stages; ynew the 7th-order solution, err = h sum e_j K_j.
  template <class T>
  __device__ static __forceinline__ void attempt(const T (&y)[D], const T *p, T h, Cache<T> &,
                                                 T (&ynew)[D], T (&err)[D]) {
    T Y[13][D], K[13][D];
    rk78_stages<Rhs, 12>(y, p, h, Y, K);
#pragma unroll
    for (int c = 0; c < D; ++c) {
      ynew[c] = smac(h, rk78_combine<13>(RK78_B, K, c), y[c]);
      err[c] = h * rk78_combine<13>(RK78_E.v, K, c);
    }
  }

  template <class T> __device__ static __forceinline__ void accepted(Cache<T> &) {}

  // Replay step: the 7th-order solution from K_1..K_11.
  template <class V, class H>
  __device__ static __forceinline__ void fwd(V (&y)[D], const V *p, H h) {
    V Y[11][D], K[11][D];
    rk78_stages<Rhs, 10>(y, p, h, Y, K);
#pragma unroll
    for (int c = 0; c < D; ++c) y[c] = smac(h, rk78_combine<11>(RK78_B, K, c), y[c]);
  }

  // Reverse of fwd at y = y_k: kbar_i = h (b_i lam + sum_{l>i} a_li w_l) for
  // i = 10..0 (terms in that order), w_i = J(Y_i)^T kbar_i,
  // g += J_p(Y_i)^T kbar_i, then lam <- lam + w_10 + w_9 + ... + w_0.
  template <class T>
  __device__ static __forceinline__ void adj(const T (&y)[D], const T *p, T h, T (&lam)[D], T *g) {
    T Y[11][D], Wv[11][D];
    {
      T K[11][D];
      rk78_stages<Rhs, 10>(y, p, h, Y, K);
    }
    T s[D];
#pragma unroll
    for (int c = 0; c < D; ++c) s[c] = lam[c];
    Rk78Rev<Rhs, 10>::run(Y, p, h, lam, Wv, s, g);
#pragma unroll
    for (int c = 0; c < D; ++c) lam[c] = s[c];
  }
};

#define DADJ_RKF78_DISPATCH(FN, ARGS)                                                      \
  do {                                                                                     \
    const bool f64 = a.pr.dtype == DA_F64;                                                 \
    switch (a.pr.rhs) {                                                                    \
      case DA_RHS_LINEAR:                                                                  \
        return f64 ? FN<double, Rkf78<Linear>> ARGS : FN<float, Rkf78<Linear>> ARGS;       \
      case DA_RHS_LORENZ63:                                                                \
        return f64 ? FN<double, Rkf78<Lorenz63>> ARGS : FN<float, Rkf78<Lorenz63>> ARGS;   \
      case DA_RHS_ROBERTSON:                                                               \
        return f64 ? FN<double, Rkf78<Robertson>> ARGS : FN<float, Rkf78<Robertson>> ARGS; \
      default:                                                                             \
        return hipErrorInvalidValue;                                                       \
    }                                                                                      \
  } while (0)

}  // namespace

hipError_t launch_rkf78_record(const RecordArgs &a, const SaveTimes &st, hipStream_t s) {
  DADJ_RKF78_DISPATCH(record_t, (a, st, s));
}
hipError_t launch_rkf78_replay_fwd(const ReplayArgs &a, hipStream_t s) {
  DADJ_RKF78_DISPATCH(replay_fwd_t, (a, s));
}
hipError_t launch_rkf78_replay_grad(const ReplayArgs &a, hipStream_t s) {
  DADJ_RKF78_DISPATCH(replay_grad_t, (a, s));
}
hipError_t launch_rkf78_replay_sens(const ReplayArgs &a, hipStream_t s) {
  DADJ_RKF78_DISPATCH(replay_sens_t, (a, s));
}

}  // namespace dadj
