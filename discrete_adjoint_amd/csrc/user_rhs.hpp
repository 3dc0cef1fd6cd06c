// Right-hand sides compiled at run time from the caller's source (the
// counterpart of registered right-hand sides: "GRADSOLVE" review, FAQ on
// which systems run in the fused kernels).  The caller writes only f, as the
// body of a function template that computes in the number type T:
//
//   template <class T, class TY, class TP>
//   void f(const TY *y, const TP *p, T *dy)                    // dy = f(y, p)
//
// using + - * /, real constants (best written T(c)) and the functions below.
// y and p hold numbers that convert to T (reals where no tangent is needed).
// The kernels evaluate f on reals and, for the derivatives, on tangent numbers
// (DualN): the vector-Jacobian products the reverse sweep needs are formed
// from the Jacobian columns of one forward-mode pass.
//
// Tangent rules (the fused schedule of dual.hpp, extended):
//   a / b         q = a.v / b.v,  tangent fma(-q, b', a') / b.v
//   c op x (c real) c is T(c) with no tangent: c*x -> (c x.v, c x'),
//                 x/c -> (x.v / c, x' / c), c/x -> (q = c / x.v, (-q x') / x.v)
//   g(x)          (g(x.v), k x') with k = g'(x.v) computed as
//                 sqrt: 0.5 / sqrt(x)    exp: exp(x)      log: 1 / x
//                 sin: cos(x)            cos: -sin(x)     tanh: fma(-t, t, 1)
//                 pow(x, c): c pow(x, c - 1)
#pragma once

#include "dual.hpp"

namespace dadj {

// ---------------------------------------------------------------------------
// Tangent arithmetic beyond dual.hpp
// ---------------------------------------------------------------------------
template <class T, int G>
__device__ __forceinline__ DualN<T, G> operator/(const DualN<T, G> &a, const DualN<T, G> &b) {
  DualN<T, G> r;
  r.v = a.v / b.v;
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = mac(-r.v, b.d[m], a.d[m]) / b.v;
  return r;
}

// Mixed operations take a real constant of a built-in arithmetic type only.
template <class S> struct RealConst {};
template <> struct RealConst<double> { typedef int ok; };
template <> struct RealConst<float> { typedef int ok; };
template <> struct RealConst<int> { typedef int ok; };
template <> struct RealConst<long> { typedef int ok; };
template <class S, class R> struct IfReal { typedef R type; };
#define DADJ_MIXED(S) typename IfReal<typename RealConst<S>::ok, DualN<T, G>>::type

template <class T, int G, class S>
__device__ __forceinline__ DADJ_MIXED(S) operator+(S c, const DualN<T, G> &x) {
  DualN<T, G> r = x;
  r.v = T(c) + x.v;
  return r;
}
template <class T, int G, class S>
__device__ __forceinline__ DADJ_MIXED(S) operator+(const DualN<T, G> &x, S c) {
  DualN<T, G> r = x;
  r.v = x.v + T(c);
  return r;
}
template <class T, int G, class S>
__device__ __forceinline__ DADJ_MIXED(S) operator-(S c, const DualN<T, G> &x) {
  DualN<T, G> r;
  r.v = T(c) - x.v;
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = -x.d[m];
  return r;
}
template <class T, int G, class S>
__device__ __forceinline__ DADJ_MIXED(S) operator-(const DualN<T, G> &x, S c) {
  DualN<T, G> r = x;
  r.v = x.v - T(c);
  return r;
}
template <class T, int G, class S>
__device__ __forceinline__ DADJ_MIXED(S) operator*(S c, const DualN<T, G> &x) {
  return cmul(double(T(c)), x);
}
template <class T, int G, class S>
__device__ __forceinline__ DADJ_MIXED(S) operator*(const DualN<T, G> &x, S c) {
  return cmul(double(T(c)), x);
}
template <class T, int G, class S>
__device__ __forceinline__ DADJ_MIXED(S) operator/(const DualN<T, G> &x, S c) {
  DualN<T, G> r;
  r.v = x.v / T(c);
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = x.d[m] / T(c);
  return r;
}
template <class T, int G, class S>
__device__ __forceinline__ DADJ_MIXED(S) operator/(S c, const DualN<T, G> &x) {
  DualN<T, G> r;
  r.v = T(c) / x.v;
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = (-r.v * x.d[m]) / x.v;
  return r;
}

#undef DADJ_MIXED

namespace user {

// ---------------------------------------------------------------------------
// Functions available to the caller's f, on reals and on tangent numbers
// ---------------------------------------------------------------------------
__device__ __forceinline__ double sqrt(double x) { return ::sqrt(x); }
__device__ __forceinline__ float sqrt(float x) { return ::sqrtf(x); }
__device__ __forceinline__ double exp(double x) { return ::exp(x); }
__device__ __forceinline__ float exp(float x) { return ::expf(x); }
__device__ __forceinline__ double log(double x) { return ::log(x); }
__device__ __forceinline__ float log(float x) { return ::logf(x); }
__device__ __forceinline__ double sin(double x) { return ::sin(x); }
__device__ __forceinline__ float sin(float x) { return ::sinf(x); }
__device__ __forceinline__ double cos(double x) { return ::cos(x); }
__device__ __forceinline__ float cos(float x) { return ::cosf(x); }
__device__ __forceinline__ double tanh(double x) { return ::tanh(x); }
__device__ __forceinline__ float tanh(float x) { return ::tanhf(x); }
__device__ __forceinline__ double pow(double x, double c) { return ::pow(x, c); }
__device__ __forceinline__ float pow(float x, double c) { return ::powf(x, float(c)); }

// (g(x.v), k x') for a unary function g with derivative factor k
template <class T, int G>
__device__ __forceinline__ DualN<T, G> chain1(T gv, T k, const DualN<T, G> &x) {
  DualN<T, G> r;
  r.v = gv;
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = k * x.d[m];
  return r;
}
template <class T, int G> __device__ __forceinline__ DualN<T, G> sqrt(const DualN<T, G> &x) {
  const T s = sqrt(x.v);
  return chain1(s, T(0.5) / s, x);
}
template <class T, int G> __device__ __forceinline__ DualN<T, G> exp(const DualN<T, G> &x) {
  const T e = exp(x.v);
  return chain1(e, e, x);
}
template <class T, int G> __device__ __forceinline__ DualN<T, G> log(const DualN<T, G> &x) {
  return chain1(log(x.v), T(1) / x.v, x);
}
template <class T, int G> __device__ __forceinline__ DualN<T, G> sin(const DualN<T, G> &x) {
  return chain1(sin(x.v), cos(x.v), x);
}
template <class T, int G> __device__ __forceinline__ DualN<T, G> cos(const DualN<T, G> &x) {
  return chain1(cos(x.v), -sin(x.v), x);
}
template <class T, int G> __device__ __forceinline__ DualN<T, G> tanh(const DualN<T, G> &x) {
  const T t = tanh(x.v);
  return chain1(t, mac(-t, t, T(1)), x);
}
template <class T, int G>
__device__ __forceinline__ DualN<T, G> pow(const DualN<T, G> &x, double c) {
  return chain1(pow(x.v, c), T(c) * pow(x.v, c - 1.0), x);
}

// ---------------------------------------------------------------------------
// A right-hand side from the caller's f: S provides D, P and
// template <class T, class TY, class TP> f(const TY *y, const TP *p, T *dy),
// T being the type the body computes in (the caller's "T").  The kernels'
// interface (f, vjp_y, vjp_p_acc) follows, the products from the Jacobian
// columns:
//   w_m = sum_i J[i][m] v_i          (first product, then fma, i ascending)
//   g_q <- g_q + sum_i Jp[i][q] v_i  (fma into g_q, i ascending)
// For J the parameters enter as reals, for Jp the states do: a tangent that
// is zero throughout is left out instead of carried (for finite values the
// result is the same as with zero tangents).
// ---------------------------------------------------------------------------
template <class S> struct AutoVjp {
  static constexpr int D = S::D, P = S::P;

  template <class T>
  __device__ static __forceinline__ void f(const T *y, const T *p, T *o) {
    S::template f<T, T, T>(y, p, o);
  }

  template <class T>
  __device__ static __forceinline__ void vjp_y(const T *y, const T *p, const T *v, T *w) {
    DualN<T, D> yd[D], od[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
      yd[c] = DualN<T, D>(y[c]);
      yd[c].d[c] = T(1);
    }
    S::template f<DualN<T, D>, DualN<T, D>, T>(yd, p, od);
#pragma unroll
    for (int m = 0; m < D; ++m) {
      T acc = od[0].d[m] * v[0];
#pragma unroll
      for (int i = 1; i < D; ++i) acc = mac(od[i].d[m], v[i], acc);
      w[m] = acc;
    }
  }

  template <class T>
  __device__ static __forceinline__ void vjp_p_acc(const T *y, const T *p, const T *v, T *g) {
    DualN<T, P> pd[P], od[D];
#pragma unroll
    for (int q = 0; q < P; ++q) {
      pd[q] = DualN<T, P>(p[q]);
      pd[q].d[q] = T(1);
    }
    S::template f<DualN<T, P>, T, DualN<T, P>>(y, pd, od);
#pragma unroll
    for (int q = 0; q < P; ++q) {
#pragma unroll
      for (int i = 0; i < D; ++i) g[q] = mac(od[i].d[q], v[i], g[q]);
    }
  }
};

}  // namespace user
}  // namespace dadj
