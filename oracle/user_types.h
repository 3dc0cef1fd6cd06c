/*
 * Number types for right-hand sides written by the caller (TEST
 * INFRASTRUCTURE, part of the CPU oracle): the caller's f is compiled as a
 * template over T into a plugin and evaluated on reals and on dual numbers
 * (value, one tangent), from which the oracle forms the Jacobian columns it
 * needs.  Written for the oracle alone; the HIP library has its own.
 *
 * UDual<S, F>: F = false rounds every operation separately (the textbook
 * rules); F = true forms tangents with fma in a fixed order:
 *   a*b   -> (a.v b.v, fma(a.d, b.v, a.v b.d))
 *   a/b   -> (q = a.v / b.v, fma(-q, b.d, a.d) / b.v)
 * A real constant c mixed with a dual is converted to S and carries no
 * tangent: c*x -> (c x.v, c x.d), x/c -> (x.v/c, x.d/c),
 * c/x -> (q = c/x.v, (-q x.d)/x.v), c+-x and x+-c act on the value.
 * Functions g(x) -> (g(x.v), k x.d) with k = g'(x.v) taken as:
 *   sqrt 0.5/sqrt(x), exp exp(x), log 1/x, sin cos(x), cos -sin(x),
 *   tanh 1 - t*t (fused: fma(-t, t, 1)), pow(x, c) c pow(x, c - 1).
 */
#ifndef ORACLE_USER_TYPES_H
#define ORACLE_USER_TYPES_H

#include <cmath>
#include <type_traits>

namespace user {

template <class S, bool F> struct UDual {
  S v, d;
  UDual() : v(0), d(0) {}
  UDual(S x) : v(x), d(0) {}
  UDual(S x, S dx) : v(x), d(dx) {}
};

template <class S, bool F> UDual<S, F> operator+(UDual<S, F> a, UDual<S, F> b) {
  return UDual<S, F>(a.v + b.v, a.d + b.d);
}
template <class S, bool F> UDual<S, F> operator-(UDual<S, F> a, UDual<S, F> b) {
  return UDual<S, F>(a.v - b.v, a.d - b.d);
}
template <class S, bool F> UDual<S, F> operator-(UDual<S, F> a) {
  return UDual<S, F>(-a.v, -a.d);
}
template <class S, bool F> UDual<S, F> operator*(UDual<S, F> a, UDual<S, F> b) {
  if (F) return UDual<S, F>(a.v * b.v, std::fma(a.d, b.v, a.v * b.d));
  return UDual<S, F>(a.v * b.v, a.d * b.v + a.v * b.d);
}
template <class S, bool F> UDual<S, F> operator/(UDual<S, F> a, UDual<S, F> b) {
  if (F) {
    const S q = a.v / b.v;
    return UDual<S, F>(q, std::fma(-q, b.d, a.d) / b.v);
  }
  return UDual<S, F>(a.v / b.v, (a.d * b.v - a.v * b.d) / (b.v * b.v));
}

template <class A>
using IfReal = typename std::enable_if<std::is_arithmetic<A>::value, int>::type;

template <class S, bool F, class A, IfReal<A> = 0> UDual<S, F> operator+(A c, UDual<S, F> x) {
  return UDual<S, F>(S(c) + x.v, x.d);
}
template <class S, bool F, class A, IfReal<A> = 0> UDual<S, F> operator+(UDual<S, F> x, A c) {
  return UDual<S, F>(x.v + S(c), x.d);
}
template <class S, bool F, class A, IfReal<A> = 0> UDual<S, F> operator-(A c, UDual<S, F> x) {
  return UDual<S, F>(S(c) - x.v, -x.d);
}
template <class S, bool F, class A, IfReal<A> = 0> UDual<S, F> operator-(UDual<S, F> x, A c) {
  return UDual<S, F>(x.v - S(c), x.d);
}
template <class S, bool F, class A, IfReal<A> = 0> UDual<S, F> operator*(A c, UDual<S, F> x) {
  return UDual<S, F>(S(c) * x.v, S(c) * x.d);
}
template <class S, bool F, class A, IfReal<A> = 0> UDual<S, F> operator*(UDual<S, F> x, A c) {
  return UDual<S, F>(S(c) * x.v, S(c) * x.d);
}
template <class S, bool F, class A, IfReal<A> = 0> UDual<S, F> operator/(UDual<S, F> x, A c) {
  return UDual<S, F>(x.v / S(c), x.d / S(c));
}
template <class S, bool F, class A, IfReal<A> = 0> UDual<S, F> operator/(A c, UDual<S, F> x) {
  const S q = S(c) / x.v;
  return UDual<S, F>(q, (-q * x.d) / x.v);
}

/* reals */
inline double sqrt(double x) { return std::sqrt(x); }
inline float sqrt(float x) { return std::sqrt(x); }
inline double exp(double x) { return std::exp(x); }
inline float exp(float x) { return std::exp(x); }
inline double log(double x) { return std::log(x); }
inline float log(float x) { return std::log(x); }
inline double sin(double x) { return std::sin(x); }
inline float sin(float x) { return std::sin(x); }
inline double cos(double x) { return std::cos(x); }
inline float cos(float x) { return std::cos(x); }
inline double tanh(double x) { return std::tanh(x); }
inline float tanh(float x) { return std::tanh(x); }
inline double pow(double x, double c) { return std::pow(x, c); }
inline float pow(float x, double c) { return std::pow(x, float(c)); }

/* duals */
template <class S, bool F> UDual<S, F> sqrt(UDual<S, F> x) {
  const S s = sqrt(x.v);
  return UDual<S, F>(s, (S(0.5) / s) * x.d);
}
template <class S, bool F> UDual<S, F> exp(UDual<S, F> x) {
  const S e = exp(x.v);
  return UDual<S, F>(e, e * x.d);
}
template <class S, bool F> UDual<S, F> log(UDual<S, F> x) {
  return UDual<S, F>(log(x.v), (S(1) / x.v) * x.d);
}
template <class S, bool F> UDual<S, F> sin(UDual<S, F> x) {
  return UDual<S, F>(sin(x.v), cos(x.v) * x.d);
}
template <class S, bool F> UDual<S, F> cos(UDual<S, F> x) {
  return UDual<S, F>(cos(x.v), (-sin(x.v)) * x.d);
}
template <class S, bool F> UDual<S, F> tanh(UDual<S, F> x) {
  const S t = tanh(x.v);
  const S k = F ? std::fma(-t, t, S(1)) : S(1) - t * t;
  return UDual<S, F>(t, k * x.d);
}
template <class S, bool F> UDual<S, F> pow(UDual<S, F> x, double c) {
  return UDual<S, F>(pow(x.v, c), (S(c) * pow(x.v, c - 1.0)) * x.d);
}

}  // namespace user

#endif
