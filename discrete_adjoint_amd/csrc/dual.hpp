// Tangent numbers for the forward-mode sensitivity kernels: a value and G
// tangent directions, carried through the replay step alongside the state
// ("Differentiable astrophysics at scale", Methodology: forward sensitivities
// integrated in the same per-trajectory kernel).
//
// Arithmetic schedule of the tangents (every multiply-add is one fma):
//   a * b        value a.v * b.v,         tangent fma(a.d, b.v, a.v * b.d)
//   fma(a, b, c) value fma(a.v, b.v, c.v), tangent fma(a.d, b.v, fma(a.v, b.d, c.d))
//   a +- b, -a   on both parts
//   1 / b        value r = 1 / b.v,      tangent fma(-r, b.d, 0) / b.v
// Coefficients and step sizes carry no tangent: c * x scales both parts,
// fma(c, x, acc) and fma(h, acc, y) act on both parts with the same c or h.
#pragma once

#include "dadj_device.hpp"

namespace dadj {

template <class T, int G> struct DualN {
  T v;
  T d[G];
  __device__ __forceinline__ DualN() {}
  __device__ __forceinline__ DualN(T x) : v(x) {
#pragma unroll
    for (int m = 0; m < G; ++m) d[m] = T(0);
  }
};

template <class T, int G>
__device__ __forceinline__ DualN<T, G> operator+(const DualN<T, G> &a, const DualN<T, G> &b) {
  DualN<T, G> r;
  r.v = a.v + b.v;
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = a.d[m] + b.d[m];
  return r;
}
template <class T, int G>
__device__ __forceinline__ DualN<T, G> operator-(const DualN<T, G> &a, const DualN<T, G> &b) {
  DualN<T, G> r;
  r.v = a.v - b.v;
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = a.d[m] - b.d[m];
  return r;
}
template <class T, int G>
__device__ __forceinline__ DualN<T, G> operator-(const DualN<T, G> &a) {
  DualN<T, G> r;
  r.v = -a.v;
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = -a.d[m];
  return r;
}
template <class T, int G>
__device__ __forceinline__ DualN<T, G> operator*(const DualN<T, G> &a, const DualN<T, G> &b) {
  DualN<T, G> r;
  r.v = a.v * b.v;
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = mac(a.d[m], b.v, a.v * b.d[m]);
  return r;
}
template <class T, int G>
__device__ __forceinline__ DualN<T, G> mac(const DualN<T, G> &a, const DualN<T, G> &b,
                                           const DualN<T, G> &c) {
  DualN<T, G> r;
  r.v = mac(a.v, b.v, c.v);
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = mac(a.d[m], b.v, mac(a.v, b.d[m], c.d[m]));
  return r;
}

// coefficient and step-size forms (no tangent on c and h)
template <class T, int G>
__device__ __forceinline__ DualN<T, G> cmul(double c, const DualN<T, G> &x) {
  DualN<T, G> r;
  r.v = T(c) * x.v;
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = T(c) * x.d[m];
  return r;
}
template <class T, int G>
__device__ __forceinline__ DualN<T, G> cmac(double c, const DualN<T, G> &x,
                                            const DualN<T, G> &acc) {
  DualN<T, G> r;
  r.v = mac(T(c), x.v, acc.v);
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = mac(T(c), x.d[m], acc.d[m]);
  return r;
}
template <class T, int G>
__device__ __forceinline__ DualN<T, G> smac(T h, const DualN<T, G> &acc, const DualN<T, G> &y) {
  DualN<T, G> r;
  r.v = mac(h, acc.v, y.v);
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = mac(h, acc.d[m], y.d[m]);
  return r;
}

template <class T, int G>
__device__ __forceinline__ DualN<T, G> smul(T h, const DualN<T, G> &x) {
  DualN<T, G> r;
  r.v = h * x.v;
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = h * x.d[m];
  return r;
}
template <class T, int G> __device__ __forceinline__ DualN<T, G> recip(const DualN<T, G> &b) {
  DualN<T, G> r;
  r.v = T(1) / b.v;
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = mac(-r.v, b.d[m], T(0)) / b.v;
  return r;
}
template <class T, int G> __device__ __forceinline__ T vpart(const DualN<T, G> &x) { return x.v; }
template <class T, int G>
__device__ __forceinline__ DualN<T, G> sel(bool c, const DualN<T, G> &a, const DualN<T, G> &b) {
  DualN<T, G> r;
  r.v = c ? a.v : b.v;
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = c ? a.d[m] : b.d[m];
  return r;
}

}  // namespace dadj
