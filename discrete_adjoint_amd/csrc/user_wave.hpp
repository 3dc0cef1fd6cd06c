// Right-hand sides compiled at run time for the wavefront-per-trajectory
// kernels: systems of dimension up to 64 ("GRADSOLVE", evolve.pub review,
// FAQ: registered right-hand sides up to state dimension 64 run in the fused
// kernels) whose component i depends on the components i + o (mod d) for a
// few fixed offsets o, a cyclic stencil such as Lorenz-96.  The caller writes
// component i of f as the body of
//
//   template <class T, class Y> T f(const Y &y, const T *p)
//
// where y(o) is the component i + o (mod d) for a declared offset o (NaN for
// an undeclared one), y.i is i, y.d is d, and p holds the P parameters.
// Lane c of the wavefront evaluates component c; the neighbours come from
// the same cross-lane moves as the built-in Lorenz-96 (DPP rotations at
// d = 64, ds_bpermute otherwise).  Vector-Jacobian products: one forward
// pass on tangent numbers with a direction per offset and per parameter
// gives D_s = df_c / dy(o_s) and df_c / dp_q in lane c; then
//   (J^T v)_c = sum_s [v D_s] taken from component c - o_s (offsets in
//               declared order, first term, then additions),
//   g_q <- fma(v, df_c / dp_q, g_q) in lane c (summed over the lanes at the
//               end of the reverse sweep).
#pragma once

#include "user_rhs.hpp"
#include "wave_kernels.hpp"

namespace dadj {
namespace user {

// NaN of a real or of a tangent number
template <class V> struct NanOf;
template <> struct NanOf<double> {
  __device__ static __forceinline__ double get() { return nanv<double>(); }
};
template <> struct NanOf<float> {
  __device__ static __forceinline__ float get() { return nanv<float>(); }
};
template <class T, int G> struct NanOf<DualN<T, G>> {
  __device__ static __forceinline__ DualN<T, G> get() { return DualN<T, G>(nanv<T>()); }
};

// The stencil values of one lane: val[s] = component i + OFF[s] (mod d).
template <class S, class V> struct StencilY {
  V val[S::NOFF];
  int i, d;
  __device__ __forceinline__ V operator()(int o) const {
    V r = NanOf<V>::get();
#pragma unroll
    for (int s = 0; s < S::NOFF; ++s)
      if (S::OFF[s] == o) r = val[s];
    return r;
  }
};

// Value of v at component c + k (k in [-3, 3]) by wavefront rotations.
template <class V> __device__ __forceinline__ V rot_by(V v, int k) {
#pragma unroll
  for (int t = 0; t < 3; ++t)
    if (t < k) v = wave::rot<wave::DPP_WAVE_ROL1>(v);
#pragma unroll
  for (int t = 0; t < 3; ++t)
    if (t < -k) v = wave::rot<wave::DPP_WAVE_ROR1>(v);
  return v;
}

// Neighbour context: FULL (d = 64) rotates; otherwise the lanes of the
// components c + OFF[s] (fw) and c - OFF[s] (bw), mod d, are read.
template <class S, bool FULL> struct StencilNb {
  int c, d;
  int fw[S::NOFF], bw[S::NOFF];
  __device__ __forceinline__ void init(int c_, int d_) {
    c = c_;
    d = d_;
    const int cc = c < d ? c : 0;
#pragma unroll
    for (int s = 0; s < S::NOFF; ++s) {
      fw[s] = ((cc + S::OFF[s]) % d + d) % d;
      bw[s] = ((cc - S::OFF[s]) % d + d) % d;
    }
  }
  template <class V> __device__ __forceinline__ V ahead(V v, int s) const {  // v_{c + OFF[s]}
    if (S::OFF[s] == 0) return v;
    if constexpr (FULL) return rot_by(v, S::OFF[s]);
    else return wave::take(v, fw[s]);
  }
  template <class V> __device__ __forceinline__ V behind(V v, int s) const {  // v_{c - OFF[s]}
    if (S::OFF[s] == 0) return v;
    if constexpr (FULL) return rot_by(v, -S::OFF[s]);
    else return wave::take(v, bw[s]);
  }
};

template <class S> struct Stencil {
  static constexpr int P = S::P, NO = S::NOFF;
  template <bool FULL> using Nb = StencilNb<S, FULL>;

  // this lane's component of f; V a real or a tangent number
  template <class V, class PV, class NB>
  __device__ static __forceinline__ V f(V x, const PV &F, const NB &nb) {
    StencilY<S, V> y;
    y.i = nb.c;
    y.d = nb.d;
#pragma unroll
    for (int s = 0; s < NO; ++s) y.val[s] = nb.ahead(x, s);
    return S::template f<V>(y, F.v);
  }

  // w = (J^T v)_c and g += this lane's terms of J_p^T v
  template <class T, class PV, class GV, class NB>
  __device__ static __forceinline__ T vjp(T x, const PV &F, T v, const NB &nb, GV &g) {
    typedef DualN<T, NO + P> DV;
    StencilY<S, DV> y;
    y.i = nb.c;
    y.d = nb.d;
#pragma unroll
    for (int s = 0; s < NO; ++s) {
      y.val[s] = DV(nb.ahead(x, s));
      y.val[s].d[s] = T(1);
    }
    DV pd[P];
#pragma unroll
    for (int q = 0; q < P; ++q) {
      pd[q] = DV(F.v[q]);
      pd[q].d[NO + q] = T(1);
    }
    const DV r = S::template f<DV>(y, pd);
    T w = T(0);
#pragma unroll
    for (int s = 0; s < NO; ++s) {
      const T t = nb.behind(v * r.d[s], s);
      w = (s == 0) ? t : w + t;
    }
#pragma unroll
    for (int q = 0; q < P; ++q) g.v[q] = mac(v, r.d[NO + q], g.v[q]);
    return w;
  }
  template <class T, class PV, class NB>
  __device__ static __forceinline__ T vjp_y(T x, const PV &F, T v, const NB &nb) {
    wave::WPar<T, P> g;
#pragma unroll
    for (int q = 0; q < P; ++q) g.v[q] = T(0);
    return vjp(x, F, v, nb, g);
  }
  template <class T, class PV, class GV, class NB>
  __device__ static __forceinline__ void vjp_p_acc(T x, const PV &F, T v, const NB &nb, GV &g) {
    (void)vjp(x, F, v, nb, g);
  }
};

}  // namespace user
}  // namespace dadj
