// Wavefront-per-trajectory kernels for systems of dimension up to 64 whose
// right-hand side couples each component only to a few neighbours (the
// cyclic Lorenz-96 stencil).  The pages' one-thread-per-trajectory design
// ("Differentiable astrophysics at scale", Methodology) would keep about
// 7 KB of stage state per lane at d = 64; here lane c of a wavefront owns
// component c of one trajectory, so every lane keeps a handful of scalars and
// the neighbours come from cross-lane shuffles.  Everything that decides the
// control flow (error norm, accept/reject, step size, loop bounds) is reduced
// across the wavefront and taken from one lane, so it is wavefront-uniform
// and the shuffles always run with every lane active.
//
//  k_wrecord<T, M, LOG>        adaptive solve (record / forward-only solve)
//  k_wreplay_fwd<T, M>         fixed-step replay
//  k_wreplay_grad<T, M, CK>    replay + reverse sweep, mesh held fixed
//  k_wreplay_sens<T, M, G>     replay with G tangent directions per lane
//                              (forward-mode sensitivities)
// each also with DENSE: save times read from the cubic Hermite interpolant of
// the accepted step that holds them, per component (lane_kernels.hpp gives
// the interpolant); whether a step holds a save is the same for all lanes.
//
// A method M provides, per lane (component) with the right-hand side's
// neighbour context: fwd(x, F, h), attempt(x, F, h, k0, xnew, err) and
// adj(x, F, h, lam, gF), where F holds the trajectory's P parameters and gF
// accumulates this lane's share of dL/dF.  A right-hand side Rhs provides P,
// its neighbour context Nb<FULL>, f(x, F, nb) for this lane's component, and
// the vector-Jacobian products vjp_y(x, F, v, nb) (this lane's component of
// J^T v), vjp_p_acc(x, F, v, nb, g) (g += this lane's terms of J_p^T v) and
// vjp(x, F, v, nb, g) (both).  At d = 64 (FULL) the neighbours are DPP
// wavefront rotations; otherwise cross-lane reads (ds_bpermute).
#pragma once

#ifndef __HIPCC_RTC__
#include <math.h>
#endif

#include "dadj_device.hpp"
#include "dadj_internal.hpp"
#include "dual.hpp"

namespace dadj {
namespace wave {

constexpr int WAVES = 4;  // trajectories (wavefronts) per workgroup
constexpr int WSENS_G = 4;  // tangent directions per lane of the sensitivity kernel

// The parameters of one trajectory (the same in every lane), as reals or as
// tangent numbers.
template <class V, int P> struct WPar {
  V v[P];
};

// ---------------------------------------------------------------------------
// wavefront helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ double uniform(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)b);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ float uniform(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Sum over the 64 lanes by a butterfly; every stage adds the same two values
// in every lane (addition commutes exactly), and lane 0's result is taken.
template <class T> __device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = v + __shfl_xor(v, off, 64);
  return uniform(v);
}

__device__ __forceinline__ bool wave_all(bool b) { return __ballot(!b) == 0ull; }

template <class T> __device__ __forceinline__ T take(T v, int src) { return __shfl(v, src, 64); }

// Whole-wavefront rotations by one lane (DPP): lane c receives lane c - 1
// (ROR) or c + 1 (ROL), cyclically over the 64 lanes.
constexpr int DPP_WAVE_ROL1 = 0x134, DPP_WAVE_ROR1 = 0x13C;
template <int CTRL> __device__ __forceinline__ double rot(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)b, CTRL, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(b >> 32), CTRL, 0xf, 0xf, true);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}
template <int CTRL> __device__ __forceinline__ float rot(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Tangent numbers move part by part.
template <int CTRL, class T, int G>
__device__ __forceinline__ DualN<T, G> rot(const DualN<T, G> &v) {
  DualN<T, G> r;
  r.v = rot<CTRL>(v.v);
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = rot<CTRL>(v.d[m]);
  return r;
}
template <class T, int G>
__device__ __forceinline__ DualN<T, G> take(const DualN<T, G> &v, int src) {
  DualN<T, G> r;
  r.v = take(v.v, src);
#pragma unroll
  for (int m = 0; m < G; ++m) r.d[m] = take(v.d[m], src);
  return r;
}

// The value of lane l (a wavefront-uniform lane index), in every lane.
__device__ __forceinline__ double lane_value(double v, int l) {
  const long long b = __double_as_longlong(v);
  const unsigned lo = __builtin_amdgcn_readlane((unsigned)b, l);
  const unsigned hi = __builtin_amdgcn_readlane((unsigned)((unsigned long long)b >> 32), l);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// The cyclic neighbours of component c in dimension d.  FULL (d = 64): the
// neighbours are wavefront rotations; otherwise cross-lane reads from the
// lanes of components c+1, c+2, c-1, c-2 (mod d).
template <bool FULL> struct Nbr {
  int p1, p2, m1, m2;
  __device__ __forceinline__ void init(int c, int d) {
    const int cc = c < d ? c : 0;
    p1 = (cc + 1) % d;
    p2 = (cc + 2) % d;
    m1 = (cc + d - 1) % d;
    m2 = (cc + d - 2) % d;
  }
  template <class T> __device__ __forceinline__ T up1(T v) const {  // v_{c+1}
    if constexpr (FULL) return rot<DPP_WAVE_ROL1>(v);
    else return take(v, p1);
  }
  template <class T> __device__ __forceinline__ T dn1(T v) const {  // v_{c-1}
    if constexpr (FULL) return rot<DPP_WAVE_ROR1>(v);
    else return take(v, m1);
  }
  // v_{c+2} and v_{c-2}, given v and its first neighbour on that side
  template <class T> __device__ __forceinline__ T up2(T v, T vp1) const {
    if constexpr (FULL) return rot<DPP_WAVE_ROL1>(vp1);
    else return take(v, p2);
  }
  template <class T> __device__ __forceinline__ T dn2(T v, T vm1) const {
    if constexpr (FULL) return rot<DPP_WAVE_ROR1>(vm1);
    else return take(v, m2);
  }
};

// ---------------------------------------------------------------------------
// Lorenz-96: x_c' = (x_{c+1} - x_{c-2}) x_{c-1} - x_c + F.  The operation
// order per component is the same as in the per-trajectory formulas:
// f_c = fma(x_{c+1} - x_{c-2}, x_{c-1}, -x_c) + F;
// (J^T v)_c = x_{c-2} v_{c-1} - v_c + (x_{c+2} - x_{c-1}) v_{c+1} - x_{c+1} v_{c+2}
// (rows c-1, c, c+1, c+2 of column c, in that order); df_c/dF = 1.
// ---------------------------------------------------------------------------
struct L96 {
  static constexpr int P = 1;
  template <bool FULL> using Nb = Nbr<FULL>;
  template <class T, class PV, class NB>
  __device__ static __forceinline__ T f(T x, const PV &F, const NB &nb) {
    const T xp1 = nb.up1(x), xm1 = nb.dn1(x), xm2 = nb.dn2(x, xm1);
    return mac(xp1 - xm2, xm1, -x) + F.v[0];
  }
  template <class T, class PV, class NB>
  __device__ static __forceinline__ T vjp_y(T x, const PV &, T v, const NB &nb) {
    const T xp1 = nb.up1(x), xp2 = nb.up2(x, xp1), xm1 = nb.dn1(x), xm2 = nb.dn2(x, xm1);
    const T vm1 = nb.dn1(v), vp1 = nb.up1(v), vp2 = nb.up2(v, vp1);
    T s = xm2 * vm1;
    s = s - v;
    s = mac(xp2 - xm1, vp1, s);
    s = mac(-xp1, vp2, s);
    return s;
  }
  template <class T, class PV, class GV, class NB>
  __device__ static __forceinline__ void vjp_p_acc(T, const PV &, T v, const NB &, GV &g) {
    g.v[0] = g.v[0] + v;
  }
  template <class T, class PV, class GV, class NB>
  __device__ static __forceinline__ T vjp(T x, const PV &F, T v, const NB &nb, GV &g) {
    const T w = vjp_y(x, F, v, nb);
    vjp_p_acc(x, F, v, nb, g);
    return w;
  }
};

// ---------------------------------------------------------------------------
// Explicit RK step per component (same arithmetic schedule as the
// lane-per-trajectory kernels: first product, then multiply-adds, left to
// right; Y_i = fma(h, acc, y)).  T is a real or a tangent number (the
// coefficients and h carry no tangent); H the real type of h.
// ---------------------------------------------------------------------------
template <class Tab, int I, class T, class H>
__device__ __forceinline__ T wstage(T y, const T (&K)[7], H h) {
  T acc = T(0);
  bool first = true;
#pragma unroll
  for (int j = 0; j < I; ++j) {
    if (Tab::a[I][j] != 0.0) {
      if (first) { acc = cmul(Tab::a[I][j], K[j]); first = false; }
      else acc = cmac(Tab::a[I][j], K[j], acc);
    }
  }
  return smac(h, acc, y);
}

template <class Tab, class Rhs, int I, int LAST, bool LASTK, class T>
struct WStages {
  template <class PV, class H, class NB>
  __device__ static __forceinline__ void run(T y, const PV &F, H h, const NB &nb, T (&Y)[7],
                                             T (&K)[7]) {
    Y[I] = wstage<Tab, I>(y, K, h);
    if (I < LAST || LASTK) K[I] = Rhs::f(Y[I], F, nb);
    WStages<Tab, Rhs, I + 1, LAST, LASTK, T>::run(y, F, h, nb, Y, K);
  }
};
template <class Tab, class Rhs, int LAST, bool LASTK, class T>
struct WStages<Tab, Rhs, LAST + 1, LAST, LASTK, T> {
  template <class PV, class H, class NB>
  __device__ static __forceinline__ void run(T, const PV &, H, const NB &, T (&)[7], T (&)[7]) {}
};

template <class Tab, class R>
struct WErk {
  using Rhs = R;
  static constexpr int order = Tab::order, err_order = Tab::err_order;

  // trial step from x with K[0] = f(x) given; returns the 5th-order value
  template <class T, class PV, class NB>
  __device__ static __forceinline__ T attempt(T x, const PV &F, T h, const NB &nb, T (&K)[7],
                                              T &err) {
    T Y[7];
    WStages<Tab, Rhs, 1, 6, true, T>::run(x, F, h, nb, Y, K);
    T acc = T(0);
    bool first = true;
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      if (Tab::e[j] != 0.0) {
        if (first) { acc = T(Tab::e[j]) * K[j]; first = false; }
        else acc = mac(T(Tab::e[j]), K[j], acc);
      }
    }
    err = h * acc;
    return Y[6];
  }

  // T: a real, or the tangent numbers of the sensitivity kernel
  template <class T, class PV, class H, class NB>
  __device__ static __forceinline__ T fwd(T x, const PV &F, H h, const NB &nb) {
    T Y[7], K[7];
    K[0] = Rhs::f(x, F, nb);
    WStages<Tab, Rhs, 1, 6, false, T>::run(x, F, h, nb, Y, K);
    return Y[6];
  }

  // Reverse of fwd at x = x_k: lam (dL/dx_{k+1} -> dL/dx_k); gF += this
  // component's share of dL/dF (its terms of J_p^T kbar at every stage).
  template <class T, class PV, class GV, class NB>
  __device__ static __forceinline__ void adj(T x, const PV &F, T h, const NB &nb, T &lam,
                                             GV &gF) {
    T Y[7], Wv[7];
    {
      T K[7];
      K[0] = Rhs::f(x, F, nb);
      WStages<Tab, Rhs, 1, 5, false, T>::run(x, F, h, nb, Y, K);
    }
    Y[0] = x;
#pragma unroll
    for (int i = 5; i >= 0; --i) {
      T acc = T(0);
      bool first = true;
      if (Tab::a[6][i] != 0.0) {
        acc = T(Tab::a[6][i]) * lam;
        first = false;
      }
#pragma unroll
      for (int l = i + 1; l <= 5; ++l) {
        if (Tab::a[l][i] != 0.0) {
          if (first) { acc = T(Tab::a[l][i]) * Wv[l]; first = false; }
          else acc = mac(T(Tab::a[l][i]), Wv[l], acc);
        }
      }
      const T kb = h * acc;
      Wv[i] = Rhs::vjp(Y[i], F, kb, nb, gF);
    }
    T s = lam;
#pragma unroll
    for (int i = 5; i >= 0; --i) s = s + Wv[i];
    lam = s;
  }
};

// Dense output, per component: the interpolant at fraction th of the step of
// size h from x0 to x1, h (H11 f(x1) + H10 f(x0)) + (H01 x1 + H00 x0).  V is
// a real or a tangent number (whose weights and step carry no tangent), T
// the real type of th and h.
template <class Rhs, class V, class T, class PV, class NB>
__device__ __forceinline__ V wdense_value(T th, T h, V x0, V x1, const PV &F, const NB &nb) {
  const HermiteW<T> w = hermite_w(th);
  const V w00(w.h00), w01(w.h01), w10(w.h10), w11(w.h11), hv(h);
  const V f0 = Rhs::f(x0, F, nb), f1 = Rhs::f(x1, F, nb);
  const V sl = mac(w11, f1, w10 * f0);
  return mac(hv, sl, mac(w01, x1, w00 * x0));
}

template <class T> __device__ __forceinline__ T wmax(T a, T b) { return (a < b) ? b : a; }
template <class T> __device__ __forceinline__ T wmin(T a, T b) { return (b < a) ? b : a; }
__device__ __forceinline__ double wpow(double a, double b) { return pow(a, b); }
__device__ __forceinline__ float wpow(float a, float b) { return powf(a, b); }
__device__ __forceinline__ double wsqrt(double a) { return sqrt(a); }
__device__ __forceinline__ float wsqrt(float a) { return sqrtf(a); }
__device__ __forceinline__ double wabs(double a) { return fabs(a); }
__device__ __forceinline__ float wabs(float a) { return fabsf(a); }

// RMS over the d live components of v / sc (lanes >= d contribute zero).
template <class T> __device__ __forceinline__ T wrms(T v, T sc, bool on, int d) {
  const T q = v / sc;
  return wsqrt(wave_sum(on ? q * q : T(0)) / T(d));
}

// One trajectory per wavefront: trajectory index of this wavefront (uniform)
// and this lane's component.
struct WaveId {
  int64_t i;
  int c;
  bool live;  // trajectory exists
};
__device__ __forceinline__ WaveId wave_id(int64_t count) {
  WaveId w;
  w.c = threadIdx.x & 63;
  w.i = (int64_t)blockIdx.x * WAVES + uniform((int)(threadIdx.x >> 6));
  w.live = w.i < count;
  return w;
}

template <class T> struct WLog {
  static constexpr int B = CHUNK_BYTES / (int)sizeof(T);
};

// ---------------------------------------------------------------------------
// Record / forward solve (same controller as the lane kernels).  Lane b of
// the wavefront holds step b of the current chunk of the step log; a full
// chunk is written by lanes 0..B-1 as one 128-byte store.
// ---------------------------------------------------------------------------
template <class T, class M, bool LOG, bool FULL, bool DENSE>
__global__ __launch_bounds__(64 * WAVES) void k_wrecord(RecordArgs a, SaveTimes stimes) {
  using Rhs = typename M::Rhs;
  constexpr int B = WLog<T>::B;
  const int64_t n = a.n;
  const WaveId w = wave_id(n);
  if (!w.live) return;  // wavefront-uniform
  const int64_t i = w.i;
  const int c = w.c;
  const ProbArgs &pr = a.pr;
  const int d = pr.dim;
  const bool on = c < d;
  typename Rhs::template Nb<FULL> nb;
  nb.init(c, d);
  const int S = pr.S;
  const bool has_saves = pr.n_save > 0;
  const int n_stops = S + ((has_saves && stimes.t[pr.n_save - 1] < pr.t1) ? 1 : 0);
  const T atol = T(pr.atol), rtol = T(pr.rtol);
  const T expo = T(-1.0) / T(M::err_order + 1);
  const T safety = T(pr.safety), fmin = T(pr.fac_min), fmax = T(pr.fac_max);
  T *H = (T *)a.h;
  T *ysave = (T *)a.y_save;
  T *theta = (T *)a.theta;

  T x = on ? ((const T *)a.u0)[c * n + i] : T(0);
  WPar<T, Rhs::P> F;
  bool finp = true;
#pragma unroll
  for (int q = 0; q < Rhs::P; ++q) {
    F.v[q] = uniform(((const T *)a.p)[(int64_t)q * n + i]);
    finp = finp && finite(F.v[q]);
  }
  for (int s = 0; s < S; ++s) {
    if (a.sidx && c == 0) a.sidx[s * n + i] = -1;
    if (theta && c == 0) theta[s * n + i] = nanv<T>();
    if (ysave && on) ysave[(s * d + c) * n + i] = nanv<T>();
  }
  int nacc = 0, natt = 0, st = LANE_OK;
  T hb = T(0);  // lane b: step b of the current chunk
  const bool fin = wave_all(finite(x)) && finp;
  if (!fin) {
    st = LANE_NONFINITE;
  } else {
    T K[7];
    K[0] = Rhs::f(x, F, nb);
    T h;
    if (pr.dt0 > 0) {
      h = T(pr.dt0);
    } else {  // Hairer, Norsett, Wanner I, section II.4
      const T sc = mac(rtol, wabs(x), atol);
      const T d0 = wrms(x, sc, on, d), d1 = wrms(K[0], sc, on, d);
      const T h0 = (d0 < T(1e-5) || d1 < T(1e-5)) ? T(1e-6) : T(0.01) * (d0 / d1);
      const T x1 = mac(h0, K[0], x);
      const T f1 = Rhs::f(x1, F, nb);
      const T d2 = wrms(f1 - K[0], sc, on, d) / h0;
      const T dm = wmax(d1, d2);
      const T h1 = (dm <= T(1e-15)) ? wmax(T(1e-6), h0 * T(1e-3))
                                    : wpow(T(0.01) / dm, T(1.0) / T(M::order + 1));
      h = uniform(wmin(T(100.0) * h0, h1));
    }
    double t = pr.t0;
    int js = 0;
    bool after_reject = false;
    for (;;) {
      const double t_stop = (!DENSE && has_saves && js < S) ? stimes.t[js] : pr.t1;
      const T rem = T(t_stop - t);
      const bool land = !(h < rem);
      const T hs = land ? rem : h;
      if (nacc >= pr.max_steps) { st = LANE_MAX_STEPS; break; }
      if (natt >= pr.max_attempts) { st = LANE_MAX_ATTEMPTS; break; }
      if (!(hs > T(0)) || t + double(hs) == t) { st = LANE_DT_UNDERFLOW; break; }
      ++natt;
      T Kt[7];
      Kt[0] = K[0];
      T err;
      const T xn = M::attempt(x, F, hs, nb, Kt, err);
      const T sc = mac(rtol, wmax(wabs(x), wabs(xn)), atol);
      const T E = wrms(err, sc, on, d);
      if (E <= T(1)) {
        if (LOG) {
          const int pos = nacc % B;
          if (c == pos) hb = hs;
          if (pos == B - 1) {
            if (c < B) H[((int64_t)(nacc / B) * n + i) * B + c] = hb;
            hb = T(0);
          }
        }
        ++nacc;
        const double t_new = land ? t_stop : t + double(hs);
        if constexpr (DENSE) {  // the save times inside this step
          for (; has_saves && js < S && stimes.t[js] <= t_new; ++js) {
            const T th = T(step_fraction(stimes.t[js], t, t_new, double(hs)));
            if (a.sidx && c == 0) a.sidx[js * n + i] = nacc;
            if (theta && c == 0) theta[js * n + i] = th;
            if (ysave) {
              const T v = wdense_value<Rhs>(th, hs, x, xn, F, nb);
              if (on) ysave[(js * d + c) * n + i] = v;
            }
          }
        }
        x = xn;
        K[0] = Kt[6];
        t = t_new;
        T fac = (E == T(0)) ? fmax : wmin(fmax, wmax(fmin, safety * ctrl_pow(E, expo)));
        if (after_reject) fac = wmin(fac, T(1));
        h = uniform(hs * fac);
        after_reject = false;
        if (DENSE && land) {
          if (!has_saves) {  // the final state is the one save
            if (a.sidx && c == 0) a.sidx[i] = nacc;
            if (theta && c == 0) theta[i] = T(1);
            if (ysave && on) ysave[c * n + i] = x;
          }
          break;
        }
        if (land) {
          if (js < S) {
            if (a.sidx && c == 0) a.sidx[js * n + i] = nacc;
            if (theta && c == 0) theta[js * n + i] = T(1);
            if (ysave && on) ysave[(js * d + c) * n + i] = x;
          }
          if (++js == n_stops) break;
        }
      } else {
        const T fac = finite(E) ? wmax(fmin, safety * ctrl_pow(E, expo)) : fmin;
        h = uniform(hs * fac);
        after_reject = true;
      }
    }
  }
  if (c == 0) {
    if (a.nsteps) a.nsteps[i] = nacc;
    if (a.status) a.status[i] = st;
    if (a.natt) a.natt[i] = natt;
  }
  if (LOG) {
    // the partial chunk, then zero chunks to the end of the log, B lanes per
    // chunk (64 lanes write 64 / B chunks per store)
    int t0 = nacc / B;
    if (nacc % B != 0) {
      if (c < B) H[((int64_t)t0 * n + i) * B + c] = hb;
      ++t0;
    }
    const int per = 64 / B;
    for (int t = a.defer_pad ? pr.n_chunks : t0; t < pr.n_chunks; t += per) {
      const int tc = t + c / B;
      if (tc < pr.n_chunks) H[((int64_t)tc * n + i) * B + (c % B)] = T(0);
    }
  }
}

// Step source of a replay wavefront: the replay table row of its lane slot,
// or its trajectory's chunks of the tiled log (uniform addresses).
template <class T> struct WSteps {
  typedef __attribute__((address_space(1))) const T GT;  // global memory
  GT *base;
  int64_t stride_chunk;
  int64_t n;
  int cap;
  bool rows;
  __device__ __forceinline__ void init(const ReplayArgs &a, int64_t j, int64_t tr) {
    n = a.n;
    rows = a.h_rows != nullptr;
    if (rows) {
      base = (GT *)a.h_rows + j;
      cap = a.rows;
    } else {
      base = (GT *)a.h + tr * WLog<T>::B;
      cap = a.pr.n_chunks * WLog<T>::B;
    }
  }
  __device__ __forceinline__ T load(int k) const {
    k = k < cap ? k : cap - 1;
    k = k < 0 ? 0 : k;
    constexpr int B = WLog<T>::B;
    return rows ? base[(int64_t)k * n] : base[(int64_t)(k / B) * n * B + (k % B)];
  }
};

// ---------------------------------------------------------------------------
// Replay forward
// ---------------------------------------------------------------------------
template <class T, class M, bool FULL, bool DENSE>
__global__ __launch_bounds__(64 * WAVES) void k_wreplay_fwd(ReplayArgs a) {
  using Rhs = typename M::Rhs;
  const int64_t n = a.n;
  const WaveId w = wave_id(n);
  if (!w.live) return;
  const int64_t j = w.i;
  const int c = w.c;
  const int d = a.pr.dim;
  const bool on = c < d;
  typename Rhs::template Nb<FULL> nb;
  nb.init(c, d);
  const int S = a.pr.S;
  T *ysave = (T *)a.y_save;
  const int64_t tr = uniform((int)(a.perm ? a.perm[j] : j));
  int N = uniform(a.nsteps[tr]);
  const int cap = a.h_rows ? a.rows : a.pr.max_steps;
  const bool ok = N >= 0 && N <= cap;
  if (!ok) N = 0;
  WSteps<T> src;
  src.init(a, j, tr);
  T x = on ? ((const T *)a.u0)[c * n + tr] : T(0);
  WPar<T, Rhs::P> F;
#pragma unroll
  for (int q = 0; q < Rhs::P; ++q) F.v[q] = uniform(((const T *)a.p)[(int64_t)q * n + tr]);
  for (int q = 0; q < S; ++q) {
    const int ix = a.sidx[q * n + tr];
    if (on && (!ok || ix < 0 || ix > N)) ysave[(q * d + c) * n + tr] = nanv<T>();
  }
  int s = 0;
  int nxt = ok ? uniform(a.sidx[tr]) : -1;
  T xp = x, hp = T(0);  // DENSE: the state before the last step, and its size
  for (int k = 0; k <= N; ++k) {
    while (s < S && nxt == k) {
      T v = x;
      if (DENSE && k > 0) v = wdense_value<Rhs>(((const T *)a.theta)[s * n + tr], hp, xp, x, F, nb);
      if (on) ysave[(s * d + c) * n + tr] = v;
      ++s;
      nxt = s < S ? uniform(a.sidx[s * n + tr]) : -1;
    }
    if (k < N) {
      hp = src.load(k);
      if (DENSE) xp = x;
      x = M::fwd(x, F, hp, nb);
    }
  }
}

// ---------------------------------------------------------------------------
// Replay + reverse sweep.  Workspace: checkpoint m of local slot jl is the
// 64-component row ws[(m * ws_lanes + jl) * 64 + c] (one contiguous 512-byte
// store per wavefront in FP64).
// ---------------------------------------------------------------------------
template <class T, class M, int CK, bool FULL, bool DENSE>
__global__ __launch_bounds__(64 * WAVES) void k_wreplay_grad(ReplayArgs a) {
  using Rhs = typename M::Rhs;
  const int64_t n = a.n;
  const WaveId w = wave_id(a.nslots);
  if (!w.live) return;
  const int64_t jl = w.i;
  const int64_t j = a.slot0 + jl;
  const int c = w.c;
  const int d = a.pr.dim;
  const bool on = c < d;
  typename Rhs::template Nb<FULL> nb;
  nb.init(c, d);
  const int64_t C = a.ws_lanes;
  const int S = a.pr.S;
  const int lk = a.loss_kind;
  const bool saves = lk != DA_LOSS_SUMSQ_FINAL;
  const T *aux = (const T *)a.aux;
  T *ws = (T *)a.ws + jl * 64 + c;
  const int64_t tr = uniform((int)(a.perm ? a.perm[j] : j));
  int N = uniform(a.nsteps[tr]);
  const int cap = a.h_rows ? a.rows : a.pr.max_steps;
  const bool ok = a.status[tr] == LANE_OK && N >= 0 && N <= cap && N <= a.max_n_steps;
  if (!ok) N = 0;
  WSteps<T> src;
  src.init(a, j, tr);
  T x = on ? ((const T *)a.u0)[c * n + tr] : T(0);
  WPar<T, Rhs::P> F;
#pragma unroll
  for (int q = 0; q < Rhs::P; ++q) F.v[q] = uniform(((const T *)a.p)[(int64_t)q * n + tr]);

  // ---- forward replay, checkpoints, loss terms ----
  const T *theta = (const T *)a.theta;
  T ss = T(0);   // this lane's share of the loss
  bool first = true;
  int s = 0;
  int nxt = (ok && saves) ? uniform(a.sidx[tr]) : -1;
  // saves with index k; DENSE (k >= 1): interpolated in the step from xp (size hk)
  auto terms = [&](int k, T xp, T hk) {
    while (s < S && nxt == k) {
      T xv = x;
      if (DENSE && k > 0) xv = wdense_value<Rhs>(theta[(int64_t)s * n + tr], hk, xp, x, F, nb);
      if (on) {
        const T av = aux[((int64_t)s * d + c) * n + tr];
        if (lk == DA_LOSS_MSE_SAVE) {
          const T r = xv - av;
          ss = first ? r * r : mac(r, r, ss);
        } else {
          ss = first ? av * xv : mac(av, xv, ss);
        }
      }
      first = false;
      ++s;
      nxt = s < S ? uniform(a.sidx[s * n + tr]) : -1;
    }
  };
  if (saves) terms(0, x, T(0));
  T hcur = src.load(0);
  for (int k = 0; k < N; ++k) {
    const T hnext = src.load(k + 1);
    if (k % CK == 0) ws[(int64_t)(k / CK) * C * 64] = x;
    const T xp = x;
    x = M::fwd(x, F, hcur, nb);
    if (saves) terms(k + 1, xp, hcur);
    hcur = hnext;
  }

  // ---- loss and seeds at the final state ----
  T lam = T(0);
  WPar<T, Rhs::P> gF;
#pragma unroll
  for (int q = 0; q < Rhs::P; ++q) gF.v[q] = T(0);
  if (!saves) {
    ss = on ? x * x : T(0);
    lam = on ? T(2.0 * a.scale) * x : T(0);
  }
  int sh = S - 1;
  int hidx = (ok && saves) ? uniform(a.sidx[(int64_t)sh * n + tr]) : -1;
  auto seeds = [&](int k, T xk) {
    while (sh >= 0 && hidx == k) {
      if (on) {
        const T av = aux[((int64_t)sh * d + c) * n + tr];
        if (lk == DA_LOSS_MSE_SAVE) lam = mac(T(2.0 * a.scale), xk - av, lam);
        else lam = mac(T(a.scale), av, lam);
      }
      --sh;
      hidx = sh >= 0 ? uniform(a.sidx[(int64_t)sh * n + tr]) : -1;
    }
  };
  if (saves && !DENSE) seeds(N, x);
  T xhi = x;  // DENSE: x_{k+1} while step k is reversed

  // ---- reverse sweep by segments of CK steps ----
  const int Mw = (N + CK - 1) / CK;
  for (int m = Mw - 1; m >= 0; --m) {
    T xs[CK], hs[CK];
    xs[0] = ws[(int64_t)m * C * 64];
#pragma unroll
    for (int b = 0; b < CK; ++b) hs[b] = src.load(m * CK + b);
#pragma unroll
    for (int b = 1; b < CK; ++b)
      xs[b] = (m * CK + b - 1 < N) ? M::fwd(xs[b - 1], F, hs[b - 1], nb) : xs[b - 1];
#pragma unroll
    for (int b = CK - 1; b >= 0; --b) {
      const int k = m * CK + b;
      if (k < N) {
        if constexpr (DENSE) {
          // saves inside step k, the last first: lam (dL/dx_{k+1}) now, mu
          // (the part of dL/dx_k that bypasses the step) after its reverse;
          // this lane's share of dL/dF gets v1, then v0
          T mu = T(0);
          bool has_mu = false;
          while (sh >= 0 && hidx == k + 1) {
            const T th = theta[(int64_t)sh * n + tr];
            const T xv = wdense_value<Rhs>(th, hs[b], xs[b], xhi, F, nb);
            T sb = T(0);
            if (on) {
              const T av = aux[((int64_t)sh * d + c) * n + tr];
              if (lk == DA_LOSS_MSE_SAVE) sb = mac(T(2.0 * a.scale), xv - av, sb);
              else sb = mac(T(a.scale), av, sb);
            }
            const HermiteW<T> w = hermite_w(th);
            const T v1 = (hs[b] * w.h11) * sb, v0 = (hs[b] * w.h10) * sb;
            const T w1 = Rhs::vjp_y(xhi, F, v1, nb), w0 = Rhs::vjp_y(xs[b], F, v0, nb);
            lam = mac(w.h01, sb, lam) + w1;
            mu = mac(w.h00, sb, mu) + w0;
            Rhs::vjp_p_acc(xhi, F, v1, nb, gF);
            Rhs::vjp_p_acc(xs[b], F, v0, nb, gF);
            has_mu = true;
            --sh;
            hidx = sh >= 0 ? uniform(a.sidx[(int64_t)sh * n + tr]) : -1;
          }
          M::adj(xs[b], F, hs[b], nb, lam, gF);
          if (has_mu) lam = lam + mu;
          if (saves && k == 0) seeds(0, xs[b]);
          xhi = xs[b];
        } else {
          M::adj(xs[b], F, hs[b], nb, lam, gF);
          if (saves) seeds(k, xs[b]);
        }
      }
    }
  }

  // ---- outputs ----
  const T L = wave_sum(on ? ss : T(0));
  if (on && a.gu0) ((T *)a.gu0)[c * n + tr] = ok ? lam : nanv<T>();
  if (c == 0 && a.loss_out) ((T *)a.loss_out)[tr] = ok ? T(a.scale) * L : nanv<T>();
#pragma unroll
  for (int q = 0; q < Rhs::P; ++q) {
    const T G = wave_sum(on ? gF.v[q] : T(0));
    if (c == 0 && a.gp) ((T *)a.gp)[(int64_t)q * n + tr] = ok ? G : nanv<T>();
  }
}

// ---------------------------------------------------------------------------
// Forward-mode sensitivities (mesh held fixed): lane c carries component c of
// the state with G tangent directions; the directions q_begin .. q_begin +
// q_count - 1 of the d + P (u0 components, then parameters) are split into groups of G
// on the second grid dimension.  Outputs as the lane-per-trajectory kernel:
// sens[S][d][q_count][n], and with a loss its value and gradient by the chain
// rule.  The gradient and loss sums run in
// save-then-component order, one component after the other (each lane's
// terms are broadcast from that lane), so they follow the same order as the
// per-trajectory formulas.
// ---------------------------------------------------------------------------
template <class T, class M, int G, bool FULL, bool DENSE>
__global__ __launch_bounds__(64 * WAVES) void k_wreplay_sens(ReplayArgs a) {
  using Rhs = typename M::Rhs;
  using DT = DualN<T, G>;
  const int64_t n = a.n;
  const WaveId w = wave_id(n);
  if (!w.live) return;
  const int64_t j = w.i;
  const int c = w.c;
  const int d = a.pr.dim;
  const int q0 = a.q_begin + (int)blockIdx.y * G, qe = a.q_begin + a.q_count, Qo = a.q_count;
  const bool on = c < d;
  typename Rhs::template Nb<FULL> nb;
  nb.init(c, d);
  const int S = a.pr.S;
  const int lk = a.loss_kind;
  const bool saves = a.has_loss && lk != DA_LOSS_SUMSQ_FINAL;
  const T *aux = (const T *)a.aux;
  T *sens = (T *)a.sens;
  const int64_t tr = uniform((int)(a.perm ? a.perm[j] : j));
  int N = uniform(a.nsteps[tr]);
  const int cap = a.h_rows ? a.rows : a.pr.max_steps;
  const bool ok = a.status[tr] == LANE_OK && N >= 0 && N <= cap;
  if (!ok) N = 0;
  WSteps<T> src;
  src.init(a, j, tr);
  DT x(on ? ((const T *)a.u0)[c * n + tr] : T(0));
  WPar<DT, Rhs::P> F;
#pragma unroll
  for (int q = 0; q < Rhs::P; ++q) {
    F.v[q] = DT(uniform(((const T *)a.p)[(int64_t)q * n + tr]));
#pragma unroll
    for (int m = 0; m < G; ++m) F.v[q].d[m] = (q0 + m == d + q) ? T(1) : T(0);
  }
#pragma unroll
  for (int m = 0; m < G; ++m) x.d[m] = (on && q0 + m == c) ? T(1) : T(0);
  if (sens && on)
    for (int s = 0; s < S; ++s) {
      const int ix = a.sidx[s * n + tr];
      if (!ok || ix < 0 || ix > N)
#pragma unroll
        for (int m = 0; m < G; ++m)
          if (q0 + m < qe) sens[((int64_t)(s * d + c) * Qo + q0 + m - a.q_begin) * n + tr] = nanv<T>();
    }

  T g[G], ss = T(0);
#pragma unroll
  for (int m = 0; m < G; ++m) g[m] = T(0);
  bool first = true;
  // terms of component l for every l < d in order: seed_l . tangent_l into g,
  // (u_l, v_l) into the loss (u v, or u u when u is v)
  auto chain = [&](T seed, const DT &yv, T u, T v) {
    for (int l = 0; l < d; ++l) {
      const T sd = lane_value(seed, l), ul = lane_value(u, l), vl = lane_value(v, l);
#pragma unroll
      for (int m = 0; m < G; ++m) {
        const T t = lane_value(yv.d[m], l);
        g[m] = first ? sd * t : mac(sd, t, g[m]);
      }
      ss = first ? ul * vl : mac(ul, vl, ss);
      first = false;
    }
  };
  int s = 0;
  int nxt = ok ? uniform(a.sidx[tr]) : -1;
  auto emit = [&](const DT &ysv) {
    if (sens && on)
#pragma unroll
      for (int m = 0; m < G; ++m)
        if (q0 + m < qe) sens[((int64_t)(s * d + c) * Qo + q0 + m - a.q_begin) * n + tr] = ysv.d[m];
    if (saves) {
      const T av = on ? aux[((int64_t)s * d + c) * n + tr] : T(0);
      const T yv = ysv.v;
      if (lk == DA_LOSS_MSE_SAVE) {
        const T r = yv - av;
        chain(T(2.0 * a.scale) * r, ysv, r, r);
      } else {
        chain(T(a.scale) * av, ysv, av, yv);
      }
    }
    ++s;
    nxt = s < S ? uniform(a.sidx[s * n + tr]) : -1;
  };
  while (s < S && nxt == 0) emit(x);
  const T *theta = (const T *)a.theta;
  T hcur = src.load(0);
  for (int k = 0; k < N; ++k) {
    const T hnext = src.load(k + 1);
    const DT xp = x;
    x = M::fwd(x, F, hcur, nb);
    while (s < S && nxt == k + 1) {
      if constexpr (DENSE) emit(wdense_value<Rhs>(theta[(int64_t)s * n + tr], hcur, xp, x, F, nb));
      else emit(x);
    }
    hcur = hnext;
  }
  if (a.has_loss && !saves) chain(T(2.0 * a.scale) * x.v, x, x.v, x.v);
  if (c == 0 && a.has_loss) {
#pragma unroll
    for (int m = 0; m < G; ++m) {
      const int q = q0 + m;
      const T v = ok ? g[m] : nanv<T>();
      if (q >= qe) continue;
      if (a.gq) {
        ((T *)a.gq)[(int64_t)(q - a.q_begin) * n + tr] = v;
      } else if (q < d) {
        if (a.gu0) ((T *)a.gu0)[(int64_t)q * n + tr] = v;
      } else {
        if (a.gp) ((T *)a.gp)[(int64_t)(q - d) * n + tr] = v;
      }
    }
    if (blockIdx.y == 0 && a.loss_out) ((T *)a.loss_out)[tr] = ok ? T(a.scale) * ss : nanv<T>();
  }
}

}  // namespace wave
}  // namespace dadj
