// Lane-per-trajectory kernels, generic over the integration method M.
//
//  k_record<T, M, LOG>    adaptive solve of one trajectory per lane; with LOG
//                         it writes every accepted step size into the tiled
//                         step log ("GRADSOLVE: fast exact gradients for ODE
//                         ensembles on GPUs", gptget.net summary, Methodology;
//                         evolve.pub review, Summary: zero-padded fixed-length
//                         mesh), without it it is the forward-only solve
//                         (summary, Key results).
//  k_replay_fwd<T, M>     fixed-step replay of a mesh (review, Summary).
//  k_replay_grad<T, M, C> replay that keeps every C-th state in the workspace,
//                         then the reverse sweep through the recomputed stages
//                         with the mesh held fixed (review, Strengths (paper
//                         section 3.1) and FAQ: the exact discrete adjoint, no
//                         derivative of the step-size choices).
//
// A method M provides:
//   using Rhs; order (for the starting step); err_order (controller exponent)
//   template <class T> struct Cache;                 per-attempt scratch
//   begin(y, p, cache)                               once per accepted state
//   attempt(y, p, h, cache, ynew, err)               one trial step
//   accepted(cache)                                  after an accepted trial
//   fwd(y, p, h)                                     one replay step
//   adj(y, p, h, lam, g)                             its reverse
//
// With dense output (template flag DENSE) save times do not end steps: each
// is read from the cubic Hermite interpolant of the accepted step that
// contains it, at the step fraction the record stores in the mesh.
//
// Memory: per-trajectory arrays are component-major ([c][n], trajectory
// fastest).  The step log is tiled [T][n][B]: each trajectory owns one 128-byte
// chunk of B steps per tile, so the record writes whole chunks and a replay
// in any lane order reads whole chunks.  The replays read step k + 1 (and the
// reverse sweep its checkpoint) while step k computes.
#pragma once

#ifndef __HIPCC_RTC__  // run-time compilation brings its own device math
#include <math.h>
#endif

#include "dadj_device.hpp"
#include "dadj_internal.hpp"

// Build option: DADJ_GRAD_WAVES_PER_EU=w asks the compiler to fit the
// gradient kernel into the registers of w wavefronts per SIMD.
#ifdef DADJ_GRAD_WAVES_PER_EU
#define DADJ_GRAD_OCCUPANCY __attribute__((amdgpu_waves_per_eu(DADJ_GRAD_WAVES_PER_EU)))
#else
#define DADJ_GRAD_OCCUPANCY
#endif

namespace dadj {

template <class T> __device__ __forceinline__ T dmax(T a, T b) { return (a < b) ? b : a; }
template <class T> __device__ __forceinline__ T dmin(T a, T b) { return (b < a) ? b : a; }
__device__ __forceinline__ double dpow(double a, double b) { return pow(a, b); }
__device__ __forceinline__ float dpow(float a, float b) { return powf(a, b); }
__device__ __forceinline__ double dsqrt(double a) { return sqrt(a); }
__device__ __forceinline__ float dsqrt(float a) { return sqrtf(a); }
__device__ __forceinline__ double dabs(double a) { return fabs(a); }
__device__ __forceinline__ float dabs(float a) { return fabsf(a); }

// ---------------------------------------------------------------------------
// Tiled step log
// ---------------------------------------------------------------------------
template <class T> struct Log {
  static constexpr int B = CHUNK_BYTES / (int)sizeof(T);
  // offset of step k from the lane's first element H + tr * B
  __device__ static __forceinline__ int64_t at(int k, int64_t n) {
    return (int64_t)(k / B) * n * B + (k % B);
  }
};

typedef double dvec2 __attribute__((ext_vector_type(2)));
typedef float fvec4 __attribute__((ext_vector_type(4)));

// One chunk (CHUNK_BYTES) from registers to memory as 16-byte stores.
constexpr int CHUNK_QUADS = CHUNK_BYTES / 16;
__device__ __forceinline__ void store_chunk(double *dst, const double (&v)[CHUNK_BYTES / 8]) {
  dvec2 *d = (dvec2 *)dst;
#pragma unroll
  for (int q = 0; q < CHUNK_QUADS; ++q) d[q] = dvec2{v[2 * q], v[2 * q + 1]};
}
__device__ __forceinline__ void store_chunk(float *dst, const float (&v)[CHUNK_BYTES / 4]) {
  fvec4 *d = (fvec4 *)dst;
#pragma unroll
  for (int q = 0; q < CHUNK_QUADS; ++q)
    d[q] = fvec4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
}

// Thread t's chunk from its column of an LDS array [position][BLOCK] to
// memory, one 16-byte piece at a time; the first `keep` positions (all of
// them by default) are copied and the rest written as zeros.
__device__ __forceinline__ void store_chunk_lds(double *dst, const double (*l)[BLOCK], int t,
                                                int keep = CHUNK_BYTES / 8) {
  dvec2 *d = (dvec2 *)dst;
#pragma unroll
  for (int q = 0; q < CHUNK_QUADS; ++q)
    d[q] = dvec2{2 * q < keep ? l[2 * q][t] : 0.0, 2 * q + 1 < keep ? l[2 * q + 1][t] : 0.0};
}
__device__ __forceinline__ void store_chunk_lds(float *dst, const float (*l)[BLOCK], int t,
                                                int keep = CHUNK_BYTES / 4) {
  fvec4 *d = (fvec4 *)dst;
#pragma unroll
  for (int q = 0; q < CHUNK_QUADS; ++q) {
    fvec4 x;
    x.x = 4 * q < keep ? l[4 * q][t] : 0.f;
    x.y = 4 * q + 1 < keep ? l[4 * q + 1][t] : 0.f;
    x.z = 4 * q + 2 < keep ? l[4 * q + 2][t] : 0.f;
    x.w = 4 * q + 3 < keep ? l[4 * q + 3][t] : 0.f;
    d[q] = x;
  }
}

// Zeros over the 64 consecutive chunks at dst (a wavefront's row segment),
// the lanes each writing CHUNK_QUADS 16-byte pieces so that every store
// covers 1 KB contiguously.
__device__ __forceinline__ void zero_row_segment(double *dst, int lane) {
  dvec2 *d = (dvec2 *)dst;
#pragma unroll
  for (int q = 0; q < CHUNK_QUADS; ++q) d[q * 64 + lane] = dvec2{0.0, 0.0};
}
__device__ __forceinline__ void zero_row_segment(float *dst, int lane) {
  fvec4 *d = (fvec4 *)dst;
#pragma unroll
  for (int q = 0; q < CHUNK_QUADS; ++q) d[q * 64 + lane] = fvec4{0.f, 0.f, 0.f, 0.f};
}

// RMS of v / sc over D components.
template <int D, class T>
__device__ __forceinline__ T rms(const T (&v)[D], const T (&sc)[D]) {
  T s = T(0);
#pragma unroll
  for (int c = 0; c < D; ++c) {
    const T q = v[c] / sc[c];
    s = (c == 0) ? q * q : mac(q, q, s);
  }
  return dsqrt(s / T(D));
}

// Error norm with scale atol + rtol max(|y|, |y+|).
template <int D, class T>
__device__ __forceinline__ T err_norm(const T (&err)[D], const T (&y)[D], const T (&yn)[D], T atol,
                                      T rtol) {
  T sc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) sc[c] = mac(rtol, dmax(dabs(y[c]), dabs(yn[c])), atol);
  return rms<D>(err, sc);
}

// ---------------------------------------------------------------------------
// Dense output ("Differentiable astrophysics at scale", Methodology: the
// solution is interpolated at observation times instead of ending steps
// there).  The interpolant is the cubic Hermite one of the accepted step
// [t_k, t_k + h] through y_k, y_{k+1} and the slopes f(y_k), f(y_{k+1}):
//   y(t_k + th h) = h (H11 f(y_{k+1}) + H10 f(y_k)) + (H01 y_{k+1} + H00 y_k)
//   H00 = (1-th)^2 (1+2th), H01 = th^2 (3-2th), H10 = th (1-th)^2,
//   H11 = -th^2 (1-th);  th = 1 gives y_{k+1} exactly.
// ---------------------------------------------------------------------------
// Interpolated state at fraction th of the step of size h from y0 to y1.  V
// is the value type (a real, or a tangent type whose weights and step carry
// no tangent), T the real type of th and h.
template <class Rhs, class V, class T>
__device__ __forceinline__ void dense_value(T th, T h, const V (&y0)[Rhs::D],
                                            const V (&y1)[Rhs::D], const V *p,
                                            V (&out)[Rhs::D]) {
  constexpr int D = Rhs::D;
  const HermiteW<T> w = hermite_w(th);
  const V w00(w.h00), w01(w.h01), w10(w.h10), w11(w.h11), hv(h);
  V f0[D], f1[D];
  Rhs::f(y0, p, f0);
  Rhs::f(y1, p, f1);
#pragma unroll
  for (int c = 0; c < D; ++c) {
    const V sl = mac(w11, f1[c], w10 * f0[c]);
    out[c] = mac(hv, sl, mac(w01, y1[c], w00 * y0[c]));
  }
}

// Starting step of Hairer, Norsett, Wanner I, section II.4, method order q.
template <class Rhs, class T>
__device__ T initial_step(const T (&y0)[Rhs::D], const T (&f0)[Rhs::D], const T *p, T atol,
                          T rtol, int q) {
  constexpr int D = Rhs::D;
  T sc[D], y1[D], f1[D], df[D];
#pragma unroll
  for (int c = 0; c < D; ++c) sc[c] = mac(rtol, dabs(y0[c]), atol);
  const T d0 = rms<D>(y0, sc);
  const T d1 = rms<D>(f0, sc);
  const T h0 = (d0 < T(1e-5) || d1 < T(1e-5)) ? T(1e-6) : T(0.01) * (d0 / d1);
#pragma unroll
  for (int c = 0; c < D; ++c) y1[c] = mac(h0, f0[c], y0[c]);
  Rhs::f(y1, p, f1);
#pragma unroll
  for (int c = 0; c < D; ++c) df[c] = f1[c] - f0[c];
  const T d2 = rms<D>(df, sc) / h0;
  const T dm = dmax(d1, d2);
  T h1;
  if (dm <= T(1e-15)) h1 = dmax(T(1e-6), h0 * T(1e-3));
  else h1 = dpow(T(0.01) / dm, T(1.0) / T(q + 1));
  return dmin(T(100.0) * h0, h1);
}

// ---------------------------------------------------------------------------
// Record / forward solve.  Controller: accept iff E <= 1; next step = used
// step * clamp(safety E^(-1/(q+1)), fac_min, fac_max), no growth right after
// a rejection, fac_max when E == 0, fac_min when E is not finite.  Steps land
// exactly on every save time and on t1 (DENSE: on t1 only; the save times
// inside an accepted step are read from its interpolant); t accumulates in
// double.  Accepted steps collect in a chunk in LDS that is written when
// full; after the last step the partial chunk follows.  The zero chunks past
// a lane's last step (unless the caller defers them to da_mesh_pad) are
// written from the end of the log downwards while the lane integrates: one
// chunk row every PadEvery<M> attempts, as long as the row index is at least
// DADJ_PAD_AHEAD times that of the chunk the next attempt would go to
// (attempts >= accepted steps, so the rule needs only the attempt count,
// which all lanes still in the loop share).  While every lane of the wavefront is still in the loop the row
// is the same for all of them, and the wavefront writes its row
// segment with each store covering 1 KB contiguously; once a lane has left,
// each lane writes its own chunk.  A lane that takes more steps than that
// overwrites the zeros later: the wavefront's stores to one address take
// effect in program order.  Spread over the integration, these stores use
// the HBM bandwidth that the arithmetic leaves free; the rows between the
// last step and the lowest zeroed row follow the loop (whole row segments
// where every lane needs the row zeroed).
// ---------------------------------------------------------------------------
// One zero row per attempt: the headline Dopri5 record (Lorenz-63, 2^20
// trajectories) takes 10.6 ms against 11.2 with one row per two attempts,
// Rodas3 on Robertson 1.71 against 1.80 ms.
#ifndef DADJ_PAD_EVERY
#define DADJ_PAD_EVERY 1
#endif
// A zero row is written during the integration only while it lies at least
// DADJ_PAD_AHEAD times the lane's current chunk row up: a row closer than
// that may still receive the lane's own steps, and zeroing it first writes
// it twice (with a factor of one the headline record wrote 37.7 GB for its
// 34.4 GB log).  Rows left over are zeroed after the loop.  Factor 4: the
// FP32 Tsit5 record (65536 trajectories) 0.278 -> 0.258 ms, the headline
// record 10.45 -> 10.28 ms; Rodas3 on Robertson and the kinetics system
// unchanged (factors 2 and 3 in between).
#ifndef DADJ_PAD_AHEAD
#define DADJ_PAD_AHEAD 4
#endif

template <class...> struct VoidT { typedef void type; };

// Methods whose steps exchange rows (the pivoted factorisation of the
// Rosenbrock methods) and that also provide the steps without exchanges
// (M::attempt_nx, M::fwd_nx, M::adj_nx: the same results wherever partial
// pivoting keeps every row in place, and `need` set where it would not).
template <class M, class = void> struct RowX { static constexpr bool value = false; };
template <class M>
struct RowX<M, typename VoidT<decltype(M::row_exchanges)>::type> {
  static constexpr bool value = M::row_exchanges;
};
// The built-in systems (R::built_in); the kernels of right-hand sides
// compiled at run time do not take the gradient kernel's branch-free path
// (their gradient kernels are often near the register limit already).
template <class R, class = void> struct BuiltIn { static constexpr bool value = false; };
template <class R>
struct BuiltIn<R, typename VoidT<decltype(R::built_in)>::type> {
  static constexpr bool value = R::built_in;
};
// One trial step of the record: without row exchanges where the method
// provides it, repeated with the pivoted step in the lanes where partial
// pivoting would have exchanged rows (the same results bit for bit).
template <class M, class T, int D, class Cache>
__device__ __forceinline__ void attempt_x(const T (&y)[D], const T *p, T h, Cache &cache,
                                          T (&ynew)[D], T (&err)[D]) {
  if constexpr (RowX<M>::value) {
    bool need = false;
    M::attempt_nx(y, p, h, cache, ynew, err, need);
    if (need) M::attempt(y, p, h, cache, ynew, err);
  } else {
    M::attempt(y, p, h, cache, ynew, err);
  }
}
// Methods that opt out of the gradient kernel's branch-free path
// (M::branch_free_replay = false).
template <class M, class = void> struct BranchFree { static constexpr bool value = true; };
template <class M>
struct BranchFree<M, typename VoidT<decltype(M::branch_free_replay)>::type> {
  static constexpr bool value = M::branch_free_replay;
};
// Attempts per zero row of the record's inline padding (M::pad_every where
// a method sets it; 0: every zero row after the integration).
template <class M, class = void> struct PadEvery { static constexpr int value = DADJ_PAD_EVERY; };
template <class M>
struct PadEvery<M, typename VoidT<decltype(M::pad_every)>::type> {
  static constexpr int value = M::pad_every;
};
template <class M, class V, class H, int D>
__device__ __forceinline__ void fwd_nx(V (&y)[D], const V *p, H h, bool &need) {
  if constexpr (RowX<M>::value) M::fwd_nx(y, p, h, need);
  else M::fwd(y, p, h);
}
template <class M, class T, int D>
__device__ __forceinline__ void adj_nx(const T (&y)[D], const T *p, T h, T (&lam)[D], T *g,
                                       bool &need) {
  if constexpr (RowX<M>::value) M::adj_nx(y, p, h, lam, g, need);
  else M::adj(y, p, h, lam, g);
}

template <class T, class M, bool LOG, bool DENSE>
__global__ __launch_bounds__(BLOCK) void k_record(RecordArgs a, SaveTimes stimes) {
  using Rhs = typename M::Rhs;
  constexpr int D = Rhs::D, P = Rhs::P;
  constexpr int B = Log<T>::B;
  const int64_t n = a.n;
  const int64_t i = (int64_t)blockIdx.x * BLOCK + threadIdx.x;
  const bool live = i < n;
  const ProbArgs &pr = a.pr;
  const int S = pr.S;
  const bool has_saves = pr.n_save > 0;
  const int n_stops = S + ((has_saves && stimes.t[pr.n_save - 1] < pr.t1) ? 1 : 0);
  const T atol = T(pr.atol), rtol = T(pr.rtol);
  const T expo = T(-1.0) / T(M::err_order + 1);
  const T safety = T(pr.safety), fmin = T(pr.fac_min), fmax = T(pr.fac_max);
  const T *u0 = (const T *)a.u0;
  const T *pp = (const T *)a.p;
  T *H = (T *)a.h;
  T *ysave = (T *)a.y_save;
  T *theta = (T *)a.theta;

  int nacc = 0, natt = 0, st = LANE_OK;
  constexpr int PE = PadEvery<M>::value;
  const bool pad = LOG && !a.defer_pad && PE > 0;  // (uniform)
  int zl = pr.n_chunks;  // rows [zl, n_chunks) of this lane are zero
  // The lane's chunk of accepted steps, filled one position per accepted
  // step and written to the log when full ([position][thread]: each thread
  // reads back only its own column).  In registers it took 16 more VGPRs
  // and a select per position on every accepted step.
  __shared__ T lchunk[LOG ? B : 1][BLOCK];
  if (live) {
    T y[D], p[P], ynew[D], err[D];
    typename M::template Cache<T> cache;
    bool fin = true;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      y[c] = u0[c * n + i];
      fin = fin && finite(y[c]);
    }
#pragma unroll
    for (int q = 0; q < P; ++q) {
      p[q] = pp[q * n + i];
      fin = fin && finite(p[q]);
    }
    for (int s = 0; s < S; ++s) {
      if (a.sidx) a.sidx[s * n + i] = -1;
      if (theta) theta[s * n + i] = nanv<T>();
      if (ysave)
#pragma unroll
        for (int c = 0; c < D; ++c) ysave[(s * D + c) * n + i] = nanv<T>();
    }
    if (!fin) {
      st = LANE_NONFINITE;
    } else {
      T f0[D];
      Rhs::f(y, p, f0);
      M::begin(y, p, f0, cache);
      T h = pr.dt0 > 0 ? T(pr.dt0) : initial_step<Rhs>(y, f0, p, atol, rtol, M::order);
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
        if (pad && natt % (PE > 0 ? PE : 1) == 0 && zl - 1 >= (DADJ_PAD_AHEAD * natt) / B) {
          --zl;
          if (__ballot(1) == ~0ull) {
            const int lane = (int)(threadIdx.x & 63u);
            zero_row_segment(H + ((int64_t)zl * n + (i - lane)) * B, lane);
          } else {
            T zb[B];
#pragma unroll
            for (int b = 0; b < B; ++b) zb[b] = T(0);
            store_chunk(H + ((int64_t)zl * n + i) * B, zb);
          }
        }
        attempt_x<M>(y, p, hs, cache, ynew, err);
        const T E = err_norm<D>(err, y, ynew, atol, rtol);
        if (E <= T(1)) {
          const double t_new = land ? t_stop : t + double(hs);
          if (LOG) {
            const int pos = nacc % B;
            lchunk[pos][threadIdx.x] = hs;
            if (pos == B - 1)
              store_chunk_lds(H + ((int64_t)(nacc / B) * n + i) * B, lchunk, threadIdx.x);
          }
          ++nacc;
          if constexpr (DENSE) {
            // the save times inside this step
            for (; has_saves && js < S && stimes.t[js] <= t_new; ++js) {
              const T th = T(step_fraction(stimes.t[js], t, t_new, double(hs)));
              if (a.sidx) a.sidx[js * n + i] = nacc;
              if (theta) theta[js * n + i] = th;
              if (ysave) {
                T ys[D];
                dense_value<Rhs>(th, hs, y, ynew, p, ys);
#pragma unroll
                for (int c = 0; c < D; ++c) ysave[(js * D + c) * n + i] = ys[c];
              }
            }
          }
#pragma unroll
          for (int c = 0; c < D; ++c) y[c] = ynew[c];
          M::accepted(cache);
          t = t_new;
          T fac = (E == T(0)) ? fmax : dmin(fmax, dmax(fmin, safety * ctrl_pow(E, expo)));
          if (after_reject) fac = dmin(fac, T(1));
          h = hs * fac;
          after_reject = false;
          if (DENSE && land) {
            if (!has_saves) {  // the final state is the one save
              if (a.sidx) a.sidx[i] = nacc;
              if (theta) theta[i] = T(1);
              if (ysave)
#pragma unroll
                for (int c = 0; c < D; ++c) ysave[c * n + i] = y[c];
            }
            break;
          }
          if (land) {
            if (js < S) {
              if (a.sidx) a.sidx[js * n + i] = nacc;
              if (theta) theta[js * n + i] = T(1);
              if (ysave)
#pragma unroll
                for (int c = 0; c < D; ++c) ysave[(js * D + c) * n + i] = y[c];
            }
            if (++js == n_stops) break;
          }
        } else {
          const T fac = finite(E) ? dmax(fmin, safety * ctrl_pow(E, expo)) : fmin;
          h = hs * fac;
          after_reject = true;
        }
      }
    }
    if (a.nsteps) a.nsteps[i] = nacc;
    if (a.status) a.status[i] = st;
    if (a.natt) a.natt[i] = natt;
    if (LOG && nacc % B != 0)
      store_chunk_lds(H + ((int64_t)(nacc / B) * n + i) * B, lchunk, threadIdx.x, nacc % B);
  }
  if (LOG && !a.defer_pad) {  // (a kernel argument: uniform)
    // the zero chunks from each lane's first chunk past its last step up to
    // its lowest zeroed row, chunk row by chunk row across the wavefront.
    // Rows [lo, hi) are zero for every lane: there the wavefront writes its
    // row segment (64 chunks) with each store covering 1 KB contiguously (the data
    // is zeros, so which lane writes which bytes does not matter); elsewhere
    // each lane writes its own chunk.
    const int Tn = pr.n_chunks;
    const int mine = live ? (nacc + B - 1) / B : Tn;
    const int upto = live ? zl : Tn;
    int tmin = mine, tmax = upto, lo = mine, hi = upto;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const int o = __shfl_xor(tmin, off, 64);
      const int u = __shfl_xor(tmax, off, 64);
      const int ol = __shfl_xor(lo, off, 64);
      const int oh = __shfl_xor(hi, off, 64);
      tmin = o < tmin ? o : tmin;
      tmax = u > tmax ? u : tmax;
      lo = ol > lo ? ol : lo;
      hi = oh < hi ? oh : hi;
    }
    tmin = __builtin_amdgcn_readfirstlane(tmin);
    tmax = __builtin_amdgcn_readfirstlane(tmax);
    lo = __builtin_amdgcn_readfirstlane(lo);
    hi = __builtin_amdgcn_readfirstlane(hi);
    T zb[B];
#pragma unroll
    for (int b = 0; b < B; ++b) zb[b] = T(0);
    // a lane past n has mine = upto = Tn, so a partial wavefront has lo = Tn
    const bool whole = lo < hi;
    const int a1 = whole ? lo : tmax;
    for (int t = tmin; t < a1; ++t)
      if (t >= mine && t < upto) store_chunk(H + ((int64_t)t * n + i) * B, zb);
    if (whole) {
      const int lane = (int)(threadIdx.x & 63u);
      const int64_t i0 = i - lane;  // the wavefront's first trajectory
      for (int t = lo; t < hi; ++t) zero_row_segment(H + ((int64_t)t * n + i0) * B, lane);
      for (int t = hi; t < tmax; ++t)
        if (t >= mine && t < upto) store_chunk(H + ((int64_t)t * n + i) * B, zb);
    }
  }
}

// ---------------------------------------------------------------------------
// Where a replay lane finds its step sizes: a row of the replay table (one
// contiguous row segment per wavefront and step) or its trajectory's chunks
// of the tiled log.  `cap` is the number of steps the source holds; loads
// are clamped to it so that prefetches past the end stay in bounds.
// ---------------------------------------------------------------------------
template <class T, bool ROWS> struct StepSrc {
  typedef __attribute__((address_space(1))) const T GT;  // global memory
  GT *base;
  int64_t n;
  int cap;
  __device__ __forceinline__ void init(const ReplayArgs &a, int64_t j, int64_t tr) {
    n = a.n;
    if constexpr (ROWS) {
      base = (GT *)a.h_rows + j;
      cap = a.rows;
    } else {
      base = (GT *)a.h + tr * Log<T>::B;
      cap = a.pr.n_chunks * Log<T>::B;
    }
  }
  __device__ __forceinline__ T load(int k) const {
    k = k < cap ? k : cap - 1;
    k = k < 0 ? 0 : k;
    if constexpr (ROWS) return base[(int64_t)k * n];
    else return base[Log<T>::at(k, n)];
  }
  // Steps k .. k + V - 1 (k a multiple of V): from the tiled log, V
  // consecutive elements of one chunk read by 16-byte loads; from the table,
  // V row loads.  A start past the source reads its last V steps.
  template <int V> __device__ __forceinline__ void loadv(int k, T (&out)[V]) const {
    constexpr int PER = 16 / (int)sizeof(T);  // elements per 16-byte piece
    if constexpr (ROWS || V % PER != 0) {
#pragma unroll
      for (int v = 0; v < V; ++v) out[v] = load(k + v);
    } else {
      k = k < cap - V ? k : cap - V;
      k = k < 0 ? 0 : k;
      typedef T Piece __attribute__((ext_vector_type(PER)));
      typedef __attribute__((address_space(1))) const Piece GP;
      GP *q = (GP *)(base + Log<T>::at(k, n));
#pragma unroll
      for (int r = 0; r < V / PER; ++r) {
        const Piece x = q[r];
#pragma unroll
        for (int e = 0; e < PER; ++e) out[r * PER + e] = x[e];
      }
    }
  }
};

// Lane j of a replay: its trajectory, step count and whether it replays.
// Lanes that need more steps than the step source holds (or than `limit`),
// and with `need_ok` lanes whose record failed, replay nothing and report
// NaN.
struct LaneInfo {
  int64_t tr;
  int N;
  bool ok;
};
__device__ __forceinline__ LaneInfo lane_info(const ReplayArgs &a, int64_t j, bool live,
                                              int limit, bool need_ok) {
  LaneInfo L{0, 0, false};
  if (live) {
    L.tr = a.perm ? a.perm[j] : j;
    const int N = a.nsteps[L.tr];
    const int cap = a.h_rows ? a.rows : a.pr.max_steps;
    L.ok = (!need_ok || a.status[L.tr] == LANE_OK) && N >= 0 && N <= cap && N <= limit;
    L.N = L.ok ? N : 0;
  }
  return L;
}

// ---------------------------------------------------------------------------
// Replay forward: the state after save_idx[s] steps goes to y_save[s]; save
// slots whose index lies outside [0, n_steps], and every slot of a lane that
// does not replay, get NaN.  DENSE: a save with index k >= 1 is the
// interpolant of step k - 1 at its recorded fraction.  Two steps per loop
// trip so that the step size of the next step is loaded into the register
// the next step reads (no copy, so no wait on the load until that step).
// ---------------------------------------------------------------------------
template <class T, class M, bool ROWS, bool DENSE>
__global__ __launch_bounds__(BLOCK) void k_replay_fwd(ReplayArgs a) {
  using Rhs = typename M::Rhs;
  constexpr int D = Rhs::D, P = Rhs::P;
  const int64_t n = a.n;
  const int64_t j = (int64_t)blockIdx.x * BLOCK + threadIdx.x;
  const bool live = j < n;
  const int S = a.pr.S;
  T *ysave = (T *)a.y_save;
  const LaneInfo L = lane_info(a, j, live, a.pr.max_steps, false);
  const int64_t tr = L.tr;
  const int N = L.N;
  StepSrc<T, ROWS> src;
  src.init(a, live ? j : 0, tr);
  T y[D], p[P];
  if (live) {
#pragma unroll
    for (int c = 0; c < D; ++c) y[c] = ((const T *)a.u0)[c * n + tr];
#pragma unroll
    for (int q = 0; q < P; ++q) p[q] = ((const T *)a.p)[q * n + tr];
    for (int q = 0; q < S; ++q) {
      const int ix = a.sidx[q * n + tr];
      if (!L.ok || ix < 0 || ix > N)
#pragma unroll
        for (int c = 0; c < D; ++c) ysave[(q * D + c) * n + tr] = nanv<T>();
    }
  }
  const int Nw = wave_max(N);
  int s = 0;
  int nxt = L.ok ? a.sidx[tr] : -1;
  auto save = [&](int k, const T (&yk)[D]) {
    while (s < S && nxt == k) {
#pragma unroll
      for (int c = 0; c < D; ++c) ysave[(s * D + c) * n + tr] = yk[c];
      ++s;
      nxt = s < S ? a.sidx[s * n + tr] : -1;
    }
  };
  save(0, y);
  // DENSE: the saves inside step k, from the state yp before it
  auto dsave = [&](int k, const T (&yp)[D], T hk) {
    while (s < S && nxt == k + 1) {
      T ys[D];
      dense_value<Rhs>(((const T *)a.theta)[(int64_t)s * n + tr], hk, yp, y, p, ys);
#pragma unroll
      for (int c = 0; c < D; ++c) ysave[(s * D + c) * n + tr] = ys[c];
      ++s;
      nxt = s < S ? a.sidx[s * n + tr] : -1;
    }
  };
  auto step = [&](int k, T hk) {
    if (k < N) {
      if constexpr (DENSE) {
        T yp[D];
#pragma unroll
        for (int c = 0; c < D; ++c) yp[c] = y[c];
        M::fwd(y, p, hk);
        dsave(k, yp, hk);
      } else {
        M::fwd(y, p, hk);
        save(k + 1, y);
      }
    }
  };
  // Branch-free units (built-in systems of up to four components, no dense
  // output), as in the gradient kernel: below the smallest step count of
  // the wavefront's trajectories, eight steps at a time with no per-lane
  // guard and, for methods with row exchanges, without exchanges; a unit in
  // which some lane would have exchanged rows is repeated with M::fwd.  Same
  // arithmetic as `step`; the saves of the unit's states follow it.
  constexpr bool FAST = !DENSE && D <= 4 && BuiltIn<Rhs>::value && BranchFree<M>::value;
  int k0 = 0;
  if constexpr (FAST) {
    constexpr int U = 8;
    const int Nmin = wave_min(N);
    T hc[U];
    src.template loadv<U>(0, hc);
    for (; k0 + U <= Nmin; k0 += U) {
      T hn[U], ys[U + 1][D];
      src.template loadv<U>(k0 + U, hn);
#pragma unroll
      for (int c = 0; c < D; ++c) ys[0][c] = y[c];
      bool need = false;
#pragma unroll
      for (int b = 0; b < U; ++b) {
#pragma unroll
        for (int c = 0; c < D; ++c) ys[b + 1][c] = ys[b][c];
        fwd_nx<M>(ys[b + 1], p, hc[b], need);
      }
      if constexpr (RowX<M>::value) {
        if (__ballot(need) != 0ull) {
#pragma unroll
          for (int b = 0; b < U; ++b) {
#pragma unroll
            for (int c = 0; c < D; ++c) ys[b + 1][c] = ys[b][c];
            M::fwd(ys[b + 1], p, hc[b]);
          }
        }
      }
#pragma unroll
      for (int b = 1; b <= U; ++b) save(k0 + b, ys[b]);
#pragma unroll
      for (int c = 0; c < D; ++c) y[c] = ys[U][c];
#pragma unroll
      for (int b = 0; b < U; ++b) hc[b] = hn[b];
    }
  }
  T hA = src.load(k0);
  for (int k = k0; k < Nw; k += 2) {
    const T hB = src.load(k + 1);
    step(k, hA);
    hA = src.load(k + 2);
    if (k + 1 < Nw) step(k + 1, hB);
  }
}

// ---------------------------------------------------------------------------
// Replay + reverse sweep
// ---------------------------------------------------------------------------
template <class T, int D>
__device__ __forceinline__ void loss_terms(int lk, const T (&y)[D], const T *aux, int64_t n, int s,
                                           int64_t tr, T &ss, bool &first) {
#pragma unroll
  for (int c = 0; c < D; ++c) {
    const T av = aux[((int64_t)s * D + c) * n + tr];
    if (lk == DA_LOSS_MSE_SAVE) {
      const T r = y[c] - av;
      ss = first ? r * r : mac(r, r, ss);
    } else {
      ss = first ? av * y[c] : mac(av, y[c], ss);
    }
    first = false;
  }
}

template <class T, int D>
__device__ __forceinline__ void seed_terms(int lk, const T (&y)[D], const T *aux, int64_t n, int s,
                                           int64_t tr, double scale, T (&lam)[D]) {
#pragma unroll
  for (int c = 0; c < D; ++c) {
    const T av = aux[((int64_t)s * D + c) * n + tr];
    if (lk == DA_LOSS_MSE_SAVE) lam[c] = mac(T(2.0 * scale), y[c] - av, lam[c]);
    else lam[c] = mac(T(scale), av, lam[c]);
  }
}

// loss_terms and seed_terms with the save's targets (MSE) or cotangents
// already in registers (the same arithmetic).
template <class T, int D>
__device__ __forceinline__ void loss_terms_v(int lk, const T (&y)[D], const T (&av)[D], T &ss,
                                             bool &first) {
#pragma unroll
  for (int c = 0; c < D; ++c) {
    if (lk == DA_LOSS_MSE_SAVE) {
      const T r = y[c] - av[c];
      ss = first ? r * r : mac(r, r, ss);
    } else {
      ss = first ? av[c] * y[c] : mac(av[c], y[c], ss);
    }
    first = false;
  }
}
template <class T, int D>
__device__ __forceinline__ void seed_terms_v(int lk, const T (&y)[D], const T (&av)[D],
                                             double scale, T (&lam)[D]) {
#pragma unroll
  for (int c = 0; c < D; ++c) {
    if (lk == DA_LOSS_MSE_SAVE) lam[c] = mac(T(2.0 * scale), y[c] - av[c], lam[c]);
    else lam[c] = mac(T(scale), av[c], lam[c]);
  }
}

// The save slots of one trajectory walked forward (the loss terms of the
// forward replay, dir = +1) or backward (the seeds of the reverse sweep,
// dir = -1): the step index and the targets or cotangents of the current
// slot q and of the next one, in registers.  The next slot's are loaded when
// the current one is taken, so that taking a save (one every few steps, at
// scattered trajectory positions in replay order) waits on no load.  Slots
// outside [0, S) read slot 0 or S - 1 (inside the buffers, never taken).
template <class T, int D> struct SaveWalk {
  int q = 0, idx = -1, idx2 = -1;
  T av[D], av2[D];
  __device__ __forceinline__ static void load(const ReplayArgs &a, int64_t tr, int r, int &i,
                                              T (&v)[D]) {
    const int S = a.pr.S;
    const int rc = r < 0 ? 0 : (r >= S ? S - 1 : r);
    i = a.sidx[(int64_t)rc * a.n + tr];
    const T *aux = (const T *)a.aux;
#pragma unroll
    for (int c = 0; c < D; ++c) v[c] = aux ? aux[((int64_t)rc * D + c) * a.n + tr] : T(0);
  }
  __device__ __forceinline__ void start(const ReplayArgs &a, int64_t tr, int q0, int dir) {
    q = q0;
    load(a, tr, q0, idx, av);
    load(a, tr, q0 + dir, idx2, av2);
  }
  __device__ __forceinline__ void take(const ReplayArgs &a, int64_t tr, int dir) {
    q += dir;
    idx = idx2;
#pragma unroll
    for (int c = 0; c < D; ++c) av[c] = av2[c];
    load(a, tr, q + dir, idx2, av2);
  }
};

// Workspace: checkpoint m (the state before step m * CK) of local lane jl at
// ws[(m * D + c) * ws_lanes + jl].  The forward replay writes the
// checkpoints; the reverse sweep walks the segments of CK steps from the
// last, recomputes the segment's states from its checkpoint in registers and
// runs the adjoint of its steps in reverse.  Segments are taken two per loop
// trip from two register sets (A, B): while one segment computes, the loads
// of the next one (its checkpoint and step sizes) are in flight.
template <class T, int D, int CK> struct Seg {
  T cp[D], h[CK];
};

// Reverse of one dense save inside the step from yk to yk1 (size h, fraction
// th), with sb = dL/dy(t_s) the save's seed:
//   lam (dL/dy_{k+1}) += H01 sb + J(yk1)^T v1,  v1 = (h H11) sb
//   mu  (the part of dL/dy_k that bypasses the step) += H00 sb + J(yk)^T v0,
//                                               v0 = (h H10) sb
//   g += J_p(yk1)^T v1, then g += J_p(yk)^T v0.
template <class Rhs, class T>
__device__ __forceinline__ void dense_seed(int lk, T th, T h, const T (&yk)[Rhs::D],
                                           const T (&yk1)[Rhs::D], const T *p, const T *aux,
                                           int64_t n, int s, int64_t tr, double scale,
                                           T (&lam)[Rhs::D], T (&mu)[Rhs::D], T *g) {
  constexpr int D = Rhs::D;
  T ys[D], sb[D], v0[D], v1[D], w0[D], w1[D];
  dense_value<Rhs>(th, h, yk, yk1, p, ys);
#pragma unroll
  for (int c = 0; c < D; ++c) sb[c] = T(0);
  seed_terms<T, D>(lk, ys, aux, n, s, tr, scale, sb);
  const HermiteW<T> w = hermite_w(th);
  const T c1 = h * w.h11, c0 = h * w.h10;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    v1[c] = c1 * sb[c];
    v0[c] = c0 * sb[c];
  }
  Rhs::vjp_y(yk1, p, v1, w1);
  Rhs::vjp_y(yk, p, v0, w0);
#pragma unroll
  for (int c = 0; c < D; ++c) {
    lam[c] = mac(w.h01, sb[c], lam[c]) + w1[c];
    mu[c] = mac(w.h00, sb[c], mu[c]) + w0[c];
  }
  Rhs::vjp_p_acc(yk1, p, v1, g);
  Rhs::vjp_p_acc(yk, p, v0, g);
}

template <class T, class M, int CK, bool ROWS, bool DENSE>
__global__ __launch_bounds__(BLOCK) DADJ_GRAD_OCCUPANCY void k_replay_grad(ReplayArgs a) {
  using Rhs = typename M::Rhs;
  constexpr int D = Rhs::D, P = Rhs::P;
  const int64_t n = a.n;
  const int64_t jl = (int64_t)blockIdx.x * BLOCK + threadIdx.x;
  const bool live = jl < a.nslots;
  const int64_t j = a.slot0 + jl;
  const int64_t C = a.ws_lanes;
  const int S = a.pr.S;
  const int lk = a.loss_kind;
  const bool saves = lk != DA_LOSS_SUMSQ_FINAL;  // loss terms at save indices
  const T *aux = (const T *)a.aux;
  // lanes past the end read (and never use) lane 0's workspace column, so
  // that the unconditional prefetches below stay inside the workspace
  T *ws = (T *)a.ws + (live ? jl : 0);
  const LaneInfo L = lane_info(a, j, live, a.max_n_steps, true);
  const int64_t tr = L.tr;
  const int N = L.N;
  const bool ok = L.ok;
  StepSrc<T, ROWS> src;
  src.init(a, live ? j : a.slot0, tr);
  T y[D], p[P];
  if (live) {
#pragma unroll
    for (int c = 0; c < D; ++c) y[c] = ((const T *)a.u0)[c * n + tr];
#pragma unroll
    for (int q = 0; q < P; ++q) p[q] = ((const T *)a.p)[q * n + tr];
  }
  const int Nw = wave_max(N);

  // ---- forward replay, keeping every CK-th state; loss terms at the saves ----
  // Built-in systems of up to four components without dense output walk the
  // saves with SaveWalk (targets loaded ahead); dense output, larger systems
  // (whose registers are full) and the kernels of registered right-hand
  // sides read each save's step index and targets when they reach it, as
  // these kernels always have (their code is kept unchanged: see BuiltIn).
  constexpr bool PF = BuiltIn<Rhs>::value && !DENSE && D <= 4;
  T ss = T(0);
  bool first = true;
  const int Sl = (ok && saves) ? S : 0;  // save slots this trajectory takes
  SaveWalk<T, D> fw;
  int s = 0;
  int nxt = (ok && saves) ? a.sidx[tr] : -1;
  if (PF && saves) fw.start(a, tr, 0, 1);
  auto terms = [&](int k, const T (&yk)[D]) {
    if constexpr (PF) {
      while (fw.q < Sl && fw.idx == k) {
        loss_terms_v<T, D>(lk, yk, fw.av, ss, first);
        fw.take(a, tr, 1);
      }
    } else {
      while (s < S && nxt == k) {
        loss_terms<T, D>(lk, yk, aux, n, s, tr, ss, first);
        ++s;
        nxt = s < S ? a.sidx[s * n + tr] : -1;
      }
    }
  };
  if (saves) terms(0, y);
  const T *theta = (const T *)a.theta;
  // DENSE: loss terms of the saves inside step k, from the state yp before it
  auto dterms = [&](int k, const T (&yp)[D], T hk) {
    if constexpr (PF) {
      while (fw.q < Sl && fw.idx == k + 1) {
        T ys[D];
        dense_value<Rhs>(theta[(int64_t)fw.q * n + tr], hk, yp, y, p, ys);
        loss_terms_v<T, D>(lk, ys, fw.av, ss, first);
        fw.take(a, tr, 1);
      }
    } else {
      while (s < S && nxt == k + 1) {
        T ys[D];
        dense_value<Rhs>(theta[(int64_t)s * n + tr], hk, yp, y, p, ys);
        loss_terms<T, D>(lk, ys, aux, n, s, tr, ss, first);
        ++s;
        nxt = s < S ? a.sidx[s * n + tr] : -1;
      }
    }
  };
  auto fstep = [&](int k, T hk) {
    if (k < N) {
      if (k % CK == 0) {
        T *wk = ws + (int64_t)(k / CK) * D * C;
#pragma unroll
        for (int c = 0; c < D; ++c) wk[c * C] = y[c];
      }
      if constexpr (DENSE) {
        T yp[D];
#pragma unroll
        for (int c = 0; c < D; ++c) yp[c] = y[c];
        M::fwd(y, p, hk);
        dterms(k, yp, hk);
      } else {
        M::fwd(y, p, hk);
        if (saves) terms(k + 1, y);
      }
    }
  };
  // Branch-free path (built-in systems of at most 4 components, checkpoint
  // interval 1, 2 or 4, no loss terms at saves, no dense output; beyond
  // these the registers of a unit spill): the steps below every lane's step
  // count (Nmin) run U at a time with no per-lane guard and, for methods
  // with row exchanges, without exchanges; if some lane would have exchanged
  // rows, the unit is repeated with M::fwd.  Same arithmetic as fstep, so
  // the same results bit for bit.
  constexpr bool PX = RowX<M>::value;
  constexpr bool FAST =
      !DENSE && CK <= 4 && D <= 4 && BuiltIn<Rhs>::value && BranchFree<M>::value;
  constexpr int U = 8;  // a multiple of CK; measured against 4 and 16
  static_assert(!FAST || U % CK == 0, "a forward unit holds whole checkpoint segments");
  const bool fast = FAST && !saves;
  const int Nmin = FAST ? wave_min(N) : 0;
  int k0 = 0;
  if constexpr (FAST) if (fast) {
    T hc[U];
    src.template loadv<U>(0, hc);
    for (; k0 + U <= Nmin; k0 += U) {
      T hn[U], ys[U + 1][D];
      src.template loadv<U>(k0 + U, hn);
#pragma unroll
      for (int c = 0; c < D; ++c) ys[0][c] = y[c];
      bool need = false;
#pragma unroll
      for (int b = 0; b < U; ++b) {
#pragma unroll
        for (int c = 0; c < D; ++c) ys[b + 1][c] = ys[b][c];
        fwd_nx<M>(ys[b + 1], p, hc[b], need);
      }
      if constexpr (PX) {
        if (__ballot(need) != 0ull) {
#pragma unroll
          for (int b = 0; b < U; ++b) {
#pragma unroll
            for (int c = 0; c < D; ++c) ys[b + 1][c] = ys[b][c];
            M::fwd(ys[b + 1], p, hc[b]);
          }
        }
      }
#pragma unroll
      for (int b = 0; b < U; b += CK) {
        T *wk = ws + (int64_t)((k0 + b) / CK) * D * C;
#pragma unroll
        for (int c = 0; c < D; ++c) wk[c * C] = ys[b][c];
      }
#pragma unroll
      for (int c = 0; c < D; ++c) y[c] = ys[U][c];
#pragma unroll
      for (int b = 0; b < U; ++b) hc[b] = hn[b];
    }
  }
  {
    T hA = src.load(k0);
    for (int k = k0; k < Nw; k += 2) {
      const T hB = src.load(k + 1);
      fstep(k, hA);
      hA = src.load(k + 2);
      if (k + 1 < Nw) fstep(k + 1, hB);
    }
  }

  // ---- loss and seeds at the final state ----
  T lam[D], g[P];
#pragma unroll
  for (int q = 0; q < P; ++q) g[q] = T(0);
  if (!saves) {
#pragma unroll
    for (int c = 0; c < D; ++c) ss = (c == 0) ? y[c] * y[c] : mac(y[c], y[c], ss);
#pragma unroll
    for (int c = 0; c < D; ++c) lam[c] = T(2.0 * a.scale) * y[c];
  } else {
#pragma unroll
    for (int c = 0; c < D; ++c) lam[c] = T(0);
  }
  SaveWalk<T, D> bw;
  if (PF && saves) bw.start(a, tr, S - 1, -1);
  bw.q = Sl - 1;
  int sh = S - 1;
  int hidx = (ok && saves) ? a.sidx[(int64_t)sh * n + tr] : -1;
  auto seeds = [&](int k, const T (&yk)[D]) {
    if constexpr (PF) {
      while (bw.q >= 0 && bw.idx == k) {
        seed_terms_v<T, D>(lk, yk, bw.av, a.scale, lam);
        bw.take(a, tr, -1);
      }
    } else {
      while (sh >= 0 && hidx == k) {
        seed_terms<T, D>(lk, yk, aux, n, sh, tr, a.scale, lam);
        --sh;
        hidx = sh >= 0 ? a.sidx[(int64_t)sh * n + tr] : -1;
      }
    }
  };
  if (saves && !DENSE) seeds(N, y);
  // DENSE: y_{k+1} while step k is reversed (starts as the final state)
  T yhi[D];
#pragma unroll
  for (int c = 0; c < D; ++c) yhi[c] = y[c];

  // ---- reverse sweep, one segment of CK steps at a time ----
  // Every index stays inside the buffers: segments m < Mw = ceil(Nw / CK);
  // the workspace holds ceil(max_n_steps / CK) >= Mw checkpoints; step loads
  // are clamped to the step source.
  const int Mw = (Nw + CK - 1) / CK;
  auto fetch = [&](int m, Seg<T, D, CK> &sg) {
    m = m < 0 ? 0 : m;
#pragma unroll
    for (int c = 0; c < D; ++c) sg.cp[c] = ws[((int64_t)m * D + c) * C];
#pragma unroll
    for (int b = 0; b < CK; ++b) sg.h[b] = src.load(m * CK + b);
  };
  auto fetchv = [&](int m, Seg<T, D, CK> &sg) {
    m = m < 0 ? 0 : m;
#pragma unroll
    for (int c = 0; c < D; ++c) sg.cp[c] = ws[((int64_t)m * D + c) * C];
    src.template loadv<CK>(m * CK, sg.h);
  };
  auto rseg = [&](int m, const Seg<T, D, CK> &sg) {
    T ys[CK][D];
#pragma unroll
    for (int c = 0; c < D; ++c) ys[0][c] = sg.cp[c];
#pragma unroll
    for (int b = 1; b < CK; ++b) {
#pragma unroll
      for (int c = 0; c < D; ++c) ys[b][c] = ys[b - 1][c];
      if (m * CK + b - 1 < N) M::fwd(ys[b], p, sg.h[b - 1]);
    }
#pragma unroll
    for (int b = CK - 1; b >= 0; --b) {
      const int k = m * CK + b;
      if (k < N) {
        if constexpr (DENSE) {
          // the saves inside step k, the last first: into lam now, into mu
          // (joining lam after the step's reverse) for the y_k part
          T mu[D];
          bool has_mu = false;
          while (sh >= 0 && hidx == k + 1) {
            if (!has_mu) {
#pragma unroll
              for (int c = 0; c < D; ++c) mu[c] = T(0);
            }
            has_mu = true;
            dense_seed<Rhs>(lk, theta[(int64_t)sh * n + tr], sg.h[b], ys[b], yhi, p, aux, n, sh,
                            tr, a.scale, lam, mu, g);
            --sh;
            hidx = sh >= 0 ? a.sidx[(int64_t)sh * n + tr] : -1;
          }
          M::adj(ys[b], p, sg.h[b], lam, g);
          if (has_mu) {
#pragma unroll
            for (int c = 0; c < D; ++c) lam[c] = lam[c] + mu[c];
          }
          if (k == 0) seeds(0, ys[b]);
#pragma unroll
          for (int c = 0; c < D; ++c) yhi[c] = ys[b][c];
        } else {
          M::adj(ys[b], p, sg.h[b], lam, g);
          if (saves) seeds(k, ys[b]);
        }
      }
    }
  };
  // Branch-free segment: no per-lane guard, no row exchanges (`need` set
  // where partial pivoting would exchange rows).
  auto rseg_nx = [&](const Seg<T, D, CK> &sg, bool &need) {
    T ys[CK][D];
#pragma unroll
    for (int c = 0; c < D; ++c) ys[0][c] = sg.cp[c];
#pragma unroll
    for (int b = 1; b < CK; ++b) {
#pragma unroll
      for (int c = 0; c < D; ++c) ys[b][c] = ys[b - 1][c];
      fwd_nx<M>(ys[b], p, sg.h[b - 1], need);
    }
#pragma unroll
    for (int b = CK - 1; b >= 0; --b) adj_nx<M>(ys[b], p, sg.h[b], lam, g, need);
  };
  if (Mw > 0) {
    Seg<T, D, CK> A, B;
    fetch(Mw - 1, A);
    int m = Mw - 1;
    // pairs of segments that hold some lane's last step, or everything when
    // the branch-free path is off: guarded
    for (; m >= 0 && !(fast && (m + 1) * CK <= Nmin); m -= 2) {
      fetch(m - 1, B);
      rseg(m, A);
      fetch(m - 2, A);
      if (m - 1 >= 0) rseg(m - 1, B);
    }
    // segments below every lane's step count: branch-free, one segment at a
    // time (a pair of one-step segments at checkpoint interval 1; measured
    // faster than pairs at intervals 2 and 4); with row exchanges, repeated
    // through rseg (from the saved lam and g, the segment read again) if some
    // lane would have exchanged rows
    constexpr int SP = CK == 1 ? 2 : 1;  // segments per check
    if constexpr (FAST) for (; m >= SP - 1; m -= SP) {
      T lam0[D], g0[P];
      if constexpr (PX) {
#pragma unroll
        for (int c = 0; c < D; ++c) lam0[c] = lam[c];
#pragma unroll
        for (int q = 0; q < P; ++q) g0[q] = g[q];
      }
      bool need = false;
      fetchv(m - 1, B);
      rseg_nx(A, need);
      if constexpr (SP == 2) {
        fetchv(m - 2, A);
        rseg_nx(B, need);
      }
      if constexpr (PX) {
        if (__ballot(need) != 0ull) {
#pragma unroll
          for (int c = 0; c < D; ++c) lam[c] = lam0[c];
#pragma unroll
          for (int q = 0; q < P; ++q) g[q] = g0[q];
          Seg<T, D, CK> R;
#pragma unroll
          for (int i = 0; i < SP; ++i) {
            fetch(m - i, R);
            rseg(m - i, R);
          }
        }
      }
      if constexpr (SP == 1) A = B;
    }
    if (m == 0) rseg(0, A);
  }

  if (live) {
    const T Lv = ok ? T(a.scale) * ss : nanv<T>();
    if (a.loss_out) ((T *)a.loss_out)[tr] = Lv;
    if (a.gu0)
#pragma unroll
      for (int c = 0; c < D; ++c) ((T *)a.gu0)[c * n + tr] = ok ? lam[c] : nanv<T>();
    if (a.gp)
#pragma unroll
      for (int q = 0; q < P; ++q) ((T *)a.gp)[q * n + tr] = ok ? g[q] : nanv<T>();
  }
}

// ---------------------------------------------------------------------------
// The replay gradient with two wavefronts per 64 trajectories, for ensembles
// that give the one-wavefront kernel about one wavefront per SIMD (65536
// trajectories), where a step's serial chain of dependent operations leaves
// the SIMD idle most of the time.
//  - Forward replay: each wavefront replays 32 of the 64 trajectories
//    (storing every state), so both are busy wherever the hardware places
//    them; the final seeds, loss sums and save cursors then pass through LDS.
//  - Reverse sweep: the first wavefront runs the adjoint of all 64 while the
//    second recomputes the forward stages of each step (M::pre) one step
//    ahead and hands them over through LDS, so that the recomputation of
//    step k - 1 runs beside the adjoint of step k (M::adj_pre).
// Checkpoint interval 1, no dense output.  The arithmetic is that of
// k_replay_grad<T, M, 1, ROWS, false> (M::adj is M::pre followed by
// M::adj_pre), so the results are the same bit for bit.  Both wavefronts
// pass the same barriers: the reverse sweep's trip count is the maximum over
// the same 64 trajectories in both.
// ---------------------------------------------------------------------------
template <class T, class M, bool ROWS>
__global__ __launch_bounds__(128) void k_replay_grad2(ReplayArgs a) {
  using Rhs = typename M::Rhs;
  using Q = typename M::template Pre<T>;
  constexpr int D = Rhs::D, P = Rhs::P, NV = Q::NV;
  __shared__ T qv[2][NV][64];
  __shared__ T qh[2][64];
  __shared__ int qb[2][64];
  __shared__ T hand[D + 1][64];  // forward -> reverse: lam, loss sum
  __shared__ int handi[1][64];   // save cursor: the next slot to seed
  const int lane = (int)(threadIdx.x & 63);
  const int wv = (int)(threadIdx.x >> 6);
  const bool helper = wv == 1;  // wavefront-uniform
  const int64_t n = a.n;
  const int64_t C = a.ws_lanes;
  const int S = a.pr.S;
  const int lk = a.loss_kind;
  const bool saves = lk != DA_LOSS_SUMSQ_FINAL;

  // ---- forward replay: slot t = 32 wv + lane of the workgroup's 64 ----
  {
    const int t = 32 * wv + lane;
    const int64_t jl = (int64_t)blockIdx.x * 64 + t;
    const bool live = lane < 32 && jl < a.nslots;
    const int64_t j = a.slot0 + jl;
    T *ws = (T *)a.ws + (live ? jl : 0);
    const LaneInfo L = lane_info(a, j, live, a.max_n_steps, true);
    const int64_t tr = L.tr;
    const int N = L.N;
    const bool ok = L.ok;
    StepSrc<T, ROWS> src;
    src.init(a, live ? j : a.slot0, tr);
    T y[D], p[P];
    if (live) {
#pragma unroll
      for (int c = 0; c < D; ++c) y[c] = ((const T *)a.u0)[c * n + tr];
#pragma unroll
      for (int q = 0; q < P; ++q) p[q] = ((const T *)a.p)[q * n + tr];
    }
    const int Nw = wave_max(N);
    T ss = T(0);
    bool first = true;
    const int Sl = (ok && saves) ? S : 0;  // save slots this trajectory takes
    SaveWalk<T, D> fw;
    if (saves) fw.start(a, tr, 0, 1);
    auto terms = [&](int k) {
      while (fw.q < Sl && fw.idx == k) {
        loss_terms_v<T, D>(lk, y, fw.av, ss, first);
        fw.take(a, tr, 1);
      }
    };
    if (saves) terms(0);
    auto fstep = [&](int k, T hk) {
      if (k < N) {
        T *wk = ws + (int64_t)k * D * C;
#pragma unroll
        for (int c = 0; c < D; ++c) wk[c * C] = y[c];
        M::fwd(y, p, hk);
        if (saves) terms(k + 1);
      }
    };
    T hA = src.load(0);
    for (int k = 0; k < Nw; k += 2) {
      const T hB = src.load(k + 1);
      fstep(k, hA);
      hA = src.load(k + 2);
      if (k + 1 < Nw) fstep(k + 1, hB);
    }
    // loss and seeds at the final state
    T lam[D];
    if (!saves) {
#pragma unroll
      for (int c = 0; c < D; ++c) ss = (c == 0) ? y[c] * y[c] : mac(y[c], y[c], ss);
#pragma unroll
      for (int c = 0; c < D; ++c) lam[c] = T(2.0 * a.scale) * y[c];
    } else {
#pragma unroll
      for (int c = 0; c < D; ++c) lam[c] = T(0);
    }
    SaveWalk<T, D> bw;
    if (saves) {
      bw.start(a, tr, S - 1, -1);
      bw.q = Sl - 1;
      while (bw.q >= 0 && bw.idx == N) {
        seed_terms_v<T, D>(lk, y, bw.av, a.scale, lam);
        bw.take(a, tr, -1);
      }
    }
    if (lane < 32) {
#pragma unroll
      for (int c = 0; c < D; ++c) hand[c][t] = lam[c];
      hand[D][t] = ss;
      handi[0][t] = saves ? bw.q : -1;
    }
  }
  __syncthreads();  // every state stored (and visible to both), seeds handed over

  // ---- reverse sweep: lane = slot t; the helper prepares step Nw - 1 - i
  // while the first wavefront reverses step Nw - i (prepared the round before)
  const int64_t jl = (int64_t)blockIdx.x * 64 + lane;
  const bool live = jl < a.nslots;
  const int64_t j = a.slot0 + jl;
  T *ws = (T *)a.ws + (live ? jl : 0);
  const LaneInfo L = lane_info(a, j, live, a.max_n_steps, true);
  const int64_t tr = L.tr;
  const int N = L.N;
  const bool ok = L.ok;
  StepSrc<T, ROWS> src;
  src.init(a, live ? j : a.slot0, tr);
  T p[P];
  if (live) {
#pragma unroll
    for (int q = 0; q < P; ++q) p[q] = ((const T *)a.p)[q * n + tr];
  }
  const int Nw = wave_max(N);
  T lam[D], g[P], ss = T(0);
  SaveWalk<T, D> bw;
#pragma unroll
  for (int q = 0; q < P; ++q) g[q] = T(0);
  if (!helper) {
#pragma unroll
    for (int c = 0; c < D; ++c) lam[c] = hand[c][lane];
    ss = hand[D][lane];
    const int q = handi[0][lane];
    if (saves) bw.start(a, tr, q, -1);
    bw.q = q;
  }
  T yn[D], hn = T(0);  // helper: the next step's state and size, loaded ahead
  if (helper && Nw > 0) {
#pragma unroll
    for (int c = 0; c < D; ++c) yn[c] = ws[((int64_t)(Nw - 1) * D + c) * C];
    hn = src.load(Nw - 1);
  }
  for (int i = 0; i <= Nw; ++i) {
    if (helper) {
      const int k = Nw - 1 - i;
      if (k >= 0) {
        T yk[D];
#pragma unroll
        for (int c = 0; c < D; ++c) yk[c] = yn[c];
        const T hk = hn;
        const int kn = k > 0 ? k - 1 : 0;
#pragma unroll
        for (int c = 0; c < D; ++c) yn[c] = ws[((int64_t)kn * D + c) * C];
        hn = src.load(kn);
        Q q;
        if (k < N) {
          M::pre(yk, p, hk, q);
        } else {
#pragma unroll
          for (int v = 0; v < NV; ++v) q.v[v] = T(0);
          q.bits = 0;
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) qv[k & 1][v][lane] = q.v[v];
        qh[k & 1][lane] = hk;
        qb[k & 1][lane] = q.bits;
      }
    } else {
      const int k = Nw - i;
      if (k < Nw && k < N) {
        Q q;
#pragma unroll
        for (int v = 0; v < NV; ++v) q.v[v] = qv[k & 1][v][lane];
        q.bits = qb[k & 1][lane];
        M::adj_pre(q, p, qh[k & 1][lane], lam, g);
        if (saves) {
          while (bw.q >= 0 && bw.idx == k) {
            T yk[D];
#pragma unroll
            for (int c = 0; c < D; ++c) yk[c] = q.v[c];
            seed_terms_v<T, D>(lk, yk, bw.av, a.scale, lam);
            bw.take(a, tr, -1);
          }
        }
      }
    }
    __syncthreads();
  }

  if (live && !helper) {
    const T Lv = ok ? T(a.scale) * ss : nanv<T>();
    if (a.loss_out) ((T *)a.loss_out)[tr] = Lv;
    if (a.gu0)
#pragma unroll
      for (int c = 0; c < D; ++c) ((T *)a.gu0)[c * n + tr] = ok ? lam[c] : nanv<T>();
    if (a.gp)
#pragma unroll
      for (int q = 0; q < P; ++q) ((T *)a.gp)[q * n + tr] = ok ? g[q] : nanv<T>();
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
#ifndef __HIPCC_RTC__
// Methods with dense output set M::dense_output; for the others the DENSE
// kernels are not built and a dense problem is refused before launch.
template <class T, class M, bool DENSE>
hipError_t record_d(const RecordArgs &a, const SaveTimes &st, hipStream_t s) {
  const unsigned grid = (unsigned)((a.n + BLOCK - 1) / BLOCK);
  if (a.h) hipLaunchKernelGGL((k_record<T, M, true, DENSE>), grid, BLOCK, 0, s, a, st);
  else hipLaunchKernelGGL((k_record<T, M, false, DENSE>), grid, BLOCK, 0, s, a, st);
  return hipGetLastError();
}

template <class T, class M>
hipError_t record_t(const RecordArgs &a, const SaveTimes &st, hipStream_t s) {
  if constexpr (M::dense_output) {
    if (a.pr.dense) return record_d<T, M, true>(a, st, s);
  } else {
    if (a.pr.dense) return hipErrorInvalidValue;
  }
  return record_d<T, M, false>(a, st, s);
}

template <class T, class M, bool DENSE>
hipError_t replay_fwd_d(const ReplayArgs &a, hipStream_t s) {
  const unsigned grid = (unsigned)((a.n + BLOCK - 1) / BLOCK);
  if (a.h_rows) hipLaunchKernelGGL((k_replay_fwd<T, M, true, DENSE>), grid, BLOCK, 0, s, a);
  else hipLaunchKernelGGL((k_replay_fwd<T, M, false, DENSE>), grid, BLOCK, 0, s, a);
  return hipGetLastError();
}

template <class T, class M>
hipError_t replay_fwd_t(const ReplayArgs &a, hipStream_t s) {
  if constexpr (M::dense_output) {
    if (a.pr.dense) return replay_fwd_d<T, M, true>(a, s);
  } else {
    if (a.pr.dense) return hipErrorInvalidValue;
  }
  return replay_fwd_d<T, M, false>(a, s);
}

// Methods whose reverse step is split into M::pre and M::adj_pre and that
// take the two-wavefront gradient kernel (M::two_wave_reverse).
template <class M, class = void> struct TwoWave { static constexpr bool value = false; };
template <class M>
struct TwoWave<M, typename VoidT<decltype(M::two_wave_reverse)>::type> {
  static constexpr bool value = M::two_wave_reverse;
};

// Ensembles of at most this many trajectories (one wavefront per SIMD for
// the one-wavefront kernel) take the two-wavefront gradient kernel.
// Measured (gradient pass): Tsit5 on Lorenz-63, FP32, 65536 trajectories
// 0.189 against 0.203 ms; FP64, 1024 trajectories 0.044 against 0.047 ms;
// Dopri5 on Lorenz-63, FP64, 2^20 trajectories 13.8 against 10.5 ms (the
// one-wavefront kernel already runs three wavefronts per SIMD there).
constexpr int64_t TWO_WAVE_MAX_LANES = 65536;

template <class T, class M, bool ROWS, bool DENSE>
hipError_t replay_grad_ck(const ReplayArgs &a, hipStream_t s) {
  if constexpr (TwoWave<M>::value && !DENSE && M::D <= 4) {
    if (a.pr.checkpoint == 1 && a.nslots <= TWO_WAVE_MAX_LANES) {
      const unsigned grid2 = (unsigned)((a.nslots + 63) / 64);
      hipLaunchKernelGGL((k_replay_grad2<T, M, ROWS>), grid2, 128, 0, s, a);
      return hipGetLastError();
    }
  }
  const unsigned grid = (unsigned)((a.nslots + BLOCK - 1) / BLOCK);
  switch (a.pr.checkpoint) {
    case 1: hipLaunchKernelGGL((k_replay_grad<T, M, 1, ROWS, DENSE>), grid, BLOCK, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_replay_grad<T, M, 2, ROWS, DENSE>), grid, BLOCK, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_replay_grad<T, M, 4, ROWS, DENSE>), grid, BLOCK, 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_replay_grad<T, M, 8, ROWS, DENSE>), grid, BLOCK, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class T, class M, bool DENSE>
hipError_t replay_grad_d(const ReplayArgs &a, hipStream_t s) {
  return a.h_rows ? replay_grad_ck<T, M, true, DENSE>(a, s)
                  : replay_grad_ck<T, M, false, DENSE>(a, s);
}

// The final-state loss reads no save, so a dense problem runs the plain
// kernel for it.
template <class T, class M>
hipError_t replay_grad_t(const ReplayArgs &a, hipStream_t s) {
  const bool dense = a.pr.dense && a.loss_kind != DA_LOSS_SUMSQ_FINAL;
  if constexpr (M::dense_output) {
    if (dense) return replay_grad_d<T, M, true>(a, s);
  } else {
    if (dense) return hipErrorInvalidValue;
  }
  return replay_grad_d<T, M, false>(a, s);
}

#endif  // __HIPCC_RTC__

}  // namespace dadj
