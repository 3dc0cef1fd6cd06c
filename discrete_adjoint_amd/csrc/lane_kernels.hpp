// Lane-per-trajectory kernels, generic over the integration method M.
//
//  k_record<T, M, LOG>   adaptive solve of one trajectory per lane; with LOG it
//                        writes every accepted step size into the mesh
//                        ("GRADSOLVE: fast exact gradients for ODE ensembles on
//                        GPUs", gptget.net summary, Methodology; evolve.pub
//                        review, Summary: zero-padded fixed-length mesh), without
//                        it it is the forward-only solve (summary, Key results).
//  k_replay_fwd<T, M>    fixed-step replay of a mesh (review, Summary).
//  k_replay_grad<T, M>   replay that keeps each y_k in the workspace, then the
//                        reverse sweep through the recomputed stages with the
//                        mesh held fixed (review, Strengths (paper section 3.1)
//                        and FAQ: the exact discrete adjoint, no derivative of
//                        the step-size choices).
//
// A method M provides:
//   using Rhs; order (for the starting step); err_order (controller exponent)
//   template <class T> struct Cache;                 per-attempt scratch
//   begin(y, p, cache)                               once per accepted state
//   attempt(y, p, h, cache, ynew, err)               one trial step
//   accepted(cache)                                  after an accepted trial
//   fwd(y, p, h)                                     one replay step
//   adj(y, p, h, lam, g)                             its reverse
#pragma once

#include <math.h>

#include "dadj_device.hpp"
#include "dadj_internal.hpp"

namespace dadj {

template <class T> __device__ __forceinline__ T dmax(T a, T b) { return (a < b) ? b : a; }
template <class T> __device__ __forceinline__ T dmin(T a, T b) { return (b < a) ? b : a; }
__device__ __forceinline__ double dpow(double a, double b) { return pow(a, b); }
__device__ __forceinline__ float dpow(float a, float b) { return powf(a, b); }
__device__ __forceinline__ double dsqrt(double a) { return sqrt(a); }
__device__ __forceinline__ float dsqrt(float a) { return sqrtf(a); }
__device__ __forceinline__ double dabs(double a) { return fabs(a); }
__device__ __forceinline__ float dabs(float a) { return fabsf(a); }

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
// exactly on every save time and on t1; t accumulates in double.
// ---------------------------------------------------------------------------
template <class T, class M, bool LOG>
__global__ __launch_bounds__(BLOCK) void k_record(RecordArgs a, SaveTimes stimes) {
  using Rhs = typename M::Rhs;
  constexpr int D = Rhs::D, P = Rhs::P;
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

  int nacc = 0, natt = 0, st = LANE_OK;
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
        const double t_stop = (has_saves && js < S) ? stimes.t[js] : pr.t1;
        const T rem = T(t_stop - t);
        const bool land = !(h < rem);
        const T hs = land ? rem : h;
        if (nacc >= pr.max_steps) { st = LANE_MAX_STEPS; break; }
        if (natt >= pr.max_attempts) { st = LANE_MAX_ATTEMPTS; break; }
        if (!(hs > T(0)) || t + double(hs) == t) { st = LANE_DT_UNDERFLOW; break; }
        ++natt;
        M::attempt(y, p, hs, cache, ynew, err);
        const T E = err_norm<D>(err, y, ynew, atol, rtol);
        if (E <= T(1)) {
          if (LOG) H[(int64_t)nacc * n + i] = hs;
          ++nacc;
#pragma unroll
          for (int c = 0; c < D; ++c) y[c] = ynew[c];
          M::accepted(cache);
          t = land ? t_stop : t + double(hs);
          T fac = (E == T(0)) ? fmax : dmin(fmax, dmax(fmin, safety * dpow(E, expo)));
          if (after_reject) fac = dmin(fac, T(1));
          h = hs * fac;
          after_reject = false;
          if (land) {
            if (js < S) {
              if (a.sidx) a.sidx[js * n + i] = nacc;
              if (ysave)
#pragma unroll
                for (int c = 0; c < D; ++c) ysave[(js * D + c) * n + i] = y[c];
            }
            if (++js == n_stops) break;
          }
        } else {
          const T fac = finite(E) ? dmax(fmin, safety * dpow(E, expo)) : fmin;
          h = hs * fac;
          after_reject = true;
        }
      }
    }
    if (a.nsteps) a.nsteps[i] = nacc;
    if (a.status) a.status[i] = st;
  }
  if (LOG) {
    // zero padding after each lane's last step, written row by row across the wave
    const int mine = live ? nacc : pr.max_steps;
    int kmin = mine;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const int o = __shfl_xor(kmin, off, 64);
      kmin = o < kmin ? o : kmin;
    }
    kmin = __builtin_amdgcn_readfirstlane(kmin);
    for (int k = kmin; k < pr.max_steps; ++k)
      if (k >= mine) H[(int64_t)k * n + i] = T(0);
  }
}

// ---------------------------------------------------------------------------
// Replay forward: the state after save_idx[s] steps goes to y_save[s]; save
// slots whose index lies outside [0, n_steps] get NaN.
// ---------------------------------------------------------------------------
template <class T, class M>
__global__ __launch_bounds__(BLOCK) void k_replay_fwd(ReplayArgs a) {
  using Rhs = typename M::Rhs;
  constexpr int D = Rhs::D, P = Rhs::P;
  const int64_t n = a.n;
  const int64_t j = (int64_t)blockIdx.x * BLOCK + threadIdx.x;
  const bool live = j < n;
  const int S = a.pr.S;
  const T *H = (const T *)a.h;
  T *ysave = (T *)a.y_save;
  int N = 0;
  int64_t tr = j;
  T y[D], p[P];
  if (live) {
    tr = a.perm ? a.perm[j] : j;
    N = a.nsteps[j];
    N = N < 0 ? 0 : (N > a.pr.max_steps ? a.pr.max_steps : N);
#pragma unroll
    for (int c = 0; c < D; ++c) y[c] = ((const T *)a.u0)[c * n + tr];
#pragma unroll
    for (int q = 0; q < P; ++q) p[q] = ((const T *)a.p)[q * n + tr];
    for (int q = 0; q < S; ++q) {
      const int ix = a.sidx[q * n + j];
      if (ix < 0 || ix > N)
#pragma unroll
        for (int c = 0; c < D; ++c) ysave[(q * D + c) * n + tr] = nanv<T>();
    }
  }
  const int Nw = wave_max(N);
  int s = 0;
  int nxt = live ? a.sidx[j] : -1;
  while (live && s < S && nxt == 0) {
#pragma unroll
    for (int c = 0; c < D; ++c) ysave[(s * D + c) * n + tr] = y[c];
    ++s;
    nxt = s < S ? a.sidx[s * n + j] : -1;
  }
  for (int k = 0; k < Nw; ++k) {
    if (k < N) {
      const T hk = H[(int64_t)k * n + j];
      M::fwd(y, p, hk);
      while (s < S && nxt == k + 1) {
#pragma unroll
        for (int c = 0; c < D; ++c) ysave[(s * D + c) * n + tr] = y[c];
        ++s;
        nxt = s < S ? a.sidx[s * n + j] : -1;
      }
    }
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

// Workspace layout: y_k of local slot jl at ws[(k * D + c) * ws_lanes + jl].
template <class T, class M>
__global__ __launch_bounds__(BLOCK) void k_replay_grad(ReplayArgs a) {
  using Rhs = typename M::Rhs;
  constexpr int D = Rhs::D, P = Rhs::P;
  const int64_t n = a.n;
  const int64_t jl = (int64_t)blockIdx.x * BLOCK + threadIdx.x;
  const bool live = jl < a.nslots;
  const int64_t j = a.slot0 + jl;
  const int64_t C = a.ws_lanes;
  const int S = a.pr.S;
  const int lk = a.loss_kind;
  const T *H = (const T *)a.h;
  const T *aux = (const T *)a.aux;
  T *ws = (T *)a.ws;
  int N = 0;
  bool ok = false;
  int64_t tr = j;
  T y[D], p[P];
  if (live) {
    tr = a.perm ? a.perm[j] : j;
    N = a.nsteps[j];
    ok = a.status[j] == LANE_OK && N >= 0 && N <= a.max_n_steps;
#pragma unroll
    for (int c = 0; c < D; ++c) y[c] = ((const T *)a.u0)[c * n + tr];
#pragma unroll
    for (int q = 0; q < P; ++q) p[q] = ((const T *)a.p)[q * n + tr];
  }
  if (!ok) N = 0;
  const int Nw = wave_max(N);

  // ---- forward replay, keeping y_k; loss terms at the save indices ----
  T ss = T(0);
  bool first = true;
  int s = 0;
  int nxt = (ok && lk != DA_LOSS_SUMSQ_FINAL) ? a.sidx[j] : -1;
  while (s < S && nxt == 0) {
    loss_terms<T, D>(lk, y, aux, n, s, tr, ss, first);
    ++s;
    nxt = s < S ? a.sidx[s * n + j] : -1;
  }
  for (int k = 0; k < Nw; ++k) {
    if (k < N) {
      T *wk = ws + (int64_t)k * D * C + jl;
#pragma unroll
      for (int c = 0; c < D; ++c) wk[c * C] = y[c];
      const T hk = H[(int64_t)k * n + j];
      M::fwd(y, p, hk);
      if (nxt == k + 1) {
        loss_terms<T, D>(lk, y, aux, n, s, tr, ss, first);
        ++s;
        nxt = s < S ? a.sidx[s * n + j] : -1;
      }
    }
  }

  // ---- loss and seeds at the final state ----
  T lam[D], g[P];
#pragma unroll
  for (int q = 0; q < P; ++q) g[q] = T(0);
  if (lk == DA_LOSS_SUMSQ_FINAL) {
#pragma unroll
    for (int c = 0; c < D; ++c) ss = (c == 0) ? y[c] * y[c] : mac(y[c], y[c], ss);
#pragma unroll
    for (int c = 0; c < D; ++c) lam[c] = T(2.0 * a.scale) * y[c];
  } else {
#pragma unroll
    for (int c = 0; c < D; ++c) lam[c] = T(0);
  }
  int sh = S - 1;
  int hidx = (ok && lk != DA_LOSS_SUMSQ_FINAL) ? a.sidx[(int64_t)sh * n + j] : -1;
  while (sh >= 0 && hidx == N) {
    seed_terms<T, D>(lk, y, aux, n, sh, tr, a.scale, lam);
    --sh;
    hidx = sh >= 0 ? a.sidx[(int64_t)sh * n + j] : -1;
  }

  // ---- reverse sweep ----
  for (int k = Nw - 1; k >= 0; --k) {
    if (k < N) {
      const T *wk = ws + (int64_t)k * D * C + jl;
      T yk[D];
#pragma unroll
      for (int c = 0; c < D; ++c) yk[c] = wk[c * C];
      const T hk = H[(int64_t)k * n + j];
      M::adj(yk, p, hk, lam, g);
      while (sh >= 0 && hidx == k) {
        seed_terms<T, D>(lk, yk, aux, n, sh, tr, a.scale, lam);
        --sh;
        hidx = sh >= 0 ? a.sidx[(int64_t)sh * n + j] : -1;
      }
    }
  }

  if (live) {
    const T L = ok ? T(a.scale) * ss : nanv<T>();
    if (a.loss_out) ((T *)a.loss_out)[tr] = L;
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
template <class T, class M>
hipError_t record_t(const RecordArgs &a, const SaveTimes &st, hipStream_t s) {
  const unsigned grid = (unsigned)((a.n + BLOCK - 1) / BLOCK);
  if (a.h) hipLaunchKernelGGL((k_record<T, M, true>), grid, BLOCK, 0, s, a, st);
  else hipLaunchKernelGGL((k_record<T, M, false>), grid, BLOCK, 0, s, a, st);
  return hipGetLastError();
}

template <class T, class M>
hipError_t replay_fwd_t(const ReplayArgs &a, hipStream_t s) {
  const unsigned grid = (unsigned)((a.n + BLOCK - 1) / BLOCK);
  hipLaunchKernelGGL((k_replay_fwd<T, M>), grid, BLOCK, 0, s, a);
  return hipGetLastError();
}

template <class T, class M>
hipError_t replay_grad_t(const ReplayArgs &a, hipStream_t s) {
  const unsigned grid = (unsigned)((a.nslots + BLOCK - 1) / BLOCK);
  hipLaunchKernelGGL((k_replay_grad<T, M>), grid, BLOCK, 0, s, a);
  return hipGetLastError();
}

}  // namespace dadj
