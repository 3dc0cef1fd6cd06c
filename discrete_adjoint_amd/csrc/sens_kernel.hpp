// Forward-mode sensitivity kernel and its launcher: the state of every lane
// carries G tangent directions (unit vectors in u0, then in p) through the
// fixed-step replay, with the mesh held fixed as in the reverse sweep ("Differentiable astrophysics at scale", Methodology:
// forward sensitivities integrated in the same per-trajectory kernel;
// "GRADSOLVE" review, FAQ on exactness: no derivative of the step sizes).
// Any method whose fwd takes tangent numbers runs here (the explicit tableaux
// and ROS2).
#pragma once

#include "dual.hpp"
#include "erk_method.hpp"

namespace dadj {

constexpr int SENS_G = 2;  // tangent directions per lane and grid row

// Directions q_begin .. q_begin + q_count - 1 of the d + P; sens and the
// gradient hold them at q - q_begin.  Gradient terms seed . dy/dtheta_q in
// save-then-component order (first product, then multiply-adds), the seeds
// being
//   final-state loss: (2 scale) y_N    MSE: (2 scale) (y_s - aux_s)
//   cotangent:        scale aux_s.
// DENSE: a save with index k >= 1 (and its tangents) is the interpolant of
// step k - 1 at the recorded fraction.
template <class T, class M, int G, bool ROWS, bool DENSE>
__global__ __launch_bounds__(BLOCK) void k_replay_sens(ReplayArgs a) {
  using Rhs = typename M::Rhs;
  constexpr int D = Rhs::D, P = Rhs::P;
  using DT = DualN<T, G>;
  const int64_t n = a.n;
  const int64_t j = (int64_t)blockIdx.x * BLOCK + threadIdx.x;
  const bool live = j < n;
  const int q0 = a.q_begin + (int)blockIdx.y * G, qe = a.q_begin + a.q_count, Qo = a.q_count;
  const int S = a.pr.S;
  const int lk = a.loss_kind;
  const bool saves = a.has_loss && lk != DA_LOSS_SUMSQ_FINAL;
  const T *aux = (const T *)a.aux;
  T *sens = (T *)a.sens;
  const LaneInfo L = lane_info(a, j, live, a.pr.max_steps, true);
  const int64_t tr = L.tr;
  const int N = L.N;
  const bool ok = L.ok;
  StepSrc<T, ROWS> src;
  src.init(a, live ? j : 0, tr);
  DT y[D], p[P];
  if (live) {
#pragma unroll
    for (int c = 0; c < D; ++c) {
      y[c] = DT(((const T *)a.u0)[c * n + tr]);
#pragma unroll
      for (int m = 0; m < G; ++m) y[c].d[m] = (q0 + m == c) ? T(1) : T(0);
    }
#pragma unroll
    for (int r = 0; r < P; ++r) {
      p[r] = DT(((const T *)a.p)[r * n + tr]);
#pragma unroll
      for (int m = 0; m < G; ++m) p[r].d[m] = (q0 + m == D + r) ? T(1) : T(0);
    }
    if (sens)
      for (int s = 0; s < S; ++s) {
        const int ix = a.sidx[s * n + tr];
        if (!ok || ix < 0 || ix > N)
#pragma unroll
          for (int c = 0; c < D; ++c)
#pragma unroll
            for (int m = 0; m < G; ++m)
              if (q0 + m < qe)
                sens[((int64_t)(s * D + c) * Qo + q0 + m - a.q_begin) * n + tr] = nanv<T>();
      }
  }
  const int Nw = wave_max(N);

  T g[G], ss = T(0);
#pragma unroll
  for (int m = 0; m < G; ++m) g[m] = T(0);
  bool gfirst = true, lfirst = true;
  auto grad_terms = [&](T seed, const DT &yc) {
#pragma unroll
    for (int m = 0; m < G; ++m) g[m] = gfirst ? seed * yc.d[m] : mac(seed, yc.d[m], g[m]);
    gfirst = false;
  };
  int s = 0;
  int nxt = ok ? a.sidx[tr] : -1;
  // save s has state (and tangents) ysv
  auto emit = [&](const DT (&ysv)[D]) {
    if (sens)
#pragma unroll
      for (int c = 0; c < D; ++c)
#pragma unroll
        for (int m = 0; m < G; ++m)
          if (q0 + m < qe) sens[((int64_t)(s * D + c) * Qo + q0 + m - a.q_begin) * n + tr] = ysv[c].d[m];
    if (saves) {
#pragma unroll
      for (int c = 0; c < D; ++c) {
        const T av = aux[((int64_t)s * D + c) * n + tr];
        const T yv = ysv[c].v;
        if (lk == DA_LOSS_MSE_SAVE) {
          grad_terms(T(2.0 * a.scale) * (yv - av), ysv[c]);
          const T r = yv - av;
          ss = lfirst ? r * r : mac(r, r, ss);
        } else {
          grad_terms(T(a.scale) * av, ysv[c]);
          ss = lfirst ? av * yv : mac(av, yv, ss);
        }
        lfirst = false;
      }
    }
    ++s;
    nxt = s < S ? a.sidx[s * n + tr] : -1;
  };
  auto at_saves = [&](int k) {
    while (s < S && nxt == k) emit(y);
  };
  at_saves(0);
  const T *theta = (const T *)a.theta;
  auto step = [&](int k, T hk) {
    if (k < N) {
      if constexpr (DENSE) {
        DT yp[D];
#pragma unroll
        for (int c = 0; c < D; ++c) yp[c] = y[c];
        M::fwd(y, p, hk);
        while (s < S && nxt == k + 1) {
          DT ys[D];
          dense_value<Rhs>(theta[(int64_t)s * n + tr], hk, yp, y, p, ys);
          emit(ys);
        }
      } else {
        M::fwd(y, p, hk);
        at_saves(k + 1);
      }
    }
  };
  // Branch-free units (built-in systems of up to four components, no dense
  // output) when nothing is read at the saves (no sensitivity output, a
  // final-state loss or none): below the smallest step count of the
  // wavefront's trajectories, U steps at a time with no per-lane guard and,
  // for methods with row exchanges, without exchanges (the tangents follow
  // the values' pivots); a unit in which some lane would have exchanged rows
  // is repeated with M::fwd.  The saves passed over are taken (nothing is
  // written for them).  Same arithmetic as `step`.
  constexpr bool FAST = !DENSE && D <= 4 && BuiltIn<Rhs>::value && BranchFree<M>::value;
  int k0 = 0;
  if constexpr (FAST) {
    if (!sens && !saves) {
      constexpr int U = 4;
      const int Nmin = wave_min(N);
      T hc[U];
#pragma unroll
      for (int b = 0; b < U; ++b) hc[b] = src.load(b);
      for (; k0 + U <= Nmin; k0 += U) {
        T hn[U];
#pragma unroll
        for (int b = 0; b < U; ++b) hn[b] = src.load(k0 + U + b);
        DT y0[D];
#pragma unroll
        for (int c = 0; c < D; ++c) y0[c] = y[c];
        bool need = false;
#pragma unroll
        for (int b = 0; b < U; ++b) fwd_nx<M>(y, p, hc[b], need);
        if constexpr (RowX<M>::value) {
          if (__ballot(need) != 0ull) {
#pragma unroll
            for (int c = 0; c < D; ++c) y[c] = y0[c];
#pragma unroll
            for (int b = 0; b < U; ++b) M::fwd(y, p, hc[b]);
          }
        }
#pragma unroll
        for (int b = 0; b < U; ++b) hc[b] = hn[b];
      }
      while (s < S && nxt >= 0 && nxt <= k0) {
        ++s;
        nxt = s < S ? a.sidx[s * n + tr] : -1;
      }
    }
  }
  T hA = src.load(k0);
  for (int k = k0; k < Nw; k += 2) {
    const T hB = src.load(k + 1);
    step(k, hA);
    hA = src.load(k + 2);
    if (k + 1 < Nw) step(k + 1, hB);
  }
  if (a.has_loss && !saves) {
#pragma unroll
    for (int c = 0; c < D; ++c) {
      grad_terms(T(2.0 * a.scale) * y[c].v, y[c]);
      ss = (c == 0) ? y[c].v * y[c].v : mac(y[c].v, y[c].v, ss);
    }
  }
  if (live && a.has_loss) {
#pragma unroll
    for (int m = 0; m < G; ++m) {
      const int q = q0 + m;
      const T v = ok ? g[m] : nanv<T>();
      if (q >= qe) continue;
      if (a.gq) {
        ((T *)a.gq)[(int64_t)(q - a.q_begin) * n + tr] = v;
      } else if (q < D) {
        if (a.gu0) ((T *)a.gu0)[q * n + tr] = v;
      } else {
        if (a.gp) ((T *)a.gp)[(q - D) * n + tr] = v;
      }
    }
    if (blockIdx.y == 0 && a.loss_out) ((T *)a.loss_out)[tr] = ok ? T(a.scale) * ss : nanv<T>();
  }
}

#ifndef __HIPCC_RTC__
// Directions per lane: SENS_G, or one for systems of eight or more
// components, whose d x d factors with two tangents each would not fit the
// registers.
template <class M> constexpr int sens_group() { return M::D >= 8 ? 1 : SENS_G; }

// Launch: one lane per trajectory, the directions in groups of G on the
// second grid dimension.
template <class T, class M, bool DENSE>
hipError_t replay_sens_d(const ReplayArgs &a, hipStream_t s) {
  constexpr int G = sens_group<M>();
  const dim3 grid((unsigned)((a.n + BLOCK - 1) / BLOCK), (unsigned)((a.q_count + G - 1) / G));
  if (a.h_rows)
    hipLaunchKernelGGL((k_replay_sens<T, M, G, true, DENSE>), grid, BLOCK, 0, s, a);
  else
    hipLaunchKernelGGL((k_replay_sens<T, M, G, false, DENSE>), grid, BLOCK, 0, s, a);
  return hipGetLastError();
}

// Dense output changes only the saves: without loss terms at the saves and
// without sensitivity output the plain kernel computes the same.  Methods
// without an interpolant never take the dense kernel (the library refuses
// dense output for them).
template <class T, class M>
hipError_t replay_sens_t(const ReplayArgs &a, hipStream_t s) {
  const bool at_saves = a.sens || (a.has_loss && a.loss_kind != DA_LOSS_SUMSQ_FINAL);
  if constexpr (M::dense_output)
    if (a.pr.dense && at_saves) return replay_sens_d<T, M, true>(a, s);
  return replay_sens_d<T, M, false>(a, s);
}
#endif

}  // namespace dadj
