// LU factorisation with partial pivoting and the two solves of the
// Rosenbrock methods (ROS2, Rodas3) in the lane-per-trajectory kernels: the
// d x d matrix W = I - gamma h J (d <= 3) of each lane in registers.  V is a
// real or a tangent number of the sensitivity kernel (pivots are chosen on
// values).
#pragma once

#include "lane_kernels.hpp"
#include "sens_kernel.hpp"

namespace dadj {
namespace {

// 1 / x for the factorisation without row exchanges, in FP64: the hardware's
// approximate reciprocal refined by three Newton steps q <- q + q (1 - x q)
// (the residual and the update one fma each).  The correctly rounded
// division 1.0 / x compiles to scalings of numerator and denominator, the
// same approximate reciprocal and two such steps, a quotient (numerator
// times reciprocal), its residual and correction, and a fix-up of special
// operands.  For |x| in [2^-600, 2^600] nothing is scaled or fixed up and
// the quotient is the reciprocal itself (the numerator is 1), so the two
// sequences are the same operations and agree bit for bit; outside that
// range (and for non-finite x) `need` is set and the caller recomputes with
// the division.  FP32 keeps the division.
__device__ __forceinline__ double recip_nx(double x, bool &need) {
  const double ax = __builtin_fabs(x);
  need = need || !(ax >= 0x1p-600 && ax <= 0x1p600);
  double q = __builtin_amdgcn_rcp(x);
#pragma unroll
  for (int it = 0; it < 3; ++it) {
    const double t = __builtin_fma(-x, q, 1.0);
    q = __builtin_fma(q, t, q);
  }
  return q;
}
__device__ __forceinline__ float recip_nx(float x, bool &) { return recip(x); }
// tangent numbers (the sensitivity kernel): the division of recip
template <class T, int G>
__device__ __forceinline__ DualN<T, G> recip_nx(const DualN<T, G> &x, bool &) {
  return recip(x);
}

// In-place LU of A (row-major) with partial pivoting; perm[i] = original row
// now in position i, swapped = some row was exchanged.  Row exchanges are
// register selects, executed only when some lane of the wavefront needs one
// (a uniform branch: where the pivot is already on the diagonal, as with
// diagonally dominant W, the selects are skipped; the values are the same
// either way).  Each pivot's reciprocal is formed once (a correctly rounded
// 1 / u) and every division by the pivot, here and in the solves, is a
// multiplication by it.  Pivots are chosen on values.
//
// X = false is the same factorisation on the assumption that no row is
// exchanged: no branch, perm the identity, swapped false, and `need` set
// where partial pivoting would have exchanged rows at some column (some
// entry below the diagonal larger in magnitude than the diagonal one, the
// comparison the pivot search makes) or where a pivot lies outside the
// range of recip_nx.  Where `need` stays false the factors are bit for bit
// those of X = true; where it is set they are not, and the caller
// recomputes with X = true.
template <int D, bool X = true, class V>
__device__ __forceinline__ void lu_factor(V (&A)[D * D], int (&perm)[D], V (&rinv)[D],
                                          bool &swapped, bool &need) {
#pragma unroll
  for (int i = 0; i < D; ++i) perm[i] = i;
  swapped = false;
#pragma unroll
  for (int k = 0; k < D; ++k) {
    if constexpr (X) {
      int piv = k;
      auto best = dabs(vpart(A[k * D + k]));
#pragma unroll
      for (int i = k + 1; i < D; ++i) {
        const auto v = dabs(vpart(A[i * D + k]));
        if (v > best) { best = v; piv = i; }
      }
      swapped = swapped || piv != k;
      if (__ballot(piv != k) != 0ull) {
#pragma unroll
        for (int r = k + 1; r < D; ++r) {
          const bool sw = piv == r;
#pragma unroll
          for (int j = 0; j < D; ++j) {
            const V top = A[k * D + j], oth = A[r * D + j];
            A[k * D + j] = sel(sw, oth, top);
            A[r * D + j] = sel(sw, top, oth);
          }
          const int pt = perm[k], po = perm[r];
          perm[k] = sw ? po : pt;
          perm[r] = sw ? pt : po;
        }
      }
    } else {
      const auto dk = dabs(vpart(A[k * D + k]));
#pragma unroll
      for (int i = k + 1; i < D; ++i) need = need || dabs(vpart(A[i * D + k])) > dk;
    }
    if constexpr (X) rinv[k] = recip(A[k * D + k]);
    else rinv[k] = recip_nx(A[k * D + k], need);
#pragma unroll
    for (int i = k + 1; i < D; ++i) {
      const V l = A[i * D + k] * rinv[k];
      A[i * D + k] = l;
#pragma unroll
      for (int j = k + 1; j < D; ++j) A[i * D + j] = mac(-l, A[k * D + j], A[i * D + j]);
    }
  }
}
template <int D, class V>
__device__ __forceinline__ void lu_factor(V (&A)[D * D], int (&perm)[D], V (&rinv)[D],
                                          bool &swapped) {
  bool need = false;
  lu_factor<D, true>(A, perm, rinv, swapped, need);
}

// Solve A x = b from the factors (P A = L U).  The right-hand side is copied
// into a private array first so that the permutation stays a register select
// (a select between loads through the argument would become an indexed load
// and keep the caller's arrays out of registers).  X = false: factors from
// lu_factor<D, false> (no permutation).
template <int D, bool X = true, class V>
__device__ __forceinline__ void lu_solve(const V (&LU)[D * D], const V (&rinv)[D],
                                         const int (&perm)[D], bool swapped, const V (&b_in)[D],
                                         V (&x)[D]) {
  V b[D];
#pragma unroll
  for (int i = 0; i < D; ++i) b[i] = b_in[i];
  if (X && __ballot(swapped) != 0ull) {  // uniform: some lane has a row exchange
#pragma unroll
    for (int i = 0; i < D; ++i) {
      V v = b[0];
#pragma unroll
      for (int q = 1; q < D; ++q) v = sel(perm[i] == q, b[q], v);
      x[i] = v;
    }
  } else {
#pragma unroll
    for (int i = 0; i < D; ++i) x[i] = b[i];
  }
#pragma unroll
  for (int i = 0; i < D; ++i)
#pragma unroll
    for (int j = 0; j < i; ++j) x[i] = mac(-LU[i * D + j], x[j], x[i]);
#pragma unroll
  for (int i = D - 1; i >= 0; --i) {
#pragma unroll
    for (int j = i + 1; j < D; ++j) x[i] = mac(-LU[i * D + j], x[j], x[i]);
    x[i] = x[i] * rinv[i];
  }
}

// Solve A^T x = b from the factors of A (A^T = U^T L^T P).
template <int D, bool X = true, class T>
__device__ __forceinline__ void lu_solve_t(const T (&LU)[D * D], const T (&rinv)[D],
                                           const int (&perm)[D], bool swapped, const T (&b)[D],
                                           T (&x)[D]) {
  T z[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    z[i] = b[i];
#pragma unroll
    for (int j = 0; j < i; ++j) z[i] = mac(-LU[j * D + i], z[j], z[i]);
    z[i] = z[i] * rinv[i];
  }
#pragma unroll
  for (int i = D - 1; i >= 0; --i)
#pragma unroll
    for (int j = i + 1; j < D; ++j) z[i] = mac(-LU[j * D + i], z[j], z[i]);
  // x[perm[i]] = z[i]
  if (X && __ballot(swapped) != 0ull) {  // uniform, as in lu_solve
#pragma unroll
    for (int c = 0; c < D; ++c) {
      T v = z[0];
#pragma unroll
      for (int i = 1; i < D; ++i) v = (perm[i] == c) ? z[i] : v;
      x[c] = v;
    }
  } else {
#pragma unroll
    for (int c = 0; c < D; ++c) x[c] = z[c];
  }
}

}  // namespace
}  // namespace dadj
