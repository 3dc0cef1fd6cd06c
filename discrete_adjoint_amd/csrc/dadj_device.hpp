// Device building blocks of libdadj: multiply-add, wave64 helpers, the
// explicit Runge-Kutta tableaux and the built-in right-hand sides.
//
// Arithmetic schedule.  Every sum of products is a chain "first product, then
// fused multiply-adds", evaluated left to right in the order written below,
// and the sources are built with -ffp-contract=off so that no other operation
// is fused.  The order is fixed so that results are reproducible and can be
// compared element by element with an independent CPU evaluation of the same
// formulas.
#pragma once

#ifndef __HIPCC_RTC__
#include <hip/hip_runtime.h>
#include <stdint.h>
#endif

namespace dadj {

// ---------------------------------------------------------------------------
// scalars
// ---------------------------------------------------------------------------
__device__ __forceinline__ double mac(double a, double b, double c) { return __builtin_fma(a, b, c); }
__device__ __forceinline__ float mac(float a, float b, float c) { return __builtin_fmaf(a, b, c); }

// Coefficient products and the step-size update of a stage sum: c * x,
// fma(c, x, acc) and fma(h, acc, y) (the tangent types of the sensitivity
// kernels provide the same three forms).
__device__ __forceinline__ double cmul(double c, double x) { return c * x; }
__device__ __forceinline__ float cmul(double c, float x) { return float(c) * x; }
__device__ __forceinline__ double cmac(double c, double x, double acc) { return mac(c, x, acc); }
__device__ __forceinline__ float cmac(double c, float x, float acc) { return mac(float(c), x, acc); }
__device__ __forceinline__ double smac(double h, double a, double y) { return mac(h, a, y); }
__device__ __forceinline__ float smac(float h, float a, float y) { return mac(h, a, y); }
// h * x for a step-size factor h, 1 / x (correctly rounded), and the value part
// of a number (the tangent types give their value; pivoting compares values).
__device__ __forceinline__ double smul(double h, double x) { return h * x; }
__device__ __forceinline__ float smul(float h, float x) { return h * x; }
__device__ __forceinline__ double recip(double x) { return 1.0 / x; }
__device__ __forceinline__ float recip(float x) { return 1.0f / x; }
__device__ __forceinline__ double vpart(double x) { return x; }
__device__ __forceinline__ float vpart(float x) { return x; }
// c ? a : b (the tangent types select part by part, which keeps them in
// registers)
__device__ __forceinline__ double sel(bool c, double a, double b) { return c ? a : b; }
__device__ __forceinline__ float sel(bool c, float a, float b) { return c ? a : b; }

__device__ __forceinline__ bool finite(double x) { return __builtin_isfinite(x); }
__device__ __forceinline__ bool finite(float x) { return __builtin_isfinite(x); }

template <class T> __device__ __forceinline__ T nanv() { return T(__builtin_nan("")); }

// Largest value of x over the active lanes of the wavefront, broadcast to all.
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const int o = __shfl_xor(x, off, 64);
    x = o > x ? o : x;
  }
  return __builtin_amdgcn_readfirstlane(x);
}
// Smallest value of x over the active lanes of the wavefront, broadcast to all.
__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const int o = __shfl_xor(x, off, 64);
    x = o < x ? o : x;
  }
  return __builtin_amdgcn_readfirstlane(x);
}

// ---------------------------------------------------------------------------
// Explicit 7-stage first-same-as-last tableaux.  Row 6 of A equals b and
// b[6] = 0, so the 7th stage state is the propagated 5th-order solution and
// only its right-hand side (for the error estimate) is extra.
// ---------------------------------------------------------------------------
struct Tsit5Tab {
  // Ch. Tsitouras, "Runge-Kutta pairs of order 5(4) satisfying only the first
  // column simplifying assumption", Comput. Math. Appl. 62 (2011) 770-775.
  static constexpr int order = 5, err_order = 4;
  static constexpr double a[7][7] = {
      {0, 0, 0, 0, 0, 0, 0},
      {0.161, 0, 0, 0, 0, 0, 0},
      {-0.008480655492356989, 0.335480655492357, 0, 0, 0, 0, 0},
      {2.897153057105493, -6.359448489975075, 4.3622954328695815, 0, 0, 0, 0},
      {5.325864828439257, -11.748883564062828, 7.4955393428898365, -0.09249506636175525, 0, 0, 0},
      {5.86145544294642, -12.92096931784711, 8.159367898576159, -0.071584973281401,
       -0.028269050394068383, 0, 0},
      {0.09646076681806523, 0.01, 0.4798896504144996, 1.379008574103742, -3.290069515436081,
       2.324710524099774, 0}};
  // error weights b - bhat
  static constexpr double e[7] = {-0.00178001105222577714, -0.0008164344596567469,
                                  0.007880878010261995,    -0.1447110071732629,
                                  0.5823571654525552,      -0.45808210592918697,
                                  0.015151515151515152};
};

struct Dopri5Tab {
  // J. R. Dormand, P. J. Prince, "A family of embedded Runge-Kutta formulae",
  // J. Comput. Appl. Math. 6 (1980) 19-26.
  static constexpr int order = 5, err_order = 4;
  static constexpr double a[7][7] = {
      {0, 0, 0, 0, 0, 0, 0},
      {1.0 / 5.0, 0, 0, 0, 0, 0, 0},
      {3.0 / 40.0, 9.0 / 40.0, 0, 0, 0, 0, 0},
      {44.0 / 45.0, -56.0 / 15.0, 32.0 / 9.0, 0, 0, 0, 0},
      {19372.0 / 6561.0, -25360.0 / 2187.0, 64448.0 / 6561.0, -212.0 / 729.0, 0, 0, 0},
      {9017.0 / 3168.0, -355.0 / 33.0, 46732.0 / 5247.0, 49.0 / 176.0, -5103.0 / 18656.0, 0, 0},
      {35.0 / 384.0, 0, 500.0 / 1113.0, 125.0 / 192.0, -2187.0 / 6784.0, 11.0 / 84.0, 0}};
  // b - bhat with bhat = (5179/57600, 0, 7571/16695, 393/640, -92097/339200,
  // 187/2100, 1/40)
  static constexpr double e[7] = {71.0 / 57600.0,       0.0,           -71.0 / 16695.0,
                                  71.0 / 1920.0,        -17253.0 / 339200.0, 22.0 / 525.0,
                                  -1.0 / 40.0};
};

// ROS2 (Verwer, Spee, Blom, Hundsdorfer 1999): gamma = 1 + 1/sqrt(2) rounded
// to double.
constexpr double ROS2_GAMMA = 1.7071067811865475;

// ---------------------------------------------------------------------------
// Right-hand sides.  vjp_y: w_j = sum_i J_ij v_i over the rows listed;
// vjp_p_acc: g_q += each (df_i/dp_q) v_i as a multiply-add into g_q;
// jac_contract_acc: gy_c (gp_q) += Jbar_ab dJ_ab/dy_c (dp_q), entries (a, b)
// in row-major order.
// ---------------------------------------------------------------------------
struct Linear {
  static constexpr int D = 1, P = 1;
  static constexpr bool built_in = true;
  template <class T> __device__ static __forceinline__ void f(const T *y, const T *p, T *o) {
    o[0] = p[0] * y[0];
  }
  template <class T>
  __device__ static __forceinline__ void vjp_y(const T *y, const T *p, const T *v, T *w) {
    w[0] = p[0] * v[0];
  }
  template <class T>
  __device__ static __forceinline__ void vjp_p_acc(const T *y, const T *p, const T *v, T *g) {
    g[0] = mac(y[0], v[0], g[0]);
  }
  template <class T> __device__ static __forceinline__ void jac(const T *y, const T *p, T *J) {
    J[0] = p[0];
  }
  template <class T>
  __device__ static __forceinline__ void jac_contract_acc(const T *y, const T *p, const T *Jb,
                                                          T *gy, T *gp) {
    gp[0] = gp[0] + Jb[0];
  }
};

struct Lorenz63 {
  // p = (sigma, rho, beta)
  static constexpr int D = 3, P = 3;
  static constexpr bool built_in = true;
  template <class T> __device__ static __forceinline__ void f(const T *y, const T *p, T *o) {
    o[0] = p[0] * (y[1] - y[0]);
    o[1] = mac(y[0], p[1] - y[2], -y[1]);
    o[2] = mac(y[0], y[1], -(p[2] * y[2]));
  }
  // J = [[-s, s, 0], [r - y3, -1, -y1], [y2, y1, -b]]
  template <class T>
  __device__ static __forceinline__ void vjp_y(const T *y, const T *p, const T *v, T *w) {
    w[0] = mac(y[1], v[2], mac(p[1] - y[2], v[1], (-p[0]) * v[0]));
    w[1] = mac(y[0], v[2], mac(p[0], v[0], -v[1]));
    w[2] = mac(-p[2], v[2], (-y[0]) * v[1]);
  }
  template <class T>
  __device__ static __forceinline__ void vjp_p_acc(const T *y, const T *p, const T *v, T *g) {
    g[0] = mac(y[1] - y[0], v[0], g[0]);
    g[1] = mac(y[0], v[1], g[1]);
    g[2] = mac(-y[2], v[2], g[2]);
  }
  template <class T> __device__ static __forceinline__ void jac(const T *y, const T *p, T *J) {
    J[0] = -p[0];        J[1] = p[0];   J[2] = T(0);
    J[3] = p[1] - y[2];  J[4] = T(-1);  J[5] = -y[0];
    J[6] = y[1];         J[7] = y[0];   J[8] = -p[2];
  }
  template <class T>
  __device__ static __forceinline__ void jac_contract_acc(const T *y, const T *p, const T *Jb,
                                                          T *gy, T *gp) {
    gp[0] = gp[0] - Jb[0];  // J11 = -s
    gp[0] = gp[0] + Jb[1];  // J12 = s
    gp[1] = gp[1] + Jb[3];  // J21 = r - y3
    gy[2] = gy[2] - Jb[3];
    gy[0] = gy[0] - Jb[5];  // J23 = -y1
    gy[1] = gy[1] + Jb[6];  // J31 = y2
    gy[0] = gy[0] + Jb[7];  // J32 = y1
    gp[2] = gp[2] - Jb[8];  // J33 = -b
  }
};

struct Robertson {
  // p = (k1, k2, k3)
  static constexpr int D = 3, P = 3;
  static constexpr bool built_in = true;
  template <class T> __device__ static __forceinline__ void f(const T *y, const T *p, T *o) {
    o[0] = mac(p[2] * y[1], y[2], (-p[0]) * y[0]);
    T s = p[0] * y[0];
    s = mac(-(p[1] * y[1]), y[1], s);
    s = mac(-(p[2] * y[1]), y[2], s);
    o[1] = s;
    o[2] = (p[1] * y[1]) * y[1];
  }
  // J = [[-k1, k3 y3, k3 y2], [k1, -2 k2 y2 - k3 y3, -k3 y2], [0, 2 k2 y2, 0]]
  template <class T>
  __device__ static __forceinline__ void vjp_y(const T *y, const T *p, const T *v, T *w) {
    w[0] = mac(p[0], v[1], (-p[0]) * v[0]);
    const T j22 = mac(-p[2], y[2], -(T(2) * p[1]) * y[1]);
    T s = (p[2] * y[2]) * v[0];
    s = mac(j22, v[1], s);
    s = mac(T(2) * p[1] * y[1], v[2], s);
    w[1] = s;
    w[2] = mac(-(p[2] * y[1]), v[1], (p[2] * y[1]) * v[0]);
  }
  template <class T>
  __device__ static __forceinline__ void vjp_p_acc(const T *y, const T *p, const T *v, T *g) {
    g[0] = mac(-y[0], v[0], g[0]);
    g[0] = mac(y[0], v[1], g[0]);
    const T y22 = y[1] * y[1];
    g[1] = mac(-y22, v[1], g[1]);
    g[1] = mac(y22, v[2], g[1]);
    const T y23 = y[1] * y[2];
    g[2] = mac(y23, v[0], g[2]);
    g[2] = mac(-y23, v[1], g[2]);
  }
  template <class T> __device__ static __forceinline__ void jac(const T *y, const T *p, T *J) {
    J[0] = -p[0];  J[1] = p[2] * y[2];  J[2] = p[2] * y[1];
    J[3] = p[0];   J[4] = mac(-p[2], y[2], -(T(2) * p[1]) * y[1]);  J[5] = -(p[2] * y[1]);
    J[6] = T(0);   J[7] = T(2) * p[1] * y[1];  J[8] = T(0);
  }
  template <class T>
  __device__ static __forceinline__ void jac_contract_acc(const T *y, const T *p, const T *Jb,
                                                          T *gy, T *gp) {
    const T k3 = p[2], two_k2 = T(2) * p[1], two_y2 = T(2) * y[1];
    gp[0] = gp[0] - Jb[0];              // J11 = -k1
    gy[2] = mac(k3, Jb[1], gy[2]);      // J12 = k3 y3
    gp[2] = mac(y[2], Jb[1], gp[2]);
    gy[1] = mac(k3, Jb[2], gy[1]);      // J13 = k3 y2
    gp[2] = mac(y[1], Jb[2], gp[2]);
    gp[0] = gp[0] + Jb[3];              // J21 = k1
    gy[1] = mac(-two_k2, Jb[4], gy[1]); // J22 = -2 k2 y2 - k3 y3
    gy[2] = mac(-k3, Jb[4], gy[2]);
    gp[1] = mac(-two_y2, Jb[4], gp[1]);
    gp[2] = mac(-y[2], Jb[4], gp[2]);
    gy[1] = mac(-k3, Jb[5], gy[1]);     // J23 = -k3 y2
    gp[2] = mac(-y[1], Jb[5], gp[2]);
    gy[1] = mac(two_k2, Jb[7], gy[1]);  // J32 = 2 k2 y2
    gp[1] = mac(two_y2, Jb[7], gp[1]);
  }
};
// ---------------------------------------------------------------------------
// Eight-species reaction cycle: a synthetic stiff system of the size of the
// HIRES test problem.  Nine mass-action reactions r0..r8 each move one unit
// of mass from species src to species dst (sum y_i is conserved):
//   r0 y0 -> y1            w = p0 y0            r5 2 y4 -> y4 + y5  ((1e-3 p1) y4) y4
//   r1 2 y1 -> y1 + y2     (p1 y1) y1           r6 y5 -> y6          (25 p0) y5
//   r2 y1 + y2 -> y0 + y2  (p2 y1) y2           r7 y6 + y2 -> y7 + y2 ((0.1 p2) y6) y2
//   r3 y2 -> y3            p3 y2                r8 y7 -> y0          (0.01 p3) y7
//   r4 y3 -> y4            (10 p3) y3
// f_a = sum_r (e_dst - e_src)_a w_r.  Every sum runs over the reactions in
// that order (a product or the first term, then multiply-adds or
// additions); a two-reactant rate k y_a y_b has the partials k y_b (in
// column a) and k y_a (column b), and k y_a^2 has (2k) y_a.
// ---------------------------------------------------------------------------
struct Kinetics8 {
  static constexpr int D = 8, P = 4;
  static constexpr bool built_in = true;
  template <class T> __device__ static __forceinline__ void f(const T *y, const T *p, T *o) {
    const T w0 = (T(1.0) * p[0]) * y[0];
    const T w1 = ((T(1.0) * p[1]) * y[1]) * y[1];
    const T w2 = ((T(1.0) * p[2]) * y[1]) * y[2];
    const T w3 = (T(1.0) * p[3]) * y[2];
    const T w4 = (T(10.0) * p[3]) * y[3];
    const T w5 = ((T(1e-3) * p[1]) * y[4]) * y[4];
    const T w6 = (T(25.0) * p[0]) * y[5];
    const T w7 = ((T(0.1) * p[2]) * y[6]) * y[2];
    const T w8 = (T(0.01) * p[3]) * y[7];
    o[0] = ((-w0) + w2) + w8;
    o[1] = (w0 - w1) - w2;
    o[2] = w1 - w3;
    o[3] = w3 - w4;
    o[4] = w4 - w5;
    o[5] = w5 - w6;
    o[6] = w6 - w7;
    o[7] = w7 - w8;
  }
  // partials of the rates: r0..r8 in order, two-reactant ones column a then b
  template <class T> struct Partials {
    T d0_0, d1_1, d2_1, d2_2, d3_2, d4_3, d5_4, d6_5, d7_6, d7_2, d8_7;
  };
  template <class T>
  __device__ static __forceinline__ Partials<T> partials(const T *y, const T *p) {
    Partials<T> d;
    const T k2 = T(1.0) * p[2], k7 = T(0.1) * p[2];
    d.d0_0 = T(1.0) * p[0];
    d.d1_1 = (T(2.0) * (T(1.0) * p[1])) * y[1];
    d.d2_1 = k2 * y[2];
    d.d2_2 = k2 * y[1];
    d.d3_2 = T(1.0) * p[3];
    d.d4_3 = T(10.0) * p[3];
    d.d5_4 = (T(2.0) * (T(1e-3) * p[1])) * y[4];
    d.d6_5 = T(25.0) * p[0];
    d.d7_6 = k7 * y[2];
    d.d7_2 = k7 * y[6];
    d.d8_7 = T(0.01) * p[3];
    return d;
  }
  // J^T v: w_b = sum_r dw_r/dy_b (v_dst - v_src)
  template <class T>
  __device__ static __forceinline__ void vjp_y(const T *y, const T *p, const T *v, T *w) {
    const Partials<T> d = partials(y, p);
    const T l0 = v[1] - v[0], l1 = v[2] - v[1], l2 = v[0] - v[1], l3 = v[3] - v[2];
    const T l4 = v[4] - v[3], l5 = v[5] - v[4], l6 = v[6] - v[5], l7 = v[7] - v[6];
    const T l8 = v[0] - v[7];
    w[0] = d.d0_0 * l0;
    w[1] = mac(d.d2_1, l2, d.d1_1 * l1);
    w[2] = mac(d.d7_2, l7, mac(d.d3_2, l3, d.d2_2 * l2));
    w[3] = d.d4_3 * l4;
    w[4] = d.d5_4 * l5;
    w[5] = d.d6_5 * l6;
    w[6] = d.d7_6 * l7;
    w[7] = d.d8_7 * l8;
  }
  // g_q += dw_r/dp_q (v_dst - v_src), reactions in order
  template <class T>
  __device__ static __forceinline__ void vjp_p_acc(const T *y, const T *p, const T *v, T *g) {
    g[0] = mac(T(1.0) * y[0], v[1] - v[0], g[0]);
    g[1] = mac((T(1.0) * y[1]) * y[1], v[2] - v[1], g[1]);
    g[2] = mac((T(1.0) * y[1]) * y[2], v[0] - v[1], g[2]);
    g[3] = mac(T(1.0) * y[2], v[3] - v[2], g[3]);
    g[3] = mac(T(10.0) * y[3], v[4] - v[3], g[3]);
    g[1] = mac((T(1e-3) * y[4]) * y[4], v[5] - v[4], g[1]);
    g[0] = mac(T(25.0) * y[5], v[6] - v[5], g[0]);
    g[2] = mac((T(0.1) * y[6]) * y[2], v[7] - v[6], g[2]);
    g[3] = mac(T(0.01) * y[7], v[0] - v[7], g[3]);
  }
  template <class T> __device__ static __forceinline__ void jac(const T *y, const T *p, T *J) {
    const Partials<T> d = partials(y, p);
#pragma unroll
    for (int i = 0; i < 64; ++i) J[i] = T(0.0);
    J[0 * 8 + 0] = -d.d0_0;       J[1 * 8 + 0] = d.d0_0;
    J[1 * 8 + 1] = -d.d1_1;       J[2 * 8 + 1] = d.d1_1;
    J[1 * 8 + 1] = J[1 * 8 + 1] - d.d2_1;
    J[0 * 8 + 1] = d.d2_1;
    J[1 * 8 + 2] = -d.d2_2;       J[0 * 8 + 2] = d.d2_2;
    J[2 * 8 + 2] = -d.d3_2;       J[3 * 8 + 2] = d.d3_2;
    J[3 * 8 + 3] = -d.d4_3;       J[4 * 8 + 3] = d.d4_3;
    J[4 * 8 + 4] = -d.d5_4;       J[5 * 8 + 4] = d.d5_4;
    J[5 * 8 + 5] = -d.d6_5;       J[6 * 8 + 5] = d.d6_5;
    J[6 * 8 + 6] = -d.d7_6;       J[7 * 8 + 6] = d.d7_6;
    J[6 * 8 + 2] = -d.d7_2;       J[7 * 8 + 2] = d.d7_2;
    J[7 * 8 + 7] = -d.d8_7;       J[0 * 8 + 7] = d.d8_7;
  }
  // sum_ab Jbar_ab dJ_ab: for each rate partial, M = Jbar[dst][col] -
  // Jbar[src][col] times its derivatives (y before p)
  template <class T>
  __device__ static __forceinline__ void jac_contract_acc(const T *y, const T *p, const T *Jb,
                                                          T *gy, T *gp) {
    gp[0] = mac(T(1.0), Jb[1 * 8 + 0] - Jb[0 * 8 + 0], gp[0]);                  // r0
    {
      const T m = Jb[2 * 8 + 1] - Jb[1 * 8 + 1];                                  // r1
      gy[1] = mac(T(2.0) * (T(1.0) * p[1]), m, gy[1]);
      gp[1] = mac((T(2.0) * T(1.0)) * y[1], m, gp[1]);
    }
    {
      const T kk = T(1.0) * p[2];                                                // r2
      const T ma = Jb[0 * 8 + 1] - Jb[1 * 8 + 1];
      gy[2] = mac(kk, ma, gy[2]);
      gp[2] = mac(T(1.0) * y[2], ma, gp[2]);
      const T mb = Jb[0 * 8 + 2] - Jb[1 * 8 + 2];
      gy[1] = mac(kk, mb, gy[1]);
      gp[2] = mac(T(1.0) * y[1], mb, gp[2]);
    }
    gp[3] = mac(T(1.0), Jb[3 * 8 + 2] - Jb[2 * 8 + 2], gp[3]);                  // r3
    gp[3] = mac(T(10.0), Jb[4 * 8 + 3] - Jb[3 * 8 + 3], gp[3]);                 // r4
    {
      const T m = Jb[5 * 8 + 4] - Jb[4 * 8 + 4];                                  // r5
      gy[4] = mac(T(2.0) * (T(1e-3) * p[1]), m, gy[4]);
      gp[1] = mac((T(2.0) * T(1e-3)) * y[4], m, gp[1]);
    }
    gp[0] = mac(T(25.0), Jb[6 * 8 + 5] - Jb[5 * 8 + 5], gp[0]);                 // r6
    {
      const T kk = T(0.1) * p[2];                                                // r7
      const T ma = Jb[7 * 8 + 6] - Jb[6 * 8 + 6];
      gy[2] = mac(kk, ma, gy[2]);
      gp[2] = mac(T(0.1) * y[2], ma, gp[2]);
      const T mb = Jb[7 * 8 + 2] - Jb[6 * 8 + 2];
      gy[6] = mac(kk, mb, gy[6]);
      gp[2] = mac(T(0.1) * y[6], mb, gp[2]);
    }
    gp[3] = mac(T(0.01), Jb[0 * 8 + 7] - Jb[7 * 8 + 7], gp[3]);                 // r8
  }
};

// ---------------------------------------------------------------------------
// Explicit RK stage machinery (one trajectory per lane, state in registers)
// ---------------------------------------------------------------------------

// Y = y + h * sum_{j<I} a[I][j] K[j]  (zero coefficients skipped).  T is the
// state type (a float type, or a tangent type), H the step-size type.
template <class Tab, int I, int D, class T, class H>
__device__ __forceinline__ void stage_state(const T (&y)[D], const T (&K)[7][D], H h,
                                            T (&Y)[D]) {
#pragma unroll
  for (int c = 0; c < D; ++c) {
    T acc = T(0);
    bool first = true;
#pragma unroll
    for (int j = 0; j < I; ++j) {
      if (Tab::a[I][j] != 0.0) {
        if (first) { acc = cmul(Tab::a[I][j], K[j][c]); first = false; }
        else acc = cmac(Tab::a[I][j], K[j][c], acc);
      }
    }
    Y[c] = smac(h, acc, y[c]);
  }
}

template <class Tab, class Rhs, int I, int LAST, bool LASTK, class T, class H>
struct StageLoop {
  __device__ static __forceinline__ void run(const T (&y)[Rhs::D], const T *p, H h,
                                             T (&Y)[7][Rhs::D], T (&K)[7][Rhs::D]) {
    stage_state<Tab, I>(y, K, h, Y[I]);
    if (I < LAST || LASTK) Rhs::f(Y[I], p, K[I]);
    StageLoop<Tab, Rhs, I + 1, LAST, LASTK, T, H>::run(y, p, h, Y, K);
  }
};
template <class Tab, class Rhs, int LAST, bool LASTK, class T, class H>
struct StageLoop<Tab, Rhs, LAST + 1, LAST, LASTK, T, H> {
  __device__ static __forceinline__ void run(const T (&)[Rhs::D], const T *, H, T (&)[7][Rhs::D],
                                             T (&)[7][Rhs::D]) {}
};

// Stages 1..LAST from y with K[0] = f(y) given; K[LAST] too when LASTK.
template <class Tab, class Rhs, int LAST, bool LASTK, class T, class H>
__device__ __forceinline__ void erk_stages(const T (&y)[Rhs::D], const T *p, H h,
                                           T (&Y)[7][Rhs::D], T (&K)[7][Rhs::D]) {
  StageLoop<Tab, Rhs, 1, LAST, LASTK, T, H>::run(y, p, h, Y, K);
}

// Power E^expo of the step-size controller, in single precision: the factor
// only scales the next trial step (the accept test E <= 1 stays in the
// state's precision), and the double-precision power would cost about as
// much as the rest of a trial step.
template <class T> __device__ __forceinline__ T ctrl_pow(T E, T expo) {
  return T(exp2f(float(expo) * log2f(float(E))));
}

// ---------------------------------------------------------------------------
// Dense output: weights of the cubic Hermite interpolant of an accepted step
// at fraction th, {H00, H01, H10, H11} = {(1-th)^2 (1+2th), th^2 (3-2th),
// th (1-th)^2, -th^2 (1-th)}, and the fraction of a save time in its step.
// ---------------------------------------------------------------------------
template <class T> struct HermiteW {
  T h00, h01, h10, h11;
};
template <class T> __device__ __forceinline__ HermiteW<T> hermite_w(T th) {
  const T u = T(1) - th;
  const T u2 = u * u, t2 = th * th;
  HermiteW<T> w;
  w.h00 = u2 * mac(T(2), th, T(1));
  w.h01 = t2 * mac(T(-2), th, T(3));
  w.h10 = th * u2;
  w.h11 = -(t2 * u);
  return w;
}

// Fraction of the accepted step [t, t_end] of size h at which save time ts
// lies (t < ts <= t_end): exactly 1 at the step's end, else (ts - t) / h in
// double, capped at 1.
__device__ __forceinline__ double step_fraction(double ts, double t, double t_end, double h) {
  if (ts >= t_end) return 1.0;
  const double th = (ts - t) / h;
  return th < 1.0 ? th : 1.0;
}

}  // namespace dadj
