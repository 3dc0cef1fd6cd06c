/*
 * Plain CPU oracle for the record-and-replay discrete adjoint of ODE ensembles.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only users of this library.  It shares
 * no code, header, table or constant with the HIP library: every tableau,
 * right-hand side, controller rule, replay and adjoint below is written here
 * from the method's definition, one lane at a time, in plain loops.
 *
 * What it computes (pages, by title and section):
 *  - "GRADSOLVE: fast exact gradients for ODE ensembles on GPUs"
 *    (gptget.net summary), Methodology: an adaptive solve per trajectory
 *    records the accepted step sizes; the gradient is taken through a
 *    fixed-step replay of those steps.  Abstract: explicit and Rosenbrock
 *    integrators; the result is the exact discrete adjoint of the replay.
 *  - same paper, evolve.pub review, Summary: the record is a zero-padded,
 *    fixed-length step mesh per trajectory; the replay is a branch-free chain
 *    and its reverse sweep gives the discrete adjoint.  Strengths (paper
 *    section 3.1) and FAQ "Is gradsolve's gradient really exact?": the mesh is
 *    held fixed (stop-gradient); no derivative of the step-size choices.
 *  - "Using GPU-accelerated Ensembles with Automatic Differentiation"
 *    (DiffEqGPU docs): the Lorenz right-hand side and parameter order
 *    (forward-mode example); per-trajectory parameters; the Enzyme example
 *    (fixed-step Tsit5 gradient of a final-state sum) used as a test pin.
 * Not from the pages (published methods, restated here):
 *  - Tsit5 tableau: Ch. Tsitouras, Comput. Math. Appl. 62 (2011) 770-775.
 *  - Dopri5 tableau: J. R. Dormand, P. J. Prince, J. Comput. Appl. Math. 6
 *    (1980) 19-26.
 *  - ROS2: J. G. Verwer, E. J. Spee, J. G. Blom, W. Hundsdorfer, SIAM J. Sci.
 *    Comput. 20 (1999) 1456-1480, with gamma = 1 + 1/sqrt(2).
 *  - Rodas3: A. Sandu et al., Atmos. Environ. 31 (1997) 3459-3472.
 *  - Fehlberg 7(8): E. Fehlberg, NASA TR R-287 (1968).
 *  - A fourth-order Rosenbrock method: L. F. Shampine, ACM TOMS 8 (1982)
 *    93-113 (its parameter set of the four-stage scheme).
 *  - Starting step: Hairer, Norsett, Wanner, Solving ODEs I, section II.4.
 *
 * Rounding modes.  Every sum of products is evaluated left to right as a
 * chain "first product, then multiply-add".  With fused = 0 each multiply and
 * add rounds separately (built with -ffp-contract=off); with fused = 1 each
 * multiply-add is one correctly rounded fma().  The fused mode also follows
 * the kernels' written schedule in three more places, each marked where it
 * occurs: pivot reciprocals in the LU and its solves, the pairwise order of
 * the Lorenz-96 parameter-gradient sum, and the step-size controller's power
 * taken in single precision.  The plain mode keeps the textbook forms there:
 * divisions by the pivot, one running sum, and the power in the state's own
 * precision.
 *
 * Layout here is lane-major: u0[n][d], p[n][P], h[n][max_steps],
 * save_idx[n][S], y_save[n][S][d] with S = max(1, n_save).
 */
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <omp.h>
#include <type_traits>
#include <vector>

#include "user_types.h"

namespace {

constexpr int MAXD = 64;  // largest state dimension handled
constexpr int MAXR = 8;   // largest state dimension of the Rosenbrock methods
constexpr int MAXP = 16;  // largest parameter count

enum { M_TSIT5 = 0, M_DOPRI5 = 1, M_ROS2 = 2, M_RODAS3 = 3, M_RKF78 = 4, M_ROS4 = 5 };
enum { R_LINEAR = 0, R_LORENZ63 = 1, R_ROBERTSON = 2, R_LORENZ96 = 3, R_KINETICS8 = 4 };
constexpr int R_USER = 1024;  /* kinds from here: the caller's right-hand side */
enum { S_OK = 0, S_MAX_STEPS = 1, S_DT_UNDERFLOW = 2, S_NONFINITE = 3,
       S_MAX_ATTEMPTS = 4 };
enum { L_SUMSQ_FINAL = 0, L_MSE_SAVE = 1, L_COTANGENT = 2 };
enum { E_OK = 0, E_INVAL = -1, E_UNSUPPORTED = -2 };

}  // namespace

extern "C" {
/* Problem description (the oracle's own struct). */
typedef struct {
  int32_t rhs, dim, n_params, method;
  double t0, t1, rtol, atol, dt0;
  int32_t max_steps, max_attempts;
  int32_t n_save;
  const double *save_times; /* host, strictly increasing in (t0, t1] */
  double safety, fac_min, fac_max;
  int32_t dense;            /* 0: steps land on save times; 1: saves read from
                               the step's interpolant (explicit methods) */
} orc_problem;
}

namespace {

/* ------------------------------------------------------------------ */
/* Scalars                                                             */
/* ------------------------------------------------------------------ */

/* Forward-mode dual number (value, one tangent) for the JVP check. */
struct Dual {
  double v, d;
  Dual() : v(0), d(0) {}
  Dual(double x) : v(x), d(0) {}
  Dual(double x, double dx) : v(x), d(dx) {}
};
inline Dual operator+(Dual a, Dual b) { return Dual(a.v + b.v, a.d + b.d); }
inline Dual operator-(Dual a, Dual b) { return Dual(a.v - b.v, a.d - b.d); }
inline Dual operator-(Dual a) { return Dual(-a.v, -a.d); }
inline Dual operator*(Dual a, Dual b) { return Dual(a.v * b.v, a.d * b.v + a.v * b.d); }
inline Dual operator/(Dual a, Dual b) {
  return Dual(a.v / b.v, (a.d * b.v - a.v * b.d) / (b.v * b.v));
}
/* Dual number of the fused-rounding mode: the tangent of every product and
 * multiply-add is formed with fma in a fixed order (the written schedule of
 * the GPU sensitivity kernels):
 *   a*b        -> (a.v*b.v,        fma(a.d, b.v, a.v*b.d))
 *   fma(a,b,c) -> (fma(a.v,b.v,c.v), fma(a.d, b.v, fma(a.v, b.d, c.d)))
 *   a/b        -> (q = a.v/b.v,     fma(-q, b.d, a.d) / b.v)
 * sums and differences act on both parts. */
struct DualF {
  double v, d;
  DualF() : v(0), d(0) {}
  DualF(double x) : v(x), d(0) {}
  DualF(double x, double dx) : v(x), d(dx) {}
};
inline DualF operator+(DualF a, DualF b) { return DualF(a.v + b.v, a.d + b.d); }
inline DualF operator-(DualF a, DualF b) { return DualF(a.v - b.v, a.d - b.d); }
inline DualF operator-(DualF a) { return DualF(-a.v, -a.d); }
inline DualF operator*(DualF a, DualF b) {
  return DualF(a.v * b.v, std::fma(a.d, b.v, a.v * b.d));
}
inline DualF operator/(DualF a, DualF b) {
  const double q = a.v / b.v;
  return DualF(q, std::fma(-q, b.d, a.d) / b.v);
}
inline bool fin(DualF a) { return std::isfinite(a.v); }
inline double val(DualF a) { return a.v; }
inline DualF absval(DualF a) { return a.v < 0 ? -a : a; }

inline bool fin(Dual a) { return std::isfinite(a.v); }
inline bool fin(double a) { return std::isfinite(a); }
inline bool fin(float a) { return std::isfinite(a); }
inline double val(Dual a) { return a.v; }
inline double val(double a) { return a; }
inline double val(float a) { return a; }
inline double absval(double a) { return std::fabs(a); }
inline float absval(float a) { return std::fabs(a); }
inline Dual absval(Dual a) { return a.v < 0 ? -a : a; }

/* The one multiply-add of this file: a*b + c. */
template <bool F> inline double mac(double a, double b, double c) {
  return F ? std::fma(a, b, c) : a * b + c;
}
template <bool F> inline float mac(float a, float b, float c) {
  return F ? std::fma(a, b, c) : a * b + c;
}
template <bool F> inline Dual mac(Dual a, Dual b, Dual c) { return a * b + c; }
template <bool F> inline DualF mac(DualF a, DualF b, DualF c) {
  return DualF(std::fma(a.v, b.v, c.v), std::fma(a.d, b.v, std::fma(a.v, b.d, c.d)));
}

/* Chain sum_k coef[k]*x[k] over nonzero coefficients: first a product, then
 * multiply-adds.  Returns 0 when every coefficient is zero. */
template <class T, bool F>
inline T chain(int m, const double *coef, const T *const *x, int c) {
  T acc = T(0.0);
  bool first = true;
  for (int k = 0; k < m; ++k) {
    if (coef[k] == 0.0) continue;
    if (first) { acc = T(coef[k]) * x[k][c]; first = false; }
    else acc = mac<F>(T(coef[k]), x[k][c], acc);
  }
  return acc;
}

/* ------------------------------------------------------------------ */
/* Tableaux (explicit, 7 stages, first-same-as-last)                   */
/* ------------------------------------------------------------------ */

struct Tableau {
  double c[7];
  double a[7][7];  /* a[i][j], j < i; row 6 equals b */
  double b[7];     /* 5th-order weights, b[6] = 0 */
  double e[7];     /* error weights b - bhat (4th-order embedded) */
  int order;       /* order of the propagated solution */
  int err_order;   /* order of the embedded solution */
};

Tableau make_tsit5() {
  /* Tsitouras (2011), decimal coefficients as published. */
  Tableau t;
  std::memset(&t, 0, sizeof t);
  t.c[1] = 0.161; t.c[2] = 0.327; t.c[3] = 0.9; t.c[4] = 0.9800255409045097;
  t.c[5] = 1.0; t.c[6] = 1.0;
  t.a[1][0] = 0.161;
  t.a[2][0] = -0.008480655492356989; t.a[2][1] = 0.335480655492357;
  t.a[3][0] = 2.897153057105493; t.a[3][1] = -6.359448489975075;
  t.a[3][2] = 4.3622954328695815;
  t.a[4][0] = 5.325864828439257; t.a[4][1] = -11.748883564062828;
  t.a[4][2] = 7.4955393428898365; t.a[4][3] = -0.09249506636175525;
  t.a[5][0] = 5.86145544294642; t.a[5][1] = -12.92096931784711;
  t.a[5][2] = 8.159367898576159; t.a[5][3] = -0.071584973281401;
  t.a[5][4] = -0.028269050394068383;
  t.a[6][0] = 0.09646076681806523; t.a[6][1] = 0.01;
  t.a[6][2] = 0.4798896504144996; t.a[6][3] = 1.379008574103742;
  t.a[6][4] = -3.290069515436081; t.a[6][5] = 2.324710524099774;
  for (int j = 0; j < 7; ++j) t.b[j] = t.a[6][j];
  t.e[0] = -0.00178001105222577714; t.e[1] = -0.0008164344596567469;
  t.e[2] = 0.007880878010261995; t.e[3] = -0.1447110071732629;
  t.e[4] = 0.5823571654525552; t.e[5] = -0.45808210592918697;
  t.e[6] = 0.015151515151515152;
  t.order = 5; t.err_order = 4;
  return t;
}

Tableau make_dopri5() {
  /* Dormand & Prince (1980), rational coefficients. */
  Tableau t;
  std::memset(&t, 0, sizeof t);
  t.c[1] = 1.0 / 5.0; t.c[2] = 3.0 / 10.0; t.c[3] = 4.0 / 5.0; t.c[4] = 8.0 / 9.0;
  t.c[5] = 1.0; t.c[6] = 1.0;
  t.a[1][0] = 1.0 / 5.0;
  t.a[2][0] = 3.0 / 40.0; t.a[2][1] = 9.0 / 40.0;
  t.a[3][0] = 44.0 / 45.0; t.a[3][1] = -56.0 / 15.0; t.a[3][2] = 32.0 / 9.0;
  t.a[4][0] = 19372.0 / 6561.0; t.a[4][1] = -25360.0 / 2187.0;
  t.a[4][2] = 64448.0 / 6561.0; t.a[4][3] = -212.0 / 729.0;
  t.a[5][0] = 9017.0 / 3168.0; t.a[5][1] = -355.0 / 33.0;
  t.a[5][2] = 46732.0 / 5247.0; t.a[5][3] = 49.0 / 176.0;
  t.a[5][4] = -5103.0 / 18656.0;
  t.a[6][0] = 35.0 / 384.0; t.a[6][1] = 0.0; t.a[6][2] = 500.0 / 1113.0;
  t.a[6][3] = 125.0 / 192.0; t.a[6][4] = -2187.0 / 6784.0; t.a[6][5] = 11.0 / 84.0;
  for (int j = 0; j < 7; ++j) t.b[j] = t.a[6][j];
  /* b - bhat, bhat = (5179/57600, 0, 7571/16695, 393/640, -92097/339200,
   * 187/2100, 1/40). */
  t.e[0] = 71.0 / 57600.0; t.e[1] = 0.0; t.e[2] = -71.0 / 16695.0;
  t.e[3] = 71.0 / 1920.0; t.e[4] = -17253.0 / 339200.0; t.e[5] = 22.0 / 525.0;
  t.e[6] = -1.0 / 40.0;
  t.order = 5; t.err_order = 4;
  return t;
}

const Tableau TSIT5 = make_tsit5();
const Tableau DOPRI5 = make_dopri5();

/* ROS2 constant gamma = 1 + 1/sqrt(2). */
const double ROS2_GAMMA = 1.0 + 1.0 / std::sqrt(2.0);

/* ------------------------------------------------------------------ */
/* The caller's right-hand side                                         */
/* ------------------------------------------------------------------ */
/* f comes from a plugin built from the caller's source (user_types.h) and
 * evaluated on reals and on dual numbers.  Its vector-Jacobian products are
 * taken column by column, one dual pass per Jacobian column:
 *   w_m = sum_i J[i][m] v_i                 (first product, then mac, i up)
 *   g_q <- g_q + sum_i Jp[i][q] v_i         (mac into g_q, i up)
 * Kinds >= R_USER all name the one right-hand side last set. */
template <class S, bool F> using UD = user::UDual<S, F>;
struct UserFns {
  int dim = 0, np = 0;
  void (*f64)(const double *, const double *, double *) = nullptr;
  void (*f32)(const float *, const float *, float *) = nullptr;
  void (*dp64)(const UD<double, false> *, const UD<double, false> *, UD<double, false> *) = nullptr;
  void (*df64)(const UD<double, true> *, const UD<double, true> *, UD<double, true> *) = nullptr;
  void (*dp32)(const UD<float, false> *, const UD<float, false> *, UD<float, false> *) = nullptr;
  void (*df32)(const UD<float, true> *, const UD<float, true> *, UD<float, true> *) = nullptr;
};
UserFns g_user;

inline void user_eval(const double *y, const double *p, double *o) { g_user.f64(y, p, o); }
inline void user_eval(const float *y, const float *p, float *o) { g_user.f32(y, p, o); }
inline void user_eval(const UD<double, false> *y, const UD<double, false> *p,
                      UD<double, false> *o) { g_user.dp64(y, p, o); }
inline void user_eval(const UD<double, true> *y, const UD<double, true> *p, UD<double, true> *o) {
  g_user.df64(y, p, o);
}
inline void user_eval(const UD<float, false> *y, const UD<float, false> *p, UD<float, false> *o) {
  g_user.dp32(y, p, o);
}
inline void user_eval(const UD<float, true> *y, const UD<float, true> *p, UD<float, true> *o) {
  g_user.df32(y, p, o);
}

/* f on the oracle's own dual types (the JVP and sensitivity checks): through
 * the plugin's dual type of the same rounding. */
template <class DT, bool FU>
void user_eval_dual(int d, const DT *y, const DT *p, DT *o) {
  UD<double, FU> yu[MAXD], pu[MAXP], ou[MAXD];
  for (int c = 0; c < d; ++c) yu[c] = UD<double, FU>(y[c].v, y[c].d);
  for (int q = 0; q < g_user.np; ++q) pu[q] = UD<double, FU>(p[q].v, p[q].d);
  user_eval(yu, pu, ou);
  for (int c = 0; c < d; ++c) o[c] = DT(ou[c].v, ou[c].d);
}

template <class T, bool F>
void user_f(int d, const T *y, const T *p, T *o);

/* Jacobian columns of the caller's f at (y, p): Jy[i][m] for the states
 * (wrt_p false) or Jp[i][q] for the parameters (wrt_p true). */
template <class T, bool F>
void user_jacobian(int d, const T *y, const T *p, bool wrt_p, T (*J)[MAXD > MAXP ? MAXD : MAXP]) {
  using U = UD<T, F>;
  const int ncol = wrt_p ? g_user.np : d;
  for (int m = 0; m < ncol; ++m) {
    U yd[MAXD], pd[MAXP], od[MAXD];
    for (int c = 0; c < d; ++c) yd[c] = U(y[c], (!wrt_p && c == m) ? T(1) : T(0));
    for (int q = 0; q < g_user.np; ++q) pd[q] = U(p[q], (wrt_p && q == m) ? T(1) : T(0));
    user_eval(yd, pd, od);
    for (int i = 0; i < d; ++i) J[i][m] = od[i].d;
  }
}

template <class T, bool F>
void user_vjp_y(int d, const T *y, const T *p, const T *v, T *w) {
  if constexpr (std::is_same<T, double>::value || std::is_same<T, float>::value) {
    T J[MAXD][MAXD > MAXP ? MAXD : MAXP];
    user_jacobian<T, F>(d, y, p, false, J);
    for (int m = 0; m < d; ++m) {
      T acc = J[0][m] * v[0];
      for (int i = 1; i < d; ++i) acc = mac<F>(J[i][m], v[i], acc);
      w[m] = acc;
    }
  } else {
    for (int m = 0; m < d; ++m) w[m] = T(NAN);
  }
}

template <class T, bool F>
void user_vjp_p_acc(int d, const T *y, const T *p, const T *v, T *g) {
  if constexpr (std::is_same<T, double>::value || std::is_same<T, float>::value) {
    T J[MAXD][MAXD > MAXP ? MAXD : MAXP];
    user_jacobian<T, F>(d, y, p, true, J);
    for (int q = 0; q < g_user.np; ++q)
      for (int i = 0; i < d; ++i) g[q] = mac<F>(J[i][q], v[i], g[q]);
  } else {
    for (int q = 0; q < g_user.np; ++q) g[q] = T(NAN);
  }
}

template <class T, bool F>
void user_f(int d, const T *y, const T *p, T *o) {
  if constexpr (std::is_same<T, double>::value || std::is_same<T, float>::value) {
    user_eval(y, p, o);
  } else if constexpr (std::is_same<T, DualF>::value) {
    user_eval_dual<DualF, true>(d, y, p, o);
  } else {
    user_eval_dual<T, false>(d, y, p, o);
  }
}

/* ------------------------------------------------------------------ */
/* Right-hand sides: f, Jacobian, vector-Jacobian products             */
/* ------------------------------------------------------------------ */
/* Conventions:
 *  vjp_y: w[j] = sum_i J[i][j] v[i], rows i in the order listed per system.
 *  vjp_p_acc: g[q] += sum_i (df_i/dp_q) v[i], each term a multiply-add into g.
 *  jac_contract_acc: gy[c] += sum_ab Jbar[a][b] dJ[a][b]/dy_c and likewise
 *  gp[q], each term a multiply-add into the accumulator, entries (a,b) in
 *  row-major order. */

/* Eight-species reaction cycle, a synthetic stiff system of the size of the
 * HIRES test problem (whose equations are not restated here).  Nine
 * mass-action reactions move one unit of mass each from species src to
 * species dst, so sum_i y_i is conserved; reaction r has rate
 *   w_r = (c_r p_{q_r}) y_a            (one reactant a), or
 *   w_r = ((c_r p_{q_r}) y_a) y_b      (two reactants, in that order),
 * and f = sum_r (e_dst - e_src) w_r.  With p = (0.04, 3e7, 1e4, 1) the rates
 * span ten orders of magnitude (the first three reactions are those of
 * Robertson's system).  Arithmetic: sums over reactions in table order (a
 * product, then multiply-adds / additions); the partial derivatives of w_r
 * with respect to its reactants in reactant order. */
struct Reaction {
  int src, dst, q, na, a, b;
  double c;
};
const Reaction KIN8[9] = {
    {0, 1, 0, 1, 0, 0, 1.0},   /* y0 -> y1           p0 y0          */
    {1, 2, 1, 2, 1, 1, 1.0},   /* 2 y1 -> y1 + y2    p1 y1 y1       */
    {1, 0, 2, 2, 1, 2, 1.0},   /* y1 + y2 -> y0 + y2 p2 y1 y2       */
    {2, 3, 3, 1, 2, 0, 1.0},   /* y2 -> y3           p3 y2          */
    {3, 4, 3, 1, 3, 0, 10.0},  /* y3 -> y4           10 p3 y3       */
    {4, 5, 1, 2, 4, 4, 1e-3},  /* 2 y4 -> y4 + y5    1e-3 p1 y4 y4  */
    {5, 6, 0, 1, 5, 0, 25.0},  /* y5 -> y6           25 p0 y5       */
    {6, 7, 2, 2, 6, 2, 0.1},   /* y6 + y2 -> y7 + y2 0.1 p2 y6 y2   */
    {7, 0, 3, 1, 7, 0, 0.01},  /* y7 -> y0           0.01 p3 y7     */
};

/* Partial derivatives of w_r: the columns cols[0..n) and their values. */
template <class T>
int kin8_partials(const Reaction &r, const T *y, const T *p, int *cols, T *vals) {
  const T k = T(r.c) * p[r.q];
  if (r.na == 1) {
    cols[0] = r.a; vals[0] = k;
    return 1;
  }
  if (r.a == r.b) {
    cols[0] = r.a; vals[0] = (T(2.0) * k) * y[r.a];
    return 1;
  }
  cols[0] = r.a; vals[0] = k * y[r.b];
  cols[1] = r.b; vals[1] = k * y[r.a];
  return 2;
}

template <class T>
T kin8_rate(const Reaction &r, const T *y, const T *p) {
  const T w = (T(r.c) * p[r.q]) * y[r.a];
  return r.na == 2 ? w * y[r.b] : w;
}

template <class T, bool F>
void rhs_f(int kind, int d, const T *y, const T *p, T *out) {
  if (kind >= R_USER) {
    user_f<T, F>(d, y, p, out);
    return;
  }
  switch (kind) {
    case R_LINEAR:  /* y' = p0 y */
      out[0] = p[0] * y[0];
      break;
    case R_LORENZ63: {  /* sigma (u2-u1), u1 (rho-u3) - u2, u1 u2 - beta u3 */
      const T s = p[0], r = p[1], b = p[2];
      out[0] = s * (y[1] - y[0]);
      out[1] = mac<F>(y[0], r - y[2], -y[1]);
      out[2] = mac<F>(y[0], y[1], -(b * y[2]));
      break;
    }
    case R_ROBERTSON: {
      /* y1' = -k1 y1 + k3 y2 y3
       * y2' =  k1 y1 - k2 y2^2 - k3 y2 y3
       * y3' =  k2 y2^2 */
      const T k1 = p[0], k2 = p[1], k3 = p[2];
      out[0] = mac<F>(k3 * y[1], y[2], (-k1) * y[0]);
      T s = k1 * y[0];
      s = mac<F>(-(k2 * y[1]), y[1], s);
      s = mac<F>(-(k3 * y[1]), y[2], s);
      out[1] = s;
      out[2] = (k2 * y[1]) * y[1];
      break;
    }
    case R_LORENZ96: {  /* x_i' = (x_{i+1} - x_{i-2}) x_{i-1} - x_i + F */
      const T Fc = p[0];
      for (int i = 0; i < d; ++i) {
        const T xp1 = y[(i + 1) % d], xm1 = y[(i + d - 1) % d], xm2 = y[(i + d - 2) % d];
        const T a = xp1 - xm2;
        out[i] = mac<F>(a, xm1, -y[i]) + Fc;
      }
      break;
    }
    case R_KINETICS8: {
      T w[9];
      for (int r = 0; r < 9; ++r) w[r] = kin8_rate(KIN8[r], y, p);
      for (int a = 0; a < 8; ++a) {
        T acc = T(0.0);
        bool first = true;
        for (int r = 0; r < 9; ++r) {
          if (KIN8[r].src == a) { acc = first ? -w[r] : acc - w[r]; first = false; }
          if (KIN8[r].dst == a) { acc = first ? w[r] : acc + w[r]; first = false; }
        }
        out[a] = acc;
      }
      break;
    }
  }
}

/* Explicit Jacobian J[a*d+b] = df_a/dy_b (small systems; Rosenbrock only). */
template <class T, bool F>
void rhs_jac(int kind, int d, const T *y, const T *p, T *J) {
  for (int i = 0; i < d * d; ++i) J[i] = T(0.0);
  switch (kind) {
    case R_LINEAR:
      J[0] = p[0];
      break;
    case R_LORENZ63: {
      const T s = p[0], r = p[1], b = p[2];
      J[0] = -s;        J[1] = s;          J[2] = T(0.0);
      J[3] = r - y[2];  J[4] = T(-1.0);    J[5] = -y[0];
      J[6] = y[1];      J[7] = y[0];       J[8] = -b;
      break;
    }
    case R_ROBERTSON: {
      const T k1 = p[0], k2 = p[1], k3 = p[2];
      J[0] = -k1;  J[1] = k3 * y[2];  J[2] = k3 * y[1];
      /* J22 = -2 k2 y2 - k3 y3 */
      J[3] = k1;   J[4] = mac<F>(-k3, y[2], -(T(2.0) * k2) * y[1]);  J[5] = -(k3 * y[1]);
      J[6] = T(0.0); J[7] = T(2.0) * k2 * y[1]; J[8] = T(0.0);
      break;
    }
    case R_KINETICS8: {
      /* J[a][b] = sum_r (e_dst - e_src)_a dw_r/dy_b, reactions in table order */
      bool set[64] = {};
      for (int r = 0; r < 9; ++r) {
        int cols[2];
        T vals[2];
        const int m = kin8_partials(KIN8[r], y, p, cols, vals);
        for (int e = 0; e < m; ++e) {
          const int b = cols[e];
          T &s = J[KIN8[r].src * 8 + b];
          s = set[KIN8[r].src * 8 + b] ? s - vals[e] : -vals[e];
          set[KIN8[r].src * 8 + b] = true;
          T &t = J[KIN8[r].dst * 8 + b];
          t = set[KIN8[r].dst * 8 + b] ? t + vals[e] : vals[e];
          set[KIN8[r].dst * 8 + b] = true;
        }
      }
      break;
    }
  }
}

template <class T, bool F>
void rhs_vjp_y(int kind, int d, const T *y, const T *p, const T *v, T *w) {
  if (kind >= R_USER) {
    user_vjp_y<T, F>(d, y, p, v, w);
    return;
  }
  switch (kind) {
    case R_LINEAR:
      w[0] = p[0] * v[0];
      break;
    case R_LORENZ63: {
      /* J = [[-s, s, 0], [r-u3, -1, -u1], [u2, u1, -b]]; rows 1,2,3 in order. */
      const T s = p[0], r = p[1], b = p[2];
      w[0] = mac<F>(y[1], v[2], mac<F>(r - y[2], v[1], (-s) * v[0]));
      w[1] = mac<F>(y[0], v[2], mac<F>(s, v[0], -v[1]));
      w[2] = mac<F>(-b, v[2], (-y[0]) * v[1]);
      break;
    }
    case R_ROBERTSON: {
      const T k1 = p[0], k2 = p[1], k3 = p[2];
      /* column 1: J11 = -k1, J21 = k1 */
      w[0] = mac<F>(k1, v[1], (-k1) * v[0]);
      /* column 2: J12 = k3 y3, J22 = -2 k2 y2 - k3 y3, J32 = 2 k2 y2 */
      const T j22 = mac<F>(-k3, y[2], -(T(2.0) * k2) * y[1]);
      T s = (k3 * y[2]) * v[0];
      s = mac<F>(j22, v[1], s);
      s = mac<F>(T(2.0) * k2 * y[1], v[2], s);
      w[1] = s;
      /* column 3: J13 = k3 y2, J23 = -k3 y2 */
      w[2] = mac<F>(-(k3 * y[1]), v[1], (k3 * y[1]) * v[0]);
      break;
    }
    case R_LORENZ96: {
      /* Column j has entries from rows j-1 (x_{j-2}), j (-1), j+1
       * (x_{j+2} - x_{j-1}) and j+2 (-x_{j+1}), taken in that order. */
      for (int j = 0; j < d; ++j) {
        const T xm2 = y[(j + d - 2) % d], xm1 = y[(j + d - 1) % d];
        const T xp1 = y[(j + 1) % d], xp2 = y[(j + 2) % d];
        const T vm1 = v[(j + d - 1) % d], vp1 = v[(j + 1) % d], vp2 = v[(j + 2) % d];
        T s = xm2 * vm1;
        s = s - v[j];
        s = mac<F>(xp2 - xm1, vp1, s);
        s = mac<F>(-xp1, vp2, s);
        w[j] = s;
      }
      break;
    }
    case R_KINETICS8: {
      /* w_b = sum_r dw_r/dy_b (v_dst - v_src), reactions in table order */
      bool set[8] = {};
      for (int r = 0; r < 9; ++r) {
        int cols[2];
        T vals[2];
        const int m = kin8_partials(KIN8[r], y, p, cols, vals);
        const T dl = v[KIN8[r].dst] - v[KIN8[r].src];
        for (int e = 0; e < m; ++e) {
          const int b = cols[e];
          w[b] = set[b] ? mac<F>(vals[e], dl, w[b]) : vals[e] * dl;
          set[b] = true;
        }
      }
      for (int b = 0; b < 8; ++b)
        if (!set[b]) w[b] = T(0.0);
      break;
    }
  }
}

template <class T, bool F>
void rhs_vjp_p_acc(int kind, int d, const T *y, const T *p, const T *v, T *g) {
  if (kind >= R_USER) {
    user_vjp_p_acc<T, F>(d, y, p, v, g);
    return;
  }
  switch (kind) {
    case R_LINEAR:  /* df/dp0 = y */
      g[0] = mac<F>(y[0], v[0], g[0]);
      break;
    case R_LORENZ63:  /* df/ds = (u2-u1,0,0), df/dr = (0,u1,0), df/db = (0,0,-u3) */
      g[0] = mac<F>(y[1] - y[0], v[0], g[0]);
      g[1] = mac<F>(y[0], v[1], g[1]);
      g[2] = mac<F>(-y[2], v[2], g[2]);
      break;
    case R_ROBERTSON: {
      /* df/dk1 = (-y1, y1, 0); df/dk2 = (0, -y2^2, y2^2);
       * df/dk3 = (y2 y3, -y2 y3, 0) */
      g[0] = mac<F>(-y[0], v[0], g[0]);
      g[0] = mac<F>(y[0], v[1], g[0]);
      const T y22 = y[1] * y[1];
      g[1] = mac<F>(-y22, v[1], g[1]);
      g[1] = mac<F>(y22, v[2], g[1]);
      const T y23 = y[1] * y[2];
      g[2] = mac<F>(y23, v[0], g[2]);
      g[2] = mac<F>(-y23, v[1], g[2]);
      break;
    }
    case R_LORENZ96:  /* df_i/dF = 1 */
      for (int i = 0; i < d; ++i) g[0] = g[0] + v[i];
      break;
    case R_KINETICS8:
      /* g_q += dw_r/dp_q (v_dst - v_src), dw_r/dp_q = c_r y_a [y_b] */
      for (int r = 0; r < 9; ++r) {
        const Reaction &k = KIN8[r];
        T dw = T(k.c) * y[k.a];
        if (k.na == 2) dw = dw * y[k.b];
        g[k.q] = mac<F>(dw, v[k.dst] - v[k.src], g[k.q]);
      }
      break;
  }
}

/* Second-derivative contraction needed by the Rosenbrock adjoint. */
template <class T, bool F>
void rhs_jac_contract_acc(int kind, int d, const T *y, const T *p, const T *Jb,
                          T *gy, T *gp) {
  switch (kind) {
    case R_LINEAR:  /* J = p0: dJ/dp0 = 1 */
      gp[0] = gp[0] + Jb[0];
      break;
    case R_LORENZ63:
      /* J11=-s, J12=s, J21=r-u3, J23=-u1, J31=u2, J32=u1, J33=-b */
      gp[0] = gp[0] - Jb[0];
      gp[0] = gp[0] + Jb[1];
      gp[1] = gp[1] + Jb[3];
      gy[2] = gy[2] - Jb[3];
      gy[0] = gy[0] - Jb[5];
      gy[1] = gy[1] + Jb[6];
      gy[0] = gy[0] + Jb[7];
      gp[2] = gp[2] - Jb[8];
      break;
    case R_ROBERTSON: {
      const T k1 = p[0], k2 = p[1], k3 = p[2];
      (void)k1;
      /* entries in row-major order:
       * J11=-k1: d/dk1=-1
       * J12=k3 y3: d/dy3=k3, d/dk3=y3
       * J13=k3 y2: d/dy2=k3, d/dk3=y2
       * J21=k1: d/dk1=1
       * J22=-2k2y2-k3y3: d/dy2=-2k2, d/dy3=-k3, d/dk2=-2y2, d/dk3=-y3
       * J23=-k3 y2: d/dy2=-k3, d/dk3=-y2
       * J32=2k2y2: d/dy2=2k2, d/dk2=2y2 */
      const T two_k2 = T(2.0) * k2, two_y2 = T(2.0) * y[1];
      gp[0] = gp[0] - Jb[0];
      gy[2] = mac<F>(k3, Jb[1], gy[2]);
      gp[2] = mac<F>(y[2], Jb[1], gp[2]);
      gy[1] = mac<F>(k3, Jb[2], gy[1]);
      gp[2] = mac<F>(y[1], Jb[2], gp[2]);
      gp[0] = gp[0] + Jb[3];
      gy[1] = mac<F>(-two_k2, Jb[4], gy[1]);
      gy[2] = mac<F>(-k3, Jb[4], gy[2]);
      gp[1] = mac<F>(-two_y2, Jb[4], gp[1]);
      gp[2] = mac<F>(-y[2], Jb[4], gp[2]);
      gy[1] = mac<F>(-k3, Jb[5], gy[1]);
      gp[2] = mac<F>(-y[1], Jb[5], gp[2]);
      gy[1] = mac<F>(two_k2, Jb[7], gy[1]);
      gp[1] = mac<F>(two_y2, Jb[7], gp[1]);
      break;
    }
    case R_KINETICS8:
      /* J = S dw/dy: for each partial dw_r/dy_b, with M = Jbar[dst][b] -
       * Jbar[src][b], add M times its derivatives (reactions in table order,
       * partials in reactant order, y before p) */
      for (int r = 0; r < 9; ++r) {
        const Reaction &k = KIN8[r];
        const T kk = T(k.c) * p[k.q];
        auto M = [&](int b) { return Jb[k.dst * 8 + b] - Jb[k.src * 8 + b]; };
        if (k.na == 1) {
          gp[k.q] = mac<F>(T(k.c), M(k.a), gp[k.q]);
        } else if (k.a == k.b) {
          const T m = M(k.a);
          gy[k.a] = mac<F>(T(2.0) * kk, m, gy[k.a]);
          gp[k.q] = mac<F>((T(2.0) * T(k.c)) * y[k.a], m, gp[k.q]);
        } else {
          const T ma = M(k.a);  /* partial k y_b in column a */
          gy[k.b] = mac<F>(kk, ma, gy[k.b]);
          gp[k.q] = mac<F>(T(k.c) * y[k.b], ma, gp[k.q]);
          const T mb = M(k.b);  /* partial k y_a in column b */
          gy[k.a] = mac<F>(kk, mb, gy[k.a]);
          gp[k.q] = mac<F>(T(k.c) * y[k.a], mb, gp[k.q]);
        }
      }
      break;
  }
}

bool rhs_shape_ok(int kind, int d, int P) {
  if (kind >= R_USER) return g_user.f64 && d == g_user.dim && P == g_user.np;
  switch (kind) {
    case R_LINEAR: return d == 1 && P == 1;
    case R_LORENZ63: return d == 3 && P == 3;
    case R_ROBERTSON: return d == 3 && P == 3;
    case R_LORENZ96: return d >= 4 && d <= MAXD && P == 1;
    case R_KINETICS8: return d == 8 && P == 4;
  }
  return false;
}

/* ------------------------------------------------------------------ */
/* Explicit RK step                                                    */
/* ------------------------------------------------------------------ */

/* Stages of one step from y with size h.  Stage 0 is y itself; K[0] must hold
 * f(y) on entry.  Computes Y[1..last] and K[1..kl] where kl = last when
 * with_last_k, else last-1.  Y[i][c] = y[c] + h * sum_{j<i} a[i][j] K[j][c]. */
template <class T, bool F>
void erk_stages(const Tableau &tb, int kind, int d, const T *y, const T *p, T h,
                int last, bool with_last_k, T (*Y)[MAXD], T (*K)[MAXD]) {
  const T *Kp[7];
  for (int j = 0; j < 7; ++j) Kp[j] = K[j];
  for (int c = 0; c < d; ++c) Y[0][c] = y[c];
  for (int i = 1; i <= last; ++i) {
    for (int c = 0; c < d; ++c) {
      const T acc = chain<T, F>(i, tb.a[i], Kp, c);
      Y[i][c] = mac<F>(h, acc, y[c]);
    }
    if (i < last || with_last_k) rhs_f<T, F>(kind, d, Y[i], p, K[i]);
  }
}

/* Replay step: y <- y + h sum_j b_j k_j (the 7th stage state). */
template <class T, bool F>
void erk_step(const Tableau &tb, int kind, int d, T *y, const T *p, T h) {
  T Y[7][MAXD], K[7][MAXD];
  rhs_f<T, F>(kind, d, y, p, K[0]);
  erk_stages<T, F>(tb, kind, d, y, p, h, 6, false, Y, K);
  for (int c = 0; c < d; ++c) y[c] = Y[6][c];
}

/* Reverse of erk_step: lam holds dL/dy_{k+1} on entry, dL/dy_k on exit;
 * gp accumulates dL/dp.  Stage states are recomputed from y = y_k. */
template <class T, bool F>
void erk_step_adjoint(const Tableau &tb, int kind, int d, const T *y, const T *p,
                      T h, T *lam, T *gp, T *gpc = nullptr) {
  T Y[7][MAXD], K[7][MAXD], Wv[7][MAXD], kb[MAXD], lacc[MAXD];
  rhs_f<T, F>(kind, d, y, p, K[0]);
  erk_stages<T, F>(tb, kind, d, y, p, h, 5, false, Y, K);
  for (int c = 0; c < d; ++c) lacc[c] = lam[c];
  for (int i = 5; i >= 0; --i) {
    /* kbar_i = h (b_i lam + sum_{l>i} a[l][i] w_l), terms in that order */
    for (int c = 0; c < d; ++c) {
      T acc = T(0.0);
      bool first = true;
      if (tb.b[i] != 0.0) { acc = T(tb.b[i]) * lam[c]; first = false; }
      for (int l = i + 1; l <= 5; ++l) {
        if (tb.a[l][i] == 0.0) continue;
        if (first) { acc = T(tb.a[l][i]) * Wv[l][c]; first = false; }
        else acc = mac<F>(T(tb.a[l][i]), Wv[l][c], acc);
      }
      kb[c] = h * acc;
    }
    rhs_vjp_y<T, F>(kind, d, Y[i], p, kb, Wv[i]);
    if (gpc)  /* Lorenz-96, df_c/dF = 1: component c contributes kb[c] */
      for (int c = 0; c < d; ++c) gpc[c] = gpc[c] + kb[c];
    else
      rhs_vjp_p_acc<T, F>(kind, d, Y[i], p, kb, gp);
    for (int c = 0; c < d; ++c) lacc[c] = lacc[c] + Wv[i][c];
  }
  for (int c = 0; c < d; ++c) lam[c] = lacc[c];
}

/* ------------------------------------------------------------------ */
/* Fehlberg 7(8)                                                       */
/* ------------------------------------------------------------------ */

/* Fehlberg's seventh-order pair with an eighth-order companion (Fehlberg
 * 1968, NASA TR R-287): 13 stages, rational coefficients.  The 7th-order
 * solution y + h sum b_j K_j uses K_1..K_11 and is propagated; the 8th-order
 * one differs by (41/840) h (K_12 + K_13 - K_1 - K_11), and that difference
 * is the error estimate (err = h sum e_j K_j, e = b7 - b8).  Not first same
 * as last.  The coefficients are typed as the published fractions; a test
 * checks them against the order conditions. */
struct Rk78Tab {
  double a[13][13];
  double b[13];  /* 7th order */
  double e[13];  /* b7 - b8 */
};

Rk78Tab make_rk78() {
  Rk78Tab t;
  std::memset(&t, 0, sizeof t);
  double (&a)[13][13] = t.a;
  a[1][0] = 2.0 / 27.0;
  a[2][0] = 1.0 / 36.0; a[2][1] = 1.0 / 12.0;
  a[3][0] = 1.0 / 24.0; a[3][2] = 1.0 / 8.0;
  a[4][0] = 5.0 / 12.0; a[4][2] = -25.0 / 16.0; a[4][3] = 25.0 / 16.0;
  a[5][0] = 1.0 / 20.0; a[5][3] = 1.0 / 4.0; a[5][4] = 1.0 / 5.0;
  a[6][0] = -25.0 / 108.0; a[6][3] = 125.0 / 108.0; a[6][4] = -65.0 / 27.0;
  a[6][5] = 125.0 / 54.0;
  a[7][0] = 31.0 / 300.0; a[7][4] = 61.0 / 225.0; a[7][5] = -2.0 / 9.0; a[7][6] = 13.0 / 900.0;
  a[8][0] = 2.0; a[8][3] = -53.0 / 6.0; a[8][4] = 704.0 / 45.0; a[8][5] = -107.0 / 9.0;
  a[8][6] = 67.0 / 90.0; a[8][7] = 3.0;
  a[9][0] = -91.0 / 108.0; a[9][3] = 23.0 / 108.0; a[9][4] = -976.0 / 135.0;
  a[9][5] = 311.0 / 54.0; a[9][6] = -19.0 / 60.0; a[9][7] = 17.0 / 6.0; a[9][8] = -1.0 / 12.0;
  a[10][0] = 2383.0 / 4100.0; a[10][3] = -341.0 / 164.0; a[10][4] = 4496.0 / 1025.0;
  a[10][5] = -301.0 / 82.0; a[10][6] = 2133.0 / 4100.0; a[10][7] = 45.0 / 82.0;
  a[10][8] = 45.0 / 164.0; a[10][9] = 18.0 / 41.0;
  a[11][0] = 3.0 / 205.0; a[11][5] = -6.0 / 41.0; a[11][6] = -3.0 / 205.0;
  a[11][7] = -3.0 / 41.0; a[11][8] = 3.0 / 41.0; a[11][9] = 6.0 / 41.0;
  a[12][0] = -1777.0 / 4100.0; a[12][3] = -341.0 / 164.0; a[12][4] = 4496.0 / 1025.0;
  a[12][5] = -289.0 / 82.0; a[12][6] = 2193.0 / 4100.0; a[12][7] = 51.0 / 82.0;
  a[12][8] = 33.0 / 164.0; a[12][9] = 12.0 / 41.0; a[12][11] = 1.0;
  double b8[13] = {};
  t.b[0] = 41.0 / 840.0; t.b[5] = 34.0 / 105.0; t.b[6] = 9.0 / 35.0; t.b[7] = 9.0 / 35.0;
  t.b[8] = 9.0 / 280.0; t.b[9] = 9.0 / 280.0; t.b[10] = 41.0 / 840.0;
  b8[5] = 34.0 / 105.0; b8[6] = 9.0 / 35.0; b8[7] = 9.0 / 35.0; b8[8] = 9.0 / 280.0;
  b8[9] = 9.0 / 280.0; b8[11] = 41.0 / 840.0; b8[12] = 41.0 / 840.0;
  for (int j = 0; j < 13; ++j) t.e[j] = t.b[j] - b8[j];
  return t;
}
const Rk78Tab RK78 = make_rk78();
constexpr int RK78_ORDER = 7, RK78_ERR_ORDER = 7;  /* error of the 7th-order solution: h^8 */

/* Stage i of a step: Y_i = fma(h, sum_{j<i} a_ij K_j, y) (a product, then
 * multiply-adds), K_i = f(Y_i), for i = 1..last. */
template <class T, bool F>
void rk78_stages(int kind, int d, const T *y, const T *p, T h, int last, T (*Y)[MAXD],
                 T (*K)[MAXD]) {
  for (int c = 0; c < d; ++c) Y[0][c] = y[c];
  rhs_f<T, F>(kind, d, y, p, K[0]);
  for (int i = 1; i <= last; ++i) {
    for (int c = 0; c < d; ++c) {
      T acc = T(0.0);
      bool first = true;
      for (int j = 0; j < i; ++j) {
        if (RK78.a[i][j] == 0.0) continue;
        acc = first ? T(RK78.a[i][j]) * K[j][c] : mac<F>(T(RK78.a[i][j]), K[j][c], acc);
        first = false;
      }
      Y[i][c] = mac<F>(h, acc, y[c]);
    }
    rhs_f<T, F>(kind, d, Y[i], p, K[i]);
  }
}

/* sum_j w_j K_j[c] over the nonzero weights (a product, then multiply-adds) */
template <class T, bool F>
T rk78_combine(const double *w, const T (*K)[MAXD], int c) {
  T acc = T(0.0);
  bool first = true;
  for (int j = 0; j < 13; ++j) {
    if (w[j] == 0.0) continue;
    acc = first ? T(w[j]) * K[j][c] : mac<F>(T(w[j]), K[j][c], acc);
    first = false;
  }
  return acc;
}

/* Trial step of the record: all 13 stages, the 7th-order solution and the
 * error estimate. */
template <class T, bool F>
void rk78_attempt(int kind, int d, const T *y, const T *p, T h, T *ynew, T *err) {
  T Y[13][MAXD], K[13][MAXD];
  rk78_stages<T, F>(kind, d, y, p, h, 12, Y, K);
  for (int c = 0; c < d; ++c) {
    ynew[c] = mac<F>(h, rk78_combine<T, F>(RK78.b, K, c), y[c]);
    err[c] = h * rk78_combine<T, F>(RK78.e, K, c);
  }
}

/* Replay step: the 7th-order solution needs K_1..K_11. */
template <class T, bool F>
void rk78_step(int kind, int d, T *y, const T *p, T h) {
  T Y[13][MAXD], K[13][MAXD];
  rk78_stages<T, F>(kind, d, y, p, h, 10, Y, K);
  for (int c = 0; c < d; ++c) y[c] = mac<F>(h, rk78_combine<T, F>(RK78.b, K, c), y[c]);
}

/* Reverse of rk78_step: kbar_i = h (b_i lam + sum_{l>i} a_li w_l) for
 * i = 10..0 (terms in that order), w_i = J(Y_i)^T kbar_i,
 * g += J_p(Y_i)^T kbar_i, then lam + w_10 + w_9 + ... + w_0. */
template <class T, bool F>
void rk78_step_adjoint(int kind, int d, const T *y, const T *p, T h, T *lam, T *gp) {
  T Y[13][MAXD], K[13][MAXD], Wv[11][MAXD], kb[MAXD], lacc[MAXD];
  rk78_stages<T, F>(kind, d, y, p, h, 10, Y, K);
  for (int c = 0; c < d; ++c) lacc[c] = lam[c];
  for (int i = 10; i >= 0; --i) {
    for (int c = 0; c < d; ++c) {
      T acc = T(0.0);
      bool first = true;
      if (RK78.b[i] != 0.0) { acc = T(RK78.b[i]) * lam[c]; first = false; }
      for (int l = i + 1; l <= 10; ++l) {
        if (RK78.a[l][i] == 0.0) continue;
        acc = first ? T(RK78.a[l][i]) * Wv[l][c] : mac<F>(T(RK78.a[l][i]), Wv[l][c], acc);
        first = false;
      }
      kb[c] = h * acc;
    }
    rhs_vjp_y<T, F>(kind, d, Y[i], p, kb, Wv[i]);
    rhs_vjp_p_acc<T, F>(kind, d, Y[i], p, kb, gp);
    for (int c = 0; c < d; ++c) lacc[c] = lacc[c] + Wv[i][c];
  }
  for (int c = 0; c < d; ++c) lam[c] = lacc[c];
}

/* ------------------------------------------------------------------ */
/* ROS2 step                                                           */
/* ------------------------------------------------------------------ */

/* LU with partial pivoting of the d x d matrix A (row-major, in place);
 * perm[i] = original row now in position i.  Ties keep the lowest row.
 * Plain mode divides by the pivot; fused mode (the kernels' schedule) forms
 * the pivot's reciprocal 1 / u once and multiplies by it, here and in both
 * solves. */
template <class T, bool F>
void lu_factor(int d, T *A, int *perm) {
  for (int i = 0; i < d; ++i) perm[i] = i;
  for (int k = 0; k < d; ++k) {
    int piv = k;
    double best = std::fabs(val(A[k * d + k]));
    for (int i = k + 1; i < d; ++i) {
      const double v = std::fabs(val(A[i * d + k]));
      if (v > best) { best = v; piv = i; }
    }
    if (piv != k) {
      for (int j = 0; j < d; ++j) std::swap(A[k * d + j], A[piv * d + j]);
      std::swap(perm[k], perm[piv]);
    }
    const T r = T(1.0) / A[k * d + k];
    for (int i = k + 1; i < d; ++i) {
      const T l = F ? A[i * d + k] * r : A[i * d + k] / A[k * d + k];
      A[i * d + k] = l;
      for (int j = k + 1; j < d; ++j) A[i * d + j] = mac<F>(-l, A[k * d + j], A[i * d + j]);
    }
  }
}

/* Solve A x = b from the factors. */
template <class T, bool F>
void lu_solve(int d, const T *LU, const int *perm, const T *b, T *x) {
  for (int i = 0; i < d; ++i) x[i] = b[perm[i]];
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < i; ++j) x[i] = mac<F>(-LU[i * d + j], x[j], x[i]);
  for (int i = d - 1; i >= 0; --i) {
    for (int j = i + 1; j < d; ++j) x[i] = mac<F>(-LU[i * d + j], x[j], x[i]);
    x[i] = F ? x[i] * (T(1.0) / LU[i * d + i]) : x[i] / LU[i * d + i];
  }
}

/* Solve A^T x = b from the factors of A (P A = L U, so A^T = U^T L^T P). */
template <class T, bool F>
void lu_solve_t(int d, const T *LU, const int *perm, const T *b, T *x) {
  T z[MAXD];
  for (int i = 0; i < d; ++i) {
    z[i] = b[i];
    for (int j = 0; j < i; ++j) z[i] = mac<F>(-LU[j * d + i], z[j], z[i]);
    z[i] = F ? z[i] * (T(1.0) / LU[i * d + i]) : z[i] / LU[i * d + i];
  }
  for (int i = d - 1; i >= 0; --i)
    for (int j = i + 1; j < d; ++j) z[i] = mac<F>(-LU[j * d + i], z[j], z[i]);
  for (int i = 0; i < d; ++i) x[perm[i]] = z[i];
}

/* Everything one ROS2 step computes from (y, h). */
template <class T>
struct Ros2Step {
  T J[MAXR * MAXR], LU[MAXR * MAXR];
  int perm[MAXR];
  T f1[MAXR], k1[MAXR], Y2[MAXR], f2[MAXR], r2[MAXR], k2[MAXR], ynew[MAXR], err[MAXR];
};

/* W = I - gamma h J; k1 = W^-1 f(y); Y2 = y + h k1;
 * k2 = W^-1 (f(Y2) - 2 k1); y+ = y + h (3/2 k1 + 1/2 k2);
 * err = h (1/2 k1 + 1/2 k2)  (difference to the first-order y + h k1). */
template <class T, bool F>
void ros2_forward(int kind, int d, const T *y, const T *p, T h, Ros2Step<T> &s) {
  rhs_jac<T, F>(kind, d, y, p, s.J);
  const T gh = T(ROS2_GAMMA) * h;
  for (int a = 0; a < d; ++a)
    for (int b = 0; b < d; ++b)
      s.LU[a * d + b] = (a == b) ? mac<F>(-gh, s.J[a * d + b], T(1.0)) : (-gh) * s.J[a * d + b];
  lu_factor<T, F>(d, s.LU, s.perm);
  rhs_f<T, F>(kind, d, y, p, s.f1);
  lu_solve<T, F>(d, s.LU, s.perm, s.f1, s.k1);
  for (int c = 0; c < d; ++c) s.Y2[c] = mac<F>(h, s.k1[c], y[c]);
  rhs_f<T, F>(kind, d, s.Y2, p, s.f2);
  for (int c = 0; c < d; ++c) s.r2[c] = mac<F>(T(-2.0), s.k1[c], s.f2[c]);
  lu_solve<T, F>(d, s.LU, s.perm, s.r2, s.k2);
  for (int c = 0; c < d; ++c) {
    const T acc = mac<F>(T(0.5), s.k2[c], T(1.5) * s.k1[c]);
    s.ynew[c] = mac<F>(h, acc, y[c]);
    const T e = mac<F>(T(0.5), s.k2[c], T(0.5) * s.k1[c]);
    s.err[c] = h * e;
  }
}

template <class T, bool F>
void ros2_step(int kind, int d, T *y, const T *p, T h) {
  Ros2Step<T> s;
  ros2_forward<T, F>(kind, d, y, p, h, s);
  for (int c = 0; c < d; ++c) y[c] = s.ynew[c];
}

/* Reverse of ros2_step (mesh fixed): transposed solves with the same factors
 * and the contraction of Jbar with the derivative of J. */
template <class T, bool F>
void ros2_step_adjoint(int kind, int d, const T *y, const T *p, T h, T *lam, T *gp) {
  Ros2Step<T> s;
  ros2_forward<T, F>(kind, d, y, p, h, s);
  T yb[MAXR], kb1[MAXR], kb2[MAXR], rb1[MAXR], rb2[MAXR], Y2b[MAXR], w[MAXR], Wb[MAXR * MAXR],
      Jb[MAXR * MAXR];
  for (int c = 0; c < d; ++c) {
    const T ab = h * lam[c];      /* adjoint of the weighted stage sum */
    kb1[c] = T(1.5) * ab;
    kb2[c] = T(0.5) * ab;
    yb[c] = lam[c];
  }
  lu_solve_t<T, F>(d, s.LU, s.perm, kb2, rb2);
  for (int a = 0; a < d; ++a)
    for (int b = 0; b < d; ++b) Wb[a * d + b] = (-rb2[a]) * s.k2[b];
  rhs_vjp_y<T, F>(kind, d, s.Y2, p, rb2, Y2b);
  rhs_vjp_p_acc<T, F>(kind, d, s.Y2, p, rb2, gp);
  for (int c = 0; c < d; ++c) {
    kb1[c] = mac<F>(T(-2.0), rb2[c], kb1[c]);
    kb1[c] = mac<F>(h, Y2b[c], kb1[c]);
    yb[c] = yb[c] + Y2b[c];
  }
  lu_solve_t<T, F>(d, s.LU, s.perm, kb1, rb1);
  for (int a = 0; a < d; ++a)
    for (int b = 0; b < d; ++b) Wb[a * d + b] = mac<F>(-rb1[a], s.k1[b], Wb[a * d + b]);
  rhs_vjp_y<T, F>(kind, d, y, p, rb1, w);
  rhs_vjp_p_acc<T, F>(kind, d, y, p, rb1, gp);
  for (int c = 0; c < d; ++c) yb[c] = yb[c] + w[c];
  const T gh = T(ROS2_GAMMA) * h;
  for (int i = 0; i < d * d; ++i) Jb[i] = (-gh) * Wb[i];
  rhs_jac_contract_acc<T, F>(kind, d, y, p, Jb, yb, gp);
  for (int c = 0; c < d; ++c) lam[c] = yb[c];
}

/* ------------------------------------------------------------------ */
/* Rodas3 step                                                         */
/* ------------------------------------------------------------------ */

/* Rodas3 (Sandu, Verwer, Blom, Spee, Carmichael and Potra 1997, the
 * Rosenbrock solvers of atmospheric chemistry): four stages, order 3,
 * stiffly accurate and L-stable, with an embedded second-order solution.
 * With the same W = I - gamma h J as ROS2 (gamma = 1/2) the stages are
 *   Y_i = y + sum_{j<i} a_ij u_j,
 *   u_i = W^-1 (gamma h f(Y_i) + sum_{j<i} gamma c_ij u_j),
 * and y+ = y + sum m_i u_i, err = sum e_i u_i (here u_4).  The published form
 * solves (I / (gamma h) - J) u_i = f(Y_i) + sum_j (c_ij / h) u_j, which is the
 * same system multiplied by gamma h.  The coefficients are the published
 * ones; a test checks that they give order 3, L-stability and a second-order
 * embedded estimate. */
struct RosTab {
  int s;
  double gamma;
  double a[4][4], c[4][4], gc[4][4];  /* gc = gamma c */
  double m[4], e[4];
  int order, err_order;
};

RosTab make_rodas3() {
  RosTab t = {};
  t.s = 4;
  t.gamma = 0.5;
  t.a[2][0] = 2.0; t.a[3][0] = 2.0; t.a[3][2] = 1.0;
  t.c[1][0] = 4.0;
  t.c[2][0] = 1.0; t.c[2][1] = -1.0;
  t.c[3][0] = 1.0; t.c[3][1] = -1.0; t.c[3][2] = -8.0 / 3.0;
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) t.gc[i][j] = t.gamma * t.c[i][j];
  t.m[0] = 2.0; t.m[1] = 0.0; t.m[2] = 1.0; t.m[3] = 1.0;
  t.e[3] = 1.0;
  t.order = 3; t.err_order = 2;
  return t;
}
const RosTab RODAS3 = make_rodas3();

/* A fourth-order Rosenbrock method with an embedded third-order solution
 * (Shampine 1982, "Implementation of Rosenbrock methods", ACM TOMS 8:93;
 * four stages, A-stable, R(-inf) = 1/3), in the same transformed form:
 * gamma = 1/2; a_21 = 2, a_31 = a_41 = 48/25, a_32 = a_42 = 6/25 (the fourth
 * stage is evaluated at the third stage's point); c_21 = -8, c_31 = 372/25,
 * c_32 = 12/5, c_41 = -112/125, c_42 = -54/125, c_43 = -2/5; m = (19/9,
 * 1/2, 25/108, 125/108); e = (17/54, 7/36, 0, 125/108), the difference of
 * the fourth- and third-order solutions.  A test checks order 4 (linear and
 * nonlinear) and order 3 for the embedded solution. */
RosTab make_ros4() {
  RosTab t = {};
  t.s = 4;
  t.gamma = 0.5;
  t.a[1][0] = 2.0;
  t.a[2][0] = 48.0 / 25.0; t.a[2][1] = 6.0 / 25.0;
  t.a[3][0] = 48.0 / 25.0; t.a[3][1] = 6.0 / 25.0;
  t.c[1][0] = -8.0;
  t.c[2][0] = 372.0 / 25.0; t.c[2][1] = 12.0 / 5.0;
  t.c[3][0] = -112.0 / 125.0; t.c[3][1] = -54.0 / 125.0; t.c[3][2] = -2.0 / 5.0;
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) t.gc[i][j] = t.gamma * t.c[i][j];
  t.m[0] = 19.0 / 9.0; t.m[1] = 0.5; t.m[2] = 25.0 / 108.0; t.m[3] = 125.0 / 108.0;
  t.e[0] = 17.0 / 54.0; t.e[1] = 7.0 / 36.0; t.e[2] = 0.0; t.e[3] = 125.0 / 108.0;
  t.order = 4; t.err_order = 3;
  return t;
}
const RosTab ROS4 = make_ros4();

/* The four-stage Rosenbrock table of a method (null for the others). */
const RosTab *ros_tab(int method) {
  return method == M_RODAS3 ? &RODAS3 : method == M_ROS4 ? &ROS4 : nullptr;
}

template <class T>
struct RodasStep {
  T J[MAXR * MAXR], LU[MAXR * MAXR];
  int perm[MAXR];
  T Y[4][MAXR], f[4][MAXR], r[4][MAXR], u[4][MAXR], ynew[MAXR], err[MAXR];
};

/* Stage sums: Y_i from y, adding a_ij u_j for j = 0, 1, ...; r_i the sum of
 * gamma c_ij u_j (first a product, then multiply-adds), then gamma h f(Y_i)
 * added last; y+ from y adding m_i u_i in stage order. */
template <class T, bool F>
void rodas_forward(const RosTab &tb, int kind, int d, const T *y, const T *p, T h,
                   RodasStep<T> &s) {
  rhs_jac<T, F>(kind, d, y, p, s.J);
  const T gh = T(tb.gamma) * h;
  for (int a = 0; a < d; ++a)
    for (int b = 0; b < d; ++b)
      s.LU[a * d + b] = (a == b) ? mac<F>(-gh, s.J[a * d + b], T(1.0)) : (-gh) * s.J[a * d + b];
  lu_factor<T, F>(d, s.LU, s.perm);
  for (int i = 0; i < tb.s; ++i) {
    for (int c = 0; c < d; ++c) {
      T acc = y[c];
      for (int j = 0; j < i; ++j)
        if (tb.a[i][j] != 0.0) acc = mac<F>(T(tb.a[i][j]), s.u[j][c], acc);
      s.Y[i][c] = acc;
    }
    rhs_f<T, F>(kind, d, s.Y[i], p, s.f[i]);
    for (int c = 0; c < d; ++c) {
      T acc = T(0.0);
      bool first = true;
      for (int j = 0; j < i; ++j)
        if (tb.gc[i][j] != 0.0) {
          acc = first ? T(tb.gc[i][j]) * s.u[j][c] : mac<F>(T(tb.gc[i][j]), s.u[j][c], acc);
          first = false;
        }
      s.r[i][c] = first ? gh * s.f[i][c] : mac<F>(gh, s.f[i][c], acc);
    }
    lu_solve<T, F>(d, s.LU, s.perm, s.r[i], s.u[i]);
  }
  for (int c = 0; c < d; ++c) {
    T acc = y[c];
    for (int i = 0; i < tb.s; ++i)
      if (tb.m[i] != 0.0) acc = mac<F>(T(tb.m[i]), s.u[i][c], acc);
    s.ynew[c] = acc;
    T e = T(0.0);
    bool first = true;
    for (int i = 0; i < tb.s; ++i)
      if (tb.e[i] != 0.0) {
        e = first ? T(tb.e[i]) * s.u[i][c] : mac<F>(T(tb.e[i]), s.u[i][c], e);
        first = false;
      }
    s.err[c] = e;
  }
}

template <class T, bool F>
void rodas_step(const RosTab &tb, int kind, int d, T *y, const T *p, T h) {
  RodasStep<T> s;
  rodas_forward<T, F>(tb, kind, d, y, p, h, s);
  for (int c = 0; c < d; ++c) y[c] = s.ynew[c];
}

/* Reverse of rodas_step (mesh fixed), stages from the last to the first:
 *   ubar_i = m_i lam + sum_{l>i} (a_li Ybar_l + gamma c_li rbar_l)
 *            (in that order: the m term, then l = i+1, ... with its a term
 *            before its c term; first a product, then multiply-adds)
 *   rbar_i = W^-T ubar_i,  Wbar -= rbar_i u_i^T,  fbar_i = gamma h rbar_i,
 *   Ybar_i = J(Y_i)^T fbar_i,  g += J_p(Y_i)^T fbar_i,  ybar += Ybar_i;
 * then Jbar = -gamma h Wbar contracted with the derivative of J at y. */
template <class T, bool F>
void rodas_step_adjoint(const RosTab &tb, int kind, int d, const T *y, const T *p, T h, T *lam,
                        T *gp) {
  RodasStep<T> s;
  rodas_forward<T, F>(tb, kind, d, y, p, h, s);
  const T gh = T(tb.gamma) * h;
  T yb[MAXR], ub[MAXR], fb[MAXR], rb[4][MAXR], Yb[4][MAXR], Wb[MAXR * MAXR], Jb[MAXR * MAXR];
  for (int c = 0; c < d; ++c) yb[c] = lam[c];
  for (int i = tb.s - 1; i >= 0; --i) {
    for (int c = 0; c < d; ++c) {
      T acc = T(0.0);
      bool first = true;
      if (tb.m[i] != 0.0) {
        acc = T(tb.m[i]) * lam[c];
        first = false;
      }
      for (int l = i + 1; l < tb.s; ++l) {
        if (tb.a[l][i] != 0.0) {
          acc = first ? T(tb.a[l][i]) * Yb[l][c] : mac<F>(T(tb.a[l][i]), Yb[l][c], acc);
          first = false;
        }
        if (tb.gc[l][i] != 0.0) {
          acc = first ? T(tb.gc[l][i]) * rb[l][c] : mac<F>(T(tb.gc[l][i]), rb[l][c], acc);
          first = false;
        }
      }
      ub[c] = acc;
    }
    lu_solve_t<T, F>(d, s.LU, s.perm, ub, rb[i]);
    for (int a = 0; a < d; ++a)
      for (int b = 0; b < d; ++b)
        Wb[a * d + b] = (i == tb.s - 1) ? (-rb[i][a]) * s.u[i][b]
                                        : mac<F>(-rb[i][a], s.u[i][b], Wb[a * d + b]);
    for (int c = 0; c < d; ++c) fb[c] = gh * rb[i][c];
    rhs_vjp_y<T, F>(kind, d, s.Y[i], p, fb, Yb[i]);
    rhs_vjp_p_acc<T, F>(kind, d, s.Y[i], p, fb, gp);
    for (int c = 0; c < d; ++c) yb[c] = yb[c] + Yb[i][c];
  }
  for (int q = 0; q < d * d; ++q) Jb[q] = (-gh) * Wb[q];
  rhs_jac_contract_acc<T, F>(kind, d, y, p, Jb, yb, gp);
  for (int c = 0; c < d; ++c) lam[c] = yb[c];
}

/* ------------------------------------------------------------------ */
/* Problem helpers                                                     */
/* ------------------------------------------------------------------ */

struct Opts {
  double safety, fac_min, fac_max;
  int max_attempts;
  int S;               /* save slots: max(1, n_save) */
  const double *saves; /* S times; the last save of n_save = 0 is t1 */
  double t1_only[1];
};

Opts make_opts(const orc_problem *P) {
  Opts o;
  o.safety = P->safety > 0 ? P->safety : 0.9;
  o.fac_min = P->fac_min > 0 ? P->fac_min : 0.2;
  o.fac_max = P->fac_max > 0 ? P->fac_max : 10.0;
  o.max_attempts = P->max_attempts > 0 ? P->max_attempts : 4 * P->max_steps;
  o.t1_only[0] = P->t1;
  if (P->n_save > 0) { o.S = P->n_save; o.saves = P->save_times; }
  else { o.S = 1; o.saves = nullptr; }
  return o;
}

int validate(const orc_problem *P) {
  if (!P) return E_INVAL;
  if (P->method < 0 || P->method > 5) return E_INVAL;
  if (!rhs_shape_ok(P->rhs, P->dim, P->n_params)) return E_INVAL;
  const bool ros = P->method == M_ROS2 || ros_tab(P->method);
  /* the Rosenbrock methods need the explicit Jacobian of the built-in systems */
  if (ros && (P->dim > MAXR || P->rhs == R_LORENZ96)) return E_UNSUPPORTED;
  if (P->dense != 0 && P->dense != 1) return E_INVAL;
  if (P->dense && (ros || P->method == M_RKF78)) return E_UNSUPPORTED;
  if (P->method == M_RKF78 && (P->rhs == R_LORENZ96 || P->rhs >= R_USER)) return E_UNSUPPORTED;
  if (P->rhs >= R_USER && ros) return E_UNSUPPORTED;
  if (!(P->t1 > P->t0)) return E_INVAL;
  if (!(P->rtol >= 0) || !(P->atol >= 0) || !(P->rtol + P->atol > 0)) return E_INVAL;
  if (P->max_steps < 1) return E_INVAL;
  if (P->n_save < 0) return E_INVAL;
  if (P->n_save > 0) {
    if (!P->save_times) return E_INVAL;
    double prev = P->t0;
    for (int s = 0; s < P->n_save; ++s) {
      if (!(P->save_times[s] > prev) || P->save_times[s] > P->t1) return E_INVAL;
      prev = P->save_times[s];
    }
  }
  return E_OK;
}

/* RMS norm of v / sc over d components. */
template <class T, bool F>
T rms(int d, const T *v, const T *sc) {
  T s = T(0.0);
  for (int c = 0; c < d; ++c) {
    const T q = v[c] / sc[c];
    s = (c == 0) ? q * q : mac<F>(q, q, s);
  }
  return std::sqrt(s / T(d));
}

/* Error norm: RMS of err / (atol + rtol max(|y|, |y+|)). */
template <class T, bool F>
T err_norm(int d, const T *err, const T *y, const T *yn, T atol, T rtol) {
  T sc[MAXD];
  for (int c = 0; c < d; ++c)
    sc[c] = mac<F>(rtol, std::max(absval(y[c]), absval(yn[c])), atol);
  return rms<T, F>(d, err, sc);
}

/* The controller's power E^expo.  Plain mode: pow in the state's precision,
 * the textbook I-controller.  Fused mode (the kernels' schedule): in single
 * precision, exp2(expo log2 E) with E and expo rounded to float; the factor
 * only scales the next trial step, so this changes which steps are tried, not
 * the accept test E <= 1 or any accepted step's arithmetic. */
template <class T, bool F>
T ctrl_pow(T E, T expo) {
  if (F) return T(std::exp2(float(expo) * std::log2(float(E))));
  return std::pow(E, expo);
}

/* Starting step (HNW I, II.4) for a method of order q. */
template <class T, bool F>
T initial_step(int kind, int d, const T *y0, const T *f0, const T *p, T atol, T rtol,
               int q) {
  T sc[MAXD] = {}, y1[MAXD] = {}, f1[MAXD] = {}, df[MAXD] = {};
  for (int c = 0; c < d; ++c) sc[c] = mac<F>(rtol, absval(y0[c]), atol);
  const T d0 = rms<T, F>(d, y0, sc);
  const T d1 = rms<T, F>(d, f0, sc);
  T h0 = (d0 < T(1e-5) || d1 < T(1e-5)) ? T(1e-6) : T(0.01) * (d0 / d1);
  for (int c = 0; c < d; ++c) y1[c] = mac<F>(h0, f0[c], y0[c]);
  rhs_f<T, F>(kind, d, y1, p, f1);
  for (int c = 0; c < d; ++c) df[c] = f1[c] - f0[c];
  const T d2 = rms<T, F>(d, df, sc) / h0;
  const T dm = std::max(d1, d2);
  T h1;
  if (dm <= T(1e-15)) h1 = std::max(T(1e-6), h0 * T(1e-3));
  else h1 = std::pow(T(0.01) / dm, T(1.0) / T(q + 1));
  return std::min(T(100.0) * h0, h1);
}

/* ------------------------------------------------------------------ */
/* Dense output: save times read inside a step                         */
/* ------------------------------------------------------------------ */
/* "Differentiable astrophysics at scale" (gist.science summary),
 * Methodology, dense output: the solution is interpolated at observation
 * times instead of forcing steps to end on them.  The page names no
 * interpolant; the one used here is the cubic Hermite interpolant of an
 * accepted step [t_k, t_k + h] through its end states and end slopes
 * f(y_k), f(y_{k+1}) (for a first-same-as-last pair these are the step's
 * first and last stage derivatives, so no extra stage is needed):
 *   y(t_k + th h) = H00 y_k + H01 y_{k+1} + h (H10 f(y_k) + H11 f(y_{k+1}))
 *   H00 = (1 - th)^2 (1 + 2 th)    H01 = th^2 (3 - 2 th)
 *   H10 = th (1 - th)^2            H11 = -th^2 (1 - th)
 * A save time t_s belongs to the accepted step with t_k < t_s <= t_k + h;
 * its fraction th = (t_s - t_k) / h is taken in double, capped at 1, and is
 * exactly 1 when t_s is the step's end (then the save is y_{k+1}).  The
 * fraction belongs to the mesh: it is recorded once and, like the step
 * sizes, carries no derivative. */

/* Fraction of the step [t, t_end] of size h at which ts lies. */
inline double step_fraction(double ts, double t, double t_end, double h) {
  if (ts >= t_end) return 1.0;
  const double th = (ts - t) / h;
  return th < 1.0 ? th : 1.0;
}

/* Hermite basis at th: w = {H00, H01, H10, H11}. */
template <class S, bool F>
void hermite_weights(S th, S *w) {
  const S u = S(1.0) - th;
  const S u2 = u * u, t2 = th * th;
  w[0] = u2 * mac<F>(S(2.0), th, S(1.0));
  w[1] = t2 * mac<F>(S(-2.0), th, S(3.0));
  w[2] = th * u2;
  w[3] = -(t2 * u);
}

/* Interpolated state at fraction th of the step from yk to yk1 of size h:
 * out = h (H11 f(yk1) + H10 f(yk)) + (H01 yk1 + H00 yk), each sum a chain as
 * written.  V is the value type (a real or a dual number), S the real type of
 * th. */
template <class V, class S, bool F>
void dense_value(int kind, int d, S th, V h, const V *yk, const V *yk1, const V *p, V *out) {
  S w[4];
  hermite_weights<S, F>(th, w);
  const V wv[4] = {V(w[0]), V(w[1]), V(w[2]), V(w[3])};
  V f0[MAXD], f1[MAXD];
  rhs_f<V, F>(kind, d, yk, p, f0);
  rhs_f<V, F>(kind, d, yk1, p, f1);
  for (int c = 0; c < d; ++c) {
    const V sl = mac<F>(wv[3], f1[c], wv[2] * f0[c]);
    out[c] = mac<F>(h, sl, mac<F>(wv[1], yk1[c], wv[0] * yk[c]));
  }
}

/* ------------------------------------------------------------------ */
/* Record (adaptive solve logging accepted steps)                      */
/* ------------------------------------------------------------------ */

template <class T>
struct LaneOut {
  T *h;            /* [max_steps] or null */
  int32_t *nsteps;
  int32_t *sidx;   /* [S] */
  T *theta;        /* [S] step fraction of each save, or null */
  int32_t *status;
  T *ysave;        /* [S][d] or null */
  int32_t *natt;   /* or null */
};

/* One adaptive integration.  Steps are clipped to land exactly on every save
 * time and on t1 (with dense output only on t1, and each save is read from
 * the interpolant of the accepted step that contains it); t accumulates in
 * double.  Controller: accept iff E <= 1;
 * h_next = h_used * clamp(safety E^(-1/(q+1)), fac_min, fac_max), no growth on
 * the step after a reject, fac_max when E == 0, fac_min on a non-finite E.
 * Stop times are the save times followed by t1 when the last save is earlier
 * (with no save times, t1 is the one save slot). */
template <class T, bool F>
void record_lane(const orc_problem *P, const Opts &o, const T *u0, const T *p,
                 const LaneOut<T> &out) {
  const int d = P->dim, kind = P->rhs;
  const RosTab *rt = ros_tab(P->method);
  const bool ros = P->method == M_ROS2 || rt;
  const Tableau &tb = (P->method == M_DOPRI5) ? DOPRI5 : TSIT5;
  const bool rk78 = P->method == M_RKF78;
  const int qerr = P->method == M_ROS2 ? 1 : rt ? rt->err_order
                 : rk78 ? RK78_ERR_ORDER : tb.err_order;
  const int qord = P->method == M_ROS2 ? 2 : rt ? rt->order
                 : rk78 ? RK78_ORDER : tb.order;
  const T atol = T(P->atol), rtol = T(P->rtol);
  const T expo = T(-1.0) / T(qerr + 1);
  const T safety = T(o.safety), fmin = T(o.fac_min), fmax = T(o.fac_max);
  const int n_stops = o.S + ((o.saves && o.saves[o.S - 1] < P->t1) ? 1 : 0);
  const bool dense = P->dense != 0;

  T y[MAXD], ynew[MAXD], err[MAXD];
  T Y[7][MAXD], K[7][MAXD];
  for (int c = 0; c < d; ++c) y[c] = u0[c];
  for (int s = 0; s < o.S; ++s) {
    out.sidx[s] = -1;
    if (out.theta) out.theta[s] = T(NAN);
    if (out.ysave)
      for (int c = 0; c < d; ++c) out.ysave[s * d + c] = T(NAN);
  }
  int nacc = 0, natt = 0, st = S_OK;
  bool finite = true;
  for (int c = 0; c < d; ++c) finite = finite && fin(y[c]);
  for (int q = 0; q < P->n_params; ++q) finite = finite && fin(p[q]);
  if (!finite) {
    st = S_NONFINITE;
  } else {
    rhs_f<T, F>(kind, d, y, p, K[0]);
    T h = P->dt0 > 0 ? T(P->dt0) : initial_step<T, F>(kind, d, y, K[0], p, atol, rtol, qord);
    double t = P->t0;
    int j = 0;  /* next stop */
    bool after_reject = false;
    for (;;) {
      const double t_stop = (!dense && o.saves && j < o.S) ? o.saves[j] : P->t1;
      const T rem = T(t_stop - t);
      const bool land = !(h < rem);
      const T hs = land ? rem : h;
      if (nacc >= P->max_steps) { st = S_MAX_STEPS; break; }
      if (natt >= o.max_attempts) { st = S_MAX_ATTEMPTS; break; }
      if (!(hs > T(0.0)) || t + double(hs) == t) { st = S_DT_UNDERFLOW; break; }
      ++natt;
      if (P->method == M_ROS2) {
        Ros2Step<T> rs;
        ros2_forward<T, F>(kind, d, y, p, hs, rs);
        for (int c = 0; c < d; ++c) { ynew[c] = rs.ynew[c]; err[c] = rs.err[c]; }
      } else if (rt) {
        RodasStep<T> rs;
        rodas_forward<T, F>(*rt, kind, d, y, p, hs, rs);
        for (int c = 0; c < d; ++c) { ynew[c] = rs.ynew[c]; err[c] = rs.err[c]; }
      } else if (rk78) {
        rk78_attempt<T, F>(kind, d, y, p, hs, ynew, err);
      } else {
        erk_stages<T, F>(tb, kind, d, y, p, hs, 6, true, Y, K);
        const T *Kp[7];
        for (int i = 0; i < 7; ++i) Kp[i] = K[i];
        for (int c = 0; c < d; ++c) {
          ynew[c] = Y[6][c];
          err[c] = hs * chain<T, F>(7, tb.e, Kp, c);
        }
      }
      const T E = err_norm<T, F>(d, err, y, ynew, atol, rtol);
      if (E <= T(1.0)) {
        const double t_new = land ? t_stop : t + double(hs);
        if (out.h) out.h[nacc] = hs;
        ++nacc;
        if (dense) /* save times inside this step */
          for (; o.saves && j < o.S && o.saves[j] <= t_new; ++j) {
            const T th = T(step_fraction(o.saves[j], t, t_new, double(hs)));
            out.sidx[j] = nacc;
            if (out.theta) out.theta[j] = th;
            if (out.ysave) dense_value<T, T, F>(kind, d, th, hs, y, ynew, p, &out.ysave[j * d]);
          }
        for (int c = 0; c < d; ++c) y[c] = ynew[c];
        if (!ros && !rk78)
          for (int c = 0; c < d; ++c) K[0][c] = K[6][c];  /* first same as last */
        t = t_new;
        T fac = (E == T(0.0)) ? fmax
                              : std::min(fmax, std::max(fmin, safety * ctrl_pow<T, F>(E, expo)));
        if (after_reject) fac = std::min(fac, T(1.0));
        h = hs * fac;
        after_reject = false;
        if (land && dense) {
          if (!o.saves) { /* the final state is the one save */
            out.sidx[0] = nacc;
            if (out.theta) out.theta[0] = T(1.0);
            if (out.ysave)
              for (int c = 0; c < d; ++c) out.ysave[c] = y[c];
          }
          break;
        }
        if (land) {
          if (j < o.S) {
            out.sidx[j] = nacc;
            if (out.theta) out.theta[j] = T(1.0);
            if (out.ysave)
              for (int c = 0; c < d; ++c) out.ysave[j * d + c] = y[c];
          }
          if (++j == n_stops) break;
        }
      } else {
        const T fac = fin(E) ? std::max(fmin, safety * ctrl_pow<T, F>(E, expo)) : fmin;
        h = hs * fac;
        after_reject = true;
      }
    }
  }
  if (out.h)
    for (int k = nacc; k < P->max_steps; ++k) out.h[k] = T(0.0);
  *out.nsteps = nacc;
  *out.status = st;
  if (out.natt) *out.natt = natt;
}

/* ------------------------------------------------------------------ */
/* Replay, loss, adjoint                                               */
/* ------------------------------------------------------------------ */

template <class T, bool F>
inline void one_step(const orc_problem *P, T *y, const T *p, T h) {
  if (P->method == M_ROS2) ros2_step<T, F>(P->rhs, P->dim, y, p, h);
  else if (ros_tab(P->method)) rodas_step<T, F>(*ros_tab(P->method), P->rhs, P->dim, y, p, h);
  else if (P->method == M_RKF78) rk78_step<T, F>(P->rhs, P->dim, y, p, h);
  else erk_step<T, F>(P->method == M_DOPRI5 ? DOPRI5 : TSIT5, P->rhs, P->dim, y, p, h);
}

template <class T, bool F>
inline void one_step_adjoint(const orc_problem *P, const T *y, const T *p, T h, T *lam, T *gp,
                             T *gpc = nullptr) {
  if (P->method == M_ROS2) ros2_step_adjoint<T, F>(P->rhs, P->dim, y, p, h, lam, gp);
  else if (ros_tab(P->method))
    rodas_step_adjoint<T, F>(*ros_tab(P->method), P->rhs, P->dim, y, p, h, lam, gp);
  else if (P->method == M_RKF78)
    rk78_step_adjoint<T, F>(P->rhs, P->dim, y, p, h, lam, gp);
  else erk_step_adjoint<T, F>(P->method == M_DOPRI5 ? DOPRI5 : TSIT5, P->rhs, P->dim, y, p,
                              h, lam, gp, gpc);
}

/* Sum of v[0..d) (d <= 64, zero beyond) by pairwise sums at offsets 32, 16,
 * ..., 1: w[c] = v[c] + v[c ^ off] for every c, then the entry at 0. */
template <class T>
T pairwise64(const T *v, int d) {
  T a[64], b[64];
  for (int c = 0; c < 64; ++c) a[c] = c < d ? v[c] : T(0.0);
  for (int off = 32; off >= 1; off >>= 1) {
    for (int c = 0; c < 64; ++c) b[c] = a[c] + a[c ^ off];
    for (int c = 0; c < 64; ++c) a[c] = b[c];
  }
  return a[0];
}

/* Fixed-step replay of a recorded mesh: writes y at every save index (with
 * dense output, theta != null, the interpolant of step sidx - 1 at the
 * save's fraction; index 0 is the initial state in both modes). */
template <class T, bool F>
void replay_lane(const orc_problem *P, int S, const T *u0, const T *p, const T *h, int N,
                 const int32_t *sidx, const T *theta, T *ysave, T *yfinal) {
  const int d = P->dim;
  T y[MAXD], yprev[MAXD];
  for (int c = 0; c < d; ++c) y[c] = u0[c];
  for (int s = 0; s < S; ++s)
    if (sidx[s] == 0)
      for (int c = 0; c < d; ++c) ysave[s * d + c] = y[c];
  for (int k = 0; k < N; ++k) {
    for (int c = 0; c < d; ++c) yprev[c] = y[c];
    one_step<T, F>(P, y, p, h[k]);
    for (int s = 0; s < S; ++s)
      if (sidx[s] == k + 1) {
        if (theta)
          dense_value<T, T, F>(P->rhs, d, theta[s], h[k], yprev, y, p, &ysave[s * d]);
        else
          for (int c = 0; c < d; ++c) ysave[s * d + c] = y[c];
      }
  }
  for (int s = 0; s < S; ++s)
    if (sidx[s] < 0 || sidx[s] > N)
      for (int c = 0; c < d; ++c) ysave[s * d + c] = T(NAN);
  if (yfinal)
    for (int c = 0; c < d; ++c) yfinal[c] = y[c];
}

/* Loss term of one save slot (MSE / cotangent kinds), accumulated into ss. */
template <class T, bool F>
void save_loss(int kind, int d, const T *y, const T *aux, T &ss, bool &first) {
  for (int c = 0; c < d; ++c) {
    if (kind == L_MSE_SAVE) {
      const T r = y[c] - aux[c];
      ss = first ? r * r : mac<F>(r, r, ss);
    } else {
      ss = first ? aux[c] * y[c] : mac<F>(aux[c], y[c], ss);
    }
    first = false;
  }
}

/* Seed of one save slot added to the adjoint: 2 scale (y - target) for MSE,
 * scale * cotangent otherwise. */
template <class T, bool F>
void save_seed(int kind, int d, const T *y, const T *aux, double scale, T *lam) {
  for (int c = 0; c < d; ++c) {
    if (kind == L_MSE_SAVE) lam[c] = mac<F>(T(2.0 * scale), y[c] - aux[c], lam[c]);
    else lam[c] = mac<F>(T(scale), aux[c], lam[c]);
  }
}

/* Reverse of one dense save inside the step from yk to yk1 (size h, fraction
 * th), given the save's seed sb = dL/dy(t_s) (save_seed from zero):
 *   lam (dL/dy_{k+1}) += H01 sb + J(yk1)^T v1,   v1 = (h H11) sb
 *   mu  (dL/dy_k part) += H00 sb + J(yk)^T v0,    v0 = (h H10) sb
 *   g += J_p(yk1)^T v1, then g += J_p(yk)^T v0
 * (with the Lorenz-96 split, df_c/dF = 1: gpc[c] += v1[c], then v0[c]). */
template <class T, bool F>
void dense_seed(const orc_problem *P, T th, T h, const T *yk, const T *yk1, const T *p,
                int loss_kind, const T *aux, double scale, T *lam, T *mu, T *g, T *gpc) {
  const int d = P->dim, kind = P->rhs;
  T ys[MAXD], sb[MAXD], v0[MAXD], v1[MAXD], w0[MAXD], w1[MAXD], w[4];
  dense_value<T, T, F>(kind, d, th, h, yk, yk1, p, ys);
  for (int c = 0; c < d; ++c) sb[c] = T(0.0);
  save_seed<T, F>(loss_kind, d, ys, aux, scale, sb);
  hermite_weights<T, F>(th, w);
  const T c1 = h * w[3], c0 = h * w[2];
  for (int c = 0; c < d; ++c) {
    v1[c] = c1 * sb[c];
    v0[c] = c0 * sb[c];
  }
  rhs_vjp_y<T, F>(kind, d, yk1, p, v1, w1);
  rhs_vjp_y<T, F>(kind, d, yk, p, v0, w0);
  for (int c = 0; c < d; ++c) {
    lam[c] = mac<F>(w[1], sb[c], lam[c]) + w1[c];
    mu[c] = mac<F>(w[0], sb[c], mu[c]) + w0[c];
  }
  if (gpc) {
    for (int c = 0; c < d; ++c) gpc[c] = gpc[c] + v1[c];
    for (int c = 0; c < d; ++c) gpc[c] = gpc[c] + v0[c];
  } else {
    rhs_vjp_p_acc<T, F>(kind, d, yk1, p, v1, g);
    rhs_vjp_p_acc<T, F>(kind, d, yk, p, v0, g);
  }
}

/* Replay + reverse sweep for one lane.  Loss kinds:
 *  SUMSQ_FINAL: L = scale sum_c y_N[c]^2
 *  MSE_SAVE:    L = scale sum_s sum_c (y_{idx_s}[c] - target[s][c])^2
 *  COTANGENT:   L = scale sum_s sum_c cot[s][c] y_{idx_s}[c]
 * The oracle keeps every forward state y_k, then runs the reverse sweep and
 * adds each save's seed once the adjoint has reached that save's index; with
 * dense output (theta != null) y_{idx_s} stands for the interpolated save
 * and its seed enters through dense_seed at step idx_s - 1. */
template <class T, bool F>
void replay_grad_lane(const orc_problem *P, int S, const T *u0, const T *p, const T *h, int N,
                      const int32_t *sidx, const T *theta, int status, int loss_kind,
                      const T *aux, double scale, T *loss, T *gu0, T *gp,
                      T *ybuf /*[(N+1)*d]*/) {
  const int d = P->dim, Pn = P->n_params;
  const bool dense = theta != nullptr;
  if (status != S_OK) {
    *loss = T(NAN);
    for (int c = 0; c < d; ++c) gu0[c] = T(NAN);
    for (int q = 0; q < Pn; ++q) gp[q] = T(NAN);
    return;
  }
  for (int c = 0; c < d; ++c) ybuf[c] = u0[c];
  for (int k = 0; k < N; ++k) {
    for (int c = 0; c < d; ++c) ybuf[(k + 1) * d + c] = ybuf[k * d + c];
    one_step<T, F>(P, &ybuf[(k + 1) * d], p, h[k]);
  }
  T lam[MAXD], g[MAXP];
  for (int c = 0; c < d; ++c) lam[c] = T(0.0);
  for (int q = 0; q < Pn; ++q) g[q] = T(0.0);
  T ss = T(0.0);
  const T *yN = &ybuf[N * d];
  if (loss_kind == L_SUMSQ_FINAL) {
    for (int c = 0; c < d; ++c) ss = (c == 0) ? yN[c] * yN[c] : mac<F>(yN[c], yN[c], ss);
    for (int c = 0; c < d; ++c) lam[c] = T(2.0 * scale) * yN[c];
  } else {
    bool first = true;
    for (int s = 0; s < S; ++s) {
      const int ix = sidx[s];
      if (dense && ix > 0) {
        T ys[MAXD];
        dense_value<T, T, F>(P->rhs, d, theta[s], h[ix - 1], &ybuf[(ix - 1) * d],
                             &ybuf[ix * d], p, ys);
        save_loss<T, F>(loss_kind, d, ys, &aux[s * d], ss, first);
      } else {
        save_loss<T, F>(loss_kind, d, &ybuf[ix * d], &aux[s * d], ss, first);
      }
    }
  }
  *loss = T(scale) * ss;
  int s_hi = S - 1;  /* highest save slot not yet seeded */
  if (loss_kind != L_SUMSQ_FINAL && !dense)
    for (; s_hi >= 0 && sidx[s_hi] == N; --s_hi)
      save_seed<T, F>(loss_kind, d, yN, &aux[s_hi * d], scale, lam);
  /* Fused mode follows the kernels' schedule also in its association order:
   * the Lorenz-96 F-gradient (a sum over components, stages and steps) is kept
   * per component over the whole sweep and the components are combined at
   * the end by pairwise sums.  Plain mode adds every term into one sum. */
  T gpc[MAXD];
  for (int c = 0; c < d; ++c) gpc[c] = T(0.0);
  T *split = (F && P->rhs == R_LORENZ96 && P->method != M_ROS2) ? gpc : nullptr;
  for (int k = N - 1; k >= 0; --k) {
    /* dense output: every save inside step k, the last first, seeds lam
     * (here dL/dy_{k+1}) now and mu, the part of dL/dy_k that bypasses the
     * step, which joins lam after the step's adjoint */
    T mu[MAXD];
    bool has_mu = false;
    if (dense && loss_kind != L_SUMSQ_FINAL)
      for (; s_hi >= 0 && sidx[s_hi] == k + 1; --s_hi) {
        if (!has_mu)
          for (int c = 0; c < d; ++c) mu[c] = T(0.0);
        has_mu = true;
        dense_seed<T, F>(P, theta[s_hi], h[k], &ybuf[k * d], &ybuf[(k + 1) * d], p, loss_kind,
                         &aux[s_hi * d], scale, lam, mu, g, split);
      }
    one_step_adjoint<T, F>(P, &ybuf[k * d], p, h[k], lam, g, split);
    if (has_mu)
      for (int c = 0; c < d; ++c) lam[c] = lam[c] + mu[c];
    if (loss_kind != L_SUMSQ_FINAL && (!dense || k == 0))
      for (; s_hi >= 0 && sidx[s_hi] == k; --s_hi)
        save_seed<T, F>(loss_kind, d, &ybuf[k * d], &aux[s_hi * d], scale, lam);
  }
  if (split) g[0] = pairwise64(gpc, d);
  for (int c = 0; c < d; ++c) gu0[c] = lam[c];
  for (int q = 0; q < Pn; ++q) gp[q] = g[q];
}

/* Re-evaluate the embedded error of every step of a given mesh along the
 * replayed states (GPU-recorded mesh check): largest E per lane. */
template <class T, bool F>
T mesh_max_err_lane(const orc_problem *P, const T *u0, const T *p, const T *h, int N) {
  const int d = P->dim, kind = P->rhs;
  const Tableau &tb = (P->method == M_DOPRI5) ? DOPRI5 : TSIT5;
  const T atol = T(P->atol), rtol = T(P->rtol);
  T y[MAXD], ynew[MAXD], err[MAXD], Y[7][MAXD], K[7][MAXD];
  for (int c = 0; c < d; ++c) y[c] = u0[c];
  T worst = T(0.0);
  for (int k = 0; k < N; ++k) {
    if (P->method == M_ROS2) {
      Ros2Step<T> rs;
      ros2_forward<T, F>(kind, d, y, p, h[k], rs);
      for (int c = 0; c < d; ++c) { ynew[c] = rs.ynew[c]; err[c] = rs.err[c]; }
    } else if (ros_tab(P->method)) {
      RodasStep<T> rs;
      rodas_forward<T, F>(*ros_tab(P->method), kind, d, y, p, h[k], rs);
      for (int c = 0; c < d; ++c) { ynew[c] = rs.ynew[c]; err[c] = rs.err[c]; }
    } else if (P->method == M_RKF78) {
      rk78_attempt<T, F>(kind, d, y, p, h[k], ynew, err);
    } else {
      rhs_f<T, F>(kind, d, y, p, K[0]);
      erk_stages<T, F>(tb, kind, d, y, p, h[k], 6, true, Y, K);
      const T *Kp[7];
      for (int j = 0; j < 7; ++j) Kp[j] = K[j];
      for (int c = 0; c < d; ++c) {
        ynew[c] = Y[6][c];
        err[c] = h[k] * chain<T, F>(7, tb.e, Kp, c);
      }
    }
    const T E = err_norm<T, F>(d, err, y, ynew, atol, rtol);
    if (!(E <= worst)) worst = E;
    for (int c = 0; c < d; ++c) y[c] = ynew[c];
  }
  return worst;
}

int set_threads(int nthreads) {
  if (nthreads > 0) omp_set_num_threads(nthreads);
  return omp_get_max_threads();
}

template <class T>
int record_all(const orc_problem *P, int64_t n, const T *u0, const T *p, int fused, T *h,
               int32_t *nsteps, int32_t *sidx, T *theta, int32_t *status, T *ysave,
               int32_t *natt, int nthreads) {
  const int rc = validate(P);
  if (rc) return rc;
  if (n < 0 || (n > 0 && (!u0 || !p || !nsteps || !sidx || !status))) return E_INVAL;
  const Opts o = make_opts(P);
  const int d = P->dim, Pn = P->n_params;
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t i = 0; i < n; ++i) {
    LaneOut<T> out;
    out.h = h ? h + i * P->max_steps : nullptr;
    out.nsteps = nsteps + i;
    out.sidx = sidx + i * o.S;
    out.theta = theta ? theta + i * o.S : nullptr;
    out.status = status + i;
    out.ysave = ysave ? ysave + i * o.S * d : nullptr;
    out.natt = natt ? natt + i : nullptr;
    if (fused) record_lane<T, true>(P, o, u0 + i * d, p + i * Pn, out);
    else record_lane<T, false>(P, o, u0 + i * d, p + i * Pn, out);
  }
  return E_OK;
}

template <class T>
int replay_all(const orc_problem *P, int64_t n, const T *u0, const T *p, int fused, const T *h,
               const int32_t *nsteps, const int32_t *sidx, const T *theta, T *ysave, T *yfinal,
               int nthreads) {
  const int rc = validate(P);
  if (rc) return rc;
  if (n < 0 || (n > 0 && (!u0 || !p || !h || !nsteps || !sidx || !ysave))) return E_INVAL;
  if (P->dense && !theta) return E_INVAL;
  const Opts o = make_opts(P);
  const int d = P->dim, Pn = P->n_params;
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t i = 0; i < n; ++i) {
    const int N = std::min(std::max(nsteps[i], 0), P->max_steps);
    T *yf = yfinal ? yfinal + i * d : nullptr;
    const T *th = P->dense ? theta + i * o.S : nullptr;
    if (fused)
      replay_lane<T, true>(P, o.S, u0 + i * d, p + i * Pn, h + i * P->max_steps, N,
                           sidx + i * o.S, th, ysave + i * o.S * d, yf);
    else
      replay_lane<T, false>(P, o.S, u0 + i * d, p + i * Pn, h + i * P->max_steps, N,
                            sidx + i * o.S, th, ysave + i * o.S * d, yf);
  }
  return E_OK;
}

template <class T>
int replay_grad_all(const orc_problem *P, int64_t n, const T *u0, const T *p, int fused,
                    const T *h, const int32_t *nsteps, const int32_t *sidx, const T *theta,
                    const int32_t *status, int loss_kind, const T *aux, double scale, T *loss,
                    T *gu0, T *gp, int nthreads) {
  const int rc = validate(P);
  if (rc) return rc;
  if (P->dense && !theta) return E_INVAL;
  if (loss_kind < 0 || loss_kind > 2) return E_INVAL;
  if (loss_kind != L_SUMSQ_FINAL && !aux) return E_INVAL;
  if (n < 0 || (n > 0 && (!u0 || !p || !h || !nsteps || !sidx || !status || !loss || !gu0 || !gp)))
    return E_INVAL;
  const Opts o = make_opts(P);
  const int d = P->dim, Pn = P->n_params;
  set_threads(nthreads);
#pragma omp parallel
  {
    T *ybuf = new T[(size_t)(P->max_steps + 1) * d];
#pragma omp for schedule(dynamic, 64)
    for (int64_t i = 0; i < n; ++i) {
      const int N = std::min(std::max(nsteps[i], 0), P->max_steps);
      const T *ax = aux ? aux + i * o.S * d : nullptr;
      const T *th = P->dense ? theta + i * o.S : nullptr;
      if (fused)
        replay_grad_lane<T, true>(P, o.S, u0 + i * d, p + i * Pn, h + i * P->max_steps, N,
                                  sidx + i * o.S, th, status[i], loss_kind, ax, scale, loss + i,
                                  gu0 + i * d, gp + i * Pn, ybuf);
      else
        replay_grad_lane<T, false>(P, o.S, u0 + i * d, p + i * Pn, h + i * P->max_steps, N,
                                   sidx + i * o.S, th, status[i], loss_kind, ax, scale,
                                   loss + i, gu0 + i * d, gp + i * Pn, ybuf);
    }
    delete[] ybuf;
  }
  return E_OK;
}

/* Forward-mode sensitivities of the replay (mesh fixed): for every direction
 * q of the d + P unit directions (u0 components, then parameters) the replay
 * runs in dual numbers (DualF with fused = 1, Dual with plain rounding),
 * giving sens[i][s][c][q] = d y(save s)[c] / d theta_q, and the loss gradient
 * by the chain rule, g_q = sum over seeds of seed . dy/dtheta_q with the
 * terms in save-then-component order (first product, then multiply-adds):
 *   final-state loss: seed = (2 scale) y_N  (the final state only)
 *   MSE:              seed = (2 scale) (y_s - aux_s)
 *   cotangent:        seed = scale aux_s.
 * A failed lane gets NaN. */
template <class D, bool F>
void sens_lane(const orc_problem *P, int S, const double *u0, const double *p, const double *h,
               int N, const int32_t *si, const double *theta, int status, int loss_kind,
               const double *aux, double scale, double *sens, double *loss, double *gu0,
               double *gp) {
  const int d = P->dim, Pn = P->n_params, Q = d + Pn;
  if (status != S_OK) {
    for (int k = 0; k < S * d * Q; ++k) sens[k] = NAN;
    *loss = NAN;
    for (int c = 0; c < d; ++c) gu0[c] = NAN;
    for (int q = 0; q < Pn; ++q) gp[q] = NAN;
    return;
  }
  double g[MAXD + MAXP];
  for (int q = 0; q < Q; ++q) {
    D yv[MAXD], pv[MAXP];
    for (int c = 0; c < d; ++c) yv[c] = D(u0[c], q == c ? 1.0 : 0.0);
    for (int r = 0; r < Pn; ++r) pv[r] = D(p[r], q == d + r ? 1.0 : 0.0);
    std::vector<D> ysl((size_t)S * d, D(NAN));
    for (int s = 0; s < S; ++s)
      if (si[s] == 0)
        for (int c = 0; c < d; ++c) ysl[s * d + c] = yv[c];
    for (int k = 0; k < N; ++k) {
      D yprev[MAXD];
      for (int c = 0; c < d; ++c) yprev[c] = yv[c];
      one_step<D, F>(P, yv, pv, D(h[k]));
      for (int s = 0; s < S; ++s)
        if (si[s] == k + 1) {
          if (theta)
            dense_value<D, double, F>(P->rhs, d, theta[s], D(h[k]), yprev, yv, pv, &ysl[s * d]);
          else
            for (int c = 0; c < d; ++c) ysl[s * d + c] = yv[c];
        }
    }
    for (int s = 0; s < S; ++s)
      for (int c = 0; c < d; ++c) sens[(s * d + c) * Q + q] = ysl[s * d + c].d;
    double acc = 0.0;
    bool first = true;
    auto add = [&](double seed, double t) {
      acc = first ? seed * t : mac<F>(seed, t, acc);
      first = false;
    };
    if (loss_kind == L_SUMSQ_FINAL) {
      for (int c = 0; c < d; ++c) add((2.0 * scale) * yv[c].v, yv[c].d);
    } else {
      for (int s = 0; s < S; ++s)
        for (int c = 0; c < d; ++c) {
          const double y = ysl[s * d + c].v, a = aux[s * d + c];
          add(loss_kind == L_MSE_SAVE ? (2.0 * scale) * (y - a) : scale * a, ysl[s * d + c].d);
        }
    }
    g[q] = acc;
    if (q == 0) {  /* the loss of the replayed states */
      double ss = 0.0;
      bool f1 = true;
      if (loss_kind == L_SUMSQ_FINAL) {
        for (int c = 0; c < d; ++c) {
          ss = f1 ? yv[c].v * yv[c].v : mac<F>(yv[c].v, yv[c].v, ss);
          f1 = false;
        }
      } else {
        for (int s = 0; s < S; ++s)
          for (int c = 0; c < d; ++c) {
            const double y = ysl[s * d + c].v, a = aux[s * d + c];
            if (loss_kind == L_MSE_SAVE) {
              const double r = y - a;
              ss = f1 ? r * r : mac<F>(r, r, ss);
            } else {
              ss = f1 ? a * y : mac<F>(a, y, ss);
            }
            f1 = false;
          }
      }
      *loss = scale * ss;
    }
  }
  for (int c = 0; c < d; ++c) gu0[c] = g[c];
  for (int r = 0; r < Pn; ++r) gp[r] = g[d + r];
}

}  // namespace

/* ------------------------------------------------------------------ */
/* C entry points (ctypes)                                             */
/* ------------------------------------------------------------------ */
extern "C" {

/* Tableau of an explicit method: c[7], a[7*7] row-major, b[7], e[7],
 * info[2] = {order, embedded order}. */
int orc_tableau(int method, double *c, double *a, double *b, double *e, int32_t *info) {
  if (method != M_TSIT5 && method != M_DOPRI5) return E_INVAL;
  const Tableau &t = method == M_TSIT5 ? TSIT5 : DOPRI5;
  for (int i = 0; i < 7; ++i) {
    c[i] = t.c[i]; b[i] = t.b[i]; e[i] = t.e[i];
    for (int j = 0; j < 7; ++j) a[i * 7 + j] = t.a[i][j];
  }
  info[0] = t.order; info[1] = t.err_order;
  return E_OK;
}

double orc_ros2_gamma(void) { return ROS2_GAMMA; }

/* The Fehlberg 7(8) coefficients as typed: a[13][13], b (7th order), e. */
int orc_rk78_tableau(double *a, double *b, double *e, int32_t *info) {
  for (int i = 0; i < 13; ++i) {
    b[i] = RK78.b[i]; e[i] = RK78.e[i];
    for (int j = 0; j < 13; ++j) a[i * 13 + j] = RK78.a[i][j];
  }
  info[0] = RK78_ORDER; info[1] = RK78_ERR_ORDER;
  return E_OK;
}

/* The caller's right-hand side from a plugin (see user_types.h): f on reals
 * (double, float) and on dual numbers (plain and fused, double and float). */
int orc_set_user_rhs(int32_t dim, int32_t n_params, void *f64, void *f32, void *dp64, void *df64,
                     void *dp32, void *df32) {
  if (dim < 1 || dim > MAXD || n_params < 1 || n_params > MAXP) return E_INVAL;
  if (!f64 || !f32 || !dp64 || !df64 || !dp32 || !df32) return E_INVAL;
  g_user.dim = dim;
  g_user.np = n_params;
  g_user.f64 = (decltype(g_user.f64))f64;
  g_user.f32 = (decltype(g_user.f32))f32;
  g_user.dp64 = (decltype(g_user.dp64))dp64;
  g_user.df64 = (decltype(g_user.df64))df64;
  g_user.dp32 = (decltype(g_user.dp32))dp32;
  g_user.df32 = (decltype(g_user.df32))df32;
  return E_OK;
}

int orc_max_threads(int nthreads) { return set_threads(nthreads); }

/* theta ([n][S] step fraction of each save) is written by the record when
 * not null, and read by the replays when the problem asks for dense output. */
int orc_record_f64(const orc_problem *P, int64_t n, const double *u0, const double *p,
                   int32_t fused, double *h, int32_t *nsteps, int32_t *sidx, double *theta,
                   int32_t *status, double *ysave, int32_t *natt, int32_t nthreads) {
  return record_all<double>(P, n, u0, p, fused, h, nsteps, sidx, theta, status, ysave, natt,
                            nthreads);
}
int orc_record_f32(const orc_problem *P, int64_t n, const float *u0, const float *p,
                   int32_t fused, float *h, int32_t *nsteps, int32_t *sidx, float *theta,
                   int32_t *status, float *ysave, int32_t *natt, int32_t nthreads) {
  return record_all<float>(P, n, u0, p, fused, h, nsteps, sidx, theta, status, ysave, natt,
                           nthreads);
}

int orc_replay_f64(const orc_problem *P, int64_t n, const double *u0, const double *p,
                   int32_t fused, const double *h, const int32_t *nsteps, const int32_t *sidx,
                   const double *theta, double *ysave, double *yfinal, int32_t nthreads) {
  return replay_all<double>(P, n, u0, p, fused, h, nsteps, sidx, theta, ysave, yfinal,
                            nthreads);
}
int orc_replay_f32(const orc_problem *P, int64_t n, const float *u0, const float *p,
                   int32_t fused, const float *h, const int32_t *nsteps, const int32_t *sidx,
                   const float *theta, float *ysave, float *yfinal, int32_t nthreads) {
  return replay_all<float>(P, n, u0, p, fused, h, nsteps, sidx, theta, ysave, yfinal, nthreads);
}

int orc_replay_grad_f64(const orc_problem *P, int64_t n, const double *u0, const double *p,
                        int32_t fused, const double *h, const int32_t *nsteps,
                        const int32_t *sidx, const double *theta, const int32_t *status,
                        int32_t loss_kind, const double *aux, double scale, double *loss,
                        double *gu0, double *gp, int32_t nthreads) {
  return replay_grad_all<double>(P, n, u0, p, fused, h, nsteps, sidx, theta, status, loss_kind,
                                 aux, scale, loss, gu0, gp, nthreads);
}
int orc_replay_grad_f32(const orc_problem *P, int64_t n, const float *u0, const float *p,
                        int32_t fused, const float *h, const int32_t *nsteps,
                        const int32_t *sidx, const float *theta, const int32_t *status,
                        int32_t loss_kind, const float *aux, double scale, float *loss,
                        float *gu0, float *gp, int32_t nthreads) {
  return replay_grad_all<float>(P, n, u0, p, fused, h, nsteps, sidx, theta, status, loss_kind,
                                aux, scale, loss, gu0, gp, nthreads);
}

int orc_replay_sens_f64(const orc_problem *P, int64_t n, const double *u0, const double *p,
                        int32_t fused, const double *h, const int32_t *nsteps,
                        const int32_t *sidx, const double *theta, const int32_t *status,
                        int32_t loss_kind, const double *aux, double scale, double *sens,
                        double *loss, double *gu0, double *gp) {
  const int rc = validate(P);
  if (rc) return rc;
  if (P->dense && !theta) return E_INVAL;
  if (loss_kind < 0 || loss_kind > 2 || (loss_kind != L_SUMSQ_FINAL && !aux)) return E_INVAL;
  const Opts o = make_opts(P);
  const int d = P->dim, Pn = P->n_params, S = o.S, Q = d + Pn;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t i = 0; i < n; ++i) {
    const int N = std::min(std::max(nsteps[i], 0), P->max_steps);
    const double *ax = aux ? aux + i * S * d : nullptr;
    const double *th = P->dense ? theta + i * S : nullptr;
    if (fused)
      sens_lane<DualF, true>(P, S, u0 + i * d, p + i * Pn, h + i * P->max_steps, N,
                             sidx + i * S, th, status[i], loss_kind, ax, scale,
                             sens + i * S * d * Q, loss + i, gu0 + i * d, gp + i * Pn);
    else
      sens_lane<Dual, false>(P, S, u0 + i * d, p + i * Pn, h + i * P->max_steps, N,
                             sidx + i * S, th, status[i], loss_kind, ax, scale,
                             sens + i * S * d * Q, loss + i, gu0 + i * d, gp + i * Pn);
  }
  return E_OK;
}

/* Forward-mode derivative of the replayed loss along (du0, dp): one dual
 * number per value, plain rounding.  Outputs the loss and its directional
 * derivative per lane, and the saved states with their tangents. */
int orc_replay_jvp_f64(const orc_problem *P, int64_t n, const double *u0, const double *p,
                       const double *du0, const double *dp, const double *h,
                       const int32_t *nsteps, const int32_t *sidx, const double *theta,
                       int32_t loss_kind, const double *aux, double scale, double *loss,
                       double *dloss, double *ysave, double *dysave) {
  const int rc = validate(P);
  if (rc) return rc;
  if (P->dense && !theta) return E_INVAL;
  if (loss_kind < 0 || loss_kind > 2 || (loss_kind != L_SUMSQ_FINAL && !aux)) return E_INVAL;
  const Opts o = make_opts(P);
  const int d = P->dim, Pn = P->n_params, S = o.S;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t i = 0; i < n; ++i) {
    Dual yv[MAXD], pv[MAXP], ys[16 * MAXD];
    const int N = std::min(std::max(nsteps[i], 0), P->max_steps);
    for (int c = 0; c < d; ++c) yv[c] = Dual(u0[i * d + c], du0[i * d + c]);
    for (int q = 0; q < Pn; ++q) pv[q] = Dual(p[i * Pn + q], dp[i * Pn + q]);
    Dual *ysl = (S <= 16) ? ys : new Dual[(size_t)S * d];
    for (int s = 0; s < S; ++s)
      for (int c = 0; c < d; ++c) ysl[s * d + c] = Dual(NAN);
    const int32_t *si = sidx + i * S;
    for (int s = 0; s < S; ++s)
      if (si[s] == 0)
        for (int c = 0; c < d; ++c) ysl[s * d + c] = yv[c];
    for (int k = 0; k < N; ++k) {
      Dual yprev[MAXD];
      const Dual hk(h[i * P->max_steps + k]);
      for (int c = 0; c < d; ++c) yprev[c] = yv[c];
      one_step<Dual, false>(P, yv, pv, hk);
      for (int s = 0; s < S; ++s)
        if (si[s] == k + 1) {
          if (P->dense)
            dense_value<Dual, double, false>(P->rhs, d, theta[i * S + s], hk, yprev, yv, pv,
                                             &ysl[s * d]);
          else
            for (int c = 0; c < d; ++c) ysl[s * d + c] = yv[c];
        }
    }
    Dual ss(0.0);
    bool first = true;
    if (loss_kind == L_SUMSQ_FINAL) {
      for (int c = 0; c < d; ++c) { ss = first ? yv[c] * yv[c] : yv[c] * yv[c] + ss; first = false; }
    } else {
      for (int s = 0; s < S; ++s)
        for (int c = 0; c < d; ++c) {
          const Dual a(aux[(i * S + s) * d + c]);
          const Dual y = ysl[s * d + c];
          const Dual term = (loss_kind == L_MSE_SAVE) ? (y - a) * (y - a) : a * y;
          ss = first ? term : term + ss;
          first = false;
        }
    }
    const Dual L = Dual(scale) * ss;
    loss[i] = L.v;
    dloss[i] = L.d;
    if (ysave)
      for (int s = 0; s < S; ++s)
        for (int c = 0; c < d; ++c) {
          ysave[(i * S + s) * d + c] = ysl[s * d + c].v;
          dysave[(i * S + s) * d + c] = ysl[s * d + c].d;
        }
    if (ysl != ys) delete[] ysl;
  }
  return E_OK;
}

int orc_mesh_max_err_f64(const orc_problem *P, int64_t n, const double *u0, const double *p,
                         int32_t fused, const double *h, const int32_t *nsteps,
                         double *max_err, int32_t nthreads) {
  const int rc = validate(P);
  if (rc) return rc;
  const int d = P->dim, Pn = P->n_params;
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t i = 0; i < n; ++i) {
    const int N = std::min(std::max(nsteps[i], 0), P->max_steps);
    max_err[i] = fused ? mesh_max_err_lane<double, true>(P, u0 + i * d, p + i * Pn,
                                                          h + i * P->max_steps, N)
                       : mesh_max_err_lane<double, false>(P, u0 + i * d, p + i * Pn,
                                                           h + i * P->max_steps, N);
  }
  return E_OK;
}
int orc_mesh_max_err_f32(const orc_problem *P, int64_t n, const float *u0, const float *p,
                         int32_t fused, const float *h, const int32_t *nsteps,
                         float *max_err, int32_t nthreads) {
  const int rc = validate(P);
  if (rc) return rc;
  const int d = P->dim, Pn = P->n_params;
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t i = 0; i < n; ++i) {
    const int N = std::min(std::max(nsteps[i], 0), P->max_steps);
    max_err[i] = fused ? mesh_max_err_lane<float, true>(P, u0 + i * d, p + i * Pn,
                                                         h + i * P->max_steps, N)
                       : mesh_max_err_lane<float, false>(P, u0 + i * d, p + i * Pn,
                                                          h + i * P->max_steps, N);
  }
  return E_OK;
}

/* Starting step of the record for one lane (for checks against the textbook). */
int orc_initial_step_f64(const orc_problem *P, const double *y0, const double *p, double *h0) {
  const int rc = validate(P);
  if (rc) return rc;
  double f0[MAXD];
  rhs_f<double, false>(P->rhs, P->dim, y0, p, f0);
  const int q = P->method == M_ROS2 ? 2 : ros_tab(P->method) ? ros_tab(P->method)->order
              : P->method == M_RKF78 ? RK78_ORDER : 5;
  *h0 = initial_step<double, false>(P->rhs, P->dim, y0, f0, p, P->atol, P->rtol, q);
  return E_OK;
}

/* One right-hand-side evaluation and its products (for direct checks). */
int orc_rhs_f64(int32_t kind, int32_t d, const double *y, const double *p, const double *v,
                double *f, double *wy, double *gp, double *J) {
  const int np = kind == R_LORENZ96 || kind == R_LINEAR ? 1 : kind == R_KINETICS8 ? 4 : 3;
  if (!rhs_shape_ok(kind, d, np)) return E_INVAL;
  rhs_f<double, false>(kind, d, y, p, f);
  rhs_vjp_y<double, false>(kind, d, y, p, v, wy);
  rhs_vjp_p_acc<double, false>(kind, d, y, p, v, gp);
  if (J && d <= MAXR && kind != R_LORENZ96) rhs_jac<double, false>(kind, d, y, p, J);
  return E_OK;
}

}  // extern "C"
