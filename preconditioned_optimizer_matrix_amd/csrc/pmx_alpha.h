// The on-device alpha fit of a PRISM update (shared by the Krylov kernel and
// the fused small-matrix kernel): from the Gram of the scaled Krylov blocks to
// the argmin of the sketched quartic on [lo, hi].
#pragma once

#include "pmx_kernels.h"

namespace pmx {

// ---------------------------------------------------------------- alpha fit
// Real roots of a x^2 + b x + c inside (lo, hi), ascending, in r0 (and r1);
// returns how many.  Scalars only: an indexed array here would live in
// scratch memory, whose store-then-load costs a memory round trip.
__device__ inline int quad_roots_in(double a, double b, double c, double lo, double hi,
                                    double& r0, double& r1) {
  const double scale = fmax(fabs(a), fmax(fabs(b), fabs(c)));
  if (scale == 0.0) return 0;
  if (fabs(a) <= 1e-14 * scale) {
    if (b != 0.0) {
      const double x = -c / b;
      if (x > lo && x < hi) {
        r0 = x;
        return 1;
      }
    }
    return 0;
  }
  const double disc = b * b - 4.0 * a * c;
  if (disc < 0.0) return 0;
  const double sq = sqrt(disc);
  const double q = -0.5 * (b + (b >= 0.0 ? sq : -sq));
  const double x1 = q / a;
  const double x2 = (q != 0.0) ? c / q : x1;
  const bool in1 = x1 > lo && x1 < hi;
  const bool in2 = x2 > lo && x2 < hi && x2 != x1;
  if (in1 && in2) {
    r0 = fmin(x1, x2);
    r1 = fmax(x1, x2);
    return 2;
  }
  if (in1 || in2) {
    r0 = in1 ? x1 : x2;
    return 1;
  }
  return 0;
}

// argmin over [lo, hi] of phi(a) = w0 + w1 a + w2 a^2 + w3 a^3 + w4 a^4.
// phi' is a cubic; the roots of phi'' split [lo, hi] into pieces on which
// phi' is monotone, and every sign change of phi' on a piece is refined to
// full double precision by bracketed Newton steps.  Candidates are both ends
// and those critical points, met in ascending order (lo, the pieces left to
// right, hi); the smallest phi wins, ties to the smaller alpha.
__device__ inline double argmin_quartic(const double (&w)[5], double lo, double hi) {
  auto phi = [&](double a) { return w[0] + a * (w[1] + a * (w[2] + a * (w[3] + a * w[4]))); };
  auto dphi = [&](double a) { return w[1] + a * (2.0 * w[2] + a * (3.0 * w[3] + a * 4.0 * w[4])); };
  auto d2phi = [&](double a) { return 2.0 * w[2] + a * (6.0 * w[3] + a * 12.0 * w[4]); };
  double best = lo, bv = phi(lo);
  auto consider = [&](double x) {
    const double v = phi(x);
    if (v < bv) {
      bv = v;
      best = x;
    }
  };
  auto piece = [&](double x0, double x1) {
    double f0 = dphi(x0);
    const double f1 = dphi(x1);
    if (f0 == 0.0) {
      if (x0 > lo && x0 < hi) consider(x0);
      return;
    }
    if ((f0 < 0.0) == (f1 < 0.0) || f1 == 0.0) return;
    // phi' is monotone on the piece: Newton steps on phi' kept inside the
    // sign-change bracket (a bisection step whenever Newton would leave it)
    // converge quadratically; stop at a step within 4 ulp or an exhausted
    // bracket.
    double x = 0.5 * (x0 + x1);
    for (int it = 0; it < 100; ++it) {
      const double fx = dphi(x);
      if (fx == 0.0) break;
      if ((fx < 0.0) == (f0 < 0.0)) {
        x0 = x;
        f0 = fx;
      } else {
        x1 = x;
      }
      const double d2 = d2phi(x);
      if (d2 != 0.0) {
        const double step = fx / d2;
        if (fabs(step) <= 8.881784197001252e-16 * fabs(x)) {
          x -= step;
          break;
        }
      }
      double xn = (d2 != 0.0) ? x - fx / d2 : 0.5 * (x0 + x1);
      if (!(xn > x0 && xn < x1)) xn = 0.5 * (x0 + x1);
      if (!(xn > x0 && xn < x1)) break;
      x = xn;
    }
    if (x > lo && x < hi) consider(x);
  };
  double q0 = hi, q1 = hi;
  const int nq = quad_roots_in(12.0 * w[4], 6.0 * w[3], 2.0 * w[2], lo, hi, q0, q1);
  if (nq == 0) {
    piece(lo, hi);
  } else {
    piece(lo, q0);
    if (nq == 1) {
      piece(q0, hi);
    } else {
      piece(q0, q1);
      piece(q1, hi);
    }
  }
  consider(hi);
  return best;
}

// alpha from the Gram G (upper triangle, row-major, of the J x J Gram of the
// scaled Krylov blocks K~_j = (R/s)^j S, j = 1..J, J = 2d + 1): the
// coefficient vectors of r(xi; alpha) are rescaled by s^j to undo the Krylov
// scaling, the quartic phi_S(alpha) = c(alpha)^T M c(alpha) is formed, and its
// argmin on [lo, hi] is taken.  A degenerate or non-finite quartic gives c_d.
template <int J>
__device__ inline double alpha_from_gram_t(const double* G, double s, const AlphaCoef& co,
                                           double lo, double hi, double* phi_out) {
  double av[3][J];
  double sp = 1.0;
#pragma unroll
  for (int j = 1; j <= J; ++j) {
    sp *= s;
#pragma unroll
    for (int i = 0; i < 3; ++i) av[i][j - 1] = co.a[i][j] * sp;
  }
  // full J x J Gram from the packed upper triangle, then u_i = M a_i
  double M[J][J];
  {
    int t = 0;
#pragma unroll
    for (int x = 0; x < J; ++x)
#pragma unroll
      for (int y = x; y < J; ++y, ++t) M[x][y] = M[y][x] = G[t];
  }
  double u[3][J];
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int x = 0; x < J; ++x) {
      double v = 0.0;
#pragma unroll
      for (int y = 0; y < J; ++y) v += M[x][y] * av[i][y];
      u[i][x] = v;
    }
  auto q = [&](int i1, int i2) {
    double t = 0.0;
#pragma unroll
    for (int x = 0; x < J; ++x) t += av[i1][x] * u[i2][x];
    return t;
  };
  double w[5];
  w[0] = q(0, 0);
  w[1] = q(0, 1) + q(1, 0);
  w[2] = q(1, 1) + q(0, 2) + q(2, 0);
  w[3] = q(1, 2) + q(2, 1);
  w[4] = q(2, 2);
  bool ok = true;
  double mx = 0.0;
#pragma unroll
  for (int e = 0; e < 5; ++e) ok = ok && isfinite(w[e]);
#pragma unroll
  for (int e = 1; e < 5; ++e) mx = fmax(mx, fabs(w[e]));
  double a;
  if (!ok || mx <= 1e-300) a = fmin(fmax(co.taylor_d, lo), hi);
  else if (hi <= lo) a = lo;
  else a = argmin_quartic(w, lo, hi);
  // phi_S at the chosen alpha (the sketched ||R_{k+1} S||_F^2)
  if (phi_out) *phi_out = w[0] + a * (w[1] + a * (w[2] + a * (w[3] + a * w[4])));
  return a;
}

// ------------------------------------------------- inverse Newton objective
// Real roots inside (lo, hi), ascending, of c[0] + c[1] x + ... + c[D] x^D.
// The roots of the derivative split [lo, hi] into pieces on which the
// polynomial is monotone; every sign change on a piece is refined by the same
// bracketed Newton steps as argmin_quartic.  At most D roots.
template <int D>
__device__ inline int poly_roots_in(const double* c, double lo, double hi, double* out) {
  if constexpr (D == 1) {
    if (c[1] == 0.0) return 0;
    const double x = -c[0] / c[1];
    if (x > lo && x < hi) {
      out[0] = x;
      return 1;
    }
    return 0;
  } else {
    double dc[D];
#pragma unroll
    for (int i = 0; i < D; ++i) dc[i] = (double)(i + 1) * c[i + 1];
    double brk[D + 1];
    int nb = 0;
    brk[nb++] = lo;
    double crit[D];
    const int nc = poly_roots_in<D - 1>(dc, lo, hi, crit);
    for (int i = 0; i < nc; ++i) brk[nb++] = crit[i];
    brk[nb++] = hi;
    auto P = [&](double x) {
      double v = c[D];
      for (int i = D - 1; i >= 0; --i) v = v * x + c[i];
      return v;
    };
    auto dP = [&](double x) {
      double v = dc[D - 1];
      for (int i = D - 2; i >= 0; --i) v = v * x + dc[i];
      return v;
    };
    int n = 0;
    for (int i = 0; i + 1 < nb; ++i) {
      double x0 = brk[i], x1 = brk[i + 1];
      double f0 = P(x0);
      const double f1 = P(x1);
      if (f0 == 0.0) {
        if (x0 > lo && x0 < hi && (n == 0 || out[n - 1] != x0)) out[n++] = x0;
        continue;
      }
      if ((f0 < 0.0) == (f1 < 0.0) || f1 == 0.0) continue;
      double x = 0.5 * (x0 + x1);
      for (int it = 0; it < 100; ++it) {
        const double fx = P(x);
        if (fx == 0.0) break;
        if ((fx < 0.0) == (f0 < 0.0)) {
          x0 = x;
          f0 = fx;
        } else {
          x1 = x;
        }
        const double d1 = dP(x);
        if (d1 != 0.0) {
          const double step = fx / d1;
          if (fabs(step) <= 8.881784197001252e-16 * fabs(x)) {
            x -= step;
            break;
          }
        }
        double xn = (d1 != 0.0) ? x - fx / d1 : 0.5 * (x0 + x1);
        if (!(xn > x0 && xn < x1)) xn = 0.5 * (x0 + x1);
        if (!(xn > x0 && xn < x1)) break;
        x = xn;
      }
      if (x > lo && x < hi) out[n++] = x;
    }
    return n;
  }
}

// alpha for the inverse Newton family from the Gram G (packed upper
// triangle of the J x J Gram of the scaled K~_j = (R/s)^j S, j = 1..J): the
// objective c(alpha)^T M c(alpha), c(alpha) = sum_{i <= NP - 1} alpha^i a_i,
// has degree 2 (NP - 1); its argmin over [lo, hi] among both ends and the
// critical points inside (ties to the smaller alpha).  A degenerate or
// non-finite objective gives the Taylor coefficient.
template <int J, int NP>
__device__ inline double alpha_from_gram_newton(const double* G, double s,
                                                const AlphaCoefN& co, double lo, double hi,
                                                double* phi_out) {
  constexpr int W = 2 * (NP - 1);  // degree of the objective
  double av[NP][J];
  double sp = 1.0;
  for (int j = 1; j <= J; ++j) {
    sp *= s;
    for (int i = 0; i < NP; ++i) av[i][j - 1] = co.a[i][j] * sp;
  }
  double M[J][J];
  {
    int t = 0;
    for (int x = 0; x < J; ++x)
      for (int y = x; y < J; ++y, ++t) M[x][y] = M[y][x] = G[t];
  }
  double w[W + 1];
  for (int e = 0; e <= W; ++e) w[e] = 0.0;
  for (int i1 = 0; i1 < NP; ++i1) {
    double u[J];
    for (int x = 0; x < J; ++x) {
      double v = 0.0;
      for (int y = 0; y < J; ++y) v += M[x][y] * av[i1][y];
      u[x] = v;
    }
    for (int i2 = 0; i2 < NP; ++i2) {
      double t = 0.0;
      for (int x = 0; x < J; ++x) t += av[i2][x] * u[x];
      w[i1 + i2] += t;
    }
  }
  auto phi = [&](double a) {
    double v = w[W];
    for (int e = W - 1; e >= 0; --e) v = v * a + w[e];
    return v;
  };
  bool ok = true;
  double mx = 0.0;
  for (int e = 0; e <= W; ++e) ok = ok && isfinite(w[e]);
  for (int e = 1; e <= W; ++e) mx = fmax(mx, fabs(w[e]));
  double best;
  if (!ok || mx <= 1e-300) {
    best = fmin(fmax(co.taylor_d, lo), hi);
  } else if (hi <= lo) {
    best = lo;
  } else {
    double dw[W];
    for (int e = 0; e < W; ++e) dw[e] = (double)(e + 1) * w[e + 1];
    double crit[W];
    const int nc = poly_roots_in<W - 1>(dw, lo, hi, crit);
    best = lo;
    double bv = phi(lo);
    for (int i = 0; i < nc; ++i) {  // ascending: strict improvement keeps the smaller
      const double v = phi(crit[i]);
      if (v < bv) {
        bv = v;
        best = crit[i];
      }
    }
    if (phi(hi) < bv) best = hi;
  }
  if (phi_out) *phi_out = phi(best);
  return best;
}

__device__ inline double alpha_from_gram(const double* G, int J, double s, const AlphaCoef& co,
                                         double lo, double hi, double* phi_out = nullptr) {
  if (J == 3) return alpha_from_gram_t<3>(G, s, co, lo, hi, phi_out);
  if (J == 5) return alpha_from_gram_t<5>(G, s, co, lo, hi, phi_out);
  return alpha_from_gram_t<7>(G, s, co, lo, hi, phi_out);
}

}  // namespace pmx
