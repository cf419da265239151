// Per-step Newton-Schulz coefficients (host only).
//
// The DMuon-2 page (App. C.3) runs its Newton-Schulz steps with per-step
// coefficients from the Polar Express method (Amsel et al., 2025), and the
// HyperParallel-FSDP evaluation runs an "asym5" set; neither page prints the
// values.  This file computes a schedule by the construction that method
// publishes: each step takes the odd quintic p(x) = a x + b x^3 + c x^5 that is
// closest to 1 in the uniform norm on the interval [l, u] that holds the
// singular values at that step, and the next interval is p's range over
// [l, u] (an odd polynomial of X maps each singular value s to p(s)).  The
// first interval is [lower, 1]: after Frobenius normalisation no singular
// value exceeds 1, and `lower` is the caller's bound on the smallest one.
//
// The best approximation is found by the exchange (Remez) iteration: the
// error 1 - p of the optimum alternates in sign with equal magnitude at four
// points l < x1 < x2 < u (the endpoints and the two interior critical points
// of p), three coefficients plus the levelled error being fixed by those four
// equations.  On a very short interval the problem degenerates; there the
// optimum tends to the quintic with p(m) = 1, p'(m) = p''(m) = 0 at the
// interval's midpoint m, which is used instead.
#include <algorithm>
#include <cmath>

#include "../../include/muon.h"

namespace {

struct Quintic {
  double a, b, c;
};

double eval(const Quintic& p, double x) {
  const double y = x * x;
  return x * (p.a + y * (p.b + y * p.c));
}

// Points x in (lo, hi) with p'(x) = a + 3b x^2 + 5c x^4 = 0, ascending.
int critical_points(const Quintic& p, double lo, double hi, double out[2]) {
  double ys[2];
  int ny = 0;
  if (p.c == 0.0) {
    if (p.b != 0.0) ys[ny++] = -p.a / (3.0 * p.b);
  } else {
    const double qa = 5.0 * p.c, qb = 3.0 * p.b, qc = p.a;
    const double disc = qb * qb - 4.0 * qa * qc;
    if (disc >= 0.0) {
      // the two roots in y = x^2, in the cancellation-free form
      const double q = -0.5 * (qb + std::copysign(std::sqrt(disc), qb));
      if (q != 0.0) {
        ys[ny++] = q / qa;
        ys[ny++] = qc / q;
      }
    }
  }
  int n = 0;
  for (int i = 0; i < ny; ++i) {
    if (!(ys[i] > 0.0)) continue;
    const double x = std::sqrt(ys[i]);
    if (x > lo && x < hi) out[n++] = x;
  }
  if (n == 2 && out[0] > out[1]) std::swap(out[0], out[1]);
  return n;
}

// Smallest and largest value of p on [lo, hi].
void range_on(const Quintic& p, double lo, double hi, double* mn, double* mx) {
  const double v0 = eval(p, lo), v1 = eval(p, hi);
  *mn = std::min(v0, v1);
  *mx = std::max(v0, v1);
  double r[2];
  const int n = critical_points(p, lo, hi, r);
  for (int i = 0; i < n; ++i) {
    const double v = eval(p, r[i]);
    *mn = std::min(*mn, v);
    *mx = std::max(*mx, v);
  }
}

// Gaussian elimination with partial pivoting on the 4 x 5 augmented system.
bool solve4(double m[4][5], double s[4]) {
  for (int col = 0; col < 4; ++col) {
    int piv = col;
    for (int r = col + 1; r < 4; ++r)
      if (std::fabs(m[r][col]) > std::fabs(m[piv][col])) piv = r;
    if (m[piv][col] == 0.0) return false;
    if (piv != col)
      for (int k = 0; k < 5; ++k) std::swap(m[piv][k], m[col][k]);
    for (int r = col + 1; r < 4; ++r) {
      const double f = m[r][col] / m[col][col];
      for (int k = col; k < 5; ++k) m[r][k] -= f * m[col][k];
    }
  }
  for (int r = 3; r >= 0; --r) {
    double v = m[r][4];
    for (int k = r + 1; k < 4; ++k) v -= m[r][k] * s[k];
    s[r] = v / m[r][r];
  }
  return true;
}

// The odd quintic closest to 1 in the uniform norm on [lo, hi], 0 < lo < hi.
bool best_quintic(double lo, double hi, Quintic* p) {
  const double pi = 3.14159265358979323846;
  double x[4], lev = 0.0;
  for (int i = 0; i < 4; ++i) x[i] = 0.5 * (lo + hi) - 0.5 * (hi - lo) * std::cos(i * pi / 3.0);
  for (int it = 0; it < 100; ++it) {
    // a x_i + b x_i^3 + c x_i^5 + (-1)^i E = 1: the error 1 - p is +E, -E, +E, -E
    double m[4][5];
    for (int i = 0; i < 4; ++i) {
      const double y = x[i] * x[i];
      m[i][0] = x[i];
      m[i][1] = x[i] * y;
      m[i][2] = x[i] * y * y;
      m[i][3] = (i & 1) ? -1.0 : 1.0;
      m[i][4] = 1.0;
    }
    double s[4];
    if (!solve4(m, s)) return false;
    *p = Quintic{s[0], s[1], s[2]};
    lev = std::fabs(s[3]);
    double r[2];
    if (critical_points(*p, lo, hi, r) != 2) return false;
    const double nx[4] = {lo, r[0], r[1], hi};
    double moved = 0.0;
    for (int i = 0; i < 4; ++i) {
      moved = std::max(moved, std::fabs(nx[i] - x[i]));
      x[i] = nx[i];
    }
    if (moved <= 1e-14 * hi) break;
  }
  // accept only a levelled solution: the largest error on [lo, hi] is E
  double mn, mx;
  range_on(*p, lo, hi, &mn, &mx);
  const double dev = std::max(1.0 - mn, mx - 1.0);
  return std::isfinite(dev) && dev <= lev * (1.0 + 1e-9) + 1e-15;
}

}  // namespace

extern "C" muon_status muon_ns_schedule(int32_t steps, double lower, double safety, double cushion,
                                        float* coeffs, double* bounds) {
  if (steps < 1 || steps > 64 || !coeffs) return MUON_ERR_INVALID_ARG;
  if (!(lower >= 1e-12 && lower < 1.0)) return MUON_ERR_INVALID_ARG;
  if (!(safety >= 1.0 && safety <= 2.0)) return MUON_ERR_INVALID_ARG;
  if (!(cushion >= 0.0 && cushion < 1.0)) return MUON_ERR_INVALID_ARG;
  double lo = lower, hi = 1.0;
  for (int k = 0; k < steps; ++k) {
    // Never design below 1e-4 u: there the levelled minimum 1 - E of p is
    // about a * 1e-4 u or less, within reach of the coefficients' float
    // rounding, and the rounded polynomial could cross zero (a sign flip of a
    // singular direction).  Below the design interval p rises from 0, so the
    // bounds still cover every value in [lo, hi].
    const double dlo = std::max({lo, cushion * hi, 1e-4 * hi});
    Quintic p;
    if (hi - dlo <= 1e-3 * hi) {
      const double mid = 0.5 * (dlo + hi);
      p = Quintic{1.875 / mid, -1.25 / (mid * mid * mid), 0.375 / (mid * mid * mid * mid * mid)};
    } else if (!best_quintic(dlo, hi, &p)) {
      return MUON_ERR_INTERNAL;
    }
    // p(x / safety): singular values up to safety * hi stay in the design range
    const double s2 = safety * safety;
    const float f[3] = {static_cast<float>(p.a / safety), static_cast<float>(p.b / (s2 * safety)),
                        static_cast<float>(p.c / (s2 * s2 * safety))};
    if (!std::isfinite(f[0]) || !std::isfinite(f[1]) || !std::isfinite(f[2])) return MUON_ERR_INTERNAL;
    // the next interval is the range of the polynomial the step will use
    double mn, mx;
    range_on(Quintic{f[0], f[1], f[2]}, lo, hi, &mn, &mx);
    if (!(mn > 0.0) || !std::isfinite(mx)) return MUON_ERR_INTERNAL;
    coeffs[3 * k + 0] = f[0];
    coeffs[3 * k + 1] = f[1];
    coeffs[3 * k + 2] = f[2];
    lo = mn;
    hi = mx;
    if (bounds) {
      bounds[2 * k] = lo;
      bounds[2 * k + 1] = hi;
    }
  }
  return MUON_OK;
}
