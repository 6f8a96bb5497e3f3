// Lloyd-Max codebook for the fixed marginal f_d (host, fp64).
//
// Method: "OrbitQuant: data-agnostic quantization for image and video"
// (rcap.io summary), "core trick" paragraph and the offline pseudo-code line
// codebook[d, b] = lloyd_max(f_d, b): after normalisation and a random
// rotation, every coordinate follows one marginal that depends only on d,
// and one optimal scalar (Lloyd-Max) quantizer is built for it offline.
//
// f_d(t) = C_d (1 - t^2)^((d-3)/2) on [-1, 1], C_d = Gamma(d/2) /
// (sqrt(pi) Gamma((d-1)/2)), the marginal of one coordinate of a uniform
// point on the unit sphere of R^d; (1 + t)/2 is Beta((d-1)/2, (d-1)/2).
//
// Numerics (own implementation):
//  * log Gamma(x + 1/2) - log Gamma(x) by upward recurrence to x >= 40 and
//    the asymptotic series 1/2 log x - 1/(8x) + 1/(192x^3) - 1/(640x^5)
//    + 17/(14336x^7); this avoids the cancellation of two large lgamma values.
//  * the lower tail P(T <= t), t <= 0, as the regularised incomplete beta
//    I_x(a, a), x = (1+t)/2, by its continued fraction (DLMF 8.17.22)
//    evaluated with the modified Lentz method; the prefactor
//    x^a (1-x)^a / (a B(a, a)) is formed as exp(a log1p(-t^2) - ...) so its
//    large terms cancel analytically (Legendre duplication formula).
//  * the partial first moment in closed form,
//    int_lo^hi t f_d = C_d / (d-1) [(1-lo^2)^((d-1)/2) - (1-hi^2)^((d-1)/2)].
//  * Lloyd steps from a compander start, then Newton on G(c) = c - m(c) with
//    the tridiagonal Jacobian (Thomas algorithm) and backtracking.
#include <cmath>
#include <vector>

#include "oq_internal.h"

namespace oq {

namespace {

constexpr double kLn2 = 0.69314718055994530942;
constexpr double kLnPi = 1.14472988584940017414;

double log_gamma_half_ratio(double x) {
  double acc = 0.0;
  while (x < 40.0) {
    acc += std::log(x) - std::log(x + 0.5);
    x += 1.0;
  }
  const double ix = 1.0 / x, ix2 = ix * ix;
  return acc + 0.5 * std::log(x) - ix / 8.0 + ix * ix2 / 192.0 - ix * ix2 * ix2 / 640.0 +
         17.0 * ix * ix2 * ix2 * ix2 / 14336.0;
}

struct Marginal {
  int d;
  double a;      // (d-1)/2
  double log_c;  // log C_d
  double log_front0;

  explicit Marginal(int d_) : d(d_), a(0.5 * (d_ - 1)) {
    log_c = log_gamma_half_ratio(a) - 0.5 * kLnPi;
    // log(1 / (a B(a, a))) + a log(x (1-x)) with x (1-x) = (1 - t^2)/4:
    //   = a log1p(-t^2) - log 2 - log a + log[Gamma(a+1/2)/Gamma(a)] - 1/2 log pi
    log_front0 = -kLn2 - std::log(a) + log_gamma_half_ratio(a) - 0.5 * kLnPi;
  }

  double pdf(double t) const {
    const double at = std::fabs(t);
    if (at > 1.0) return 0.0;
    if (at == 1.0) return d == 3 ? std::exp(log_c) : 0.0;
    return std::exp(log_c + 0.5 * (d - 3) * std::log1p(-t * t));
  }

  // P(T <= t) for t <= 0.
  double lower_tail(double t) const {
    if (t <= -1.0) return 0.0;
    const double x = 0.5 * (1.0 + t);
    const double front = std::exp(a * std::log1p(-t * t) + log_front0);
    // continued fraction 1 + d1/(1 + d2/(1 + ...)), modified Lentz
    const double tiny = 1e-300;
    double f = 1.0, C = 1.0, D = 0.0;
    for (int j = 1; j < 100000; ++j) {
      double dj;
      const int m = j / 2;
      if (j & 1) {
        dj = -(a + m) * (a + a + m) * x / ((a + 2 * m) * (a + 2 * m + 1));
      } else {
        dj = m * (a - m) * x / ((a + 2 * m - 1) * (a + 2 * m));
      }
      D = 1.0 + dj * D;
      if (std::fabs(D) < tiny) D = tiny;
      C = 1.0 + dj / C;
      if (std::fabs(C) < tiny) C = tiny;
      D = 1.0 / D;
      const double delta = C * D;
      f *= delta;
      if (std::fabs(delta - 1.0) < 1e-16) break;
    }
    return front / f;
  }

  double upper_tail(double t) const { return lower_tail(-t); }  // P(T > t), t >= 0

  double mass(double lo, double hi) const {
    if (hi <= 0.0) return lower_tail(hi) - lower_tail(lo);
    if (lo >= 0.0) return upper_tail(lo) - upper_tail(hi);
    return 1.0 - lower_tail(lo) - upper_tail(hi);
  }

  double moment1(double lo, double hi) const {
    const double e = 0.5 * (d - 1);
    auto g = [&](double t) {
      if (std::fabs(t) >= 1.0) return 0.0;
      return std::exp(e * std::log1p(-t * t));
    };
    return std::exp(log_c) / (d - 1) * (g(lo) - g(hi));
  }
};

double inv_normal_cdf(double p) {
  // bisection on Phi(x) = erfc(-x / sqrt 2) / 2; monotone, exact to fp64
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 200; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (0.5 * std::erfc(-mid / std::sqrt(2.0)) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

struct Eval {
  std::vector<double> m, P, M, G;
  double resid;
};

void evaluate(const Marginal& f, const std::vector<double>& c, Eval& e) {
  const int L = (int)c.size();
  e.m.resize(L); e.P.resize(L); e.M.resize(L); e.G.resize(L);
  e.resid = 0.0;
  for (int j = 0; j < L; ++j) {
    const double lo = j == 0 ? -1.0 : 0.5 * (c[j - 1] + c[j]);
    const double hi = j == L - 1 ? 1.0 : 0.5 * (c[j] + c[j + 1]);
    e.P[j] = f.mass(lo, hi);
    e.M[j] = f.moment1(lo, hi);
    e.m[j] = e.M[j] / e.P[j];
    e.G[j] = c[j] - e.m[j];
    e.resid = std::fmax(e.resid, std::fabs(e.G[j]));
  }
}

void symmetrize(std::vector<double>& c) {
  const int L = (int)c.size();
  for (int j = 0; j < L / 2; ++j) {
    const double v = 0.5 * (c[L - 1 - j] - c[j]);
    c[j] = -v;
    c[L - 1 - j] = v;
  }
  if (L & 1) c[L / 2] = 0.0;
}

bool increasing(const std::vector<double>& c) {
  for (size_t j = 1; j < c.size(); ++j)
    if (!(c[j] > c[j - 1])) return false;
  return true;
}

}  // namespace

int lloyd_max_fd(int d, int bits, int max_newton, double* centroids, double* thresholds, double* mse_out,
                 double* resid_out) {
  const Marginal f(d);
  const int L = 1 << bits;
  std::vector<double> c(L);
  const double sig3 = std::sqrt(3.0 / d);
  double cmax0 = 0.0;
  for (int j = 0; j < L; ++j) {
    c[j] = sig3 * inv_normal_cdf((j + 0.5) / L);
    cmax0 = std::fmax(cmax0, std::fabs(c[j]));
  }
  if (cmax0 > 0.95)  // small d: shrink the start into the support [-1, 1], keeping its order
    for (int j = 0; j < L; ++j) c[j] *= 0.95 / cmax0;
  symmetrize(c);

  Eval e;
  for (int it = 0; it < 50; ++it) {
    evaluate(f, c, e);
    c = e.m;
    symmetrize(c);
  }
  evaluate(f, c, e);

  std::vector<double> lo_d(L), di(L), up(L), rhs(L), step(L), cn(L);
  Eval en;
  for (int it = 0; it < max_newton; ++it) {
    double cmax = 0.0;
    for (double v : c) cmax = std::fmax(cmax, std::fabs(v));
    if (e.resid <= 1e-15 * cmax) break;
    // J = I - dm/dc; dm_j/dtheta_{j-1} = f(theta_{j-1}) (m_j - theta_{j-1}) / P_j,
    // dm_j/dtheta_j = f(theta_j) (theta_j - m_j) / P_j, dtheta/dc = 1/2.
    for (int j = 0; j < L; ++j) {
      double aj = 0.0, bj = 0.0;
      if (j > 0) {
        const double th = 0.5 * (c[j - 1] + c[j]);
        aj = f.pdf(th) * (e.m[j] - th) / e.P[j];
      }
      if (j < L - 1) {
        const double th = 0.5 * (c[j] + c[j + 1]);
        bj = f.pdf(th) * (th - e.m[j]) / e.P[j];
      }
      di[j] = 1.0 - 0.5 * (aj + bj);
      lo_d[j] = -0.5 * aj;  // coefficient of c_{j-1}
      up[j] = -0.5 * bj;    // coefficient of c_{j+1}
      rhs[j] = -e.G[j];
    }
    // Thomas algorithm
    for (int j = 1; j < L; ++j) {
      const double w = lo_d[j] / di[j - 1];
      di[j] -= w * up[j - 1];
      rhs[j] -= w * rhs[j - 1];
    }
    step[L - 1] = rhs[L - 1] / di[L - 1];
    for (int j = L - 2; j >= 0; --j) step[j] = (rhs[j] - up[j] * step[j + 1]) / di[j];

    bool improved = false;
    for (double lam = 1.0; lam > 1e-6; lam *= 0.5) {
      for (int j = 0; j < L; ++j) cn[j] = c[j] + lam * step[j];
      symmetrize(cn);
      if (!increasing(cn) || cn[0] <= -1.0 || cn[L - 1] >= 1.0) continue;
      evaluate(f, cn, en);
      if (en.resid < e.resid) {
        c = cn;
        e = en;
        improved = true;
        break;
      }
    }
    if (!improved) break;
  }

  double cmax = 0.0, mse = 1.0 / d;
  for (int j = 0; j < L; ++j) {
    cmax = std::fmax(cmax, std::fabs(c[j]));
    mse += -2.0 * c[j] * e.M[j] + c[j] * c[j] * e.P[j];
  }
  for (int j = 0; j < L; ++j) centroids[j] = c[j];
  for (int j = 0; j + 1 < L; ++j) thresholds[j] = 0.5 * (c[j] + c[j + 1]);
  if (mse_out) *mse_out = mse;
  const double rel = e.resid / cmax;
  if (resid_out) *resid_out = rel;
  return rel <= 1e-10 ? 0 : -1;
}

}  // namespace oq
