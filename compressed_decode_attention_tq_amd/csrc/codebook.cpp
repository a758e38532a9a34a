// Host-side Lloyd-Max codebook for the rotated-coordinate density.
//
// [tq-80] "TurboQuant：让大模型本地推理内存占用降低80%的KV缓存压缩技术", §核心创新: after a
// random orthogonal rotation each coordinate of a unit vector follows a known, highly
// concentrated Beta law, so an optimal scalar (Lloyd-Max) quantizer can be precomputed
// once, independently of any data.  For a uniform point on the sphere S^{d-1} one
// coordinate has density proportional to (1 - x^2)^((d-3)/2) on [-1, 1].
//
// The quantizer satisfies the two Lloyd-Max conditions: each boundary is the midpoint of
// its neighbouring centroids, and each centroid is the conditional mean of its cell.  The
// density is log-concave, so that fixed point is unique.  It is found by Lloyd steps
// followed by Newton steps on c - Phi(c) = 0, whose Jacobian is tridiagonal.
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <vector>

#include "tq.h"

namespace {

struct Quadrature {
  double x[24];
  double w[24];
  int n;
};

// Gauss-Legendre nodes and weights on [-1, 1] by Newton iteration on P_n.
Quadrature gauss_legendre(int n) {
  Quadrature q;
  q.n = n;
  for (int i = 0; i < (n + 1) / 2; ++i) {
    double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
    double dp = 0.0;
    for (int it = 0; it < 100; ++it) {
      double p0 = 1.0, p1 = z;
      for (int k = 2; k <= n; ++k) {
        double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = p2;
      }
      dp = n * (z * p1 - p0) / (z * z - 1.0);
      double dz = p1 / dp;
      z -= dz;
      if (std::fabs(dz) < 1e-16) break;
    }
    {
      double p0 = 1.0, p1 = z;
      for (int k = 2; k <= n; ++k) {
        double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = p2;
      }
      dp = n * (z * p1 - p0) / (z * z - 1.0);
    }
    double w = 2.0 / ((1.0 - z * z) * dp * dp);
    q.x[i] = -z;
    q.w[i] = w;
    q.x[n - 1 - i] = z;
    q.w[n - 1 - i] = w;
  }
  return q;
}

struct Density {
  double alpha;
  double operator()(double x) const {
    double s = 1.0 - x * x;
    return s > 0.0 ? std::pow(s, alpha) : 0.0;
  }
  // Antiderivative of x (1-x^2)^alpha.
  double moment_primitive(double x) const {
    double s = 1.0 - x * x;
    return s > 0.0 ? -std::pow(s, alpha + 1.0) / (2.0 * (alpha + 1.0)) : 0.0;
  }
};

// Mass of the density over [a, b]: composite Gauss-Legendre, pieces of width <= 0.005.
double cell_mass(const Density &f, const Quadrature &q, double a, double b) {
  if (b <= a) return 0.0;
  int pieces = (int)std::ceil((b - a) / 0.005);
  if (pieces < 1) pieces = 1;
  double h = (b - a) / pieces, sum = 0.0;
  for (int p = 0; p < pieces; ++p) {
    double mid = a + (p + 0.5) * h, half = 0.5 * h, s = 0.0;
    for (int j = 0; j < q.n; ++j) s += q.w[j] * f(mid + half * q.x[j]);
    sum += s * half;
  }
  return sum;
}

// Centroid map Phi(c) and the Lloyd-Max Jacobian terms for the current centroids.
void centroid_map(const Density &f, const Quadrature &q, const std::vector<double> &c,
                  std::vector<double> &phi, std::vector<double> &lo_term,
                  std::vector<double> &hi_term) {
  const int L = (int)c.size();
  for (int k = 0; k < L; ++k) {
    double a = k == 0 ? -1.0 : 0.5 * (c[k - 1] + c[k]);
    double b = k == L - 1 ? 1.0 : 0.5 * (c[k] + c[k + 1]);
    double m0 = cell_mass(f, q, a, b);
    double m1 = f.moment_primitive(b) - f.moment_primitive(a);
    double mean = m1 / m0;
    phi[k] = mean;
    // d Phi_k / d a = f(a) (mean - a) / m0,  d Phi_k / d b = f(b) (b - mean) / m0
    lo_term[k] = k == 0 ? 0.0 : f(a) * (mean - a) / m0;
    hi_term[k] = k == L - 1 ? 0.0 : f(b) * (b - mean) / m0;
  }
}

double inverse_normal_cdf(double p) {
  // bisection on the normal CDF 0.5 * erfc(-x / sqrt(2))
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 200; ++i) {
    double mid = 0.5 * (lo + hi);
    double cdf = 0.5 * std::erfc(-mid / std::sqrt(2.0));
    if (cdf < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

double residual(const std::vector<double> &c, const std::vector<double> &phi) {
  double r = 0.0;
  for (size_t k = 0; k < c.size(); ++k) r = std::fmax(r, std::fabs(c[k] - phi[k]));
  return r;
}

bool increasing(const std::vector<double> &c) {
  for (size_t k = 1; k < c.size(); ++k)
    if (!(c[k] > c[k - 1])) return false;
  return c.front() > -1.0 && c.back() < 1.0;
}

}  // namespace

extern "C" float tq_value_table_scale(const float *c, int n_levels) {
  if (c == nullptr || n_levels != 4) return 1.f;
  const double a = c[2], b = c[3];
  if (!(a > 0.0) || !(b > a) || c[1] != -c[2] || c[0] != -c[3]) return 1.f;
  const double r = b / a;
  if (!(r < 2047.0)) return 1.f;
  // convergents p_k / q_k of r: p_k = a_k p_{k-1} + p_{k-2}, the same for q
  double p0 = 1.0, q0 = 0.0, p1 = std::floor(r), q1 = 1.0, x = r - p1;
  for (int k = 0; k < 64 && x > 1e-12; ++k) {
    x = 1.0 / x;
    const double ak = std::floor(x);
    x -= ak;
    const double p2 = ak * p1 + p0, q2 = ak * q1 + q0;
    if (p2 > 2047.0) break;
    p0 = p1;
    q0 = q1;
    p1 = p2;
    q1 = q2;
  }
  // q 2^j in [a, 2a)
  const double qj = q1 * std::exp2(std::floor(std::log2(a / q1)));
  const double s = (qj < a ? 2.0 * qj : qj) / a;
  return (float)s;
}

extern "C" int tq_make_codebook_table(int d, int bits, float *centroids, float *boundaries) {
  if (centroids == nullptr || boundaries == nullptr || d < 4) return TQ_ERR_INVALID_ARG;
  if (bits < 1 || bits > 8) return TQ_ERR_UNSUPPORTED;
  const int L = 1 << bits;
  const Density f{(d - 3) / 2.0};
  const Quadrature q = gauss_legendre(20);

  std::vector<double> c(L), phi(L), lo(L), hi(L), delta(L);
  for (int k = 0; k < L; ++k) c[k] = inverse_normal_cdf((k + 0.5) / L) / std::sqrt((double)d);

  // A few plain Lloyd steps bring the centroids into Newton's basin.
  for (int it = 0; it < 50; ++it) {
    centroid_map(f, q, c, phi, lo, hi);
    c = phi;
  }
  // Newton on F(c) = c - Phi(c): J = I - dPhi/dc with
  // dPhi_k/dc_{k-1} = lo_k / 2, dPhi_k/dc_k = (lo_k + hi_k) / 2, dPhi_k/dc_{k+1} = hi_k / 2.
  for (int it = 0; it < 100; ++it) {
    centroid_map(f, q, c, phi, lo, hi);
    double r0 = residual(c, phi);
    if (r0 < 1e-16) break;
    std::vector<double> sub(L), diag(L), sup(L), rhs(L);
    for (int k = 0; k < L; ++k) {
      sub[k] = -0.5 * lo[k];
      diag[k] = 1.0 - 0.5 * (lo[k] + hi[k]);
      sup[k] = -0.5 * hi[k];
      rhs[k] = phi[k] - c[k];
    }
    // Thomas algorithm
    for (int k = 1; k < L; ++k) {
      double m = sub[k] / diag[k - 1];
      diag[k] -= m * sup[k - 1];
      rhs[k] -= m * rhs[k - 1];
    }
    delta[L - 1] = rhs[L - 1] / diag[L - 1];
    for (int k = L - 2; k >= 0; --k) delta[k] = (rhs[k] - sup[k] * delta[k + 1]) / diag[k];
    // damped step: keep the centroids ordered and the residual decreasing
    double step = 1.0;
    std::vector<double> trial(L);
    bool accepted = false;
    for (int half = 0; half < 40; ++half, step *= 0.5) {
      for (int k = 0; k < L; ++k) trial[k] = c[k] + step * delta[k];
      if (!increasing(trial)) continue;
      std::vector<double> p2(L), l2(L), h2(L);
      centroid_map(f, q, trial, p2, l2, h2);
      if (residual(trial, p2) < r0 || r0 < 1e-14) {
        accepted = true;
        break;
      }
    }
    if (!accepted) {  // fall back to a Lloyd step
      c = phi;
      continue;
    }
    bool tiny = true;
    for (int k = 0; k < L; ++k) {
      if (std::fabs(trial[k] - c[k]) > 1e-17) tiny = false;
      c[k] = trial[k];
    }
    if (tiny) break;
  }
  // The density is even: symmetrise, which makes the middle boundary exactly 0.
  std::vector<double> s(L);
  for (int k = 0; k < L; ++k) s[k] = 0.5 * (c[k] - c[L - 1 - k]);
  for (int k = 0; k < L; ++k) {
    if (!std::isfinite(s[k])) return TQ_ERR_INVALID_ARG;
    centroids[k] = (float)s[k];
  }
  for (int k = 0; k + 1 < L; ++k) boundaries[k] = (float)(0.5 * (s[k] + s[k + 1]));
  return TQ_OK;
}
