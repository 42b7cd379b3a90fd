// Host-side math of libtq: the Beta and Gaussian Lloyd-Max codebooks, the
// SplitMix64 streams of the rotation and the sketch, and the eigenbases of
// HeadQ and SpectralQuant calibration.
//
// [P1] = "Resumen Técnico: Inferencia Estadística y Medidas de Calidad de
//        Cuantizaciones de Cache KV Inspiradas en TurboQuant"
// [P2] = "Resumo Técnico: Ablação, Inferência Estatística e Validação para
//        Compressão de KV-Cache"
// [P3] = "Resumo Técnico: HeadQ: Distorção Visível ao Modelo e Correção no
//        Espaço de Pontuação para Quantização de KV-Cache"
#include <algorithm>
#include <cmath>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "internal.h"

namespace tq {
namespace {

// ---- regularised incomplete beta I_x(a, b) ---------------------------------
// Continued fraction of DLMF 8.17.22 evaluated with the modified Lentz method;
// for x beyond the mean the symmetry I_x(a,b) = 1 - I_{1-x}(b,a) is used.
// log B(a, b) in long double: at a = b = 511.5 the three log-gamma terms are
// ~2.6e3, so double would leave ~1e-13 relative error in B.
long double lbeta(long double a, long double b) { return lgammal(a) + lgammal(b) - lgammal(a + b); }

double beta_cf(double a, double b, double x) {
  const double tiny = 1e-300, eps = 1e-17;
  double c = 1.0, dd = 1.0 - (a + b) * x / (a + 1.0);
  if (std::fabs(dd) < tiny) dd = tiny;
  dd = 1.0 / dd;
  double h = dd;
  for (int m = 1; m < 200000; ++m) {
    double m2 = 2.0 * m;
    double num = m * (b - m) * x / ((a + m2 - 1.0) * (a + m2));
    dd = 1.0 + num * dd; if (std::fabs(dd) < tiny) dd = tiny;
    c = 1.0 + num / c;   if (std::fabs(c) < tiny) c = tiny;
    dd = 1.0 / dd; h *= dd * c;
    num = -(a + m) * (a + b + m) * x / ((a + m2) * (a + m2 + 1.0));
    dd = 1.0 + num * dd; if (std::fabs(dd) < tiny) dd = tiny;
    c = 1.0 + num / c;   if (std::fabs(c) < tiny) c = tiny;
    dd = 1.0 / dd;
    double del = dd * c;
    h *= del;
    if (std::fabs(del - 1.0) < eps) break;
  }
  return h;
}

double inc_beta(double a, double b, double x) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  if (a == b && x == 0.5) return 0.5;
  const long double lf = (long double)a * logl((long double)x) + (long double)b * log1pl(-(long double)x) - lbeta(a, b);
  const double f = (double)expl(lf);
  if (x < (a + 1.0) / (a + b + 2.0)) return f * beta_cf(a, b, x) / a;
  return 1.0 - f * beta_cf(b, a, 1.0 - x) / b;
}

// Lower tail P(T <= t) of one coordinate t of a uniform unit vector in R^d,
// for t <= 0 only (the upper tail follows by symmetry, keeping precision).
double lower_tail(double t, double a) { return inc_beta(a, a, 0.5 * (1.0 + t)); }

// Probability of the cell [lo, hi) under f_d(t) = (1-t^2)^(a-1) / B(1/2, a),
// a = (d-1)/2 ([P1] "Marco Teórico": the Beta((d-1)/2,(d-1)/2) marginal).
double cell_mass(double lo, double hi, double a) {
  if (hi <= 0.0) return lower_tail(hi, a) - lower_tail(lo, a);
  if (lo >= 0.0) return lower_tail(-lo, a) - lower_tail(-hi, a);
  return 1.0 - lower_tail(lo, a) - lower_tail(-hi, a);
}

// Integral of t f_d(t) over [lo, hi]; d/dt of -(1-t^2)^a / (2a) is t (1-t^2)^(a-1).
double cell_moment(double lo, double hi, double a, double log_norm) {
  auto g = [a](double t) { return std::fabs(t) >= 1.0 ? 0.0 : std::exp(a * std::log1p(-t * t)); };
  return (g(lo) - g(hi)) / (2.0 * a * std::exp(log_norm));
}

std::mutex g_cb_mu;
std::map<std::pair<int, int>, std::pair<std::vector<double>, std::vector<double>>> g_cb_cache;

uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kTagSign = 0x243F6A8885A308D3ull;
constexpr uint64_t kTagGauss = 0x13198A2E03707344ull;

}  // namespace

// Lloyd-Max fixed point: boundaries at midpoints, centroids at the
// conditional means of their cells ([P2] "Configuração Experimental": a
// data-oblivious Beta Lloyd-Max codebook).  Starts from evenly spaced levels
// in +-2/sqrt(d); the density is log-concave, so the fixed point is unique.
bool codebook(int d, int bits, std::vector<double>* centroids, std::vector<double>* boundaries) {
  if (d < 2 || bits < 1 || bits > 8) return false;
  {
    std::lock_guard<std::mutex> lk(g_cb_mu);
    auto it = g_cb_cache.find({d, bits});
    if (it != g_cb_cache.end()) {
      *centroids = it->second.first;
      *boundaries = it->second.second;
      return true;
    }
  }
  const int K = 1 << bits;
  const double a = 0.5 * (d - 1);
  const double log_norm = (double)(lgammal(0.5L) + lgammal((long double)a) - lgammal((long double)a + 0.5L));
  std::vector<double> c(K), t(K - 1), e(K + 1);
  for (int k = 0; k < K; ++k) c[k] = (2.0 * k - (K - 1)) / (K - 1 > 0 ? K - 1 : 1) * 2.0 / std::sqrt((double)d);
  for (int it = 0; it < 100000; ++it) {
    e[0] = -1.0; e[K] = 1.0;
    for (int k = 0; k + 1 < K; ++k) e[k + 1] = 0.5 * (c[k] + c[k + 1]);
    double delta = 0.0;
    for (int k = 0; k < K; ++k) {
      double m0 = cell_mass(e[k], e[k + 1], a);
      double m1 = cell_moment(e[k], e[k + 1], a, log_norm);
      double nc = m1 / m0;
      delta = std::max(delta, std::fabs(nc - c[k]));
      c[k] = nc;
    }
    if (delta < 1e-15) break;
  }
  std::vector<double> cs(K);
  for (int k = 0; k < K; ++k) cs[k] = 0.5 * (c[k] - c[K - 1 - k]);
  for (int k = 0; k + 1 < K; ++k) t[k] = 0.5 * (cs[k] + cs[k + 1]);
  t[K / 2 - 1] = 0.0;
  *centroids = cs;
  *boundaries = t;
  std::lock_guard<std::mutex> lk(g_cb_mu);
  g_cb_cache[{d, bits}] = {cs, t};
  return true;
}

// Relative MSE d * E[(T - c[idx(T)])^2] of the b-bit Beta Lloyd-Max code of
// one coordinate T of a uniform unit vector in R^d: at the fixed point every
// centroid is its cell's conditional mean, so the per-coordinate distortion is
// E[T^2] - sum_k P_k c_k^2 with E[T^2] = 1/d.
double codebook_distortion(int d, int bits) {
  std::vector<double> c, t;
  if (!codebook(d, bits, &c, &t)) return NAN;
  const double a = 0.5 * (d - 1);
  const int K = (int)c.size();
  double s = 0.0;
  for (int k = 0; k < K; ++k) {
    const double lo = k == 0 ? -1.0 : t[k - 1], hi = k == K - 1 ? 1.0 : t[k];
    s += cell_mass(lo, hi, a) * c[k] * c[k];
  }
  return d * (1.0 / d - s);
}

// Sign vector of the randomised Walsh-Hadamard rotation ([P2]
// "Configuração Experimental"): D_i = -1 iff bit 63 of the i-th output of
// the SplitMix64 stream started at seed ^ kTagSign is set.
void sign_vector(uint64_t seed, int d, float* signs) {
  uint64_t base = seed ^ kTagSign;
  for (int i = 0; i < d; ++i) {
    uint64_t o = mix64(base + (uint64_t)(i + 1) * kGamma);
    signs[i] = (o >> 63) ? -1.0f : 1.0f;
  }
}

// Gaussian sketch S (m = d rows) of the QJL stage ([P1] "Contribuciones
// Clave" 1): Box-Muller pairs in double from the stream at seed ^ kTagGauss,
// each rounded straight from double to the nearest fp16 value (so S is exact
// in fp16, which the sketch projection on fp16 matrix cores relies on), and
// returned as float.
void gaussian_sketch(uint64_t seed, int d, float* S) {
  const uint64_t base = seed ^ kTagGauss;
  const size_t n = (size_t)d * d;
  const double two_pi = 6.283185307179586;
  for (size_t p = 0; 2 * p < n; ++p) {
    uint64_t o1 = mix64(base + (uint64_t)(2 * p + 1) * kGamma) >> 11;
    uint64_t o2 = mix64(base + (uint64_t)(2 * p + 2) * kGamma) >> 11;
    double u1 = ((double)o1 + 1.0) * 0x1.0p-53;
    double u2 = (double)o2 * 0x1.0p-53;
    double r = std::sqrt(-2.0 * std::log(u1));
    S[2 * p] = (float)(_Float16)(r * std::cos(two_pi * u2));
    if (2 * p + 1 < n) S[2 * p + 1] = (float)(_Float16)(r * std::sin(two_pi * u2));
  }
}

// [P3] section 3 ("Calibração"): rank-r PCA of the calibration queries.
// Centred covariance in double, cyclic Jacobi rotations to diagonal form,
// eigenvectors of the r largest eigenvalues, each flipped so that its
// largest-magnitude entry is positive.
bool pca_basis(const float* X, int N, int d, int rank, float* U, float* eigenvalues, float* mean_out) {
  if (N < 2 || d < 1 || rank < 1 || rank > d) return false;
  std::vector<double> mean(d, 0.0), A((size_t)d * d, 0.0), V((size_t)d * d, 0.0);
  for (int n = 0; n < N; ++n)
    for (int i = 0; i < d; ++i) mean[i] += X[(size_t)n * d + i];
  for (int i = 0; i < d; ++i) mean[i] /= N;
  std::vector<double> row(d);
  for (int n = 0; n < N; ++n) {
    for (int i = 0; i < d; ++i) row[i] = X[(size_t)n * d + i] - mean[i];
    for (int i = 0; i < d; ++i)
      for (int j = i; j < d; ++j) A[(size_t)i * d + j] += row[i] * row[j];
  }
  for (int i = 0; i < d; ++i)
    for (int j = i; j < d; ++j) {
      A[(size_t)i * d + j] /= N;
      A[(size_t)j * d + i] = A[(size_t)i * d + j];
    }
  for (int i = 0; i < d; ++i) V[(size_t)i * d + i] = 1.0;
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0, diag = 0.0;
    for (int i = 0; i < d; ++i) {
      diag += A[(size_t)i * d + i] * A[(size_t)i * d + i];
      for (int j = i + 1; j < d; ++j) off += A[(size_t)i * d + j] * A[(size_t)i * d + j];
    }
    if (off <= 1e-30 * diag) break;
    for (int p = 0; p < d; ++p)
      for (int q = p + 1; q < d; ++q) {
        double apq = A[(size_t)p * d + q];
        if (std::fabs(apq) < 1e-300) continue;
        double app = A[(size_t)p * d + p], aqq = A[(size_t)q * d + q];
        double theta = (aqq - app) / (2.0 * apq);
        double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        double c = 1.0 / std::sqrt(t * t + 1.0), s = t * c;
        // A <- J^T A J with J the rotation in the (p, q) plane.
        for (int k = 0; k < d; ++k) {
          double akp = A[(size_t)k * d + p], akq = A[(size_t)k * d + q];
          A[(size_t)k * d + p] = c * akp - s * akq;
          A[(size_t)k * d + q] = s * akp + c * akq;
        }
        for (int k = 0; k < d; ++k) {
          double apk = A[(size_t)p * d + k], aqk = A[(size_t)q * d + k];
          A[(size_t)p * d + k] = c * apk - s * aqk;
          A[(size_t)q * d + k] = s * apk + c * aqk;
        }
        for (int k = 0; k < d; ++k) {
          double vkp = V[(size_t)k * d + p], vkq = V[(size_t)k * d + q];
          V[(size_t)k * d + p] = c * vkp - s * vkq;
          V[(size_t)k * d + q] = s * vkp + c * vkq;
        }
      }
  }
  std::vector<int> order(d);
  for (int i = 0; i < d; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return A[(size_t)x * d + x] > A[(size_t)y * d + y]; });
  for (int j = 0; j < rank; ++j) {
    int col = order[j];
    int arg = 0;
    for (int i = 1; i < d; ++i)
      if (std::fabs(V[(size_t)i * d + col]) > std::fabs(V[(size_t)arg * d + col])) arg = i;
    double sgn = V[(size_t)arg * d + col] < 0 ? -1.0 : 1.0;
    for (int i = 0; i < d; ++i) U[(size_t)i * rank + j] = (float)(sgn * V[(size_t)i * d + col]);
    if (eigenvalues) eigenvalues[j] = (float)std::max(0.0, A[(size_t)col * d + col]);
  }
  if (mean_out)
    for (int i = 0; i < d; ++i) mean_out[i] = (float)mean[i];
  return true;
}

// Lloyd-Max codebook of N(0, 1) at `bits` bits: boundaries at midpoints,
// centroids at the conditional means (phi(a) - phi(b)) / (Phi(b) - Phi(a)) of
// their cells, from the quantile midpoints to a fixed point; made exactly
// symmetric (the middle boundary 0).  Cached per bits.
bool gaussian_codebook(int bits, std::vector<double>* centroids, std::vector<double>* boundaries) {
  if (bits < 1 || bits > 8) return false;
  static std::mutex mu;
  static std::map<int, std::pair<std::vector<double>, std::vector<double>>> cache;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(bits);
  if (it == cache.end()) {
    const int K = 1 << bits;
    const double inv_sqrt2 = 0.70710678118654752440, inv_sqrt2pi = 0.39894228040143267794;
    auto pdf = [&](double x) { return std::isinf(x) ? 0.0 : inv_sqrt2pi * std::exp(-0.5 * x * x); };
    auto sf = [&](double x) { return 0.5 * std::erfc(x * inv_sqrt2); };   // upper tail, exact far out
    // Start: levels spread over +-2 standard deviations.
    std::vector<double> c(K), t(K - 1);
    for (int k = 0; k < K; ++k) c[k] = -2.0 + 4.0 * (k + 0.5) / K;
    for (int iter = 0; iter < 200000; ++iter) {
      double delta = 0.0;
      std::vector<double> e(K + 1);
      e[0] = -INFINITY;
      e[K] = INFINITY;
      for (int k = 1; k < K; ++k) e[k] = 0.5 * (c[k - 1] + c[k]);
      for (int k = 0; k < K; ++k) {
        const double m0 = sf(e[k]) - sf(e[k + 1]);
        const double m1 = pdf(e[k]) - pdf(e[k + 1]);
        const double nc = m1 / m0;
        delta = std::max(delta, std::fabs(nc - c[k]));
        c[k] = nc;
      }
      if (delta < 1e-15) break;
    }
    std::vector<double> cs(K);
    for (int k = 0; k < K; ++k) cs[k] = 0.5 * (c[k] - c[K - 1 - k]);
    for (int k = 0; k + 1 < K; ++k) t[k] = 0.5 * (cs[k] + cs[k + 1]);
    t[K / 2 - 1] = 0.0;
    it = cache.emplace(bits, std::make_pair(cs, t)).first;
  }
  *centroids = it->second.first;
  *boundaries = it->second.second;
  return true;
}

}  // namespace tq
