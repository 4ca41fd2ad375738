// Host setup of a TurboQuant codebook handle: the Lloyd-Max codebook for the
// coordinate law of a rotated unit vector, the seeded Haar rotation and the
// QJL Gaussian matrix.  Pure C++ (double precision), no HIP calls.
//
// [admirer.cn memory-wall article, section 2, stage one]: after a random
// rotation each coordinate of a unit vector follows a known Beta-type law, so
// a Lloyd-Max quantizer (1-D continuous k-means) for that law can be solved
// once per bit width and stored; inference only looks it up.
// [cc-newplayer explainer, technical breakdown item 2] and
// [intelliparadigm "3-bit" article, §2.1.1]: the rotation is a Haar-random
// orthogonal matrix.  [same article, §2.1.2]: S has Gaussian entries.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr double kPi = 3.14159265358979323846;

// log of the normalizing constant of f_d(t) = C_d (1 - t^2)^((d-3)/2).
double log_norm_const(int d) {
  return std::lgamma(0.5 * d) - 0.5 * std::log(kPi) - std::lgamma(0.5 * (d - 1));
}

// Continued fraction of the regularized incomplete beta function
// (DLMF 8.17.22), evaluated with the modified Lentz method.  Valid and fast
// for x < (a + 1) / (a + b + 2).
double beta_cf(double a, double b, double x) {
  const double tiny = 1e-300;
  double f = 1.0, C = 1.0, D = 0.0;
  for (int j = 1; j < 10000; ++j) {
    const int mm = j / 2;
    double coef;
    if (j % 2 == 0) {
      coef = mm * (b - mm) * x / ((a + 2.0 * mm - 1.0) * (a + 2.0 * mm));
    } else {
      coef = -(a + mm) * (a + b + mm) * x / ((a + 2.0 * mm) * (a + 2.0 * mm + 1.0));
    }
    D = 1.0 + coef * D;
    if (std::fabs(D) < tiny) D = tiny;
    D = 1.0 / D;
    C = 1.0 + coef / C;
    if (std::fabs(C) < tiny) C = tiny;
    const double delta = C * D;
    f *= delta;
    if (std::fabs(delta - 1.0) < 4e-16) break;
  }
  return f;
}

// I_x(a, b), regularized incomplete beta.
double incomplete_beta(double a, double b, double x) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  if (x > (a + 1.0) / (a + b + 2.0)) return 1.0 - incomplete_beta(b, a, 1.0 - x);
  const double lbeta = std::lgamma(a) + std::lgamma(b) - std::lgamma(a + b);
  const double front = std::exp(a * std::log(x) + b * std::log1p(-x) - lbeta) / a;
  return front / beta_cf(a, b, x);
}

// Integral of s f_d(s) ds over [-1, t]: (1 - t^2)^((d-1)/2) is an
// antiderivative of -(d-1) t (1 - t^2)^((d-3)/2).
double sphere_coord_first_moment(double t, int d) {
  t = std::min(1.0, std::max(-1.0, t));
  const double k1 = 0.5 * (d - 1);
  return -std::exp(log_norm_const(d)) * std::pow(1.0 - t * t, k1) / (2.0 * k1);
}

// SplitMix64 output for counter i (i >= 1) of state `seed`
// (Steele, Lea & Flood 2014; Stafford's variant-13 finalizer).
inline uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
  uint64_t z = seed + i * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace

double sphere_coord_cdf(double t, int d) {
  t = std::min(1.0, std::max(-1.0, t));
  const double a = 0.5 * (d - 1);
  return incomplete_beta(a, a, 0.5 * (1.0 + t));
}

void lloyd_max_sphere(int d, int bits, std::vector<double> *centroids,
                      std::vector<double> *thresholds, int *iterations) {
  const int L = 1 << bits;
  std::vector<double> c(L), t(L - 1), edge(L + 1);
  // Symmetric start: L equal steps over +-2 sigma (clipped inside [-1, 1]).
  const double spread = std::min(0.95, 2.0 / std::sqrt(static_cast<double>(d)));
  for (int i = 0; i < L; ++i) c[i] = spread * (2.0 * i + 1.0 - L) / L;
  int it = 0;
  for (it = 1; it <= 200000; ++it) {
    for (int i = 0; i + 1 < L; ++i) t[i] = 0.5 * (c[i] + c[i + 1]);
    edge[0] = -1.0;
    edge[L] = 1.0;
    for (int i = 0; i + 1 < L; ++i) edge[i + 1] = t[i];
    std::vector<double> cn(L);
    for (int i = 0; i < L; ++i) {
      const double mass = sphere_coord_cdf(edge[i + 1], d) - sphere_coord_cdf(edge[i], d);
      const double mom = sphere_coord_first_moment(edge[i + 1], d) - sphere_coord_first_moment(edge[i], d);
      cn[i] = mom / mass;
    }
    // The law is even: keep the iterate exactly antisymmetric.
    double step = 0.0;
    for (int i = 0; i < L; ++i) {
      const double v = 0.5 * (cn[i] - cn[L - 1 - i]);
      step = std::max(step, std::fabs(v - c[i]));
      c[i] = v;
    }
    if (step < 1e-15) break;
  }
  for (int i = 0; i + 1 < L; ++i) t[i] = 0.5 * (c[i] + c[i + 1]);
  *centroids = c;
  *thresholds = t;
  if (iterations) *iterations = it;
}

void seeded_normals(uint64_t seed, size_t count, double *out) {
  // Box-Muller on consecutive SplitMix64 outputs: u1 = 1 - (z >> 11) 2^-53 in
  // (0, 1], u2 = (z' >> 11) 2^-53 in [0, 1); radius sqrt(-2 ln u1); the even
  // normal takes cos(2 pi u2), the odd one sin(2 pi u2).
  const double two53 = 1.0 / 9007199254740992.0;
  for (size_t pair = 0; 2 * pair < count; ++pair) {
    const uint64_t za = splitmix64_at(seed, 2 * pair + 1);
    const uint64_t zb = splitmix64_at(seed, 2 * pair + 2);
    const double u1 = 1.0 - static_cast<double>(za >> 11) * two53;
    const double u2 = static_cast<double>(zb >> 11) * two53;
    const double rad = std::sqrt(-2.0 * std::log(u1));
    out[2 * pair] = rad * std::cos(2.0 * kPi * u2);
    if (2 * pair + 1 < count) out[2 * pair + 1] = rad * std::sin(2.0 * kPi * u2);
  }
}

void haar_orthogonal(int d, uint64_t seed, double *pi_rowmajor) {
  // Householder QR of the seeded Gaussian matrix G = Q R, then
  // Pi = Q diag(sign(R_kk)): the unique Q with positive-diagonal R, which is
  // Haar-distributed on O(d).
  std::vector<double> A(static_cast<size_t>(d) * d);
  seeded_normals(seed, A.size(), A.data());
  std::vector<double> Q(static_cast<size_t>(d) * d, 0.0);
  for (int i = 0; i < d; ++i) Q[static_cast<size_t>(i) * d + i] = 1.0;
  std::vector<double> v(d), rdiag(d);
  auto a = [&](int r, int c) -> double & { return A[static_cast<size_t>(r) * d + c]; };
  auto q = [&](int r, int c) -> double & { return Q[static_cast<size_t>(r) * d + c]; };
  for (int k = 0; k < d; ++k) {
    double norm2 = 0.0;
    for (int r = k; r < d; ++r) norm2 += a(r, k) * a(r, k);
    const double norm = std::sqrt(norm2);
    if (norm == 0.0) {
      rdiag[k] = 0.0;
      continue;
    }
    // Reflect column k onto alpha e_k with alpha = -sign(a_kk) * norm (no cancellation).
    const double alpha = a(k, k) >= 0.0 ? -norm : norm;
    double vnorm2 = 0.0;
    for (int r = k; r < d; ++r) {
      v[r] = a(r, k) - (r == k ? alpha : 0.0);
      vnorm2 += v[r] * v[r];
    }
    rdiag[k] = alpha;
    if (vnorm2 == 0.0) continue;
    // A <- (I - 2 v v^T / |v|^2) A on rows k.., columns k..
    for (int c = k; c < d; ++c) {
      double s = 0.0;
      for (int r = k; r < d; ++r) s += v[r] * a(r, c);
      s *= 2.0 / vnorm2;
      for (int r = k; r < d; ++r) a(r, c) -= s * v[r];
    }
    // Q <- Q (I - 2 v v^T / |v|^2) on columns k..
    for (int r = 0; r < d; ++r) {
      double s = 0.0;
      for (int c = k; c < d; ++c) s += q(r, c) * v[c];
      s *= 2.0 / vnorm2;
      for (int c = k; c < d; ++c) q(r, c) -= s * v[c];
    }
  }
  for (int r = 0; r < d; ++r)
    for (int c = 0; c < d; ++c)
      pi_rowmajor[static_cast<size_t>(r) * d + c] = q(r, c) * (rdiag[c] < 0.0 ? -1.0 : 1.0);
}

uint16_t bf16_bits_rne(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);  // quiet NaN
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return static_cast<uint16_t>(u >> 16);
}

float bf16_bits_to_float(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

bool build_host_tables(int d, int bits, int n_wide, int m, uint64_t rot_seed, uint64_t qjl_seed,
                       HostTables *out, std::string *err) {
  if (d < 2 || d > 4096) {
    *err = "head_dim must be in [2, 4096]";
    return false;
  }
  if (bits < 1 || bits > 4) {
    *err = "mse_bits must be in [1, 4]";
    return false;
  }
  if (m < 0 || m % 32 != 0 || m > 4096) {
    *err = "qjl_dim must be 0 or a positive multiple of 32 (<= 4096)";
    return false;
  }
  if (n_wide < 0 || n_wide > d || (n_wide > 0 && bits > 3)) {
    *err = "wide_coords must be in [0, head_dim], and mse_bits <= 3 when it is positive";
    return false;
  }
  HostTables h;
  h.d = d;
  h.bits = bits;
  h.m = m;
  h.levels = 1 << bits;
  h.n_wide = n_wide;
  int iters = 0;
  lloyd_max_sphere(d, bits, &h.centroids64, &h.thresholds64, &iters);
  // [cc-newplayer explainer, technical breakdown item 1] and [intelliparadigm
  // "3-bit" article, §2.1 and §5.1]: fractional average widths; every rotated
  // coordinate has the same law, so the wide part takes the plain
  // (bits + 1)-bit Lloyd-Max codebook of that law.
  if (n_wide > 0) lloyd_max_sphere(d, bits + 1, &h.wide_centroids64, &h.wide_thresholds64, &iters);
  h.rotation64.resize(static_cast<size_t>(d) * d);
  haar_orthogonal(d, rot_seed, h.rotation64.data());
  if (m > 0) {
    h.qjl64.resize(static_cast<size_t>(m) * d);
    seeded_normals(qjl_seed, h.qjl64.size(), h.qjl64.data());
  }
  auto to_f32 = [](const std::vector<double> &src, std::vector<float> *dst) {
    dst->resize(src.size());
    for (size_t i = 0; i < src.size(); ++i) (*dst)[i] = static_cast<float>(src[i]);
  };
  to_f32(h.centroids64, &h.centroids);
  to_f32(h.thresholds64, &h.thresholds);
  to_f32(h.rotation64, &h.rotation);
  to_f32(h.qjl64, &h.qjl);
  to_f32(h.wide_centroids64, &h.wide_centroids);
  to_f32(h.wide_thresholds64, &h.wide_thresholds);
  *out = std::move(h);
  return true;
}

}  // namespace tq
