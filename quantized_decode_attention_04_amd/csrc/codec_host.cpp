// Host-side codec builder: deterministic in (head_dim, bits, seed, mode).
//
// The pages fix that TurboQuant rotates each head vector with a seeded random
// orthogonal matrix and maps each rotated coordinate to a Lloyd-Max centroid,
// and that the codec is rebuilt from (head_dim, bits, seed) alone
// ("omlx turboquant_kv.py", _rebuild_codecs); Prod keys add a d x d QJL
// matrix S ("turboquant validate_moe_phase2.py", Test 2).  The generator,
// factorisation and density are this library's reading:
//   * standard normals: counter-based SplitMix64 (Steele, Lea & Flood 2014)
//     feeding Box-Muller; stream s of a seed starts at seed XOR s*GAMMA;
//     stream 0 is the rotation's Gaussian, stream 1 is S (stream 2: the
//     high part's rotation of a split codec); row-major fill;
//   * rotation: Householder QR G = QR, Pi = Q diag(sign R_ii) (positive
//     diagonal, unique), y = Pi x;
//   * codebook: Lloyd-Max for the density of one coordinate of a uniform unit
//     vector in R^d, f(y) ~ (1 - y^2)^((d-3)/2), cell masses by composite
//     Gauss-Legendre quadrature, first moments in closed form; then made odd
//     symmetric and rounded onto the grid 2^-E (largest E with
//     max|c| 2^E <= 16256); boundaries are midpoints of the stored values.
#include <cmath>
#include <cstring>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ULL;

uint64_t splitmix_out(uint64_t state) {
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

// n standard normals (n even) of stream `stream` of `seed`.
void standard_normals(uint64_t seed, uint64_t stream, size_t n, std::vector<double>& out) {
  out.resize(n);
  const uint64_t start = seed ^ (stream * kGamma);
  const double two_pi = 2.0 * M_PI;
  for (size_t i = 0; i < n; i += 2) {
    const uint64_t a = splitmix_out(start + (uint64_t)(i + 1) * kGamma);
    const uint64_t b = splitmix_out(start + (uint64_t)(i + 2) * kGamma);
    const double u1 = ((double)(a >> 11) + 1.0) * 0x1p-53;
    const double u2 = ((double)(b >> 11) + 1.0) * 0x1p-53;
    const double r = std::sqrt(-2.0 * std::log(u1));
    const double th = two_pi * u2;
    out[i] = r * std::cos(th);
    out[i + 1] = r * std::sin(th);
  }
}

// Householder QR of the row-major d x d matrix g; returns Q diag(sign R_ii).
std::vector<double> orthogonal_factor(const std::vector<double>& g, int d) {
  std::vector<double> a(g);
  std::vector<double> vs((size_t)d * d, 0.0);  // Householder vector k in row k (entries k..d-1)
  std::vector<double> vn2(d, 0.0), rdiag(d, 0.0);
  for (int k = 0; k < d; ++k) {
    double nrm2 = 0.0;
    for (int i = k; i < d; ++i) nrm2 += a[(size_t)i * d + k] * a[(size_t)i * d + k];
    const double nrm = std::sqrt(nrm2);
    const double x0 = a[(size_t)k * d + k];
    const double alpha = x0 > 0.0 ? -nrm : nrm;
    double* v = &vs[(size_t)k * d];
    for (int i = k; i < d; ++i) v[i] = a[(size_t)i * d + k];
    v[k] -= alpha;
    double s = 0.0;
    for (int i = k; i < d; ++i) s += v[i] * v[i];
    vn2[k] = s;
    rdiag[k] = alpha;
    if (s == 0.0) { rdiag[k] = x0; continue; }
    for (int j = k; j < d; ++j) {
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += v[i] * a[(size_t)i * d + j];
      const double f = 2.0 * dot / s;
      for (int i = k; i < d; ++i) a[(size_t)i * d + j] -= f * v[i];
    }
  }
  // Q = H_0 H_1 ... H_{d-1}: apply to the identity from the last reflector on.
  std::vector<double> q((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) q[(size_t)i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    if (vn2[k] == 0.0) continue;
    const double* v = &vs[(size_t)k * d];
    for (int j = 0; j < d; ++j) {
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += v[i] * q[(size_t)i * d + j];
      const double f = 2.0 * dot / vn2[k];
      for (int i = k; i < d; ++i) q[(size_t)i * d + j] -= f * v[i];
    }
  }
  for (int j = 0; j < d; ++j) {
    if (rdiag[j] < 0.0)
      for (int i = 0; i < d; ++i) q[(size_t)i * d + j] = -q[(size_t)i * d + j];
  }
  return q;
}

// Gauss-Legendre nodes and weights on [-1, 1] (Newton on P_n).
struct GaussLegendre {
  static constexpr int n = 20;
  double x[n], w[n];
  GaussLegendre() {
    for (int i = 0; i < n; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
      double dp = 0.0;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= n; ++k) {
          const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        dp = n * (z * p1 - p0) / (z * z - 1.0);
        const double dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-16) break;
      }
      double p0 = 1.0, p1 = z;
      for (int k = 2; k <= n; ++k) {
        const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = p2;
      }
      dp = n * (z * p1 - p0) / (z * z - 1.0);
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

struct SphereCoordinate {
  int d;
  double a;     // (d-1)/2
  double logc;  // log of 1/B(1/2, a)
  const GaussLegendre& gl;
  SphereCoordinate(int d_, const GaussLegendre& g) : d(d_), a((d_ - 1) / 2.0), gl(g) {
    logc = std::lgamma(d / 2.0) - std::lgamma(a) - 0.5 * std::log(M_PI);
  }
  double density(double y) const { return std::exp((a - 1.0) * std::log1p(-y * y) + logc); }
  double mass(double lo, double hi) const {
    const int panels = 48;
    const double h = (hi - lo) / panels;
    double s = 0.0;
    for (int p = 0; p < panels; ++p) {
      const double c = lo + (p + 0.5) * h;
      double ps = 0.0;
      for (int i = 0; i < GaussLegendre::n; ++i) ps += gl.w[i] * density(c + 0.5 * h * gl.x[i]);
      s += 0.5 * h * ps;
    }
    return s;
  }
  // int_lo^hi y f(y) dy = C [(1-lo^2)^a - (1-hi^2)^a] / (2a)
  double first_moment(double lo, double hi) const {
    const double plo = lo <= -1.0 || lo >= 1.0 ? 0.0 : std::exp(a * std::log1p(-lo * lo));
    const double phi = hi <= -1.0 || hi >= 1.0 ? 0.0 : std::exp(a * std::log1p(-hi * hi));
    return std::exp(logc) * (plo - phi) / (2.0 * a);
  }
};

void lloyd_max(int d, int bits, std::vector<double>& c) {
  static const GaussLegendre gl;
  const SphereCoordinate f(d, gl);
  const int L = 1 << bits;
  c.resize(L);
  for (int k = 0; k < L; ++k) c[k] = (2.0 * k + 1.0 - L) / L * (2.5 / std::sqrt((double)d));
  std::vector<double> nxt(L);
  for (int it = 0; it < 20000; ++it) {
    double step = 0.0;
    for (int k = 0; k < L; ++k) {
      const double lo = k == 0 ? -1.0 : 0.5 * (c[k - 1] + c[k]);
      const double hi = k == L - 1 ? 1.0 : 0.5 * (c[k] + c[k + 1]);
      nxt[k] = f.first_moment(lo, hi) / f.mass(lo, hi);
      step = std::fmax(step, std::fabs(nxt[k] - c[k]));
    }
    c.swap(nxt);
    if (step <= 1e-14) break;
  }
  std::vector<double> sym(L);
  for (int k = 0; k < L; ++k) sym[k] = 0.5 * (c[k] - c[L - 1 - k]);
  c.swap(sym);
}

}  // namespace

bool build_codec(int d, int bits, uint64_t seed, int mode, HostCodec* out, std::string* err, int rot_stream) {
  if (d < 32 || d > 256 || d % 32 != 0) {
    *err = "head_dim must be a multiple of 32 in [32, 256]";
    return false;
  }
  HostCodec h;
  h.d = d;
  h.bits = bits;
  h.mode = mode;
  h.seed = seed;
  if (mode == TQ_MODE_GROUP) {
    if (bits < 1 || bits > 4) {
      *err = "group mode supports 1..4 bits";
      return false;
    }
    h.mse_bits = bits;
    h.levels = 0;
    *out = std::move(h);
    return true;
  }
  if (mode != TQ_MODE_MSE && mode != TQ_MODE_PROD) {
    *err = "unknown mode";
    return false;
  }
  h.mse_bits = mode == TQ_MODE_PROD ? bits - 1 : bits;
  if (h.mse_bits < 1 || h.mse_bits > 4) {
    *err = mode == TQ_MODE_PROD ? "Prod mode supports 2..5 bits" : "MSE mode supports 1..4 bits";
    return false;
  }
  h.levels = 1 << h.mse_bits;

  std::vector<double> g;
  standard_normals(seed, (uint64_t)rot_stream, (size_t)d * d, g);
  const std::vector<double> pi = orthogonal_factor(g, d);
  h.rot.resize((size_t)d * d);
  for (size_t i = 0; i < pi.size(); ++i) h.rot[i] = (float)pi[i];

  if (mode == TQ_MODE_PROD) {
    std::vector<double> s;
    standard_normals(seed, 1, (size_t)d * d, s);
    h.sketch.resize(s.size());
    for (size_t i = 0; i < s.size(); ++i) h.sketch[i] = (float)s[i];
  }

  std::vector<double> c;
  lloyd_max(d, h.mse_bits, c);
  double m = 0.0;
  for (double v : c) m = std::fmax(m, std::fabs(v));
  int e = (int)std::floor(std::log2(kGridMax / m));
  while (std::ldexp(m, e + 1) <= kGridMax) ++e;
  while (std::ldexp(m, e) > kGridMax) --e;
  h.grid_exp = e;
  h.centroids.resize(h.levels);
  for (int k = 0; k < h.levels; ++k) h.centroids[k] = (float)std::ldexp(std::nearbyint(std::ldexp(c[k], e)), -e);
  h.boundaries.resize(h.levels - 1);
  for (int k = 0; k + 1 < h.levels; ++k)
    h.boundaries[k] = (float)(0.5 * ((double)h.centroids[k] + (double)h.centroids[k + 1]));
  *out = std::move(h);
  return true;
}

}  // namespace tq
