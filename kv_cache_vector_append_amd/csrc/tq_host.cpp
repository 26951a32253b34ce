// Host-side construction of the parameter blob: Lloyd-Max codebooks for the
// rotated-coordinate density, the seeded Rademacher signs, and (dense variant)
// the Haar rotations and the Gaussian QJL matrix.
//
// [Reconstruction] = "Mathematical Reconstruction, Lineage, and Accuracy Limits
// of TurboQuant and TurboVec"; [Design Study] = "TurboQuant Family Design
// Study for CPU and Browser WASM KV Caches".
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "tq_internal.h"

namespace tqi {
namespace {

// ------------------------------------------------------------------ PRNG
// SplitMix64 in counter form: out(k) = mix(seed + (k + 1) * golden_gamma)
// (Steele, Lea and Flood 2014; 64-bit finaliser of Vigna's splitmix64.c).
// Stream layout: counter = (role << 48) | index.
constexpr uint64_t kGoldenGamma = 0x9E3779B97F4A7C15ull;
enum Role : uint64_t { kKeySigns = 0, kSketchSigns1 = 1, kSketchSigns2 = 2, kValueSigns = 3,
                       kKeyGauss = 4, kSketchGauss = 5, kValueGauss = 6 };

uint64_t splitmix64(uint64_t seed, uint64_t counter) {
  uint64_t z = seed + (counter + 1) * kGoldenGamma;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t ctr(uint64_t role, uint64_t i) { return (role << 48) | i; }

// Box-Muller (Box and Muller, 1958): element 2k = r cos(2 pi u2), 2k+1 = r sin(2 pi u2),
// u1 = (top53(out(2k)) + 1) 2^-53 in (0, 1], u2 = top53(out(2k+1)) 2^-53.
std::vector<double> gaussian(uint64_t seed, uint64_t role, int rows, int cols) {
  const int n = rows * cols;
  std::vector<double> g(n);
  for (int k = 0; 2 * k < n; ++k) {
    const double u1 = (double((splitmix64(seed, ctr(role, 2 * k)) >> 11)) + 1.0) * 0x1.0p-53;
    const double u2 = double(splitmix64(seed, ctr(role, 2 * k + 1)) >> 11) * 0x1.0p-53;
    const double r = std::sqrt(-2.0 * std::log(u1));
    g[2 * k] = r * std::cos(2.0 * M_PI * u2);
    if (2 * k + 1 < n) g[2 * k + 1] = r * std::sin(2.0 * M_PI * u2);
  }
  return g;
}

// Householder QR of a square row-major matrix; returns Q * diag(sign(diag R)),
// the unique orthogonal factor whose R has a positive diagonal
// ([Reconstruction] section 5 "Step 2": QR of a standard Gaussian matrix).
std::vector<double> haar_from_gaussian(std::vector<double> a, int d) {
  std::vector<double> q(size_t(d) * d, 0.0);
  for (int i = 0; i < d; ++i) q[size_t(i) * d + i] = 1.0;
  std::vector<double> v(d);
  for (int k = 0; k < d; ++k) {
    double norm2 = 0.0;
    for (int i = k; i < d; ++i) norm2 += a[size_t(i) * d + k] * a[size_t(i) * d + k];
    const double norm = std::sqrt(norm2);
    if (norm == 0.0) continue;
    const double x0 = a[size_t(k) * d + k];
    const double alpha = x0 >= 0 ? -norm : norm;  // reflect x onto alpha e_k
    for (int i = k; i < d; ++i) v[i] = a[size_t(i) * d + k];
    v[k] -= alpha;
    double vv = 0.0;
    for (int i = k; i < d; ++i) vv += v[i] * v[i];
    if (vv == 0.0) continue;
    // A <- (I - 2 v v^T / v^T v) A on rows k.., columns k..
    for (int j = k; j < d; ++j) {
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += v[i] * a[size_t(i) * d + j];
      const double f = 2.0 * dot / vv;
      for (int i = k; i < d; ++i) a[size_t(i) * d + j] -= f * v[i];
    }
    // Q <- Q (I - 2 v v^T / v^T v) on columns k..
    for (int i = 0; i < d; ++i) {
      double dot = 0.0;
      for (int j = k; j < d; ++j) dot += q[size_t(i) * d + j] * v[j];
      const double f = 2.0 * dot / vv;
      for (int j = k; j < d; ++j) q[size_t(i) * d + j] -= f * v[j];
    }
  }
  for (int j = 0; j < d; ++j) {
    if (a[size_t(j) * d + j] < 0) {
      for (int i = 0; i < d; ++i) q[size_t(i) * d + j] = -q[size_t(i) * d + j];
    }
  }
  return q;
}

// ------------------------------------------------------------------ codebook
// Density of one coordinate of a uniform point on S^{d-1}:
//   f_d(x) = (1 - x^2)^((d-3)/2) / B(1/2, (d-1)/2),  (1 + x)/2 ~ Beta(a, a), a = (d-1)/2
// ([Reconstruction] section 5 "Step 2": scaled Beta marginal).

double log_beta(double a, double b) { return std::lgamma(a) + std::lgamma(b) - std::lgamma(a + b); }

// Continued fraction of the regularised incomplete beta function evaluated by
// the modified Lentz method:
//   I_x(a,b) = x^a (1-x)^b / (a B(a,b)) * 1/(1 + e1/(1 + e2/(1 + ...))),
//   e_{2m+1} = -(a+m)(a+b+m) x / ((a+2m)(a+2m+1)),  e_{2m} = m(b-m) x / ((a+2m-1)(a+2m)).
double beta_cf(double a, double b, double x) {
  const double tiny = 1e-300;
  double c = 1.0;
  double dd = 1.0 - (a + b) * x / (a + 1.0);
  if (std::fabs(dd) < tiny) dd = tiny;
  dd = 1.0 / dd;
  double h = dd;
  for (int m = 1; m < 10000; ++m) {
    const double m2 = 2.0 * m;
    double e = m * (b - m) * x / ((a + m2 - 1.0) * (a + m2));
    dd = 1.0 + e * dd;
    if (std::fabs(dd) < tiny) dd = tiny;
    c = 1.0 + e / c;
    if (std::fabs(c) < tiny) c = tiny;
    dd = 1.0 / dd;
    h *= dd * c;
    e = -(a + m) * (a + b + m) * x / ((a + m2) * (a + m2 + 1.0));
    dd = 1.0 + e * dd;
    if (std::fabs(dd) < tiny) dd = tiny;
    c = 1.0 + e / c;
    if (std::fabs(c) < tiny) c = tiny;
    dd = 1.0 / dd;
    const double del = dd * c;
    h *= del;
    if (std::fabs(del - 1.0) < 1e-16) break;
  }
  return h;
}

double reg_inc_beta(double a, double b, double x) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  const double front = std::exp(a * std::log(x) + b * std::log1p(-x) - log_beta(a, b));
  if (x < (a + 1.0) / (a + b + 2.0)) return front * beta_cf(a, b, x) / a;
  return 1.0 - front * beta_cf(b, a, 1.0 - x) / b;
}

struct Marginal {
  double a, log_norm;  // log((d-1) B(1/2, a))
  int d;
  explicit Marginal(int d_) : a((d_ - 1) / 2.0), d(d_) { log_norm = std::log(double(d_ - 1)) + log_beta(0.5, a); }
  double cdf(double x) const {
    if (x <= -1.0) return 0.0;
    if (x >= 1.0) return 1.0;
    return reg_inc_beta(a, a, 0.5 * (1.0 + x));
  }
  // antiderivative of x f_d(x): -(1-x^2)^((d-1)/2) / ((d-1) B(1/2, a))
  double moment(double x) const {
    if (x <= -1.0 || x >= 1.0) return 0.0;
    return -std::exp(a * std::log1p(-x * x) - log_norm);
  }
};

// Lloyd-Max iteration ([Reconstruction] "Step 4: Lloyd-Max Boundaries and
// Centroids"): boundaries at centroid midpoints, centroids at the conditional
// means of their cells, until the largest move is below 1e-14 of the largest
// centroid.  The density is even, so the codebook is kept odd.
std::vector<double> lloyd_max(int d, int bits) {
  const int L = 1 << bits;
  const Marginal f(d);
  std::vector<double> c(L), cn(L), edges(L + 1);
  // start: a uniform grid over +-2.5 standard deviations of N(0, 1/d)
  for (int j = 0; j < L; ++j) c[j] = (2.0 * j + 1.0 - L) / L * 2.5 / std::sqrt(double(d));
  for (int it = 0; it < 100000; ++it) {
    edges[0] = -1.0;
    edges[L] = 1.0;
    for (int j = 1; j < L; ++j) edges[j] = 0.5 * (c[j - 1] + c[j]);
    for (int j = 0; j < L; ++j) {
      const double mass = f.cdf(edges[j + 1]) - f.cdf(edges[j]);
      const double mom = f.moment(edges[j + 1]) - f.moment(edges[j]);
      cn[j] = mom / mass;
    }
    double delta = 0.0, cmax = 0.0;
    for (int j = 0; j < L; ++j) {
      const double v = 0.5 * (cn[j] - cn[L - 1 - j]);
      delta = std::fmax(delta, std::fabs(v - c[j]));
      cmax = std::fmax(cmax, std::fabs(v));
    }
    for (int j = 0; j < L; ++j) c[j] = 0.5 * (cn[j] - cn[L - 1 - j]);
    if (delta < 1e-14 * cmax) break;
  }
  return c;
}

void write_codebook(uint8_t* blob, int off_c, int off_t, int off_coef, int d, int bits) {
  const int L = 1 << bits;
  const std::vector<double> c = lloyd_max(d, bits);
  float* cf = reinterpret_cast<float*>(blob + off_c);
  float* tf = reinterpret_cast<float*>(blob + off_t);
  float* af = reinterpret_cast<float*>(blob + off_coef);
  for (int j = 0; j < 16; ++j) {
    cf[j] = j < L ? float(c[j]) : 0.0f;
    tf[j] = j + 1 < L ? float(0.5 * (c[j] + c[j + 1])) : INFINITY;
  }
  for (int S = 0; S < 16; ++S) {
    double acc = 0.0;
    if (S < L) {
      for (int idx = 0; idx < L; ++idx) {
        double sgn = 1.0;
        for (int k = 0; k < bits; ++k)
          if ((S >> k) & 1) sgn *= ((idx >> k) & 1) ? -1.0 : 1.0;
        acc += c[idx] * sgn;
      }
      acc /= L;
    }
    af[S] = float(acc);
  }
}

void write_signs(uint8_t* blob, uint64_t seed, int d) {
  const uint64_t roles[4] = {kKeySigns, kSketchSigns1, kSketchSigns2, kValueSigns};
  for (int r = 0; r < 4; ++r) {
    uint32_t* w = reinterpret_cast<uint32_t*>(blob + kOffSigns + r * kSignRoleBytes);
    for (int i = 0; i < d / 32; ++i) {
      const uint64_t word = splitmix64(seed, ctr(roles[r], uint64_t(i / 2)));
      w[i] = uint32_t(word >> (32 * (i & 1)));
    }
  }
}

}  // namespace

// Context splits per (sequence, KV head): enough work items to fill the
// chip's resident wavefront slots (two per SIMD, 1024 SIMDs) and no more, each
// a whole number of tiles (the matrix-core kernel's 128-token blocks, the
// plain kernel's 64-token tiles).
SplitPlan plan_splits(const tq_config& cfg, int num_seqs, int max_ctx) {
  const bool mfma = decode_mfma_supported(cfg);
  const int units = (num_seqs > 0 ? num_seqs : 1) * cfg.num_kv_heads;
  const int tile = mfma ? 128 : 64;
  const int items = mfma ? decode_mfma_items(cfg) : 2048;
  // 64-bit arithmetic: max_ctx may be up to TQ_MAX_CONTEXT
  const long long ctx = max_ctx > 0 ? max_ctx : 1;
  const long long max_tiles = (ctx + tile - 1) / tile;
  long long splits = (items + units - 1) / units;
  if (splits > max_tiles) splits = max_tiles;
  if (splits > kMaxSplits) splits = kMaxSplits;
  if (splits < 1) splits = 1;
  const long long per = (ctx + splits - 1) / splits;
  long long split_tokens = ((per + tile - 1) / tile) * tile;
  if (split_tokens < tile) split_tokens = tile;
  splits = (ctx + split_tokens - 1) / split_tokens;
  if (splits < 1) splits = 1;
  // The window's items run after the compressed ones: kWindowRecords short
  // ones per (sequence, KV head) where they fit in the slots the compressed
  // items leave, else one (the compressed items already fill the GPU).
  const int window_items = units * kWindowRecords <= items ? kWindowRecords : 1;
  return {int(splits), int(split_tokens), window_items};
}

Codec make_codec(const tq_config& c) {
  Codec k{};
  const int d = c.head_dim, P = c.page_tokens;
  k.key_mode = c.key_mode;
  k.value_mode = c.value_mode;
  k.qjl = c.key_mode == TQ_KEY_QJL ? 1 : 0;
  k.kbits[0] = c.key_bits - k.qjl;
  k.kbits[1] = (c.key_bits_hi ? c.key_bits_hi : c.key_bits) - k.qjl;
  k.vbits[0] = c.value_bits;
  k.vbits[1] = c.value_bits_hi ? c.value_bits_hi : c.value_bits;
  k.outliers = c.key_outliers;
  k.ext = c.key_mode != TQ_KEY_QJL || c.value_mode != TQ_VALUE_LLOYD || k.kbits[0] != k.kbits[1] ||
          k.vbits[0] != k.vbits[1] || c.key_outliers != 0;
  const int half_groups = d / (2 * kGroup);
  k.key_row_words = half_groups * (k.kbits[0] + k.qjl) + half_groups * (k.kbits[1] + k.qjl);
  k.key_norm_off = 4 * P * k.key_row_words;
  k.key_side_off = k.key_norm_off + 8 * P;
  k.side_val_off = 1 + k.outliers + ((1 + k.outliers) & 1);
  k.side_bytes = k.outliers ? (k.side_val_off + 2 * k.outliers + 3) / 4 * 4 : 0;
  k.key_block = k.key_side_off + P * k.side_bytes;
  k.value_words = (d / 4) * (k.vbits[0] + k.vbits[1]);
  k.value_tail_off = 4 * k.value_words;
  k.value_block = k.value_tail_off + (c.value_mode == TQ_VALUE_GROUP ? P * (d / kGroup) * 4 : 4 * P);
  return k;
}

void build_params(const tq_config& cfg, uint8_t* blob) {
  const int d = cfg.head_dim;
  const Codec k = make_codec(cfg);
  std::memset(blob, 0, params_bytes(d, cfg.rotation));
  ParamsHeader h{};
  h.magic = kParamsMagic;
  h.version = 2;
  h.head_dim = d;
  h.key_mse_bits = k.kbits[0];
  h.value_bits = k.vbits[0];
  h.rotation = cfg.rotation;
  h.seed = cfg.seed;
  h.total_bytes = uint32_t(params_bytes(d, cfg.rotation));
  h.key_mse_bits_hi = k.kbits[1];
  h.value_bits_hi = k.vbits[1];
  h.key_mode = cfg.key_mode;
  h.value_mode = cfg.value_mode;
  h.key_outliers = cfg.key_outliers;
  std::memcpy(blob, &h, sizeof(h));
  for (int half = 0; half < 2; ++half) {
    const int o = half ? kOffUpperHalf : 0;
    write_codebook(blob, kOffKeyCentroids + o, kOffKeyThresholds + o, kOffKeyPlaneCoef + o, d, k.kbits[half]);
    write_codebook(blob, kOffValueCentroids + o, kOffValueThresholds + o, kOffValuePlaneCoef + o, d, k.vbits[half]);
  }
  write_signs(blob, cfg.seed, d);
  if (cfg.rotation == TQ_ROT_DENSE) {
    float* dst = reinterpret_cast<float*>(blob + kOffDense);
    const uint64_t roles[3] = {kKeyGauss, kSketchGauss, kValueGauss};
    std::vector<double> exact[2];  // Pi_K and G in double, for the query preparation's matrices
    for (int m = 0; m < 3; ++m) {
      std::vector<double> g = gaussian(cfg.seed, roles[m], d, d);
      if (m != 1) g = haar_from_gaussian(std::move(g), d);
      for (size_t i = 0; i < size_t(d) * d; ++i) dst[size_t(m) * d * d + i] = float(g[i]);
      if (m < 2) exact[m] = g;
      if (m > 0) {  // G^T and Pi_V^T for the short appends
        float* t = reinterpret_cast<float*>(blob + dense_t_offset(d, m + 1));
        for (int r = 0; r < d; ++r)
          for (int c = 0; c < d; ++c) t[size_t(c) * d + r] = dst[size_t(m) * d * d + size_t(r) * d + c];
      }
      // fp16 hi / lo split of the scaled fp32 matrix for the matrix cores
      _Float16* hi = reinterpret_cast<_Float16*>(blob + dense16_offset(d, m));
      _Float16* lo = hi + size_t(d) * d;
      for (size_t i = 0; i < size_t(d) * d; ++i) {
        const float v = dst[size_t(m) * d * d + i] * kDense16Scale[m];
        hi[i] = _Float16(v);
        lo[i] = _Float16(v - float(hi[i]));
      }
    }
    // The query preparation's matrices, transposed: Pi_K^T, and (G Pi_K)^T,
    // which maps the query straight to its sketch (qh = G Pi_K q), formed in
    // double and rounded once.
    float* t0 = reinterpret_cast<float*>(blob + dense_t_offset(d, 0));
    float* t1 = reinterpret_cast<float*>(blob + dense_t_offset(d, 1));
    std::vector<double> row(d);
    for (int r = 0; r < d; ++r) {
      std::fill(row.begin(), row.end(), 0.0);
      for (int k = 0; k < d; ++k) {
        const double gk = exact[1][size_t(r) * d + k];
        const double* pk = exact[0].data() + size_t(k) * d;
        for (int c = 0; c < d; ++c) row[c] += gk * pk[c];
      }
      for (int c = 0; c < d; ++c) {
        t0[size_t(c) * d + r] = float(exact[0][size_t(r) * d + c]);
        t1[size_t(c) * d + r] = float(row[c]);
      }
    }
  }
}

}  // namespace tqi
