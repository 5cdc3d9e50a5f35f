// Host-side setup math for libkvq: Lloyd-Max centroid solver, seeded sign
// generator, row sizes, status strings and the thread-local error text.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"

namespace {

thread_local char g_last_error[512] = "";

// Standard normal density and the probability mass of (a, b], written so that
// cells far out in a tail do not lose digits to cancellation.
double normal_pdf(double x) {
  if (std::isinf(x)) return 0.0;
  return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
}

double upper_tail(double x) { return 0.5 * std::erfc(x / std::sqrt(2.0)); }  // P(X > x)

double cell_probability(double a, double b) {
  if (a >= 0.0) return upper_tail(a) - upper_tail(b);
  if (b <= 0.0) return upper_tail(-b) - upper_tail(-a);
  return 1.0 - upper_tail(-a) - upper_tail(b);
}

// Mean of N(0,1) restricted to (a, b]: integral of x*pdf over the cell is
// pdf(a) - pdf(b); divide by the cell's mass.
double cell_mean(double a, double b) { return (normal_pdf(a) - normal_pdf(b)) / cell_probability(a, b); }

// Start point: the level-centred quantiles of N(0,1), found by bisection.
double normal_quantile(double p) {
  double lo = -12.0, hi = 12.0;
  for (int i = 0; i < 200; ++i) {
    double mid = 0.5 * (lo + hi);
    if (1.0 - upper_tail(mid) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

// Fixed point of the Lloyd map for N(0,1): boundaries at centroid midpoints,
// each centroid the mean of its cell.  The Gaussian density is log-concave, so
// the fixed point is unique and the plain iteration converges to it.  Levels
// are kept exactly antisymmetric.
std::vector<double> gaussian_lloyd_max(int levels) {
  std::vector<double> c(levels), next(levels), edge(levels + 1);
  for (int i = 0; i < levels; ++i) c[i] = normal_quantile((i + 0.5) / levels);
  for (int i = 0; i < levels / 2; ++i) {
    double v = 0.5 * (c[levels - 1 - i] - c[i]);
    c[i] = -v;
    c[levels - 1 - i] = v;
  }
  for (int iter = 0; iter < 1000000; ++iter) {
    edge[0] = -INFINITY;
    edge[levels] = INFINITY;
    for (int i = 1; i < levels; ++i) edge[i] = 0.5 * (c[i - 1] + c[i]);
    double change = 0.0;
    for (int i = 0; i < levels; ++i) next[i] = cell_mean(edge[i], edge[i + 1]);
    for (int i = 0; i < levels / 2; ++i) {
      double v = 0.5 * (next[levels - 1 - i] - next[i]);
      next[i] = -v;
      next[levels - 1 - i] = v;
    }
    for (int i = 0; i < levels; ++i) change = std::fmax(change, std::fabs(next[i] - c[i]));
    c.swap(next);
    if (change < 1e-15) break;
  }
  return c;
}

}  // namespace

namespace kvq {

kvq_status fail(kvq_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_last_error[0] = '\0'; }

bool valid_head_dim(int32_t d) { return d == 64 || d == 128 || d == 256; }

int format_bits(int32_t f) {
  switch (f) {
    case KVQ_LM2: return 2;
    case KVQ_LM3: return 3;
    case KVQ_LM4: return 4;
    case KVQ_FP8_E4M3: return 8;
    default: return 0;
  }
}

}  // namespace kvq

extern "C" {

size_t kvq_row_bytes(int32_t format, int32_t head_dim) {
  int bits = kvq::format_bits(format);
  if (!bits || !kvq::valid_head_dim(head_dim)) return 0;
  return (size_t)head_dim * bits / 8;
}

kvq_status kvq_lloyd_max(int32_t bits, int32_t head_dim, float *centroids_host) {
  kvq::clear_error();
  if (!centroids_host) return kvq::fail(KVQ_EINVAL, "kvq_lloyd_max: centroids_host is NULL");
  if (bits < 1 || bits > 4) return kvq::fail(KVQ_EINVAL, "kvq_lloyd_max: bits=%d not in 1..4", bits);
  if (head_dim < 1) return kvq::fail(KVQ_EINVAL, "kvq_lloyd_max: head_dim=%d", head_dim);
  std::vector<double> g = gaussian_lloyd_max(1 << bits);
  const double root = std::sqrt((double)head_dim);
  for (int i = 0; i < (1 << bits); ++i) centroids_host[i] = (float)(g[i] / root);
  return KVQ_OK;
}

kvq_status kvq_make_signs(uint64_t seed, int32_t head_dim, int8_t *signs_host) {
  kvq::clear_error();
  if (!signs_host) return kvq::fail(KVQ_EINVAL, "kvq_make_signs: signs_host is NULL");
  if (head_dim < 1) return kvq::fail(KVQ_EINVAL, "kvq_make_signs: head_dim=%d", head_dim);
  uint64_t state = seed;
  for (int32_t j = 0; j < head_dim; ++j) {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    signs_host[j] = (z >> 63) ? -1 : 1;
  }
  return KVQ_OK;
}

size_t kvq_partials_floats(int32_t batch, int32_t q_heads, int32_t total_splits, int32_t head_dim) {
  if (batch < 0 || q_heads < 0 || total_splits < 0 || head_dim < 0) return 0;
  return (size_t)batch * q_heads * total_splits * head_dim;
}

const char *kvq_status_string(kvq_status status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument";
    case KVQ_EUNSUPPORTED: return "unsupported configuration";
    case KVQ_ERANGE: return "token range outside cache capacity";
    case KVQ_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *kvq_last_error(void) { return g_last_error; }

}  // extern "C"
