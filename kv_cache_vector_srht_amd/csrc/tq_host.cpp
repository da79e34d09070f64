// Host-only part of libtq: codebooks, layer randomness, sizes, validation,
// status strings.  No HIP calls here, so every function works without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "tq_internal.h"

namespace tq {

static thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return TQ_OK;
}

// ---------------------------------------------------------------------------
// Gaussian helpers in long double (64-bit mantissa on x86-64).
// ---------------------------------------------------------------------------
typedef long double ld;
static const ld kInvSqrt2Pi = 0.398942280401432677939946059934381868L;
static const ld kInvSqrt2 = 0.707106781186547524400844362104849039L;

static ld pdf(ld x) { return isinf(x) ? 0.0L : kInvSqrt2Pi * expl(-0.5L * x * x); }
// Upper tail P(Z >= x), accurate for large positive x.
static ld upper(ld x) { return isinf(x) ? (x > 0 ? 0.0L : 1.0L) : 0.5L * erfcl(x * kInvSqrt2); }

// Densities the Lloyd-Max quantiser is solved for.  Each gives, for x >= 0,
// the density f(x), the upper tail P(X >= x), and the partial first moment
// E[X; X >= x] (for N(0,1) this is f(x) itself); `end` is the top of the
// support.
struct GaussianModel {
  ld end() const { return INFINITY; }
  ld density(ld x) const { return pdf(x); }
  ld tail(ld x) const { return upper(x); }
  ld moment(ld x) const { return pdf(x); }
};

// Regularised incomplete beta I_x(a, b) from the continued fraction of
// Abramowitz & Stegun 26.5.8,
//   I_x(a, b) = x^a (1-x)^b / (a B(a, b)) * 1 / (1 + d1 / (1 + d2 / (1 + ...))),
//   d(2m+1) = -(a+m)(a+b+m) x / ((a+2m)(a+2m+1)),  d(2m) = m(b-m) x / ((a+2m-1)(a+2m)),
// evaluated front to back with the modified Lentz method, on the side of the
// symmetry I_x(a, b) = 1 - I_{1-x}(b, a) where the fraction converges fast.
// log Gamma(x) for x > 0.  lgammal also stores the sign of Gamma in the
// process-wide signgam, a data race between host threads; lgammal_r returns
// it through an argument instead.
static ld log_gamma(ld x) {
  int sign = 0;
  return lgammal_r(x, &sign);
}

static ld incomplete_beta(ld a, ld b, ld x) {
  if (x <= 0.0L) return 0.0L;
  if (x >= 1.0L) return 1.0L;
  if (x > (a + 1.0L) / (a + b + 2.0L)) return 1.0L - incomplete_beta(b, a, 1.0L - x);
  const ld tiny = 1e-4000L;
  auto guard = [&](ld v) { return fabsl(v) < tiny ? tiny : v; };
  // value = 1 / (1 + d1 / (1 + d2 / ...)): C_k, D_k of the Lentz recurrences
  ld C = 1.0L;
  ld Dk = 1.0L / guard(1.0L - (a + b) * x / (a + 1.0L));   // 1 + d1
  ld value = Dk;
  for (int m = 1; m < 5000; ++m) {
    const ld even = (ld)m * (b - (ld)m) * x / ((a + 2 * m - 1) * (a + 2 * m));
    Dk = 1.0L / guard(1.0L + even * Dk);
    C = guard(1.0L + even / C);
    value *= Dk * C;
    const ld odd = -(a + m) * (a + b + m) * x / ((a + 2 * m) * (a + 2 * m + 1));
    Dk = 1.0L / guard(1.0L + odd * Dk);
    C = guard(1.0L + odd / C);
    const ld step = Dk * C;
    value *= step;
    if (fabsl(step - 1.0L) < 1e-21L) break;
  }
  const ld lfront = a * logl(x) + b * log1pl(-x) - (log_gamma(a) + log_gamma(b) - log_gamma(a + b)) - logl(a);
  return expl(lfront) * value;
}

// One coordinate of sqrt(d) times a uniformly random unit vector of R^d (the
// distribution a rotated, normalised head vector's coordinate has when its
// direction is random): f(u) = c (1 - u^2/d)^((d-3)/2) on |u| < sqrt(d), with
// c = Gamma(d/2) / (sqrt(pi d) Gamma((d-1)/2)); u^2/d ~ Beta(1/2, (d-1)/2).
struct SphereModel {
  ld d, c;
  explicit SphereModel(int dim) : d((ld)dim) {
    c = expl(log_gamma(0.5L * d) - log_gamma(0.5L * (d - 1.0L))) / sqrtl(3.14159265358979323846264338327950288L * d);
  }
  ld end() const { return sqrtl(d); }
  ld density(ld x) const {
    const ld y = 1.0L - x * x / d;
    return y <= 0.0L ? 0.0L : c * powl(y, 0.5L * (d - 3.0L));
  }
  ld tail(ld x) const {
    const ld y = 1.0L - x * x / d;
    return y <= 0.0L ? 0.0L : 0.5L * incomplete_beta(0.5L * (d - 1.0L), 0.5L, y);
  }
  ld moment(ld x) const {
    // integral of u f(u) from x to sqrt(d)
    const ld y = 1.0L - x * x / d;
    return y <= 0.0L ? 0.0L : c * d / (d - 1.0L) * powl(y, 0.5L * (d - 1.0L));
  }
};

// The Rayleigh(1) law of the radius of a standard 2-D Gaussian pair:
// f(r) = r exp(-r^2/2), P(R >= x) = exp(-x^2/2),
// E[R; R >= x] = x exp(-x^2/2) + sqrt(2 pi) P(Z >= x).
struct RayleighModel {
  ld end() const { return INFINITY; }
  ld density(ld x) const { return isinf(x) ? 0.0L : x * expl(-0.5L * x * x); }
  ld tail(ld x) const { return isinf(x) ? 0.0L : expl(-0.5L * x * x); }
  ld moment(ld x) const {
    return isinf(x) ? 0.0L : x * expl(-0.5L * x * x) + 2.50662827463100050241576528481104525L * upper(x);
  }
};

// Lloyd-Max quantiser of a symmetric density with L = 2^bits levels.  By
// symmetry only the positive centroids c[0..h-1] (h = L/2) are unknowns; cell i
// of the positive half is [a_i, b_i) with a_0 = 0, a_i = (c[i-1] + c[i]) / 2,
// b_i = a_{i+1}, b_{h-1} = the end of the support, and the conditions are
// c[i] = E[X | a_i <= X < b_i].  Solved by a few Lloyd sweeps followed by
// Newton's method with the exact tridiagonal Jacobian (Thomas algorithm), all
// in long double.
template <class Model>
static void lloyd_max(int bits, const Model& M, std::vector<ld>& cpos) {
  const int h = 1 << (bits - 1);
  cpos.assign(h, 0.0L);
  // Start: centroids of equal-probability cells of N(0, 3) (companding shape).
  for (int i = 0; i < h; ++i) {
    // bisection for the quantile of (h + i + 0.5) / (2h) of N(0, 3)
    ld p = (ld)(h + i) + 0.5L;
    p /= (ld)(2 * h);
    ld lo = 0.0L, hi = 20.0L;
    for (int it = 0; it < 200; ++it) {
      ld mid = 0.5L * (lo + hi);
      if (1.0L - upper(mid / sqrtl(3.0L)) < p) lo = mid; else hi = mid;
    }
    cpos[i] = std::min(0.5L * (lo + hi), M.end() * (ld)(i + 1) / (ld)(h + 1));
  }
  auto cond_means = [&](const std::vector<ld>& c, std::vector<ld>& m,
                        std::vector<ld>* dm_da, std::vector<ld>* dm_db) {
    for (int i = 0; i < h; ++i) {
      ld a = i == 0 ? 0.0L : 0.5L * (c[i - 1] + c[i]);
      ld b = i == h - 1 ? M.end() : 0.5L * (c[i] + c[i + 1]);
      ld P = M.tail(a) - M.tail(b);
      ld mean = (M.moment(a) - M.moment(b)) / P;
      m[i] = mean;
      if (dm_da) (*dm_da)[i] = M.density(a) * (mean - a) / P;
      if (dm_db) (*dm_db)[i] = i == h - 1 ? 0.0L : M.density(b) * (b - mean) / P;
    }
  };
  std::vector<ld> m(h), da(h), db(h);
  for (int it = 0; it < 300; ++it) {
    cond_means(cpos, m, nullptr, nullptr);
    cpos = m;
  }
  // Newton on F(c) = c - m(c).
  std::vector<ld> lower(h), diag(h), upperd(h), rhs(h);
  for (int it = 0; it < 100; ++it) {
    cond_means(cpos, m, &da, &db);
    ld maxstep = 0.0L;
    for (int i = 0; i < h; ++i) {
      rhs[i] = -(cpos[i] - m[i]);
      // m_i depends on a_i (through c[i-1], c[i]) for i > 0 and on b_i
      // (through c[i], c[i+1]) for i < h-1; each edge is a midpoint.
      ld dii = 0.0L;
      if (i > 0) dii += 0.5L * da[i];
      if (i < h - 1) dii += 0.5L * db[i];
      diag[i] = 1.0L - dii;
      lower[i] = i > 0 ? -0.5L * da[i] : 0.0L;
      upperd[i] = i < h - 1 ? -0.5L * db[i] : 0.0L;
    }
    // Thomas algorithm.
    for (int i = 1; i < h; ++i) {
      ld w = lower[i] / diag[i - 1];
      diag[i] -= w * upperd[i - 1];
      rhs[i] -= w * rhs[i - 1];
    }
    std::vector<ld> step(h);
    step[h - 1] = rhs[h - 1] / diag[h - 1];
    for (int i = h - 2; i >= 0; --i) step[i] = (rhs[i] - upperd[i] * step[i + 1]) / diag[i];
    for (int i = 0; i < h; ++i) {
      cpos[i] += step[i];
      maxstep = std::max(maxstep, fabsl(step[i]));
    }
    if (maxstep < 1e-18L) break;
  }
}

// Mid-rise uniform grid with the MSE-optimal step for N(0,1): the step solves
// g(delta) = delta * sum m_k^2 P_k - sum m_k (pdf(a_k) - pdf(b_k)) = 0, i.e.
// d MSE / d delta = 0, summed over the positive half (the negative half adds
// the same terms).  g < 0 below the optimum and > 0 above; found by bisection.
static ld uniform_step(int bits) {
  const int L = 1 << bits, h = L / 2;
  auto g = [&](ld delta) {
    ld num = 0.0L, den = 0.0L;
    for (int i = 0; i < h; ++i) {
      ld mk = (ld)i + 0.5L;
      ld a = (ld)i * delta;
      ld b = i == h - 1 ? INFINITY : (ld)(i + 1) * delta;
      num += mk * (pdf(a) - pdf(b));
      den += mk * mk * (upper(a) - upper(b));
    }
    return delta * den - num;
  };
  ld lo = 0.01L * 8.0L / L, hi = 8.0L * 8.0L / L;
  for (int it = 0; it < 200; ++it) {
    ld mid = 0.5L * (lo + hi);
    if (g(mid) < 0.0L) lo = mid; else hi = mid;
    if (hi - lo <= 1e-21L * hi) break;
  }
  return 0.5L * (lo + hi);
}

}  // namespace tq

using namespace tq;

extern "C" {

const char* tq_last_error(void) { return g_last_error; }

const char* tq_status_string(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case TQ_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case TQ_ERR_WORKSPACE: return "workspace too small";
    case TQ_ERR_DEVICE: return "device error";
    default: return "unknown status";
  }
}

size_t tq_page_bytes(int k_bits, int v_bits, int qjl) {
  if (k_bits == 0) {
    if (v_bits != 0 || qjl) return 0;
    return (size_t)2 * TQ_PAGE_TOKENS * TQ_HEAD_DIM * 2;
  }
  if (k_bits < 1 || k_bits > 8 || v_bits < 1 || v_bits > 8) return 0;
  return (size_t)1024 * (k_bits + v_bits) + 512 + (qjl ? 1280 : 0);
}

uint64_t tq_page_descriptor(uint64_t offset, int k_bits, int v_bits, int qjl) {
  if (tq_page_bytes(k_bits, v_bits, qjl) == 0) return 0;
  if ((offset & 255) || offset > TQ_PAGE_OFFSET_MASK) return 0;
  return offset | ((uint64_t)k_bits << 48) | ((uint64_t)v_bits << 52) |
         (qjl ? TQ_PAGE_QJL : 0) | TQ_PAGE_PRESENT;
}

int tq_build_codebook(int bits, int kind, float* centroids, float* boundaries) {
  if (bits < 1 || bits > 8) return fail(TQ_ERR_UNSUPPORTED, "bits must be in 1..8 (got %d)", bits);
  if (!centroids || !boundaries) return fail(TQ_ERR_INVALID_ARG, "null output array");
  const int L = 1 << bits, h = L / 2;
  std::vector<ld> c(L);
  if (kind == TQ_CODEBOOK_LLOYD_MAX || kind == TQ_CODEBOOK_BETA) {
    std::vector<ld> cpos;
    if (kind == TQ_CODEBOOK_LLOYD_MAX)
      lloyd_max(bits, GaussianModel(), cpos);
    else
      lloyd_max(bits, SphereModel(TQ_HEAD_DIM), cpos);
    for (int i = 0; i < h; ++i) {
      c[h + i] = cpos[i];
      c[h - 1 - i] = -cpos[i];
    }
  } else if (kind == TQ_CODEBOOK_UNIFORM) {
    ld delta = uniform_step(bits);
    for (int k = 0; k < L; ++k) c[k] = ((ld)k - 0.5L * (ld)(L - 1)) * delta;
  } else if (kind == TQ_CODEBOOK_POLAR) {
    // the positive-half solver with 2^bits cells from 0 is the one-sided one
    std::vector<ld> cpos;
    lloyd_max(bits + 1, RayleighModel(), cpos);
    for (int k = 0; k < L; ++k) c[k] = cpos[k];
  } else {
    return fail(TQ_ERR_INVALID_ARG, "unknown codebook kind %d", kind);
  }
  for (int k = 0; k < L; ++k) centroids[k] = (float)c[k];
  for (int k = 0; k + 1 < L; ++k) boundaries[k] = (float)(0.5L * (c[k] + c[k + 1]));
  return ok();
}

}  // extern "C"

namespace tq {

// Pair section of a table (widths 1..4): entry lo | hi << b of width b holds
// the values of a coordinate pair whose codes are lo (first coordinate) and hi
// (second).  A scalar codebook's pair is (c[lo], c[hi]).
static void build_scalar_pairs(float* table) {
  for (int b = 1; b <= 4; ++b) {
    const int L = 1 << b;
    const float* c = table + centroid_offset(b);
    float* p = table + kPairOffset + 2 * pair_offset_host(b);
    for (int i = 0; i < L * L; ++i) {
      p[2 * i] = c[i & (L - 1)];
      p[2 * i + 1] = c[i >> b];
    }
  }
}

// PolarQuant's pair at width b with angle shift t: the pair field
// F = rc | tc << r (r = b - t radius bits, a = b + t angle bits) holds radius
// level rc (Lloyd-Max of Rayleigh(1) at r bits) in the direction of angle
// sector tc's middle, -pi + (2 tc + 1) pi / 2^a.  The levels are solved again
// in long double for the products.  A width that cannot carry the shift (r or
// a outside 1..8) keeps a zero table; the encoders refuse its pages.
static void build_polar_pairs(float* table, int shift) {
  const ld pi = 3.14159265358979323846264338327950288L;
  for (int b = 1; b <= 4; ++b) {
    const int rb = b - shift, ab = b + shift;
    if (rb < 1 || rb > 8 || ab < 1 || ab > 8) continue;
    std::vector<ld> r;
    lloyd_max(rb + 1, RayleighModel(), r);
    float* p = table + kPairOffset + 2 * pair_offset_host(b);
    for (int i = 0; i < (1 << (2 * b)); ++i) {
      const ld a = -pi + (ld)(2 * (i >> rb) + 1) * pi / (ld)(1 << ab);
      p[2 * i] = (float)(r[i & ((1 << rb) - 1)] * cosl(a));
      p[2 * i + 1] = (float)(r[i & ((1 << rb) - 1)] * sinl(a));
    }
  }
}

// The encoder's lookup grids of a table whose centroids and boundaries are in
// place (layout in tq_codebook_table's description).
static int build_grids(float* table, int max_bits = 8) {
  uint32_t* words = reinterpret_cast<uint32_t*>(table);
  int next = kLutEntriesOffset;
  for (int b = 1; b <= max_bits; ++b) {
    float* t = table + boundary_offset(b);
    // Quantiser lookup grid: bins of width h over [-T, T) with
    // idx = floor(u * S + O), S = 1/h, O = T/h.  Bin i, widened by h/4 on each
    // side, holds at most one boundary; base = boundaries below the widened bin.
    // (The widening makes an index off by one at a bin edge harmless.)  The
    // boundary is stored in the grid's own coordinate, fma(t, S, O) rounded
    // once to float32, so that the encoder compares its fma(u, S, O) with it
    // (an exact tie u = t stays a tie: both sides round the same expression).
    const int nt = (1 << b) - 1;
    double gap = 2.0, tmax = 0.0;
    for (int k = 0; k + 1 < nt; ++k) gap = std::min(gap, (double)t[k + 1] - (double)t[k]);
    for (int k = 0; k < nt; ++k) tmax = std::max(tmax, fabs((double)t[k]));
    // A grid of at most 256 bins is stored as exactly 256 and indexed by the
    // saturating round-to-nearest byte conversion of u S + O - 1/2 (bins past
    // the grid's end hold the top code), which saves the clamp.
    if (!(gap > 0.0) || 2.0 * (tmax / gap + 1.0) * 2.5 > TQ_CODEBOOK_TABLE_FLOATS)
      return fail(TQ_ERR_UNSUPPORTED, "boundaries of width %d too close for the lookup grid", b);
    const double h = gap / 2.5, T = tmax + 2.0 * h;
    const float S = (float)(1.0 / h), O = (float)(T / h);
    int nb = (int)ceil(2.0 * T / h) + 1;
    const bool byte_grid = nb <= kLutByteBins;
    if (byte_grid) nb = kLutByteBins;
    if (nb > kLutMaxBins)   // the encoder stages at most this many bins in LDS
      return fail(TQ_ERR_UNSUPPORTED, "boundaries of width %d too close for the lookup grid", b);
    if (next + 2 * nb > TQ_CODEBOOK_TABLE_FLOATS)
      return fail(TQ_ERR_UNSUPPORTED, "codebook lookup grid does not fit the table");
    float* hdr = table + kLutHeaderOffset + 4 * (b - 1);
    hdr[0] = S;
    hdr[1] = byte_grid ? O - 0.5f : O;
    reinterpret_cast<uint32_t*>(hdr)[2] = (uint32_t)nb;
    reinterpret_cast<uint32_t*>(hdr)[3] = (uint32_t)next;
    const float Oh = hdr[1];
    for (int i = 0; i < nb; ++i) {
      const long double lo = ((long double)i - (long double)O) / (long double)S - 0.25L / (long double)S;
      const long double hi = ((long double)i + 1.0L - (long double)O) / (long double)S + 0.25L / (long double)S;
      uint32_t base = 0;
      float thr = 3.0e38f;
      int inside = 0;
      for (int k = 0; k < nt; ++k) {
        if ((long double)t[k] < lo) ++base;
        else if ((long double)t[k] < hi) { thr = fmaf(t[k], S, Oh); ++inside; }
      }
      if (inside > 1) return fail(TQ_ERR_UNSUPPORTED, "lookup bin with two boundaries (bits %d)", b);
      words[next + 2 * i] = base;
      table[next + 2 * i + 1] = thr;
    }
    next += 2 * nb;
  }
  return ok();
}

// Magnitudes |u| of the rotated, normalised coordinates
// u = D H D x / ||x|| (= sqrt(d) R x / ||x||) of the nonzero sample vectors, in
// double, sorted.
static std::vector<double> sample_magnitudes(const float* vectors, size_t n, const int8_t* signs) {
  const int d = TQ_HEAD_DIM;
  std::vector<double> u;
  u.reserve(n * d);
  double y[TQ_HEAD_DIM];
  for (size_t v = 0; v < n; ++v) {
    const float* x = vectors + v * d;
    double ss = 0.0;
    for (int j = 0; j < d; ++j) ss += (double)x[j] * (double)x[j];
    if (!(ss > 0.0)) continue;
    const double inv = 1.0 / sqrt(ss);
    for (int j = 0; j < d; ++j) y[j] = signs[j] * (double)x[j];
    for (int h = 1; h < d; h <<= 1)
      for (int i = 0; i < d; i += 2 * h)
        for (int j = i; j < i + h; ++j) {
          const double a = y[j], b = y[j + h];
          y[j] = a + b;
          y[j + h] = a - b;
        }
    for (int j = 0; j < d; ++j) u.push_back(fabs(y[j]) * inv);
  }
  std::sort(u.begin(), u.end());
  return u;
}

// A symmetric codebook fitted to the samples and their mirror images (the
// encoder relies on t_k = -t_{L-2-k}): Lloyd's iteration (k-means in one
// dimension) on the positive half, over the sorted magnitudes.  The positive
// cells are [0, t_1), [t_1, t_2), ..., [t_{h-1}, inf) with t_i the midpoints of
// the current levels; each level moves to the mean of its cell (an empty cell
// keeps its level) until no sample changes cell or kFitSweeps sweeps.  Starts
// from the Gaussian Lloyd-Max levels.  Writes the 2^bits levels and their
// midpoints.
constexpr int kFitSweeps = 200;

static int fit_levels(const std::vector<double>& u, int bits, float* centroids, float* boundaries) {
  const int L = 1 << bits, h = L / 2;
  std::vector<float> c0(L), t0(L);
  int st = tq_build_codebook(bits, TQ_CODEBOOK_LLOYD_MAX, c0.data(), t0.data());
  if (st != TQ_OK) return st;
  std::vector<double> c(c0.begin() + h, c0.end());
  std::vector<size_t> pos(h + 1), prev(h + 1, (size_t)-1);
  for (int sweep = 0; sweep < kFitSweeps; ++sweep) {
    pos[0] = 0;
    pos[h] = u.size();
    for (int k = 1; k < h; ++k)
      pos[k] = (size_t)(std::lower_bound(u.begin(), u.end(), 0.5 * (c[k - 1] + c[k])) - u.begin());
    if (pos == prev) break;
    for (int k = 0; k < h; ++k) {
      if (pos[k + 1] <= pos[k]) continue;
      long double sum = 0.0L;
      for (size_t i = pos[k]; i < pos[k + 1]; ++i) sum += u[i];
      c[k] = (double)(sum / (long double)(pos[k + 1] - pos[k]));
    }
    prev = pos;
  }
  std::vector<double> full(L);
  for (int i = 0; i < h; ++i) {
    full[h + i] = c[i];
    full[h - 1 - i] = -c[i];
  }
  for (int k = 0; k < L; ++k) centroids[k] = (float)full[k];
  for (int k = 0; k + 1 < L; ++k) boundaries[k] = (float)(0.5 * (full[k] + full[k + 1]));
  return TQ_OK;
}

}  // namespace tq

extern "C" {

int tq_codebook_table(int kind, float* table) {
  if (!table) return fail(TQ_ERR_INVALID_ARG, "null table");
  memset(table, 0, sizeof(float) * TQ_CODEBOOK_TABLE_FLOATS);
  for (int b = 1; b <= 8; ++b) {
    int st = tq_build_codebook(b, kind, table + centroid_offset(b), table + boundary_offset(b));
    if (st != TQ_OK) return st;
  }
  if (kind == TQ_CODEBOOK_POLAR) return tq_polar_table(0, table);
  build_scalar_pairs(table);
  return build_grids(table);
}

int tq_polar_table(int angle_shift, float* table) {
  if (!table) return fail(TQ_ERR_INVALID_ARG, "null table");
  if (angle_shift < -3 || angle_shift > 3)
    return fail(TQ_ERR_UNSUPPORTED, "angle shift %d outside -3..3", angle_shift);
  memset(table, 0, sizeof(float) * TQ_CODEBOOK_TABLE_FLOATS);
  for (int b = 1; b <= 8; ++b) {
    int st = tq_build_codebook(b, TQ_CODEBOOK_POLAR, table + centroid_offset(b), table + boundary_offset(b));
    if (st != TQ_OK) return st;
  }
  // pages are at most 4 bits wide; their radius grids go up to 4 - shift bits
  build_polar_pairs(table, angle_shift);
  table[kPolarShiftSlot] = (float)angle_shift;
  return build_grids(table, std::min(8, 4 - std::min(angle_shift, 0)));
}

int tq_fit_codebook(const float* vectors, size_t n, const int8_t* signs, int bits, float* centroids,
                    float* boundaries) {
  if (bits < 1 || bits > 8) return fail(TQ_ERR_UNSUPPORTED, "bits must be in 1..8 (got %d)", bits);
  if (!vectors || !signs || !centroids || !boundaries) return fail(TQ_ERR_INVALID_ARG, "null pointer");
  for (int j = 0; j < TQ_HEAD_DIM; ++j)
    if (signs[j] != 1 && signs[j] != -1) return fail(TQ_ERR_INVALID_ARG, "sign %d is not +-1", j);
  const std::vector<double> u = sample_magnitudes(vectors, n, signs);
  if (u.empty()) return fail(TQ_ERR_INVALID_ARG, "no nonzero sample vector");
  int st = fit_levels(u, bits, centroids, boundaries);
  return st != TQ_OK ? st : ok();
}

int tq_calibrated_table(const float* vectors, size_t n, const int8_t* signs, float* table) {
  if (!table) return fail(TQ_ERR_INVALID_ARG, "null table");
  if (!vectors || !signs) return fail(TQ_ERR_INVALID_ARG, "null pointer");
  for (int j = 0; j < TQ_HEAD_DIM; ++j)
    if (signs[j] != 1 && signs[j] != -1) return fail(TQ_ERR_INVALID_ARG, "sign %d is not +-1", j);
  const std::vector<double> u = sample_magnitudes(vectors, n, signs);
  if (u.empty()) return fail(TQ_ERR_INVALID_ARG, "no nonzero sample vector");
  memset(table, 0, sizeof(float) * TQ_CODEBOOK_TABLE_FLOATS);
  for (int b = 1; b <= 8; ++b) {
    int st = fit_levels(u, b, table + centroid_offset(b), table + boundary_offset(b));
    if (st != TQ_OK) return st;
  }
  build_scalar_pairs(table);
  return build_grids(table);
}

static uint64_t splitmix64_at(uint64_t seed, uint64_t index) {
  // Output `index` (1-based) of SplitMix64 seeded with `seed`.
  uint64_t z = seed + index * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int tq_layer_params(uint64_t seed, int layer, int head_dim, int jl_dim, int8_t* signs,
                    float* qjl_s) {
  if (head_dim != TQ_HEAD_DIM) return fail(TQ_ERR_UNSUPPORTED, "head_dim must be 128");
  if (qjl_s && jl_dim != TQ_JL_DIM) return fail(TQ_ERR_UNSUPPORTED, "jl_dim must be 128");
  if (!signs) return fail(TQ_ERR_INVALID_ARG, "null signs");
  const uint64_t s = seed + (uint64_t)(int64_t)layer;
  for (int j = 0; j < head_dim; ++j) signs[j] = (splitmix64_at(s, j + 1) >> 63) ? -1 : 1;
  if (qjl_s) {
    const int n = jl_dim * head_dim;
    const double two_pi = 2.0 * M_PI;
    uint64_t idx = head_dim + 1;
    for (int i = 0; i < n; i += 2) {
      double u1 = (double)(splitmix64_at(s, idx++) >> 11) * (1.0 / 9007199254740992.0);
      double u2 = (double)(splitmix64_at(s, idx++) >> 11) * (1.0 / 9007199254740992.0);
      double r = sqrt(-2.0 * log(1.0 - u1));
      double a = two_pi * u2;
      qjl_s[i] = (float)(r * cos(a));
      if (i + 1 < n) qjl_s[i + 1] = (float)(r * sin(a));
    }
  }
  return ok();
}

int tq_sign_mask(const int8_t* signs, int head_dim, uint32_t* mask) {
  if (!signs || !mask) return fail(TQ_ERR_INVALID_ARG, "null pointer");
  if (head_dim != TQ_HEAD_DIM) return fail(TQ_ERR_UNSUPPORTED, "head_dim must be 128");
  for (int w = 0; w < 4; ++w) mask[w] = 0;
  for (int j = 0; j < head_dim; ++j) {
    if (signs[j] != 1 && signs[j] != -1) return fail(TQ_ERR_INVALID_ARG, "sign %d is not +-1", j);
    if (signs[j] < 0) mask[j >> 5] |= 1u << (j & 31);
  }
  return ok();
}

size_t tq_cache_bytes(const uint64_t* host_pages, size_t n) {
  if (!host_pages) return 0;
  size_t total = 0;
  for (size_t i = 0; i < n; ++i) {
    uint64_t d = host_pages[i];
    if (!(d & TQ_PAGE_PRESENT)) continue;
    total += (d & TQ_PAGE_PENDING) ? tq_page_bytes(0, 0, 0)
                                   : tq_page_bytes((int)((d >> 48) & 15), (int)((d >> 52) & 15),
                                                   (d & TQ_PAGE_QJL) ? 1 : 0);
  }
  return total;
}

size_t tq_decode_workspace_bytes(const tq_cache* cache, int n_q_heads) {
  if (!cache || cache->n_sessions <= 0 || cache->n_kv_heads <= 0 || cache->max_pages <= 0 ||
      n_q_heads <= 0)
    return 0;
  SplitPlan sp = split_plan(cache->n_sessions, cache->n_kv_heads, cache->max_pages);
  return decode_workspace_bytes(cache->n_sessions, n_q_heads, sp);
}

}  // extern "C"

namespace tq {

SplitPlan split_plan(int n_sessions, int n_kv_heads, int max_pages) {
  // Enough workgroups to fill the GPU several times over, each with at least
  // one page per wave: ranges of total / kTargetSplitGroups pages.  The other
  // class (half as long) keeps that length.  The common and wide classes cut
  // ranges longer than kLongRangePages to about 3 kTargetSplitGroups of them
  // (not below kLongRangePages): with long contexts their ranges, all
  // resident at once, would otherwise wait for the slowest (tiers mix cheap
  // and dear pages), while several rounds of shorter ones balance.  Wide
  // ranges are as long as common ones when those are not cut (the merged
  // launch of a layer with hub heads then stays one round of workgroups;
  // shorter wide ranges added a round of their own; the launch may shorten
  // them down to a quarter, balancing them against longer common ranges),
  // and a quarter of that length when they are.
  const int64_t units = (int64_t)n_sessions * n_kv_heads;
  const int64_t total_pages = units * max_pages;
  auto clamp_len = [&](int64_t p) {
    p = std::max<int64_t>(p, kDecodeWaves);
    p = std::min<int64_t>(p, kMaxPagesPerSplit);
    return std::min<int64_t>(p, max_pages);
  };
  const int64_t pps = clamp_len((total_pages + kTargetSplitGroups - 1) / kTargetSplitGroups);
  const int64_t short_len = (total_pages + 3 * kTargetSplitGroups - 1) / (3 * kTargetSplitGroups);
  int64_t ppc = std::max<int64_t>(std::min<int64_t>(pps, kLongRangePages), short_len);
  // at most kTargetSplitGroups ranges per unit (the partials' slots)
  ppc = clamp_len(std::max<int64_t>(ppc, (max_pages + kTargetSplitGroups - 1) / kTargetSplitGroups));
  SplitPlan sp;
  sp.pages_per_split = (int)ppc;
  sp.n_splits = (int)((max_pages + ppc - 1) / ppc);
  sp.pages_per_split_general = (int)((pps + 1) / 2);
  sp.n_splits_general = (max_pages + sp.pages_per_split_general - 1) / sp.pages_per_split_general;
  sp.cut = pps > kLongRangePages;
  sp.min_pages_per_split_wide = (sp.pages_per_split + 3) / 4;
  sp.max_splits_wide = (max_pages + sp.min_pages_per_split_wide - 1) / sp.min_pages_per_split_wide;
  sp.pages_per_split_wide = sp.cut ? sp.min_pages_per_split_wide : sp.pages_per_split;
  sp.n_splits_wide = (max_pages + sp.pages_per_split_wide - 1) / sp.pages_per_split_wide;
  return sp;
}

size_t decode_workspace_bytes(int n_sessions, int n_q_heads, const SplitPlan& sp) {
  const size_t rows = (size_t)n_sessions * n_q_heads;
  // query prep, then the partials of the three page classes
  return sizeof(float) * rows *
         (kQPrepFloats + (size_t)(sp.n_splits + sp.max_splits_wide + sp.n_splits_general) * kPartialFloats);
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int check_layer(const tq_layer* L) {
  if (!L) return fail(TQ_ERR_INVALID_ARG, "null layer descriptor");
  if (L->head_dim != TQ_HEAD_DIM) return fail(TQ_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", L->head_dim);
  if (L->k_codebook < TQ_CODEBOOK_LLOYD_MAX || L->k_codebook > TQ_CODEBOOK_POLAR)
    return fail(TQ_ERR_INVALID_ARG, "unknown k_codebook %d", L->k_codebook);
  if (L->v_codebook < TQ_CODEBOOK_LLOYD_MAX || L->v_codebook > TQ_CODEBOOK_POLAR)
    return fail(TQ_ERR_INVALID_ARG, "unknown v_codebook %d", L->v_codebook);
  if (!L->sign_mask || !L->k_table || !L->v_table) return fail(TQ_ERR_INVALID_ARG, "null layer table");
  if (!aligned16(L->sign_mask) || !aligned16(L->k_table) || !aligned16(L->v_table))
    return fail(TQ_ERR_ALIGNMENT, "layer tables must be 16-byte aligned");
  if (L->qjl_s) {
    if (L->jl_dim != TQ_JL_DIM) return fail(TQ_ERR_UNSUPPORTED, "jl_dim must be 128 (got %d)", L->jl_dim);
    if (!aligned16(L->qjl_s)) return fail(TQ_ERR_ALIGNMENT, "qjl_s must be 16-byte aligned");
  }
  return TQ_OK;
}

int check_cache(const tq_cache* C) {
  if (!C) return fail(TQ_ERR_INVALID_ARG, "null cache descriptor");
  if (C->n_sessions <= 0 || C->n_kv_heads <= 0 || C->max_pages <= 0)
    return fail(TQ_ERR_INVALID_ARG, "cache sizes must be positive (B=%d H_kv=%d max_pages=%d)",
                C->n_sessions, C->n_kv_heads, C->max_pages);
  if ((int64_t)C->max_pages * TQ_PAGE_TOKENS > (int64_t)0x7fffffff)
    return fail(TQ_ERR_INVALID_ARG, "max_pages too large");
  if (!C->n_tokens || !C->pages || !C->pool) return fail(TQ_ERR_INVALID_ARG, "null cache pointer");
  if (((uintptr_t)C->pool & 255) != 0) return fail(TQ_ERR_ALIGNMENT, "pool must be 256-byte aligned");
  if (((uintptr_t)C->pages & 7) != 0 || ((uintptr_t)C->n_tokens & 3) != 0)
    return fail(TQ_ERR_ALIGNMENT, "page table / token counts misaligned");
  if (C->pool_bytes == 0) return fail(TQ_ERR_INVALID_ARG, "empty pool");
  if (C->page_classes & ~(TQ_CACHE_COMMON_PAGES | TQ_CACHE_OTHER_PAGES | TQ_CACHE_WIDE_PAGES))
    return fail(TQ_ERR_INVALID_ARG, "unknown page_classes bits 0x%x", C->page_classes);
  if (C->unit_classes) {
    const int64_t units = (int64_t)C->n_sessions * C->n_kv_heads;
    for (int64_t u = 0; u < units; ++u)
      if (C->unit_classes[u] & ~(TQ_CACHE_COMMON_PAGES | TQ_CACHE_OTHER_PAGES | TQ_CACHE_WIDE_PAGES))
        return fail(TQ_ERR_INVALID_ARG, "unknown unit_classes bits 0x%x at unit %lld",
                    (unsigned)C->unit_classes[u], (long long)u);
  }
  return TQ_OK;
}

}  // namespace tq
