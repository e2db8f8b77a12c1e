// Build-time generator of the codec's fixed scalar codebooks.
//
// The page "TACT-KV: Tri-Axis Cosine Transform ..." (section "Methodology in
// Plain English", stage 4) quantizes each coordinate of a gain-normalized
// bin with a precomputed Lloyd-Max table at the bin's bit width.  The tables
// here are the minimum-MSE quantizers of a unit Gaussian for 1..8 bits,
// solved in double precision:
//   * the quantizer is symmetric, 0 is a threshold, so only the 2^(b-1)
//     positive levels y_1 < ... < y_m are unknowns;
//   * thresholds are midpoints t_j = (y_j + y_{j+1}) / 2, t_0 = 0, t_m = inf;
//   * each level is the centroid of its cell,
//       y_j = (phi(t_{j-1}) - phi(t_j)) / (Q(t_{j-1}) - Q(t_j)),
//     with phi the density and Q the upper tail of N(0, 1);
//   * solved by fixed-point (Lloyd) sweeps followed by Newton's method on
//     F(y) = centroid(y) - y, whose Jacobian is tridiagonal (Thomas solve).
// It also writes the two other quantizers of the page's comparison (a
// symmetric uniform grid and NormalFloat, both of [-1, 1]).
// Output: a C include with the tables as exact hexadecimal float literals
// (rounded to fp32), ascending, code c = c-th level from the most negative.
#include <cfloat>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

double density(double x) {
  if (!std::isfinite(x)) return 0.0;
  return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
}

double upper_tail(double x) {
  if (x == INFINITY) return 0.0;
  return 0.5 * std::erfc(x / std::sqrt(2.0));
}

struct Cells {
  std::vector<double> lo, hi, mass, centroid;
};

Cells cells_of(const std::vector<double>& y) {
  const size_t m = y.size();
  Cells c;
  c.lo.resize(m);
  c.hi.resize(m);
  c.mass.resize(m);
  c.centroid.resize(m);
  for (size_t j = 0; j < m; ++j) {
    c.lo[j] = (j == 0) ? 0.0 : 0.5 * (y[j - 1] + y[j]);
    c.hi[j] = (j + 1 == m) ? INFINITY : 0.5 * (y[j] + y[j + 1]);
    c.mass[j] = upper_tail(c.lo[j]) - upper_tail(c.hi[j]);
    c.centroid[j] = (density(c.lo[j]) - density(c.hi[j])) / c.mass[j];
  }
  return c;
}

std::vector<double> solve_positive_levels(int bits) {
  const int m = 1 << (bits - 1);
  std::vector<double> y(m);
  for (int j = 0; j < m; ++j) y[j] = (j + 0.5) * 4.0 / m;
  for (int it = 0; it < 3000; ++it) y = cells_of(y).centroid;
  for (int it = 0; it < 100; ++it) {
    Cells c = cells_of(y);
    double worst = 0.0;
    std::vector<double> f(m), sub(m, 0.0), dia(m, -1.0), sup(m, 0.0);
    for (int j = 0; j < m; ++j) {
      f[j] = c.centroid[j] - y[j];
      worst = std::fmax(worst, std::fabs(f[j]));
      // d centroid / d lower edge, d centroid / d upper edge
      const double dlo = density(c.lo[j]) * (c.centroid[j] - c.lo[j]) / c.mass[j];
      const double dhi = std::isfinite(c.hi[j])
                             ? density(c.hi[j]) * (c.hi[j] - c.centroid[j]) / c.mass[j]
                             : 0.0;
      if (j > 0) {  // lower edge = (y[j-1] + y[j]) / 2
        sub[j] += 0.5 * dlo;
        dia[j] += 0.5 * dlo;
      }
      if (j + 1 < m) {  // upper edge = (y[j] + y[j+1]) / 2
        dia[j] += 0.5 * dhi;
        sup[j] += 0.5 * dhi;
      }
    }
    if (worst < 1e-15) break;
    // Thomas algorithm for J * delta = -f
    std::vector<double> cp(m), dp(m);
    cp[0] = sup[0] / dia[0];
    dp[0] = -f[0] / dia[0];
    for (int j = 1; j < m; ++j) {
      const double den = dia[j] - sub[j] * cp[j - 1];
      cp[j] = sup[j] / den;
      dp[j] = (-f[j] - sub[j] * dp[j - 1]) / den;
    }
    std::vector<double> delta(m);
    delta[m - 1] = dp[m - 1];
    for (int j = m - 2; j >= 0; --j) delta[j] = dp[j] - cp[j] * delta[j + 1];
    for (int j = 0; j < m; ++j) y[j] += delta[j];
  }
  return y;
}

}  // namespace

// Standard normal quantile by bisection on the lower tail 0.5 erfc(-x/sqrt2)
double normal_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 200; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (0.5 * std::erfc(-mid / std::sqrt(2.0)) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

void emit(const char* name, const std::vector<float>& v) {
  std::printf("#define %s \\\n", name);
  for (size_t i = 0; i < v.size(); ++i)
    std::printf("  %a%s", (double)v[i], i + 1 < v.size() ? ",\\\n" : "\n");
}

// Midpoint thresholds of an ascending level table, rounded to fp32.
void midpoints(const std::vector<double>& lv, std::vector<float>& thr) {
  for (size_t j = 0; j + 1 < lv.size(); ++j) thr.push_back((float)(0.5 * (lv[j] + lv[j + 1])));
}

int main() {
  std::vector<float> levels, thresholds;
  // the comparison backends of the page's "Main Findings": a symmetric
  // uniform quantizer (2^b equal cells of [-1, 1], levels at the cell
  // centres) and NormalFloat (normal quantiles at (k + 1/2) / 2^b, outermost
  // levels at +-1); both scale by the bin's absolute maximum
  std::vector<float> ulevels, uthresholds, nlevels, nthresholds;
  for (int b = 1; b <= 8; ++b) {
    const std::vector<double> y = solve_positive_levels(b);
    const int m = (int)y.size();
    for (int j = m - 1; j >= 0; --j) levels.push_back((float)-y[j]);
    for (int j = 0; j < m; ++j) levels.push_back((float)y[j]);
    for (int j = m - 2; j >= 0; --j) thresholds.push_back((float)(-0.5 * (y[j] + y[j + 1])));
    thresholds.push_back(0.0f);
    for (int j = 0; j + 1 < m; ++j) thresholds.push_back((float)(0.5 * (y[j] + y[j + 1])));
    const int n = 1 << b;
    std::vector<double> ul(n), nl(n);
    const double zmax = normal_quantile((n - 0.5) / n);
    for (int k = 0; k < n; ++k) ul[k] = (2.0 * k + 1.0 - n) / n;
    // the quantiles mirror about 1/2: the upper half, mirrored, keeps the
    // table exactly symmetric (middle threshold 0)
    for (int k = n / 2; k < n; ++k) {
      nl[k] = normal_quantile((k + 0.5) / n) / zmax;
      nl[n - 1 - k] = -nl[k];
    }
    for (int k = 0; k < n; ++k) {
      ulevels.push_back((float)ul[k]);
      nlevels.push_back((float)nl[k]);
    }
    midpoints(ul, uthresholds);
    midpoints(nl, nthresholds);
  }
  std::printf("/* Generated by gen_codebooks.cpp: Gaussian Lloyd-Max tables, 1..8 bits,\n"
              " * fp32, ascending, and the uniform and NormalFloat tables of the same\n"
              " * sizes.  Level table of b bits starts at (1<<b) - 2, threshold table\n"
              " * at (1<<b) - b - 1. */\n");
  std::printf("#define TACT_CODEBOOK_LEVELS %zu\n#define TACT_CODEBOOK_THRESHOLDS %zu\n",
              levels.size(), thresholds.size());
  emit("TACT_CODEBOOK_LEVEL_VALUES", levels);
  emit("TACT_CODEBOOK_THRESHOLD_VALUES", thresholds);
  emit("TACT_UNIFORM_LEVEL_VALUES", ulevels);
  emit("TACT_UNIFORM_THRESHOLD_VALUES", uthresholds);
  emit("TACT_NF_LEVEL_VALUES", nlevels);
  emit("TACT_NF_THRESHOLD_VALUES", nthresholds);
  return 0;
}
