// NF4 table and the bucket table of the nearest-row search (host side).
//
// "QLoRA Explained: A 4-Bit Base, NF4, and What It Really Costs", sections "Put
// the rows where the weights are" and "That is NF4": the sixteen rows are
// quantiles of a standard normal, computed once, one of them exactly zero, the
// table spanning [-1, 1] once the block scale is divided out.
//
// Reading of the unspecified details: probabilities evenly spaced within each
// half; 7 rows below zero, zero, 8 rows above; the outermost rows at tail
// probability delta = (1/30 + 1/32)/2 = 31/960; every quantile divided by
// z* = Phi^-1(1 - delta).
//
// The inverse normal CDF here is Newton's method on Phi(z) - p = 0 with
// Phi(z) = erfc(-z/sqrt 2)/2 from the C library and Phi'(z) = exp(-z^2/2)/sqrt(2 pi).
// Started at z = 0, the iteration approaches the root monotonically (Phi is
// convex below zero and concave above), and it stops when the step no longer
// changes z.  Accuracy is that of erfc (about 1 ulp of fp64), far finer than
// the fp32 rounding that follows.

#include <cfloat>
#include <cmath>
#include <cstring>
#include <mutex>

#include "qn_internal.h"

namespace qn {
namespace {

double normal_cdf(double z) { return 0.5 * std::erfc(-z / std::sqrt(2.0)); }

double normal_quantile(double p) {
  const double inv_sqrt_2pi = 0.39894228040143267794;
  double z = 0.0;
  for (int it = 0; it < 200; ++it) {
    double f = normal_cdf(z) - p;
    double d = inv_sqrt_2pi * std::exp(-0.5 * z * z);
    double zn = z - f / d;
    if (zn == z) break;
    // Stop once the step is below the fp64 resolution around z.
    if (std::fabs(zn - z) <= 4 * DBL_EPSILON * std::fmax(1.0, std::fabs(z))) {
      z = zn;
      // One more step to settle the last ulp, then stop.
      f = normal_cdf(z) - p;
      d = inv_sqrt_2pi * std::exp(-0.5 * z * z);
      z = z - f / d;
      break;
    }
    z = zn;
  }
  return z;
}

// Smallest fp32 strictly greater than the (exact) fp64 value m.
float next_f32_above(double m) {
  float f = (float)m;
  if ((double)f > m) {
    // f is the nearest; it may still not be the smallest above m if rounding
    // went up by more than one ulp, which cannot happen for round-to-nearest.
    return f;
  }
  return std::nextafterf(f, INFINITY);
}

CodecTables g_tables;
double g_rows64[16];
std::once_flag g_once;
bool g_ok = true;

void build() {
  const double delta = (1.0 / 30.0 + 1.0 / 32.0) / 2.0;  // 31/960
  const double zstar = normal_quantile(1.0 - delta);
  for (int i = 0; i < 7; ++i) {
    double p = delta + i * (0.5 - delta) / 7.0;
    g_rows64[i] = normal_quantile(p) / zstar;
  }
  g_rows64[7] = 0.0;
  for (int j = 1; j <= 8; ++j) {
    double p = 0.5 + j * (0.5 - delta) / 8.0;
    g_rows64[7 + j] = normal_quantile(p) / zstar;
  }
  g_rows64[0] = -1.0;
  g_rows64[15] = 1.0;
  for (int i = 0; i < 16; ++i) g_tables.code[i] = (float)g_rows64[i];

  // Decision thresholds: the row index of n is #{i : n >= T_i}, T_i being the
  // smallest fp32 above the exact midpoint of rows i and i+1 (an fp32 n equal
  // to a representable midpoint stays with the lower row).
  float T[15];
  for (int i = 0; i < 15; ++i) {
    double m = ((double)g_tables.code[i] + (double)g_tables.code[i + 1]) / 2.0;
    T[i] = next_f32_above(m);
  }
  // Buckets of width 1/16 over [-1, 1].
  for (int b = 0; b < 32; ++b) {
    double lo = b / 16.0 - 1.0, hi = (b + 1) / 16.0 - 1.0;
    uint32_t below = 0;
    float inside = INFINITY;
    int n_inside = 0;
    for (int i = 0; i < 15; ++i) {
      if ((double)T[i] < lo) ++below;
      else if ((double)T[i] < hi) { inside = T[i]; ++n_inside; }
    }
    if (n_inside > 1) g_ok = false;
    g_tables.base[b] = below;
    g_tables.thr[b] = inside;
  }
  for (int i = 0; i < 15; ++i) {
    double t = ((double)T[i] + 1.0) * 16.0;
    double frac = t - std::floor(t);
    double dist = std::fmin(frac, 1.0 - frac) / 16.0;
    if (dist < 1e-4) g_ok = false;
  }
}

}  // namespace

const CodecTables &codec_tables() {
  std::call_once(g_once, build);
  return g_tables;
}

bool codec_tables_ok() {
  codec_tables();
  return g_ok;
}

Code16 code16() {
  Code16 c;
  const CodecTables &t = codec_tables();
  for (int i = 0; i < 16; ++i) c.v[i] = t.code[i];
  return c;
}

void nf4_rows_f64(double out[16]) {
  codec_tables();
  std::memcpy(out, g_rows64, sizeof(g_rows64));
}

}  // namespace qn
