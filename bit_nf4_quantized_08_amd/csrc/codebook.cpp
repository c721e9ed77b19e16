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

#include <algorithm>
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

CodecTables g_tables[2];
double g_rows64[16];
std::once_flag g_once;
bool g_ok = true;

// The 4-bit float of the second table: sign, two exponent bits, one mantissa
// bit (exponent bias 1), divided by the largest magnitude 6 so that the table
// spans [-1, 1].  Codes 0 and 8 are +0 and -0.
double fp4_value(int c) {
  const int s = c >> 3, e = (c >> 1) & 3, m = c & 1;
  const double mag = e == 0 ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, e - 1);
  return (s ? -mag : mag) / 6.0;
}

// Decision table of one 16-entry table (values by code): the distinct values
// ascending (a repeated value keeps its smaller code); threshold i is the
// smallest fp32 strictly above the exact midpoint of levels i and i+1, so an
// fp32 value equal to a representable midpoint stays with the lower level.
// Buckets of width 1/16 over [-1, 1 + 1/16) each hold at most one threshold:
// base[b] = levels below the bucket, thr[b] = its threshold (or +inf),
// lohi[b] = code of level base[b] | code of level base[b] + 1 << 8.  The
// kernel takes the bucket from the fp32 sum n + 5 (rounded once, in [4, 8)),
// whose edges 5 + b/16 - 1 are representable, so the bucket can only come
// out one too high, for an n within 2^-22 below an edge; no threshold may lie
// that close below an edge (checked, with a margin of 1e-6).
void build_decisions(CodecTables &t) {
  int order[16];
  for (int i = 0; i < 16; ++i) order[i] = i;
  std::sort(order, order + 16, [&](int x, int y) {
    return t.code[x] < t.code[y] || (t.code[x] == t.code[y] && x < y);
  });
  float lev[16];
  uint32_t lcode[16];
  int L = 0;
  for (int k = 0; k < 16; ++k) {
    const int c = order[k];
    if (L > 0 && t.code[c] == lev[L - 1]) continue;   // same value: the smaller code was taken
    lev[L] = t.code[c];
    lcode[L] = (uint32_t)c;
    ++L;
  }
  float T[15];
  for (int i = 0; i + 1 < L; ++i) T[i] = next_f32_above(((double)lev[i] + (double)lev[i + 1]) / 2.0);
  for (int b = 0; b < kBuckets; ++b) {
    const double lo = b / 16.0 - 1.0, hi = (b + 1) / 16.0 - 1.0;
    uint32_t below = 0;
    float inside = INFINITY;
    int n_inside = 0;
    for (int i = 0; i + 1 < L; ++i) {
      if ((double)T[i] < lo) ++below;
      else if ((double)T[i] < hi) { inside = T[i]; ++n_inside; }
    }
    if (n_inside > 1) g_ok = false;
    t.base[b] = below;
    t.thr[b] = inside;
    const uint32_t c_lo = lcode[below], c_hi = lcode[below + 1 < (uint32_t)L ? below + 1 : below];
    t.lohi[b] = c_lo | (c_hi << 8);
  }
  for (int i = 0; i + 1 < L; ++i) {
    const double u = ((double)T[i] + 1.0) * 16.0;
    const double to_edge = (std::ceil(u) - u) / 16.0;   // distance up to the next edge
    if (to_edge > 0.0 && to_edge < 1e-6) g_ok = false;
  }
}

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
  for (int i = 0; i < 16; ++i) g_tables[QN_NF4].code[i] = (float)g_rows64[i];
  for (int i = 0; i < 16; ++i) g_tables[QN_FP4].code[i] = (float)fp4_value(i);
  build_decisions(g_tables[QN_NF4]);
  build_decisions(g_tables[QN_FP4]);
  // The NF4 rows are distinct and ascending: the code of a level is its rank,
  // which the quantiser's NF4 path relies on.
  for (int b = 0; b < kBuckets; ++b) {
    const uint32_t lo = g_tables[QN_NF4].lohi[b] & 0xFF;
    if (lo != g_tables[QN_NF4].base[b]) g_ok = false;
  }
}

}  // namespace

const CodecTables &codec_tables(int qtype) {
  std::call_once(g_once, build);
  return g_tables[qtype == QN_FP4 ? QN_FP4 : QN_NF4];
}

bool codec_tables_ok() {
  codec_tables(QN_NF4);
  return g_ok;
}

Code16 code16(int qtype) {
  Code16 c;
  const CodecTables &t = codec_tables(qtype);
  for (int i = 0; i < 16; ++i) c.v[i] = t.code[i];
  return c;
}

void nf4_rows_f64(double out[16]) {
  codec_tables(QN_NF4);
  std::memcpy(out, g_rows64, sizeof(g_rows64));
}

}  // namespace qn
