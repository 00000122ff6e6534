// NF4 codebook for the library (host code).
//
// NF4 places its 16 levels at normal-distribution quantiles of evenly spaced
// probabilities so that every bin is equally likely and the levels crowd
// around 0 ("LLM quantization selection: five mainstream schemes compared",
// section 6.1; the concepts article, section 七).  The pages print no level
// values; this library uses 8 positive levels at probabilities evenly spaced
// in (1/2, 31/32], 7 negative levels mirrored from probabilities evenly
// spaced in (1/2, 31/32], and an exact 0, all divided by PhiInv(31/32) so
// the range is exactly [-1, 1].  31/32 is the centre of the outermost of 16
// equal-probability bins, which keeps the quantiles finite.
//
// The quantile function here is Newton's method on Phi(x) = erfc(-x/sqrt2)/2
// in double precision; each level is rounded once to fp32.  The decision
// midpoints are (L_i + L_{i+1}) * 0.5 evaluated in fp32.
#include <cmath>

#include "internal.h"

namespace wq {
namespace {

double phi(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double phi_inv(double p) {
  // p is in [1/2, 31/32] here; Newton from 0 converges monotonically there
  // because Phi is concave on x >= 0.
  const double inv_sqrt_2pi = 0.39894228040143267794;
  double x = 0.0;
  for (int it = 0; it < 100; ++it) {
    double f = phi(x) - p;
    double d = inv_sqrt_2pi * std::exp(-0.5 * x * x);
    double step = f / d;
    x -= step;
    if (std::fabs(step) <= 1e-17 * (1.0 + std::fabs(x))) break;
  }
  return x;
}

struct Table {
  float levels[16];
  float thresholds[15];
  Table() {
    const double pmax = 1.0 - 1.0 / 32.0;
    const double top = phi_inv(pmax);
    levels[7] = 0.0f;
    for (int i = 1; i <= 8; ++i)
      levels[7 + i] = (float)(phi_inv(0.5 + (pmax - 0.5) * i / 8.0) / top);
    for (int i = 1; i <= 7; ++i)
      levels[7 - i] = (float)(-phi_inv(0.5 + (pmax - 0.5) * i / 7.0) / top);
    for (int i = 0; i < 15; ++i) {
      volatile float s = levels[i] + levels[i + 1];  // fp32 sum
      thresholds[i] = s * 0.5f;
    }
  }
};

const Table& table() {
  static const Table t;
  return t;
}

// FP4: the E2M1 values of codes 0..15 (sign bit 3, exponent bits 2-1 with
// bias 1, mantissa bit 0: magnitudes 0, 1/2, 1, 3/2, 2, 3, 4, 6) divided by
// 6, and the fp32 midpoints between adjacent magnitudes.
struct Fp4Table {
  float levels[16];
  float thresholds[15];
  Fp4Table() {
    for (int c = 0; c < 16; ++c) {
      const int e = (c >> 1) & 3, m = c & 1;
      const double mag = e == 0 ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, e - 1);
      const float v = (float)(mag / 6.0);
      levels[c] = (c & 8) ? -v : v;
    }
    for (int i = 0; i < 15; ++i) thresholds[i] = 0.0f;
    for (int i = 0; i < 7; ++i) {
      volatile float s = levels[i] + levels[i + 1];  // fp32 sum
      thresholds[i] = s * 0.5f;
    }
  }
};

const Fp4Table& fp4_table() {
  static const Fp4Table t;
  return t;
}

}  // namespace

const float* nf4_levels() { return table().levels; }
const float* nf4_thresholds() { return table().thresholds; }
const float* fp4_levels() { return fp4_table().levels; }
const float* fp4_thresholds() { return fp4_table().thresholds; }

}  // namespace wq
