// Host derivation of the NF4 code book and of the thresholds the quantizer
// compares against.
//
// Bitsandbytes tool page (ozercemkelahmet.com/tools/bitsandbytes), "How NF4
// works": the 16 code values are placed so that each covers an equal share of
// the bell curve.  The construction used is the asymmetric equal-probability
// one that came with NF4 (the QLoRA paper named on that page): with
// delta = 1 - (1/30 + 1/32)/2, the positive levels are the normal quantiles at
// 8 probabilities stepping evenly from delta toward 1/2, the negative levels
// the negated quantiles at 7 such probabilities, 1/2 itself excluded, plus an
// exact zero; all are divided by the quantile at delta so the ends are +-1.
//
// Quantiles are found by bisection on the upper tail 0.5*erfc(x/sqrt 2) in
// x87 extended precision and rounded once to float32.
#include <cfloat>
#include <cmath>

#include "nf4_internal.h"

namespace nf4i {
namespace {

long double upper_tail(long double x) { return 0.5L * erfcl(x / sqrtl(2.0L)); }

// x >= 0 with upper_tail(x) = q, for 0 < q < 1/2.
long double upper_tail_inverse(long double q) {
  long double lo = 0.0L, hi = 16.0L;
  for (int it = 0; it < 400; ++it) {
    long double mid = 0.5L * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (upper_tail(mid) > q) lo = mid; else hi = mid;
  }
  return 0.5L * (lo + hi);
}

// Smallest float t such that every float v >= t is nearer (ties: farther from
// zero) to level[i+1] than to level[i].
float decision_threshold(float lo, float hi) {
  const double mid = 0.5 * (static_cast<double>(lo) + static_cast<double>(hi));  // exact
  const float f = static_cast<float>(mid);
  const double fd = static_cast<double>(f);
  if (fd == mid) return mid > 0.0 ? f : std::nextafterf(f, INFINITY);  // tie rule
  return fd > mid ? f : std::nextafterf(f, INFINITY);
}

Codebook build() {
  Codebook cb{};
  // 1 - p for the positive side: p_i = delta - (delta - 1/2) i/8, i = 0..7, so
  // 1 - p_i = (248 + 449 i) / 7680; negative side: (217 + 449 j) / 6720.
  const long double top = upper_tail_inverse(31.0L / 960.0L);
  for (int j = 0; j < 7; ++j) {
    const long double q = (217.0L + 449.0L * j) / 6720.0L;
    cb.level[j] = static_cast<float>(-(upper_tail_inverse(q) / top));
  }
  cb.level[7] = 0.0f;
  for (int i = 0; i < 8; ++i) {
    const long double q = (248.0L + 449.0L * i) / 7680.0L;
    cb.level[15 - i] = static_cast<float>(upper_tail_inverse(q) / top);
  }
  for (int i = 0; i < 15; ++i) cb.thresh[i] = decision_threshold(cb.level[i], cb.level[i + 1]);
  cb.thresh[15] = INFINITY;
  return cb;
}

}  // namespace

const Codebook& codebook() {
  static const Codebook cb = build();
  return cb;
}

}  // namespace nf4i
