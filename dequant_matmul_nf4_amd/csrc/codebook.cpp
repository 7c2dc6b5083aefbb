// Host derivation of the NF4 code book (and of the FP4 one) and of the
// thresholds the quantizer compares against.
//
// FP4: the bitsandbytes tool page lists FP4 beside NF4 among the 4-bit formats
// ("What it is") and calls it a 4-bit floating-point type ("Glossary"),
// without values.  The reading used is the E2M1 element type of the Open
// Compute Project's microscaling formats specification, divided by 6.
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
#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdio>
#include <cstring>

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

uint32_t count_code(float v, const Codebook& cb) {
  uint32_t c = 0;
  for (int i = 0; i < 15; ++i) c += (v >= cb.thresh[i]) ? 1u : 0u;
  return c;
}

float from_bits(uint32_t u) {
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

}  // namespace

// Builds the bucket table and checks, for every one of the 2048 buckets, that
// the bucket rule reproduces the threshold count at both ends of the bucket
// (the count is monotone, so that covers every value inside).  A failed check
// is reported through `err` (and the function returns false); the table is
// then unusable and the quantizer refuses to run.
bool build_lut(const Codebook& cb, QuantLut* out, char* err, size_t err_len) {
  QuantLut lut{};
  for (int b = 0; b < kLutBuckets; ++b) {
    const uint32_t sign = static_cast<uint32_t>(b) >> 10;
    const uint32_t lo_mag = static_cast<uint32_t>(b & 1023) << 21, hi_mag = lo_mag | 0x1FFFFFu;
    if ((lo_mag >> 23) > 127 || ((lo_mag >> 23) == 127 && lo_mag != 0x3F800000u)) continue;  // |v| > 1 never occurs
    const uint32_t hi_bits = std::min(hi_mag, 0x3F800000u);
    const float lo_v = from_bits((sign << 31) | (sign ? hi_bits : lo_mag));  // smallest value in bucket
    const float hi_v = from_bits((sign << 31) | (sign ? lo_mag : hi_bits));  // largest value in bucket
    const uint32_t c_lo = count_code(lo_v, cb), c_hi = count_code(hi_v, cb);
    const int e = static_cast<int>(lo_mag >> 23);
    if (c_hi > c_lo + 1) {
      std::snprintf(err, err_len, "quantizer table self-check: bucket %d holds two decision thresholds", b);
      return false;
    }
    if (e < kLutFirstExp) {
      if (c_lo != 7 || c_hi != 7) {
        std::snprintf(err, err_len, "quantizer table self-check: bucket %d below 2^-5 is not the zero level", b);
        return false;
      }
      continue;
    }
    int t = -1;
    for (int k = 0; k < kLutSpecial; ++k)
      if (lut_special_index(k) == b) t = k;
    if (t < 0) {
      std::snprintf(err, err_len, "quantizer table self-check: bucket %d is missing from the table", b);
      return false;
    }
    lut.base[t] = c_lo;
    lut.thr[t] = (c_hi == c_lo) ? INFINITY : cb.thresh[c_lo];
  }
  *out = lut;
  if (err_len) err[0] = '\0';
  return true;
}

namespace {

// FP4 (the E2M1 reading): a 4-bit pattern is a sign bit, two exponent bits
// with bias 1 and one mantissa bit, exponent field 0 being subnormal (m / 2);
// the level is that value divided by 6, so the largest magnitude is 1.
double e2m1(int code) {
  const int e = (code >> 1) & 3, m = code & 1;
  const double mag = e == 0 ? 0.5 * m : (1.0 + 0.5 * m) * std::ldexp(1.0, e - 1);
  return (code & 8) ? -mag : mag;
}

Codebook build_fp4() {
  Codebook cb{};
  for (int c = 0; c < 16; ++c) cb.level[c] = static_cast<float>(e2m1(c) / 6.0);
  for (int i = 0; i < 16; ++i) cb.thresh[i] = INFINITY;  // unused: the quantizer uses the ascending form
  return cb;
}

// The 15 producible FP4 levels in ascending order (index c <-> pattern
// c >= 7 ? c - 7 : 15 - c), with a 16th entry equal to the last whose
// threshold is never reached, so that the NF4 bucket construction applies.
Codebook build_fp4_ascending() {
  const Codebook by_code = build_fp4();
  Codebook cb{};
  for (int c = 0; c < 15; ++c) cb.level[c] = by_code.level[c >= 7 ? c - 7 : 15 - c];
  cb.level[15] = cb.level[14];
  for (int i = 0; i < 14; ++i) cb.thresh[i] = decision_threshold(cb.level[i], cb.level[i + 1]);
  cb.thresh[14] = INFINITY;
  cb.thresh[15] = INFINITY;
  return cb;
}

}  // namespace

const Codebook& codebook(int fp4) {
  static const Codebook nf4 = build();
  static const Codebook f4 = build_fp4();
  return fp4 ? f4 : nf4;
}

namespace {

struct LutState {
  QuantLut lut;
  bool ok;
  char err[160];
};

LutState make_lut_state(const Codebook& cb) {
  LutState st{};
  st.ok = build_lut(cb, &st.lut, st.err, sizeof st.err);
  return st;
}

}  // namespace

const QuantLut* quant_lut(int fp4, const char** err) {
  static const LutState nf4 = make_lut_state(codebook(0));
  static const LutState f4 = make_lut_state(build_fp4_ascending());
  const LutState& st = fp4 ? f4 : nf4;
  if (!st.ok) {
    if (err) *err = st.err;
    return nullptr;
  }
  return &st.lut;
}

}  // namespace nf4i
