// Host construction of the read-only tables: code points (NF4 or FP4), the
// exact fp32 decision thresholds of the nearest-code search, the 8-bit level
// table of the double quantisation, and the byte-pair decode tables.
//
// NF4 code points: [kwkr "QLoRA原理深入" §2.2] standard-normal quantiles as
// code points; [rkmt "QLORA技术解析" §2.2.1] quantiles of a truncated normal
// splitting the area into equal parts; [czcl "QLoRA技術解析" §2.1] exact zero.
// Construction: 8 equal probability steps from 1/2 to P on the positive
// side, 7 on the negative side, plus 0, divided by the quantile at P, with
// P = 1 - (1/32 + 1/30)/2 (the truncation point is not given on the pages;
// this is the value chosen).
//
// FP4 code points: [kwkr "QLoRA原理深入" §4.1] names fp4 as the alternative
// type (made for floating-point distributions, worse than NF4 for weights)
// without giving its format.  Taken as E2M1 (sign, 2 exponent bits, 1
// mantissa bit: magnitudes 0, 1/2, 1, 3/2, 2, 3, 4, 6) divided by 6, so the
// block absmax maps to the largest code; its 15 values fill 16 ascending
// entries with 0 at indices 7 and 8.

#include "qn_tables.h"

#include <cmath>
#include <cstring>
#include <mutex>

namespace qn {

// Inverse standard-normal CDF in fp64.  Initial value: P. J. Acklam's
// rational approximation ("An algorithm for computing the inverse normal
// cumulative distribution function", 2003; relative error < 1.15e-9),
// followed by Halley steps on the residual Phi(x) - p computed with erfc,
// as Acklam describes, which brings it to fp64 rounding level.
double inv_norm_cdf(double p) {
  static const double a[6] = {-3.969683028665376e+01, 2.209460984245205e+02,
                              -2.759285104469687e+02, 1.383577518672690e+02,
                              -3.066479806614716e+01, 2.506628277459239e+00};
  static const double b[5] = {-5.447609879822406e+01, 1.615858368580409e+02,
                              -1.556989798598866e+02, 6.680131188771972e+01,
                              -1.328068155288572e+01};
  static const double c[6] = {-7.784894002430293e-03, -3.223964580411365e-01,
                              -2.400758277161838e+00, -2.549732539343734e+00,
                              4.374664141464968e+00, 2.938163982698783e+00};
  static const double d[4] = {7.784695709041462e-03, 3.224671290700398e-01,
                              2.445134137142996e+00, 3.754408661907416e+00};
  const double p_low = 0.02425, p_high = 1.0 - p_low;
  double x;
  if (p < p_low) {
    double q = std::sqrt(-2.0 * std::log(p));
    x = (((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
        ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1.0);
  } else if (p <= p_high) {
    double q = p - 0.5, r = q * q;
    x = (((((a[0] * r + a[1]) * r + a[2]) * r + a[3]) * r + a[4]) * r + a[5]) * q /
        (((((b[0] * r + b[1]) * r + b[2]) * r + b[3]) * r + b[4]) * r + 1.0);
  } else {
    double q = std::sqrt(-2.0 * std::log1p(-p));
    x = -(((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
        ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1.0);
  }
  const double sqrt2 = std::sqrt(2.0), sqrt2pi = std::sqrt(2.0 * M_PI);
  for (int it = 0; it < 3; ++it) {
    double e = 0.5 * std::erfc(-x / sqrt2) - p;
    double u = e * sqrt2pi * std::exp(0.5 * x * x);
    x = x - u / (1.0 + 0.5 * x * u);
  }
  return x;
}

namespace {

// Largest fp32 <= m.
float round_down_f32(double m) {
  float f = static_cast<float>(m);
  if (static_cast<double>(f) > m) f = std::nextafter(f, -INFINITY);
  return f;
}

uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Same bucket function as the quantiser kernel.
uint32_t bucket_of(float v, float scale, int nb) {
  float f = std::fmaf(v, scale, scale);
  f = std::fmin(std::fmax(f, 0.0f), static_cast<float>(nb - 1));
  return static_cast<uint32_t>(f);
}

bool build_buckets(Tables& t) {
  // Every threshold must sit at least `margin` inside its bucket (the
  // kernel's fast path compares an approximate quotient, see quantiser).
  const float margin = std::ldexp(1.0f, -19);
  // Integer scales put v = 0 on a bucket edge; FP4 has a threshold there,
  // so half-integer scales follow.
  static const float scales[] = {32.f, 31.f, 33.f, 30.f, 34.f, 29.f, 35.f, 28.f,
                                 36.f, 27.f, 37.f, 40.f, 44.f, 48.f, 24.5f, 25.5f,
                                 26.5f, 27.5f, 28.5f, 29.5f, 30.5f, 31.5f, 36.5f, 48.5f};
  for (float s : scales) {
    int nb = static_cast<int>(2 * s) + 1;
    if (nb > kMaxBuckets) continue;
    uint32_t bidx[15];
    bool ok = true;
    for (int i = 0; i < 15 && ok; ++i) {
      bidx[i] = bucket_of(t.thr[i], s, nb);
      ok = bucket_of(t.thr[i] - margin, s, nb) == bidx[i] &&
           bucket_of(t.thr[i] + margin, s, nb) == bidx[i] &&
           (i == 0 || bidx[i] > bidx[i - 1]);
    }
    if (!ok) continue;
    t.bucket_scale = s;
    t.nbuckets = nb;
    for (int b = 0; b < nb; ++b) {
      t.buckets[b].thr = INFINITY;
      uint32_t base = 0;
      for (int i = 0; i < 15; ++i) {
        if (bidx[i] < static_cast<uint32_t>(b)) ++base;
        if (bidx[i] == static_cast<uint32_t>(b)) t.buckets[b].thr = t.thr[i];
      }
      t.buckets[b].base = base;
    }
    return true;
  }
  return false;
}

Tables g_tables[2];
const Tables* g_ptr[2] = {nullptr, nullptr};
std::once_flag g_once;

// NF4 code points, fp64, ascending.
void nf4_points(double q[16]) {
  const double pmax = 929.0 / 960.0;  // 1 - (1/32 + 1/30) / 2, exact ratio
  const double top = inv_norm_cdf(pmax);
  for (int j = 1; j <= 7; ++j)  // negative side: probabilities 1/2 + 449 j / 6720
    q[7 - j] = -inv_norm_cdf((3360.0 + 449.0 * j) / 6720.0) / top;
  q[7] = 0.0;
  for (int j = 1; j <= 8; ++j)  // positive side: probabilities 1/2 + 449 j / 7680
    q[7 + j] = inv_norm_cdf((3840.0 + 449.0 * j) / 7680.0) / top;
  // Both ends evaluate the quantile at exactly P (6503/6720 = 7432/7680 =
  // 929/960), so they come out as exactly -1 and +1; checked below.
}

// FP4 code points: E2M1 magnitudes / 6, negatives mirrored, 0 twice.
void fp4_points(double q[16]) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  for (int i = 0; i < 8; ++i) {
    q[8 + i] = mag[i] / 6.0;
    q[7 - i] = -mag[i] / 6.0;
  }
  q[7] = 0.0;  // +0, not -0
}

bool build_one(Tables& t, const double q[16], bool twin_zero) {
  for (int i = 0; i < 16; ++i) t.q32[i] = static_cast<float>(q[i]);
  for (int i = 0; i < 15; ++i)
    t.thr[i] = round_down_f32((static_cast<double>(t.q32[i]) + t.q32[i + 1]) * 0.5);
  for (int k = 0; k < 256; ++k) t.l8[k] = static_cast<float>(k) / 255.0f;
  for (int k = 0; k < 255; ++k)
    t.thr8[k] = round_down_f32((static_cast<double>(t.l8[k]) + t.l8[k + 1]) * 0.5);
  for (int b = 0; b < 256; ++b) {
    float hi = t.q32[b >> 4], lo = t.q32[b & 15];
    t.pair_bf16[b] = static_cast<uint32_t>(bf16_rne(hi)) |
                     (static_cast<uint32_t>(bf16_rne(lo)) << 16);
    t.pair_f32[2 * b] = hi;
    t.pair_f32[2 * b + 1] = lo;
  }
  bool ok = build_buckets(t);
  for (int i = 0; i < 15; ++i)
    ok = ok && (t.q32[i] < t.q32[i + 1] || (twin_zero && i == 7 && t.q32[i] == t.q32[i + 1]));
  uint32_t zbits;
  std::memcpy(&zbits, &t.q32[7], 4);
  ok = ok && zbits == 0u && t.q32[0] == -1.0f && t.q32[15] == 1.0f;
  return ok;
}

void build() {
  double q[16];
  nf4_points(q);
  if (build_one(g_tables[kQuantNF4], q, false)) g_ptr[kQuantNF4] = &g_tables[kQuantNF4];
  fp4_points(q);
  if (build_one(g_tables[kQuantFP4], q, true)) g_ptr[kQuantFP4] = &g_tables[kQuantFP4];
}

}  // namespace

const Tables* tables(int quant_type) {
  std::call_once(g_once, build);
  return quant_type == kQuantNF4 || quant_type == kQuantFP4 ? g_ptr[quant_type] : nullptr;
}

}  // namespace qn
