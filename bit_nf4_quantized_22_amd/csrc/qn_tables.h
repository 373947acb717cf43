// Host-built, read-only tables shared by the launchers of the QLoRA NF4
// library.  Built once (thread-safe) on first use; never written afterwards.
#pragma once

#include <cstdint>

namespace qn {

// Bucket table of the quantiser: the fp32 value v = w / c (|v| <= 1) maps to
// bucket idx = min((uint32)fmaf(v, scale, scale), nb - 1); each bucket holds
// at most one code threshold `thr` and `base` = number of thresholds in the
// lower buckets, so code(v) = base + (v > thr).
constexpr int kMaxBuckets = 160;

struct QuantBucket {
  float thr;      // threshold inside the bucket (+inf if none)
  uint32_t base;  // codes below the bucket
};

// Code tables of the 4-bit weight: NF4, or FP4 (E2M1 / 6, zero twice).
constexpr int kQuantNF4 = 0;
constexpr int kQuantFP4 = 1;

struct Tables {
  float q32[16];         // code points, fp32, ascending
  float thr[15];         // largest fp32 <= fp64 mid-point of q32[i], q32[i+1]
  float l8[256];         // level-2 code values fl32(q / 255)
  float thr8[255];       // largest fp32 <= fp64 mid-point of l8[j], l8[j+1]
  float bucket_scale;    // see QuantBucket
  int nbuckets;
  QuantBucket buckets[kMaxBuckets];
  uint32_t pair_bf16[256];  // byte -> bf16(q32[hi nibble]) | bf16(q32[lo]) << 16
  float pair_f32[512];      // byte -> q32[hi nibble], q32[lo nibble]
};

// The tables of a code type (kQuantNF4 or kQuantFP4), built on first call.
// Returns nullptr for an unknown type or if construction failed its own
// consistency checks (never expected).
const Tables* tables(int quant_type = kQuantNF4);

// fp64 inverse of the standard normal CDF (exposed for the codebook).
double inv_norm_cdf(double p);

}  // namespace qn
