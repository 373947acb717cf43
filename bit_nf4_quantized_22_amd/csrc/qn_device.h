// Device-side helpers shared by the HIP kernels of the library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qn_tables.h"

namespace qn {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Level-2 value fl32(q / 255), by IEEE division (same value as the host table).
__device__ __forceinline__ float l8_value(uint32_t q) {
  return __fdiv_rn(static_cast<float>(q), 255.0f);
}

// Block constant c' of block `bi` of a quantised weight: double-dequantised
// fl32(L8[q8] * c2) when qscale != nullptr, else the stored fp32 absmax.
__device__ __forceinline__ float block_scale(const uint8_t* __restrict__ qscale,
                                             const float* __restrict__ gscale,
                                             const float* __restrict__ absmax, int64_t bi) {
  if (qscale) return __fmul_rn(l8_value(qscale[bi]), gscale[bi >> 8]);
  return absmax[bi];
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Kernel parameter blocks (passed by value, copied to LDS by each workgroup).
struct QuantParams {
  float scale;
  uint32_t nbuckets;
  QuantBucket bk[kMaxBuckets];
};

struct DqParams {
  float thr8[256];  // thr8[255] = +inf sentinel
};

struct PairF32Params {
  float pair[512];
};

struct PairBf16Params {
  uint32_t pair[256];
};

}  // namespace qn
