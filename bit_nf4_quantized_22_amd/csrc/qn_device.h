// Device-side helpers shared by the HIP kernels of the library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qn_launch.h"
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

// Level-2 value fl32(q / 255) (same value as the host table): x = q r with
// r = fl32(1 / 255), then one Newton correction x + fma(-x, 255, q) r.  For
// every q = 0..255 this is the correctly rounded IEEE quotient (checked
// exhaustively with exact rationals), at three operations instead of a
// division sequence.
__device__ __forceinline__ float l8_value(uint32_t q) {
  const float qf = static_cast<float>(q), r = 1.0f / 255.0f;
  const float x = qf * r;
  return fmaf(fmaf(-x, 255.0f, qf), r, x);
}

// Value of a non-negative E4M3 code q < 0x7F (4 exponent bits, bias 7, 3
// mantissa bits; subnormals m 2^-9), exact in fp32.
__device__ __forceinline__ float e4m3_value(uint32_t q) {
  const uint32_t e = q >> 3, m = q & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : static_cast<float>(m) * 0x1p-9f;
}

// Nearest E4M3 code of v in [0, 1], ties to the even code: below 2^-6 the
// subnormal k 2^-9 with k = rne(512 v) (exact scaling; k = 8 is the first
// normal code), above it the fp32 significand rounded to 3 bits.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  if (v < 0x1p-6f) return static_cast<uint32_t>(__builtin_rintf(v * 512.0f));
  const uint32_t b = __float_as_uint(v);
  const uint32_t m = b & 0x7FFFFFu, rem = m & 0xFFFFFu;
  const uint32_t code = (((b >> 23) - 120u) << 3) | (m >> 20);
  return code + ((rem > 0x80000u || (rem == 0x80000u && (code & 1u))) ? 1u : 0u);
}

// Level of a signed code byte q (two's complement k): fl32(k / 127), by the
// same three operations as l8_value (correctly rounded for every k in
// -128..127, checked exhaustively with exact rationals).
__device__ __forceinline__ float s8_value(uint32_t q) {
  const float kf = static_cast<float>(static_cast<int>(static_cast<int8_t>(q & 0xFFu)));
  const float r = 1.0f / 127.0f;
  const float x = kf * r;
  return fmaf(fmaf(-x, 127.0f, kf), r, x);
}

// Level-2 value of code q of the given kind.
__device__ __forceinline__ float l2_value(uint32_t q, int kind) {
  return kind == kL2E4M3 ? e4m3_value(q) : kind == kL2Centred ? s8_value(q) : l8_value(q);
}

// fl32(fl32(a b) + c), rounded twice.  hipcc contracts a multiply feeding
// an add into one fused multiply-add (a single rounding) even through
// __fmul_rn / __fadd_rn; the empty asm hides the product from that.
__device__ __forceinline__ float mul_then_add(float a, float b, float c) {
  float p = a * b;
  asm("" : "+v"(p));
  return p + c;
}

// Double-dequantised block constant c' = fl32(fl32(L2[q] * c2) + mu); mu is
// the centred code's offset and 0 for the others (adding +0 leaves the
// non-negative product unchanged, bit for bit).
__device__ __forceinline__ float dq_value(uint32_t q, float c2, int kind, float mu) {
  return mul_then_add(l2_value(q, kind), c2, mu);
}

// Block constant c' of block `bi` of a quantised weight: double-dequantised
// when qscale != nullptr, else the stored fp32 absmax.
__device__ __forceinline__ float block_scale(const uint8_t* __restrict__ qscale,
                                             const float* __restrict__ gscale,
                                             const float* __restrict__ absmax, int64_t bi,
                                             int kind, float mu) {
  if (qscale) return dq_value(qscale[bi], gscale[bi >> 8], kind, mu);
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

// Kernel parameters.  Tables are never indexed per lane out of the kernel
// argument segment (that becomes a vector load per lane at the start of
// every workgroup); each kernel builds its LDS tables from a few scalars
// read with wave-uniform indices.

// The 16 code values of the weight's table (fp32, ascending), the kind of
// its level-2 code (kL2*) and, for the centred code, the device address of
// its offset mu (nullptr otherwise).
struct CodeParams {
  float q[16];
  int l2;
  const float* mu;
};

// The offset to add to every double-dequantised constant (one scalar load,
// wave-uniform).
__device__ __forceinline__ float l2_offset(const CodeParams& P) {
  return P.mu ? *P.mu : 0.0f;
}

// The 16 code values spread over lanes 0..15 of one VGPR (v_writelane of
// the scalar kernel arguments).  q[c] for a per-lane c is then a
// ds_bpermute from lane c: no memory access and no per-lane select, which
// the compiler would otherwise turn back into an indexed load from the
// argument segment or a scratch array.
struct CodeRegs {
  int lanes;
};

__device__ __forceinline__ CodeRegs code_regs(const CodeParams& P) {
  int v = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(__float_as_int(P.q[i])), "n"(i));
  return CodeRegs{v};
}

__device__ __forceinline__ float code_value(const CodeRegs& R, uint32_t c) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(static_cast<int>(c << 2), R.lanes));
}

// Same for a wave-uniform c: v_readlane, no LDS operation.
__device__ __forceinline__ float code_value_uniform(const CodeRegs& R, uint32_t c) {
  return __int_as_float(__builtin_amdgcn_readlane(R.lanes, static_cast<int>(c)));
}

// LDS byte table, `copies` interleaved copies: entry e of copy k at
// e * copies + k holds (q[e >> 4], q[e & 15]) (even element first).
__device__ __forceinline__ void fill_pair_f32(float2* tab, const CodeParams& P, int copies) {
  const CodeRegs R = code_regs(P);
  for (int i = threadIdx.x; i < 256 * copies; i += blockDim.x) {
    const uint32_t e = i / copies;
    tab[i] = make_float2(code_value(R, e >> 4), code_value(R, e & 15));
  }
}

// Same, as packed bf16 pairs (RNE), low half = even element.
__device__ __forceinline__ void fill_pair_bf16(uint32_t* tab, const CodeParams& P, int copies) {
  const CodeRegs R = code_regs(P);
  for (int i = threadIdx.x; i < 256 * copies; i += blockDim.x) {
    const uint32_t e = i / copies;
    tab[i] = pack_bf16x2(code_value(R, e >> 4), code_value(R, e & 15));
  }
}

// Quantiser: bucket scale, bucket count and the 15 fp32 decision
// thresholds; the bucket table itself is rebuilt in LDS by each workgroup.
struct QuantParams {
  float scale;
  uint32_t nbuckets;
  float thr[15];
};

}  // namespace qn
