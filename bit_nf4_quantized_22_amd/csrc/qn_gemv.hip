// Decode-path kernels (gfx950): the skinny LoRA projections u = x A^T and
// t = dy B, and the dequant-GEMV y = x W^T + s u B^T for M <= 16 tokens.
//
// [kwkr "QLoRA原理深入" §2.3] the 4-bit weight is expanded to 16 bits only
// inside the product; [rkmt "QLORA技术解析" §2.1, §3.3] LoRA bypass B A
// scaled by alpha / r.
//
// GEMV design: the weight stream (0.516 byte per weight) is the only HBM
// traffic that matters, so the kernel keeps the VALU work per weight small.
// The 16x16x32 bf16 MFMA does the multiply-adds (VALU would need 16 FMAs per
// weight at M = 16); the weight operand is the *unscaled* code value
// bf16(q[code]) looked up two codes at a time from a 256-entry byte table in
// LDS, and the block constant c' is applied once per 64-weight block to the
// fp32 partial sum (4 FMAs per lane per block).  Every MFMA therefore covers
// the 16 rows x 32 k-slots of one block: lane (n = l%16, g = l/16) holds codes
// k = 64b + 16g + [0, 16) of row n (one 8-byte load), and the two MFMAs of a
// block take the first and second 8 of them; the x operand uses the same
// k-slot map.

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// out[M, r] = in[M, L] * P^T.  One workgroup per 16 rows of `in`; its 4
// waves split L in 32-wide slices; MFMA 16x16x32 with in-rows as the M side
// and up to 8 column tiles of 16 (r <= 128).
template <bool kPRowMajor>
__global__ __launch_bounds__(256) void skinny_kernel(const uint16_t* __restrict__ in, int64_t M,
                                                     int64_t L, const uint16_t* __restrict__ P,
                                                     int r, float scale,
                                                     float* __restrict__ out_f32,
                                                     uint16_t* __restrict__ out_sbf16,
                                                     uint16_t* __restrict__ out_bf16) {
  __shared__ float sred[4][8][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mi = lane & 15, g = lane >> 4;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 16 + mi;
  const int ncol = (r + 15) >> 4;
  f32x4_t acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = 32 * wave; k0 < L; k0 += 128) {
    const int64_t kk = k0 + 8 * g;
    uint4 a = make_uint4(0, 0, 0, 0);
    if (m < M) a = *reinterpret_cast<const uint4*>(in + m * L + kk);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (c < ncol) {
        const int j = c * 16 + mi;
        uint4 b = make_uint4(0, 0, 0, 0);
        if (j < r) {
          if constexpr (kPRowMajor) {
            b = *reinterpret_cast<const uint4*>(P + static_cast<int64_t>(j) * L + kk);
          } else {
            uint32_t e[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) e[t] = P[(kk + t) * r + j];
            b = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                           e[6] | (e[7] << 16));
          }
        }
        acc[c] = mfma16(a, b, acc[c]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c)
    if (c < ncol)
#pragma unroll
      for (int v = 0; v < 4; ++v) sred[wave][c][4 * g + v][mi] = acc[c][v];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 16 * ncol * 16; idx += 256) {
    const int row = idx / (ncol * 16), col = idx % (ncol * 16);
    const int c = col >> 4, cj = col & 15;
    const int64_t mm = static_cast<int64_t>(blockIdx.x) * 16 + row;
    if (mm >= M || col >= r) continue;
    const float v = sred[0][c][row][cj] + sred[1][c][row][cj] + sred[2][c][row][cj] +
                    sred[3][c][row][cj];
    const int64_t o = mm * r + col;
    if (out_f32) out_f32[o] = v;
    if (out_sbf16) out_sbf16[o] = static_cast<uint16_t>(pack_bf16x2(scale * v, 0.f) & 0xFFFF);
    if (out_bf16) out_bf16[o] = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xFFFF);
  }
}

// Dequant-GEMV.  One workgroup per 16 output features (rows of W); its NW
// waves take groups of 4 consecutive blocks round-robin along K and the
// partial sums meet in LDS; the workgroup then adds the LoRA term and
// writes y as bf16.
template <int NW>
__global__ __launch_bounds__(NW * 64) void gemv_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ gscale, const float* __restrict__ absmax, int64_t N, int64_t K,
    const uint16_t* __restrict__ x, int M, const float* __restrict__ u,
    const uint16_t* __restrict__ B, int r, float s, uint16_t* __restrict__ y,
    PairBf16Params P) {
  __shared__ uint32_t spair[256];
  __shared__ float spart[NW][16][17];
  for (int i = threadIdx.x; i < 256; i += NW * 64) spair[i] = P.pair[i];
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t n = n0 + nl;
  const int64_t nblk = K >> 6;
  const uint8_t* wrow = packed + n * (K >> 1);
  const bool xvalid = nl < M;
  const uint16_t* xrow = x + static_cast<int64_t>(xvalid ? nl : 0) * K;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};

  for (int64_t b0 = 4 * wave; b0 < nblk; b0 += 4 * NW) {
    uint2 wv[4];
    float cs[4];
    uint4 xa[4][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t b = b0 + q;
      wv[q] = make_uint2(0, 0);
      cs[q] = 0.f;
      xa[q][0] = xa[q][1] = make_uint4(0, 0, 0, 0);
      if (b < nblk) {
        wv[q] = *reinterpret_cast<const uint2*>(wrow + b * 32 + g * 8);
        cs[q] = block_scale(qscale, gscale, absmax, n * nblk + b);
        if (xvalid) {
          const uint4* xp = reinterpret_cast<const uint4*>(xrow + b * 64 + g * 16);
          xa[q][0] = xp[0];
          xa[q][1] = xp[1];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w0 = wv[q].x, w1 = wv[q].y;
      const uint4 d0 = make_uint4(spair[w0 & 0xFF], spair[(w0 >> 8) & 0xFF],
                                  spair[(w0 >> 16) & 0xFF], spair[w0 >> 24]);
      const uint4 d1 = make_uint4(spair[w1 & 0xFF], spair[(w1 >> 8) & 0xFF],
                                  spair[(w1 >> 16) & 0xFF], spair[w1 >> 24]);
      f32x4_t t = mfma16(xa[q][0], d0, zero);
      t = mfma16(xa[q][1], d1, t);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] = fmaf(cs[q], t[v], acc[v]);
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) spart[wave][4 * g + v][nl] = acc[v];
  __syncthreads();

  for (int idx = threadIdx.x; idx < 16 * M; idx += NW * 64) {
    const int m = idx >> 4, nn = idx & 15;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += spart[w][m][nn];
    if (r > 0) {
      float lora = 0.f;
      const uint16_t* brow = B + (n0 + nn) * r;
      const float* urow = u + static_cast<int64_t>(m) * r;
      for (int j = 0; j < r; ++j) lora = fmaf(urow[j], bf16_to_f32(brow[j]), lora);
      v = fmaf(s, lora, v);
    }
    y[static_cast<int64_t>(m) * N + n0 + nn] = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xFFFF);
  }
}

}  // namespace

hipError_t launch_skinny(const uint16_t* in, int64_t M, int64_t L, const uint16_t* P,
                         bool p_is_rl, int r, float scale, float* out_f32,
                         uint16_t* out_scaled_bf16, uint16_t* out_bf16, hipStream_t s) {
  if (M == 0 || r == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>((M + 15) / 16));
  if (p_is_rl)
    hipLaunchKernelGGL(skinny_kernel<true>, grid, dim3(256), 0, s, in, M, L, P, r, scale,
                       out_f32, out_scaled_bf16, out_bf16);
  else
    hipLaunchKernelGGL(skinny_kernel<false>, grid, dim3(256), 0, s, in, M, L, P, r, scale,
                       out_f32, out_scaled_bf16, out_bf16);
  return hipGetLastError();
}

hipError_t launch_gemv(const WeightView& w, const uint16_t* x, int M, const float* u,
                       const uint16_t* B, int r, float s, uint16_t* y, hipStream_t st) {
  if (M == 0 || w.N == 0) return hipSuccess;
  const Tables* t = tables();
  PairBf16Params P;
  for (int i = 0; i < 256; ++i) P.pair[i] = t->pair_bf16[i];
  const dim3 grid(static_cast<uint32_t>(w.N / 16));
  constexpr int NW = 8;
  hipLaunchKernelGGL(gemv_kernel<NW>, grid, dim3(NW * 64), 0, st, w.packed, w.qscale, w.gscale,
                     w.absmax, w.N, w.K, x, M, u, B, r, s, y, P);
  return hipGetLastError();
}

}  // namespace qn
