// Decode-path kernels (gfx950): the skinny LoRA projections u = x A^T and
// t = dy B, and the dequant-GEMV y = x W^T + s u B^T for M <= 16 tokens.
//
// [kwkr "QLoRA原理深入" §2.3] the 4-bit weight is expanded to 16 bits only
// inside the product; [rkmt "QLORA技术解析" §2.1, §3.3] LoRA bypass B A
// scaled by alpha / r.
//
// GEMV design: the weight stream (0.516 byte per weight) is the only HBM
// traffic that matters.  The 16x16x32 bf16 MFMA does the multiply-adds
// (VALU would need 16 FMAs per weight at M = 16); the weight operand is the
// *unscaled* code value bf16(q[code]) looked up two codes at a time from a
// 256-entry byte table in LDS, and the block constant c' is applied once per
// 64-weight block to the fp32 partial sum (4 FMAs per lane per block).  Every
// MFMA therefore covers the 16 rows x 32 k-slots of one block: lane
// (n = l%16, g = l/16) holds codes k = 64b + 16g + [0, 16) of row n (one
// 8-byte load), and the two MFMAs of a block take the first and second 8 of
// them; the x operand uses the same k-slot map.  Each wave works through
// groups of 4 consecutive blocks and issues the loads of its next group
// before computing the current one.

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

constexpr int kGemvWaves = 8;
constexpr int kUParts = 16;  // LoRA partial sums held per thread in the GEMV
constexpr int kPairCopies = 8;  // lane l uses copy l % 8 (fewer LDS bank conflicts)

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// out[M, r] = in[M, L] * P^T.  Grid: (16-row tiles of `in`) x ksplit; the 4
// waves of a workgroup split its L-slice in 32-wide chunks; MFMA 16x16x32
// with in-rows as the M side and up to 8 column tiles of 16 (r <= 128).
// ksplit == 1: writes the finished result (fp32 and/or bf16 forms).
// ksplit > 1: writes fp32 partial sums out_f32[slice][M][r].
template <bool kPRowMajor>
__global__ __launch_bounds__(256) void skinny_kernel(const uint16_t* __restrict__ in, int64_t M,
                                                     int64_t L, const uint16_t* __restrict__ P,
                                                     int r, float scale, int ksplit,
                                                     float* __restrict__ out_f32,
                                                     uint16_t* __restrict__ out_sbf16,
                                                     uint16_t* __restrict__ out_bf16) {
  __shared__ float sred[4][8][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mi = lane & 15, g = lane >> 4;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 16 + mi;
  const int64_t mc = m < M ? m : M - 1;  // clamped: rows >= M are never stored
  const int ncol = (r + 15) >> 4;
  const int64_t nchunk = L >> 5;
  const int64_t c_lo = nchunk * blockIdx.y / ksplit, c_hi = nchunk * (blockIdx.y + 1) / ksplit;
  f32x4_t acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t ch = c_lo + wave; ch < c_hi; ch += 4) {
    const int64_t kk = ch * 32 + 8 * g;
    const uint4 a = *reinterpret_cast<const uint4*>(in + mc * L + kk);
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
    if (ksplit > 1) {
      out_f32[static_cast<int64_t>(blockIdx.y) * M * r + o] = v;
      continue;
    }
    if (out_f32) out_f32[o] = v;
    if (out_sbf16) out_sbf16[o] = static_cast<uint16_t>(pack_bf16x2(scale * v, 0.f) & 0xFFFF);
    if (out_bf16) out_bf16[o] = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xFFFF);
  }
}

// Dequant-GEMV.  One workgroup (8 waves) per band of 16 output features
// (rows of W).  Wave w owns a contiguous slice of at most kGemvMaxBlocks
// blocks of the band's K range (longer rows are done in several passes) and
// issues all of its weight loads (8 bytes per lane per block) and block
// constants at once, before anything else: the whole weight matrix is in
// flight almost from the start, which is what an HBM-latency-bound stream
// needs.  x is read per block, two blocks ahead.  Partial sums meet in LDS;
// the workgroup adds the LoRA term (u as `usplit` fp32 partial sums
// [usplit][M][r]) and writes y as bf16.
constexpr int kGemvMaxBlocks = 24;

template <bool kDQ>
__global__ __launch_bounds__(kGemvWaves * 64) void gemv_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ gscale, const float* __restrict__ absmax, int64_t N, int64_t K,
    const uint16_t* __restrict__ x, int M, const float* __restrict__ u, int usplit,
    const uint16_t* __restrict__ B, int r, float s, uint16_t* __restrict__ y,
    uint16_t* __restrict__ u_out, CodeParams P) {
  __shared__ uint32_t spair[256 * kPairCopies];
  __shared__ float sl8[256];
  __shared__ float spart[kGemvWaves][16][17];
  __shared__ float su[16 * 128];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int nl = lane & 15, g = lane >> 4;
  const int64_t nblk = K >> 6;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t n = n0 + nl;
  const uint8_t* wrow = packed + n * (K >> 1);
  // Lanes of token rows >= M read row M - 1 (unconditional loads keep the
  // load counter exact) and zero the value.
  const bool xvalid = nl < M;
  const uint16_t* xrow = x + static_cast<int64_t>(xvalid ? nl : M - 1) * K;
  const int64_t rowblk0 = n * nblk;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc = zero;

  // LoRA partial sums: loaded first (thread t owns elements t, t + 512, ..
  // of u[M][r], kUParts values in all), summed after the main loop, so their
  // latency hides behind the weight stream.  The host keeps
  // usplit * ceil(M r / 512) <= kUParts.
  const int mr = M * r;
  const int ue = (mr + kGemvWaves * 64 - 1) / (kGemvWaves * 64);
  float upart[kUParts];
#pragma unroll
  for (int q = 0; q < kUParts; ++q) {
    const int e = q / usplit, sp = q % usplit;
    const int idx = threadIdx.x + e * kGemvWaves * 64;
    upart[q] = (e < ue && idx < mr) ? u[static_cast<int64_t>(sp) * mr + idx] : 0.f;
  }

  const int64_t per_pass = static_cast<int64_t>(kGemvWaves) * kGemvMaxBlocks;
  bool tables_ready = false;
  for (int64_t pass0 = 0; pass0 < nblk; pass0 += per_pass) {
    const int64_t pass_n = min(per_pass, nblk - pass0);
    const int64_t b_lo = pass0 + pass_n * wave / kGemvWaves;
    const int64_t b_hi = pass0 + pass_n * (wave + 1) / kGemvWaves;
    const int nb = static_cast<int>(b_hi - b_lo);

    // 1. all weight loads and block constants of this wave's slice
    uint2 w[kGemvMaxBlocks];
    float cq[kGemvMaxBlocks];
#pragma unroll
    for (int i = 0; i < kGemvMaxBlocks; ++i) {
      // clamped into the slice (an empty slice reads its first block, which
      // exists since b_lo < nblk); blocks past the slice are skipped below
      const int64_t b = b_lo + min(i, max(nb - 1, 0));
      w[i] = *reinterpret_cast<const uint2*>(wrow + b * 32 + g * 8);
      if constexpr (kDQ) cq[i] = __uint_as_float(static_cast<uint32_t>(qscale[rowblk0 + b]));
      else cq[i] = absmax[rowblk0 + b];
    }
    float g_lo = 0.f, g_hi = 0.f;
    if constexpr (kDQ) {
      g_lo = gscale[(rowblk0 + b_lo) >> 8];
      g_hi = gscale[(rowblk0 + max(b_hi - 1, b_lo)) >> 8];
    }

    // 2. tables (once), overlapping the loads
    if (!tables_ready) {
      fill_pair_bf16(spair, P, kPairCopies);
      for (int i = threadIdx.x; i < 256; i += kGemvWaves * 64) sl8[i] = l8_value(i);
      __syncthreads();
      tables_ready = true;
    }

    // 3. walk the slice: x two blocks ahead, decode, MFMA, block scale
    const int cp = threadIdx.x & (kPairCopies - 1);
    uint4 xa[3][2];  // x of blocks i, i+1, i+2 in slots i % 3, ...
    auto load_x = [&](int i) {
      const uint4* xp = reinterpret_cast<const uint4*>(xrow + (b_lo + i) * 64 + g * 16);
      xa[i % 3][0] = xp[0];
      xa[i % 3][1] = xp[1];
    };
    auto x_of = [&](int slot, int h) {
      const uint4 v = xa[slot][h];
      return xvalid ? v : make_uint4(0, 0, 0, 0);
    };
    if (nb > 0) load_x(0);
    if (nb > 1) load_x(1);
#pragma unroll
    for (int i = 0; i < kGemvMaxBlocks; ++i) {
      if (i < nb) {
        if (i + 2 < nb) load_x(i + 2);
        const uint32_t w0 = w[i].x, w1 = w[i].y;
        const uint4 d0 = make_uint4(spair[(w0 & 0xFF) * kPairCopies + cp],
                                    spair[((w0 >> 8) & 0xFF) * kPairCopies + cp],
                                    spair[((w0 >> 16) & 0xFF) * kPairCopies + cp],
                                    spair[(w0 >> 24) * kPairCopies + cp]);
        const uint4 d1 = make_uint4(spair[(w1 & 0xFF) * kPairCopies + cp],
                                    spair[((w1 >> 8) & 0xFF) * kPairCopies + cp],
                                    spair[((w1 >> 16) & 0xFF) * kPairCopies + cp],
                                    spair[(w1 >> 24) * kPairCopies + cp]);
        f32x4_t t = mfma16(x_of(i % 3, 0), d0, zero);
        t = mfma16(x_of(i % 3, 1), d1, t);
        float cs;
        if constexpr (kDQ) {
          const int64_t b = b_lo + i;
          const float c2 = ((rowblk0 + b) >> 8) == ((rowblk0 + b_lo) >> 8) ? g_lo : g_hi;
          cs = __fmul_rn(sl8[__float_as_uint(cq[i])], c2);
        } else {
          cs = cq[i];
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = fmaf(cs, t[v], acc[v]);
      }
    }
  }
  // LoRA down-projection: sum the partials loaded at the start.
#pragma unroll
  for (int e = 0; e < kUParts; ++e) {
    if (e < ue) {
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < kUParts; ++q)
        if (q / usplit == e) v += upart[q];
      const int idx = threadIdx.x + e * kGemvWaves * 64;
      if (idx < mr) su[idx] = v;
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) spart[wave][4 * g + v][nl] = acc[v];
  __syncthreads();
  if (u_out && blockIdx.x == 0)
    for (int i = threadIdx.x; i < M * r; i += kGemvWaves * 64)
      u_out[i] = static_cast<uint16_t>(pack_bf16x2(su[i], 0.f) & 0xFFFF);
  for (int idx = threadIdx.x; idx < 16 * M; idx += kGemvWaves * 64) {
    const int m = idx >> 4, nn = idx & 15;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < kGemvWaves; ++ww) v += spart[ww][m][nn];
    if (r > 0) {
      float lora = 0.f;
      const uint16_t* brow = B + (n0 + nn) * r;
      for (int j = 0; j < r; ++j) lora = fmaf(su[m * r + j], bf16_to_f32(brow[j]), lora);
      v = fmaf(s, lora, v);
    }
    y[static_cast<int64_t>(m) * N + n0 + nn] = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xFFFF);
  }
}

}  // namespace

int skinny_splits(int64_t M, int64_t L, int r) {
  if (M > 16 || r == 0) return 1;
  // the GEMV holds usplit * ceil(M r / 512) partials per thread
  const int64_t per_thread = (M * r + kGemvWaves * 64 - 1) / (kGemvWaves * 64);
  int ks = static_cast<int>(kUParts / per_thread);
  const int64_t chunks = L >> 5;
  if (ks > chunks / 4) ks = static_cast<int>(chunks / 4);
  return ks < 1 ? 1 : ks;
}

hipError_t launch_skinny(const uint16_t* in, int64_t M, int64_t L, const uint16_t* P,
                         bool p_is_rl, int r, float scale, float* out_f32,
                         uint16_t* out_scaled_bf16, uint16_t* out_bf16, int ksplit,
                         hipStream_t s) {
  if (M == 0 || r == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>((M + 15) / 16), static_cast<uint32_t>(ksplit));
  if (p_is_rl)
    hipLaunchKernelGGL(skinny_kernel<true>, grid, dim3(256), 0, s, in, M, L, P, r, scale, ksplit,
                       out_f32, out_scaled_bf16, out_bf16);
  else
    hipLaunchKernelGGL(skinny_kernel<false>, grid, dim3(256), 0, s, in, M, L, P, r, scale, ksplit,
                       out_f32, out_scaled_bf16, out_bf16);
  return hipGetLastError();
}

hipError_t launch_gemv(const WeightView& w, const uint16_t* x, int M, const float* u, int usplit,
                       const uint16_t* B, int r, float s, uint16_t* y, uint16_t* u_out,
                       hipStream_t st) {
  if (M == 0 || w.N == 0) return hipSuccess;
  const Tables* t = tables();
  CodeParams P;
  for (int i = 0; i < 16; ++i) P.q[i] = t->q32[i];
  const dim3 grid(static_cast<uint32_t>(w.N / 16));
  if (w.qscale)
    hipLaunchKernelGGL(gemv_kernel<true>, grid, dim3(kGemvWaves * 64), 0, st, w.packed, w.qscale,
                       w.gscale, w.absmax, w.N, w.K, x, M, u, usplit, B, r, s, y, u_out, P);
  else
    hipLaunchKernelGGL(gemv_kernel<false>, grid, dim3(kGemvWaves * 64), 0, st, w.packed, w.qscale,
                       w.gscale, w.absmax, w.N, w.K, x, M, u, usplit, B, r, s, y, u_out, P);
  return hipGetLastError();
}

}  // namespace qn
