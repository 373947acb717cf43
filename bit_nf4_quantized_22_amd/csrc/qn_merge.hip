// LoRA merge (gfx950): out[n, k] = bf16(fl32(q[code] c') + fl32(s * (B A)[n, k])),
// s = alpha / r, the rank-r product accumulated in fp32 by MFMA.
//
// [rkmt "QLORA技术解析" §2.1] for inference the adapter is folded into the
// weight, W <- W + B A, so it costs no latency; [tgd "QLoRA微调" §7] a QLoRA
// adapter is merged into a 16-bit weight, never into the 4-bit form.  The
// weight here is the dequantised 4-bit weight (the value the adapter was
// trained against), expanded on the fly: the merged bf16 weight is the only
// 16-bit copy that is written.  Re-quantising it (nf4_quantize) gives a
// merged 4-bit model.
//
// HBM-bound streaming kernel: per weight it reads half a byte of codes and
// writes two bytes.  The rank-r product runs on the 16x16x32 bf16 MFMA as
// the transposed product (B A)^T = A^T B^T, so a lane's four outputs per
// MFMA are four k of one row n; the k order inside each 64-block is
// permuted so that over the block's four MFMAs a lane owns 16 consecutive
// k.  A lane then reads 8 bytes of codes and one block constant and writes
// 32 bytes per block, and a wave's rows are 32-byte code reads and 128-byte
// stores.  A workgroup (4 waves) owns 64 rows x 256 columns; A's columns
// for them are staged transposed in LDS, B's rows sit in registers.

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

constexpr int kMRows = 64;    // rows of W per workgroup (16 per wave)
constexpr int kMCols = 256;   // columns of W per workgroup (4 blocks)

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// kR: rank capacity (0, 32, 64 or 128); kD = kR / 32 MFMAs per 16 x 16 tile.
template <int kR, bool kDQ>
__global__ __launch_bounds__(256) void merge_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ gscale, const float* __restrict__ absmax, int64_t N, int64_t K,
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int r, float s,
    uint16_t* __restrict__ out, CodeParams P) {
  constexpr int kD = kR / 32;
  constexpr int kRS = kR + 8;  // bf16 per row of the transposed A tile (16-byte pad)
  __shared__ float scode[16 * 64];  // q[c] for lane l at [64 c + l]: no bank conflicts
  __shared__ __attribute__((aligned(16))) uint16_t sat[kR > 0 ? kMCols * kRS : 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * kMRows;
  const int64_t k0 = static_cast<int64_t>(blockIdx.x) * kMCols;
  const int64_t n = n0 + 16 * wave + nl;  // N % 64 == 0: always a valid row
  // The weight loads of all four blocks go first, before the LoRA operands
  // are staged (blocks past K re-read the last block and store nothing):
  // their latency then overlaps the staging and its barrier instead of
  // following it.
  constexpr int kBlk = kMCols / 64;
  uint2 cw[kBlk];
  uint32_t q8[kBlk];
  float c2[kBlk];
#pragma unroll
  for (int blk = 0; blk < kBlk; ++blk) {
    const int64_t kb = k0 + 64 * blk < K ? k0 + 64 * blk : K - 64;
    const int64_t bi = n * (K >> 6) + (kb >> 6);
    // codes of k = kb + 16 g .. + 15 (8 bytes; byte i: k 2i high nibble, 2i + 1 low)
    cw[blk] = *reinterpret_cast<const uint2*>(packed + (n * K + kb + 16 * g) / 2);
    if constexpr (kDQ) {
      q8[blk] = qscale[bi];
      c2[blk] = gscale[bi >> 8];
    } else {
      q8[blk] = 0;
      c2[blk] = absmax[bi];
    }
  }
  const float mu = kDQ ? l2_offset(P) : 0.0f;
  {
    const CodeRegs R = code_regs(P);
    for (int i = tid; i < 16 * 64; i += 256) scode[i] = code_value(R, i >> 6);
  }
  // B row n, columns 32 d + 8 g .. + 7 (zero past r), as MFMA operands
  uint4 bfrag[kD > 0 ? kD : 1];
  if constexpr (kR > 0) {
    // A tile transposed: sat[kk][j] = A[j][k0 + kk], zero for j >= r or
    // columns past K.  Thread tid handles column kk = tid of every row j;
    // all loads are unconditional from clamped addresses (a branch around a
    // load would wait for it at the join), the zeros selected afterwards.
    // Rows j >= r are zero and need no load (r is uniform); each thread's
    // column goes to LDS as 16-byte runs of 8 ranks.
    {
      const int kk = tid;
      const int64_t kc = k0 + kk < K ? k0 + kk : K - 1;
      const bool kin = k0 + kk < K;
      uint32_t av[kR];
#pragma unroll
      for (int j = 0; j < kR; ++j) av[j] = j < r ? A[static_cast<int64_t>(j) * K + kc] : 0u;
#pragma unroll
      for (int q = 0; q < kR / 8; ++q) {
        uint32_t w4[4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
          w4[h] = kin ? ((av[8 * q + 2 * h] & 0xFFFFu) | (av[8 * q + 2 * h + 1] << 16)) : 0u;
        *reinterpret_cast<uint4*>(sat + kk * kRS + 8 * q) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
    }
    // B's row n as one 16-byte load per 8 ranks when r is a multiple of 8
    // (rows of 16-byte multiples; B itself 16-byte aligned), else element
    // by element
    const bool bvec = (r & 7) == 0 && (reinterpret_cast<uintptr_t>(B) & 15) == 0;
#pragma unroll
    for (int d = 0; d < kD; ++d) {
      const int j0 = 32 * d + 8 * g;
      if (bvec) {
        bfrag[d] = j0 < r ? *reinterpret_cast<const uint4*>(B + n * r + j0) : make_uint4(0, 0, 0, 0);
      } else {
        uint32_t bv[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const int j = j0 + h;
          bv[h] = B[n * r + (j < r ? j : r - 1)];
        }
        uint32_t w4[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int j = j0 + 2 * h;
          w4[h] = (j < r ? bv[2 * h] : 0u) | ((j + 1 < r ? bv[2 * h + 1] : 0u) << 16);
        }
        bfrag[d] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
    }
  }
  __syncthreads();

  const uint32_t lane4 = static_cast<uint32_t>(lane) << 2;
  const char* tab = reinterpret_cast<const char*>(scode);
#pragma unroll
  for (int blk = 0; blk < kBlk; ++blk) {
    const int64_t kb = k0 + 64 * blk;  // first column of the block
    const float cs = kDQ ? dq_value(q8[blk], c2[blk], P.l2, mu) : c2[blk];
    f32x4_t t[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      t[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (kR > 0) {
        // MFMA b: output row i is column kb + 16 (i / 4) + 4 b + i % 4, so
        // lane (nl, g) gets k = kb + 16 g + 4 b + [0, 4)
        const int krow = 64 * blk + 16 * (nl >> 2) + 4 * b + (nl & 3);
#pragma unroll
        for (int d = 0; d < kD; ++d) {
          const uint4 af = *reinterpret_cast<const uint4*>(sat + krow * kRS + 32 * d + 8 * g);
          t[b] = mfma16(af, bfrag[d], t[b]);
        }
      }
    }
    const uint32_t words[2] = {cw[blk].x, cw[blk].y};
    uint32_t o[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const uint32_t byte = (words[e >> 3] >> (8 * ((e & 7) >> 1))) & 0xFFu;
      const float q0 = *reinterpret_cast<const float*>(tab + (((byte >> 4) << 8) | lane4));
      const float q1 = *reinterpret_cast<const float*>(tab + (((byte & 15u) << 8) | lane4));
      float m0 = __fmul_rn(q0, cs), m1 = __fmul_rn(q1, cs);
      if constexpr (kR > 0) {
        m0 = __fadd_rn(m0, __fmul_rn(s, t[e >> 2][e & 3]));
        m1 = __fadd_rn(m1, __fmul_rn(s, t[(e + 1) >> 2][(e + 1) & 3]));
      }
      o[e >> 1] = pack_bf16x2(m0, m1);
    }
    if (kb < K) {  // uniform: whole blocks only (K % 64 == 0)
      uint4* dst = reinterpret_cast<uint4*>(out + n * K + kb + 16 * g);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
}

template <int kR>
void merge_launch(const WeightView& w, const uint16_t* A, const uint16_t* B, int r, float s,
                  uint16_t* out, const CodeParams& P, hipStream_t st) {
  const dim3 grid(static_cast<uint32_t>((w.K + kMCols - 1) / kMCols),
                  static_cast<uint32_t>(w.N / kMRows));
  if (w.qscale)
    hipLaunchKernelGGL((merge_kernel<kR, true>), grid, dim3(256), 0, st, w.packed, w.qscale,
                       w.gscale, w.absmax, w.N, w.K, A, B, r, s, out, P);
  else
    hipLaunchKernelGGL((merge_kernel<kR, false>), grid, dim3(256), 0, st, w.packed, w.qscale,
                       w.gscale, w.absmax, w.N, w.K, A, B, r, s, out, P);
}

}  // namespace

hipError_t launch_merge(const WeightView& w, const uint16_t* A, const uint16_t* B, int r, float s,
                        uint16_t* out, hipStream_t st) {
  if (w.N == 0 || w.K == 0) return hipSuccess;
  const CodeParams P = code_params(w);
  if (r == 0) merge_launch<0>(w, A, B, r, s, out, P, st);  // frozen weight: A, B unused
  else if (r <= 32) merge_launch<32>(w, A, B, r, s, out, P, st);
  else if (r <= 64) merge_launch<64>(w, A, B, r, s, out, P, st);
  else merge_launch<128>(w, A, B, r, s, out, P, st);
  return hipGetLastError();
}

}  // namespace qn
