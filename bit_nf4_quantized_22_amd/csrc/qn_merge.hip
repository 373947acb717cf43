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
// k.  A lane then reads 8 bytes of codes and one block constant per block.
// A workgroup (4 waves) owns 256 columns and a run of 64-row groups: A's
// columns for them are staged transposed in LDS once, then the workgroup
// walks its row groups with the next group's codes, constants and B rows
// (in registers) in flight.  Each wave's 16 x 64 output block goes out
// through a small LDS slot as 8 rows x 128 bytes per store instruction.

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

constexpr int kMRows = 64;    // rows of W per row group (16 per wave)
constexpr int kMCols = 256;   // columns of W per workgroup (4 blocks)
constexpr int kBlk = kMCols / 64;
constexpr int kSP = 64 + 8;   // row pitch (bf16) of a wave's staged 16 x 64 output block
// Workgroups to aim for: each stages its A tile once and then walks
// ceil(row groups x column blocks / kTargetWgs) row groups (two or three
// at the 7B shapes).  Measured at 4096 x 11008 and 11008 x 4096: 512 is
// 8-17% faster than one row group per workgroup (2752 workgroups) at
// r = 16, 64 and 128, within 2% of 1024 at r = 16 and 9-17% faster than
// 1024 at r = 64 and 128.
constexpr int kTargetWgs = 512;

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// A lane's loads for one row group: the codes of its row n, columns
// k0 + 64 blk + 16 g .. + 15 of each block (8 bytes; byte i holds k 2i in
// the high nibble and 2i + 1 in the low one), the blocks' constants, and
// B's row n, columns 32 d + 8 g .. + 7, raw (kVec: one 16-byte load, else
// eight 2-byte loads): they are masked and packed only when used, since any
// use right after a load makes the compiler wait for it.
template <int kD, bool kVec>
struct MergeRow {
  uint2 cw[kBlk];
  uint32_t q8[kBlk];
  float c2[kBlk];
  uint32_t bv[kD > 0 ? kD : 1][kVec ? 4 : 8];
};

// All loads unconditional from clamped addresses (blocks past K re-read the
// last block and store nothing; a branch around a load would make the join
// wait for it).
template <int kR, bool kDQ, bool kVec>
__device__ __forceinline__ void merge_load(const uint8_t* __restrict__ packed,
                                           const uint8_t* __restrict__ qscale,
                                           const float* __restrict__ gscale,
                                           const float* __restrict__ absmax, int64_t K,
                                           const uint16_t* __restrict__ B, int r, int64_t n,
                                           int64_t k0, int g, MergeRow<kR / 32, kVec>& L) {
#pragma unroll
  for (int blk = 0; blk < kBlk; ++blk) {
    const int64_t kb = k0 + 64 * blk < K ? k0 + 64 * blk : K - 64;
    const int64_t bi = n * (K >> 6) + (kb >> 6);
    L.cw[blk] = *reinterpret_cast<const uint2*>(packed + (n * K + kb + 16 * g) / 2);
    if constexpr (kDQ) {
      L.q8[blk] = qscale[bi];
      L.c2[blk] = gscale[bi >> 8];
    } else {
      L.q8[blk] = 0;
      L.c2[blk] = absmax[bi];
    }
  }
  if constexpr (kR > 0) {
    // one 16-byte load per 8 ranks when r is a multiple of 8 (rows of
    // 16-byte multiples; B itself 16-byte aligned; ranks past r re-read the
    // last 8), else element by element (ranks past r re-read rank r - 1)
#pragma unroll
    for (int d = 0; d < kR / 32; ++d) {
      const int j0 = 32 * d + 8 * g;
      if constexpr (kVec) {
        const uint4 v = *reinterpret_cast<const uint4*>(B + n * r + (j0 < r ? j0 : r - 8));
        L.bv[d][0] = v.x;
        L.bv[d][1] = v.y;
        L.bv[d][2] = v.z;
        L.bv[d][3] = v.w;
      } else {
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const int j = j0 + h;
          L.bv[d][h] = B[n * r + (j < r ? j : r - 1)];
        }
      }
    }
  }
}

// B fragment d of a row group's loads, zero past rank r.
template <int kD, bool kVec>
__device__ __forceinline__ uint4 merge_bfrag(const MergeRow<kD, kVec>& L, int d, int r, int g) {
  const int j0 = 32 * d + 8 * g;
  if constexpr (kVec) {
    return j0 < r ? make_uint4(L.bv[d][0], L.bv[d][1], L.bv[d][2], L.bv[d][3]) : make_uint4(0, 0, 0, 0);
  } else {
    uint32_t w4[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int j = j0 + 2 * h;
      w4[h] = (j < r ? L.bv[d][2 * h] : 0u) | ((j + 1 < r ? L.bv[d][2 * h + 1] : 0u) << 16);
    }
    return make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
}

// kR: rank capacity (0, 32, 64 or 128); kD = kR / 32 MFMAs per 16 x 16 tile;
// kVec: B's rows are read as 16-byte runs (r % 8 == 0, B 16-byte aligned).
// Workgroup (x, y) owns columns 256 x .. + 255 and row groups gpw y ..
// gpw (y + 1) - 1 (64 rows each, the last one clipped to N / 64); it stages
// its slice of A once and walks its row groups with the next group's loads
// in flight.
template <int kR, bool kDQ, bool kVec>
__global__ __launch_bounds__(256) void merge_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ gscale, const float* __restrict__ absmax, int64_t N, int64_t K,
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int r, float s,
    uint16_t* __restrict__ out, CodeParams P, int gpw) {
  constexpr int kD = kR / 32;
  constexpr int kRS = kR + 8;  // bf16 per row of the transposed A tile (16-byte pad)
  __shared__ float scode[16 * 64];  // q[c] for lane l at [64 c + l]: no bank conflicts
  __shared__ __attribute__((aligned(16))) uint16_t sat[kR > 0 ? kMCols * kRS : 8];
  __shared__ __attribute__((aligned(16))) uint16_t stg[4][16 * kSP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int64_t k0 = static_cast<int64_t>(blockIdx.x) * kMCols;
  const int ngroups = static_cast<int>(N / kMRows);  // N % 64 == 0: every row valid
  const int gb = static_cast<int>(blockIdx.y) * gpw;
  const int ge = gb + gpw < ngroups ? gb + gpw : ngroups;
  // The first row group's loads go first, before the LoRA operands are
  // staged: their latency then overlaps the staging and its barrier.
  MergeRow<kD, kVec> cur;
  merge_load<kR, kDQ, kVec>(packed, qscale, gscale, absmax, K, B, r,
                            static_cast<int64_t>(gb) * kMRows + 16 * wave + nl, k0, g, cur);
  const float mu = kDQ ? l2_offset(P) : 0.0f;
  {
    const CodeRegs R = code_regs(P);
    for (int i = tid; i < 16 * 64; i += 256) scode[i] = code_value(R, i >> 6);
  }
  if constexpr (kR > 0) {
    // A tile transposed: sat[kk][j] = A[j][k0 + kk], zero for j >= r or
    // columns past K.  Thread tid handles column kk = tid of every row j.
    // The loads go in runs of 8 ranks, only as many runs as r needs, each
    // from clamped addresses (rows j >= r re-read row r - 1); the values are
    // first used after all loads are issued, where the zeros are selected.
    // (Loading rank by rank behind the test j < r, with the packing next to
    // the load, made the compiler wait for every pair: one memory round trip
    // per two ranks.)  Each thread's column goes to LDS as 16-byte runs of 8
    // ranks.
    const int kk = tid;
    const int64_t kc = k0 + kk < K ? k0 + kk : K - 1;
    const bool kin = k0 + kk < K;
    uint32_t av[kR];
#pragma unroll
    for (int q = 0; q < kR / 8; ++q) {
      if (8 * q < r) {  // uniform
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const int j = 8 * q + h;
          av[j] = A[static_cast<int64_t>(j < r ? j : r - 1) * K + kc];
        }
      } else {
#pragma unroll
        for (int h = 0; h < 8; ++h) av[8 * q + h] = 0u;
      }
    }
    // first use of the loaded values here, after every run is issued (else
    // the compiler packs each run inside its branch and waits there)
#pragma unroll
    for (int j = 0; j < kR; ++j) asm volatile("" : "+v"(av[j]));
#pragma unroll
    for (int q = 0; q < kR / 8; ++q) {
      uint32_t w4[4];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        w4[h] = kin ? ((8 * q + 2 * h < r ? av[8 * q + 2 * h] & 0xFFFFu : 0u) |
                       (8 * q + 2 * h + 1 < r ? av[8 * q + 2 * h + 1] << 16 : 0u))
                    : 0u;
      *reinterpret_cast<uint4*>(sat + kk * kRS + 8 * q) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
  }
  __syncthreads();

  const uint32_t lane4 = static_cast<uint32_t>(lane) << 2;
  const char* tab = reinterpret_cast<const char*>(scode);
  uint16_t* stw = stg[wave];
  for (int gi = gb; gi < ge; ++gi) {
    MergeRow<kD, kVec> nxt;  // the next row group's loads, in flight during this one
    if (gi + 1 < ge)         // uniform
      merge_load<kR, kDQ, kVec>(packed, qscale, gscale, absmax, K, B, r,
                                static_cast<int64_t>(gi + 1) * kMRows + 16 * wave + nl, k0, g, nxt);
    const int64_t nb = static_cast<int64_t>(gi) * kMRows + 16 * wave;  // the wave's first row
#pragma unroll
    for (int blk = 0; blk < kBlk; ++blk) {
      const int64_t kb = k0 + 64 * blk;  // first column of the block
      const float cs = kDQ ? dq_value(cur.q8[blk], cur.c2[blk], P.l2, mu) : cur.c2[blk];
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
            t[b] = mfma16(af, merge_bfrag(cur, d, r, g), t[b]);
          }
        }
      }
      const uint32_t words[2] = {cur.cw[blk].x, cur.cw[blk].y};
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
        // Lane (nl, g) holds row nb + nl, columns kb + 16 g .. + 15.  The
        // wave stages its 16 x 64 block in its own LDS slot and stores it
        // as 8 rows x 128 bytes per instruction (a 16-row x 64-byte pattern
        // straight from the registers streams about 10% slower).  LDS
        // instructions of one wave complete in order, so the slot is free
        // again for the next block once these reads are issued.
        *reinterpret_cast<uint4*>(stw + nl * kSP + 16 * g) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(stw + nl * kSP + 16 * g + 8) = make_uint4(o[4], o[5], o[6], o[7]);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int lr = lane >> 3, ch = lane & 7;
        const uint4 v0 = *reinterpret_cast<const uint4*>(stw + lr * kSP + 8 * ch);
        const uint4 v1 = *reinterpret_cast<const uint4*>(stw + (lr + 8) * kSP + 8 * ch);
        *reinterpret_cast<uint4*>(out + (nb + lr) * K + kb + 8 * ch) = v0;
        *reinterpret_cast<uint4*>(out + (nb + lr + 8) * K + kb + 8 * ch) = v1;
      }
    }
    cur = nxt;
  }
}

template <int kR>
void merge_launch(const WeightView& w, const uint16_t* A, const uint16_t* B, int r, float s,
                  uint16_t* out, const CodeParams& P, hipStream_t st) {
  const int64_t gx = (w.K + kMCols - 1) / kMCols, ngroups = w.N / kMRows;
  int64_t gpw = (gx * ngroups + kTargetWgs - 1) / kTargetWgs;
  if (gpw < 1) gpw = 1;
  const dim3 grid(static_cast<uint32_t>(gx), static_cast<uint32_t>((ngroups + gpw - 1) / gpw));
  const bool vec = (r & 7) == 0 && (reinterpret_cast<uintptr_t>(B) & 15) == 0;
#define QN_MERGE_GO(DQ, VEC)                                                                   \
  hipLaunchKernelGGL((merge_kernel<kR, DQ, VEC>), grid, dim3(256), 0, st, w.packed, w.qscale, \
                     w.gscale, w.absmax, w.N, w.K, A, B, r, s, out, P, static_cast<int>(gpw))
  if (w.qscale) {
    if (vec) QN_MERGE_GO(true, true); else QN_MERGE_GO(true, false);
  } else {
    if (vec) QN_MERGE_GO(false, true); else QN_MERGE_GO(false, false);
  }
#undef QN_MERGE_GO
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
