// Decode-path kernels (gfx950): the skinny LoRA projections u = x A^T and
// t = dy B, and the dequant-GEMV y = x W^T + s u B^T for M <= 16 tokens.
//
// [kwkr "QLoRA原理深入" §2.3] the 4-bit weight is expanded to 16 bits only
// inside the product; [rkmt "QLORA技术解析" §2.1, §3.3] LoRA bypass B A
// scaled by alpha / r.
//
// GEMV design: the weight stream (0.516 byte per weight) is the only HBM
// traffic that matters, and at 4096 x 4096 the whole matrix is about one
// memory latency's worth of bytes for the chip, so the kernel is built to
// put every weight byte in flight at once and to serialise nothing behind
// it.  The 16x16x32 bf16 MFMA does the multiply-adds (VALU would need 16
// FMAs per weight at M = 16); the weight operand is the *unscaled* code
// value bf16(q[code]) looked up two codes at a time from a 256-entry byte
// table in LDS, and the block constant c' is applied once per 64-weight
// block to the fp32 partial sum.  Every MFMA covers 16 rows x 32 k-slots of
// one block: lane (n = l%16, g = l/16) holds codes k = 64b + 16g + [0, 16)
// of row n (one 8-byte load), the two MFMAs of a block take the first and
// second 8 of them, and the x operand uses the same k-slot map.
//
// The byte table has 32 copies (64 in 16-wave workgroups), lane l reading
// copy l mod copies, so the random lookups of a wave spread over all LDS
// banks (a single shared copy halves the lookup rate on gfx950).

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

constexpr int kUParts = 8;   // LoRA partial sums held per thread in the GEMV
constexpr int kXAhead = 3;   // x prefetch distance, in blocks (register ring)

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Skinny projection out[M, r] = in[M, L] * P^T, P row-major [r, L].
//
// Grid: (row groups of 16 kRT rows of `in`) x ksplit L-slices; kWaves waves
// per workgroup split the slice in 32-wide chunks, wave w taking chunks w,
// w + kWaves, ...  Each round a wave issues the loads of kCh chunks (in: one
// 16-byte load per lane per chunk and 16-row tile; P: one per lane per
// 16-column tile) before any MFMA, so a round costs one memory latency.
// 16x16x32 MFMA with in-rows on the M side and kCols column tiles of 16
// (r <= 16 kCols); the kRT row tiles of a workgroup share each P load.
// ksplit == 1: writes the finished result (fp32 and/or bf16 forms).
// ksplit > 1: writes fp32 partial sums out_f32[slice][M][r].
template <int kCols, int kWaves, int kRT>
__global__ __launch_bounds__(kWaves * 64) void skinny_kernel(
    const uint16_t* __restrict__ in, int64_t M, int64_t L, const uint16_t* __restrict__ P, int r,
    float scale, int ksplit, float* __restrict__ out_f32, uint16_t* __restrict__ out_sbf16,
    uint16_t* __restrict__ out_bf16) {
  constexpr int kCh = kCols * kRT >= 8 ? 1 : 8 / (kCols * kRT);
  __shared__ float sred[kWaves][16][17];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mi = lane & 15, g = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 16 * kRT;
  const int64_t nchunk = L >> 5;
  const int64_t c_lo = nchunk * blockIdx.y / ksplit, c_hi = nchunk * (blockIdx.y + 1) / ksplit;
  // rows >= M read row M - 1 and are never stored
  const uint16_t* arow[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int64_t m = row0 + 16 * rt + mi;
    arow[rt] = in + (m < M ? m : M - 1) * L + 8 * g;
  }
  // Column j = 16 c + mi of P, clamped into [0, r); columns >= r read row
  // r - 1 and are zeroed.
  const uint16_t* prow[kCols];
  bool pvalid[kCols];
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
    const int j = c * 16 + mi;
    pvalid[c] = j < r;
    prow[c] = P + static_cast<int64_t>(j < r ? j : r - 1) * L + 8 * g;
  }
  f32x4_t acc[kRT][kCols];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int c = 0; c < kCols; ++c) acc[rt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // chunks of this wave: c_lo + wave + kWaves * i, i < cnt.  Each round
  // issues all of its loads (clamped to valid chunks) before any MFMA, and
  // has no branches: chunks past cnt have their P operand masked to zero
  // with an integer AND (a select would become a branch around the load).
  const int64_t first = c_lo + wave;
  const int64_t cnt = first < c_hi ? (c_hi - first + kWaves - 1) / kWaves : 0;
  for (int64_t i0 = 0; i0 < cnt; i0 += kCh) {
    uint4 a[kCh][kRT], b[kCh][kCols];
#pragma unroll
    for (int i = 0; i < kCh; ++i) {
      const int64_t ii = i0 + i < cnt ? i0 + i : cnt - 1;
      const int64_t kk = (first + ii * kWaves) * 32;
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) a[i][rt] = *reinterpret_cast<const uint4*>(arow[rt] + kk);
#pragma unroll
      for (int c = 0; c < kCols; ++c) b[i][c] = *reinterpret_cast<const uint4*>(prow[c] + kk);
    }
#pragma unroll
    for (int i = 0; i < kCh; ++i) {
      const uint32_t im = i0 + i < cnt ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int c = 0; c < kCols; ++c) {
        const uint32_t bm = pvalid[c] ? im : 0u;
        const uint4 bb = make_uint4(b[i][c].x & bm, b[i][c].y & bm, b[i][c].z & bm, b[i][c].w & bm);
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) acc[rt][c] = mfma16(a[i][rt], bb, acc[rt][c]);
      }
    }
  }

  // Cross-wave sum, one 16 x 16 tile at a time, fixed order.
  const int ncol = (r + 15) >> 4;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      if (c < ncol) {
#pragma unroll
        for (int v = 0; v < 4; ++v) sred[wave][4 * g + v][mi] = acc[rt][c][v];
        __syncthreads();
        for (int idx = threadIdx.x; idx < 256; idx += kWaves * 64) {
          const int row = idx >> 4, cj = idx & 15;
          const int col = c * 16 + cj;
          const int64_t mm = row0 + 16 * rt + row;
          if (mm < M && col < r) {
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) v += sred[w][row][cj];
            const int64_t o = mm * r + col;
            if (ksplit > 1) {
              out_f32[static_cast<int64_t>(blockIdx.y) * M * r + o] = v;
            } else {
              if (out_f32) out_f32[o] = v;
              if (out_sbf16) out_sbf16[o] = static_cast<uint16_t>(pack_bf16x2(scale * v, 0.f) & 0xFFFF);
              if (out_bf16) out_bf16[o] = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xFFFF);
            }
          }
        }
        __syncthreads();
      }
    }
  }
}

// Fixed-order sum of the L-sliced partial sums of a LoRA projection: one
// element per thread, the loads of all slices issued before they are added
// up in slice order (bit-reproducible).
__global__ __launch_bounds__(256) void lora_reduce_kernel(const float* __restrict__ part,
                                                          int nslice, int64_t n, float scale,
                                                          uint16_t* __restrict__ out_scaled,
                                                          uint16_t* __restrict__ out) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t ec = e < n ? e : n - 1;  // past n: re-read the last element, store nothing
  float v[kWideMaxSlices];
#pragma unroll
  for (int q = 0; q < kWideMaxSlices; ++q) v[q] = part[static_cast<int64_t>(q < nslice ? q : 0) * n + ec];
  float sum = v[0];
#pragma unroll
  for (int q = 1; q < kWideMaxSlices; ++q)
    if (q < nslice) sum += v[q];
  if (e < n) {
    out_scaled[e] = static_cast<uint16_t>(pack_bf16x2(scale * sum, 0.f) & 0xFFFF);
    if (out) out[e] = static_cast<uint16_t>(pack_bf16x2(sum, 0.f) & 0xFFFF);
  }
}

// out[c][l] = in[l][c] for a row-major [L, C] bf16 matrix (C <= 128): turns
// B [N, r] into the row-major [r, N] operand of the skinny kernel.  One
// workgroup per 64 rows of `in`, staged through LDS.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ in,
                                                        int64_t L, int C,
                                                        uint16_t* __restrict__ out) {
  __shared__ uint16_t t[64][129];
  const int64_t l0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int rows = static_cast<int>(L - l0 < 64 ? L - l0 : 64);
  for (int idx = threadIdx.x; idx < rows * C; idx += 256) {
    const int lr = idx / C, c = idx % C;
    t[lr][c] = in[(l0 + lr) * C + c];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < rows * C; idx += 256) {
    const int c = idx / rows, lr = idx % rows;
    out[static_cast<int64_t>(c) * L + l0 + lr] = t[lr][c];
  }
}

// ---------------------------------------------------------------------------
// Dequant-GEMV.  One workgroup of kWaves waves per band of 16 output
// features (rows of W).  Wave w owns a contiguous slice of at most kS
// blocks of the band's K range (longer rows take several passes) and issues
// all of its weight loads (8 bytes per lane per block) and block constants
// before anything else.  x is read per block, kXAhead blocks ahead (it is
// small and L2-resident).  The LoRA inputs (u as `usplit` fp32 partial
// sums [usplit][M][r], and the band's 16 rows of B) are loaded at the start
// with plain indexing and only consumed in the epilogue.  Partial sums meet
// in LDS in a fixed order (bit-reproducible).
//
// Everything before the weight loads is kept to a few instructions: at
// these sizes the whole matrix is in flight within a microsecond or two,
// so every serial step (a division in address arithmetic, an LDS round trip
// per block) shows up directly in the kernel time.
struct GemvArgs {
  const uint8_t* packed;
  const uint8_t* qscale;
  const float* gscale;
  const float* absmax;
  int64_t N, K;
  const uint16_t* x;
  const float* u;
  const uint16_t* B;
  uint16_t* y;
  uint16_t* u_out;
  int M, usplit, r;
  float s;
};

// kXM: token rows of x staged in LDS per wave (1; 0: no staging, x
// read per block from memory into a register ring).  kCopiesT: pair-table
// copies, 64 for 16-wave workgroups (entry address (e << 8) | 4 lane is one
// v_perm), else 32 (LDS for several workgroups per CU).
template <int kWaves, int kS, bool kDQ, int kXM>
__global__ __launch_bounds__(kWaves * 64) void gemv_kernel(const GemvArgs a, const CodeParams P) {
  constexpr int kThreads = kWaves * 64;
  constexpr int kCopiesT = kWaves == 16 ? 64 : 32;
  constexpr int kTabWords = 256 * kCopiesT;
  constexpr int kBPer = (16 * 128 + kThreads - 1) / kThreads;  // B-tile elements per thread
  constexpr bool kXL = kXM > 0;
  // staged x per wave: [token m < kXM][block i < kS][64 bf16]
  constexpr int kXBytes = kXL ? kXM * kS * 128 : 16;
  constexpr int kXPer = kXL ? (kXM * kS * 8 + 63) / 64 : 1;  // 16-byte chunks per lane
  // Pair table during the walk; afterwards the same memory holds u and the
  // band's B rows for the epilogue.
  __shared__ __attribute__((aligned(16))) uint32_t stab[kTabWords];
  __shared__ float sl8[256];
  __shared__ float spart[kWaves][16][17];
  __shared__ __attribute__((aligned(16))) char sx[kXL ? kWaves * kXBytes : 16];
  __shared__ __attribute__((aligned(16))) uint4 sxz[kXL ? kS * 8 + 8 : 1];  // zeros
  // epilogue: su [M r <= 2048] + sB [16 r <= 2048 bf16] + group sums [<= 1024]
  static_assert(kTabWords >= 16 * 128 + 16 * 128 / 2 + 1024, "epilogue buffers must fit");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, g = lane >> 4;
  const int64_t K = a.K, nblk = K >> 6;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t n = n0 + nl;
  const int M = a.M, r = a.r, mr = M * r, usplit = a.usplit;

  // -- LoRA inputs (consumed only in the epilogue) --
  // Issued without any branch (a branch join would wait for them); with
  // r == 0 the host points B and u at valid memory and element 0 is read.
  // u arrives as usplit partial sums [usplit][M][r].  Thread t works on
  // element e = t % (M r) for slices sg, sg + G, sg + 2 G, .. (sg = t / (M r),
  // G = threads / (M r) groups), kUParts of them at most: the host keeps
  // usplit <= G kUParts.  Unused slots read slice 0 and are masked in the
  // epilogue, which sums each thread's slots, then the groups, in a fixed
  // order.  With M r > threads, elements >= threads are summed from memory
  // in the epilogue.
  uint32_t bt[kBPer];  // 32-bit so the compiler does not pack them (that waits on the loads)
  float upart[kUParts];
  {
    const int nbt = 16 * r;
#pragma unroll
    for (int q = 0; q < kBPer; ++q) {
      const int e = tid + q * kThreads;
      bt[q] = a.B[n0 * r + (e < nbt ? e : (nbt > 0 ? nbt - 1 : 0))];
    }
    const int ugroups = mr > 0 && mr <= kThreads ? kThreads / mr : 1;
    const int ue = mr > 0 ? tid % mr : 0, ug = mr > 0 ? tid / mr : 0;
    const float* ut = a.u + (ug < ugroups ? ue : 0);
#pragma unroll
    for (int q = 0; q < kUParts; ++q) {
      const int sl = ug + q * ugroups;
      upart[q] = ut[static_cast<int64_t>(sl < usplit && ug < ugroups ? sl : 0) * mr];
    }
  }

  // Weight loads: lane l reads 8 bytes of row n0 + l / 4 at byte 8 (l % 4)
  // of the block, so each group of 4 consecutive lanes reads 32 contiguous
  // bytes (one row's block); ds_bpermute then moves them to the MFMA lane
  // (row l % 16, byte group l / 16), i.e. from lane 4 (l % 16) + l / 16.
  // (Loading in MFMA lane order directly, consecutive lanes in different
  // rows, streams about a third slower.)
  const uint8_t* wrow = a.packed + (n0 + (lane >> 2)) * (K >> 1) + 8 * (lane & 3);
  const int wperm = ((lane & 15) * 4 + (lane >> 4)) * 4;
  // Token rows >= M: the ring path reads row M - 1 and zeroes the value;
  // the staged path reads a zero region.
  const bool xvalid = nl < M;
  const int xm = xvalid ? nl : M - 1;
  const uint16_t* xrow = a.x + static_cast<int64_t>(xm) * K + 16 * g;
  const int64_t rowblk0 = n * nblk;
  const uint32_t lane4 = static_cast<uint32_t>(lane) << 2;
  char* sxw = sx + (kXL ? wave * kXBytes : 0);
  const char* xbase = kXL ? (xvalid ? sxw + xm * (kS * 128) + g * 32
                                    : reinterpret_cast<const char*>(sxz) + g * 32)
                          : nullptr;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc = zero;

  const int64_t per_pass = static_cast<int64_t>(kWaves) * kS;
  for (int64_t p0 = 0; p0 < nblk; p0 += per_pass) {
    const int64_t pn = min(per_pass, nblk - p0);
    const int64_t b_lo = p0 + pn * wave / kWaves;  // <= nblk - 1 even for an empty slice
    const int nb = static_cast<int>(p0 + pn * (wave + 1) / kWaves - b_lo);
    const int nbc = nb > 0 ? nb - 1 : 0;

    // 1. tables (first pass only): the barrier they need comes before the
    // loads of the slice, so no wave then waits for another wave's loads
    if (p0 == 0) {
      // uint4 f of the table holds entry f / (kCopiesT / 4), copies
      // 4 (f % (kCopiesT / 4)) .. + 3; for f = tid + i kThreads the odd
      // element (low nibble, e & 15) is fixed per thread and the even
      // element (e >> 4) is wave-uniform.
      const CodeRegs R = code_regs(P);
      constexpr int kPer = kCopiesT / 4;  // uint4 per entry
      const int e_hi0 = __builtin_amdgcn_readfirstlane(tid / (16 * kPer));
      constexpr int kFill = kTabWords / 4 / kThreads;
      const float q_odd = code_value(R, static_cast<uint32_t>((tid / kPer) & 15));
#pragma unroll
      for (int i = 0; i < kFill; ++i) {
        const uint32_t wv = pack_bf16x2(
            code_value_uniform(R, static_cast<uint32_t>(e_hi0 + i * (kThreads / (16 * kPer)))), q_odd);
        reinterpret_cast<uint4*>(stab)[tid + i * kThreads] = make_uint4(wv, wv, wv, wv);
      }
      for (int i = tid; i < 256; i += kThreads) sl8[i] = l2_value(static_cast<uint32_t>(i), P.fp8);
      if constexpr (kXL)
        for (int i = tid; i < kS * 8 + 8; i += kThreads) sxz[i] = make_uint4(0, 0, 0, 0);
      __syncthreads();
    }

    // 2. x of the slice into registers (staged path): 16-byte chunk c of
    // the wave's [m][i][128 B] staging area; rows >= M and blocks past the
    // slice re-read valid data and are never used.
    uint4 xs[kXPer];
    int xc[kXPer];
    if constexpr (kXL) {
#pragma unroll
      for (int q = 0; q < kXPer; ++q) {
        int c = lane + 64 * q;
        c = c < kXM * kS * 8 ? c : kXM * kS * 8 - 1;
        xc[q] = c;
        const int cm = c / (kS * 8), ci = (c >> 3) % kS;
        const int64_t m = cm < M ? cm : M - 1;
        const int64_t bi = b_lo + (ci < nbc ? ci : nbc);
        xs[q] = *reinterpret_cast<const uint4*>(a.x + m * K + bi * 64 + (c & 7) * 8);
      }
    }

    // 3. block constants and all weight loads of this wave's slice
    const int64_t qb = rowblk0 + b_lo;  // index of the slice's first block constant
    constexpr int kQD = kS / 4 + 1;
    uint32_t qd[kQD];
    float cq[kDQ ? 1 : kS];
    float g_lo = 0.f, g_hi = 0.f;
    if constexpr (kDQ) {
      // 8-bit constants of the slice: aligned dwords covering
      // [qb, qb + kS); the total count N K / 64 is a multiple of 4, so the
      // clamp keeps every dword inside the array.
      const uint32_t* q32 = reinterpret_cast<const uint32_t*>(a.qscale);
      const int64_t dmax = ((a.N * nblk) >> 2) - 1;
#pragma unroll
      for (int j = 0; j < kQD; ++j) {
        const int64_t d = (qb >> 2) + j;
        qd[j] = q32[d < dmax ? d : dmax];
      }
      g_lo = a.gscale[qb >> 8];
      g_hi = a.gscale[(qb + nbc) >> 8];
    } else {
#pragma unroll
      for (int i = 0; i < kS; ++i) cq[i] = a.absmax[qb + (i < nbc ? i : nbc)];
    }
    uint2 w[kS];
#pragma unroll
    for (int i = 0; i < kS; ++i)
      w[i] = *reinterpret_cast<const uint2*>(wrow + (b_lo + (i < nbc ? i : nbc)) * 32);

    // 4. x: staged slice to LDS (read back only by this wave), or the
    // first blocks of the register ring
    uint4 xr[kXL ? 1 : kXAhead + 1][2];
    auto load_x = [&](int i) {
      if constexpr (!kXL) {
        const int ic = i < nbc ? i : nbc;
        const uint4* xp = reinterpret_cast<const uint4*>(xrow + (b_lo + ic) * 64);
        xr[i % (kXAhead + 1)][0] = xp[0];
        xr[i % (kXAhead + 1)][1] = xp[1];
      }
    };
    if constexpr (kXL) {
#pragma unroll
      for (int q = 0; q < kXPer; ++q) *reinterpret_cast<uint4*>(sxw + xc[q] * 16) = xs[q];
    } else {
#pragma unroll
      for (int i = 0; i < kXAhead; ++i) load_x(i);
    }
    auto x_of = [&](int i, int h) -> uint4 {
      if constexpr (kXL) {
        return *reinterpret_cast<const uint4*>(xbase + i * 128 + h * 16);
      } else {
        const uint4 v = xr[i % (kXAhead + 1)][h];
        return xvalid ? v : make_uint4(0, 0, 0, 0);
      }
    };

    // 5. block constants c' of every block of the slice (one LDS round trip)
    float cs[kS];
    if constexpr (kDQ) {
      const uint32_t sh = static_cast<uint32_t>(qb & 3);
      const int gfirst = static_cast<int>(qb & 255);
#pragma unroll
      for (int j = 0; j < kS / 4; ++j) {
        const uint32_t al = __builtin_amdgcn_alignbyte(qd[j + 1], qd[j], sh);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = 4 * j + b;
          const float c = __fmul_rn(sl8[(al >> (8 * b)) & 0xFFu], gfirst + i < 256 ? g_lo : g_hi);
          cs[i] = i < nb ? c : 0.f;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kS; ++i) cs[i] = i < nb ? cq[i] : 0.f;
    }

    // 6. walk the slice; the pair lookups of block i + 1 are issued before
    // the MFMAs of block i.  No control flow: blocks past the slice (the
    // last wave of an uneven split) re-read valid data and have c' = 0 (a
    // branch here lets the compiler sink the weight loads into it).
    auto look = [&](uint32_t word, int byte) -> uint32_t {
      uint32_t addr;
      if constexpr (kCopiesT == 64) {
        // bytes [4 lane, e, 0, 0]: (e << 8) | 4 lane
        addr = __builtin_amdgcn_perm(word, lane4, 0x0C0C0400u + (static_cast<uint32_t>(byte) << 8));
      } else {
        addr = (((word >> (8 * byte)) & 0xFFu) << 7) | (lane4 & 0x7Cu);
      }
      return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(stab) + addr);
    };
    uint4 d[kS][2];
#pragma unroll
    for (int i = 0; i < kS; ++i) {
      const uint32_t w0 = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(wperm, static_cast<int>(w[i].x)));
      const uint32_t w1 = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(wperm, static_cast<int>(w[i].y)));
      d[i][0] = make_uint4(look(w0, 0), look(w0, 1), look(w0, 2), look(w0, 3));
      d[i][1] = make_uint4(look(w1, 0), look(w1, 1), look(w1, 2), look(w1, 3));
      if (i > 0) {
        f32x4_t t = mfma16(x_of(i - 1, 0), d[i - 1][0], zero);
        t = mfma16(x_of(i - 1, 1), d[i - 1][1], t);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = fmaf(cs[i - 1], t[v], acc[v]);
      }
      load_x(i + kXAhead);
    }
    {
      f32x4_t t = mfma16(x_of(kS - 1, 0), d[kS - 1][0], zero);
      t = mfma16(x_of(kS - 1, 1), d[kS - 1][1], t);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] = fmaf(cs[kS - 1], t[v], acc[v]);
    }
  }

  // -- epilogue --
#pragma unroll
  for (int v = 0; v < 4; ++v) spart[wave][4 * g + v][nl] = acc[v];
  __syncthreads();  // every wave is done with the pair table
  float* su = reinterpret_cast<float*>(stab);                  // [M][r] fp32
  uint16_t* sB = reinterpret_cast<uint16_t*>(stab + 16 * 128);  // [16][r] bf16
  float* sug = reinterpret_cast<float*>(stab + 16 * 128 + 16 * 128 / 2);  // [groups][M r]
  if (r > 0) {
    const int ugroups = mr <= kThreads ? kThreads / mr : 1;
    const int ue = tid % mr, ug = tid / mr;
    if (ug < ugroups) {
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < kUParts; ++q) {
        const uint32_t mask = ug + q * ugroups < usplit ? 0xFFFFFFFFu : 0u;  // an AND, not a select
        v += __uint_as_float(__float_as_uint(upart[q]) & mask);
      }
      sug[ug * mr + ue] = v;
    }
    for (int idx = tid + kThreads; idx < mr; idx += kThreads) {
      float v = 0.f;
      for (int q = 0; q < usplit; ++q) v += a.u[static_cast<int64_t>(q) * mr + idx];
      su[idx] = v;
    }
#pragma unroll
    for (int q = 0; q < kBPer; ++q) {
      const int e = tid + q * kThreads;
      if (e < 16 * r) sB[e] = static_cast<uint16_t>(bt[q]);
    }
    __syncthreads();
    if (tid < mr && tid < kThreads) {
      float v = 0.f;
      for (int gq = 0; gq < ugroups; ++gq) v += sug[gq * mr + tid];
      su[tid] = v;
    }
  }
  __syncthreads();
  if (a.u_out && blockIdx.x == 0)
    for (int i = tid; i < mr; i += kThreads)
      a.u_out[i] = static_cast<uint16_t>(pack_bf16x2(su[i], 0.f) & 0xFFFF);
  for (int idx = tid; idx < 16 * M; idx += kThreads) {
    const int m = idx >> 4, nn = idx & 15;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) v += spart[ww][m][nn];
    if (r > 0) {
      float lora = 0.f;
      for (int j = 0; j < r; ++j) lora = fmaf(su[m * r + j], bf16_to_f32(sB[nn * r + j]), lora);
      v = fmaf(a.s, lora, v);
    }
    a.y[static_cast<int64_t>(m) * a.N + n0 + nn] = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xFFFF);
  }
}

// One GEMV configuration: the single token row staged in LDS (xmode 1), or
// the register ring.
template <int W, int S>
void gemv_config(int xmode, bool dq, dim3 grid, hipStream_t st, const GemvArgs& a,
                 const CodeParams& P) {
  if (xmode == 1) {
    hipLaunchKernelGGL((gemv_kernel<W, S, true, 1>), grid, dim3(W * 64), 0, st, a, P);
  } else if (dq) {
    hipLaunchKernelGGL((gemv_kernel<W, S, true, 0>), grid, dim3(W * 64), 0, st, a, P);
  } else {
    hipLaunchKernelGGL((gemv_kernel<W, S, false, 0>), grid, dim3(W * 64), 0, st, a, P);
  }
}

template <int kCols>
void skinny_launch(int rows, hipStream_t s, const uint16_t* in, int64_t M, int64_t L,
                   const uint16_t* P, int r, float scale, int ksplit, float* out_f32,
                   uint16_t* out_sbf16, uint16_t* out_bf16) {
  const dim3 grid(static_cast<uint32_t>((M + rows - 1) / rows), static_cast<uint32_t>(ksplit));
  if constexpr (kCols <= 4) {
    if (rows == 64) {
      hipLaunchKernelGGL((skinny_kernel<kCols, 16, 4>), grid, dim3(1024), 0, s, in, M, L, P, r,
                         scale, ksplit, out_f32, out_sbf16, out_bf16);
      return;
    }
  }
  if (M > 16)
    hipLaunchKernelGGL((skinny_kernel<kCols, 16, 1>), grid, dim3(1024), 0, s, in, M, L, P, r, scale,
                       ksplit, out_f32, out_sbf16, out_bf16);
  else
    hipLaunchKernelGGL((skinny_kernel<kCols, 1, 1>), grid, dim3(64), 0, s, in, M, L, P, r, scale,
                       ksplit, out_f32, out_sbf16, out_bf16);
}

int skinny_cols(int r) { return r <= 16 ? 1 : r <= 32 ? 2 : r <= 64 ? 4 : 8; }

}  // namespace

int gemv_threads(int64_t N, int64_t K) {
  int wv = 4;
  while (wv < 16 && (N / 16) * wv * 2 <= 4096) wv *= 2;
  (void)K;
  return wv * 64;
}

int skinny_splits(int64_t M, int64_t L, int r, int gemv_thr) {
  if (M > 16 || r == 0) return 1;
  // one single-wave slice per 32-wide chunk (a wave per workgroup, no
  // cross-wave reduction: the partials go straight to the GEMV, which sums
  // at most (threads / (M r)) * kUParts of them per element).  Against 8
  // waves per slice this takes 10% off a decode call (one LDS reduction and
  // barrier fewer in the kernel that the weight stream waits for).
  const int64_t mr = M * r;
  const int64_t groups = mr <= gemv_thr ? gemv_thr / mr : 1;
  int64_t ks = L >> 5;
  if (ks > groups * kUParts) ks = groups * kUParts;
  if (ks > kDecodeMaxSlices) ks = kDecodeMaxSlices;
  return ks < 1 ? 1 : static_cast<int>(ks);
}

int skinny_wide_splits(int64_t M, int64_t L) {
  // about 256 workgroups of 64 rows, at least one 32-wide chunk per wave
  const int64_t groups = (M + 63) / 64;
  int64_t ks = (256 + groups - 1) / groups;
  const int64_t maxk = (L >> 5) / 16;
  if (ks > maxk) ks = maxk;
  if (ks > kWideMaxSlices) ks = kWideMaxSlices;
  return ks < 1 ? 1 : static_cast<int>(ks);
}

hipError_t launch_skinny(const uint16_t* in, int64_t M, int64_t L, const uint16_t* P, int r,
                         float scale, float* out_f32, uint16_t* out_scaled_bf16,
                         uint16_t* out_bf16, int ksplit, hipStream_t s) {
  if (M == 0 || r == 0) return hipSuccess;
  // Decode (M <= 16): one 16-row tile, one wave per 32-wide L-slice.  Token batches:
  // 64-row workgroups of 16 waves (each load of P serves four row tiles);
  // r > 64 keeps 16-row workgroups (the accumulators of 4 x 8 tiles would
  // not fit).
  const int rows = M > 16 && r <= 64 ? 64 : 16;
  switch (skinny_cols(r)) {
    case 1: skinny_launch<1>(rows, s, in, M, L, P, r, scale, ksplit, out_f32, out_scaled_bf16, out_bf16); break;
    case 2: skinny_launch<2>(rows, s, in, M, L, P, r, scale, ksplit, out_f32, out_scaled_bf16, out_bf16); break;
    case 4: skinny_launch<4>(rows, s, in, M, L, P, r, scale, ksplit, out_f32, out_scaled_bf16, out_bf16); break;
    default: skinny_launch<8>(rows, s, in, M, L, P, r, scale, ksplit, out_f32, out_scaled_bf16, out_bf16); break;
  }
  return hipGetLastError();
}

hipError_t launch_lora_reduce(const float* part, int nslice, int64_t n, float scale,
                              uint16_t* out_scaled, uint16_t* out, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(lora_reduce_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256),
                     0, st, part, nslice, n, scale, out_scaled, out);
  return hipGetLastError();
}

hipError_t launch_transpose(const uint16_t* in, int64_t L, int C, uint16_t* out, hipStream_t s) {
  if (L == 0 || C == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_kernel, dim3(static_cast<uint32_t>((L + 63) / 64)), dim3(256), 0, s,
                     in, L, C, out);
  return hipGetLastError();
}

hipError_t launch_gemv(const WeightView& w, const uint16_t* x, int M, const float* u, int usplit,
                       const uint16_t* B, int r, float s, uint16_t* y, uint16_t* u_out,
                       hipStream_t st) {
  if (M == 0 || w.N == 0) return hipSuccess;
  const CodeParams P = code_params(w);
  GemvArgs a;
  a.packed = w.packed;
  a.qscale = w.qscale;
  a.gscale = w.gscale;
  a.absmax = w.absmax;
  a.N = w.N;
  a.K = w.K;
  a.x = x;
  // with r == 0 the kernel still reads element 0 of u and B (never used)
  a.u = r > 0 ? u : reinterpret_cast<const float*>(x);
  a.B = r > 0 ? B : x;
  a.y = y;
  a.u_out = u_out;
  a.M = M;
  a.usplit = usplit < 1 ? 1 : usplit;
  a.r = r;
  a.s = s;
  const int64_t nbands = w.N / 16, nblk = w.K >> 6;
  const dim3 grid(static_cast<uint32_t>(nbands));
  // About 16 resident waves per CU in one round: waves per band from
  // 4096 / bands (4, 8 or 16), blocks per wave the smallest of 4, 8, 12, 16
  // that covers the row (longer rows: 16 per pass, several passes).
  const int wv = gemv_threads(w.N, w.K) / 64;
  const int64_t need = (nblk + wv - 1) / wv;
  int sb = need <= 4 ? 4 : need <= 8 ? 8 : need <= 12 ? 12 : 16;
  if (wv == 16 && sb == 16) sb = 12;  // 16 x 16 would spill at 1024 threads
  const bool dq = w.qscale != nullptr;
  // x staging: the one row for M == 1, the register ring above (also for
  // M <= 4: staging four rows was 15% slower at 11008 x 4096, M = 4); the
  // unscaled-constant path (no double quantisation) uses the ring.
  const int xmode = !dq ? 0 : M == 1 ? 1 : 0;
#define QN_GEMV(W, S) \
  if (wv == W && sb == S) gemv_config<W, S>(xmode, dq, grid, st, a, P);
  QN_GEMV(4, 4) QN_GEMV(4, 8) QN_GEMV(4, 12) QN_GEMV(4, 16)
  QN_GEMV(8, 4) QN_GEMV(8, 8) QN_GEMV(8, 12) QN_GEMV(8, 16)
  QN_GEMV(16, 4) QN_GEMV(16, 8) QN_GEMV(16, 12)
#undef QN_GEMV
  return hipGetLastError();
}

}  // namespace qn
