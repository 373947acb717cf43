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
constexpr int kSelfUMaxBlocks = 8;  // one round of A loads after the walk: 2 kS uint4 per lane
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
template <int kCols, int kWaves, int kRT, bool kPT>
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
  // r - 1 and are zeroed.  kPT: P is stored [L, r] (B for t = dy B, read
  // where it lies), and a lane's 8 consecutive l of column j are 8 loads
  // r elements apart.
  const uint16_t* prow[kCols];
  bool pvalid[kCols];
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
    const int j = c * 16 + mi;
    pvalid[c] = j < r;
    const int jc = j < r ? j : r - 1;
    prow[c] = kPT ? P + static_cast<int64_t>(8 * g) * r + jc
                  : P + static_cast<int64_t>(jc) * L + 8 * g;
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
      for (int c = 0; c < kCols; ++c) {
        if constexpr (kPT) {
          const uint16_t* pc = prow[c] + kk * r;
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = pc[static_cast<int64_t>(e) * r];
          b[i][c] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                               h[6] | (h[7] << 16));
        } else {
          b[i][c] = *reinterpret_cast<const uint4*>(prow[c] + kk);
        }
      }
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

// Token-batch projection out[M, r] = in[M, L] * P^T (M > 16, r <= 16 kCols
// <= 64): workgroups of 16 waves own 64 rows of `in` and an L-slice, as in
// skinny_kernel<kCols, 16, 4>, with the same per-wave chunk order and
// cross-wave sum order (bit-identical results).  The slice is taken in
// stages of 16 chunks (512 columns): each wave loads 4 whole rows of the
// stage, 1 KB per load instruction, into a padded LDS tile (the next
// stage's rows in flight meanwhile), and wave w then multiplies chunk w of
// the stage from LDS.  Loading the MFMA operands straight from memory reads
// 16 rows x 64 bytes per instruction, and the launch ran about 30% longer.
// The cross-wave sum takes four 16 x 16 tiles per pair of barriers.
template <int kCols, bool kPT>
__global__ __launch_bounds__(1024) void skinny_batch_kernel(
    const uint16_t* __restrict__ in, int64_t M, int64_t L, const uint16_t* __restrict__ P, int r,
    float scale, int ksplit, float* __restrict__ out_f32, uint16_t* __restrict__ out_sbf16,
    uint16_t* __restrict__ out_bf16) {
  constexpr int kWaves = 16, kRT = 4, kStage = 16;  // chunks per stage: one per wave
  constexpr int kXP = kStage * 32 + 8;  // LDS row pitch (bf16): rows 16 bytes apart in bank terms
  constexpr int kTiles = kRT * kCols, kTB = 4;
  __shared__ __attribute__((aligned(16))) uint16_t sx[64 * kXP];
  __shared__ float sred[kWaves][kTB][16][17];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mi = lane & 15, g = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int64_t nchunk = L >> 5;
  const int64_t c_lo = nchunk * blockIdx.y / ksplit, c_hi = nchunk * (blockIdx.y + 1) / ksplit;
  const int nstage = static_cast<int>((c_hi - c_lo + kStage - 1) / kStage);
  // P columns as in skinny_kernel (clamped into [0, r), zeroed past r)
  const uint16_t* prow[kCols];
  bool pvalid[kCols];
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
    const int j = c * 16 + mi;
    pvalid[c] = j < r;
    const int jc = j < r ? j : r - 1;
    prow[c] = kPT ? P + static_cast<int64_t>(8 * g) * r + jc
                  : P + static_cast<int64_t>(jc) * L + 8 * g;
  }
  // stage loads: wave w, rows 4 w + q; lane l, columns 8 l .. + 7 of the
  // stage (past the slice: its last 8 columns, never multiplied); rows past
  // M read row M - 1 and are never stored
  const int64_t colmax = c_hi * 32 - 8;
  const uint16_t* xrow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t m = row0 + 4 * wave + q;
    xrow[q] = in + (m < M ? m : M - 1) * L;
  }
  auto stage_col = [&](int st) -> int64_t {
    const int64_t col = (c_lo + static_cast<int64_t>(st) * kStage) * 32 + 8 * lane;
    return col < colmax ? col : colmax;
  };
  f32x4_t acc[kRT][kCols];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int c = 0; c < kCols; ++c) acc[rt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the stage's four rows in named registers (an array carried across the
  // stage loop was kept in scratch memory)
  uint4 xr0, xr1, xr2, xr3;
  auto load_rows = [&](int64_t col) {
    xr0 = *reinterpret_cast<const uint4*>(xrow[0] + col);
    xr1 = *reinterpret_cast<const uint4*>(xrow[1] + col);
    xr2 = *reinterpret_cast<const uint4*>(xrow[2] + col);
    xr3 = *reinterpret_cast<const uint4*>(xrow[3] + col);
  };
  load_rows(stage_col(0));  // an empty slice reads valid data it never uses
  for (int st = 0; st < nstage; ++st) {
    // this wave's chunk of the stage and its P operand (chunks past the
    // slice read the last chunk and are masked to zero)
    const int64_t cw = c_lo + static_cast<int64_t>(st) * kStage + wave;
    const uint32_t im = cw < c_hi ? 0xFFFFFFFFu : 0u;
    const int64_t kk = (cw < c_hi ? cw : c_hi - 1) * 32;
    uint4 b[kCols];
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      if constexpr (kPT) {
        const uint16_t* pc = prow[c] + kk * r;
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = pc[static_cast<int64_t>(e) * r];
        b[c] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                          h[6] | (h[7] << 16));
      } else {
        b[c] = *reinterpret_cast<const uint4*>(prow[c] + kk);
      }
    }
    if (st > 0) __syncthreads();  // the previous stage's operand reads are done
    uint16_t* srow = sx + 4 * wave * kXP + 8 * lane;
    *reinterpret_cast<uint4*>(srow) = xr0;
    *reinterpret_cast<uint4*>(srow + kXP) = xr1;
    *reinterpret_cast<uint4*>(srow + 2 * kXP) = xr2;
    *reinterpret_cast<uint4*>(srow + 3 * kXP) = xr3;
    if (st + 1 < nstage) load_rows(stage_col(st + 1));  // uniform
    __syncthreads();  // the stage is in LDS
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      const uint32_t bm = pvalid[c] ? im : 0u;
      b[c] = make_uint4(b[c].x & bm, b[c].y & bm, b[c].z & bm, b[c].w & bm);
    }
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const uint4 a = *reinterpret_cast<const uint4*>(sx + (16 * rt + mi) * kXP + 32 * wave + 8 * g);
#pragma unroll
      for (int c = 0; c < kCols; ++c) acc[rt][c] = mfma16(a, b[c], acc[rt][c]);
    }
  }

  // Cross-wave sum, kTB tiles (t = kCols rt + c) per round, waves in order.
  const int ncol = (r + 15) >> 4;
#pragma unroll
  for (int t0 = 0; t0 < kTiles; t0 += kTB) {
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) {
      const int t = t0 + tb;
      if (t < kTiles && t % kCols < ncol) {
#pragma unroll
        for (int v = 0; v < 4; ++v) sred[wave][tb][4 * g + v][mi] = acc[t / kCols][t % kCols][v];
      }
    }
    __syncthreads();
    {
      const int idx = threadIdx.x;  // kTB x 256 outputs: one per thread
      const int tb = idx >> 8, row = (idx >> 4) & 15, cj = idx & 15;
      const int t = t0 + tb;
      const int c = t % kCols, col = c * 16 + cj;
      const int64_t mm = row0 + 16 * (t / kCols) + row;
      if (t < kTiles && c < ncol && mm < M && col < r) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) v += sred[w][tb][row][cj];
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

// ---------------------------------------------------------------------------
// Dequant-GEMV, M <= 16 tokens.  One workgroup of kWaves waves per band of
// 16 output features (rows of W).  Wave w owns a contiguous slice of at most
// kS blocks of the band's K range (longer rows take several passes).  The
// LoRA inputs (u as `usplit` fp32 partial sums [usplit][M][r], and the
// band's 16 rows of B) are loaded at the start and only consumed in the
// epilogue.  Partial sums meet in LDS in a fixed order (bit-reproducible).
//
// What paces a decode call (measured with per-wave timestamps): every
// wave's weight loads are issued into a memory system that is already
// saturated, so issuing them stalls for microseconds, and any work placed
// behind the loads in program order (a table fill, a barrier) waits that
// long.  The table is therefore built and published before the first load;
// all loads of a slice are then issued in a pinned order (x, constants,
// weights, with scheduling barriers so the compiler cannot move a use of a
// late load ahead of an early one), and the walk waits for one block at a
// time, so decoding overlaps the rest of the stream.
struct GemvArgs {
  const uint8_t* packed;
  const uint8_t* qscale;
  const float* gscale;
  const float* absmax;
  int64_t N, K;
  const uint16_t* x;
  const float* u;   // usplit fp32 partial sums [usplit][M][r] of x A^T
  const uint16_t* B;
  uint16_t* y;
  uint16_t* u_out;
  int M, usplit, r;
  float s;
  // One token, one pass, r <= 16, in the kernel that computes u = x A^T
  // itself from the x slices it staged: A [r, K] (u and usplit unused).
  const uint16_t* A;
};

// The decode's LDS tables: kCopiesT interleaved copies of the 256-entry
// byte table (entry e = (bf16(q[e >> 4]), bf16(q[e & 15])), the even
// element first) and the 256 level-2 values.  uint4 f of the table holds
// entry f / (kCopiesT / 4), copies 4 (f % (kCopiesT / 4)) .. + 3; for f =
// tid + i kThreads the odd element (low nibble, e & 15) is fixed per thread
// and the even element (e >> 4) is wave-uniform.
template <int kCopiesT, int kThreads>
__device__ __forceinline__ void gemv_tables(uint32_t* stab, float* sl8, const CodeParams& P,
                                            int tid) {
  const CodeRegs R = code_regs(P);
  constexpr int kPer = kCopiesT / 4;  // uint4 per entry
  const int e_hi0 = __builtin_amdgcn_readfirstlane(tid / (16 * kPer));
  constexpr int kFill = 256 * kCopiesT / 4 / kThreads;
  const float q_odd = code_value(R, static_cast<uint32_t>((tid / kPer) & 15));
#pragma unroll
  for (int i = 0; i < kFill; ++i) {
    const uint32_t wv = pack_bf16x2(
        code_value_uniform(R, static_cast<uint32_t>(e_hi0 + i * (kThreads / (16 * kPer)))), q_odd);
    reinterpret_cast<uint4*>(stab)[tid + i * kThreads] = make_uint4(wv, wv, wv, wv);
  }
  for (int i = tid; i < 256; i += kThreads) sl8[i] = l2_value(static_cast<uint32_t>(i), P.l2);
}

// Pair of bf16 code values of byte `byte` of `word` from lane `lane`'s copy
// of the table (lane4 = 4 lane).  With 64 copies the entry address
// (e << 8) | 4 lane is a single byte permute.
template <int kCopiesT>
__device__ __forceinline__ uint32_t pair_lookup(const uint32_t* stab, uint32_t word, int byte,
                                                uint32_t lane4) {
  uint32_t addr;
  if constexpr (kCopiesT == 64) {
    addr = __builtin_amdgcn_perm(word, lane4, 0x0C0C0400u + (static_cast<uint32_t>(byte) << 8));
  } else {
    addr = (((word >> (8 * byte)) & 0xFFu) << 7) | (lane4 & 0x7Cu);
  }
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(stab) + addr);
}

// Workgroup barrier for LDS data only: waits for this wave's LDS stores,
// not for its loads in flight (a __syncthreads() also waits for those),
// and keeps the compiler from scheduling anything across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// LoRA inputs of the epilogue.  u arrives as usplit partial sums
// [usplit][M][r]: thread t works on element e = t % (M r) for slices sg,
// sg + G, .. (sg = t / (M r), G = threads / (M r) groups), kUParts of them
// at most (the host keeps usplit <= G kUParts).  Unused slots read slice 0
// and are masked when summed.  With M r > threads, elements >= threads are
// summed from memory later.
template <int kThreads, int kBPer, int kUParts>
__device__ __forceinline__ void gemv_lora_loads(const GemvArgs& a, int64_t n0, int tid,
                                                uint32_t (&bt)[kBPer], float (&upart)[kUParts]) {
  const int r = a.r, mr = a.M * a.r;
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
    upart[q] = ut[static_cast<int64_t>(sl < a.usplit && ug < ugroups ? sl : 0) * mr];
  }
}

// Epilogue: the waves' partial sums meet in LDS in a fixed order, u is
// summed from its partials (fixed order), and s u B^T is added to the band.
// The LoRA inputs are loaded here, after the weight stream, so no register
// holds them during the walk.  The table memory holds u and the band's B
// rows once every wave is done with the table (the first barrier below).
template <int kWaves, int kUParts>
__device__ __forceinline__ void gemv_epilogue(const GemvArgs& a, const f32x4_t& acc,
                                              float (*spart)[16][17], uint32_t* stab, int tid,
                                              const float (*su_w)[16] = nullptr) {
  constexpr int kThreads = kWaves * 64;
  constexpr int kBPer = (16 * 128 + kThreads - 1) / kThreads;
  const int lane = tid & 63, wave = tid >> 6, nl = lane & 15, g = lane >> 4;
  const int M = a.M, r = a.r, mr = M * r, usplit = a.usplit;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
#pragma unroll
  for (int v = 0; v < 4; ++v) spart[wave][4 * g + v][nl] = acc[v];
  __syncthreads();  // every wave is done with the pair table
  float* su = reinterpret_cast<float*>(stab);                  // [M][r] fp32
  uint16_t* sB = reinterpret_cast<uint16_t*>(stab + 16 * 128);  // [16][r] bf16
  float* sug = reinterpret_cast<float*>(stab + 16 * 128 + 16 * 128 / 2);  // [groups][M r]
  if (r > 0 && su_w) {
    // the band's B rows; u (one token) is the waves' partial sums, added in
    // wave order
#pragma unroll
    for (int q = 0; q < kBPer; ++q) {
      const int e = tid + q * kThreads;
      if (e < 16 * r) sB[e] = a.B[n0 * r + e];
    }
    if (tid < r) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += su_w[w][tid];
      su[tid] = v;
    }
    __syncthreads();
  } else if (r > 0) {
    uint32_t bt[kBPer];
    float upart[kUParts];
    gemv_lora_loads<kThreads, kBPer, kUParts>(a, n0, tid, bt, upart);
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
    __syncthreads();
  }
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

// Register-ring GEMV for 2 <= M <= 16 tokens: x is read per block from
// memory into a register ring kXAhead blocks ahead (x of 16 tokens is too
// large to stage in LDS per wave).  Rows >= M read row M - 1 and are
// zeroed.
template <int kWaves, int kS, bool kDQ>
__global__ __launch_bounds__(kWaves * 64) void gemv_ring_kernel(const GemvArgs a, const CodeParams P) {
  constexpr int kThreads = kWaves * 64;
  constexpr int kCopiesT = kWaves == 16 ? 64 : 32;
  constexpr int kTabWords = 256 * kCopiesT;
  constexpr int kQD = (kS + 3) / 4 + 1;  // dwords covering constant bytes sh .. sh + kS - 1, sh < 4
  // Pair table during the walk; afterwards the same memory holds u and the
  // band's B rows for the epilogue.
  __shared__ __attribute__((aligned(16))) uint32_t stab[kTabWords];
  __shared__ float sl8[256];
  __shared__ float spart[kWaves][16][17];
  // epilogue: su [M r <= 2048] + sB [16 r <= 2048 bf16] + group sums [<= 1024]
  static_assert(kTabWords >= 16 * 128 + 16 * 128 / 2 + 1024, "epilogue buffers must fit");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, g = lane >> 4;
  const int64_t K = a.K, nblk = K >> 6;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int M = a.M;

  // tables first, published before any load is in flight
  gemv_tables<kCopiesT, kThreads>(stab, sl8, P, tid);
  const float mu = kDQ ? l2_offset(P) : 0.0f;
  lds_barrier();

  // Weight loads: lane l reads 8 bytes of row n0 + l / 4 at byte 8 (l % 4)
  // of the block, so each group of 4 consecutive lanes reads 32 contiguous
  // bytes (one row's block); ds_bpermute then moves them to the MFMA lane
  // (row l % 16, byte group l / 16), i.e. from lane 4 (l % 16) + l / 16.
  // (Loading in MFMA lane order directly, consecutive lanes in different
  // rows, streams about a third slower.)
  const uint8_t* wrow = a.packed + (n0 + (lane >> 2)) * (K >> 1) + 8 * (lane & 3);
  const int wperm = ((lane & 15) * 4 + (lane >> 4)) * 4;
  const bool xvalid = nl < M;
  const int xm = xvalid ? nl : M - 1;
  const uint16_t* xrow = a.x + static_cast<int64_t>(xm) * K + 16 * g;
  const int64_t rowblk0 = (n0 + nl) * nblk;
  const uint32_t lane4 = static_cast<uint32_t>(lane) << 2;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc = zero;

  const int64_t per_pass = static_cast<int64_t>(kWaves) * kS;
  for (int64_t p0 = 0; p0 < nblk; p0 += per_pass) {
    const int64_t pn = min(per_pass, nblk - p0);
    const int64_t b_lo = p0 + pn * wave / kWaves;  // <= nblk - 1 even for an empty slice
    const int nb = static_cast<int>(p0 + pn * (wave + 1) / kWaves - b_lo);
    const int nbc = nb > 0 ? nb - 1 : 0;

    // block constants and all weight loads of this wave's slice
    const int64_t qb = rowblk0 + b_lo;  // index of the slice's first block constant
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

    // the first blocks of the x ring
    uint4 xr[kXAhead + 1][2];
    auto load_x = [&](int i) {
      const int ic = i < nbc ? i : nbc;
      const uint4* xp = reinterpret_cast<const uint4*>(xrow + (b_lo + ic) * 64);
      xr[i % (kXAhead + 1)][0] = xp[0];
      xr[i % (kXAhead + 1)][1] = xp[1];
    };
#pragma unroll
    for (int i = 0; i < kXAhead; ++i) load_x(i);
    auto x_of = [&](int i, int h) -> uint4 {
      const uint4 v = xr[i % (kXAhead + 1)][h];
      return xvalid ? v : make_uint4(0, 0, 0, 0);
    };

    // block constants c' of every block of the slice (one LDS round trip)
    float cs[kS];
    if constexpr (kDQ) {
      const uint32_t sh = static_cast<uint32_t>(qb & 3);
      const int gfirst = static_cast<int>(qb & 255);
#pragma unroll
      for (int j = 0; j < (kS + 3) / 4; ++j) {
        const uint32_t al = __builtin_amdgcn_alignbyte(qd[j + 1], qd[j], sh);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = 4 * j + b;
          if (i < kS) {
            const float c = mul_then_add(sl8[(al >> (8 * b)) & 0xFFu], gfirst + i < 256 ? g_lo : g_hi, mu);
            cs[i] = i < nb ? c : 0.f;
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kS; ++i) cs[i] = i < nb ? cq[i] : 0.f;
    }

    // walk the slice; the pair lookups of block i + 1 are issued before
    // the MFMAs of block i.  No control flow: blocks past the slice (the
    // last wave of an uneven split) re-read valid data and have c' = 0 (a
    // branch here lets the compiler sink the weight loads into it).
    auto look = [&](uint32_t word, int byte) -> uint32_t {
      return pair_lookup<kCopiesT>(stab, word, byte, lane4);
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

  gemv_epilogue<kWaves, kUParts>(a, acc, spart, stab, tid);
}

// Staged GEMV for one token (M == 1).  The 16 x kS x 64 x-values of a wave's
// slice are copied to that wave's LDS region once per pass; in the walk only
// the four lanes that hold token row 0 of the MFMA's x operand read them
// (the other rows of the product are never stored), so x costs no vector
// memory bandwidth per block.  Loads of a pass, in issue order: the x slice,
// the 8-bit block constants (aligned dwords covering the slice) and group
// constants, then the weights block by block; the walk waits for one more
// block per step.
template <int kWaves, int kS, bool kDQ, bool kSelfU = false>
__global__ __launch_bounds__(kWaves * 64) void gemv1_kernel(const GemvArgs a, const CodeParams P) {
  static_assert(!kSelfU || kS <= kSelfUMaxBlocks, "one round of A loads");
  constexpr int kThreads = kWaves * 64;
  constexpr int kCopiesT = kWaves == 16 ? 64 : 32;
  constexpr int kTabWords = 256 * kCopiesT;
  constexpr int kXBytes = kS * 128;                            // a wave's x slice
  constexpr int kXPer = (kS * 8 + 63) / 64;                    // its 16-byte chunks per lane
  constexpr int kQD = (kS + 3) / 4 + 1;  // dwords covering constant bytes sh .. sh + kS - 1, sh < 4
  // the waves' partial sums share memory with the x staging area, which is
  // free once the walk has ended
  constexpr int kXAll = kWaves * kXBytes > kWaves * 16 * 17 * 4 ? kWaves * kXBytes : kWaves * 16 * 17 * 4;
  __shared__ __attribute__((aligned(16))) uint32_t stab[kTabWords];
  __shared__ float sl8[256];
  __shared__ __attribute__((aligned(16))) char sx[kXAll];
  float (*spart)[16][17] = reinterpret_cast<float (*)[16][17]>(sx);
  static_assert(kTabWords >= 16 * 128 + 16 * 128 / 2 + 1024, "epilogue buffers must fit");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, g = lane >> 4;
  const int64_t K = a.K, nblk = K >> 6;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;

  // 1. tables, published before any load is in flight
  gemv_tables<kCopiesT, kThreads>(stab, sl8, P, tid);
  const float mu = kDQ ? l2_offset(P) : 0.0f;
  lds_barrier();

  // the band's 16 rows as a buffer: lane offset in a VGPR, block offset
  // (wave-uniform) in an SGPR, so a slice's loads need no 64-bit addresses
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.packed + n0 * (K >> 1)), static_cast<short>(0),
      static_cast<int>(16 * (K >> 1)), 0x00020000);
  const int wlane = static_cast<int>((lane >> 2) * (K >> 1) + 8 * (lane & 3));
  const int wperm = ((lane & 15) * 4 + (lane >> 4)) * 4;
  const uint32_t lane4 = static_cast<uint32_t>(lane) << 2;
  char* sxw = sx + wave * kXBytes;
  const char* xb = sxw + g * 32;
  const bool xon = nl == 0;  // lanes holding token row 0 of the x operand
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc = zero;

  const int64_t per_pass = static_cast<int64_t>(kWaves) * kS;
  for (int64_t p0 = 0; p0 < nblk; p0 += per_pass) {
    const int64_t pn = min(per_pass, nblk - p0);
    const int64_t b_lo = p0 + pn * wave / kWaves;  // <= nblk - 1 even for an empty slice
    const int nb = static_cast<int>(p0 + pn * (wave + 1) / kWaves - b_lo);
    const int nbc = nb > 0 ? nb - 1 : 0;
    __builtin_amdgcn_sched_barrier(0);

    // x slice: 16-byte chunk c of block c / 8 (blocks past the slice re-read
    // a valid one and are never used)
    uint4 xs[kXPer];
    int xc[kXPer];
#pragma unroll
    for (int q = 0; q < kXPer; ++q) {
      int c = lane + 64 * q;
      c = c < kS * 8 ? c : kS * 8 - 1;
      xc[q] = c;
      const int ci = c >> 3;
      xs[q] = *reinterpret_cast<const uint4*>(a.x + (b_lo + (ci < nbc ? ci : nbc)) * 64 + (c & 7) * 8);
    }
    __builtin_amdgcn_sched_barrier(0);

    // block constants of row n0 + nl over the slice
    const int64_t qb = (n0 + nl) * nblk + b_lo;
    uint32_t qd[kQD];
    float cq[kDQ ? 1 : kS];
    float g_lo = 0.f, g_hi = 0.f;
    if constexpr (kDQ) {
      // aligned dwords covering [qb, qb + kS); the count N K / 64 is a
      // multiple of 4, so the clamp keeps every dword inside the array
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
    __builtin_amdgcn_sched_barrier(0);

    // weights: lane l reads 8 bytes of row n0 + l / 4 at byte 8 (l % 4) of
    // the block (four lanes cover a row's 32-byte block); ds_bpermute then
    // moves them to the MFMA lane (row l % 16, byte group l / 16)
    uint2 w[kS];
#pragma unroll
    for (int i = 0; i < kS; ++i) {
      const int boff = __builtin_amdgcn_readfirstlane(static_cast<int>((b_lo + (i < nbc ? i : nbc)) * 32));
      w[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(wr, wlane, boff, 0));
      __builtin_amdgcn_sched_barrier(0);
    }

    // x to this wave's LDS region (read back only by this wave); the empty
    // asm keeps the stores, and their wait for x, behind the weight loads
#pragma unroll
    for (int q = 0; q < kXPer; ++q) {
      asm volatile("" : "+v"(xs[q].x), "+v"(xs[q].y), "+v"(xs[q].z), "+v"(xs[q].w)::"memory");
      *reinterpret_cast<uint4*>(sxw + xc[q] * 16) = xs[q];
    }

    // c' of block i of the slice, from the 8-bit constants in registers
    // (blocks past the slice get 0)
    const uint32_t sh = static_cast<uint32_t>(qb & 3);
    const int gfirst = static_cast<int>(qb & 255);
    auto cscale = [&](int i) -> float {
      float c;
      if constexpr (kDQ) {
        const uint32_t al = __builtin_amdgcn_alignbyte(qd[i / 4 + 1], qd[i / 4], sh);
        c = mul_then_add(sl8[(al >> (8 * (i % 4))) & 0xFFu], gfirst + i < 256 ? g_lo : g_hi, mu);
      } else {
        c = cq[i];
      }
      return i < nb ? c : 0.f;
    };
    __builtin_amdgcn_sched_barrier(0);

    // walk: decode block i + 1 (its lookups in flight) while block i multiplies
    uint4 dcur[2], dnext[2];
    auto decode = [&](int i, uint4 (&d)[2]) {
      const uint32_t w0 = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(wperm, static_cast<int>(w[i].x)));
      const uint32_t w1 = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(wperm, static_cast<int>(w[i].y)));
      d[0] = make_uint4(pair_lookup<kCopiesT>(stab, w0, 0, lane4), pair_lookup<kCopiesT>(stab, w0, 1, lane4),
                        pair_lookup<kCopiesT>(stab, w0, 2, lane4), pair_lookup<kCopiesT>(stab, w0, 3, lane4));
      d[1] = make_uint4(pair_lookup<kCopiesT>(stab, w1, 0, lane4), pair_lookup<kCopiesT>(stab, w1, 1, lane4),
                        pair_lookup<kCopiesT>(stab, w1, 2, lane4), pair_lookup<kCopiesT>(stab, w1, 3, lane4));
    };
    uint4 x0 = make_uint4(0, 0, 0, 0), x1 = x0;
    decode(0, dcur);
    float ccur = cscale(0), cnext = 0.f;
#pragma unroll
    for (int i = 0; i < kS; ++i) {
      if (i + 1 < kS) {
        decode(i + 1, dnext);
        cnext = cscale(i + 1);
      }
      if (xon) {
        x0 = *reinterpret_cast<const uint4*>(xb + i * 128);
        x1 = *reinterpret_cast<const uint4*>(xb + i * 128 + 16);
      }
      f32x4_t t = mfma16(x0, dcur[0], zero);
      t = mfma16(x1, dcur[1], t);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] = fmaf(ccur, t[v], acc[v]);
      __builtin_amdgcn_sched_barrier(0);
      dcur[0] = dnext[0];
      dcur[1] = dnext[1];
      ccur = cnext;
    }
  }
  // LoRA-down in the same launch (one pass, r <= 16): this wave's share of
  // u = x A^T over its blocks, from its x slice still in LDS, with A's rows
  // loaded in one round after the walk (the weight stream is done) and the
  // same k-slot map as the walk's two MFMAs per block; row 0 of the
  // product holds the wave's partial u.
  if constexpr (kSelfU) {
    __shared__ float su_w[kWaves][16];
    const int64_t b_lo = nblk * wave / kWaves;
    const int nb = static_cast<int>(nblk * (wave + 1) / kWaves - b_lo);
    const int nbc = nb > 0 ? nb - 1 : 0;
    const int r = a.r;
    const uint16_t* arow = a.A + static_cast<int64_t>(nl < r ? nl : r - 1) * K + 16 * g;
    uint4 af[kS][2];
#pragma unroll
    for (int i = 0; i < kS; ++i) {
      const int64_t bi = b_lo + (i < nbc ? i : nbc);
      af[i][0] = *reinterpret_cast<const uint4*>(arow + bi * 64);
      af[i][1] = *reinterpret_cast<const uint4*>(arow + bi * 64 + 8);
    }
    f32x4_t au = zero;
#pragma unroll
    for (int i = 0; i < kS; ++i) {
      uint4 x0 = make_uint4(0, 0, 0, 0), x1 = x0;
      if (xon) {
        x0 = *reinterpret_cast<const uint4*>(xb + i * 128);
        x1 = *reinterpret_cast<const uint4*>(xb + i * 128 + 16);
      }
      const uint32_t m = i < nb && nl < r ? 0xFFFFFFFFu : 0u;  // an AND, not a select
      au = mfma16(x0, make_uint4(af[i][0].x & m, af[i][0].y & m, af[i][0].z & m, af[i][0].w & m), au);
      au = mfma16(x1, make_uint4(af[i][1].x & m, af[i][1].y & m, af[i][1].z & m, af[i][1].w & m), au);
    }
    if (g == 0) su_w[wave][nl] = au[0];
    __syncthreads();  // the partial sums below overwrite the x staging area
    gemv_epilogue<kWaves, kUParts>(a, acc, spart, stab, tid, su_w);
  } else {
    __syncthreads();  // the partial sums below overwrite the x staging area
    gemv_epilogue<kWaves, kUParts>(a, acc, spart, stab, tid);
  }
}

// One GEMV configuration: the staged kernel for one token, the register
// ring above.
template <int W, int S>
void gemv_config(int M, bool dq, dim3 grid, hipStream_t st, const GemvArgs& a,
                 const CodeParams& P, bool self_u) {
  if constexpr (W == 16 && (S == 4 || S == 8)) {
    if (self_u) {
      if (dq)
        hipLaunchKernelGGL((gemv1_kernel<W, S, true, true>), grid, dim3(W * 64), 0, st, a, P);
      else
        hipLaunchKernelGGL((gemv1_kernel<W, S, false, true>), grid, dim3(W * 64), 0, st, a, P);
      return;
    }
  }
  if (M == 1) {
    if (dq)
      hipLaunchKernelGGL((gemv1_kernel<W, S, true>), grid, dim3(W * 64), 0, st, a, P);
    else
      hipLaunchKernelGGL((gemv1_kernel<W, S, false>), grid, dim3(W * 64), 0, st, a, P);
  } else if (dq) {
    hipLaunchKernelGGL((gemv_ring_kernel<W, S, true>), grid, dim3(W * 64), 0, st, a, P);
  } else {
    hipLaunchKernelGGL((gemv_ring_kernel<W, S, false>), grid, dim3(W * 64), 0, st, a, P);
  }
}

template <int kCols, bool kPT>
void skinny_launch(int rows, hipStream_t s, const uint16_t* in, int64_t M, int64_t L,
                   const uint16_t* P, int r, float scale, int ksplit, float* out_f32,
                   uint16_t* out_sbf16, uint16_t* out_bf16) {
  const dim3 grid(static_cast<uint32_t>((M + rows - 1) / rows), static_cast<uint32_t>(ksplit));
  if constexpr (kCols <= 4) {
    if (rows == 64) {
      hipLaunchKernelGGL((skinny_batch_kernel<kCols, kPT>), grid, dim3(1024), 0, s, in, M, L, P,
                         r, scale, ksplit, out_f32, out_sbf16, out_bf16);
      return;
    }
  }
  if (M > 16)
    hipLaunchKernelGGL((skinny_kernel<kCols, 16, 1, kPT>), grid, dim3(1024), 0, s, in, M, L, P, r,
                       scale, ksplit, out_f32, out_sbf16, out_bf16);
  else
    hipLaunchKernelGGL((skinny_kernel<kCols, 1, 1, kPT>), grid, dim3(64), 0, s, in, M, L, P, r,
                       scale, ksplit, out_f32, out_sbf16, out_bf16);
}

int skinny_cols(int r) { return r <= 16 ? 1 : r <= 32 ? 2 : r <= 64 ? 4 : 8; }

}  // namespace

int gemv_threads(int64_t N, int64_t K) {
  // about 16-24 resident waves per CU in one round: 16 waves per band up
  // to 384 bands, 8 up to 768, else 4 (11008 x 4096 at M = 1 ran about 10%
  // faster with 8 waves than with 4)
  const int64_t bands = N / 16;
  (void)K;
  return (bands <= 384 ? 16 : bands <= 768 ? 8 : 4) * 64;
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
                         uint16_t* out_bf16, int ksplit, hipStream_t s, bool p_rows_l) {
  if (M == 0 || r == 0) return hipSuccess;
  // Decode (M <= 16): one 16-row tile, one wave per 32-wide L-slice.  Token batches:
  // 64-row workgroups of 16 waves (each load of P serves four row tiles);
  // r > 64 keeps 16-row workgroups (the accumulators of 4 x 8 tiles would
  // not fit).
  const int rows = M > 16 && r <= 64 ? 64 : 16;
#define QN_SKINNY(C)                                                                          \
  if (p_rows_l)                                                                               \
    skinny_launch<C, true>(rows, s, in, M, L, P, r, scale, ksplit, out_f32, out_scaled_bf16,  \
                           out_bf16);                                                         \
  else                                                                                        \
    skinny_launch<C, false>(rows, s, in, M, L, P, r, scale, ksplit, out_f32, out_scaled_bf16, \
                            out_bf16);
  switch (skinny_cols(r)) {
    case 1: QN_SKINNY(1) break;
    case 2: QN_SKINNY(2) break;
    case 4: QN_SKINNY(4) break;
    default: QN_SKINNY(8) break;
  }
#undef QN_SKINNY
  return hipGetLastError();
}

hipError_t launch_lora_reduce(const float* part, int nslice, int64_t n, float scale,
                              uint16_t* out_scaled, uint16_t* out, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(lora_reduce_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256),
                     0, st, part, nslice, n, scale, out_scaled, out);
  return hipGetLastError();
}

namespace {

// Waves per band and blocks per wave of the GEMV for an N x K weight.
// Waves per band from gemv_threads; blocks per wave the smallest of 4, 8,
// 11, 12, 16 that covers the row (11: 172 blocks of a 11008-long row over
// 16 waves); longer rows take several passes of 16 (of 12 at 16 waves,
// where 16 x 16 would spill).
void gemv_shape(int64_t N, int64_t K, int M, int& wv, int& sb) {
  const int64_t nblk = K >> 6;
  wv = gemv_threads(N, K) / 64;
  const int64_t need = (nblk + wv - 1) / wv;
  sb = need <= 4 ? 4 : need <= 8 ? 8 : need <= 11 ? 11 : need <= 12 ? 12 : 16;
  if (wv == 16 && sb == 16) sb = 12;
  // one token over 8 waves: two passes of 4 blocks rather than one of 8
  // (the 8-block kernel needs 89 VGPRs, which allows two workgroups per CU
  // instead of three; 11008 x 4096: 10.4 us against 10.9)
  if (M == 1 && wv == 8 && sb == 8) sb = 4;
}

}  // namespace

bool gemv_self_u(const WeightView& w, int M, int r) {
  if (M != 1 || r <= 0 || r > 16 || w.N == 0) return false;
  int wv, sb;
  gemv_shape(w.N, w.K, M, wv, sb);
  // one pass of the 16-wave kernel with 4 or 8 blocks per wave, and every
  // band reads all of A [r, K] from L2: at about 10 TB/s that costs more
  // than the LoRA-down launch it replaces (about 4.5 us) beyond some 40 MB
  // (4096 x 4096, r = 16: 33.5 MB, 9.6 against 10.9 us per call; 4096 x
  // 11008: 90 MB, 19.8 against 15.4 us)
  const double a_bytes = static_cast<double>(w.N / 16) * r * static_cast<double>(w.K) * 2;
  return wv == 16 && (sb == 4 || sb == 8) && (w.K >> 6) <= 16 * sb && a_bytes <= 40e6;
}

hipError_t launch_gemv(const WeightView& w, const uint16_t* x, int M, const float* u, int usplit,
                       const uint16_t* B, int r, float s, uint16_t* y, uint16_t* u_out,
                       hipStream_t st, const uint16_t* A_self) {
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
  // with r == 0 the kernel reads neither; both still point at valid memory
  a.u = r > 0 ? u : reinterpret_cast<const float*>(x);
  a.B = r > 0 ? B : x;
  a.y = y;
  a.u_out = u_out;
  a.M = M;
  a.usplit = usplit < 1 ? 1 : usplit;
  a.r = r;
  a.s = s;
  a.A = A_self;
  const bool self_u = A_self != nullptr && r > 0;
  const int64_t nbands = w.N / 16;
  const dim3 grid(static_cast<uint32_t>(nbands));
  int wv, sb;
  gemv_shape(w.N, w.K, M, wv, sb);
  if (self_u && !gemv_self_u(w, M, r)) return hipErrorInvalidValue;
  const bool dq = w.qscale != nullptr;
#define QN_GEMV(W, S) \
  if (wv == W && sb == S) gemv_config<W, S>(M, dq, grid, st, a, P, self_u);
  QN_GEMV(4, 4) QN_GEMV(4, 8) QN_GEMV(4, 11) QN_GEMV(4, 12) QN_GEMV(4, 16)
  QN_GEMV(8, 4) QN_GEMV(8, 8) QN_GEMV(8, 11) QN_GEMV(8, 12) QN_GEMV(8, 16)
  QN_GEMV(16, 4) QN_GEMV(16, 8) QN_GEMV(16, 11) QN_GEMV(16, 12)
#undef QN_GEMV
  return hipGetLastError();
}

}  // namespace qn
