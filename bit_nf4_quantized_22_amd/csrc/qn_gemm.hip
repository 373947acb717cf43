// Fused dequant -> bf16 MFMA GEMMs for token batches (gfx950).
//
// Forward  y[M, N]  = x[M, K] W^T + (s u)[M, r] B^T      (contraction over K)
// Backward dx[M, K] = dy[M, N] W  + (s t)[M, r] A        (contraction over N)
//
// [kwkr "QLoRA原理深入" §2.3] the 4-bit weight is expanded to 16 bits for the
// matrix product and never written back; [rkmt "QLORA技术解析" §3.2] compute
// type bf16.  The weight tile is dequantised straight into LDS as
// bf16(fl32(q[code] * c')), the same bf16 value nf4_dequant produces, and
// never exists in HBM in 16-bit form.  The LoRA term rides on the same
// accumulators as one extra contraction of depth r: the A-side operand is
// bf16(s u) (or bf16(s t)), the B-side operand is B (or A^T).
//
// Tiling.  Workgroup tile BM x BN = 256 x 128, K step 64 (one quantisation
// block), one workgroup of 8 waves per CU with two LDS buffers per operand
// (rows padded by 16 bytes, 112 KB).  The waves are specialised: waves 0-3
// only read MFMA fragments from LDS and run the 32x32x16 bf16 MFMAs (2 x 2
// grid of 128 x 64 wave tiles), waves 4-7 only load from HBM and
// dequantise into LDS, so each SIMD holds one MFMA wave and one producer
// wave whose LDS latency chains no longer stall the MFMA issue.  While the
// MFMA waves consume step k from one buffer, the producers fill the other
// with step k+1 from registers loaded two steps earlier (a ring of three
// register sets); one barrier per K step.  The 256-row tile halves the
// dequantisation per flop against 128 rows, which is what bounds the kernel:
// the producers, not the MFMAs, set the pace.  All global loads are
// unconditional (edge rows re-read a valid row), which keeps the compiler
// from serialising them behind branches.
// The dequantisation looks each 4-bit code up in a 64-copy fp32 table in
// LDS (lane l reads copy l, so a wave never has a bank conflict), multiplies
// by the block constant and packs to bf16.  The forward stages the weight
// tile row-major ([n][k]); the backward needs 8 consecutive n per MFMA
// lane, so it writes the dequantised tile transposed ([k][n]).

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

constexpr int kBM = 256, kBN = 128, kBK = 64;
constexpr int kLD = kBK + 8;    // bf16 per LDS operand row (padded by 16 bytes)
constexpr int kTM = kBM / 64, kTN = kBN / 64;  // MFMA tiles per wave (wave tile kBM/2 x kBN/2)
constexpr int kWGPerCU = kBM == 256 ? 1 : 2;
constexpr int kParts = kBK / 16;               // 16-deep MFMA steps per K step
constexpr int kAChunks = kBM * kBK / 8 / 256;  // 16-byte activation chunks per thread
constexpr int kACols = kBK / 8;                // 16-byte chunks per activation row
constexpr int kCodes = kBN * kBK / 256;        // weight codes per thread per K step
constexpr int kWords = kCodes / 8;             // their 32-bit words
static_assert(kWords * 8 == kCodes, "whole words of codes per thread");

struct GemmArgs {
  const uint8_t* packed;
  const uint8_t* qscale;
  const float* gscale;
  const float* absmax;
  int64_t N, K, M;
  const uint16_t* act;   // x [M, K] (fwd) or dy [M, N] (bwd)
  const uint16_t* lact;  // bf16(s u) or bf16(s t), [M, r]
  const uint16_t* lw;    // B [N, r] (fwd) or A [r, K] (bwd)
  int r;
  uint16_t* out;         // y [M, N] or dx [M, K]
};

// Registers of the next K step: activation chunks, the thread's weight
// codes (kCodes consecutive codes of one block) and their block constant
// (q8 code + group constant, or absmax).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t wvec_t __attribute__((ext_vector_type(kWords)));

struct Prefetch {
  u32x4 a[kAChunks];
  wvec_t w;
  uint32_t q8;
  float c;
};

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Global loads of contraction step kt into registers.
//   activation: thread t owns rows t / kACols + (256 / kACols) i, 16 bytes
//     at column 8 (t % kACols)
//   forward weight: thread t owns row c0 + t/2, codes k0 + kCodes (t%2) ..
//   backward weight: thread t owns row k0 + t % kBK, codes c0 + kCodes (t / kBK) ..
template <bool kBwd, bool kDQ>
__device__ __forceinline__ void load_step(const GemmArgs& g, int64_t m0, int64_t c0, int kt,
                                          Prefetch& pf, int t) {
  const int64_t L = kBwd ? g.N : g.K;
  const int64_t k0 = static_cast<int64_t>(kt) * kBK;
  // Rows past M and weight rows/columns past the output edge re-read a
  // valid row: they only feed outputs that are never stored.
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    const int row = t / kACols + (256 / kACols) * i, col = (t % kACols) * 8;
    const int64_t m = m0 + row < g.M ? m0 + row : g.M - 1;
    pf.a[i] = *reinterpret_cast<const u32x4*>(g.act + m * L + k0 + col);
  }
  int64_t n, k;
  if constexpr (kBwd) {
    n = k0 + (t % kBK);
    k = c0 + kCodes * (t / kBK);
    k = k < g.K ? k : g.K - kCodes;
  } else {
    n = c0 + (t >> 1);
    k = k0 + kCodes * (t & 1);
    n = n < g.N ? n : g.N - 1;
  }
  pf.w = *reinterpret_cast<const wvec_t*>(g.packed + n * (g.K >> 1) + (k >> 1));
  const int64_t bi = n * (g.K >> 6) + (k >> 6);
  if constexpr (kDQ) {
    pf.q8 = g.qscale[bi];
    pf.c = g.gscale[bi >> 8];
  } else {
    pf.q8 = 0;
    pf.c = g.absmax[bi];
  }
}

// Block constant of a prefetched weight chunk.
template <bool kDQ>
__device__ __forceinline__ float chunk_scale(const Prefetch& pf) {
  return kDQ ? __fmul_rn(l8_value(pf.q8), pf.c) : pf.c;
}

// Register -> LDS store of one K step: the weight codes dequantised, then
// the activation chunks as they are.  All table lookups are issued first
// and the LDS stores last, so the in-order LDS return queue holds only
// lookups while the arithmetic waits on them.
template <bool kBwd>
__device__ __forceinline__ void store_step(const Prefetch& pf, float cs,
                                           const float* __restrict__ scode,
                                           uint16_t* __restrict__ sA, uint16_t* __restrict__ sB,
                                           int t) {
  // Byte b of a word holds element 2b (high nibble) and 2b+1 (low nibble).
  // Code c of lane l sits at byte offset 256 c + 4 l of the 64-copy table,
  // so a wave's 64 lookups hit 64 different banks; the offset is one v_perm
  // of the code byte and 4 l.
  const uint32_t lane4 = static_cast<uint32_t>(threadIdx.x & 63) << 2;
  const char* tab = reinterpret_cast<const char*>(scode);
  float q[kWords][8];
#pragma unroll
  for (int i = 0; i < kWords; ++i) {
    const uint32_t word = pf.w[i];
    const uint32_t hi = (word >> 4) & 0x0F0F0F0Fu, lo = word & 0x0F0F0F0Fu;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t sel = 0x0C0C0400u + (static_cast<uint32_t>(b) << 8);
      q[i][2 * b] = *reinterpret_cast<const float*>(tab + __builtin_amdgcn_perm(hi, lane4, sel));
      q[i][2 * b + 1] = *reinterpret_cast<const float*>(tab + __builtin_amdgcn_perm(lo, lane4, sel));
    }
  }
#pragma unroll
  for (int i = 0; i < kWords; ++i) {
    uint32_t d[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
      d[b] = pack_bf16x2(__fmul_rn(q[i][2 * b], cs), __fmul_rn(q[i][2 * b + 1], cs));
    if constexpr (kBwd) {
      const int row = t % kBK, qd = t / kBK;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        sB[(kCodes * qd + 8 * i + 2 * b) * kLD + row] = static_cast<uint16_t>(d[b] & 0xFFFF);
        sB[(kCodes * qd + 8 * i + 2 * b + 1) * kLD + row] = static_cast<uint16_t>(d[b] >> 16);
      }
    } else {
      *reinterpret_cast<u32x4*>(sB + (t >> 1) * kLD + kCodes * (t & 1) + 8 * i) = u32x4{d[0], d[1], d[2], d[3]};
    }
  }
#pragma unroll
  for (int c = 0; c < kAChunks; ++c) {
    const int row = t / kACols + (256 / kACols) * c, col = (t % kACols) * 8;
    *reinterpret_cast<u32x4*>(sA + row * kLD + col) = pf.a[c];
  }
}

// One 16-deep MFMA step of the wave's 64 x 64 tile from LDS.
__device__ __forceinline__ void mma_k16(const uint16_t* __restrict__ sA,
                                        const uint16_t* __restrict__ sB, int kk,
                                        f32x16_t (&acc)[kTM][kTN]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, lg = lane >> 5;
  uint4 a[kTM], b[kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
    a[i] = *reinterpret_cast<const uint4*>(sA + (wm * (kBM / 2) + i * 32 + li) * kLD + kk * 16 + 8 * lg);
#pragma unroll
  for (int j = 0; j < kTN; ++j)
    b[j] = *reinterpret_cast<const uint4*>(sB + (wn * (kBN / 2) + j * 32 + li) * kLD + kk * 16 + 8 * lg);
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
}

__device__ __forceinline__ void mma_steps(const uint16_t* __restrict__ sA,
                                          const uint16_t* __restrict__ sB, int ksteps,
                                          f32x16_t (&acc)[kTM][kTN]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, lg = lane >> 5;
  for (int kk = 0; kk < ksteps; ++kk) {
    uint4 a[kTM], b[kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
      a[i] = *reinterpret_cast<const uint4*>(sA + (wm * (kBM / 2) + i * 32 + li) * kLD + kk * 16 + 8 * lg);
#pragma unroll
    for (int j = 0; j < kTN; ++j)
      b[j] = *reinterpret_cast<const uint4*>(sB + (wn * (kBN / 2) + j * 32 + li) * kLD + kk * 16 + 8 * lg);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
  }
}

// Output tile of workgroup `bid` (1-D grid over nr x nc tiles).  Workgroups
// are dealt to the 8 XCDs round-robin (bid % 8) and each XCD has its own
// L2, so when the tile count divides by 8 each XCD gets one contiguous run
// of the tile order below: bands of kBandRows row tiles, column-major
// inside a band.  An XCD then works on a few row tiles x a slice of the
// columns, which keeps its share of x and W small enough to be reused from
// its L2 instead of being fetched by all 8 XCDs.
constexpr int kBandRows = 4;

__device__ __forceinline__ void tile_of(int bid, int nc, int nr, int& row, int& col) {
  const int total = nc * nr;
  int q = bid;
  if ((total & 7) == 0) q = (bid & 7) * (total >> 3) + (bid >> 3);
  const int band = q / (kBandRows * nc);
  const int local = q - band * kBandRows * nc;
  const int rows = nr - band * kBandRows < kBandRows ? nr - band * kBandRows : kBandRows;
  col = local / rows;
  row = band * kBandRows + local % rows;
}

template <bool kBwd, bool kDQ>
__global__ __launch_bounds__(512, kWGPerCU) void gemm_kernel(GemmArgs g, CodeParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kLD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBN * kLD];
  __shared__ __attribute__((aligned(16))) float scode[16 * 64];  // q[c] for lane l at [64 c + l]
  const int t = threadIdx.x;
  {
    const CodeRegs R = code_regs(P);
    for (int i = t; i < 16 * 64; i += blockDim.x) scode[i] = code_value(R, i >> 6);
  }

  const int64_t ncols = kBwd ? g.K : g.N;
  int trow, tcol;
  tile_of(blockIdx.x, static_cast<int>((ncols + kBN - 1) / kBN),
          static_cast<int>((g.M + kBM - 1) / kBM), trow, tcol);
  const int64_t m0 = static_cast<int64_t>(trow) * kBM;
  const int64_t c0 = static_cast<int64_t>(tcol) * kBN;  // output column tile
  const int nk = static_cast<int>((kBwd ? g.N : g.K) / kBK);

  f32x16_t acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Waves 0-3 run the MFMAs, waves 4-7 load and dequantise; each SIMD holds
  // one of each.  Two LDS buffers: while the MFMA waves consume step k from
  // buffer k % 2, the producer waves dequantise step k + 1 into the other
  // buffer from registers loaded two steps earlier (a ring of three register
  // sets, loads of steps k + 2 and k + 3 in flight).  One barrier per K
  // step.  Steps past the end re-load the last step; what they store is
  // never read.
  if (t >= 256) {
    const int pt = t - 256;
    Prefetch p0, p1, p2;
    load_step<kBwd, kDQ>(g, m0, c0, 0, p0, pt);
    load_step<kBwd, kDQ>(g, m0, c0, nk > 1 ? 1 : nk - 1, p1, pt);
    load_step<kBwd, kDQ>(g, m0, c0, nk > 2 ? 2 : nk - 1, p2, pt);
    __syncthreads();  // code table visible
    {
      const float cs = chunk_scale<kDQ>(p0);
      store_step<kBwd>(p0, cs, scode, sA[0], sB[0], pt);
    }
    __syncthreads();
    auto step = [&](int k, Prefetch& dec, Prefetch& ld) {
      const int kl = k + 3 < nk ? k + 3 : nk - 1;
      const int nxt = (k & 1) ^ 1;
      // Pin the first use of the registers loaded two steps ago here, after
      // the barrier, so the compiler cannot hoist their address arithmetic
      // next to the loads it has just issued and wait for those.
      asm volatile("" : "+v"(dec.w), "+v"(dec.q8), "+v"(dec.c));
      const float cs = chunk_scale<kDQ>(dec);
      load_step<kBwd, kDQ>(g, m0, c0, kl, ld, pt);
      store_step<kBwd>(dec, cs, scode, sA[nxt], sB[nxt], pt);
      __syncthreads();
    };
    int k = 0;
    for (; k + 2 < nk; k += 3) {
      step(k, p1, p0);
      step(k + 1, p2, p1);
      step(k + 2, p0, p2);
    }
    if (k < nk) step(k, p1, p0);
    if (k + 1 < nk) step(k + 1, p2, p1);
  } else {
    __syncthreads();
    __syncthreads();
    for (int k = 0; k < nk; ++k) {
      const int cur = k & 1;
#pragma unroll
      for (int kk = 0; kk < kParts; ++kk) mma_k16(sA[cur], sB[cur], kk, acc);
      __syncthreads();
    }
  }

  // LoRA contraction of depth r, kBK at a time, through buffer 0.
  for (int j0 = 0; j0 < g.r; j0 += kBK) {
    for (int c = t; c < kBM * kBK; c += 512) {
      const int row = c / kBK, col = c % kBK;
      const int64_t m = m0 + row;
      uint16_t v = 0;
      if (m < g.M && j0 + col < g.r) v = g.lact[m * g.r + j0 + col];
      sA[0][row * kLD + col] = v;
    }
    for (int c = t; c < kBN * kBK; c += 512) {
      uint16_t v = 0;
      if constexpr (kBwd) {  // sB[kcol][j] = A[j0 + j][c0 + kcol]
        const int kcol = c % kBN, j = c / kBN;
        if (j0 + j < g.r && c0 + kcol < g.K) v = g.lw[static_cast<int64_t>(j0 + j) * g.K + c0 + kcol];
        sB[0][kcol * kLD + j] = v;
      } else {               // sB[n][j] = B[c0 + n][j0 + j]
        const int n = c / kBK, j = c % kBK;
        if (c0 + n < g.N && j0 + j < g.r) v = g.lw[(c0 + n) * g.r + j0 + j];
        sB[0][n * kLD + j] = v;
      }
    }
    __syncthreads();
    const int depth = g.r - j0 < kBK ? g.r - j0 : kBK;
    if (t < 256) mma_steps(sA[0], sB[0], (depth + 15) >> 4, acc);
    __syncthreads();
  }
  if (t >= 256) return;

  // Epilogue: accumulators straight to bf16 in HBM.  Lane (li, lg) of an
  // MFMA tile holds column li of rows 8 (v / 4) + 4 lg + v % 4, so each
  // store instruction writes 32 consecutive columns of two rows.
  {
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 31, lg = lane >> 5;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * (kBM / 2) + i * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
          const int col = wn * (kBN / 2) + j * 32 + li;
          const int64_t m = m0 + row, n = c0 + col;
          if (m < g.M && n < ncols)
            g.out[m * ncols + n] = static_cast<uint16_t>(pack_bf16x2(acc[i][j][v], 0.f) & 0xFFFF);
        }
  }
}

CodeParams code_params() {
  const Tables* t = tables();
  CodeParams P;
  for (int i = 0; i < 16; ++i) P.q[i] = t->q32[i];
  return P;
}

}  // namespace

hipError_t launch_gemm_fwd(const WeightView& w, const uint16_t* x, int64_t M,
                           const uint16_t* us, const uint16_t* B, int r, uint16_t* y,
                           hipStream_t st) {
  if (M == 0 || w.N == 0) return hipSuccess;
  GemmArgs g{w.packed, w.qscale, w.gscale, w.absmax, w.N, w.K, M, x, us, B, r, y};
  const dim3 grid(static_cast<uint32_t>(((w.N + kBN - 1) / kBN) * ((M + kBM - 1) / kBM)));
  if (w.qscale)
    hipLaunchKernelGGL((gemm_kernel<false, true>), grid, dim3(512), 0, st, g, code_params());
  else
    hipLaunchKernelGGL((gemm_kernel<false, false>), grid, dim3(512), 0, st, g, code_params());
  return hipGetLastError();
}

hipError_t launch_gemm_bwd(const WeightView& w, const uint16_t* dy, int64_t M,
                           const uint16_t* ts, const uint16_t* A, int r, uint16_t* dx,
                           hipStream_t st) {
  if (M == 0 || w.K == 0) return hipSuccess;
  GemmArgs g{w.packed, w.qscale, w.gscale, w.absmax, w.N, w.K, M, dy, ts, A, r, dx};
  const dim3 grid(static_cast<uint32_t>(((w.K + kBN - 1) / kBN) * ((M + kBM - 1) / kBM)));
  if (w.qscale)
    hipLaunchKernelGGL((gemm_kernel<true, true>), grid, dim3(512), 0, st, g, code_params());
  else
    hipLaunchKernelGGL((gemm_kernel<true, false>), grid, dim3(512), 0, st, g, code_params());
  return hipGetLastError();
}

}  // namespace qn
