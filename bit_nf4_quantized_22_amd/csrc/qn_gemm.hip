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
// Tiling.  Workgroup tile BM x BN = 128 x 128, 4 waves in a 2 x 2 grid, each
// wave 64 x 64 = 2 x 2 tiles of the 32x32x16 bf16 MFMA; K step 64 (one
// quantisation block).  Two LDS buffers per operand (rows padded by 16
// bytes, 74 KB per workgroup, two workgroups per CU).  While the MFMAs of
// step k read one buffer, the same waves dequantise step k+1 from registers
// into the other, a quarter per 16-deep MFMA step, and the global loads of
// step k+2 are in flight: one barrier per K step.  All global loads are
// unconditional (edge rows re-read a valid row), which keeps the compiler
// from serialising them behind branches.
// The dequantisation is a byte -> (q[hi], q[lo]) lookup in an LDS table,
// a multiply by the block constant and a packed bf16 conversion.  The
// forward stages the weight tile row-major ([n][k]); the backward needs 8
// consecutive n per MFMA lane, so it writes the dequantised tile transposed
// ([k][n]).

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLD = kBK + 8;    // bf16 per LDS operand row (144 bytes)
constexpr int kTM = kBM / 64, kTN = kBN / 64;  // MFMA tiles per wave (wave tile 64 x 64)
constexpr int kAChunks = kBM * 8 / 256;        // 16-byte activation chunks per thread

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

// Registers of the next K step: activation chunks, one 16-byte weight chunk
// (32 codes of one block) and its block constant (q8 code + group
// constant, or absmax).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Prefetch {
  u32x4 a[kAChunks];
  u32x4 w;
  uint32_t q8;
  float c;
};

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Global loads of contraction step kt into registers.
//   activation: thread t owns rows (t/8) + 32 i, 16 bytes at column 8 (t%8)
//   forward weight: thread t owns row c0 + t/2, codes k0 + 32 (t%2) .. +32
//   backward weight: thread t owns row k0 + t%64, codes c0 + 32 (t/64) .. +32
template <bool kBwd, bool kDQ>
__device__ __forceinline__ void load_step(const GemmArgs& g, int64_t m0, int64_t c0, int kt,
                                          Prefetch& pf) {
  const int t = threadIdx.x;
  const int64_t L = kBwd ? g.N : g.K;
  const int64_t k0 = static_cast<int64_t>(kt) * kBK;
  // Rows past M and weight rows/columns past the output edge re-read a
  // valid row: they only feed outputs that are never stored.
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    const int row = (t >> 3) + 32 * i, col = (t & 7) * 8;
    const int64_t m = m0 + row < g.M ? m0 + row : g.M - 1;
    pf.a[i] = *reinterpret_cast<const u32x4*>(g.act + m * L + k0 + col);
  }
  int64_t n, k;
  if constexpr (kBwd) {
    n = k0 + (t & 63);
    k = c0 + 32 * (t >> 6);
    k = k < g.K ? k : g.K - 32;
  } else {
    n = c0 + (t >> 1);
    k = k0 + 32 * (t & 1);
    n = n < g.N ? n : g.N - 1;
  }
  pf.w = *reinterpret_cast<const u32x4*>(g.packed + n * (g.K >> 1) + (k >> 1));
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

// Part i (of 4) of the register -> LDS store of one K step: activation
// chunk i as is, weight word i (8 codes) dequantised.
template <bool kBwd>
__device__ __forceinline__ void store_part(int i, const Prefetch& pf, float cs,
                                           const float2* __restrict__ spair,
                                           uint16_t* __restrict__ sA, uint16_t* __restrict__ sB) {
  const int t = threadIdx.x;
  if (i < kAChunks) {
    const int row = (t >> 3) + 32 * i, col = (t & 7) * 8;
    *reinterpret_cast<u32x4*>(sA + row * kLD + col) = pf.a[i];
  }
  const uint32_t word = pf.w[i];
  uint32_t d[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float2 pr = spair[(word >> (8 * b)) & 0xFF];
    d[b] = pack_bf16x2(__fmul_rn(pr.x, cs), __fmul_rn(pr.y, cs));
  }
  if constexpr (kBwd) {
    const int row = t & 63, q = t >> 6;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      sB[(32 * q + 8 * i + 2 * b) * kLD + row] = static_cast<uint16_t>(d[b] & 0xFFFF);
      sB[(32 * q + 8 * i + 2 * b + 1) * kLD + row] = static_cast<uint16_t>(d[b] >> 16);
    }
  } else {
    *reinterpret_cast<u32x4*>(sB + (t >> 1) * kLD + 32 * (t & 1) + 8 * i) = u32x4{d[0], d[1], d[2], d[3]};
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

template <bool kBwd, bool kDQ>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs g, CodeParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kLD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBN * kLD];
  __shared__ float2 spair[256];
  const int t = threadIdx.x;
  fill_pair_f32(spair, P, 1);

  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kBN;  // output column tile
  const int64_t ncols = kBwd ? g.K : g.N;
  const int nk = static_cast<int>((kBwd ? g.N : g.K) / kBK);

  f32x16_t acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Two register sets and two LDS buffers.  While the MFMAs consume step k
  // from LDS buffer k % 2, the same waves dequantise step k + 1 (loaded one
  // step earlier) into the other buffer, and the loads of step k + 2 are in
  // flight: one barrier per K step.  Steps past the end re-load the last
  // step; what they store is never read.
  Prefetch p0, p1;
  load_step<kBwd, kDQ>(g, m0, c0, 0, p0);
  load_step<kBwd, kDQ>(g, m0, c0, nk > 1 ? 1 : 0, p1);
  __syncthreads();  // spair visible
  {
    const float cs = chunk_scale<kDQ>(p0);
#pragma unroll
    for (int i = 0; i < 4; ++i) store_part<kBwd>(i, p0, cs, spair, sA[0], sB[0]);
  }
  __syncthreads();
  auto step = [&](int k, Prefetch& dec, Prefetch& ld, int cur) {
    const int kl = k + 2 < nk ? k + 2 : nk - 1;
    const float cs = chunk_scale<kDQ>(dec);
    load_step<kBwd, kDQ>(g, m0, c0, kl, ld);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      mma_k16(sA[cur], sB[cur], kk, acc);
      store_part<kBwd>(kk, dec, cs, spair, sA[cur ^ 1], sB[cur ^ 1]);
    }
    __syncthreads();
  };
  int k = 0;
  for (; k + 1 < nk; k += 2) {
    step(k, p1, p0, 0);
    step(k + 1, p0, p1, 1);
  }
  if (k < nk) step(k, p1, p0, 0);

  // LoRA contraction of depth r, 64 at a time, through buffer 0.
  for (int j0 = 0; j0 < g.r; j0 += kBK) {
    for (int c = t; c < kBM * kBK; c += 256) {
      const int row = c >> 6, col = c & 63;
      const int64_t m = m0 + row;
      uint16_t v = 0;
      if (m < g.M && j0 + col < g.r) v = g.lact[m * g.r + j0 + col];
      sA[0][row * kLD + col] = v;
    }
    for (int c = t; c < kBN * kBK; c += 256) {
      uint16_t v = 0;
      if constexpr (kBwd) {  // sB[kcol][j] = A[j0 + j][c0 + kcol]
        const int kcol = c % kBN, j = c / kBN;
        if (j0 + j < g.r && c0 + kcol < g.K) v = g.lw[static_cast<int64_t>(j0 + j) * g.K + c0 + kcol];
        sB[0][kcol * kLD + j] = v;
      } else {               // sB[n][j] = B[c0 + n][j0 + j]
        const int n = c >> 6, j = c & 63;
        if (c0 + n < g.N && j0 + j < g.r) v = g.lw[(c0 + n) * g.r + j0 + j];
        sB[0][n * kLD + j] = v;
      }
    }
    __syncthreads();
    const int depth = g.r - j0 < kBK ? g.r - j0 : kBK;
    mma_steps(sA[0], sB[0], (depth + 15) >> 4, acc);
    __syncthreads();
  }

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
  const dim3 grid(static_cast<uint32_t>((w.N + kBN - 1) / kBN),
                  static_cast<uint32_t>((M + kBM - 1) / kBM));
  if (w.qscale)
    hipLaunchKernelGGL((gemm_kernel<false, true>), grid, dim3(256), 0, st, g, code_params());
  else
    hipLaunchKernelGGL((gemm_kernel<false, false>), grid, dim3(256), 0, st, g, code_params());
  return hipGetLastError();
}

hipError_t launch_gemm_bwd(const WeightView& w, const uint16_t* dy, int64_t M,
                           const uint16_t* ts, const uint16_t* A, int r, uint16_t* dx,
                           hipStream_t st) {
  if (M == 0 || w.K == 0) return hipSuccess;
  GemmArgs g{w.packed, w.qscale, w.gscale, w.absmax, w.N, w.K, M, dy, ts, A, r, dx};
  const dim3 grid(static_cast<uint32_t>((w.K + kBN - 1) / kBN),
                  static_cast<uint32_t>((M + kBM - 1) / kBM));
  if (w.qscale)
    hipLaunchKernelGGL((gemm_kernel<true, true>), grid, dim3(256), 0, st, g, code_params());
  else
    hipLaunchKernelGGL((gemm_kernel<true, false>), grid, dim3(256), 0, st, g, code_params());
  return hipGetLastError();
}

}  // namespace qn
