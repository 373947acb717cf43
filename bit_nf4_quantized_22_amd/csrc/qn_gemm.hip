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
// quantisation block).  One LDS buffer per operand (rows padded by 16
// bytes, 37 KB per workgroup), so several workgroups share a CU and the
// hardware overlaps one workgroup's dequantise/store phase with another's
// MFMAs.  The global loads of step k+1 are issued before the MFMAs of step
// k and written to LDS after them, between two barriers.  (Measured on
// MI355X: double-buffered LDS, deeper register prefetch, a branch-free loop
// with clamped loads, an XCD-grouped tile order, 256 x 128 tiles, a
// replicated decode table and a 128 x 256 tile with the weight decoded into
// MFMA registers were all slower than this configuration.)
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
struct Prefetch {
  uint4 a[kAChunks];
  uint4 w;
  uint32_t q8;
  float c;
};

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Dequantise 32 consecutive codes (16 packed bytes, one block constant) to
// 16 bf16 pairs.
__device__ __forceinline__ void decode32(const float2* __restrict__ spair, const uint4& pk,
                                         float cs, uint32_t out[16]) {
  const uint32_t words[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
  for (int wi = 0; wi < 4; ++wi)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float2 pr = spair[(words[wi] >> (8 * b)) & 0xFF];
      out[4 * wi + b] = pack_bf16x2(__fmul_rn(pr.x, cs), __fmul_rn(pr.y, cs));
    }
}

// Global loads of contraction step kt into registers.
//   activation: thread t owns rows (t/8) + 32 i, 16 bytes at column 8 (t%8)
//   forward weight: thread t owns row c0 + t/2, codes k0 + 32 (t%2) .. +32
//   backward weight: thread t owns row k0 + t%64, codes c0 + 32 (t/64) .. +32
template <bool kBwd>
__device__ __forceinline__ void load_step(const GemmArgs& g, int64_t m0, int64_t c0, int kt,
                                          Prefetch& pf) {
  const int t = threadIdx.x;
  const int64_t L = kBwd ? g.N : g.K;
  const int64_t k0 = static_cast<int64_t>(kt) * kBK;
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    const int row = (t >> 3) + 32 * i, col = (t & 7) * 8;
    const int64_t m = m0 + row;
    pf.a[i] = m < g.M ? *reinterpret_cast<const uint4*>(g.act + m * L + k0 + col)
                      : make_uint4(0, 0, 0, 0);
  }
  int64_t n, k;
  if constexpr (kBwd) {
    n = k0 + (t & 63);
    k = c0 + 32 * (t >> 6);
  } else {
    n = c0 + (t >> 1);
    k = k0 + 32 * (t & 1);
  }
  const bool live = kBwd ? (k < g.K) : (n < g.N);
  pf.w = make_uint4(0, 0, 0, 0);
  pf.q8 = 0;
  pf.c = 0.f;
  if (live) {
    pf.w = *reinterpret_cast<const uint4*>(g.packed + n * (g.K >> 1) + (k >> 1));
    const int64_t bi = n * (g.K >> 6) + (k >> 6);
    if (g.qscale) {
      pf.q8 = g.qscale[bi];
      pf.c = g.gscale[bi >> 8];
    } else {
      pf.c = g.absmax[bi];
    }
  }
}

// Registers -> LDS buffer (dequantising the weight chunk).
template <bool kBwd>
__device__ __forceinline__ void store_step(const GemmArgs& g, const Prefetch& pf,
                                           const float2* __restrict__ spair,
                                           uint16_t* __restrict__ sA, uint16_t* __restrict__ sB) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    const int row = (t >> 3) + 32 * i, col = (t & 7) * 8;
    *reinterpret_cast<uint4*>(sA + row * kLD + col) = pf.a[i];
  }
  const float cs = g.qscale ? __fmul_rn(l8_value(pf.q8), pf.c) : pf.c;
  uint32_t d[16];
  decode32(spair, pf.w, cs, d);
  if constexpr (kBwd) {
    const int row = t & 63, q = t >> 6;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sB[(32 * q + 2 * i) * kLD + row] = static_cast<uint16_t>(d[i] & 0xFFFF);
      sB[(32 * q + 2 * i + 1) * kLD + row] = static_cast<uint16_t>(d[i] >> 16);
    }
  } else {
    uint4* dst = reinterpret_cast<uint4*>(sB + (t >> 1) * kLD + 32 * (t & 1));
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]);
  }
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

template <bool kBwd>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs g, CodeParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[1][kBM * kLD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[1][kBN * kLD];
  __shared__ float2 spair[256];
  const int t = threadIdx.x;
  fill_pair_f32(spair, P, 1);

  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kBN;  // output column tile
  const int64_t L = kBwd ? g.N : g.K;
  const int64_t ncols = kBwd ? g.K : g.N;
  const int nk = static_cast<int>(L / kBK);

  f32x16_t acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  Prefetch pf;
  load_step<kBwd>(g, m0, c0, 0, pf);
  __syncthreads();  // spair visible
  store_step<kBwd>(g, pf, spair, sA[0], sB[0]);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_step<kBwd>(g, m0, c0, kt + 1, pf);
    mma_steps(sA[0], sB[0], kBK / 16, acc);
    __syncthreads();
    if (kt + 1 < nk) store_step<kBwd>(g, pf, spair, sA[0], sB[0]);
    __syncthreads();
  }

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
  hipLaunchKernelGGL(gemm_kernel<false>, grid, dim3(256), 0, st, g, code_params());
  return hipGetLastError();
}

hipError_t launch_gemm_bwd(const WeightView& w, const uint16_t* dy, int64_t M,
                           const uint16_t* ts, const uint16_t* A, int r, uint16_t* dx,
                           hipStream_t st) {
  if (M == 0 || w.K == 0) return hipSuccess;
  GemmArgs g{w.packed, w.qscale, w.gscale, w.absmax, w.N, w.K, M, dy, ts, A, r, dx};
  const dim3 grid(static_cast<uint32_t>((w.K + kBN - 1) / kBN),
                  static_cast<uint32_t>((M + kBM - 1) / kBM));
  hipLaunchKernelGGL(gemm_kernel<true>, grid, dim3(256), 0, st, g, code_params());
  return hipGetLastError();
}

}  // namespace qn
