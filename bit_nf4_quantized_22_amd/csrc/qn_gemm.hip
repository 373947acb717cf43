// Fused dequant -> bf16 MFMA GEMMs for token batches (gfx950).
//
// Forward  y[M, N]  = x[M, K] W^T + (s u)[M, r] B^T      (contraction over K)
// Backward dx[M, K] = dy[M, N] W  + (s t)[M, r] A        (contraction over N)
//
// [kwkr "QLoRA原理深入" §2.3] the 4-bit weight is expanded to 16 bits for the
// matrix product and never written back; [rkmt "QLORA技术解析" §3.2] compute
// type bf16.  The weight tile is dequantised straight into LDS as
// bf16(fl32(q[code] * c')), the same bf16 value nf4_dequant produces, and
// never touches HBM in 16-bit form.  The LoRA term rides on the same
// accumulators as one extra contraction of depth r: the A-side operand is
// bf16(s u) (or bf16(s t)), the B-side operand is B (or A^T).
//
// Tiling: workgroup tile BM x BN, 4 waves in a 2 x 2 grid, each wave
// (BM/2) x (BN/2) made of 32x32x16 bf16 MFMA tiles; K step 64 staged
// through LDS (rows padded by 16 bytes).  The forward stages the weight tile
// row-major ([n][k]); the backward needs k-major columns of 8 consecutive n
// per MFMA lane, so it writes the dequantised tile transposed ([k][n]).

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

constexpr int kBK = 64;
constexpr int kLD = kBK + 8;  // bf16 per LDS row (144 bytes)

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Dequantise 32 consecutive codes (16 packed bytes, one block constant) to
// bf16 pairs.
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

template <int BM, int BN>
__device__ __forceinline__ void mma_tile(const uint16_t* __restrict__ As,
                                         const uint16_t* __restrict__ Bs, int ksteps,
                                         f32x16_t (&acc)[BM / 64][BN / 64]) {
  constexpr int TM = BM / 64, TN = BN / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, lg = lane >> 5;
  for (int kk = 0; kk < ksteps; ++kk) {
    uint4 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      a[i] = *reinterpret_cast<const uint4*>(As + (wm * (BM / 2) + i * 32 + li) * kLD + kk * 16 + 8 * lg);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      b[j] = *reinterpret_cast<const uint4*>(Bs + (wn * (BN / 2) + j * 32 + li) * kLD + kk * 16 + 8 * lg);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
  }
}

template <int BM, int BN>
__device__ __forceinline__ void store_tile(const f32x16_t (&acc)[BM / 64][BN / 64],
                                           uint16_t* __restrict__ out, int64_t rows,
                                           int64_t cols, int64_t r0, int64_t c0) {
  constexpr int TM = BM / 64, TN = BN / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, lg = lane >> 5;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = c0 + wn * (BN / 2) + j * 32 + li;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = r0 + wm * (BM / 2) + i * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
        if (row < rows && col < cols)
          out[row * cols + col] = static_cast<uint16_t>(pack_bf16x2(acc[i][j][v], 0.f) & 0xFFFF);
      }
    }
}

// Stage rows [r0, r0 + ROWS) x cols [c0, c0 + 64) of a bf16 row-major matrix
// (row stride ld) into LDS, zero outside [0, nrows).
template <int ROWS>
__device__ __forceinline__ void stage_rows(uint16_t* __restrict__ S, const uint16_t* __restrict__ g,
                                           int64_t ld, int64_t nrows, int64_t r0, int64_t c0) {
  for (int c = threadIdx.x; c < ROWS * 8; c += 256) {
    const int row = c >> 3, col = (c & 7) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + row < nrows) v = *reinterpret_cast<const uint4*>(g + (r0 + row) * ld + c0 + col);
    *reinterpret_cast<uint4*>(S + row * kLD + col) = v;
  }
}

// Stage a [ROWS, 64] window of a small bf16 matrix with `width` valid
// columns (element loads; columns >= width and rows >= nrows are zero).
template <int ROWS>
__device__ __forceinline__ void stage_small(uint16_t* __restrict__ S, const uint16_t* __restrict__ g,
                                            int64_t ld, int64_t nrows, int width, int64_t r0,
                                            int c0) {
  for (int c = threadIdx.x; c < ROWS * 64; c += 256) {
    const int row = c >> 6, col = c & 63;
    uint16_t v = 0;
    if (r0 + row < nrows && c0 + col < width) v = g[(r0 + row) * ld + c0 + col];
    S[row * kLD + col] = v;
  }
}

template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_fwd_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ gscale, const float* __restrict__ absmax, int64_t N, int64_t K,
    const uint16_t* __restrict__ x, int64_t M, const uint16_t* __restrict__ us,
    const uint16_t* __restrict__ B, int r, uint16_t* __restrict__ y, PairF32Params P) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * kLD];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[BN * kLD];
  __shared__ float2 spair[256];
  spair[threadIdx.x] = make_float2(P.pair[2 * threadIdx.x], P.pair[2 * threadIdx.x + 1]);

  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;
  const int64_t nblk = K >> 6;
  f32x16_t acc[BM / 64][BN / 64];
#pragma unroll
  for (int i = 0; i < BM / 64; ++i)
#pragma unroll
    for (int j = 0; j < BN / 64; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  __syncthreads();

  for (int64_t k0 = 0; k0 < K; k0 += kBK) {
    stage_rows<BM>(As, x, K, M, m0, k0);
    for (int c = threadIdx.x; c < BN * 2; c += 256) {
      const int row = c >> 1, half = c & 1;
      const int64_t n = n0 + row;
      uint32_t d[16];
      if (n < N) {
        const uint4 pk = *reinterpret_cast<const uint4*>(packed + n * (K >> 1) + (k0 >> 1) + half * 16);
        decode32(spair, pk, block_scale(qscale, gscale, absmax, n * nblk + (k0 >> 6)), d);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) d[i] = 0;
      }
      uint4* dst = reinterpret_cast<uint4*>(Ws + row * kLD + half * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = make_uint4(d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]);
    }
    __syncthreads();
    mma_tile<BM, BN>(As, Ws, kBK / 16, acc);
    __syncthreads();
  }
  for (int j0 = 0; j0 < r; j0 += kBK) {
    stage_small<BM>(As, us, r, M, r, m0, j0);
    stage_small<BN>(Ws, B, r, N, r, n0, j0);
    __syncthreads();
    const int depth = r - j0 < kBK ? r - j0 : kBK;
    mma_tile<BM, BN>(As, Ws, (depth + 15) >> 4, acc);
    __syncthreads();
  }
  store_tile<BM, BN>(acc, y, M, N, m0, n0);
}

template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_bwd_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ gscale, const float* __restrict__ absmax, int64_t N, int64_t K,
    const uint16_t* __restrict__ dy, int64_t M, const uint16_t* __restrict__ ts,
    const uint16_t* __restrict__ A, int r, uint16_t* __restrict__ dx, PairF32Params P) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * kLD];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[BN * kLD];  // [k][n] (transposed)
  __shared__ float2 spair[256];
  spair[threadIdx.x] = make_float2(P.pair[2 * threadIdx.x], P.pair[2 * threadIdx.x + 1]);

  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
  const int64_t kc0 = static_cast<int64_t>(blockIdx.x) * BN;  // output columns (k)
  const int64_t nblk = K >> 6;
  f32x16_t acc[BM / 64][BN / 64];
#pragma unroll
  for (int i = 0; i < BM / 64; ++i)
#pragma unroll
    for (int j = 0; j < BN / 64; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  __syncthreads();

  for (int64_t nc = 0; nc < N; nc += kBK) {
    stage_rows<BM>(As, dy, N, M, m0, nc);
    // weight rows nc..nc+63, columns kc0..kc0+BN-1, written as Ws[k][n]
    for (int c = threadIdx.x; c < kBK * (BN / 32); c += 256) {
      const int row = c & 63, q = c >> 6;
      const int64_t n = nc + row;
      const int64_t k = kc0 + 32 * q;
      uint32_t d[16];
      if (k < K) {
        const uint4 pk = *reinterpret_cast<const uint4*>(packed + n * (K >> 1) + (k >> 1));
        decode32(spair, pk, block_scale(qscale, gscale, absmax, n * nblk + (k >> 6)), d);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) d[i] = 0;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        Ws[(32 * q + 2 * i) * kLD + row] = static_cast<uint16_t>(d[i] & 0xFFFF);
        Ws[(32 * q + 2 * i + 1) * kLD + row] = static_cast<uint16_t>(d[i] >> 16);
      }
    }
    __syncthreads();
    mma_tile<BM, BN>(As, Ws, kBK / 16, acc);
    __syncthreads();
  }
  for (int j0 = 0; j0 < r; j0 += kBK) {
    stage_small<BM>(As, ts, r, M, r, m0, j0);
    // Ws[kcol][j] = A[j0 + j][kc0 + kcol]
    for (int c = threadIdx.x; c < BN * kBK; c += 256) {
      const int kcol = c % BN, j = c / BN;
      uint16_t v = 0;
      if (j0 + j < r && kc0 + kcol < K) v = A[static_cast<int64_t>(j0 + j) * K + kc0 + kcol];
      Ws[kcol * kLD + j] = v;
    }
    __syncthreads();
    const int depth = r - j0 < kBK ? r - j0 : kBK;
    mma_tile<BM, BN>(As, Ws, (depth + 15) >> 4, acc);
    __syncthreads();
  }
  store_tile<BM, BN>(acc, dx, M, K, m0, kc0);
}

PairF32Params pair_params() {
  const Tables* t = tables();
  PairF32Params P;
  for (int i = 0; i < 512; ++i) P.pair[i] = t->pair_f32[i];
  return P;
}

}  // namespace

hipError_t launch_gemm_fwd(const WeightView& w, const uint16_t* x, int64_t M,
                           const uint16_t* us, const uint16_t* B, int r, uint16_t* y,
                           hipStream_t st) {
  if (M == 0 || w.N == 0) return hipSuccess;
  constexpr int BM = 128, BN = 128;
  const dim3 grid(static_cast<uint32_t>((w.N + BN - 1) / BN), static_cast<uint32_t>((M + BM - 1) / BM));
  hipLaunchKernelGGL((gemm_fwd_kernel<BM, BN>), grid, dim3(256), 0, st, w.packed, w.qscale,
                     w.gscale, w.absmax, w.N, w.K, x, M, us, B, r, y, pair_params());
  return hipGetLastError();
}

hipError_t launch_gemm_bwd(const WeightView& w, const uint16_t* dy, int64_t M,
                           const uint16_t* ts, const uint16_t* A, int r, uint16_t* dx,
                           hipStream_t st) {
  if (M == 0 || w.K == 0) return hipSuccess;
  constexpr int BM = 128, BN = 128;
  const dim3 grid(static_cast<uint32_t>((w.K + BN - 1) / BN), static_cast<uint32_t>((M + BM - 1) / BM));
  hipLaunchKernelGGL((gemm_bwd_kernel<BM, BN>), grid, dim3(256), 0, st, w.packed, w.qscale,
                     w.gscale, w.absmax, w.N, w.K, dy, M, ts, A, r, dx, pair_params());
  return hipGetLastError();
}

}  // namespace qn
