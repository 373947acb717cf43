// LoRA gradients (gfx950):  dA = s (dy B)^T x,  dB = s dy^T (x A^T).
//
// [kwkr "QLoRA原理深入" §2.3] gradients flow only into the LoRA bypass; the
// 4-bit weight and its constants get none, so this is all the backward
// produces besides dx.
//
// Both are reductions over the M tokens of a product of a wide bf16 matrix
// (x [M, K] or dy [M, N]) with a narrow fp32/bf16 one (t or u, [M, r]).  The
// wide matrix is read once: workgroups own 256 consecutive columns and one
// chunk of 256 tokens, keep r fp32 accumulators per column, and write a
// partial [chunk][r][cols]; a second pass sums the chunks in a fixed order
// and applies s.  Bit-reproducible run to run.

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

constexpr int kChunk = 256;  // tokens per partial
constexpr int kRows = 32;    // tokens staged in LDS at a time

template <typename T>
__device__ __forceinline__ float ld_narrow(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld_narrow<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_narrow<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

template <int RT, typename T>
__global__ __launch_bounds__(256) void grads_partial_kernel(const uint16_t* __restrict__ X,
                                                            int64_t M, int64_t C,
                                                            const T* __restrict__ Tn, int r,
                                                            float* __restrict__ part) {
  __shared__ float sT[kRows][RT];
  const int64_t col = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t chunk = blockIdx.y;
  const int64_t mstart = chunk * kChunk;
  const int64_t mend = (mstart + kChunk < M) ? mstart + kChunk : M;
  float acc[RT];
#pragma unroll
  for (int j = 0; j < RT; ++j) acc[j] = 0.f;
  for (int64_t mb = mstart; mb < mend; mb += kRows) {
    for (int idx = threadIdx.x; idx < kRows * RT; idx += 256) {
      const int mm = idx / RT, j = idx % RT;
      sT[mm][j] = (mb + mm < mend && j < r) ? ld_narrow(Tn, (mb + mm) * r + j) : 0.f;
    }
    __syncthreads();
    // Rows past mend have sT == 0; their loads are clamped to a valid row.
    if (col < C) {
#pragma unroll 1
      for (int mm = 0; mm < kRows; mm += 8) {
        float xv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int64_t row = min(mb + mm + q, mend - 1);
          xv[q] = bf16_to_f32(X[row * C + col]);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int j = 0; j < RT; ++j) acc[j] = fmaf(sT[mm + q][j], xv[q], acc[j]);
      }
    }
    __syncthreads();
  }
  if (col < C)
    for (int j = 0; j < r; ++j) part[(chunk * r + j) * C + col] = acc[j];
}

// out = s * sum over chunks (fixed order); transposed writes out[col][j].
__global__ __launch_bounds__(256) void grads_reduce_kernel(const float* __restrict__ part,
                                                           int nchunk, int r, int64_t C,
                                                           float s, bool transposed,
                                                           float* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(r) * C) return;
  const int64_t j = idx / C, col = idx % C;
  float v = 0.f;
  for (int c = 0; c < nchunk; ++c) v += part[(c * r + j) * C + col];
  v *= s;
  if (transposed) out[col * r + j] = v;
  else out[j * C + col] = v;
}

template <typename T>
hipError_t launch_partial(const uint16_t* X, int64_t M, int64_t C, const T* Tn, int r,
                          float* part, hipStream_t st) {
  const dim3 grid(static_cast<uint32_t>((C + 255) / 256), static_cast<uint32_t>((M + kChunk - 1) / kChunk));
  if (r <= 16) hipLaunchKernelGGL((grads_partial_kernel<16, T>), grid, dim3(256), 0, st, X, M, C, Tn, r, part);
  else if (r <= 32) hipLaunchKernelGGL((grads_partial_kernel<32, T>), grid, dim3(256), 0, st, X, M, C, Tn, r, part);
  else if (r <= 64) hipLaunchKernelGGL((grads_partial_kernel<64, T>), grid, dim3(256), 0, st, X, M, C, Tn, r, part);
  else hipLaunchKernelGGL((grads_partial_kernel<128, T>), grid, dim3(256), 0, st, X, M, C, Tn, r, part);
  return hipGetLastError();
}

}  // namespace

size_t grads_workspace_bytes(int64_t M, int64_t N, int64_t K, int r) {
  const int64_t nchunk = (M + kChunk - 1) / kChunk;
  return static_cast<size_t>(nchunk) * static_cast<size_t>(r) * static_cast<size_t>(N + K) * 4;
}

hipError_t launch_grads_impl(const uint16_t* x, const uint16_t* dy, const void* u, bool u_bf16,
                             const void* t, bool t_bf16, int64_t M, int64_t N, int64_t K,
                             int r, float s, float* dA, float* dB, void* ws, hipStream_t st) {
  if (r == 0) return hipSuccess;
  const int nchunk = static_cast<int>((M + kChunk - 1) / kChunk);
  float* partA = static_cast<float*>(ws);
  float* partB = partA + static_cast<int64_t>(nchunk) * r * K;
  hipError_t e;
  if (M > 0) {
    e = t_bf16 ? launch_partial(x, M, K, static_cast<const uint16_t*>(t), r, partA, st)
               : launch_partial(x, M, K, static_cast<const float*>(t), r, partA, st);
    if (e != hipSuccess) return e;
    e = u_bf16 ? launch_partial(dy, M, N, static_cast<const uint16_t*>(u), r, partB, st)
               : launch_partial(dy, M, N, static_cast<const float*>(u), r, partB, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(grads_reduce_kernel, dim3(static_cast<uint32_t>((r * K + 255) / 256)), dim3(256), 0,
                     st, partA, nchunk, r, K, s, false, dA);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(grads_reduce_kernel, dim3(static_cast<uint32_t>((r * N + 255) / 256)), dim3(256), 0,
                     st, partB, nchunk, r, N, s, true, dB);
  return hipGetLastError();
}

}  // namespace qn
