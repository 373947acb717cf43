// LoRA gradients (gfx950):  dA = s (dy B)^T x,  dB = s dy^T (x A^T).
//
// [kwkr "QLoRA原理深入" §2.3] gradients flow only into the LoRA bypass; the
// 4-bit weight and its constants get none, so this is all the backward
// produces besides dx.
//
// Both are out[r, C] = P^T X summed over the M tokens, with X the wide bf16
// matrix (x [M, K] or dy [M, N]) and P the narrow one (t or u, [M, r], fp32
// or bf16): a contraction along M, the slow dimension of both row-major
// inputs.  MFMA 16x16x32 needs each lane to hold 8 consecutive tokens of
// one column, so every 64-token step of X is loaded with coalesced 16-byte
// loads and written *transposed* into LDS as bf16 pairs (column-major
// [column][token], row pitch 72 halves so the operand reads are
// conflict-free); P is staged the same way.  The next step's loads are in
// flight during a step's MFMAs: 32 KB per workgroup, since with about one
// workgroup per CU the bytes in flight set the streaming rate.  Workgroups own 256 columns and
// a token chunk, write fp32 partial sums [chunk][r][C], and a second pass
// sums the chunks in a fixed order and applies s (bit-reproducible).  The
// wide matrix is read once; the partials are a small fraction of it.

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

constexpr int kCols = 256;    // columns of X per workgroup (4 waves x 64)
constexpr int kStep = 64;     // tokens per step (two 32-deep MFMA steps)
constexpr int kQ = kStep / 16;  // 16-token row groups per step
constexpr int kPitch = kStep + 8;  // LDS row pitch of the transposed tiles, in bf16

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ float ld_narrow(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld_narrow<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_narrow<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// RT: rank tile (r <= RT, a multiple of 16).  Grid: (ceil(C / 256), chunks).
// Thread t loads, per step, rows 2 (t % 8) + {0, 1} + 16 q (q < kQ) of
// columns 8 (t / 8) .. + 7: 2 kQ 16-byte loads, 8 rows x 128 bytes per wave
// instruction.  Each pair of rows is packed per column into one 32-bit word
// and stored at [column][row pair] of the transposed tile.
template <int RT, typename T>
__global__ __launch_bounds__(256) void grads_mfma_kernel(const uint16_t* __restrict__ X, int64_t M,
                                                         int64_t C, const T* __restrict__ P, int r,
                                                         int64_t chunk, float* __restrict__ part) {
  constexpr int kPer = (kStep * RT + 255) / 256;  // P elements per thread per step
  __shared__ __attribute__((aligned(16))) uint16_t sX[kCols * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sP[RT * kPitch];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kCols;
  const int64_t m_lo = static_cast<int64_t>(blockIdx.y) * chunk;
  const int64_t m_hi = m_lo + chunk < M ? m_lo + chunk : M;
  const int nsteps = static_cast<int>((m_hi - m_lo + kStep - 1) / kStep);

  // loader roles
  const int lcg = tid >> 3;         // column group: columns 8 lcg .. + 7
  const int lrp = tid & 7;          // row pair within 16 rows
  const int64_t lcol = c0 + 8 * lcg;
  const int64_t lcolc = lcol + 8 <= C ? lcol : C - 8;  // C % 64 == 0: a valid 8-column group
  auto load_x = [&](int s, uint4 (&v)[2 * kQ]) {
#pragma unroll
    for (int q = 0; q < kQ; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int64_t m = m_lo + static_cast<int64_t>(s) * kStep + 16 * q + 2 * lrp + h;
        m = m < m_hi ? m : m_hi - 1;  // rows past the chunk: valid data, P zeroed
        v[2 * q + h] = *reinterpret_cast<const uint4*>(X + m * C + lcolc);
      }
  };
  auto load_p = [&](int s, float (&pv)[kPer]) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + 256 * i;
      const int mm = idx / RT, j = idx % RT;
      const int64_t m = m_lo + static_cast<int64_t>(s) * kStep + mm;
      const bool ok = idx < kStep * RT && j < r && m < m_hi;
      const float v = ld_narrow(P, (ok ? m : m_lo) * r + (ok ? j : 0));
      pv[i] = ok ? v : 0.f;
    }
  };

  f32x4_t acc[RT / 16][4];
#pragma unroll
  for (int a = 0; a < RT / 16; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 xv[2 * kQ];
  float pv[kPer];
  load_x(0, xv);
  load_p(0, pv);
  const int l16 = lane & 15, g = lane >> 4;
  for (int s = 0; s < nsteps; ++s) {
    __syncthreads();  // the previous step's operand reads are done
    // transposed stores: word (row pair lrp + 8 q) of column 8 lcg + e
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const uint32_t a0[4] = {xv[2 * q].x, xv[2 * q].y, xv[2 * q].z, xv[2 * q].w};
      const uint32_t a1[4] = {xv[2 * q + 1].x, xv[2 * q + 1].y, xv[2 * q + 1].z, xv[2 * q + 1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = e & 1 ? a0[e >> 1] >> 16 : a0[e >> 1] & 0xFFFFu;
        const uint32_t hi = e & 1 ? a1[e >> 1] & 0xFFFF0000u : a1[e >> 1] << 16;
        *reinterpret_cast<uint32_t*>(&sX[(8 * lcg + e) * kPitch + 16 * q + 2 * lrp]) = lo | hi;
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + 256 * i;
      if (idx < kStep * RT) {
        const int mm = idx / RT, j = idx % RT;
        sP[j * kPitch + mm] = static_cast<uint16_t>(pack_bf16x2(pv[i], 0.f) & 0xFFFF);
      }
    }
    __syncthreads();
    // next step's loads (clamped to the last step) before this step's MFMAs
    {
      const int sn = s + 1 < nsteps ? s + 1 : s;
      load_x(sn, xv);
      load_p(sn, pv);
    }
#pragma unroll
    for (int kk = 0; kk < kStep / 32; ++kk) {
      uint4 pa[RT / 16];
#pragma unroll
      for (int a = 0; a < RT / 16; ++a)
        pa[a] = *reinterpret_cast<const uint4*>(&sP[(16 * a + l16) * kPitch + 32 * kk + 8 * g]);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint4 xb = *reinterpret_cast<const uint4*>(
            &sX[(wave * 64 + 16 * b + l16) * kPitch + 32 * kk + 8 * g]);
#pragma unroll
        for (int a = 0; a < RT / 16; ++a) acc[a][b] = mfma16(pa[a], xb, acc[a][b]);
      }
    }
  }

  // lane (column l16, group g) holds rows j = 16 a + 4 g + v of columns
  // c0 + 64 wave + 16 b + l16
#pragma unroll
  for (int a = 0; a < RT / 16; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t col = c0 + wave * 64 + 16 * b + l16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 16 * a + 4 * g + v;
        if (j < r && col < C)
          part[(static_cast<int64_t>(blockIdx.y) * r + j) * C + col] = acc[a][b][v];
      }
    }
}

// out = s * sum over chunks (fixed order); transposed writes out[col][j].
__global__ __launch_bounds__(256) void grads_reduce_kernel(const float* __restrict__ part,
                                                           int nchunk, int r, int64_t C,
                                                           float s, bool transposed,
                                                           float* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(r) * C) return;
  const int64_t j = idx / C, col = idx % C;
  // 16 loads in flight per batch (clamped to the last chunk, not added),
  // then the additions in chunk order
  constexpr int kBatch = 16;
  float v = 0.f;
  for (int c0 = 0; c0 < nchunk; c0 += kBatch) {
    float pv[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c = c0 + i < nchunk ? c0 + i : nchunk - 1;
      pv[i] = part[(static_cast<int64_t>(c) * r + j) * C + col];
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (c0 + i < nchunk) v += pv[i];
  }
  v *= s;
  if (transposed) out[col * r + j] = v;
  else out[j * C + col] = v;
}

// Token chunks for C columns: about 256 workgroups, chunks a multiple of 32.
int64_t grads_chunk(int64_t M, int64_t C) {
  const int64_t nct = (C + kCols - 1) / kCols;
  int64_t nch = 256 / nct;
  if (nch < 1) nch = 1;
  int64_t chunk = (M + nch - 1) / nch;
  chunk = (chunk + kStep - 1) / kStep * kStep;
  return chunk < kStep ? kStep : chunk;
}

int64_t grads_nchunk(int64_t M, int64_t C) {
  if (M <= 0) return 0;
  const int64_t chunk = grads_chunk(M, C);
  return (M + chunk - 1) / chunk;
}

template <typename T>
hipError_t launch_partial(const uint16_t* X, int64_t M, int64_t C, const T* Pn, int r,
                          float* part, hipStream_t st) {
  const int64_t chunk = grads_chunk(M, C);
  const dim3 grid(static_cast<uint32_t>((C + kCols - 1) / kCols),
                  static_cast<uint32_t>((M + chunk - 1) / chunk));
  if (r <= 16) hipLaunchKernelGGL((grads_mfma_kernel<16, T>), grid, dim3(256), 0, st, X, M, C, Pn, r, chunk, part);
  else if (r <= 32) hipLaunchKernelGGL((grads_mfma_kernel<32, T>), grid, dim3(256), 0, st, X, M, C, Pn, r, chunk, part);
  else if (r <= 64) hipLaunchKernelGGL((grads_mfma_kernel<64, T>), grid, dim3(256), 0, st, X, M, C, Pn, r, chunk, part);
  else hipLaunchKernelGGL((grads_mfma_kernel<128, T>), grid, dim3(256), 0, st, X, M, C, Pn, r, chunk, part);
  return hipGetLastError();
}

}  // namespace

size_t grads_workspace_bytes(int64_t M, int64_t N, int64_t K, int r) {
  const int64_t elems = (grads_nchunk(M, K) * K + grads_nchunk(M, N) * N) * r;
  return static_cast<size_t>(elems) * 4;
}

hipError_t launch_grads_impl(const uint16_t* x, const uint16_t* dy, const void* u, bool u_bf16,
                             const void* t, bool t_bf16, int64_t M, int64_t N, int64_t K,
                             int r, float s, float* dA, float* dB, void* ws, hipStream_t st) {
  if (r == 0) return hipSuccess;
  const int nchA = static_cast<int>(grads_nchunk(M, K));
  const int nchB = static_cast<int>(grads_nchunk(M, N));
  float* partA = static_cast<float*>(ws);
  float* partB = partA + static_cast<int64_t>(nchA) * r * K;
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
                     st, partA, nchA, r, K, s, false, dA);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(grads_reduce_kernel, dim3(static_cast<uint32_t>((r * N + 255) / 256)), dim3(256), 0,
                     st, partB, nchB, r, N, s, true, dB);
  return hipGetLastError();
}

}  // namespace qn
