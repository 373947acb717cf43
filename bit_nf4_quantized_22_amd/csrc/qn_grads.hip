// LoRA gradients (gfx950):  dA = s (dy B)^T x,  dB = s dy^T (x A^T).
//
// [kwkr "QLoRA原理深入" §2.3] gradients flow only into the LoRA bypass; the
// 4-bit weight and its constants get none, so this is all the backward
// produces besides dx.
//
// Both are out[r, C] = P^T X summed over the M tokens, with X the wide bf16
// matrix (x [M, K] or dy [M, N]) and P the narrow one (t or u, [M, r],
// bf16): a contraction along M, the slow dimension of both row-major
// inputs.  MFMA 16x16x32 needs each lane to hold 8 consecutive tokens of
// one column, so every 64-token step of X is loaded with coalesced 16-byte
// loads and written *transposed* into LDS as bf16 pairs (column-major
// [column][token], row pitch 72 halves so the operand reads are
// conflict-free); P is staged the same way.  Loads run two steps ahead
// (64 KB in flight per workgroup): with one or two workgroups per CU the
// bytes in flight set the streaming rate.  Workgroups own 256 columns and a
// token chunk, write fp32 partial sums [chunk][r][C], and a second pass
// sums the chunks in a fixed order and applies s (bit-reproducible).  Both
// products share each of the two launches.  The wide matrices are read
// once; the chunks are long enough that the partials stay a quarter of
// them or less.

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

constexpr int kCols = 256;    // columns of X per workgroup (4 waves x 64)
constexpr int kStep = 64;     // tokens per step (two 32-deep MFMA steps)
constexpr int kQ = kStep / 16;  // 16-token row groups per step
constexpr int kPitch = kStep + 8;  // LDS row pitch of the transposed tiles, in bf16

// The transposed X tile holds column c's 64 tokens as 8 chunks of 16 bytes;
// chunk h of row c sits in slot h ^ ((c >> 3) & 7).  A loader lane writes
// one 32-bit token pair into each of 8 rows that are 8 apart in one
// instruction: without the swizzle those rows share their banks (row pitch
// 36 words) and the stores serialise eight ways.
__device__ __forceinline__ int xslot(int row, int chunk) { return chunk ^ ((row >> 3) & 7); }

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// One of the two products: X [M, C] bf16 (x or dy), P [M, r] bf16 (t or
// u), partial sums part[chunk][r][C] over token chunks of `chunk` rows.
struct GradJob {
  const uint16_t* X;
  const uint16_t* P;
  float* part;
  int64_t C, chunk;
  int ncol;  // 256-column tiles
  int nwg;   // workgroups: ncol x chunks
};

// RT: rank tile (r <= RT, a multiple of 16).  1-D grid: the workgroups of
// job a, then those of job b (dA and dB in one launch); inside a job the
// column tile runs fastest.  Thread t loads, per step, rows 2 (t % 8) +
// {0, 1} + 16 q (q < kQ) of columns 8 (t / 8) .. + 7: 2 kQ 16-byte loads,
// 8 rows x 128 bytes per wave instruction.  Each pair of rows is packed
// per column into one 32-bit word and stored at [column][row pair] of the
// transposed tile.  kDepth register sets of loads are in flight: step s + 2
// is loaded while step s is computed (one set for RT = 128, whose
// accumulators leave no room for two).  Steps past the chunk read clamped
// rows and a zero P, so the loop runs in pairs without branches.
template <int RT>
__global__ __launch_bounds__(256) void grads_mfma_kernel(const GradJob ja, const GradJob jb,
                                                         int64_t M, int r) {
  constexpr int kPer = (kStep * RT + 255) / 256;  // P elements per thread per step
  constexpr int kDepth = RT <= 64 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint16_t sX[kCols * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sP[RT * kPitch];

  const bool second = static_cast<int>(blockIdx.x) >= ja.nwg;  // uniform
  const uint16_t* X = second ? jb.X : ja.X;
  const uint16_t* P = second ? jb.P : ja.P;
  float* part = second ? jb.part : ja.part;
  const int64_t C = second ? jb.C : ja.C;
  const int64_t chunk = second ? jb.chunk : ja.chunk;
  const int ncol = second ? jb.ncol : ja.ncol;
  const int bid = static_cast<int>(blockIdx.x) - (second ? ja.nwg : 0);
  const int ct = bid % ncol, ch = bid / ncol;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t c0 = static_cast<int64_t>(ct) * kCols;
  const int64_t m_lo = static_cast<int64_t>(ch) * chunk;
  const int64_t m_hi = m_lo + chunk < M ? m_lo + chunk : M;
  const int nsteps = static_cast<int>((m_hi - m_lo + kStep - 1) / kStep);

  // loader roles
  const int lcg = tid >> 3;         // column group: columns 8 lcg .. + 7
  const int lrp = tid & 7;          // row pair within 16 rows
  const int64_t lcol = c0 + 8 * lcg;
  const int64_t lcolc = lcol + 8 <= C ? lcol : C - 8;  // C % 64 == 0: a valid 8-column group
  auto load_step = [&](int s, uint4 (&v)[2 * kQ], uint32_t (&pv)[kPer]) {
#pragma unroll
    for (int q = 0; q < kQ; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int64_t m = m_lo + static_cast<int64_t>(s) * kStep + 16 * q + 2 * lrp + h;
        m = m < m_hi ? m : m_hi - 1;  // rows past the chunk: valid data, P zeroed
        v[2 * q + h] = *reinterpret_cast<const uint4*>(X + m * C + lcolc);
      }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + 256 * i;
      const int mm = idx / RT, j = idx % RT;
      const int64_t m = m_lo + static_cast<int64_t>(s) * kStep + mm;
      const bool ok = idx < kStep * RT && j < r && m < m_hi;
      const uint32_t val = P[(ok ? m : m_lo) * r + (ok ? j : 0)];
      pv[i] = ok ? val : 0u;
    }
  };

  f32x4_t acc[RT / 16][4];
#pragma unroll
  for (int a = 0; a < RT / 16; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int l16 = lane & 15, g = lane >> 4;
  // Step s: its loads (issued kDepth steps earlier) into the transposed LDS
  // tiles, the loads of step s + kDepth into the same registers, then the
  // MFMAs of step s.
  auto step = [&](int s, uint4 (&xv)[2 * kQ], uint32_t (&pv)[kPer]) {
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
        const int row = 8 * lcg + e, tok = 16 * q + 2 * lrp;  // tok: first of the pair
        *reinterpret_cast<uint32_t*>(&sX[row * kPitch + 8 * xslot(row, tok >> 3) + (tok & 7)]) =
            lo | hi;
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + 256 * i;
      if (idx < kStep * RT) {
        const int mm = idx / RT, j = idx % RT;
        sP[j * kPitch + mm] = static_cast<uint16_t>(pv[i]);
      }
    }
    __syncthreads();
    load_step(s + kDepth, xv, pv);
#pragma unroll
    for (int kk = 0; kk < kStep / 32; ++kk) {
      uint4 pa[RT / 16];
#pragma unroll
      for (int a = 0; a < RT / 16; ++a)
        pa[a] = *reinterpret_cast<const uint4*>(&sP[(16 * a + l16) * kPitch + 32 * kk + 8 * g]);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int xrow = wave * 64 + 16 * b + l16;
        const uint4 xb = *reinterpret_cast<const uint4*>(
            &sX[xrow * kPitch + 8 * xslot(xrow, 4 * kk + g)]);
#pragma unroll
        for (int a = 0; a < RT / 16; ++a) acc[a][b] = mfma16(pa[a], xb, acc[a][b]);
      }
    }
  };
  uint4 xv0[2 * kQ];
  uint32_t pv0[kPer];
  load_step(0, xv0, pv0);
  if constexpr (kDepth == 2) {
    uint4 xv1[2 * kQ];
    uint32_t pv1[kPer];
    load_step(1, xv1, pv1);
    for (int s = 0; s < nsteps; s += 2) {
      step(s, xv0, pv0);
      step(s + 1, xv1, pv1);  // past the chunk when nsteps is odd: adds zeros
    }
  } else {
    for (int s = 0; s < nsteps; ++s) step(s, xv0, pv0);
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
          part[(static_cast<int64_t>(ch) * r + j) * C + col] = acc[a][b][v];
      }
    }
}

// dA[j][k] = s * sum over chunks of partA, then dB[n][j] (transposed) from
// partB, in one launch; each element's chunks are added in a fixed order.
__global__ __launch_bounds__(256) void grads_reduce_kernel(const float* __restrict__ partA,
                                                           int nchA, int64_t K,
                                                           float* __restrict__ dA,
                                                           const float* __restrict__ partB,
                                                           int nchB, int64_t N,
                                                           float* __restrict__ dB, int r,
                                                           float s) {
  int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nA = static_cast<int64_t>(r) * K;
  const bool second = idx >= nA;
  if (second) idx -= nA;
  const int64_t C = second ? N : K;
  if (idx >= static_cast<int64_t>(r) * C) return;
  const float* part = second ? partB : partA;
  const int nchunk = second ? nchB : nchA;
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
  if (second) dB[col * r + j] = v;
  else dA[j * C + col] = v;
}

// Token chunks for C columns: about 256 workgroups, chunks a multiple of
// 64, and at least 8 max(r, 16) tokens each, so that the fp32 partial sums
// (chunks x r x C x 4 bytes, written and read back) stay within a quarter
// of the bf16 input (M x C x 2 bytes).  At M = 2048, r = 64 the 16 chunks
// of a 4096-column product had made the partials as large as the input
// (44.8 against 40.4 us per call at 4096 x 4096).
int64_t grads_chunk(int64_t M, int64_t C, int r) {
  const int64_t nct = (C + kCols - 1) / kCols;
  int64_t nch = 256 / nct;
  const int64_t cap = M / (8 * (r > 16 ? r : 16));
  if (nch > cap) nch = cap;
  if (nch < 1) nch = 1;
  int64_t chunk = (M + nch - 1) / nch;
  chunk = (chunk + kStep - 1) / kStep * kStep;
  return chunk < kStep ? kStep : chunk;
}

int64_t grads_nchunk(int64_t M, int64_t C, int r) {
  if (M <= 0) return 0;
  const int64_t chunk = grads_chunk(M, C, r);
  return (M + chunk - 1) / chunk;
}

GradJob grad_job(const uint16_t* X, const uint16_t* P, int64_t M, int64_t C, float* part, int r) {
  GradJob j;
  j.X = X;
  j.P = P;
  j.part = part;
  j.C = C;
  j.chunk = grads_chunk(M, C, r);
  j.ncol = static_cast<int>((C + kCols - 1) / kCols);
  j.nwg = j.ncol * static_cast<int>(grads_nchunk(M, C, r));
  return j;
}

}  // namespace

size_t grads_workspace_bytes(int64_t M, int64_t N, int64_t K, int r) {
  const int64_t elems = (grads_nchunk(M, K, r) * K + grads_nchunk(M, N, r) * N) * r;
  return static_cast<size_t>(elems) * 4;
}

hipError_t launch_grads_impl(const uint16_t* x, const uint16_t* dy, const uint16_t* u,
                             const uint16_t* t, int64_t M, int64_t N, int64_t K, int r, float s,
                             float* dA, float* dB, void* ws, hipStream_t st) {
  if (r == 0) return hipSuccess;
  const int nchA = static_cast<int>(grads_nchunk(M, K, r));
  const int nchB = static_cast<int>(grads_nchunk(M, N, r));
  float* partA = static_cast<float*>(ws);
  float* partB = partA + static_cast<int64_t>(nchA) * r * K;
  if (M > 0) {
    const GradJob ja = grad_job(x, t, M, K, partA, r), jb = grad_job(dy, u, M, N, partB, r);
    const dim3 grid(static_cast<uint32_t>(ja.nwg + jb.nwg));
    if (r <= 16) hipLaunchKernelGGL((grads_mfma_kernel<16>), grid, dim3(256), 0, st, ja, jb, M, r);
    else if (r <= 32) hipLaunchKernelGGL((grads_mfma_kernel<32>), grid, dim3(256), 0, st, ja, jb, M, r);
    else if (r <= 64) hipLaunchKernelGGL((grads_mfma_kernel<64>), grid, dim3(256), 0, st, ja, jb, M, r);
    else hipLaunchKernelGGL((grads_mfma_kernel<128>), grid, dim3(256), 0, st, ja, jb, M, r);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n = static_cast<int64_t>(r) * (K + N);
  hipLaunchKernelGGL(grads_reduce_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0,
                     st, partA, nchA, K, dA, partB, nchB, N, dB, r, s);
  return hipGetLastError();
}

}  // namespace qn
