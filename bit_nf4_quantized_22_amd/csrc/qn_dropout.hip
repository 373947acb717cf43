// LoRA dropout on the adapter branch (gfx950).
//
// [rkmt "QLORA技术解析" §3.3] gives the LoRA layer a dropout rate (0.1;
// [czcl "QLoRA技術解析" §3.2] and [kwkr "QLoRA原理深入" §4] use 0.05).  The
// dropout acts on the adapter's input only:
//   y  = x W^T + s ((x * D) A^T) B^T,        D = keep / (1 - p)
//   dx = dy W + D * (s (dy B) A)
// and the LoRA gradients take the dropped input x * D.
//
// The keep mask is regenerated, never stored.  It comes from the counter-
// based generator Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC 2011):
// element (m, k) of a row-major [M, K] input uses the block at counter
// (k, m / 8, 0, 0) with key (seed, 0); row m % 8 takes the 32-bit half
// (m % 8) % 2 (low first) of 64-bit word (m % 8) / 2, and the element is kept
// iff that half >= floor(p 2^32).  One block thus serves eight rows of one
// column, and a thread that walks a column makes one block per eight rows.
//
// Two streaming kernels:
//   dropout_kernel   x -> bf16(x * fl32(1 / (1 - p))) or +0, 8 rows x 8
//                    columns per thread (16-byte loads and stores)
//   dx_lora_kernel   dx = bf16(dy W + D * (s t A)) from the fp32 product
//                    dy W (one rounding), one column per thread with A's
//                    column in registers and the rows of bf16(s t) in LDS;
//                    32 rows per workgroup

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

// the published Philox4x64 round multipliers and Weyl key increments
constexpr uint64_t kPhiloxMul0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxMul1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxWeyl0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxWeyl1 = 0xBB67AE8584CAA73Bull;

// Keep bits of the eight rows 8 g .. 8 g + 7 of column k: bit i is row 8 g + i.
__device__ __forceinline__ uint32_t keep_bits(uint64_t k, uint64_t g, uint64_t seed, uint32_t thr) {
  uint64_t x0 = k, x1 = g, x2 = 0, x3 = 0;
  uint64_t k0 = seed, k1 = 0;
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd) {
      k0 += kPhiloxWeyl0;
      k1 += kPhiloxWeyl1;
    }
    const uint64_t hi0 = __umul64hi(kPhiloxMul0, x0), lo0 = kPhiloxMul0 * x0;
    const uint64_t hi1 = __umul64hi(kPhiloxMul1, x2), lo1 = kPhiloxMul1 * x2;
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
  }
  const uint64_t w[4] = {x0, x1, x2, x3};
  uint32_t bits = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bits |= static_cast<uint32_t>(static_cast<uint32_t>(w[j]) >= thr) << (2 * j);
    bits |= static_cast<uint32_t>(static_cast<uint32_t>(w[j] >> 32) >= thr) << (2 * j + 1);
  }
  return bits;
}

__device__ __forceinline__ uint32_t drop_pair(uint32_t xv, bool keep_lo, bool keep_hi, float inv_keep) {
  const uint32_t lo = keep_lo ? (pack_bf16x2(__fmul_rn(bf16_lo(xv), inv_keep), 0.f) & 0xFFFFu) : 0u;
  const uint32_t hi = keep_hi ? (pack_bf16x2(0.f, __fmul_rn(bf16_hi(xv), inv_keep)) & 0xFFFF0000u) : 0u;
  return lo | hi;
}

// One thread: rows 8 g .. 8 g + 7 (g = row group) of columns 8 c .. 8 c + 7.
__global__ __launch_bounds__(256) void dropout_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                     int64_t K, uint64_t seed, uint32_t thr,
                                                     float inv_keep, uint16_t* __restrict__ out) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int64_t cgroups = K >> 3;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= cgroups) return;
  const int64_t col0 = c << 3;
  for (int64_t g = blockIdx.y; g < (M + 7) >> 3; g += gridDim.y) {
    const int64_t row0 = g << 3;
    const int rows = M - row0 < 8 ? static_cast<int>(M - row0) : 8;
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < rows) v[i] = *reinterpret_cast<const u32x4*>(x + (row0 + i) * K + col0);
    uint32_t bits[8];  // bits[j]: keep bits of column col0 + j, bit i = row row0 + i
#pragma unroll
    for (int j = 0; j < 8; ++j) bits[j] = keep_bits(static_cast<uint64_t>(col0 + j), g, seed, thr);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < rows) {
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = drop_pair(v[i][q], (bits[2 * q] >> i) & 1u, (bits[2 * q + 1] >> i) & 1u, inv_keep);
        *reinterpret_cast<u32x4*>(out + (row0 + i) * K + col0) = o;
      }
    }
  }
}

constexpr int kDxRows = 32;  // rows of dx per workgroup (four Philox blocks per column)

// dx[m, k] <- bf16(dx[m, k] + keep(m, k) * fl32(inv_keep * sum_j ts[m, j] A[j, k]))
// with ts = bf16(s t); the sum is an fp32 fma chain in j order.
template <int kR>
__global__ __launch_bounds__(256) void dx_lora_kernel(const float* __restrict__ base,
                                                      uint16_t* __restrict__ dx,
                                                      const uint16_t* __restrict__ ts,
                                                      const uint16_t* __restrict__ A, int64_t M,
                                                      int64_t K, int r, uint64_t seed,
                                                      uint32_t thr, float inv_keep) {
  constexpr bool kPacked = kR > 64;  // A's column as bf16 pairs above rank 64
  constexpr int kAR = kPacked ? kR / 2 : kR;
  __shared__ __attribute__((aligned(16))) float st[kDxRows][kR];
  const int tid = threadIdx.x;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kDxRows;
  for (int i = tid; i < kDxRows * kR; i += 256) {
    const int rr = i / kR, j = i % kR;
    const int64_t m = m0 + rr;
    const bool ok = m < M && j < r;
    const float v = bf16_to_f32(ts[(m < M ? m : M - 1) * r + (j < r ? j : r - 1)]);
    st[rr][j] = ok ? v : 0.f;
  }
  __syncthreads();
  const int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + tid;
  const bool kvalid = k < K;
  const int64_t kc = kvalid ? k : K - 1;
  uint32_t a[kAR];
#pragma unroll
  for (int i = 0; i < kAR; ++i) {
    if constexpr (kPacked) {
      const int j0 = 2 * i, j1 = 2 * i + 1;
      const uint32_t v0 = A[static_cast<int64_t>(j0 < r ? j0 : r - 1) * K + kc];
      const uint32_t v1 = A[static_cast<int64_t>(j1 < r ? j1 : r - 1) * K + kc];
      a[i] = (j0 < r ? v0 : 0u) | ((j1 < r ? v1 : 0u) << 16);
    } else {
      const uint32_t v = A[static_cast<int64_t>(i < r ? i : r - 1) * K + kc];
      a[i] = i < r ? (v << 16) : 0u;
    }
  }
  const int64_t mlast = (m0 + kDxRows < M ? m0 + kDxRows : M) - 1;
  for (int rb = 0; rb < kDxRows; rb += 8) {
    const int64_t g = (m0 + rb) >> 3;
    float d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = m0 + rb + i < mlast ? m0 + rb + i : mlast;
      d[i] = base[m * K + kc];
    }
    const uint32_t bits = keep_bits(static_cast<uint64_t>(kc), static_cast<uint64_t>(g), seed, thr);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = m0 + rb + i;
      const float* trow = st[rb + i];
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < kR; ++j) {
        float aj;
        if constexpr (kPacked)
          aj = __uint_as_float((j & 1) ? (a[j >> 1] & 0xFFFF0000u) : (a[j >> 1] << 16));
        else
          aj = __uint_as_float(a[j]);
        acc = __fmaf_rn(trow[j], aj, acc);
      }
      const float add = ((bits >> i) & 1u) ? __fmul_rn(inv_keep, acc) : 0.f;
      const float val = __fadd_rn(d[i], add);
      if (kvalid && m <= mlast) dx[m * K + k] = static_cast<uint16_t>(pack_bf16x2(val, 0.f) & 0xFFFF);
    }
  }
}

template <int kR>
void dx_lora_launch(const float* base, uint16_t* dx, const uint16_t* ts, const uint16_t* A,
                    int64_t M, int64_t K, int r, uint64_t seed, uint32_t thr, float inv_keep,
                    hipStream_t st) {
  const dim3 grid(static_cast<uint32_t>((K + 255) / 256),
                  static_cast<uint32_t>((M + kDxRows - 1) / kDxRows));
  hipLaunchKernelGGL((dx_lora_kernel<kR>), grid, dim3(256), 0, st, base, dx, ts, A, M, K, r, seed,
                     thr, inv_keep);
}

}  // namespace

DropoutParams dropout_params(float p) {
  DropoutParams d;
  d.threshold = static_cast<uint32_t>(static_cast<double>(p) * 4294967296.0);  // floor, p < 1
  d.inv_keep = static_cast<float>(1.0 / (1.0 - static_cast<double>(p)));
  return d;
}

hipError_t launch_dropout(const uint16_t* x, int64_t M, int64_t K, float p, uint64_t seed,
                          uint16_t* out, hipStream_t st) {
  if (M == 0 || K == 0) return hipSuccess;
  const DropoutParams d = dropout_params(p);
  const int64_t cgroups = K >> 3;
  const int64_t rgroups = (M + 7) >> 3;
  const dim3 grid(static_cast<uint32_t>((cgroups + 255) / 256),
                  static_cast<uint32_t>(rgroups < 65535 ? rgroups : 65535));
  hipLaunchKernelGGL(dropout_kernel, grid, dim3(256), 0, st, x, M, K, seed, d.threshold,
                     d.inv_keep, out);
  return hipGetLastError();
}

hipError_t launch_dx_lora_dropout(const float* base, uint16_t* dx, const uint16_t* ts,
                                  const uint16_t* A, int64_t M, int64_t K, int r, float p,
                                  uint64_t seed, hipStream_t st) {
  if (M == 0 || K == 0 || r == 0) return hipSuccess;
  const DropoutParams d = dropout_params(p);
  if (r <= 16) dx_lora_launch<16>(base, dx, ts, A, M, K, r, seed, d.threshold, d.inv_keep, st);
  else if (r <= 32) dx_lora_launch<32>(base, dx, ts, A, M, K, r, seed, d.threshold, d.inv_keep, st);
  else if (r <= 64) dx_lora_launch<64>(base, dx, ts, A, M, K, r, seed, d.threshold, d.inv_keep, st);
  else dx_lora_launch<128>(base, dx, ts, A, M, K, r, seed, d.threshold, d.inv_keep, st);
  return hipGetLastError();
}

}  // namespace qn
