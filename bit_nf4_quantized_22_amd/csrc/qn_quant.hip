// Blockwise NF4 quantisation, double quantisation of the block constants,
// and dequantisation (gfx950).
//
// [rkmt "QLORA技术解析" §2.2.1-2.2.2] blocks of 64 weights, one fp32 constant
// per block, nearest NF4 code per weight; second quantisation of the
// constants to 8 bits.  [kwkr "QLoRA原理深入" §2.3, §3.1] 4-bit storage,
// dequantised for compute; block size 64; 8-bit constants.
//
// All kernels here are HBM-streaming: one pass over the input, one write
// of the output, no re-reads.

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

constexpr int kQThreads = 256;     // 4 waves
constexpr int kQPerThread = 16;    // 16 weights per lane, 4 lanes per block of 64
constexpr int kQPerGroup = kQThreads * kQPerThread;  // 4096 weights per workgroup
constexpr float kDanger = 0x1p-20f;  // see the fast path below
constexpr float kTiny = 0x1p-100f;

template <bool kBf16>
__device__ __forceinline__ void load16(const void* __restrict__ w, int64_t e0, int64_t numel,
                                       float x[16]) {
  if (e0 + 16 <= numel) {
    if constexpr (kBf16) {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w) + e0);
      uint4 a = p[0], b = p[1];
      uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[2 * i] = bf16_lo(v[i]);
        x[2 * i + 1] = bf16_hi(v[i]);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(w) + e0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 f = p[i];
        x[4 * i] = f.x;
        x[4 * i + 1] = f.y;
        x[4 * i + 2] = f.z;
        x[4 * i + 3] = f.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int64_t e = e0 + i;
      float v = 0.0f;
      if (e < numel) {
        if constexpr (kBf16) v = bf16_to_f32(static_cast<const uint16_t*>(w)[e]);
        else v = static_cast<const float*>(w)[e];
      }
      x[i] = v;
    }
  }
}

// Code of v: base + (v > thr) of v's bucket.  Exact for any fp32 v in
// [-1, 1] because each bucket holds at most one threshold and the bucket
// function is monotone (the host built the table with the same function).
__device__ __forceinline__ uint32_t bucket_code(const QuantBucket* sbk, float v, float sc,
                                                float top, float& thr) {
  // median of (v sc + sc, 0, top): the clamp min(max(., 0), top) in one
  // instruction (a NaN, which the clamp maps to 0, converts to bucket 0 too)
  float f = __builtin_amdgcn_fmed3f(fmaf(v, sc, sc), 0.0f, top);
  QuantBucket e = sbk[static_cast<uint32_t>(f)];
  thr = e.thr;
  return e.base + (v > e.thr ? 1u : 0u);
}

// Bucket table: bucket b holds the threshold whose bucket is b (if any)
// and counts the thresholds in lower buckets (same bucket function as
// bucket_code; the host checked that buckets hold at most one threshold
// with a margin).
__device__ __forceinline__ void fill_buckets(QuantBucket* sbk, const QuantParams& P, int nthreads) {
  const float sc = P.scale;
  const float top = static_cast<float>(P.nbuckets - 1);
  for (uint32_t b = threadIdx.x; b < P.nbuckets; b += nthreads) {
    uint32_t base = 0;
    float thr = INFINITY;
#pragma unroll
    for (int i = 0; i < 15; ++i) {
      const float ti = P.thr[i];
      const uint32_t bi = static_cast<uint32_t>(fminf(fmaxf(fmaf(ti, sc, sc), 0.0f), top));
      base += bi < b ? 1u : 0u;
      thr = bi == b ? ti : thr;
    }
    sbk[b] = QuantBucket{thr, base};
  }
}

// Each lane owns 16 consecutive weights from e0; the 4 lanes of a
// 64-weight block reduce their absmax with two cross-lane steps.  Code of
// a weight:
//   fast path  q = w * rcp(c) (|q - fl32(w/c)| <= 2^-22 for |w| <= c,
//              c >= 2^-100); the bucket lookup on q gives the code of q.
//              It equals the code of fl32(w/c) unless a threshold lies
//              within 2^-22 of q.  Thresholds sit >= 2^-19 inside their
//              bucket (host-checked), so only the bucket's own threshold
//              can; a lane whose q comes within 2^-20 of it ("danger"),
//              or whose block constant is below 2^-100, redoes its 16
//              weights on the exact path.
//   exact path q = fl32(w / c) by IEEE division, then the same lookup
//              (q = w for an all-zero block: the code of v = 0).
// Writes the 8 packed bytes (numel is even) and returns the block constant.
__device__ __forceinline__ float quantize16_loaded(const QuantBucket* sbk, const QuantParams& P,
                                                   const float (&x)[16], int64_t e0,
                                                   int64_t numel, uint8_t* __restrict__ packed) {
  const float sc = P.scale;
  const float top = static_cast<float>(P.nbuckets - 1);

  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(x[i]));
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  const float c = m;

  const float rc = c > 0.0f ? __builtin_amdgcn_rcpf(c) : 0.0f;
  bool danger = (c > 0.0f) && (c < kTiny);
  uint32_t code[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float thr;
    const float q = x[i] * rc;
    code[i] = bucket_code(sbk, q, sc, top, thr);
    danger |= fabsf(q - thr) <= kDanger;
  }
  if (danger) {
    // an all-zero block (c = 0) takes the code of v = 0, as in the fast
    // path: with a threshold at 0 (FP4's two zeros) it lands here, and 0 / 0
    // would be NaN
    const float cd = c > 0.0f ? c : 1.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float thr;
      code[i] = bucket_code(sbk, x[i] / cd, sc, top, thr);
    }
  }

  if (e0 < numel) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= ((code[2 * i] << 4) | code[2 * i + 1]) << (8 * i);
      hi |= ((code[8 + 2 * i] << 4) | code[8 + 2 * i + 1]) << (8 * i);
    }
    uint8_t* dst = packed + e0 / 2;
    if (e0 + 16 <= numel) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
    } else {
      const int64_t nbytes = (numel - e0) / 2;  // numel is even
      for (int64_t b = 0; b < nbytes; ++b)
        dst[b] = static_cast<uint8_t>(((b < 4 ? lo : hi) >> (8 * (b & 3))) & 0xFF);
    }
  }
  return c;
}

template <bool kBf16>
__device__ __forceinline__ float quantize16(const QuantBucket* sbk, const QuantParams& P,
                                            const void* __restrict__ w, int64_t e0, int64_t numel,
                                            uint8_t* __restrict__ packed) {
  float x[16];
  load16<kBf16>(w, e0, numel, x);
  return quantize16_loaded(sbk, P, x, e0, numel, packed);
}

template <bool kBf16>
__global__ __launch_bounds__(kQThreads) void nf4_quantize_kernel(
    const void* __restrict__ w, int64_t numel, uint8_t* __restrict__ packed,
    float* __restrict__ absmax, QuantParams P) {
  __shared__ QuantBucket sbk[kMaxBuckets];
  fill_buckets(sbk, P, kQThreads);
  __syncthreads();
  const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * kQThreads + threadIdx.x) * kQPerThread;
  const float c = quantize16<kBf16>(sbk, P, w, e0, numel, packed);
  if (e0 < numel && (threadIdx.x & 3) == 0) absmax[e0 / 64] = c;
}

// Decision thresholds of the 8-bit grid, one per thread j < 256: the
// largest fp32 <= the fp64 mid-point of adjacent levels fl32(j / 255)
// (exact in fp64); +inf last.
__device__ __forceinline__ void fill_l8_thresholds(float* sthr, int j) {
  float thr = INFINITY;
  if (j < 255) {
    const double m = (static_cast<double>(l8_value(j)) + static_cast<double>(l8_value(j + 1))) * 0.5;
    thr = static_cast<float>(m);
    if (static_cast<double>(thr) > m) thr = nextafterf(thr, -INFINITY);
  }
  sthr[j] = thr;
}

// Level-2 code of a block constant c in a group with maximum c2: v =
// fl32(c / c2), the nearest level of the uint8 grid fl32(q / 255), or (kFP8)
// the nearest E4M3 number ([kwkr] §3.1 names fp8 for the constants).
template <bool kFP8>
__device__ __forceinline__ uint8_t dq_code(float c, float c2, const float* sthr) {
  int q = 0;
  if (c2 > 0.0f) {
    const float v = c / c2;  // IEEE division
    if constexpr (kFP8) {
      q = static_cast<int>(e4m3_code(v));
    } else {
      q = static_cast<int>(fminf(fmaxf(fmaf(v, 255.0f, 0.5f), 0.0f), 255.0f));
      while (q < 255 && v > sthr[q]) ++q;
      while (q > 0 && !(v > sthr[q - 1])) --q;
    }
  }
  return static_cast<uint8_t>(q);
}

// Quantisation and double quantisation in one launch: a workgroup takes
// one group of 256 blocks (16384 weights: 4 x 16 per lane; for bf16 all 64
// are loaded before the first is quantised, 128 bytes per lane in flight),
// keeps the group's block constants in LDS and ends with their level-2
// codes and the group maximum: the same values as nf4_quantize_kernel
// followed by dq_quantize_kernel.  The block constants themselves are
// written too when absmax is not null.
constexpr int kQDPasses = 4;

// LDS of one group's quantise + double-quantise.
struct QdqShared {
  QuantBucket sbk[kMaxBuckets];
  float sthr[256];
  float sconst[256];
  float smax[4];
};

// Group `grp` (256 blocks of 64 weights) of one weight: its 4-bit codes,
// block constants, their 8-bit codes and the group constant.
template <bool kBf16, bool kFP8>
__device__ __forceinline__ void quantize_dq_group(QdqShared& sh, const void* __restrict__ w,
                                                  int64_t numel, uint8_t* __restrict__ packed,
                                                  float* __restrict__ absmax,
                                                  uint8_t* __restrict__ qscale,
                                                  float* __restrict__ gscale,
                                                  const QuantParams& P, int64_t grp) {
  static_assert(kQDPasses * kQPerGroup == 256 * 64, "one workgroup per 256-block group");
  QuantBucket* sbk = sh.sbk;
  float* sthr = sh.sthr;
  float* sconst = sh.sconst;
  float* smax = sh.smax;
  const int64_t g0 = grp * (kQDPasses * kQPerGroup);
  const bool full = g0 + kQDPasses * kQPerGroup <= numel;  // uniform
  // whole groups of bf16 weights: the raw 16-byte words of all passes are
  // loaded first (32 registers) and widened pass by pass
  uint4 raw[kBf16 ? kQDPasses : 1][2];
  if (kBf16 && full) {
#pragma unroll
    for (int s = 0; s < (kBf16 ? kQDPasses : 1); ++s) {
      const uint4* p = reinterpret_cast<const uint4*>(
          static_cast<const uint16_t*>(w) + g0 +
          (static_cast<int64_t>(s) * kQThreads + threadIdx.x) * kQPerThread);
      raw[s][0] = p[0];
      raw[s][1] = p[1];
    }
  }
  fill_buckets(sbk, P, kQThreads);
  if constexpr (!kFP8) fill_l8_thresholds(sthr, threadIdx.x);
  __syncthreads();
  float cmax = 0.0f;
#pragma unroll
  for (int s = 0; s < kQDPasses; ++s) {
    const int64_t e0 = g0 + (static_cast<int64_t>(s) * kQThreads + threadIdx.x) * kQPerThread;
    float x[16];
    if (kBf16 && full) {
      const uint4 a = raw[kBf16 ? s : 0][0], b = raw[kBf16 ? s : 0][1];
      const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[2 * i] = bf16_lo(v[i]);
        x[2 * i + 1] = bf16_hi(v[i]);
      }
    } else {
      load16<kBf16>(w, e0, numel, x);
    }
    const float c = quantize16_loaded(sbk, P, x, e0, numel, packed);  // 0 past numel
    if ((threadIdx.x & 3) == 0) {
      sconst[s * (kQThreads / 4) + threadIdx.x / 4] = c;
      if (absmax && e0 < numel) absmax[e0 / 64] = c;
    }
    cmax = fmaxf(cmax, c);
  }
  const float wm = wave_max(cmax);
  if ((threadIdx.x & 63) == 0) smax[threadIdx.x >> 6] = wm;
  __syncthreads();
  const float c2 = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
  const int64_t nblocks = (numel + 63) / 64;
  const int64_t bi = grp * 256 + threadIdx.x;
  if (threadIdx.x == 0) gscale[grp] = c2;
  if (bi < nblocks) qscale[bi] = dq_code<kFP8>(sconst[threadIdx.x], c2, sthr);
}

template <bool kBf16, bool kFP8>
__global__ __launch_bounds__(kQThreads) void quantize_dq_kernel(
    const void* __restrict__ w, int64_t numel, uint8_t* __restrict__ packed,
    float* __restrict__ absmax, uint8_t* __restrict__ qscale, float* __restrict__ gscale,
    QuantParams P) {
  __shared__ QdqShared sh;
  quantize_dq_group<kBf16, kFP8>(sh, w, numel, packed, absmax, qscale, gscale, P, blockIdx.x);
}

// Several weights in one launch: workgroup b serves entry j, the first with
// b < gend[j], at group b - gend[j - 1] (j and the entry's fields are
// uniform, read from the kernel arguments with scalar loads).
template <bool kBf16, bool kFP8>
__global__ __launch_bounds__(kQThreads) void quantize_dq_batch_kernel(QdqBatch B, QuantParams P) {
  __shared__ QdqShared sh;
  const uint32_t b = blockIdx.x;
  int j = 0;
  while (j + 1 < B.n && b >= B.gend[j]) ++j;
  j = __builtin_amdgcn_readfirstlane(j);
  const uint32_t g = b - (j > 0 ? B.gend[j - 1] : 0u);
  quantize_dq_group<kBf16, kFP8>(sh, B.w[j], B.numel[j], B.packed[j], B.absmax[j], B.qscale[j],
                                 B.gscale[j], P, g);
}

// One workgroup of 256 lanes per group of 256 block constants.
template <bool kFP8>
__global__ __launch_bounds__(256) void dq_quantize_kernel(const float* __restrict__ absmax,
                                                          int64_t nblocks,
                                                          uint8_t* __restrict__ qscale,
                                                          float* __restrict__ gscale) {
  __shared__ float sthr[256];
  __shared__ float smax[4];
  fill_l8_thresholds(sthr, threadIdx.x);
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const float c = i < nblocks ? absmax[i] : 0.0f;
  const float wm = wave_max(c);
  if ((threadIdx.x & 63) == 0) smax[threadIdx.x >> 6] = wm;
  __syncthreads();
  const float c2 = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
  if (threadIdx.x == 0) gscale[blockIdx.x] = c2;
  if (i < nblocks) qscale[i] = dq_code<kFP8>(c, c2, sthr);
}

// ---- mean-centred level-2 code ----------------------------------------
// The offset mu is the mean of the block constants, summed in fp64 by
// adjacent pairs (the constants zero-padded to a power of two, added 0+1,
// 2+3, ..., then the partial sums likewise), so its value does not depend
// on the launch shape.  A workgroup sums 4096 consecutive values: each lane
// 16 as a balanced tree in registers, then the 256 lane sums pair up in LDS.
// 4096-aligned chunks are subtrees of the whole tree, so partial sums of
// partial sums give the same result.

__device__ __forceinline__ double tree_input(const float* p, int64_t i) {
  return static_cast<double>(p[i]);
}
// fp64 partial sums are kept as pairs of 32-bit words (the scratch area is
// only 4-byte aligned)
__device__ __forceinline__ double tree_input(const uint32_t* p, int64_t i) {
  const uint64_t b = static_cast<uint64_t>(p[2 * i]) | (static_cast<uint64_t>(p[2 * i + 1]) << 32);
  return __longlong_as_double(static_cast<long long>(b));
}

constexpr int kTreeChunk = 4096;

// kFinal: one workgroup, n <= 4096, writes mu = fl32(sum / count);
// otherwise workgroup b writes the sum of chunk b to part[2b], part[2b + 1].
template <typename T, bool kFinal>
__global__ __launch_bounds__(256) void mean_tree_kernel(const T* __restrict__ in, int64_t n,
                                                        uint32_t* __restrict__ part,
                                                        int64_t count, float* __restrict__ mu) {
  __shared__ double sp[256];
  const int t = threadIdx.x;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kTreeChunk + t * 16;
  double v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = base + i < n ? tree_input(in, base + i) : 0.0;
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1) {
#pragma unroll
    for (int i = 0; i < w; ++i) v[i] = __dadd_rn(v[2 * i], v[2 * i + 1]);
  }
  sp[t] = v[0];
  __syncthreads();
  for (int st = 1; st < 256; st *= 2) {
    if ((t & (2 * st - 1)) == 0) sp[t] = __dadd_rn(sp[t], sp[t + st]);
    __syncthreads();
  }
  if (t == 0) {
    if constexpr (kFinal) {
      *mu = __double2float_rn(__ddiv_rn(sp[0], static_cast<double>(count)));
    } else {
      const uint64_t b = static_cast<uint64_t>(__double_as_longlong(sp[0]));
      part[2 * static_cast<int64_t>(blockIdx.x)] = static_cast<uint32_t>(b);
      part[2 * static_cast<int64_t>(blockIdx.x) + 1] = static_cast<uint32_t>(b >> 32);
    }
  }
}

// Largest fp32 not above the fp64 mid-point of the signed-grid levels j / 127
// and (j + 1) / 127, j = 0..126 (the mid-point is exact in fp64); +inf last.
__device__ __forceinline__ void fill_s8_thresholds(float* sthr, int j) {
  float thr = INFINITY;
  if (j < 127) {
    const double m =
        (static_cast<double>(s8_value(j)) + static_cast<double>(s8_value(j + 1))) * 0.5;
    thr = static_cast<float>(m);
    if (static_cast<double>(thr) > m) thr = nextafterf(thr, -INFINITY);
  }
  sthr[j] = thr;
}

// Code of a centred constant d in a group with c2 = max |d|: t = fl32(d / c2),
// the level j / 127 nearest to |t| (ties toward 0), signed like t, as a
// two's-complement byte.
__device__ __forceinline__ uint8_t s8_code(float d, float c2, const float* sthr) {
  if (!(c2 > 0.0f)) return 0;
  const float t = d / c2;  // IEEE division
  const float a = fabsf(t);
  int j = static_cast<int>(fminf(fmaxf(fmaf(a, 127.0f, 0.5f), 0.0f), 127.0f));
  while (j < 127 && a > sthr[j]) ++j;
  while (j > 0 && !(a > sthr[j - 1])) --j;
  return static_cast<uint8_t>((t < 0.0f ? -j : j) & 0xFF);
}

// One workgroup of 256 lanes per group of 256 block constants.
__global__ __launch_bounds__(256) void dq_centred_kernel(const float* __restrict__ absmax,
                                                         int64_t nblocks,
                                                         const float* __restrict__ mu,
                                                         uint8_t* __restrict__ qscale,
                                                         float* __restrict__ gscale) {
  __shared__ float sthr[128];
  __shared__ float smax[4];
  if (threadIdx.x < 128) fill_s8_thresholds(sthr, threadIdx.x);
  const float off = *mu;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const float d = i < nblocks ? __fsub_rn(absmax[i], off) : 0.0f;
  const float wm = wave_max(fabsf(d));
  if ((threadIdx.x & 63) == 0) smax[threadIdx.x >> 6] = wm;
  __syncthreads();
  const float c2 = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
  if (threadIdx.x == 0) gscale[blockIdx.x] = c2;
  if (i < nblocks) qscale[i] = s8_code(d, c2, sthr);
}

// Each thread expands 32 codes: four runs of 8 (4 packed bytes, one block
// constant each), 2048 codes apart.
template <bool kOutBf16>
__global__ __launch_bounds__(256) void nf4_dequant_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ gscale, const float* __restrict__ absmax, int64_t numel,
    void* __restrict__ out, CodeParams P) {
  __shared__ float2 spair[256];
  fill_pair_f32(spair, P, 1);
  const float mu = l2_offset(P);
  __syncthreads();
  // Run i of thread t: codes wbase + 2048 i .. + 7, so every load and
  // store instruction of a wave covers one contiguous range (256 bytes of
  // codes, 1 KB of bf16 or 2 KB of fp32).  Lane-strided 16-byte stores (a
  // lane's 32 codes contiguous) streamed at 3.5 TB/s; this order at 5.7.
  // Runs past numel (a multiple of 32) re-read the last run and store
  // nothing.
  const int64_t wbase = static_cast<int64_t>(blockIdx.x) * 8192 + threadIdx.x * 8;
  int64_t e[4];
  uint32_t words[4];
  float cs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t ei = wbase + i * 2048;
    e[i] = ei < numel ? ei : numel - 8;
    words[i] = *reinterpret_cast<const uint32_t*>(packed + e[i] / 2);
    cs[i] = block_scale(qscale, gscale, absmax, e[i] >> 6, P.l2, mu);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[8];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float2 pr = spair[(words[i] >> (8 * b)) & 0xFF];
      v[2 * b] = __fmul_rn(pr.x, cs[i]);
      v[2 * b + 1] = __fmul_rn(pr.y, cs[i]);
    }
    if (wbase + i * 2048 < numel) {
      if constexpr (kOutBf16) {
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + e[i]) =
            make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7]));
      } else {
        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + e[i]);
        dst[0] = make_float4(v[0], v[1], v[2], v[3]);
        dst[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
}

}  // namespace

CodeParams code_params(const WeightView& w) {
  const Tables* t = tables(w.quant_type);
  CodeParams P;
  for (int i = 0; i < 16; ++i) P.q[i] = t->q32[i];
  P.l2 = w.l2;
  P.mu = w.l2 == kL2Centred ? w.mu : nullptr;
  return P;
}

hipError_t launch_quantize(const void* w, bool bf16, int64_t numel, int quant_type,
                           uint8_t* packed, float* absmax, hipStream_t s) {
  if (numel == 0) return hipSuccess;
  const Tables* t = tables(quant_type);
  QuantParams P;
  P.scale = t->bucket_scale;
  P.nbuckets = static_cast<uint32_t>(t->nbuckets);
  for (int i = 0; i < 15; ++i) P.thr[i] = t->thr[i];
  const int64_t groups = (numel + kQPerGroup - 1) / kQPerGroup;
  if (bf16)
    hipLaunchKernelGGL(nf4_quantize_kernel<true>, dim3(static_cast<uint32_t>(groups)),
                       dim3(kQThreads), 0, s, w, numel, packed, absmax, P);
  else
    hipLaunchKernelGGL(nf4_quantize_kernel<false>, dim3(static_cast<uint32_t>(groups)),
                       dim3(kQThreads), 0, s, w, numel, packed, absmax, P);
  return hipGetLastError();
}

hipError_t launch_quantize_dq(const void* w, bool bf16, int64_t numel, int quant_type, bool fp8,
                              uint8_t* packed, float* absmax, uint8_t* qscale, float* gscale,
                              hipStream_t s) {
  if (numel == 0) return hipSuccess;
  const Tables* t = tables(quant_type);
  QuantParams P;
  P.scale = t->bucket_scale;
  P.nbuckets = static_cast<uint32_t>(t->nbuckets);
  for (int i = 0; i < 15; ++i) P.thr[i] = t->thr[i];
  const int64_t per = static_cast<int64_t>(kQDPasses) * kQPerGroup;
  const dim3 grid(static_cast<uint32_t>((numel + per - 1) / per));
#define QN_QDQ(B, F)                                                                            \
  if (bf16 == B && fp8 == F)                                                                   \
    hipLaunchKernelGGL((quantize_dq_kernel<B, F>), grid, dim3(kQThreads), 0, s, w, numel, packed, \
                       absmax, qscale, gscale, P);
  QN_QDQ(true, false) QN_QDQ(true, true) QN_QDQ(false, false) QN_QDQ(false, true)
#undef QN_QDQ
  return hipGetLastError();
}

hipError_t launch_quantize_dq_batch(const QdqBatch& batch, bool bf16, int quant_type, bool fp8,
                                    hipStream_t s) {
  const uint32_t groups = batch.n > 0 ? batch.gend[batch.n - 1] : 0u;
  if (groups == 0) return hipSuccess;
  const Tables* t = tables(quant_type);
  QuantParams P;
  P.scale = t->bucket_scale;
  P.nbuckets = static_cast<uint32_t>(t->nbuckets);
  for (int i = 0; i < 15; ++i) P.thr[i] = t->thr[i];
#define QN_QDQB(B, F)                                                                          \
  if (bf16 == B && fp8 == F)                                                                   \
    hipLaunchKernelGGL((quantize_dq_batch_kernel<B, F>), dim3(groups), dim3(kQThreads), 0, s,  \
                       batch, P);
  QN_QDQB(true, false) QN_QDQB(true, true) QN_QDQB(false, false) QN_QDQB(false, true)
#undef QN_QDQB
  return hipGetLastError();
}

hipError_t launch_dq(const float* absmax, int64_t nblocks, bool fp8, uint8_t* qscale,
                     float* gscale, hipStream_t s) {
  if (nblocks == 0) return hipSuccess;
  const int64_t groups = (nblocks + 255) / 256;
  if (fp8)
    hipLaunchKernelGGL(dq_quantize_kernel<true>, dim3(static_cast<uint32_t>(groups)), dim3(256), 0,
                       s, absmax, nblocks, qscale, gscale);
  else
    hipLaunchKernelGGL(dq_quantize_kernel<false>, dim3(static_cast<uint32_t>(groups)), dim3(256),
                       0, s, absmax, nblocks, qscale, gscale);
  return hipGetLastError();
}

hipError_t launch_dq_centred(const float* absmax, int64_t nblocks, uint8_t* qscale, float* gscale,
                             float* mu, hipStream_t s) {
  if (nblocks == 0) return hipSuccess;
  // partial sums go to gscale (ceil(nblocks / 256) words) before its final
  // values: level 1 needs 2 ceil(nblocks / 4096) words, which fit once
  // nblocks > 4096; deeper levels follow it and are smaller still
  uint32_t* stage = reinterpret_cast<uint32_t*>(gscale);
  if (nblocks <= kTreeChunk) {
    hipLaunchKernelGGL((mean_tree_kernel<float, true>), dim3(1), dim3(256), 0, s, absmax, nblocks,
                       nullptr, nblocks, mu);
  } else {
    int64_t cnt = (nblocks + kTreeChunk - 1) / kTreeChunk;
    hipLaunchKernelGGL((mean_tree_kernel<float, false>), dim3(static_cast<uint32_t>(cnt)),
                       dim3(256), 0, s, absmax, nblocks, stage, nblocks, nullptr);
    const uint32_t* cur = stage;
    uint32_t* next = stage + 2 * cnt;
    while (cnt > kTreeChunk) {
      const int64_t m = (cnt + kTreeChunk - 1) / kTreeChunk;
      hipLaunchKernelGGL((mean_tree_kernel<uint32_t, false>), dim3(static_cast<uint32_t>(m)),
                         dim3(256), 0, s, cur, cnt, next, nblocks, nullptr);
      cur = next;
      next += 2 * m;
      cnt = m;
    }
    hipLaunchKernelGGL((mean_tree_kernel<uint32_t, true>), dim3(1), dim3(256), 0, s, cur, cnt,
                       nullptr, nblocks, mu);
  }
  const int64_t groups = (nblocks + 255) / 256;
  hipLaunchKernelGGL(dq_centred_kernel, dim3(static_cast<uint32_t>(groups)), dim3(256), 0, s,
                     absmax, nblocks, mu, qscale, gscale);
  return hipGetLastError();
}

hipError_t launch_dequant(const WeightView& w, bool out_bf16, void* out, hipStream_t s) {
  const int64_t numel = w.N * w.K;
  if (numel == 0) return hipSuccess;
  const CodeParams P = code_params(w);
  const int64_t groups = (numel / 32 + 255) / 256;
  if (out_bf16)
    hipLaunchKernelGGL(nf4_dequant_kernel<true>, dim3(static_cast<uint32_t>(groups)), dim3(256),
                       0, s, w.packed, w.qscale, w.gscale, w.absmax, numel, out, P);
  else
    hipLaunchKernelGGL(nf4_dequant_kernel<false>, dim3(static_cast<uint32_t>(groups)), dim3(256),
                       0, s, w.packed, w.qscale, w.gscale, w.absmax, numel, out, P);
  return hipGetLastError();
}

}  // namespace qn
