// LoRA merge (gfx950): out[n, k] = bf16(fl32(q[code] c') + fl32(s * sum_j B[n, j] A[j, k])),
// s = alpha / r, the sum an fp32 fma chain over j = 0 .. r - 1.
//
// [rkmt "QLORA技术解析" §2.1] for inference the adapter is folded into the
// weight, W <- W + B A, so it costs no latency; [tgd "QLoRA微调" §7] a QLoRA
// adapter is merged into a 16-bit weight, never into the 4-bit form.  The
// weight here is the dequantised NF4 weight (the value the adapter was
// trained against), expanded on the fly: the merged bf16 weight is the only
// 16-bit copy that is written.  Re-quantising it (nf4_quantize) gives a
// merged 4-bit model.
//
// HBM-bound streaming kernel: per weight it reads half a byte of codes and
// writes two bytes.  A workgroup of 256 threads owns 256 consecutive columns
// and kRowsPerWG rows; each thread keeps the r values of A's column in
// registers for all its rows, the workgroup's rows of B sit in LDS as fp32
// (one broadcast read per value), and the loads of kRowBatch rows are
// issued together, so the rank-r update costs r fp32 FMAs per weight.

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

constexpr int kRowsPerWG = 32;
constexpr int kRowBatch = 8;  // rows whose loads are issued together

template <int kR, bool kDQ>
__global__ __launch_bounds__(256) void merge_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ gscale, const float* __restrict__ absmax, int64_t N, int64_t K,
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int r, float s,
    uint16_t* __restrict__ out, CodeParams P) {
  // A's column in registers: fp32 for r <= 64, bf16 pairs above (register budget)
  constexpr bool kPacked = kR > 64;
  constexpr int kAR = kR == 0 ? 1 : (kPacked ? kR / 2 : kR);
  __shared__ float scode[16];
  __shared__ __attribute__((aligned(16))) float sB[kRowsPerWG][kR == 0 ? 4 : kR];  // B rows, fp32
  const int tid = threadIdx.x;
  {
    const CodeRegs R = code_regs(P);
    const float qv = code_value(R, tid & 15);
    if (tid < 16) scode[tid] = qv;
  }
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * kRowsPerWG;
  if constexpr (kR > 0) {
    // the workgroup's rows of B (rows past N and columns past r: zero)
    for (int i = tid; i < kRowsPerWG * kR; i += 256) {
      const int rr = i / kR, j = i % kR;
      const int64_t n = n0 + rr;
      const bool ok = n < N && j < r;
      const float v = bf16_to_f32(B[(n < N ? n : N - 1) * r + (j < r ? j : r - 1)]);
      sB[rr][j] = ok ? v : 0.f;
    }
  }
  __syncthreads();
  const int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + tid;
  const bool kvalid = k < K;
  const int64_t kc = kvalid ? k : K - 1;  // columns past K read column K - 1, store nothing
  // A[:, k] for j < r, zero beyond r (loads clamped to row r - 1, so every
  // load is unconditional and in bounds; kR == 0 is the frozen weight)
  uint32_t a[kAR];
#pragma unroll
  for (int i = 0; i < kAR; ++i) {
    if constexpr (kR == 0) {
      a[i] = 0;
    } else if constexpr (kPacked) {
      const int j0 = 2 * i, j1 = 2 * i + 1;
      const uint32_t v0 = A[static_cast<int64_t>(j0 < r ? j0 : r - 1) * K + kc];
      const uint32_t v1 = A[static_cast<int64_t>(j1 < r ? j1 : r - 1) * K + kc];
      a[i] = (j0 < r ? v0 : 0u) | ((j1 < r ? v1 : 0u) << 16);
    } else {
      const uint32_t v = A[static_cast<int64_t>(i < r ? i : r - 1) * K + kc];
      a[i] = i < r ? (v << 16) : 0u;  // fp32 bit pattern of the bf16 value
    }
  }
  const int shift = (kc & 1) ? 0 : 4;  // even column: high nibble
  const int64_t nlast = (n0 + kRowsPerWG < N ? n0 + kRowsPerWG : N) - 1;
  for (int rb = 0; rb < kRowsPerWG; rb += kRowBatch) {
    // all loads of the batch first (rows past N re-read the last row)
    uint32_t byte[kRowBatch], q8[kRowBatch];
    float c2[kRowBatch];
#pragma unroll
    for (int i = 0; i < kRowBatch; ++i) {
      const int64_t n = n0 + rb + i < nlast ? n0 + rb + i : nlast;
      const int64_t bi = n * (K >> 6) + (kc >> 6);
      byte[i] = packed[n * (K >> 1) + (kc >> 1)];
      if constexpr (kDQ) {
        q8[i] = qscale[bi];
        c2[i] = gscale[bi >> 8];
      } else {
        q8[i] = 0;
        c2[i] = absmax[bi];
      }
    }
#pragma unroll
    for (int i = 0; i < kRowBatch; ++i) {
      const int64_t n = n0 + rb + i;
      const float cs = kDQ ? __fmul_rn(l2_value(q8[i], P.fp8), c2[i]) : c2[i];
      const float w = __fmul_rn(scode[(byte[i] >> shift) & 15], cs);
      float merged = w;
      if constexpr (kR > 0) {
        const float* brow = sB[rb + i];
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < kR; ++j) {
          float aj;
          if constexpr (kPacked)
            aj = __uint_as_float((j & 1) ? (a[j >> 1] & 0xFFFF0000u) : (a[j >> 1] << 16));
          else
            aj = __uint_as_float(a[j]);
          t = __fmaf_rn(brow[j], aj, t);
        }
        merged = __fadd_rn(w, __fmul_rn(s, t));
      }
      if (kvalid && n <= nlast) out[n * K + k] = static_cast<uint16_t>(pack_bf16x2(merged, 0.f) & 0xFFFF);
    }
  }
}

template <int kR>
void merge_launch(const WeightView& w, const uint16_t* A, const uint16_t* B, int r, float s,
                  uint16_t* out, const CodeParams& P, hipStream_t st) {
  const dim3 grid(static_cast<uint32_t>((w.K + 255) / 256),
                  static_cast<uint32_t>((w.N + kRowsPerWG - 1) / kRowsPerWG));
  if (w.qscale)
    hipLaunchKernelGGL((merge_kernel<kR, true>), grid, dim3(256), 0, st, w.packed, w.qscale,
                       w.gscale, w.absmax, w.N, w.K, A, B, r, s, out, P);
  else
    hipLaunchKernelGGL((merge_kernel<kR, false>), grid, dim3(256), 0, st, w.packed, w.qscale,
                       w.gscale, w.absmax, w.N, w.K, A, B, r, s, out, P);
}

}  // namespace

hipError_t launch_merge(const WeightView& w, const uint16_t* A, const uint16_t* B, int r, float s,
                        uint16_t* out, hipStream_t st) {
  if (w.N == 0 || w.K == 0) return hipSuccess;
  const CodeParams P = code_params(w);
  if (r == 0) merge_launch<0>(w, A, B, r, s, out, P, st);  // frozen weight: A, B unused
  else if (r <= 16) merge_launch<16>(w, A, B, r, s, out, P, st);
  else if (r <= 32) merge_launch<32>(w, A, B, r, s, out, P, st);
  else if (r <= 64) merge_launch<64>(w, A, B, r, s, out, P, st);
  else merge_launch<128>(w, A, B, r, s, out, P, st);
  return hipGetLastError();
}

}  // namespace qn
