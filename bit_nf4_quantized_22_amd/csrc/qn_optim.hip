// AdamW step on the LoRA matrices (gfx950), fp32 parameters and states.
//
// [rkmt "QLORA技术解析" §3.5], [czcl "QLoRA技術解析" §3.2]: the adapter is
// trained with AdamW (32-bit states, learning rate 2e-4); only A and B have
// optimizer state.  The update is the published AdamW with decoupled weight
// decay, in this order per element (all fp32, IEEE operations):
//   p <- p * (1 - lr wd)
//   m <- b1 m + (1 - b1) g;   v <- b2 v + (1 - b2) g^2
//   p <- p - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps)
// The bias corrections come from the host (fp64, rounded to fp32).  An
// optional bf16 copy of the new p is the operand of the next forward.
//
// HBM-bound: 16 bytes read and 12 (+2) written per parameter, four
// parameters per thread with 16-byte loads.

#include <cmath>

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

struct AdamArgs {
  float lr, beta1, beta2, eps, decay;  // decay = 1 - lr wd
  float step_size;                     // lr / (1 - beta1^t)
  float inv_bc2_sqrt;                  // 1 / sqrt(1 - beta2^t)
};

__device__ __forceinline__ void adam_one(float& p, float g, float& m, float& v, const AdamArgs& a) {
  p = __fmul_rn(p, a.decay);
  m = __fadd_rn(__fmul_rn(a.beta1, m), __fmul_rn(1.0f - a.beta1, g));
  v = __fadd_rn(__fmul_rn(a.beta2, v), __fmul_rn(1.0f - a.beta2, __fmul_rn(g, g)));
  const float denom = __fadd_rn(__fmul_rn(__fsqrt_rn(v), a.inv_bc2_sqrt), a.eps);
  p = __fsub_rn(p, __fmul_rn(a.step_size, __fdiv_rn(m, denom)));
}

__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p,
                                                    const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    uint16_t* __restrict__ p_bf16, int64_t n,
                                                    AdamArgs a) {
  typedef float f4_t __attribute__((ext_vector_type(4)));
  const int64_t i4 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i4 + 4 <= n) {
    f4_t pv = *reinterpret_cast<const f4_t*>(p + i4);
    const f4_t gv = *reinterpret_cast<const f4_t*>(g + i4);
    f4_t mv = *reinterpret_cast<const f4_t*>(m + i4);
    f4_t vv = *reinterpret_cast<const f4_t*>(v + i4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float pj = pv[j], mj = mv[j], vj = vv[j];
      adam_one(pj, gv[j], mj, vj, a);
      pv[j] = pj;
      mv[j] = mj;
      vv[j] = vj;
    }
    *reinterpret_cast<f4_t*>(p + i4) = pv;
    *reinterpret_cast<f4_t*>(m + i4) = mv;
    *reinterpret_cast<f4_t*>(v + i4) = vv;
    if (p_bf16)
      *reinterpret_cast<uint2*>(p_bf16 + i4) =
          make_uint2(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]));
  } else {
    for (int64_t i = i4; i < n; ++i) {  // the last 1..3 parameters
      float pj = p[i], mj = m[i], vj = v[i];
      adam_one(pj, g[i], mj, vj, a);
      p[i] = pj;
      m[i] = mj;
      v[i] = vj;
      if (p_bf16) p_bf16[i] = static_cast<uint16_t>(pack_bf16x2(pj, 0.f) & 0xFFFF);
    }
  }
}

}  // namespace

hipError_t launch_adamw(float* p, const float* g, float* m, float* v, uint16_t* p_bf16, int64_t n,
                        float lr, float beta1, float beta2, float eps, float weight_decay, int step,
                        hipStream_t st) {
  if (n == 0) return hipSuccess;
  AdamArgs a;
  a.lr = lr;
  a.beta1 = beta1;
  a.beta2 = beta2;
  a.eps = eps;
  a.decay = static_cast<float>(1.0 - static_cast<double>(lr) * static_cast<double>(weight_decay));
  const double bc1 = 1.0 - std::pow(static_cast<double>(beta1), step);
  const double bc2 = 1.0 - std::pow(static_cast<double>(beta2), step);
  a.step_size = static_cast<float>(static_cast<double>(lr) / bc1);
  a.inv_bc2_sqrt = static_cast<float>(1.0 / std::sqrt(bc2));
  const int64_t threads = (n + 3) / 4;
  hipLaunchKernelGGL(adamw_kernel, dim3(static_cast<uint32_t>((threads + 255) / 256)), dim3(256), 0,
                     st, p, g, m, v, p_bf16, n, a);
  return hipGetLastError();
}

}  // namespace qn
