// Host-side launch functions, one per kernel family.  The C ABI in
// qn_api.cpp validates arguments and then calls these; each returns the
// hipError_t of its launch(es).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qn {

struct CodeParams;  // qn_device.h

// Kinds of level-2 code of the block constants.
constexpr int kL2Grid8 = 0;    // uint8 grid fl32(q / 255) of c / c2
constexpr int kL2E4M3 = 1;     // E4M3 number of c / c2
constexpr int kL2Centred = 2;  // signed grid fl32(k / 127) of (c - mu) / c2

struct WeightView {
  const uint8_t* packed;
  const uint8_t* qscale;  // nullptr: not double-quantised
  const float* gscale;
  const float* absmax;
  int64_t N, K;
  int quant_type;  // kQuantNF4 or kQuantFP4 (the code table)
  int l2;          // level-2 code: 0 uint8 grid, 1 E4M3, 2 mean-centred signed grid
  const float* mu; // the centred code's offset (device, one fp32), else nullptr
};

// Code values and level-2 kind of a weight, for the kernels.
CodeParams code_params(const WeightView& w);

hipError_t launch_quantize(const void* w, bool bf16, int64_t numel, int quant_type,
                           uint8_t* packed, float* absmax, hipStream_t s);
hipError_t launch_dq(const float* absmax, int64_t nblocks, bool fp8, uint8_t* qscale,
                     float* gscale, hipStream_t s);
// Both in one launch (one workgroup per 256-block group); absmax may be
// nullptr.
hipError_t launch_quantize_dq(const void* w, bool bf16, int64_t numel, int quant_type, bool fp8,
                              uint8_t* packed, float* absmax, uint8_t* qscale, float* gscale,
                              hipStream_t s);
// Several weights of one dtype and code type in one launch: entry i is
// weight w[i] of numel[i] elements and its outputs; gend[i] is one past the
// last group (workgroup) of entries 0..i.  The struct travels by value as
// a kernel argument.
constexpr int kQdqMaxBatch = 8;
struct QdqBatch {
  const void* w[kQdqMaxBatch];
  int64_t numel[kQdqMaxBatch];
  uint8_t* packed[kQdqMaxBatch];
  float* absmax[kQdqMaxBatch];
  uint8_t* qscale[kQdqMaxBatch];
  float* gscale[kQdqMaxBatch];
  uint32_t gend[kQdqMaxBatch];
  int n;
};
hipError_t launch_quantize_dq_batch(const QdqBatch& batch, bool bf16, int quant_type, bool fp8,
                                    hipStream_t s);
// Mean-centred level-2 code: mu (pairwise fp64 sum of the constants / n,
// written to *mu), then per 256-group c2 = max |c - mu| and signed codes.
// gscale doubles as scratch for the partial sums before its final values.
hipError_t launch_dq_centred(const float* absmax, int64_t nblocks, uint8_t* qscale, float* gscale,
                             float* mu, hipStream_t s);
hipError_t launch_dequant(const WeightView& w, bool out_bf16, void* out, hipStream_t s);

// out[M, r] = in[M, L] * P^T, P row-major [r, L] (in and P 16-byte
// aligned, L % 32 == 0).  ksplit == 1 writes any of: fp32 result,
// bf16(scale * result), bf16(result); ksplit > 1 splits L over ksplit
// workgroups and writes fp32 partial sums out_f32[ksplit][M][r].
// With p_rows_l, P is stored [L, r] instead (B for t = dy B, read in place).
hipError_t launch_skinny(const uint16_t* in, int64_t M, int64_t L, const uint16_t* P, int r,
                         float scale, float* out_f32, uint16_t* out_scaled_bf16,
                         uint16_t* out_bf16, int ksplit, hipStream_t s, bool p_rows_l = false);
// Largest number of L-slices of the decode LoRA-down (the forward
// workspace holds that many fp32 partial sums of u).
constexpr int kDecodeMaxSlices = 512;
// Largest number of L-slices of the token-batch LoRA projections u = x A^T
// and t = dy B, whose fp32 partial sums the fused GEMM adds up.
constexpr int kWideMaxSlices = 16;
// Number of L-slices launch_skinny uses for M > 16 tokens.
int skinny_wide_splits(int64_t M, int64_t L);

// Streaming read of `bytes` (a multiple of 16) with 16-byte loads (a
// measurement aid).
hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t st);

// Size of the library's own per-device scratch array (qn_scratch.hip), the
// workspace of the allocation-free forward.
constexpr size_t kScratchBytes = static_cast<size_t>(64) << 20;
// Device address of the scratch array of the device that `stream` belongs
// to (the current device for the null stream), resolved once per device
// with that device current, then cached.
hipError_t scratch_address(hipStream_t stream, void** out);

// Threads per workgroup of the decode GEMV for an N x K weight.
int gemv_threads(int64_t N, int64_t K);
// Number of L-slices launch_skinny uses for the decode path (M <= 16),
// given the GEMV's threads per workgroup (which bounds the partial sums it
// can take).
int skinny_splits(int64_t M, int64_t L, int r, int gemv_thr);

// Decode path (M <= 16): y = x W^T + s u B^T with u given as usplit fp32
// partial sums [usplit][M][r]; optionally writes bf16(u) to u_out.
// With A_self (A [r, K]; only where gemv_self_u holds) the GEMV launch
// computes u itself from x, and u / usplit are not read.
hipError_t launch_gemv(const WeightView& w, const uint16_t* x, int M, const float* u, int usplit,
                       const uint16_t* B, int r, float s, uint16_t* y, uint16_t* u_out,
                       hipStream_t st, const uint16_t* A_self = nullptr);
// Whether the GEMV for this weight, M and r computes the LoRA-down in the
// same launch (one token, r <= 16, one pass of the 16-wave kernel, and A
// re-read by all bands in at most about 40 MB).
bool gemv_self_u(const WeightView& w, int M, int r);

// Fused dequant GEMM, forward: y[M,N] = x W^T + us B^T (us = bf16(s*u), [M, r]).
hipError_t launch_gemm_fwd(const WeightView& w, const uint16_t* x, int64_t M,
                           const uint16_t* us, const uint16_t* B, int r, uint16_t* y,
                           hipStream_t st);

// Fused dequant GEMM, backward to the input: dx[M,K] = dy W + ts A; with
// dx32 the fp32 result goes to dx32 [M, K] instead (dx untouched).
hipError_t launch_gemm_bwd(const WeightView& w, const uint16_t* dy, int64_t M,
                           const uint16_t* ts, const uint16_t* A, int r, uint16_t* dx,
                           hipStream_t st, float* dx32 = nullptr);

// Sum of nslice (<= kWideMaxSlices) fp32 partial sums part[nslice][n] in
// slice order: writes bf16(scale * sum) to out_scaled (and bf16(sum) to out
// if non-null).
hipError_t launch_lora_reduce(const float* part, int nslice, int64_t n, float scale,
                              uint16_t* out_scaled, uint16_t* out, hipStream_t st);

// LoRA merge: out[N, K] = bf16(dequant(W) + s B A) (A [r, K], B [N, r]).
hipError_t launch_merge(const WeightView& w, const uint16_t* A, const uint16_t* B, int r, float s,
                        uint16_t* out, hipStream_t st);

// AdamW step (see lora_adamw_step in the C ABI).
hipError_t launch_adamw(float* p, const float* g, float* m, float* v, uint16_t* p_bf16, int64_t n,
                        float lr, float beta1, float beta2, float eps, float weight_decay, int step,
                        hipStream_t st);

// LoRA dropout on the adapter branch (see lora_dropout in the C ABI):
// threshold = floor(p 2^32) on the 32-bit Philox halves, inv_keep =
// fl32(1 / (1 - p)), both from fp64 on the host.
struct DropoutParams {
  uint32_t threshold;
  float inv_keep;
};
DropoutParams dropout_params(float p);
// out[M, K] = x * keep / (1 - p) in bf16 (dropped elements +0); K % 8 == 0.
hipError_t launch_dropout(const uint16_t* x, int64_t M, int64_t K, float p, uint64_t seed,
                          uint16_t* out, hipStream_t st);
// dx[M, K] = bf16(base[M, K] + keep * (ts A) / (1 - p)), base the fp32
// product dy W, ts = bf16(s t) [M, r], A [r, K]: one rounding.
hipError_t launch_dx_lora_dropout(const float* base, uint16_t* dx, const uint16_t* ts,
                                  const uint16_t* A, int64_t M, int64_t K, int r, float p,
                                  uint64_t seed, hipStream_t st);

// LoRA gradients (see lora_grads in the C ABI).  u and t are bf16 [M, r];
// ws holds grads_workspace_bytes() of split-M partials.
size_t grads_workspace_bytes(int64_t M, int64_t N, int64_t K, int r);
hipError_t launch_grads_impl(const uint16_t* x, const uint16_t* dy, const uint16_t* u,
                             const uint16_t* t, int64_t M, int64_t N, int64_t K, int r, float s,
                             float* dA, float* dB, void* ws, hipStream_t st);

}  // namespace qn
