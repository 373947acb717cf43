// C ABI of the QLoRA NF4 library: argument validation on the host, then the
// launches on the caller's stream.  See include/qlora_nf4.h for the contract
// of every entry point.

#include "qlora_nf4.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "qn_launch.h"
#include "qn_tables.h"

namespace {

constexpr int kBlock = 64;
constexpr int kGroup = 256;
constexpr int kMaxRank = 128;
constexpr int64_t kGemvMaxM = 16;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int hip_status(hipError_t e) { return e == hipSuccess ? QN_OK : QN_ERR_HIP; }

// The adapter of a call: r == 0, or A and B both NULL, is the frozen layer
// (rank 0); exactly one of A, B NULL with r > 0 is an error.
int adapter_rank(int32_t r, const void* A, const void* B, int32_t& r_eff) {
  r_eff = r;
  if (r > 0 && !A && !B) r_eff = 0;
  else if (r > 0 && (!A || !B)) return QN_ERR_NULL;
  return QN_OK;
}

// Validates a quantised weight for the linear ops and fills a view.
int check_weight(const qn_weight* w, qn::WeightView& v, bool linear) {
  if (!w || !w->packed) return QN_ERR_NULL;
  if (w->blocksize != kBlock || w->group != kGroup) return QN_ERR_UNSUPPORTED;
  if (w->quant_type != QN_NF4 && w->quant_type != QN_FP4) return QN_ERR_UNSUPPORTED;
  if (w->scale_type != QN_SCALE_U8 && w->scale_type != QN_SCALE_FP8 &&
      w->scale_type != QN_SCALE_CENTRED)
    return QN_ERR_UNSUPPORTED;
  if (!qn::tables(w->quant_type)) return QN_ERR_UNSUPPORTED;
  if (w->N < 0 || w->K < 0) return QN_ERR_SHAPE;
  if (linear && (w->N <= 0 || w->K <= 0 || w->N % 64 != 0 || w->K % 64 != 0)) return QN_ERR_SHAPE;
  const bool centred = w->qscale && w->scale_type == QN_SCALE_CENTRED;
  if (w->qscale) {
    if (!w->gscale || (centred && !w->offset)) return QN_ERR_NULL;
  } else if (!w->absmax) {
    return QN_ERR_NULL;
  }
  if (!aligned(w->packed, 16)) return QN_ERR_ALIGN;
  if ((w->gscale && !aligned(w->gscale, 4)) || (w->absmax && !aligned(w->absmax, 4)) ||
      (centred && !aligned(w->offset, 4)))
    return QN_ERR_ALIGN;
  v.packed = w->packed;
  v.qscale = w->qscale;
  v.gscale = w->gscale;
  v.absmax = w->qscale ? nullptr : w->absmax;
  v.N = w->N;
  v.K = w->K;
  v.quant_type = w->quant_type == QN_FP4 ? qn::kQuantFP4 : qn::kQuantNF4;
  v.l2 = !w->qscale ? qn::kL2Grid8
        : w->scale_type == QN_SCALE_FP8 ? qn::kL2E4M3
        : w->scale_type == QN_SCALE_CENTRED ? qn::kL2Centred
                                            : qn::kL2Grid8;
  v.mu = centred ? w->offset : nullptr;
  return QN_OK;
}

// fp32 partial sums of u (or t) over L-slices: up to kDecodeMaxSlices of
// them on the decode path, kWideMaxSlices for token batches.
size_t lora_part_bytes(int64_t M, int32_t r) {
  const size_t mr = static_cast<size_t>(M) * static_cast<size_t>(r);
  const size_t slices = M <= kGemvMaxM ? qn::kDecodeMaxSlices : qn::kWideMaxSlices;
  return round_up(mr * 4 * slices, 256);
}

// bf16(s u) or bf16(s t), the LoRA operand of the fused GEMM.
size_t lora_bf16_bytes(int64_t M, int32_t r) {
  return round_up(static_cast<size_t>(M) * static_cast<size_t>(r) * 2, 256);
}

// Forward workspace: the partial sums of u, then bf16(s u).
size_t fwd_ws(int64_t M, int32_t r) {
  if (r == 0 || M == 0) return 0;
  return lora_part_bytes(M, r) + lora_bf16_bytes(M, r);
}

// Backward workspace: the partial sums of t, then bf16(s t).
size_t bwd_ws(int64_t M, int64_t N, int32_t r) {
  (void)N;
  if (r == 0 || M == 0) return 0;
  return lora_part_bytes(M > kGemvMaxM ? M : kGemvMaxM + 1, r) + lora_bf16_bytes(M, r);
}

// Backward with dropout: the backward's workspace, then the fp32 product
// dy W [M, K] that the masked LoRA pass adds to before rounding once.
size_t bwd_drop_ws(int64_t M, int64_t N, int64_t K, int32_t r) {
  if (r == 0 || M == 0) return 0;
  return bwd_ws(M, N, r) + round_up(static_cast<size_t>(M) * static_cast<size_t>(K) * 4, 256);
}

// Gradient workspace: bf16 u and t (recomputed when not given), the
// partial sums of those projections, then the split-M partial sums.
size_t grads_ws(int64_t M, int64_t N, int64_t K, int32_t r) {
  if (r == 0) return 0;
  return 2 * lora_bf16_bytes(M, r) + lora_part_bytes(M > kGemvMaxM ? M : kGemvMaxM + 1, r) +
         round_up(qn::grads_workspace_bytes(M, N, K, r), 256);
}

int codebook(int qt, float out[16]) {
  if (!out) return QN_ERR_NULL;
  const qn::Tables* t = qn::tables(qt);
  if (!t) return QN_ERR_UNSUPPORTED;
  std::memcpy(out, t->q32, sizeof(t->q32));
  return QN_OK;
}

int quantize(int qt, const void* w, int32_t dtype, int64_t numel, int32_t blocksize,
             uint8_t* packed, float* absmax, void* stream) {
  if (blocksize != kBlock) return QN_ERR_UNSUPPORTED;
  if (dtype != QN_F32 && dtype != QN_BF16) return QN_ERR_UNSUPPORTED;
  if (numel < 0 || (numel & 1)) return QN_ERR_SHAPE;
  if (numel == 0) return QN_OK;
  if (!w || !packed || !absmax) return QN_ERR_NULL;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(absmax, 4)) return QN_ERR_ALIGN;
  if (!qn::tables(qt)) return QN_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return hip_status(
      qn::launch_quantize(w, dtype == QN_BF16, numel, qt, packed, absmax, as_stream(stream)));
}

int dq(bool fp8, const float* absmax, int64_t nblocks, int32_t group, uint8_t* qscale,
       float* gscale, void* stream) {
  if (group != kGroup) return QN_ERR_UNSUPPORTED;
  if (nblocks < 0) return QN_ERR_SHAPE;
  if (nblocks == 0) return QN_OK;
  if (!absmax || !qscale || !gscale) return QN_ERR_NULL;
  if (!aligned(absmax, 4) || !aligned(gscale, 4)) return QN_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(qn::launch_dq(absmax, nblocks, fp8, qscale, gscale, as_stream(stream)));
}

// Forward with the LoRA-down input xa (x itself, or the dropped x).
int fwd_impl(const qn_weight* w, const qn_bf16* x, const qn_bf16* xa, int64_t M, const qn_bf16* A,
             const qn_bf16* B, int32_t r, float alpha, qn_bf16* y, qn_bf16* u_out, void* ws,
             size_t ws_bytes, void* stream, bool own_scratch = false) {
  qn::WeightView v;
  int st = check_weight(w, v, true);
  if (st != QN_OK) return st;
  if (M < 0 || r < 0) return QN_ERR_SHAPE;
  if (r > kMaxRank) return QN_ERR_UNSUPPORTED;
  if (M == 0 || w->N == 0) return QN_OK;
  if ((st = adapter_rank(r, A, B, r)) != QN_OK) return st;
  if (!x || !xa || !y) return QN_ERR_NULL;
  if (!aligned(x, 16) || !aligned(xa, 16) || !aligned(y, 2) || (r > 0 && (!aligned(A, 16) || !aligned(B, 2))) ||
      (u_out && !aligned(u_out, 2)))
    return QN_ERR_ALIGN;
  const size_t need = fwd_ws(M, r);
  if (own_scratch) {
    // the library's per-device array stands in for the caller's workspace
    if (need > qn::kScratchBytes) return QN_ERR_WORKSPACE;
    ws = nullptr;
    ws_bytes = 0;
    if (need > 0) {
      if (qn::scratch_address(as_stream(stream), &ws) != hipSuccess) return QN_ERR_HIP;
      ws_bytes = qn::kScratchBytes;
    }
  }
  if (need > 0 && (!ws || ws_bytes < need)) return QN_ERR_WORKSPACE;
  if (need > 0 && !aligned(ws, 16)) return QN_ERR_ALIGN;
  if (!qn::tables()) return QN_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  (void)hipGetLastError();
  const float scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
  // u = x A^T as fp32 partial sums over L-slices, added up (in slice order)
  // by the GEMV or GEMM that applies the LoRA-up term
  float* u32 = static_cast<float*>(ws);
  const bool decode = M <= kGemvMaxM;
  const int ks = decode ? qn::skinny_splits(M, w->K, r, qn::gemv_threads(w->N, w->K))
                        : qn::skinny_wide_splits(M, w->K);
  // one token on a one-pass GEMV (and no dropout): the GEMV launch computes
  // u from the x it stages, and no LoRA-down launch runs
  const bool self_u = decode && r > 0 && xa == x && qn::gemv_self_u(v, static_cast<int>(M), r);
  if (r > 0 && !self_u) {
    if (qn::launch_skinny(xa, M, w->K, A, r, scale, u32, nullptr, nullptr, ks, s) != hipSuccess)
      return QN_ERR_HIP;
  }
  if (decode)
    return hip_status(qn::launch_gemv(v, x, static_cast<int>(M), u32, ks, B, r, scale, y,
                                      r > 0 ? u_out : nullptr, s, self_u ? A : nullptr));
  uint16_t* us = nullptr;
  if (r > 0) {
    us = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + lora_part_bytes(M, r));
    if (qn::launch_lora_reduce(u32, ks, M * r, scale, us, u_out, s) != hipSuccess) return QN_ERR_HIP;
  }
  return hip_status(qn::launch_gemm_fwd(v, x, M, us, B, r, y, s));
}

// Backward to the input; with drop, the LoRA term is masked by the dropout
// of the adapter's input (base GEMM alone, then dx += D * (s t A)).
int bwd_impl(const qn_weight* w, const qn_bf16* dy, int64_t M, const qn_bf16* A, const qn_bf16* B,
             int32_t r, float alpha, const float* drop_p, uint64_t seed, qn_bf16* dx,
             qn_bf16* t_out, void* ws, size_t ws_bytes, void* stream) {
  qn::WeightView v;
  int st = check_weight(w, v, true);
  if (st != QN_OK) return st;
  if (M < 0 || r < 0) return QN_ERR_SHAPE;
  if (r > kMaxRank) return QN_ERR_UNSUPPORTED;
  if (M == 0 || w->K == 0) return QN_OK;
  if ((st = adapter_rank(r, A, B, r)) != QN_OK) return st;
  if (!dy || !dx) return QN_ERR_NULL;
  if (!aligned(dy, 16) || !aligned(dx, 2) || (r > 0 && (!aligned(A, 2) || !aligned(B, 2))) ||
      (t_out && !aligned(t_out, 2)))
    return QN_ERR_ALIGN;
  const size_t need = drop_p ? bwd_drop_ws(M, w->N, w->K, r) : bwd_ws(M, w->N, r);
  if (need > 0 && (!ws || ws_bytes < need)) return QN_ERR_WORKSPACE;
  if (need > 0 && !aligned(ws, 16)) return QN_ERR_ALIGN;
  if (!qn::tables()) return QN_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  (void)hipGetLastError();
  const float scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
  // t = dy B as fp32 partial sums over N-slices (B read where it lies,
  // [N, r]), added up in slice order into bf16(s t), the GEMM's operand
  uint16_t* ts = nullptr;
  const int64_t mp = M > kGemvMaxM ? M : kGemvMaxM + 1;
  const int ks = qn::skinny_wide_splits(mp, w->N);
  if (r > 0) {
    char* base = static_cast<char*>(ws);
    float* t32 = reinterpret_cast<float*>(base);
    ts = reinterpret_cast<uint16_t*>(base + lora_part_bytes(mp, r));
    if (qn::launch_skinny(dy, M, w->N, B, r, scale, t32, nullptr, nullptr, ks, s, true) !=
        hipSuccess)
      return QN_ERR_HIP;
    if (qn::launch_lora_reduce(t32, ks, M * r, scale, ts, t_out, s) != hipSuccess) return QN_ERR_HIP;
  }
  if (!drop_p || r == 0) return hip_status(qn::launch_gemm_bwd(v, dy, M, ts, A, r, dx, s));
  float* base32 = reinterpret_cast<float*>(static_cast<char*>(ws) + bwd_ws(M, w->N, r));
  if (qn::launch_gemm_bwd(v, dy, M, nullptr, nullptr, 0, dx, s, base32) != hipSuccess)
    return QN_ERR_HIP;
  return hip_status(qn::launch_dx_lora_dropout(base32, dx, ts, A, M, w->K, r, *drop_p, seed, s));
}

}  // namespace

extern "C" {

const char* qn_status_string(int status) {
  switch (status) {
    case QN_OK: return "ok";
    case QN_ERR_NULL: return "a required pointer is NULL";
    case QN_ERR_SHAPE: return "invalid or inconsistent sizes";
    case QN_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QN_ERR_UNSUPPORTED: return "unsupported parameter (blocksize 64, group 256, fp32/bf16 only)";
    case QN_ERR_WORKSPACE: return "workspace missing or too small";
    case QN_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int nf4_codebook(float out[16]) { return codebook(qn::kQuantNF4, out); }

int fp4_codebook(float out[16]) { return codebook(qn::kQuantFP4, out); }

int nf4_quantize(const void* w, int32_t dtype, int64_t numel, int32_t blocksize,
                 uint8_t* packed, float* absmax, void* stream) {
  return quantize(qn::kQuantNF4, w, dtype, numel, blocksize, packed, absmax, stream);
}

int fp4_quantize(const void* w, int32_t dtype, int64_t numel, int32_t blocksize,
                 uint8_t* packed, float* absmax, void* stream) {
  return quantize(qn::kQuantFP4, w, dtype, numel, blocksize, packed, absmax, stream);
}

int dq_quantize_scales(const float* absmax, int64_t nblocks, int32_t group, uint8_t* qscale,
                       float* gscale, void* stream) {
  return dq(false, absmax, nblocks, group, qscale, gscale, stream);
}

int dq_quantize_scales_fp8(const float* absmax, int64_t nblocks, int32_t group,
                           uint8_t* qscale, float* gscale, void* stream) {
  return dq(true, absmax, nblocks, group, qscale, gscale, stream);
}

int nf4_quantize_dq(const void* w, int32_t dtype, int64_t numel, int32_t blocksize, int32_t group,
                    int32_t quant_type, int32_t scale_type, uint8_t* packed, float* absmax,
                    uint8_t* qscale, float* gscale, void* stream) {
  if (blocksize != kBlock || group != kGroup) return QN_ERR_UNSUPPORTED;
  if (dtype != QN_F32 && dtype != QN_BF16) return QN_ERR_UNSUPPORTED;
  if (quant_type != QN_NF4 && quant_type != QN_FP4) return QN_ERR_UNSUPPORTED;
  if (scale_type != QN_SCALE_U8 && scale_type != QN_SCALE_FP8) return QN_ERR_UNSUPPORTED;
  if (numel < 0 || (numel & 1)) return QN_ERR_SHAPE;
  if (numel == 0) return QN_OK;
  if (!w || !packed || !qscale || !gscale) return QN_ERR_NULL;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(gscale, 4) ||
      (absmax && !aligned(absmax, 4)))
    return QN_ERR_ALIGN;
  const int qt = quant_type == QN_FP4 ? qn::kQuantFP4 : qn::kQuantNF4;
  if (!qn::tables(qt)) return QN_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return hip_status(qn::launch_quantize_dq(w, dtype == QN_BF16, numel, qt,
                                           scale_type == QN_SCALE_FP8, packed, absmax, qscale,
                                           gscale, as_stream(stream)));
}

int nf4_quantize_dq_batch(int32_t n, const void* const* w, const int64_t* numel, int32_t dtype,
                          int32_t blocksize, int32_t group, int32_t quant_type,
                          int32_t scale_type, uint8_t* const* packed, float* const* absmax,
                          uint8_t* const* qscale, float* const* gscale, void* stream) {
  if (blocksize != kBlock || group != kGroup) return QN_ERR_UNSUPPORTED;
  if (dtype != QN_F32 && dtype != QN_BF16) return QN_ERR_UNSUPPORTED;
  if (quant_type != QN_NF4 && quant_type != QN_FP4) return QN_ERR_UNSUPPORTED;
  if (scale_type != QN_SCALE_U8 && scale_type != QN_SCALE_FP8) return QN_ERR_UNSUPPORTED;
  if (n < 0 || n > qn::kQdqMaxBatch) return QN_ERR_SHAPE;
  if (n == 0) return QN_OK;
  if (!w || !numel || !packed || !qscale || !gscale) return QN_ERR_NULL;
  qn::QdqBatch b{};
  const int64_t per = static_cast<int64_t>(kBlock) * kGroup;  // weights per group
  int64_t groups = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t m = numel[i];
    if (m < 0 || (m & 1)) return QN_ERR_SHAPE;
    if (m > 0) {
      float* am = absmax ? absmax[i] : nullptr;
      if (!w[i] || !packed[i] || !qscale[i] || !gscale[i]) return QN_ERR_NULL;
      if (!aligned(w[i], 16) || !aligned(packed[i], 16) || !aligned(gscale[i], 4) ||
          (am && !aligned(am, 4)))
        return QN_ERR_ALIGN;
      b.w[b.n] = w[i];
      b.numel[b.n] = m;
      b.packed[b.n] = packed[i];
      b.absmax[b.n] = am;
      b.qscale[b.n] = qscale[i];
      b.gscale[b.n] = gscale[i];
      groups += (m + per - 1) / per;
      if (groups > INT32_MAX) return QN_ERR_SHAPE;
      b.gend[b.n] = static_cast<uint32_t>(groups);
      ++b.n;
    }
  }
  if (b.n == 0) return QN_OK;
  const int qt = quant_type == QN_FP4 ? qn::kQuantFP4 : qn::kQuantNF4;
  if (!qn::tables(qt)) return QN_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return hip_status(qn::launch_quantize_dq_batch(b, dtype == QN_BF16, qt,
                                                 scale_type == QN_SCALE_FP8, as_stream(stream)));
}

int dq_quantize_scales_centred(const float* absmax, int64_t nblocks, int32_t group,
                               uint8_t* qscale, float* gscale, float* offset, void* stream) {
  if (group != kGroup) return QN_ERR_UNSUPPORTED;
  if (nblocks < 0) return QN_ERR_SHAPE;
  if (nblocks == 0) return QN_OK;
  if (!absmax || !qscale || !gscale || !offset) return QN_ERR_NULL;
  if (!aligned(absmax, 4) || !aligned(gscale, 4) || !aligned(offset, 4)) return QN_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(
      qn::launch_dq_centred(absmax, nblocks, qscale, gscale, offset, as_stream(stream)));
}

int nf4_dequant(const qn_weight* w, int32_t out_dtype, void* out, void* stream) {
  qn::WeightView v;
  int st = check_weight(w, v, false);
  if (st != QN_OK) return st;
  if (out_dtype != QN_F32 && out_dtype != QN_BF16) return QN_ERR_UNSUPPORTED;
  if ((w->N * w->K) % 32 != 0) return QN_ERR_SHAPE;
  if (w->N * w->K == 0) return QN_OK;
  if (!out) return QN_ERR_NULL;
  if (!aligned(out, 16)) return QN_ERR_ALIGN;
  if (!qn::tables()) return QN_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return hip_status(qn::launch_dequant(v, out_dtype == QN_BF16, out, as_stream(stream)));
}

size_t qn_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K, int32_t r) {
  if (M < 0 || N < 0 || K < 0 || r < 0 || r > kMaxRank) return 0;
  switch (op) {
    case QN_OP_FWD: return fwd_ws(M, r);
    case QN_OP_BWD_DX: return bwd_ws(M, N, r);
    case QN_OP_LORA_GRADS: return grads_ws(M, N, K, r);
    case QN_OP_BWD_DX_DROPOUT: return bwd_drop_ws(M, N, K, r);
    default: return 0;
  }
}

int qlora_linear_fwd(const qn_weight* w, const qn_bf16* x, int64_t M, const qn_bf16* A,
                     const qn_bf16* B, int32_t r, float alpha, qn_bf16* y, qn_bf16* u_out,
                     void* ws, size_t ws_bytes, void* stream) {
  return fwd_impl(w, x, x, M, A, B, r, alpha, y, u_out, ws, ws_bytes, stream);
}

int qn_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return QN_ERR_SHAPE;
  if (bytes == 0) return QN_OK;
  if (!buf || !sink) return QN_ERR_NULL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return QN_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(qn::launch_read_probe(buf, bytes, sink, as_stream(stream)));
}

int qlora_linear_fwd_noalloc(const qn_weight* w, const qn_bf16* x, int64_t M, const qn_bf16* A,
                             const qn_bf16* B, int32_t r, float alpha, qn_bf16* y,
                             qn_bf16* u_out, void* stream) {
  return fwd_impl(w, x, x, M, A, B, r, alpha, y, u_out, nullptr, 0, stream, true);
}

int qlora_linear_fwd_dropout(const qn_weight* w, const qn_bf16* x, const qn_bf16* x_drop,
                             int64_t M, const qn_bf16* A, const qn_bf16* B, int32_t r,
                             float alpha, qn_bf16* y, qn_bf16* u_out, void* ws, size_t ws_bytes,
                             void* stream) {
  return fwd_impl(w, x, x_drop, M, A, B, r, alpha, y, u_out, ws, ws_bytes, stream);
}

int qlora_linear_bwd_dx(const qn_weight* w, const qn_bf16* dy, int64_t M, const qn_bf16* A,
                        const qn_bf16* B, int32_t r, float alpha, qn_bf16* dx, qn_bf16* t_out,
                        void* ws, size_t ws_bytes, void* stream) {
  return bwd_impl(w, dy, M, A, B, r, alpha, nullptr, 0, dx, t_out, ws, ws_bytes, stream);
}

int qlora_linear_bwd_dx_dropout(const qn_weight* w, const qn_bf16* dy, int64_t M,
                                const qn_bf16* A, const qn_bf16* B, int32_t r, float alpha,
                                float p, uint64_t seed, qn_bf16* dx, qn_bf16* t_out, void* ws,
                                size_t ws_bytes, void* stream) {
  if (!(p >= 0.0f && p < 1.0f)) return QN_ERR_SHAPE;
  return bwd_impl(w, dy, M, A, B, r, alpha, &p, seed, dx, t_out, ws, ws_bytes, stream);
}

int lora_dropout(const qn_bf16* x, int64_t M, int64_t K, float p, uint64_t seed, qn_bf16* x_drop,
                 void* stream) {
  if (M < 0 || K < 0 || K % 8 != 0 || !(p >= 0.0f && p < 1.0f)) return QN_ERR_SHAPE;
  if (M == 0 || K == 0) return QN_OK;
  if (!x || !x_drop) return QN_ERR_NULL;
  if (!aligned(x, 16) || !aligned(x_drop, 16)) return QN_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(qn::launch_dropout(x, M, K, p, seed, x_drop, as_stream(stream)));
}

int qlora_merge(const qn_weight* w, const qn_bf16* A, const qn_bf16* B, int32_t r, float alpha,
                qn_bf16* out, void* stream) {
  qn::WeightView v;
  int st = check_weight(w, v, true);
  if (st != QN_OK) return st;
  if (r < 0) return QN_ERR_SHAPE;
  if (r > kMaxRank) return QN_ERR_UNSUPPORTED;
  if ((st = adapter_rank(r, A, B, r)) != QN_OK) return st;
  if (!out) return QN_ERR_NULL;
  if (!aligned(out, 16) || (r > 0 && (!aligned(A, 2) || !aligned(B, 2)))) return QN_ERR_ALIGN;
  if (!qn::tables()) return QN_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  const float scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
  return hip_status(qn::launch_merge(v, A, B, r, scale, out, as_stream(stream)));
}

int lora_adamw_step(float* p, const float* g, float* m, float* v, qn_bf16* p_bf16, int64_t n,
                    float lr, float beta1, float beta2, float eps, float weight_decay, int32_t step,
                    void* stream) {
  if (n < 0 || step < 1) return QN_ERR_SHAPE;
  if (n == 0) return QN_OK;
  if (!p || !g || !m || !v) return QN_ERR_NULL;
  if (!aligned(p, 16) || !aligned(g, 16) || !aligned(m, 16) || !aligned(v, 16) ||
      (p_bf16 && !aligned(p_bf16, 8)))
    return QN_ERR_ALIGN;
  if (!(lr >= 0.0f) || !(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) ||
      !(eps > 0.0f) || !(weight_decay >= 0.0f))
    return QN_ERR_SHAPE;
  (void)hipGetLastError();
  return hip_status(qn::launch_adamw(p, g, m, v, p_bf16, n, lr, beta1, beta2, eps, weight_decay,
                                     step, as_stream(stream)));
}

int lora_grads(const qn_bf16* x, const qn_bf16* dy, const qn_bf16* u, const qn_bf16* t,
               const qn_bf16* A, const qn_bf16* B, int64_t M, int64_t N, int64_t K, int32_t r,
               float alpha, float* dA, float* dB, void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || N < 0 || K < 0 || r < 0) return QN_ERR_SHAPE;
  if (r == 0) return QN_ERR_SHAPE;
  if (r > kMaxRank) return QN_ERR_UNSUPPORTED;
  if (N == 0 || K == 0 || N % 64 != 0 || K % 64 != 0) return QN_ERR_SHAPE;
  if (!dA || !dB) return QN_ERR_NULL;
  if (M > 0 && (!x || !dy || (!u && !A) || (!t && !B))) return QN_ERR_NULL;
  if ((x && !aligned(x, 16)) || (dy && !aligned(dy, 16)) || (A && !aligned(A, 16)) ||
      (B && !aligned(B, 2)) || (u && !aligned(u, 2)) || (t && !aligned(t, 2)) ||
      !aligned(dA, 4) || !aligned(dB, 4))
    return QN_ERR_ALIGN;
  const size_t need = grads_ws(M, N, K, r);
  if (!ws || ws_bytes < need) return QN_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return QN_ERR_ALIGN;
  if (!qn::tables()) return QN_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  (void)hipGetLastError();
  const float scale = alpha / static_cast<float>(r);
  // u and t, when not given, are recomputed as bf16 by the launches the
  // forward and the backward use for u_out and t_out (same splits, same
  // fixed-order sums), so they equal the saved ones bit for bit for M > 16
  // (t at every M)
  char* base = static_cast<char*>(ws);
  const int64_t mp = M > kGemvMaxM ? M : kGemvMaxM + 1;
  uint16_t* u16 = reinterpret_cast<uint16_t*>(base);
  uint16_t* t16 = reinterpret_cast<uint16_t*>(base + lora_bf16_bytes(M, r));
  float* lpart = reinterpret_cast<float*>(base + 2 * lora_bf16_bytes(M, r));
  void* part = base + 2 * lora_bf16_bytes(M, r) + lora_part_bytes(mp, r);
  if (M > 0 && !u) {
    const int ks = qn::skinny_wide_splits(mp, K);
    if (qn::launch_skinny(x, M, K, A, r, 1.0f, lpart, nullptr, nullptr, ks, s) != hipSuccess ||
        qn::launch_lora_reduce(lpart, ks, M * r, 1.0f, u16, nullptr, s) != hipSuccess)
      return QN_ERR_HIP;
  }
  if (M > 0 && !t) {
    const int ks = qn::skinny_wide_splits(mp, N);
    if (qn::launch_skinny(dy, M, N, B, r, 1.0f, lpart, nullptr, nullptr, ks, s, true) != hipSuccess ||
        qn::launch_lora_reduce(lpart, ks, M * r, 1.0f, t16, nullptr, s) != hipSuccess)
      return QN_ERR_HIP;
  }
  return hip_status(qn::launch_grads_impl(x, dy, u ? u : u16, t ? t : t16, M, N, K, r, scale, dA,
                                          dB, part, s));
}

}  // extern "C"
