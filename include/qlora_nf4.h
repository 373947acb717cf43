/*
 * qlora_nf4.h -- C ABI of the QLoRA NF4 hot path for AMD Instinct MI355X
 * (gfx950, CDNA4).
 *
 * What it computes is described on these pages (cited by title, site in
 * brackets, and the page's own section number):
 *   [rkmt] "QLORA技术解析：4-bit量化与LoRA结合，单卡微调百亿大模型" (rkmt.cn)
 *   [czcl] "QLoRA技術解析：4-bit量化與高效微調實戰" (czchanglian.com)
 *   [tgd]  "QLoRA微调" (theguodong.com)
 *   [kwkr] "【79.PythonAI】QLoRA原理深入：4-bit量化+LoRA，24G显存也能微调7B模型" (kwkr.cn)
 *
 * General rules for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, unless a
 *     function says "host".  Tensors are dense, row-major, and 16-byte
 *     aligned.  The library never keeps a pointer after a call returns.
 *   - Every device call is asynchronous on `stream` (a hipStream_t passed
 *     as void*; NULL means the default stream).  No call synchronises.
 *   - Every call returns an int status: QN_OK (0) or a negative QN_ERR_*.
 *     Argument errors are found on the host before anything is launched;
 *     when one is returned nothing was launched and no output was touched.
 *     QN_ERR_HIP means a launch failed (hipGetLastError after the launch);
 *     outputs are then undefined.  No C++ exception crosses the ABI.
 *   - The library allocates no device memory.  Scratch space comes from a
 *     caller-provided workspace sized by qn_workspace_bytes().  One
 *     workspace serves every operation, but calls that may run at the same
 *     time (on different streams) need workspaces of their own.
 *   - Inputs must be finite.  NaN or Inf in a weight or activation gives
 *     undefined (but memory-safe) results.
 *   - Calls are thread-safe; the only global state is a read-only table
 *     built once on first use.
 *   - Only block size 64 and double-quantisation group 256 are built; other
 *     values return QN_ERR_UNSUPPORTED.  fp16 compute is not offered: the
 *     pages require bf16 ([rkmt] §3.2, [kwkr] §4.1).
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define QN_API __attribute__((visibility("default")))
#else
#define QN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define QN_OK                0
#define QN_ERR_NULL         -1  /* a required pointer is NULL              */
#define QN_ERR_SHAPE        -2  /* a size is negative, odd or inconsistent */
#define QN_ERR_ALIGN        -3  /* a pointer is not 16-byte aligned        */
#define QN_ERR_UNSUPPORTED  -4  /* valid request this build does not offer */
#define QN_ERR_WORKSPACE    -5  /* workspace missing or too small          */
#define QN_ERR_HIP          -6  /* a HIP launch failed                      */

/* element types */
#define QN_F32   0
#define QN_BF16  1

/* operation ids for qn_workspace_bytes */
#define QN_OP_FWD         0
#define QN_OP_BWD_DX      1
#define QN_OP_LORA_GRADS  2
#define QN_OP_BWD_DX_DROPOUT 3

typedef uint16_t qn_bf16; /* bf16 bit pattern */

/* code table of the 4-bit weight (qn_weight.quant_type) */
#define QN_NF4  0
#define QN_FP4  1
/* level-2 code of the block constants (qn_weight.scale_type) */
#define QN_SCALE_U8   0
#define QN_SCALE_FP8  1
#define QN_SCALE_CENTRED 2

/*
 * A quantised weight W[N, K] (N = out_features, K = in_features).
 *   packed  uint8[N*K/2]: 4-bit codes of the row-major flattening of W, two
 *           per byte, the even element in the high nibble.
 *   qscale  uint8[N*K/64]: 8-bit code of each block constant, or NULL when
 *           the weight is not double-quantised.
 *   gscale  fp32[ceil((N*K/64)/256)]: one constant per 256 blocks; required
 *           iff qscale != NULL.
 *   absmax  fp32[N*K/64]: the block constants themselves; used iff
 *           qscale == NULL.
 *   blocksize must be 64 and group 256.  The linear ops (and lora_grads)
 *   need N and K to be positive multiples of 64, so a block never crosses a
 *   row; other sizes return QN_ERR_SHAPE.
 *   quant_type  QN_NF4 (the NF4 table of nf4_codebook) or QN_FP4 (that of
 *           fp4_codebook); the codes must come from the matching quantiser.
 *   scale_type  QN_SCALE_U8 (qscale from dq_quantize_scales),
 *           QN_SCALE_FP8 (from dq_quantize_scales_fp8) or QN_SCALE_CENTRED
 *           (from dq_quantize_scales_centred); ignored when qscale == NULL.
 *           Other values return QN_ERR_UNSUPPORTED.  A zero-initialised
 *           struct means NF4 with the uint8 code.
 *   offset  device fp32[1]: the mean subtracted by the centred code;
 *           required (QN_ERR_NULL) iff qscale != NULL and scale_type ==
 *           QN_SCALE_CENTRED, ignored otherwise.
 */
typedef struct qn_weight {
  const uint8_t* packed;
  const uint8_t* qscale;
  const float* gscale;
  const float* absmax;
  int64_t N;
  int64_t K;
  int32_t blocksize;
  int32_t group;
  int32_t quant_type;
  int32_t scale_type;
  const float* offset;
} qn_weight;

/* Human-readable text for a status code (static storage, never NULL). */
QN_API const char* qn_status_string(int status);

/*
 * nf4_codebook -- HOST function.  Writes the 16 NF4 code points (ascending,
 * fp32) to out[16].
 * [kwkr] §2.2: the codes are standard-normal quantiles, dense near zero and
 * sparse in the tails; [rkmt] §2.2.1: quantiles of a truncated normal that
 * split the area into equal parts; [czcl] §2.1: zero is represented exactly.
 * Built in fp64 as 7 negative quantiles, 0 and 8 positive quantiles of the
 * normal truncated at probability 1 - (1/32 + 1/30)/2, divided by the
 * largest, then rounded to fp32: out[0] = -1, out[7] = +0, out[15] = +1.
 * Returns QN_ERR_NULL if out is NULL.
 */
QN_API int nf4_codebook(float out[16]);

/*
 * nf4_quantize -- blockwise absmax NF4 quantisation of numel weights.
 * [rkmt] §2.2.1-2.2.2, [kwkr] §3.1: blocks of 64 weights, one fp32 constant
 * (the block's max |w|) each, every weight normalised by it and mapped to
 * the nearest code point; only the 4-bit index is stored.
 *   w        device, numel elements of type dtype (QN_F32 or QN_BF16), the
 *            row-major flattening of the weight.
 *   numel    even, >= 0; the last block may be partial.
 *   packed   device uint8[numel/2] out.
 *   absmax   device fp32[ceil(numel/blocksize)] out.
 * Code of w: nearest code to fl32(w / absmax) (IEEE fp32 division), ties to
 * the lower code; an all-zero block stores code 7 (exact zero).  Results
 * are bit-identical on every run and on every device.
 */
QN_API int nf4_quantize(const void* w, int32_t dtype, int64_t numel, int32_t blocksize,
                 uint8_t* packed, float* absmax, void* stream);

/*
 * dq_quantize_scales -- double quantisation of the block constants.
 * [rkmt] §2.2.2, [kwkr] §3.1, [tgd] §2: the fp32 block constants are
 * quantised again to 8 bits, with fp32 constants for that second level,
 * saving about 0.37 bit per weight.
 *   absmax   device fp32[nblocks] in (non-negative, finite).
 *   qscale   device uint8[nblocks] out: nearest level of fl32(q/255),
 *            q = 0..255, to fl32(absmax / gscale), ties to the lower code.
 *   gscale   device fp32[ceil(nblocks/group)] out: max of each group of 256.
 */
QN_API int dq_quantize_scales(const float* absmax, int64_t nblocks, int32_t group,
                       uint8_t* qscale, float* gscale, void* stream);

/*
 * fp4_codebook -- HOST function.  Writes the 16 FP4 code points (ascending,
 * fp32) to out[16].  [kwkr] §4.1 names fp4 as the alternative 4-bit type
 * (made for floating-point distributions; worse than NF4 for weights)
 * without a format: taken as E2M1 (magnitudes 0, 1/2, 1, 3/2, 2, 3, 4, 6)
 * divided by 6, negatives mirrored, +0 at both out[7] and out[8]; each
 * value is the fp32 nearest to the exact ratio.  QN_ERR_NULL if out is NULL.
 */
QN_API int fp4_codebook(float out[16]);

/*
 * fp4_quantize -- nf4_quantize with the FP4 table: same arguments, layout,
 * block constants and errors; code = index of the nearest entry of
 * fp4_codebook (ties to the lower index, so v <= 0 within the zero bin
 * takes code 7 and v > 0 code 8, both +0).  Use quant_type = QN_FP4.
 */
QN_API int fp4_quantize(const void* w, int32_t dtype, int64_t numel, int32_t blocksize,
                        uint8_t* packed, float* absmax, void* stream);

/*
 * dq_quantize_scales_fp8 -- dq_quantize_scales with an FP8 level-2 code.
 * [kwkr] §3.1 compresses the fp32 block constants to fp8: here the ratio
 * v = fl32(c / c2) in [0, 1] (c2 the group max, stored in gscale as for the
 * uint8 code) is stored as the nearest E4M3 number (4 exponent bits, bias
 * 7, 3 mantissa bits, subnormals below 2^-6), ties to the even code; the
 * dequantised constant is fl32(value * c2).  Same arguments and errors as
 * dq_quantize_scales; use scale_type = QN_SCALE_FP8.
 */
QN_API int dq_quantize_scales_fp8(const float* absmax, int64_t nblocks, int32_t group,
                                  uint8_t* qscale, float* gscale, void* stream);

/*
 * nf4_quantize_dq -- nf4_quantize (or fp4_quantize) and dq_quantize_scales
 * (or dq_quantize_scales_fp8) in one call: [rkmt] §2.2.1-2.2.2 and [kwkr]
 * §3.1, the 4-bit codes and the 8-bit codes of their block constants.
 * Same packed, qscale and gscale bytes as the two calls, bit for bit; one
 * pass over the weight, no round trip of the constants through memory.
 *   quant_type  QN_NF4 or QN_FP4;  scale_type QN_SCALE_U8 or QN_SCALE_FP8
 *               (the centred code needs the mean of all constants first:
 *               QN_ERR_UNSUPPORTED here, use dq_quantize_scales_centred).
 *   absmax  fp32[ceil(numel/64)] out (the block constants), or NULL to
 *           skip writing them.
 * Other arguments and errors as nf4_quantize and dq_quantize_scales.
 */
QN_API int nf4_quantize_dq(const void* w, int32_t dtype, int64_t numel, int32_t blocksize,
                           int32_t group, int32_t quant_type, int32_t scale_type,
                           uint8_t* packed, float* absmax, uint8_t* qscale, float* gscale,
                           void* stream);

/*
 * nf4_quantize_dq_batch -- nf4_quantize_dq over n weights in one launch,
 * for callers that quantise many weights at once (the projections of a
 * layer, a model at load time): [rkmt] §2.2.1-2.2.2 and [kwkr] §3.1 per
 * weight, as in nf4_quantize_dq.  Entry i is the weight w[i] of numel[i]
 * elements with its own outputs packed[i], qscale[i], gscale[i] and
 * absmax[i] (absmax itself may be NULL: no constants written for any
 * entry; a NULL absmax[i] skips entry i's).  All entries share dtype,
 * quant_type and scale_type.  The bytes written equal those of n separate
 * nf4_quantize_dq calls, bit for bit; outputs of different entries must
 * not overlap.  The host arrays are read during the call only.
 *   n  0..8 (QN_ERR_SHAPE otherwise); entries with numel[i] == 0 are
 *      skipped (their pointers are not read).
 * Other arguments and errors as nf4_quantize_dq, checked for every entry
 * before anything runs.
 */
QN_API int nf4_quantize_dq_batch(int32_t n, const void* const* w, const int64_t* numel,
                                 int32_t dtype, int32_t blocksize, int32_t group,
                                 int32_t quant_type, int32_t scale_type, uint8_t* const* packed,
                                 float* const* absmax, uint8_t* const* qscale,
                                 float* const* gscale, void* stream);

/*
 * dq_quantize_scales_centred -- mean-centred double quantisation.
 * [rkmt] §2.2.2 and [kwkr] §3.1 quantise the block constants to 8 bits a
 * second time; the publication the pages summarise subtracts the constants'
 * mean first so that a symmetric signed code serves them.  Here:
 *   mu = fl32(S / nblocks), S the fp64 sum of the constants by adjacent
 *        pairs (zero-padded to a power of two, added 0+1, 2+3, ... level by
 *        level): one fixed order, bit-reproducible;
 *   d = fl32(c - mu); per group of 256, gscale = max |d|;
 *   qscale = k as a two's-complement byte, k in -127..127 the nearest level
 *        fl32(k / 127) to fl32(d / gscale) (ties toward k = 0; 0 when
 *        gscale == 0);
 *   the dequantised constant is fl32(fl32(fl32(k / 127) * gscale) + mu).
 *   absmax  device fp32[nblocks] in;  qscale uint8[nblocks] out;
 *   gscale  fp32[ceil(nblocks/256)] out (also scratch during the call);
 *   offset  device fp32[1] out (mu).  4-byte alignment suffices.
 * Use scale_type = QN_SCALE_CENTRED and qn_weight.offset = offset.  Other
 * errors as dq_quantize_scales; nblocks == 0 writes nothing.
 */
QN_API int dq_quantize_scales_centred(const float* absmax, int64_t nblocks, int32_t group,
                                      uint8_t* qscale, float* gscale, float* offset,
                                      void* stream);

/*
 * nf4_dequant -- materialise the weight.
 * [rkmt] §2.2.1: look the 4-bit index up in the code table and scale it;
 * [kwkr] §2.3: the 16-bit copy is a compute-time value.
 *   out      device [N, K] of out_dtype (QN_F32 or QN_BF16), 16-byte
 *            aligned.  N * K must be a multiple of 32 (QN_ERR_SHAPE
 *            otherwise: a thread expands whole 32-code runs); N and K need
 *            not be multiples of 64 (a block may cross a row).
 * Value: c' = fl32(fl32(q/255) * gscale) (or absmax when not
 * double-quantised), w = fl32(code_value * c'); bf16 output is the RNE of
 * that fp32.  Bit-identical to the definition, including -0.0.
 */
QN_API int nf4_dequant(const qn_weight* w, int32_t out_dtype, void* out, void* stream);

/*
 * qn_workspace_bytes -- HOST function.  Bytes of device workspace that op
 * (QN_OP_FWD, QN_OP_BWD_DX, QN_OP_LORA_GRADS or QN_OP_BWD_DX_DROPOUT)
 * needs for these sizes.
 * Returns 0 for invalid arguments.  The forward and backward keep the LoRA
 * projection (x A^T or dy B) there as fp32 partial sums over slices of the
 * contraction (at most 512 slices for M <= 16, 16 above), which are added
 * up in a fixed order, so results are bit-reproducible.
 */
QN_API size_t qn_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K, int32_t r);

/*
 * qlora_linear_fwd -- y = x * dequant(W)^T + (alpha/r) * (x * A^T) * B^T.
 * [kwkr] §2.3: the 4-bit weight is expanded to 16 bits for the product and
 * never stored back; [rkmt] §2.1 and §3.3: LoRA bypass B*A scaled by
 * alpha/r.  bf16 operands, fp32 accumulation, bf16 output.
 *   x      device bf16[M, K];  A bf16[r, K];  B bf16[N, r].
 *   y      device bf16[M, N] out.
 *   u_out  device bf16[M, r] out (x * A^T, kept for the backward), or NULL.
 *   r      0 (frozen layer: A, B ignored) or 1..128.  A == B == NULL with
 *          r > 0 is the frozen layer too (no workspace needed, u_out left
 *          untouched); exactly one of them NULL with r > 0 is QN_ERR_NULL.
 *   ws     device workspace of ws_bytes >= qn_workspace_bytes(QN_OP_FWD,..).
 */
QN_API int qlora_linear_fwd(const qn_weight* w, const qn_bf16* x, int64_t M,
                     const qn_bf16* A, const qn_bf16* B, int32_t r, float alpha,
                     qn_bf16* y, qn_bf16* u_out, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * qn_hbm_read_probe -- a measurement aid, not an operation of the method:
 * reads `bytes` bytes of device memory at buf with 16-byte loads (2048
 * workgroups, a grid-stride loop) and discards them, so its duration gives
 * the streaming-read rate that the HBM-bound kernels are measured against.
 *   buf   device, 16-byte aligned;  bytes a multiple of 16 (QN_ERR_SHAPE).
 *   sink  device uint32[1]; written only when the XOR of all the data equals
 *         a fixed sentinel (it keeps the loads from being optimised away).
 */
QN_API int qn_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/*
 * qlora_linear_fwd_noalloc -- qlora_linear_fwd without a workspace
 * argument, for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, hosts that forbid allocation).
 * Same arguments (minus ws, ws_bytes), same kernels and the same results
 * bit for bit.  The workspace is a fixed 64 MiB array inside the library,
 * one per GPU, created when the library is first used on that GPU and held
 * until the process ends; this call allocates nothing.  Sizes whose
 * forward workspace (qn_workspace_bytes(QN_OP_FWD, M, N, K, r)) exceeds
 * 64 MiB return QN_ERR_WORKSPACE before anything runs (r = 64: M up to
 * 15887 tokens; r = 128: 7943).  The first call on a device resolves that
 * device's array address (hipGetSymbolAddress, with the stream's device
 * made current for it and the caller's device restored); make it once
 * before capturing a graph.  Every call on one GPU
 * shares its array and nothing in it needs to start at zero, but calls
 * that may overlap on one GPU (different streams, or threads without
 * ordering) race on it and must be serialised by the caller.
 */
QN_API int qlora_linear_fwd_noalloc(const qn_weight* w, const qn_bf16* x, int64_t M,
                                    const qn_bf16* A, const qn_bf16* B, int32_t r,
                                    float alpha, qn_bf16* y, qn_bf16* u_out, void* stream);

/*
 * qlora_linear_bwd_dx -- dx = dy * dequant(W) + (alpha/r) * (dy * B) * A.
 * [kwkr] §2.3: the gradient flows through the frozen 4-bit weight to the
 * input and into the LoRA bypass only.
 *   dy     device bf16[M, N];  dx device bf16[M, K] out.
 *   t_out  device bf16[M, r] out (dy * B), or NULL.
 *   r == 0, or A == B == NULL, is the frozen layer (as in qlora_linear_fwd).
 */
QN_API int qlora_linear_bwd_dx(const qn_weight* w, const qn_bf16* dy, int64_t M,
                        const qn_bf16* A, const qn_bf16* B, int32_t r, float alpha,
                        qn_bf16* dx, qn_bf16* t_out, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * qlora_merge -- out = bf16(dequant(W) + (alpha/r) B A), the merged 16-bit
 * weight.  [rkmt] §2.1: for inference the adapter is folded into the
 * weight (W <- W + B A, no added latency); [tgd] §7: a QLoRA adapter is
 * merged into a 16-bit weight, never into the 4-bit form.  W is the
 * dequantised NF4 weight the adapter was trained against; re-quantise the
 * result with nf4_quantize for a merged 4-bit model.
 *   A bf16[r, K], B bf16[N, r] (device; ignored when r == 0).
 *   out device bf16[N, K], 16-byte aligned, overwritten.  Per element: the
 *   rank-r product of the bf16 operands accumulated in fp32 (MFMA), scaled
 *   by alpha/r in fp32, added to the fp32 dequantised weight, then rounded
 *   to bf16 (nearest even); r == 0 writes bf16(dequant(W)) exactly.
 *   r must be 0..128; A == B == NULL with r > 0 is taken as r == 0.  N and
 *   K must be positive multiples of 64.
 */
QN_API int qlora_merge(const qn_weight* w, const qn_bf16* A, const qn_bf16* B, int32_t r,
                       float alpha, qn_bf16* out, void* stream);

/*
 * lora_grads -- dA = (alpha/r) (dy B)^T x,  dB = (alpha/r) dy^T (x A^T).
 * [kwkr] §2.3: only the LoRA matrices receive gradients; the 4-bit weight
 * and its constants get none.
 *   x bf16[M, K], dy bf16[M, N], A bf16[r, K], B bf16[N, r] (device).
 *   u bf16[M, r] (x A^T, the forward's u_out) or NULL to recompute it;
 *   t bf16[M, r] (dy B, the backward's t_out) or NULL to recompute it.
 *   A recomputed u or t is the bf16 value the forward or backward returns
 *   in u_out / t_out (same launches and summation order), so both ways
 *   give the same dA (any M) and dB (M > 16) bit for bit when the given
 *   u and t are 16-byte aligned (as the library's own workspace copies are).
 *   ws     device workspace of ws_bytes >= qn_workspace_bytes(QN_OP_LORA_GRADS,..).
 *   dA fp32[r, K] and dB fp32[N, r] out (overwritten, not accumulated).
 *   r must be 1..128.  The sum over M is taken in a fixed order, so results
 *   are bit-reproducible: with r % 8 == 0 and u, t 16-byte aligned one
 *   launch, each workgroup summing all M tokens for its columns; otherwise
 *   fixed token chunks whose partial sums (in ws) a second launch adds.
 */
QN_API int lora_grads(const qn_bf16* x, const qn_bf16* dy, const qn_bf16* u,
               const qn_bf16* t, const qn_bf16* A, const qn_bf16* B,
               int64_t M, int64_t N, int64_t K, int32_t r, float alpha,
               float* dA, float* dB, void* ws, size_t ws_bytes, void* stream);

/*
 * lora_dropout -- the dropped input of the LoRA branch, x * keep / (1 - p).
 * [rkmt] §3.3 gives the LoRA layer a dropout rate (0.1; [czcl] §3.2 and
 * [kwkr] §4 use 0.05); it acts on the adapter's input only, the frozen
 * path sees x.  The keep mask is a pure function of (seed, m, k), so the
 * backward regenerates it: element (m, k) uses the Philox4x64-10 block
 * (Salmon et al., SC 2011) at counter (k, m / 8, 0, 0), key (seed, 0); row
 * m % 8 reads the 32-bit half (m % 8) % 2 (low first) of 64-bit word
 * (m % 8) / 2 and is kept iff it is >= floor(p * 2^32).
 *   x       device bf16[M, K], 16-byte aligned; K % 8 == 0.
 *   x_drop  device bf16[M, K] out, 16-byte aligned, not overlapping x.
 *           Kept: bf16(fl32(x * fl32(1 / (1 - p)))); dropped: +0.
 *   p       0 <= p < 1 (else QN_ERR_SHAPE); p = 0 copies x bit for bit.
 * Feed x_drop to qlora_linear_fwd_dropout and, as its x, to lora_grads.
 * Use a distinct seed per layer and step.
 */
QN_API int lora_dropout(const qn_bf16* x, int64_t M, int64_t K, float p, uint64_t seed,
                        qn_bf16* x_drop, void* stream);

/*
 * qlora_linear_fwd_dropout -- y = x * dequant(W)^T + (alpha/r) *
 * (x_drop * A^T) * B^T: the forward with LoRA dropout ([rkmt] §3.3), the
 * base product on x and the adapter on x_drop (from lora_dropout).
 * Arguments, workspace (QN_OP_FWD) and errors as qlora_linear_fwd; x_drop
 * is device bf16[M, K], 16-byte aligned; u_out receives x_drop * A^T.
 */
QN_API int qlora_linear_fwd_dropout(const qn_weight* w, const qn_bf16* x,
                                    const qn_bf16* x_drop, int64_t M, const qn_bf16* A,
                                    const qn_bf16* B, int32_t r, float alpha, qn_bf16* y,
                                    qn_bf16* u_out, void* ws, size_t ws_bytes, void* stream);

/*
 * qlora_linear_bwd_dx_dropout -- dx = dy * dequant(W) + D * ((alpha/r) *
 * (dy * B) * A), D = keep / (1 - p) with the mask of lora_dropout for the
 * same (p, seed) regenerated in place: the chain rule through the dropped
 * adapter input ([rkmt] §3.3; [kwkr] §2.3).  The base product dy * W is
 * kept in fp32 in the workspace and the masked LoRA term is added to it
 * before the one rounding to bf16, as on the plain path.
 * Workspace: ws_bytes >= qn_workspace_bytes(QN_OP_BWD_DX_DROPOUT, ..), the
 * backward's workspace plus M * K fp32.  Arguments and errors as
 * qlora_linear_bwd_dx; p outside [0, 1) is QN_ERR_SHAPE.
 */
QN_API int qlora_linear_bwd_dx_dropout(const qn_weight* w, const qn_bf16* dy, int64_t M,
                                       const qn_bf16* A, const qn_bf16* B, int32_t r,
                                       float alpha, float p, uint64_t seed, qn_bf16* dx,
                                       qn_bf16* t_out, void* ws, size_t ws_bytes, void* stream);

/*
 * lora_adamw_step -- one AdamW step on a LoRA matrix (A or B), in place.
 * [rkmt] §3.5, [czcl] §3.2: the adapter is trained with AdamW (32-bit
 * states, learning rate 2e-4), the only trainable parameters being A and
 * B.  Decoupled weight decay, per element in fp32:
 *   p <- p (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;
 *   p <- p - (lr / (1 - b1^step)) m / (sqrt(v) / sqrt(1 - b2^step) + eps)
 * (the bias corrections computed on the host in fp64).
 *   p, m, v  device fp32[n], updated in place; g device fp32[n] (dA or dB
 *            from lora_grads).  16-byte aligned.
 *   p_bf16   device bf16[n] out (the new p rounded to bf16, the operand of
 *            the next forward), 8-byte aligned, or NULL.
 *   step     1 for the first step.  lr >= 0, 0 <= b1, b2 < 1, eps > 0,
 *            weight_decay >= 0, else QN_ERR_SHAPE.
 * The paged optimizer of the pages (host unified memory) is not part of it.
 */
QN_API int lora_adamw_step(float* p, const float* g, float* m, float* v, qn_bf16* p_bf16,
                           int64_t n, float lr, float beta1, float beta2, float eps,
                           float weight_decay, int32_t step, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
