// Fused dequant -> bf16 MFMA GEMMs for token batches (gfx950).
//
// Forward  y[M, N]  = x[M, K] W^T + (s u)[M, r] B^T      (contraction over K)
// Backward dx[M, K] = dy[M, N] W  + (s t)[M, r] A        (contraction over N)
//
// [kwkr "QLoRA原理深入" §2.3] the 4-bit weight is expanded to 16 bits for the
// matrix product and never written back; [rkmt "QLORA技术解析" §3.2] compute
// type bf16.  The weight tile is dequantised straight into LDS as
// bf16(fl32(q[code] * c')), the same bf16 value nf4_dequant produces, and
// never exists in HBM in 16-bit form.  The LoRA term rides on the same
// accumulators as one extra contraction of depth r: the A-side operand is
// bf16(s u) (or bf16(s t)), the B-side operand is B (or A^T).
//
// Tiling.  Workgroup tile BM x BN = 256 x 128, K step 64 (one quantisation
// block), one workgroup of 8 waves per CU.  The waves are specialised, one
// of each kind per SIMD:
//   * waves 0-3 run the 32x32x16 bf16 MFMAs (2 x 2 grid of 128 x 64 wave
//     tiles) and bring in the activation tile by direct-to-LDS DMA two K
//     steps ahead (three activation buffers, 128-byte rows with an XOR
//     swizzle instead of padding, so each 1 KB DMA fills whole rows and the
//     fragment reads stay free of bank conflicts);
//   * waves 4-7 load the 4-bit weight and its constants three steps ahead
//     (a ring of four register sets) and dequantise one step ahead into the
//     other of two weight buffers.
// One barrier per K step.  The 256-row tile halves the dequantisation per
// flop against 128 rows, and moving the activation copy to DMA leaves the
// producer waves only the dequantisation.  All global loads are
// unconditional (edge rows re-read a valid row), which keeps the compiler
// from serialising them behind branches.  A producer lane's 32 codes per
// step lie in one 64-block: it forms the block's 16 products
// bf16(fl32(q[c] c')) and decodes its codes with byte permutes from
// registers, so the LDS carries only the activation DMA, the weight tile
// and the MFMA fragment reads.  The forward stages the weight tile
// row-major ([n][k]); the backward needs 8 consecutive n per MFMA lane, so
// it writes the dequantised tile transposed ([k][n]), as pairs of rows.

#include "qn_device.h"
#include "qn_launch.h"

namespace qn {

namespace {

constexpr int kBM = 256, kBN = 128, kBK = 64;
constexpr int kLD = kBK + 8;    // bf16 per row of the weight tile in LDS (padded by 16 bytes)
constexpr int kTM = kBM / 64, kTN = kBN / 64;  // MFMA tiles per wave (wave tile kBM/2 x kBN/2)
constexpr int kParts = kBK / 16;               // 16-deep MFMA steps per K step
constexpr int kMmaWaves = 4;                   // 2 x 2 grid of MFMA wave tiles
constexpr int kProdWaves = 4;                  // dequantising waves
constexpr int kProd = 64 * kProdWaves;         // producer threads
constexpr int kThreads = 64 * (kMmaWaves + kProdWaves);
constexpr int kCodes = kBN * kBK / kProd;      // weight codes per producer thread per K step
constexpr int kCodeThreads = kBK / kCodes;     // producer threads per weight row (forward)
constexpr int kWords = kCodes / 8;             // their 32-bit words
constexpr int kADma = kBM * kBK * 2 / 1024 / kMmaWaves;  // 1 KB activation DMAs per MFMA wave
static_assert(kWords * 8 == kCodes && kADma * 1024 * kMmaWaves == kBM * kBK * 2, "tile split");

struct GemmArgs {
  const uint8_t* packed;
  const uint8_t* qscale;
  const float* gscale;
  const float* absmax;
  int64_t N, K, M;
  const uint16_t* act;   // x [M, K] (fwd) or dy [M, N] (bwd)
  const uint16_t* lact;  // bf16(s u) or bf16(s t), [M, r]
  const uint16_t* lw;    // B [N, r] (fwd) or A [r, K] (bwd)
  int r;
  uint16_t* out;         // y [M, N] or dx [M, K]
  float* out32;          // if not null: the fp32 result goes here instead of out
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t wvec_t __attribute__((ext_vector_type(kWords)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Registers of one K step of a producer thread: its weight codes (kCodes
// consecutive codes of one block) and their block constant (q8 code +
// group constant, or absmax).
struct Prefetch {
  wvec_t w;
  uint32_t q8;
  float c;
};

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Activation tile layout in LDS: kBM rows of 128 bytes (8 chunks of 16 B),
// chunk c of row r in slot c ^ swz(r).  The swizzle makes the MFMA
// fragment reads (16 lanes = 16 consecutive rows, one chunk) hit 16
// distinct 4-bank groups without padding, so a 1 KB DMA fills 8 whole rows.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Weight loads of contraction step kt (producer thread t):
//   forward: row c0 + t / kCodeThreads, codes k0 + kCodes (t % kCodeThreads) ..
//   backward: row k0 + t % kBK, codes c0 + kCodes (t / kBK) ..
// Weight rows/columns past the output edge re-read a valid one: they only
// feed outputs that are never stored.
template <bool kBwd, bool kDQ>
__device__ __forceinline__ void load_step(const GemmArgs& g, int64_t c0, int kt, Prefetch& pf,
                                          int t) {
  const int64_t k0 = static_cast<int64_t>(kt) * kBK;
  int64_t n, k;
  if constexpr (kBwd) {
    n = k0 + (t % kBK);
    k = c0 + kCodes * (t / kBK);
    k = k < g.K ? k : g.K - kCodes;
  } else {
    n = c0 + t / kCodeThreads;
    k = k0 + kCodes * (t % kCodeThreads);
    n = n < g.N ? n : g.N - 1;
  }
  pf.w = *reinterpret_cast<const wvec_t*>(g.packed + n * (g.K >> 1) + (k >> 1));
  const int64_t bi = n * (g.K >> 6) + (k >> 6);
  if constexpr (kDQ) {
    pf.q8 = g.qscale[bi];
    pf.c = g.gscale[bi >> 8];
  } else {
    pf.q8 = 0;
    pf.c = g.absmax[bi];
  }
}

// Block constant of a prefetched weight chunk.
template <bool kDQ>
__device__ __forceinline__ float chunk_scale(const Prefetch& pf, int kind, float mu) {
  return kDQ ? dq_value(pf.q8, pf.c, kind, mu) : pf.c;
}

// Dequantise one K step of weight codes into the LDS weight tile.  A
// producer lane's 32 codes all belong to one 64-block, so it first forms
// that block's 16 products bf16(fl32(Q[c] cs)) (the same rounding as
// nf4_dequant) and then decodes every code with byte permutes from
// registers: no code-table reads through LDS, whose bandwidth the MFMA
// fragment reads and the activation DMAs already use.
template <bool kBwd>
__device__ __forceinline__ void store_step(const Prefetch& pf, float cs, const CodeParams& P,
                                           uint16_t* __restrict__ sB, int t) {
  // tl[j] / th[j]: low / high bytes of the products of codes 4 j .. 4 j + 3
  uint32_t tl[4], th[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t d0 = pack_bf16x2(__fmul_rn(P.q[4 * j], cs), __fmul_rn(P.q[4 * j + 1], cs));
    const uint32_t d1 = pack_bf16x2(__fmul_rn(P.q[4 * j + 2], cs), __fmul_rn(P.q[4 * j + 3], cs));
    tl[j] = __builtin_amdgcn_perm(d1, d0, 0x06040200u);
    th[j] = __builtin_amdgcn_perm(d1, d0, 0x07050301u);
  }
  // Bytes of c are four codes: look each up in both 8-entry halves (index
  // c & 7), then keep byte k of the low or the high half by bit 3 of c.
  auto look = [&](uint32_t c, uint32_t& lo8, uint32_t& hi8) {
    const uint32_t s7 = c & 0x07070707u;
    const uint32_t half = ((c >> 1) & 0x04040404u) | 0x03020100u;
    lo8 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(tl[3], tl[2], s7),
                                __builtin_amdgcn_perm(tl[1], tl[0], s7), half);
    hi8 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(th[3], th[2], s7),
                                __builtin_amdgcn_perm(th[1], th[0], s7), half);
  };
#pragma unroll
  for (int i = 0; i < kWords; ++i) {
    // byte b of a word holds element 2b (high nibble) and 2b+1 (low nibble)
    const uint32_t word = pf.w[i];
    uint32_t el, eh, ol, oh;
    look((word >> 4) & 0x0F0F0F0Fu, el, eh);  // elements 0, 2, 4, 6
    look(word & 0x0F0F0F0Fu, ol, oh);         // elements 1, 3, 5, 7
    const uint32_t e0 = __builtin_amdgcn_perm(eh, el, 0x05010400u);  // bf16 pair: elements 0, 2
    const uint32_t e1 = __builtin_amdgcn_perm(eh, el, 0x07030602u);  // 4, 6
    const uint32_t o0 = __builtin_amdgcn_perm(oh, ol, 0x05010400u);  // 1, 3
    const uint32_t o1 = __builtin_amdgcn_perm(oh, ol, 0x07030602u);  // 5, 7
    uint32_t d[4];  // d[b]: elements 2b, 2b + 1
    d[0] = __builtin_amdgcn_perm(o0, e0, 0x05040100u);
    d[1] = __builtin_amdgcn_perm(o0, e0, 0x07060302u);
    d[2] = __builtin_amdgcn_perm(o1, e1, 0x05040100u);
    d[3] = __builtin_amdgcn_perm(o1, e1, 0x07060302u);
    if constexpr (kBwd) {
      // Transposed tile sB[column][row]: lane l holds row l (rows are the
      // contraction).  Adjacent lanes swap halves (one DPP move) so the even
      // lane stores rows l, l+1 of column 2b and the odd lane those of
      // column 2b + 1, as one 4-byte store each.
      const int lane = t & 63, qd = t / kBK;
      const uint32_t sel = (lane & 1) ? 0x03020706u : 0x05040100u;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t nb = static_cast<uint32_t>(
            __builtin_amdgcn_mov_dpp(static_cast<int>(d[b]), 0xB1, 0xF, 0xF, false));  // lane l ^ 1
        *reinterpret_cast<uint32_t*>(sB + (kCodes * qd + 8 * i + 2 * b + (lane & 1)) * kLD +
                                     (lane & ~1)) = __builtin_amdgcn_perm(nb, d[b], sel);
      }
    } else {
      *reinterpret_cast<u32x4*>(sB + (t / kCodeThreads) * kLD + kCodes * (t % kCodeThreads) + 8 * i) =
          u32x4{d[0], d[1], d[2], d[3]};
    }
  }
}

// Per-lane byte offsets of an MFMA wave's activation DMAs: DMA j of wave w
// fills rows 64 w + 8 j .. +8; lane L writes slot L % 8 of row 64 w + 8 j +
// L / 8, so it fetches chunk (L % 8) ^ swz(row) of that row.  Rows past M
// re-read row M - 1.
struct ADma {
  uint32_t off[kADma];  // byte offset of the lane's chunk from the tile's row m0, column 0
};

__device__ __forceinline__ ADma adma_offsets(int64_t m0, int64_t M, int64_t L) {
  ADma d;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < kADma; ++j) {
    const int row = 64 * w + 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);
    const int64_t m = m0 + row < M ? row : M - 1 - m0;
    d.off[j] = static_cast<uint32_t>(m * L * 2 + chunk * 16);
  }
  return d;
}

// Issue the activation DMAs of K step kt into buffer `dst` (MFMA waves).
// Written as inline assembly: for a DMA the compiler knows about it waits
// for every outstanding one at each barrier, which would leave no time for
// the DMA of step k + 2.  The MFMA waves issue no other vector-memory
// instruction inside the K loop, so the explicit waits below count exactly
// these DMAs.  M0 holds the wave's LDS destination; lane L writes 16 bytes
// at M0 + 16 L.
__device__ __forceinline__ void adma_issue(const ADma& d, const uint16_t* act_tile, int kt,
                                           uint16_t* dst) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const char* base = reinterpret_cast<const char*>(act_tile) + static_cast<int64_t>(kt) * kBK * 2;
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint16_t*)(dst + 64 * w * kBK)));
#pragma unroll
  for (int j = 0; j < kADma; ++j) {
    const void* src = base + d.off[j];
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds + 8 * j * kBK * 2)
                 : "memory", "m0");
  }
}

// Wait until at most one K step of activation DMAs is outstanding.
__device__ __forceinline__ void adma_wait_one_step() {
  static_assert(kADma == 8, "the wait count below is kADma");
  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
}

// MFMA fragments of one 16-deep step of the wave's tile: activation rows
// from the swizzled tile, weight rows from the padded tile.
struct Frags {
  uint4 a[kTM], b[kTN];
};

__device__ __forceinline__ void load_frags(const uint16_t* __restrict__ sA,
                                           const uint16_t* __restrict__ sB, int kk, Frags& f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, lg = lane >> 5;
  const int aslot = (2 * kk + lg) ^ swz(li);  // wave rows start at multiples of 32
#pragma unroll
  for (int i = 0; i < kTM; ++i)
    f.a[i] = *reinterpret_cast<const uint4*>(sA + (wm * (kBM / 2) + i * 32 + li) * kBK + aslot * 8);
#pragma unroll
  for (int j = 0; j < kTN; ++j)
    f.b[j] = *reinterpret_cast<const uint4*>(sB + (wn * (kBN / 2) + j * 32 + li) * kLD + kk * 16 + 8 * lg);
}

// Rank <= 16 LoRA tiles staged at the start: activation [kBM][16] and weight
// [kBN][16], rows of 32 bytes (a wave's 16-byte fragment reads cover 1 KB
// contiguously: no bank conflicts).
constexpr int kLoraEarly = 16;
constexpr int kLoraPer = (kBM + kBN) * kLoraEarly / kThreads;  // elements per thread

__device__ __forceinline__ void load_frags_lora(const uint16_t* __restrict__ sLA,
                                                const uint16_t* __restrict__ sLW, Frags& f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, lg = lane >> 5;
#pragma unroll
  for (int i = 0; i < kTM; ++i)
    f.a[i] = *reinterpret_cast<const uint4*>(sLA + (wm * (kBM / 2) + i * 32 + li) * kLoraEarly + 8 * lg);
#pragma unroll
  for (int j = 0; j < kTN; ++j)
    f.b[j] = *reinterpret_cast<const uint4*>(sLW + (wn * (kBN / 2) + j * 32 + li) * kLoraEarly + 8 * lg);
}

// acc[i][j] += (weight tile j) (activation tile i)^T: the transposed
// output tile, so a lane's registers run along output columns.
__device__ __forceinline__ void mma_frags(const Frags& f, f32x16_t (&acc)[kTM][kTN]) {
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = mfma32(f.b[j], f.a[i], acc[i][j]);
}

__device__ __forceinline__ void mma_k16(const uint16_t* __restrict__ sA,
                                        const uint16_t* __restrict__ sB, int kk,
                                        f32x16_t (&acc)[kTM][kTN]) {
  Frags f;
  load_frags(sA, sB, kk, f);
  mma_frags(f, acc);
}

// One K step (kParts 16-deep steps) with the fragments of step kk + 1 in
// flight while the MFMAs of step kk run.
__device__ __forceinline__ void mma_step(const uint16_t* __restrict__ sA,
                                         const uint16_t* __restrict__ sB,
                                         f32x16_t (&acc)[kTM][kTN]) {
  static_assert(kParts % 2 == 0, "fragment double buffer");
  Frags f0, f1;
  load_frags(sA, sB, 0, f0);
#pragma unroll
  for (int kk = 0; kk < kParts; kk += 2) {
    load_frags(sA, sB, kk + 1, f1);
    mma_frags(f0, acc);
    if (kk + 2 < kParts) load_frags(sA, sB, kk + 2, f0);
    mma_frags(f1, acc);
  }
}

// Output tile of workgroup `bid` (1-D grid over nr x nc tiles).  Workgroups
// are dealt to the 8 XCDs round-robin (bid % 8) and each XCD has its own
// L2, so when the tile count divides by 8 each XCD gets one contiguous run
// of the tile order below: bands of kBandRows row tiles, column-major
// inside a band.  An XCD then works on two row tiles x a slice of the
// columns: its 32 concurrent tiles share the K window of x and of W, and
// two row tiles of x (2-5.6 MB each at K = 4096-11008) are the most its
// 4 MB L2 can keep between rounds.  Against bands of 4 (measured) this
// fetches about 19% fewer bytes from beyond L2 and runs 1-2% faster;
// bands of 1 re-fetch W per XCD and fetch more.
constexpr int kBandRows = 2;

__device__ __forceinline__ void tile_of(int bid, int nc, int nr, int& row, int& col) {
  const int total = nc * nr;
  int q = bid;
  if ((total & 7) == 0) q = (bid & 7) * (total >> 3) + (bid >> 3);
  const int band = q / (kBandRows * nc);
  const int local = q - band * kBandRows * nc;
  const int rows = nr - band * kBandRows < kBandRows ? nr - band * kBandRows : kBandRows;
  col = local / rows;
  row = band * kBandRows + local % rows;
}

template <bool kBwd, bool kDQ>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmArgs g, CodeParams P) {
  // Three activation buffers (filled by DMA two steps ahead) and two weight
  // buffers (dequantised one step ahead).  Separate arrays, so the compiler
  // can tell a DMA into one activation buffer from reads of another.
  __shared__ __attribute__((aligned(16))) uint16_t sA0[kBM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t sA1[kBM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t sA2[kBM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBN * kLD];
  __shared__ __attribute__((aligned(16))) uint16_t sLA[kBM * kLoraEarly];
  __shared__ __attribute__((aligned(16))) uint16_t sLW[kBN * kLoraEarly];
  const int t = threadIdx.x;

  const int64_t ncols = kBwd ? g.K : g.N;
  const int64_t L = kBwd ? g.N : g.K;  // contraction length
  int trow, tcol;
  tile_of(blockIdx.x, static_cast<int>((ncols + kBN - 1) / kBN),
          static_cast<int>((g.M + kBM - 1) / kBM), trow, tcol);
  const int64_t m0 = static_cast<int64_t>(trow) * kBM;
  const int64_t c0 = static_cast<int64_t>(tcol) * kBN;  // output column tile
  const int nk = static_cast<int>(L / kBK);

  f32x16_t acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // LoRA operands of rank <= 16: loaded here, from clamped in-bounds
  // addresses, and written to sLA / sLW after each role has issued its
  // prologue loads, so their latency overlaps the pipeline start.  Element
  // c < kBM * 16 is lact[m0 + c / 16][c % 16]; the rest is the weight side:
  // B[c0 + n][j] (forward) or A[j][c0 + kcol] (backward).
  const bool early = g.r > 0 && g.r <= kLoraEarly;
  uint32_t lv[kLoraPer];
  uint32_t lok = 0;
  if (early) {
#pragma unroll
    for (int i = 0; i < kLoraPer; ++i) {
      const int ci = i * kThreads;  // thread-independent: which tile
      const int c = ci + t;
      if (ci < kBM * kLoraEarly) {
        const int row = c / kLoraEarly, col = c % kLoraEarly;
        const int64_t m = m0 + row;
        lok |= static_cast<uint32_t>(m < g.M && col < g.r) << i;
        lv[i] = g.lact[(m < g.M ? m : g.M - 1) * g.r + (col < g.r ? col : g.r - 1)];
      } else {
        const int e = c - kBM * kLoraEarly;
        if constexpr (kBwd) {
          const int j = e / kBN, kcol = e % kBN;
          lok |= static_cast<uint32_t>(j < g.r && c0 + kcol < g.K) << i;
          lv[i] = g.lw[static_cast<int64_t>(j < g.r ? j : g.r - 1) * g.K +
                       (c0 + kcol < g.K ? c0 + kcol : g.K - 1)];
        } else {
          const int n = e / kLoraEarly, j = e % kLoraEarly;
          lok |= static_cast<uint32_t>(c0 + n < g.N && j < g.r) << i;
          lv[i] = g.lw[(c0 + n < g.N ? c0 + n : g.N - 1) * g.r + (j < g.r ? j : g.r - 1)];
        }
      }
    }
  }
  auto store_lora = [&]() {
    if (!early) return;
#pragma unroll
    for (int i = 0; i < kLoraPer; ++i) {
      const int ci = i * kThreads;
      const int c = ci + t;
      const uint16_t val = (lok >> i) & 1u ? static_cast<uint16_t>(lv[i]) : uint16_t{0};
      if (ci < kBM * kLoraEarly) {
        sLA[c] = val;
      } else {
        const int e = c - kBM * kLoraEarly;
        if constexpr (kBwd)
          sLW[(e % kBN) * kLoraEarly + e / kBN] = val;
        else
          sLW[e] = val;
      }
    }
  };

  // Waves 0-3 run the MFMAs and fetch the activation tiles by DMA; waves
  // 4-7 load and dequantise the weight.  Per K step k: the MFMA waves
  // consume activation buffer k % 3 and weight buffer k % 2, and start the
  // DMA of step k + 2; the producers dequantise step k + 1 (loaded three
  // steps earlier, a ring of four register sets) into the other weight
  // buffer.
  // One barrier per K step.  Steps past the end re-load the last step; what
  // they store is never read.
  if (t >= 64 * kMmaWaves) {
    const int pt = t - 64 * kMmaWaves;
    const float mu = kDQ ? l2_offset(P) : 0.0f;
    Prefetch p0, p1, p2, p3;
    load_step<kBwd, kDQ>(g, c0, 0, p0, pt);
    load_step<kBwd, kDQ>(g, c0, nk > 1 ? 1 : nk - 1, p1, pt);
    load_step<kBwd, kDQ>(g, c0, nk > 2 ? 2 : nk - 1, p2, pt);
    load_step<kBwd, kDQ>(g, c0, nk > 3 ? 3 : nk - 1, p3, pt);
    store_lora();
    __syncthreads();  // the LoRA tiles visible
    store_step<kBwd>(p0, chunk_scale<kDQ>(p0, P.l2, mu), P, sB[0], pt);
    __syncthreads();
    auto step = [&](int k, Prefetch& dec, Prefetch& ld) {
      const int kl = k + 4 < nk ? k + 4 : nk - 1;
      // Pin the first use of the registers loaded three steps ago here, after
      // the barrier, so the compiler cannot hoist their address arithmetic
      // next to the loads it has just issued and wait for those.
      asm volatile("" : "+v"(dec.w), "+v"(dec.q8), "+v"(dec.c));
      const float cs = chunk_scale<kDQ>(dec, P.l2, mu);
      load_step<kBwd, kDQ>(g, c0, kl, ld, pt);
      store_step<kBwd>(dec, cs, P, sB[(k & 1) ^ 1], pt);
      __syncthreads();
    };
    int k = 0;
    for (; k + 3 < nk; k += 4) {
      step(k, p1, p0);
      step(k + 1, p2, p1);
      step(k + 2, p3, p2);
      step(k + 3, p0, p3);
    }
    if (k < nk) step(k, p1, p0);
    if (k + 1 < nk) step(k + 1, p2, p1);
    if (k + 2 < nk) step(k + 2, p3, p2);
  } else {
    const ADma ad = adma_offsets(m0, g.M, L);
    const uint16_t* act_tile = g.act + m0 * L;
    adma_issue(ad, act_tile, 0, sA0);
    adma_issue(ad, act_tile, nk > 1 ? 1 : nk - 1, sA1);
    store_lora();
    __syncthreads();
    adma_wait_one_step();  // step 0 landed
    __syncthreads();
    auto step = [&](int k, const uint16_t* cur, uint16_t* next2) {
      adma_issue(ad, act_tile, k + 2 < nk ? k + 2 : nk - 1, next2);
      mma_step(cur, sB[k & 1], acc);
      adma_wait_one_step();  // step k + 1 landed
      __syncthreads();
    };
    int k = 0;
    for (; k + 2 < nk; k += 3) {
      step(k, sA0, sA2);
      step(k + 1, sA1, sA0);
      step(k + 2, sA2, sA1);
    }
    if (k < nk) step(k, sA0, sA2);
    if (k + 1 < nk) step(k + 1, sA1, sA0);
    // drain the DMAs of the steps past the end before the buffers are reused
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();

  // LoRA contraction of depth r, kBK at a time, through sA0 and sB[0].  Only
  // the dp = ceil16(depth) columns the MFMAs read are filled (zero past r).
  // The elements of both tiles form one list, taken 16 per thread at a time:
  // all 16 loads are issued before the first LDS store, so r <= 16 costs one
  // memory round trip (12 elements per thread) and r = 64 three.
  // Consecutive threads read consecutive elements of a row of lact, B or A.
  constexpr int kBatch = 16;
  if (early) {
    if (t < 64 * kMmaWaves) {
      Frags f;
      load_frags_lora(sLA, sLW, f);
      mma_frags(f, acc);
    }
  }
  for (int j0 = 0; !early && j0 < g.r; j0 += kBK) {
    const int depth = g.r - j0 < kBK ? g.r - j0 : kBK;
    const int dp = (depth + 15) & ~15;
    const int na = kBM * dp, ntot = na + kBN * dp;  // both multiples of kThreads
    for (int base = 0; base < ntot; base += kBatch * kThreads) {
      // loads from clamped, in-bounds addresses; invalid elements are zeroed
      // at the LDS store (no write to a register with a load in flight)
      uint32_t v[kBatch];
      uint32_t ok = 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int ci = base + i * kThreads;  // thread-independent: which tile
        const int c = ci + t;
        if (ci < na) {
          const int row = c / dp, col = c % dp;
          const int64_t m = m0 + row;
          ok |= static_cast<uint32_t>(m < g.M && col < depth) << i;
          v[i] = g.lact[(m < g.M ? m : g.M - 1) * g.r + j0 + (col < depth ? col : depth - 1)];
        } else if (ci < ntot) {
          const int e = c - na;
          if constexpr (kBwd) {  // A[j0 + j][c0 + kcol]
            const int j = e / kBN, kcol = e % kBN;
            ok |= static_cast<uint32_t>(j < depth && c0 + kcol < g.K) << i;
            v[i] = g.lw[static_cast<int64_t>(j0 + (j < depth ? j : depth - 1)) * g.K +
                        (c0 + kcol < g.K ? c0 + kcol : g.K - 1)];
          } else {               // B[c0 + n][j0 + j]
            const int n = e / dp, j = e % dp;
            ok |= static_cast<uint32_t>(c0 + n < g.N && j < depth) << i;
            v[i] = g.lw[(c0 + n < g.N ? c0 + n : g.N - 1) * g.r + j0 + (j < depth ? j : depth - 1)];
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int ci = base + i * kThreads;
        const int c = ci + t;
        const uint16_t val = (ok >> i) & 1u ? static_cast<uint16_t>(v[i]) : uint16_t{0};
        if (ci < na) {
          const int row = c / dp, col = c % dp;
          sA0[row * kBK + (((col >> 3) ^ swz(row)) << 3) + (col & 7)] = val;
        } else if (ci < ntot) {
          const int e = c - na;
          if constexpr (kBwd)  // sB[kcol][j]
            sB[0][(e % kBN) * kLD + e / kBN] = val;
          else                 // sB[n][j]
            sB[0][(e / dp) * kLD + e % dp] = val;
        }
      }
    }
    __syncthreads();
    if (t < 64 * kMmaWaves)
      for (int kk = 0; kk < dp >> 4; ++kk) mma_k16(sA0, sB[0], kk, acc);
    __syncthreads();
  }
  if (t >= 64 * kMmaWaves) return;

  // Epilogue.  The MFMAs take the weight fragment as their first operand,
  // so each 32 x 32 tile holds the transposed product: lane (li, lg) holds
  // token row li, output columns 8 q + 4 lg + [0, 4) in registers
  // 4 q .. 4 q + 3.  With a 16-byte aligned y whose rows are whole 16-byte
  // chunks, each wave stages its tile in LDS and stores whole 128-byte row
  // segments (8 rows per instruction): 1.4-5.3% faster per launch than
  // storing the registers' 8-byte runs directly (32 rows x 16 bytes per
  // instruction), which remains for other y.  One 2-byte store per register
  // was 3-6 us slower again.
  {
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 31, lg = lane >> 5;
    if (g.out32) {
      // fp32 result (a later pass adds to it and rounds once): each lane's
      // four adjacent columns as one 16-byte store (ncols % 64 == 0)
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t m = m0 + wm * (kBM / 2) + i * 32 + li;
            const int64_t n = c0 + wn * (kBN / 2) + j * 32 + 8 * q + 4 * lg;
            if (m < g.M && n < ncols)
              *reinterpret_cast<float4*>(g.out32 + m * ncols + n) =
                  make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                              acc[i][j][4 * q + 3]);
          }
      return;
    }
    const bool vec16 = (ncols & 7) == 0 && (reinterpret_cast<uintptr_t>(g.out) & 15) == 0;
    if (vec16) {
      // stage the wave's 128 x 64 tile in LDS (the activation buffers and
      // weight buffer 0 are free now), then write whole 128-byte row
      // segments: 8 rows per 16-byte store instruction
      constexpr int kSP = kBN / 2 + 8;  // staged row pitch in bf16
      uint16_t* stg = wave == 0 ? sA0 : wave == 1 ? sA1 : wave == 2 ? sA2 : sB[0];
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = i * 32 + li, col = j * 32 + 8 * q + 4 * lg;
            *reinterpret_cast<uint2*>(stg + row * kSP + col) =
                make_uint2(pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                           pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
          }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int s = 0; s < (kBM / 2) * (kBN / 2) / 8 / 64; ++s) {
        const int row = s * 8 + (lane >> 3), ch = lane & 7;
        const uint4 v = *reinterpret_cast<const uint4*>(stg + row * kSP + ch * 8);
        const int64_t m = m0 + wm * (kBM / 2) + row;
        const int64_t n = c0 + wn * (kBN / 2) + ch * 8;
        if (m < g.M && n < ncols) *reinterpret_cast<uint4*>(g.out + m * ncols + n) = v;
      }
      return;
    }
    const bool vec = (ncols & 3) == 0 && (reinterpret_cast<uintptr_t>(g.out) & 7) == 0;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t m = m0 + wm * (kBM / 2) + i * 32 + li;
          const int64_t n = c0 + wn * (kBN / 2) + j * 32 + 8 * q + 4 * lg;
          const uint32_t lo = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
          const uint32_t hi = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          if (m < g.M) {
            if (vec) {
              if (n < ncols) *reinterpret_cast<uint2*>(g.out + m * ncols + n) = make_uint2(lo, hi);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (n + e < ncols)
                  g.out[m * ncols + n + e] = static_cast<uint16_t>(((e < 2 ? lo : hi) >> (16 * (e & 1))) & 0xFFFF);
            }
          }
        }
  }
}


}  // namespace

hipError_t launch_gemm_fwd(const WeightView& w, const uint16_t* x, int64_t M,
                           const uint16_t* us, const uint16_t* B, int r, uint16_t* y,
                           hipStream_t st) {
  if (M == 0 || w.N == 0) return hipSuccess;
  GemmArgs g{w.packed, w.qscale, w.gscale, w.absmax, w.N, w.K, M, x, us, B, r, y, nullptr};
  const dim3 grid(static_cast<uint32_t>(((w.N + kBN - 1) / kBN) * ((M + kBM - 1) / kBM)));
  if (w.qscale)
    hipLaunchKernelGGL((gemm_kernel<false, true>), grid, dim3(kThreads), 0, st, g, code_params(w));
  else
    hipLaunchKernelGGL((gemm_kernel<false, false>), grid, dim3(kThreads), 0, st, g, code_params(w));
  return hipGetLastError();
}

hipError_t launch_gemm_bwd(const WeightView& w, const uint16_t* dy, int64_t M,
                           const uint16_t* ts, const uint16_t* A, int r, uint16_t* dx,
                           hipStream_t st, float* dx32) {
  if (M == 0 || w.K == 0) return hipSuccess;
  GemmArgs g{w.packed, w.qscale, w.gscale, w.absmax, w.N, w.K, M, dy, ts, A, r, dx, dx32};
  const dim3 grid(static_cast<uint32_t>(((w.K + kBN - 1) / kBN) * ((M + kBM - 1) / kBM)));
  if (w.qscale)
    hipLaunchKernelGGL((gemm_kernel<true, true>), grid, dim3(kThreads), 0, st, g, code_params(w));
  else
    hipLaunchKernelGGL((gemm_kernel<true, false>), grid, dim3(kThreads), 0, st, g, code_params(w));
  return hipGetLastError();
}

}  // namespace qn
