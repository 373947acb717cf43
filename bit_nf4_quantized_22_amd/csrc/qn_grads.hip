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
// bytes in flight set the streaming rate.  Both products share each launch.
// Two forms, each bit-reproducible:
//   * column tiles (r % 8 == 0, u and t 16-byte aligned): a workgroup owns
//     64 columns over all M tokens and writes s * sum directly, one launch;
//   * token chunks (any r): workgroups own 256 columns and a token chunk,
//     write fp32 partial sums [chunk][r][C], and a second pass sums the
//     chunks in a fixed order and applies s.  The chunks are long enough
//     that the partials stay a quarter of the input or less.
// The wide matrices are read once in both.

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
  int pair;  // column-tile kernel: adjacent tiles on one XCD (see grads_cols_kernel)
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

// Column-tile form, no partial sums: a workgroup owns kCW (64 or 32) columns of X over
// all M tokens and writes s * sum straight into dA or dB, so one launch
// does what the chunked kernel and its reduction do in two.  The four waves
// take interleaved 64-token steps (wave w: steps w, w + 4, ...), each in its
// own LDS region, so the main loop has no workgroup barrier: a wave's LDS
// instructions are processed in issue order, which orders its transposed
// stores, its operand reads and the next step's stores.  The waves' sums
// are added in LDS in wave order at the end.  Needs r % 8 == 0 and P
// 16-byte aligned: a lane loads 8 consecutive ranks of two adjacent tokens
// as two 16-byte loads and stores them transposed as token pairs.
//   X: lane (cg = lane / kRPn, rp = lane % kRPn, kRPn = 512 / kCW) loads rows
//      2 kRPn q + 2 rp + {0, 1} of columns 8 cg .. + 7: 8 rows x 128 bytes
//      (kCW = 64) or 16 rows x 64 bytes (kCW = 32) per instruction.
//   P: lane (tp = lane % 32, jh = lane / 32) loads tokens 2 tp + {0, 1},
//      ranks 8 (jh + 2 q) .. + 7 (q < RT / 16).
// Tokens past M read row M - 1 and are stored as zero P, ranks past r read
// a valid chunk and are stored as zero.
template <int RT, int kCW>
__global__ __launch_bounds__(256) void grads_cols_kernel(const GradJob ja, const GradJob jb,
                                                         int64_t M, int r, float s,
                                                         float* __restrict__ dA,
                                                         float* __restrict__ dB) {
  // steps in flight per wave (four at r <= 32 was slower: 17.4 against 16.2 us at
  // 11008 x 4096, M = 2048, r = 16)
  constexpr int kDepth = RT <= 64 ? 2 : 1;
  constexpr int kPV = RT / 8;                       // 16-byte P loads per lane per step
  constexpr int kCG = kCW / 8;        // 8-column groups of the tile
  constexpr int kRPn = 64 / kCG;      // lanes per column group: token pairs per load
  constexpr int kQn = kStep / (2 * kRPn);  // loads of each row of a pair per step
  constexpr int kCT = kCW / 16;       // 16-column MFMA tiles
  constexpr int kSX = kCW * kPitch, kSP = RT * kPitch;  // bf16 per wave region
  constexpr int kSlab = RT < 64 ? RT : 64;          // ranks per cross-wave pass
  constexpr int kRP = 65;                           // fp32 pitch of the pass buffer
  constexpr int kStage = 4 * (kSX + kSP) * 2, kRed = 4 * kSlab * kRP * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStage > kRed ? kStage : kRed];

  const bool second = static_cast<int>(blockIdx.x) >= ja.nwg;  // uniform
  const uint16_t* X = second ? jb.X : ja.X;
  const uint16_t* P = second ? jb.P : ja.P;
  const int64_t C = second ? jb.C : ja.C;
  int ct = static_cast<int>(blockIdx.x) - (second ? ja.nwg : 0);
  // Workgroup b runs on XCD b mod 8.  With 32-column tiles two tiles share
  // each 128-byte line of a row; with pair set (both jobs' tile counts
  // multiples of 16, so b mod 8 is the job-local index mod 8) each group of
  // 16 workgroups takes its 16 tiles as 8 adjacent pairs, a pair on one XCD.
  if (kCW == 32 && (second ? jb.pair : ja.pair)) ct = (ct & ~15) | ((ct & 7) << 1) | ((ct >> 3) & 1);
  const int64_t c0 = static_cast<int64_t>(ct) * kCW;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint16_t* sX = reinterpret_cast<uint16_t*>(smem) + wave * (kSX + kSP);
  uint16_t* sP = sX + kSX;
  const int nsteps = static_cast<int>((M + kStep - 1) / kStep);
  const int nown = (nsteps + 3) / 4;                          // steps of wave 0
  const int niter = (nown + kDepth - 1) / kDepth * kDepth;    // same count for every wave

  const int cg = lane / kRPn, rp = lane % kRPn;
  const int tp = lane & 31, jh = lane >> 5;
  const int rc = r >> 3;  // valid 8-rank chunks
  const uint16_t* Xc = X + c0 + 8 * cg;
  auto load_step = [&](int i, uint4 (&xv)[2 * kQn], uint4 (&pv)[kPV]) {
    const int64_t mb = static_cast<int64_t>(4 * i + wave) * kStep;
#pragma unroll
    for (int q = 0; q < kQn; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int64_t m = mb + 2 * kRPn * q + 2 * rp + h;
        m = m < M ? m : M - 1;
        xv[2 * q + h] = *reinterpret_cast<const uint4*>(Xc + m * C);
      }
#pragma unroll
    for (int q = 0; q < RT / 16; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int64_t m = mb + 2 * tp + h;
        m = m < M ? m : M - 1;
        int jc = jh + 2 * q;
        jc = jc < rc ? jc : rc - 1;
        pv[2 * q + h] = *reinterpret_cast<const uint4*>(P + m * r + 8 * jc);
      }
  };

  f32x4_t acc[RT / 16][kCT];
#pragma unroll
  for (int a = 0; a < RT / 16; ++a)
#pragma unroll
    for (int b = 0; b < kCT; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int l16 = lane & 15, g = lane >> 4;
  auto step = [&](int i, uint4 (&xv)[2 * kQn], uint4 (&pv)[kPV]) {
    const int64_t mb = static_cast<int64_t>(4 * i + wave) * kStep;
    // X transposed: word (token pair rp + kRPn q) of column 8 cg + e
#pragma unroll
    for (int q = 0; q < kQn; ++q) {
      const uint32_t a0[4] = {xv[2 * q].x, xv[2 * q].y, xv[2 * q].z, xv[2 * q].w};
      const uint32_t a1[4] = {xv[2 * q + 1].x, xv[2 * q + 1].y, xv[2 * q + 1].z, xv[2 * q + 1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = e & 1 ? a0[e >> 1] >> 16 : a0[e >> 1] & 0xFFFFu;
        const uint32_t hi = e & 1 ? a1[e >> 1] & 0xFFFF0000u : a1[e >> 1] << 16;
        const int row = 8 * cg + e, tok = 2 * kRPn * q + 2 * rp;
        *reinterpret_cast<uint32_t*>(&sX[row * kPitch + 8 * xslot(row, tok >> 3) + (tok & 7)]) =
            lo | hi;
      }
    }
    // P transposed: word (token pair tp) of rank 8 jc + e
    const bool ok0 = mb + 2 * tp < M, ok1 = mb + 2 * tp + 1 < M;
#pragma unroll
    for (int q = 0; q < RT / 16; ++q) {
      const int jc = jh + 2 * q;
      const bool okj = jc < rc;
      const uint4 p0 = pv[2 * q], p1 = pv[2 * q + 1];
      const uint32_t w0[4] = {p0.x, p0.y, p0.z, p0.w}, w1[4] = {p1.x, p1.y, p1.z, p1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = e & 1 ? w0[e >> 1] >> 16 : w0[e >> 1] & 0xFFFFu;
        const uint32_t hi = e & 1 ? w1[e >> 1] & 0xFFFF0000u : w1[e >> 1] << 16;
        const uint32_t word = (okj && ok0 ? lo : 0u) | (okj && ok1 ? hi : 0u);
        *reinterpret_cast<uint32_t*>(&sP[(8 * jc + e) * kPitch + 2 * tp]) = word;
      }
    }
    load_step(i + kDepth, xv, pv);
#pragma unroll
    for (int kk = 0; kk < kStep / 32; ++kk) {
      uint4 pa[RT / 16];
#pragma unroll
      for (int a = 0; a < RT / 16; ++a)
        pa[a] = *reinterpret_cast<const uint4*>(&sP[(16 * a + l16) * kPitch + 32 * kk + 8 * g]);
#pragma unroll
      for (int b = 0; b < kCT; ++b) {
        const int xrow = 16 * b + l16;
        const uint4 xb = *reinterpret_cast<const uint4*>(
            &sX[xrow * kPitch + 8 * xslot(xrow, 4 * kk + g)]);
#pragma unroll
        for (int a = 0; a < RT / 16; ++a) acc[a][b] = mfma16(pa[a], xb, acc[a][b]);
      }
    }
    asm volatile("" ::: "memory");  // keep this step's reads before the next step's stores
  };
  if (niter > 0) {
    uint4 xv[kDepth][2 * kQn];
    uint4 pv[kDepth][kPV];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) load_step(d, xv[d], pv[d]);
    for (int i = 0; i < niter; i += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) step(i + d, xv[d], pv[d]);
    }
  }

  // Cross-wave sum in wave order, kSlab ranks per pass.  Lane (l16, g)
  // holds ranks 16 a + 4 g + v of columns 16 b + l16.
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int sl = 0; sl < RT; sl += kSlab) {
    __syncthreads();  // staging reads (or the previous pass's reads) are done
#pragma unroll
    for (int a = sl / 16; a < (sl + kSlab) / 16; ++a)
#pragma unroll
      for (int b = 0; b < kCT; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          red[(wave * kSlab + 16 * a + 4 * g + v - sl) * kRP + 16 * b + l16] = acc[a][b][v];
    __syncthreads();
    const int nj = r - sl < kSlab ? r - sl : kSlab;  // ranks of this pass
    if (nj > 0) {
      auto sum4 = [&](int jj, int c) {
        const float* p = red + jj * kRP + c;
        return s * (((p[0] + p[kSlab * kRP]) + p[2 * kSlab * kRP]) + p[3 * kSlab * kRP]);
      };
      if (!second) {  // dA [r, C]: kCW consecutive columns per rank
        for (int idx = tid; idx < nj * kCW; idx += 256) {
          const int jj = idx / kCW, c = idx % kCW;
          dA[static_cast<int64_t>(sl + jj) * C + c0 + c] = sum4(jj, c);
        }
      } else {  // dB [C, r]: the tile's rows are contiguous
        for (int idx = tid; idx < nj * kCW; idx += 256) {
          const int c = idx / nj, jj = idx - c * nj;
          dB[(c0 + c) * r + sl + jj] = sum4(jj, c);
        }
      }
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
  if (r % 8 == 0 && reinterpret_cast<uintptr_t>(u) % 16 == 0 &&
      reinterpret_cast<uintptr_t>(t) % 16 == 0) {
    // 32-column tiles where 64-column ones would leave most CUs idle, for
    // r > 16, whose t/u staging dominates a step (4096 x 4096, M = 2048: 128
    // workgroups; r = 64 22.4 -> 19.6 us, while r = 16 went 13.6 -> 14.2 us)
    const int cw = r > 16 && (K / 64 + N / 64) < 200 ? 32 : 64;
    GradJob ja{}, jb{};
    ja.X = x; ja.P = t; ja.C = K; ja.ncol = static_cast<int>(K / cw); ja.nwg = ja.ncol;
    jb.X = dy; jb.P = u; jb.C = N; jb.ncol = static_cast<int>(N / cw); jb.nwg = jb.ncol;
    ja.pair = jb.pair = ja.ncol % 16 == 0 && jb.ncol % 16 == 0;
    const dim3 grid(static_cast<uint32_t>(ja.nwg + jb.nwg));
#define QN_GRADS_COLS(RT, CW) \
  hipLaunchKernelGGL((grads_cols_kernel<RT, CW>), grid, dim3(256), 0, st, ja, jb, M, r, s, dA, dB)
    if (cw == 64) {
      if (r <= 16) QN_GRADS_COLS(16, 64);
      else if (r <= 32) QN_GRADS_COLS(32, 64);
      else if (r <= 64) QN_GRADS_COLS(64, 64);
      else QN_GRADS_COLS(128, 64);
    } else {
      if (r <= 16) QN_GRADS_COLS(16, 32);
      else if (r <= 32) QN_GRADS_COLS(32, 32);
      else if (r <= 64) QN_GRADS_COLS(64, 32);
      else QN_GRADS_COLS(128, 32);
    }
#undef QN_GRADS_COLS
    return hipGetLastError();
  }
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
