// Measurement aid: a plain streaming read, the rate the memory system gives
// a kernel that does nothing but load.  It is the context for the fractions
// of the HBM peak that the quantiser, dequant, GEMV and merge reach.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qn_launch.h"

namespace qn {

namespace {

// Grid-stride loop over 16-byte words, four loads in flight per lane and
// iteration (consecutive lanes read consecutive words, so every load
// instruction of a wave covers 1 KB).  All 16 bytes of every word feed the
// XOR, so no load narrows; the store fires only on a sentinel value.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) *sink = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  // 8 workgroups per CU on the 256 CUs
  hipLaunchKernelGGL(read_probe_kernel, dim3(2048), dim3(256), 0, st,
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace qn
