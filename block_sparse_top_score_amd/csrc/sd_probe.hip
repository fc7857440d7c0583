// Streaming-read probe: a measurement aid, no part of the decode path.  It
// gives the HBM read rate a plain kernel reaches on this GPU, against which
// the decode step's own rate can be read.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "sparse_decode.h"

namespace {
// Plain streaming read: every 16-byte word of src once, grid-stride with
// eight words in flight per thread (consecutive threads read consecutive
// words); the XOR of a workgroup's words goes to its sink word, so no load is
// dead.  (Four in flight reach 0.70 of the HBM peak on this GPU, eight about
// 0.77 at 4096 workgroups.)
constexpr int kInFlight = 8;
__global__ __launch_bounds__(256) void k_read_probe(const uint4 *__restrict__ src, size_t n16,
                                                    uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    uint4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  __shared__ uint32_t w[4];
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = w[0] ^ w[1] ^ w[2] ^ w[3];
}
}  // namespace

extern "C" sd_status sd_read_probe(const void *src, size_t bytes, uint32_t *sink,
                                   int32_t sink_words, void *stream) {
  if (!src || !sink || sink_words < 1 || bytes == 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return SD_EINVAL;
  hipLaunchKernelGGL(k_read_probe, dim3((unsigned)sink_words), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4 *>(src), bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? SD_OK : SD_EHIP;
}
