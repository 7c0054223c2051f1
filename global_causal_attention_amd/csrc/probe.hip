// Measurement helper: streaming-read bandwidth of HBM on this device, the reference the
// memory-bound kernels are compared with beside the 8 TB/s specification. Every lane reads
// 16-byte pieces with non-temporal loads (four in flight per lane per round) and folds them into
// one word per wave, written to `sink` so that the loads cannot be removed.
#include "zg_common.hpp"

namespace zg {

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= (a[0] ^ a[1] ^ a[2] ^ a[3]) ^ (b[0] ^ b[1] ^ b[2] ^ b[3]) ^ (c[0] ^ c[1] ^ c[2] ^ c[3]) ^
           (d[0] ^ d[1] ^ d[2] ^ d[3]);
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if ((threadIdx.x & 63) == 0) sink[(int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* sink, int32_t n_blocks,
                             hipStream_t s) {
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)n_blocks), dim3(256), 0, s,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace zg
