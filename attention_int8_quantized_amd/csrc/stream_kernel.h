// A plain read of a device buffer, for measuring the practical HBM read
// bandwidth next to the attention kernels (the attention kernels' bytes are
// priced against it as well as against the 8 TB/s peak).  Each workgroup XORs
// the 32-bit words it reads, so the XOR of all workgroup results is the XOR of
// the buffer: a value that depends on every byte read and can be checked.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnq8 {

constexpr int kStreamBlocks = 1024;   // workgroups (four per CU)
constexpr int kStreamThreads = 256;

__device__ __forceinline__ uint32_t xor4(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// p: n16 16-byte vectors; sink: kStreamBlocks words, one per workgroup
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                                     uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)kStreamBlocks * kStreamThreads;
  size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
  uint32_t acc = 0;
  // four 16-byte loads in flight per lane
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= xor4(a) ^ xor4(b) ^ xor4(c) ^ xor4(d);
  }
  for (; i < n16; i += stride) acc ^= xor4(p[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  __shared__ uint32_t w[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int k = 0; k < kStreamThreads / 64; ++k) r ^= w[k];
    sink[blockIdx.x] = r;
  }
}

}  // namespace attnq8
