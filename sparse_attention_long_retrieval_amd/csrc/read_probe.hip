// Streaming-read probe for the benchmark's attainable-bandwidth figure (not part of
// the attention path, and built into its own library, libreadprobe.so).  Every
// thread reads 16-byte words in a grid-stride loop, four in flight, and folds them
// into one word so the loads cannot be dropped; each block writes one word.
#include <hip/hip_runtime.h>
#include <stdint.h>

__global__ __launch_bounds__(256) void k_read_probe(const uint4* __restrict__ src, size_t n16,
                                                    unsigned* out) {
  unsigned acc = 0u;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ unsigned part[256];
  part[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned r = 0u;
    for (int k = 0; k < 256; ++k) r ^= part[k];
    out[blockIdx.x] = r;
  }
}

// Read nbytes (a multiple of 16) at src with `blocks` blocks; out holds `blocks` words.
extern "C" int read_probe(const void* src, size_t nbytes, void* out, int blocks, void* stream) {
  if (!src || !out || blocks < 1 || nbytes % 16) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_read_probe, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, nbytes / 16, (unsigned*)out);
  return (int)hipGetLastError();
}
