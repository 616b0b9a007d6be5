// Diagnostics: a plain read of a device buffer, the practical ceiling of a kernel that only
// streams bytes in.  The roofline of the streaming kernels is the published HBM peak; this
// kernel shows how much of it a read with nothing else to do reaches on the same part.
#include <hip/hip_runtime.h>

#include "sv_launch.h"

namespace sv {

// Grid-stride read of n 16-byte words: every thread keeps four loads in flight per round and
// folds the words with xor; each workgroup writes one word (so the loads are not dead).
__global__ __launch_bounds__(256) void sv_read_probe_kernel(const uint4* __restrict__ p, int64_t n,
                                                             uint32_t* out) {
  constexpr int U = 4;
  uint32_t acc = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * U;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 256 * U + threadIdx.x; base < n; base += stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * 256;
      v[u] = i < n ? p[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t red[4];
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

hipError_t launch_read_probe(const void* data, int64_t n_words, uint32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(sv_read_probe_kernel, dim3(kReadProbeBlocks), dim3(256), 0, st,
                     static_cast<const uint4*>(data), n_words, out);
  return hipGetLastError();
}

}  // namespace sv
