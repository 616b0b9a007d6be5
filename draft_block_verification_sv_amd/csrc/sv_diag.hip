// Diagnostics: a plain read of a device buffer, the practical ceiling of a kernel that only
// streams bytes in.  The roofline of the streaming kernels is the published HBM peak; this
// kernel shows how much of it a read with nothing else to do reaches on the same part.
#include <hip/hip_runtime.h>

#include "sv_launch.h"

namespace sv {

// Block-contiguous read of n 16-byte words: workgroup g reads words [g per, (g + 1) per) front
// to back, every thread two nontemporal loads per round (8 KiB per workgroup in flight), and
// folds the words with xor; each workgroup writes one word (so the loads are not dead).  Of the
// read patterns measured on this part (grid-stride and contiguous, 1024 to 65536 workgroups,
// 1 to 8 loads in flight per thread, plain and nontemporal), this one read fastest.
typedef unsigned int probe_u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void sv_read_probe_kernel(const uint4* __restrict__ p, int64_t n,
                                                             uint32_t* out) {
  const int64_t per = (n + gridDim.x - 1) / gridDim.x;
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t hi = lo + per < n ? lo + per : n;
  const probe_u32x4* q = reinterpret_cast<const probe_u32x4*>(p);
  uint32_t acc = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += 512) {
    probe_u32x4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
    if (i < hi) v0 = __builtin_nontemporal_load(q + i);
    if (i + 256 < hi) v1 = __builtin_nontemporal_load(q + i + 256);
    acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
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
