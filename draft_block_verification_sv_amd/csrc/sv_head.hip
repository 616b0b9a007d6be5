// The adaptive length head (AdaFlash paper, Section 3.2 "Design of the Adaptive Length Head"
// and "Online Update of the Length Head"; Section 3.3 "Adaptive Request Scheduling" for the
// packed layout), on gfx950 matrix cores.
//
//   sv_head_feat   per request b and 16-feature slab: the k x 16 block of W1 h_b^T on MFMA
//                  (v_mfma_f32_16x16x32_bf16, 16-position tiles, K = H in steps of 32 split
//                  four ways across the waves, eight steps of loads in flight, partial tiles
//                  summed in LDS in wave order), then + b1, SiLU and the mean over the k
//                  positions, written as the pooled features of b (fp32).
//   sv_head_out    one workgroup: a_hat_b = sigmoid(w2 . pooled_b + b2) (fp64 dot, fixed
//                  combination order), k_hat_b = clamp(floor(a_hat_b gamma k), 1, k) in fp64, and the
//                  packed target-row offsets off_t[b] = sum_{c<b} (k_hat_c + 1).
//   sv_len_loss    l_len_b = (a_hat_b - a_b / k_hat_b)^2 and its derivative in a_hat.
//
// MFMA lane layout of the 16x16x32 bf16 instruction (checked on the device): lane l holds
// A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16], e = 0..7, and its four results
// are D[4 (l / 16) + i][l % 16], i = 0..3.  A is the 16-row tile of h (positions x H), B the
// transposed 16-column tile of W1 (H x features), so both operands are 16-byte loads of 8
// consecutive elements of one row.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_device.h"
#include "sv_launch.h"

namespace sv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& w) {
  bf16x8_t v;
  __builtin_memcpy(&v, &w, 16);
  return v;
}

constexpr int kHeadCols = 16;   // features per workgroup (one 16 x 16 MFMA tile)
constexpr int kHeadSplit = 4;   // the workgroup's waves split K four ways
constexpr int kHeadUnroll = 8;  // K steps whose loads are in flight together

// One workgroup: request b, features n0 .. n0 + 15.  Wave w accumulates the w-th quarter of
// the K steps of every 16-position tile; the four partial tiles are summed in LDS
// in wave order, then wave 0 adds b1, applies SiLU and pools over the k positions.
__global__ __launch_bounds__(64 * kHeadSplit) void sv_head_feat_kernel(HeadArgs a) {
  __shared__ float part[kHeadSplit][64][4];
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.y * kHeadCols;
  const int r = lane & 15, kg = (lane >> 4) * 8;  // operand row / column, k offset
  const int n = n0 + r;                            // the W1 row this lane loads
  const bool n_ok = n < a.Hf;
  const int steps = a.H / 32;  // MFMA K steps (H is a multiple of 32), shared out in order
  const int k_lo = 32 * ((wave * steps) / kHeadSplit);
  const int k_hi = 32 * (((wave + 1) * steps) / kHeadSplit);
  const uint16_t* Wrow = static_cast<const uint16_t*>(a.W1) + (n_ok ? n : 0) * a.ld_w + kg;
  float colsum = 0.0f;
  for (int r0 = 0; r0 < a.k; r0 += 16) {
    const int pos = r0 + r;
    const bool p_ok = pos < a.k;
    const uint16_t* Hrow =
        static_cast<const uint16_t*>(a.h) + (b * a.k + (p_ok ? pos : 0)) * a.ld_h + kg;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    int kk = k_lo;
    for (; kk + 32 * kHeadUnroll <= k_hi; kk += 32 * kHeadUnroll) {
      uint4 av[kHeadUnroll], bv[kHeadUnroll];
#pragma unroll
      for (int u = 0; u < kHeadUnroll; ++u) {
        av[u] = p_ok ? *reinterpret_cast<const uint4*>(Hrow + kk + 32 * u) : make_uint4(0, 0, 0, 0);
        bv[u] = n_ok ? *reinterpret_cast<const uint4*>(Wrow + kk + 32 * u) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kHeadUnroll; ++u)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[u]), as_bf16x8(bv[u]), acc, 0,
                                                     0, 0);
    }
    for (; kk + 32 <= k_hi; kk += 32) {
      const uint4 av = p_ok ? *reinterpret_cast<const uint4*>(Hrow + kk) : make_uint4(0, 0, 0, 0);
      const uint4 bv = n_ok ? *reinterpret_cast<const uint4*>(Wrow + kk) : make_uint4(0, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bv), acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wave][lane][i] = acc[i];
    __syncthreads();
    if (wave == 0) {
      // lane holds D[4 (l/16) + i][l % 16]: positions r0 + 4 (l/16) + i, feature n0 + l % 16
      const float bias = (a.b1 && n0 + (lane & 15) < a.Hf) ? a.b1[n0 + (lane & 15)] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float z = 0.0f;
#pragma unroll
        for (int w = 0; w < kHeadSplit; ++w) z += part[w][lane][i];
        z += bias;
        const int p = r0 + 4 * (lane >> 4) + i;
        if (p < a.k) colsum += z / (1.0f + __expf(-z));
      }
    }
    __syncthreads();
  }
  if (wave == 0) {
    // the four lanes of a feature column (l, l + 16, l + 32, l + 48) hold its row groups
    colsum += __shfl_xor(colsum, 16, 64);
    colsum += __shfl_xor(colsum, 32, 64);
    const int fc = n0 + (lane & 15);
    if (lane < 16 && fc < a.Hf) a.pooled[b * a.Hf + fc] = colsum / static_cast<float>(a.k);
  }
}

__device__ __forceinline__ int block_excl_scan_1024_head(int v, int* lds_waves, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(x, d, 64);
    if (lane >= d) x += o;
  }
  if (lane == 63) lds_waves[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) base += lds_waves[w];
    tot += lds_waves[w];
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// One workgroup of 16 waves.  a_hat and k_hat: wave w takes requests w, w + 16, ..., its
// lanes stride the features (coalesced), fp64 partial dots combined by a fixed butterfly.
// Then the fixed-order scan of k_hat + 1 gives the packed offsets.
__global__ __launch_bounds__(1024) void sv_head_out_kernel(HeadArgs a) {
  __shared__ int s_waves[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int64_t b = wave; b < a.B; b += 16) {
    const float* pb = a.pooled + b * a.Hf;
    double dot = 0.0;
    for (int n = lane; n < a.Hf; n += 64) dot += static_cast<double>(pb[n]) * static_cast<double>(a.w2[n]);
    dot = wave_sum_d(dot) + static_cast<double>(a.b2);
    if (lane == 0) {
      const double ah = 1.0 / (1.0 + exp(-dot));
      double t = floor(ah * static_cast<double>(a.gamma) * static_cast<double>(a.k));
      t = t < 1.0 ? 1.0 : (t > a.k ? static_cast<double>(a.k) : t);
      a.a_hat[b] = static_cast<float>(ah);
      a.k_hat[b] = static_cast<int>(t);
    }
  }
  if (!a.off_t) return;
  __syncthreads();  // k_hat written by this workgroup, read back below
  int carry = 0;
  for (int64_t base = 0; base < a.B; base += 1024) {
    const int64_t b = base + tid;
    const int kh = b < a.B ? a.k_hat[b] : 0;
    int total = 0;
    const int excl = block_excl_scan_1024_head(b < a.B ? kh + 1 : 0, s_waves, &total);
    if (b < a.B) a.off_t[b] = carry + excl;
    carry += total;
  }
  if (tid == 0) a.off_t[a.B] = carry;
}

__global__ __launch_bounds__(256) void sv_len_loss_kernel(int64_t B, const float* a_hat,
                                                          const int32_t* accept_len,
                                                          const int32_t* k_hat, float* loss,
                                                          float* dloss) {
  const int64_t b = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (b >= B) return;
  const int al = accept_len[b], kh = k_hat[b];
  const bool ok = al >= 0 && kh >= 1 && al <= kh;
  const double e = static_cast<double>(a_hat[b]) - static_cast<double>(al) / static_cast<double>(kh);
  loss[b] = ok ? static_cast<float>(e * e) : NAN;
  if (dloss) dloss[b] = ok ? static_cast<float>(2.0 * e) : NAN;
}

hipError_t launch_head(const HeadArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.B), static_cast<unsigned>((a.Hf + kHeadCols - 1) / kHeadCols));
  hipLaunchKernelGGL(sv_head_feat_kernel, grid, dim3(64 * kHeadSplit), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return hipSuccess;
}

hipError_t launch_head_out(const HeadArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(sv_head_out_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_len_loss(int64_t B, const float* a_hat, const int32_t* accept_len,
                           const int32_t* k_hat, float* loss, float* dloss, hipStream_t st) {
  hipLaunchKernelGGL(sv_len_loss_kernel, dim3(static_cast<unsigned>((B + 255) / 256)), dim3(256), 0,
                     st, B, a_hat, accept_len, k_hat, loss, dloss);
  return hipGetLastError();
}

}  // namespace sv
