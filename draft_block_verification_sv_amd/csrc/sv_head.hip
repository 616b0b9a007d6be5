// The adaptive length head (AdaFlash paper, Section 3.2 "Design of the Adaptive Length Head"
// and "Online Update of the Length Head"; Section 3.3 "Adaptive Request Scheduling" for the
// packed layout), on gfx950 matrix cores.
//
//   sv_head_feat   the projection z = W1 h^T as a split-K GEMM on v_mfma_f32_16x16x32_bf16.
//                  A request's positions form ceil(k / 16) blocks of 16 rows; a workgroup
//                  takes four blocks against all features (up to 256; wave w a quarter of
//                  them) over one K-chunk, staged through LDS 32 columns at a time with
//                  several stages in flight, and writes the fp32 partial sums of that chunk.
//   sv_head_pool   one workgroup per request: z = sum of the K-chunks' partials in chunk order
//                  + b1, SiLU, the mean over the k positions, a_hat = sigmoid(w2 . pooled + b2)
//                  (fp64 dot, fixed combination order) and k_hat = clamp(floor(a_hat gamma k),
//                  1, k) in fp64; the workgroup that finishes last writes the packed
//                  target-row offsets off_t[b] = sum_{c<b} (k_hat_c + 1).
//   sv_len_loss    l_len_b = (a_hat_b - a_b / k_hat_b)^2 and its derivative in a_hat.
//
// MFMA lane layout of the 16x16x32 bf16 instruction (checked on the device): lane l holds
// A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16], e = 0..7, and its four results
// are D[4 (l / 16) + i][l % 16], i = 0..3.  A is the 16-row tile of h (positions x H), B the
// transposed 16-column tile of W1 (H x features), so both operands are 16-byte loads of 8
// consecutive elements of one row.  Rows past a request's k (and past the last request) and
// features past H' are read from clamped, in-bounds rows: an MFMA output row depends only
// on its own A row and an output column only on its own B column, so those rows and columns
// are simply never used, and every load is issued without a condition.
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

constexpr int kHeadStages = 4;   // 32-column K stages whose loads are in flight
constexpr int kLdsRow = 32 + 8;  // bf16 per LDS row: one K stage plus 16 B of padding
constexpr int kHeadThreads = 64 * kHeadBlocks;
// 16-byte pieces of a stage each thread copies: one of the 64-row A stage, kBPieces of the
// kHeadTileN-row B stage (64 bytes per row)
constexpr int kBPieces = kHeadTileN * 4 / kHeadThreads;
static_assert(kHeadBlocks == 4 && kBPieces == 4 && kBPieces * kHeadThreads == kHeadTileN * 4,
              "stage copy layout: four B pieces per thread, named below");
constexpr int kWaveFeatures = kHeadTileN / kHeadBlocks;  // features per wave
constexpr int kWaveTiles = kWaveFeatures / 16;           // 16-feature MFMA tiles per wave

// One workgroup: blocks 4 g .. 4 g + 3 (64 rows), features n0 .. n0 + kHeadTileN - 1 (all of
// H' up to 256), K-chunk c, in stages of 32 columns.  Wave w computes every block against
// features n0 + 64 w .. + 63 (4 blocks x 4 feature tiles = 16 MFMAs a stage), so each wave
// reads 4 A and 4 B fragments per stage from LDS and h is read once per K-chunk.  Each thread
// copies one 16-byte piece of the A stage (row tid / 4) and kBPieces of the B stage (feature
// rows tid / 4 + 64 j): every row of a stage is read as a full 64-byte run.  kHeadStages stages
// are in flight in registers; a stage is written to one of two LDS buffers (rows padded to 80
// bytes, so the 16 rows a fragment read touches fall on distinct banks), the workgroup barrier
// publishes it, the next stage's loads are issued, and each wave reads its fragments.  Stage
// indices past the chunk are clamped (the last stage again, from cache; never used).  Writes
// partial[((c NB + blk) 16 + row) H' + n].
__global__ __launch_bounds__(kHeadThreads) void sv_head_feat_kernel(HeadArgs a) {
  __shared__ __align__(16) uint16_t sA[2][64 * kLdsRow];
  __shared__ __align__(16) uint16_t sB[2][kHeadTileN * kLdsRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n_rows = a.B * static_cast<int64_t>(a.k);
  // this thread's copy pieces: row cr of the A stage and feature rows cr + 64 j of the B stage,
  // 16 bytes at column cc
  const int cr = tid >> 2, cc = (tid & 3) * 8;
  const int64_t cblk = static_cast<int64_t>(blockIdx.x) * kHeadBlocks + cr / 16;
  const int64_t cb = cblk / a.R;
  const int cpos = static_cast<int>(cblk - cb * a.R) * 16 + (cr & 15);
  int64_t hrow = cb * a.k + cpos;
  if (cpos >= a.k || hrow >= n_rows) hrow = n_rows - 1;  // clamped: row never used
  const int n0 = blockIdx.y * kHeadTileN;
  const uint16_t* gA = static_cast<const uint16_t*>(a.h) + hrow * a.ld_h + cc;
  // (clamped rows: columns never stored)
  auto w1_row = [&](int j) {
    return static_cast<const uint16_t*>(a.W1) +
           static_cast<int64_t>(min(n0 + cr + 64 * j, a.Hf - 1)) * a.ld_w + cc;
  };
  const uint16_t* const gB0 = w1_row(0);
  const uint16_t* const gB1 = w1_row(1);
  const uint16_t* const gB2 = w1_row(2);
  const uint16_t* const gB3 = w1_row(3);
  const int lds_w = cr * kLdsRow + cc;
  // this lane's fragment reads: row r of each block / of each of its wave's feature tiles,
  // k offset kg
  const int r = lane & 15, kg = (lane >> 4) * 8;
  const int ldsA = r * kLdsRow + kg;
  const int ldsB = (wave * kWaveFeatures + r) * kLdsRow + kg;

  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && tid == 0) *a.ticket = 0;
  const int c = blockIdx.z;
  const int steps = a.H / 32;
  const int s_lo = (c * steps) / a.S, s_hi = ((c + 1) * steps) / a.S;
  const int n_st = s_hi - s_lo;
  f32x4_t acc[kHeadBlocks][kWaveTiles];
#pragma unroll
  for (int bb = 0; bb < kHeadBlocks; ++bb)
#pragma unroll
    for (int t = 0; t < kWaveTiles; ++t) acc[bb][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the ring of stages in flight, as named registers (an array here would live in scratch)
  uint4 ra0, ra1, ra2, ra3;
  uint4 rb0_0, rb0_1, rb0_2, rb0_3, rb1_0, rb1_1, rb1_2, rb1_3;
  uint4 rb2_0, rb2_1, rb2_2, rb2_3, rb3_0, rb3_1, rb3_2, rb3_3;
#define SV_HEAD_FETCH(J, st)                                                                \
  {                                                                                         \
    const int col_ = 32 * (s_lo + min((st), n_st - 1));                                     \
    ra##J = *reinterpret_cast<const uint4*>(gA + col_);                                     \
    rb##J##_0 = *reinterpret_cast<const uint4*>(gB0 + col_);                                \
    rb##J##_1 = *reinterpret_cast<const uint4*>(gB1 + col_);                                \
    rb##J##_2 = *reinterpret_cast<const uint4*>(gB2 + col_);                                \
    rb##J##_3 = *reinterpret_cast<const uint4*>(gB3 + col_);                                \
  }
  SV_HEAD_FETCH(0, 0)
  SV_HEAD_FETCH(1, 1)
  SV_HEAD_FETCH(2, 2)
  SV_HEAD_FETCH(3, 3)
  // stage i: publish it in LDS buffer i % 2, refill its ring slot with stage i + kHeadStages,
  // then 16 MFMAs from LDS.  Full rounds run without a condition (a load under a branch would
  // make the wait at the join count the refills too); the last partial round is guarded by its
  // stage index, uniform across the workgroup.
#define SV_HEAD_STEP(J, i)                                                                  \
  {                                                                                         \
    uint16_t* bA = sA[(J) & 1];                                                             \
    uint16_t* bB = sB[(J) & 1];                                                             \
    *reinterpret_cast<uint4*>(&bA[lds_w]) = ra##J;                                          \
    *reinterpret_cast<uint4*>(&bB[lds_w]) = rb##J##_0;                                      \
    *reinterpret_cast<uint4*>(&bB[lds_w + 64 * kLdsRow]) = rb##J##_1;                       \
    *reinterpret_cast<uint4*>(&bB[lds_w + 128 * kLdsRow]) = rb##J##_2;                      \
    *reinterpret_cast<uint4*>(&bB[lds_w + 192 * kLdsRow]) = rb##J##_3;                      \
    __syncthreads();                                                                        \
    SV_HEAD_FETCH(J, (i) + kHeadStages)                                                     \
    uint4 av[kHeadBlocks], bv[kWaveTiles];                                                  \
    _Pragma("unroll") for (int bb = 0; bb < kHeadBlocks; ++bb)                              \
      av[bb] = *reinterpret_cast<const uint4*>(&bA[ldsA + bb * 16 * kLdsRow]);              \
    _Pragma("unroll") for (int t = 0; t < kWaveTiles; ++t)                                  \
      bv[t] = *reinterpret_cast<const uint4*>(&bB[ldsB + t * 16 * kLdsRow]);                \
    _Pragma("unroll") for (int bb = 0; bb < kHeadBlocks; ++bb)                              \
      _Pragma("unroll") for (int t = 0; t < kWaveTiles; ++t)                                \
        acc[bb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[bb]),             \
                                                             as_bf16x8(bv[t]), acc[bb][t],   \
                                                             0, 0, 0);                      \
  }
  int i0 = 0;
  for (; i0 + kHeadStages <= n_st; i0 += kHeadStages) {
    SV_HEAD_STEP(0, i0)
    SV_HEAD_STEP(1, i0 + 1)
    SV_HEAD_STEP(2, i0 + 2)
    SV_HEAD_STEP(3, i0 + 3)
  }
  if (i0 < n_st) {
    SV_HEAD_STEP(0, i0)
    if (i0 + 1 < n_st) SV_HEAD_STEP(1, i0 + 1)
    if (i0 + 2 < n_st) SV_HEAD_STEP(2, i0 + 2)
  }
#undef SV_HEAD_STEP
#undef SV_HEAD_FETCH
  // lane holds D[4 (l/16) + i][l % 16] of each (block, feature tile)
#pragma unroll
  for (int bb = 0; bb < kHeadBlocks; ++bb) {
    const int64_t blk = static_cast<int64_t>(blockIdx.x) * kHeadBlocks + bb;
    if (blk >= a.NB) continue;
    float* P = a.partial + ((static_cast<int64_t>(c) * a.NB + blk) * 16 + 4 * (lane >> 4)) * a.Hf;
#pragma unroll
    for (int t = 0; t < kWaveTiles; ++t) {
      const int n = n0 + wave * kWaveFeatures + 16 * t + r;
      if (n < a.Hf)
#pragma unroll
        for (int i = 0; i < 4; ++i) P[static_cast<int64_t>(i) * a.Hf + n] = acc[bb][t][i];
    }
  }
}

// s_waitcnt operand that waits for every outstanding vector memory operation of the wave
// (vmcnt = 0) and leaves the export and LDS/scalar counters at their maxima (gfx9 encoding).
constexpr int kWaitVmcnt0 = 0x0F70;

// Fixed-order exclusive scan of k_hat + 1 over all requests by one 256-thread workgroup: each
// thread sums a contiguous run of requests, the run totals are scanned in thread order, then
// each thread writes its run's offsets.  k_hat is read with device-scope loads (it was written
// by other workgroups of the same launch).
__device__ void head_offsets(const HeadArgs& a, int* s_tot) {
  const int tid = threadIdx.x;
  const int64_t per = (a.B + 255) / 256;
  const int64_t lo = min<int64_t>(a.B, tid * per), hi = min<int64_t>(a.B, lo + per);
  int tot = 0;
  for (int64_t b = lo; b < hi; ++b)
    tot += __hip_atomic_load(a.k_hat + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
  s_tot[tid] = tot;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int t = 0; t < 256; ++t) {
      const int v = s_tot[t];
      s_tot[t] = run;
      run += v;
    }
    a.off_t[a.B] = run;
  }
  __syncthreads();
  int off = s_tot[tid];
  for (int64_t b = lo; b < hi; ++b) {
    a.off_t[b] = off;
    off += __hip_atomic_load(a.k_hat + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
  }
}

// One workgroup per request: thread t takes features t, t + 256, ...; for each, the partials
// of 32 / SP positions x SP chunk slots (SP = 4 when S <= 4, else 8) are loaded before any is
// used, indices past k or S clamped in bounds and their values dropped, so no load sits under
// a branch; z of a position is the sum of its chunks in chunk order, then + b1, SiLU, summed
// over the positions.  The dot with w2 is taken in fp64 over the thread's features, then over
// the threads in a fixed order.  With off_t, the workgroup that takes the last ticket of the
// launch (a device-scope counter the projection kernel zeroes) scans k_hat into the packed
// offsets; k_hat goes out as device-scope stores before the ticket.
template <int SP>
__device__ __forceinline__ float pool_feature(const HeadArgs& a, int64_t b, int n, float bias,
                                              int64_t chunk_stride) {
  constexpr int RP = 32 / SP;  // positions per round
  float colsum = 0.0f;
  for (int i0 = 0; i0 < a.k; i0 += RP) {
    float v[RP][SP];
#pragma unroll
    for (int ii = 0; ii < RP; ++ii) {
      const int i = min(i0 + ii, a.k - 1);
      const float* P = a.partial + ((b * a.R + i / 16) * 16 + (i % 16)) * a.Hf + n;
#pragma unroll
      for (int c = 0; c < SP; ++c) v[ii][c] = P[min(c, a.S - 1) * chunk_stride];
    }
#pragma unroll
    for (int ii = 0; ii < RP; ++ii) {
      float z = 0.0f;
#pragma unroll
      for (int c = 0; c < SP; ++c)
        if (c < a.S) z += v[ii][c];
      z += bias;
      if (i0 + ii < a.k) colsum += z / (1.0f + __expf(-z));
    }
  }
  return colsum;
}

__global__ __launch_bounds__(256) void sv_head_pool_kernel(HeadArgs a) {
  __shared__ double s_w[4];
  __shared__ int s_tot[256];
  __shared__ int s_last;
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t chunk_stride = a.NB * 16 * static_cast<int64_t>(a.Hf);
  double dot = 0.0;
  for (int n = tid; n < a.Hf; n += 256) {
    const float bias = a.b1 ? a.b1[n] : 0.0f;
    const float colsum = a.S <= 4 ? pool_feature<4>(a, b, n, bias, chunk_stride)
                                  : pool_feature<kHeadMaxSplit>(a, b, n, bias, chunk_stride);
    const float pooled = colsum / static_cast<float>(a.k);
    dot += static_cast<double>(pooled) * static_cast<double>(a.w2[n]);
  }
  dot = wave_sum_d(dot);
  if (lane == 0) s_w[wave] = dot;
  __syncthreads();
  if (tid == 0) {
    const double z = s_w[0] + s_w[1] + s_w[2] + s_w[3] + static_cast<double>(a.b2);
    const double ah = 1.0 / (1.0 + exp(-z));
    double t = floor(ah * static_cast<double>(a.gamma) * static_cast<double>(a.k));
    t = t < 1.0 ? 1.0 : (t > a.k ? static_cast<double>(a.k) : t);
    a.a_hat[b] = static_cast<float>(ah);
    __hip_atomic_store(a.k_hat + b, static_cast<int>(t), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a.off_t) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // k_hat is out before the ticket
      s_last = (__hip_atomic_fetch_add(a.ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                a.B - 1) ? 1 : 0;
    }
  }
  if (!a.off_t) return;
  __syncthreads();
  if (s_last) head_offsets(a, s_tot);
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
  const dim3 grid(static_cast<unsigned>((a.NB + kHeadBlocks - 1) / kHeadBlocks),
                  static_cast<unsigned>((a.Hf + kHeadTileN - 1) / kHeadTileN),
                  static_cast<unsigned>(a.S));
  hipLaunchKernelGGL(sv_head_feat_kernel, grid, dim3(kHeadThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_head_pool(const HeadArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(sv_head_pool_kernel, dim3(static_cast<unsigned>(a.B)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_len_loss(int64_t B, const float* a_hat, const int32_t* accept_len,
                           const int32_t* k_hat, float* loss, float* dloss, hipStream_t st) {
  hipLaunchKernelGGL(sv_len_loss_kernel, dim3(static_cast<unsigned>((B + 255) / 256)), dim3(256), 0,
                     st, B, a_hat, accept_len, k_hat, loss, dloss);
  return hipGetLastError();
}

}  // namespace sv
