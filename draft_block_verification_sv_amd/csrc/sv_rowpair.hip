// The streaming pass of the verification path on gfx950 (MI355X), fused with the
// per-row finalize.
//
// One 256-thread workgroup owns one target row t and, when t scores a draft
// (position i < k_b), the draft row d it pairs with.  Its four wavefronts stream the
// row (pair) in slices of 64 lanes x kElemsPerLane columns, each wave double-buffering
// its next slice's 16-byte loads behind the current slice's arithmetic, so every logit
// is read from HBM exactly once.  Per slice a wave reduces:
//   m      max (wave butterfly); the exp2 offset is the fp32 product m * L2E;
//   S      sum 2^(l L2E - fp32(m L2E))                      softmax sum at T = 1;
//   S_T    sum 2^(l beta - fp32(m beta))                    rows with T_b not in {0, 1};
//   arg    first column attaining m                         greedy rows (target row);
//   W, G   sum / max of E_y (l_q - l_p), E_y = 2^(l_q L2E - fp32(m_q L2E)) (draft row),
// into a record in LDS.  The workgroup then finishes the row from the records:
//   log2 normalisers LZ = K + log2(sum_s S_s 2^(K_s - K)), fp64, fixed order;
//   the clipped reverse-KL R = sum_y min(delta, q log(q/p)) at T = 1 (AdaFlash paper,
//     Section 3.1 equation; Appendix B.1 for the temperature): per slice,
//       sum_{y in s} t_y  = ln2 2^(K_s - LZq) (L2E W_s + c2 S_s)     exactly, and
//       max_{y in s} t_y <= ln2 2^(K_s - LZq) (L2E G_s + max(c2, 0)),   c2 = LZp - LZq;
//     a slice whose bound stays below delta contributes its exact unclipped sum, any
//     other slice is re-read (it was just streamed, so it comes from cache) and summed
//     entry by entry;
//   the acceptance test u < min(1, p_T(x)/q_T(x)) (paper, Section 2.1), or for T = 0
//     the argmax match (DFlash notes, Section 5.2, worked example #4);
//   the offsets the sampler needs to rebuild p_T and q_T of this row.
//
// Request layout: for batches up to kInlinePlanMaxB requests every workgroup scans k
// itself (no separate plan launch); larger batches read per-row descriptors.
//
// Built with IEEE mode off and NaN-free arithmetic assumed: logits are finite by the
// library's contract, the max reductions then need no NaN-quieting instructions, every
// validity test on inputs is done on bit patterns, and NaN outputs are stored as bits.
#include <float.h>
#include <math.h>

#include "sv_device.h"
#include "sv_layout.h"
#include "sv_launch.h"

#ifndef SV_ROWS_NT
#define SV_ROWS_NT 1
#endif
#ifndef SV_ROWS_PREFETCH
#define SV_ROWS_PREFETCH 1
#endif
#ifndef SV_ROWS_WAVES_PER_EU
#define SV_ROWS_WAVES_PER_EU 1
#endif

namespace sv {

constexpr uint32_t kNaNBits = 0x7fc00000u;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store_nan(float* p) { *reinterpret_cast<uint32_t*>(p) = kNaNBits; }

// Uniform valid iff in [0, 1) (-0 allowed); decided on the bits.
__device__ __forceinline__ bool uniform_ok(float u) {
  const uint32_t b = __float_as_uint(u);
  return b < 0x3f800000u || b == 0x80000000u;
}
// Temperature valid iff +-0 or a positive normal finite number.
__device__ __forceinline__ bool temperature_ok(float T) {
  const uint32_t b = __float_as_uint(T);
  return (b & 0x7fffffffu) == 0u || (b >= 0x00800000u && b < 0x7f800000u);
}

// One 16-byte streaming load (nontemporal: every byte is read once).
template <class T>
__device__ __forceinline__ T stream_load(const T* p) {
  static_assert(sizeof(T) == 16, "16-byte loads");
#if SV_ROWS_NT
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
#else
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
#endif
  T r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// ----------------------------------------------------------------------------- lane data
// A lane's share of one row slice.  Full bf16 slices stay packed, two elements per
// register; everything else (fp32 inputs, ragged tails, unaligned rows) is fp32.
struct PackedRow {
  uint32_t w[kElemsPerLane / 2];
  __device__ __forceinline__ float at(int e) const {
    return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
  }
  // The high element of each word is maxed on the raw 32-bit pattern read as fp32 (the
  // low 16 bits only move the value inside the high element's bf16 ulp, which never
  // reorders distinct bf16 values) and masked at the end; low elements are unpacked.
  __device__ __forceinline__ float max() const {
    float mh = __uint_as_float(w[0]), ml = bf16_lo(w[0]);
#pragma unroll
    for (int i = 1; i < kElemsPerLane / 2; ++i) {
      mh = fmaxf(mh, __uint_as_float(w[i]));
      ml = fmaxf(ml, bf16_lo(w[i]));
    }
    return fmaxf(bf16_hi(__float_as_uint(mh)), ml);
  }
  __device__ __forceinline__ void load(const uint16_t* p) {  // p: this lane's first column
#pragma unroll
    for (int c = 0; c < kGroups; ++c) {
      const uint4 v = stream_load(reinterpret_cast<const uint4*>(p + c * 512));
      w[c * 4 + 0] = v.x;
      w[c * 4 + 1] = v.y;
      w[c * 4 + 2] = v.z;
      w[c * 4 + 3] = v.w;
    }
  }
};

struct FloatRow {
  float x[kElemsPerLane];
  __device__ __forceinline__ float at(int e) const { return x[e]; }
  __device__ __forceinline__ float max() const {
    float m0 = x[0], m1 = x[1];
#pragma unroll
    for (int j = 2; j < kElemsPerLane; j += 2) {
      m0 = fmaxf(m0, x[j]);
      m1 = fmaxf(m1, x[j + 1]);
    }
    return fmaxf(m0, m1);
  }
  // Columns >= V read as -inf.  VEC: the row allows 16-byte loads.
  template <int DT, bool VEC>
  __device__ __forceinline__ void load(const void* row, int64_t col_lane, int V) {
#pragma unroll
    for (int c = 0; c < kGroups; ++c) {
      const int64_t col = col_lane + c * 512;
      if constexpr (DT == 0) {
        const uint16_t* p = static_cast<const uint16_t*>(row) + col;
        if (VEC && col + 8 <= V) {
          const uint4 r = stream_load(reinterpret_cast<const uint4*>(p));
          x[c * 8 + 0] = bf16_lo(r.x);
          x[c * 8 + 1] = bf16_hi(r.x);
          x[c * 8 + 2] = bf16_lo(r.y);
          x[c * 8 + 3] = bf16_hi(r.y);
          x[c * 8 + 4] = bf16_lo(r.z);
          x[c * 8 + 5] = bf16_hi(r.z);
          x[c * 8 + 6] = bf16_lo(r.w);
          x[c * 8 + 7] = bf16_hi(r.w);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[c * 8 + e] = (col + e < V) ? bf16_at(p + e) : -INFINITY;
        }
      } else {
        const float* p = static_cast<const float*>(row) + col;
        if (VEC && col + 8 <= V) {
          const float4 r0 = stream_load(reinterpret_cast<const float4*>(p));
          const float4 r1 = stream_load(reinterpret_cast<const float4*>(p + 4));
          x[c * 8 + 0] = r0.x;
          x[c * 8 + 1] = r0.y;
          x[c * 8 + 2] = r0.z;
          x[c * 8 + 3] = r0.w;
          x[c * 8 + 4] = r1.x;
          x[c * 8 + 5] = r1.y;
          x[c * 8 + 6] = r1.z;
          x[c * 8 + 7] = r1.w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[c * 8 + e] = (col + e < V) ? p[e] : -INFINITY;
        }
      }
    }
  }
};

// ----------------------------------------------------------------------------- slice records
struct SliceRecs {  // LDS, structure of arrays, one entry per slice
  float mp[kMaxSlices], sp[kMaxSlices], stp[kMaxSlices];
  int ap[kMaxSlices];
  float mq[kMaxSlices], sq[kMaxSlices], stq[kMaxSlices], w[kMaxSlices], g[kMaxSlices];
};

// Statistics of one slice of the row (pair); lane 0 writes the record of slice s.
// col_lane: column of the lane's first element (argmax positions, padding mask).
// MASK: columns >= V are padding (-inf) whose difference term must be zeroed.
template <bool PAIR, int MODE, bool MASK, class Row>
__device__ __forceinline__ void slice_stats(const Row& rp, const Row& rq, float beta, int s,
                                            int64_t col_lane, int V, int lane, SliceRecs& R) {
  const float mp = wave_max(rp.max());
  const float op = -(mp * kL2E);
  float mq = 0.0f, oq = 0.0f;
  if constexpr (PAIR) {
    mq = wave_max(rq.max());
    oq = -(mq * kL2E);
  }
  float otp = 0.0f, otq = 0.0f;
  if constexpr (MODE == 2) {
    otp = -(mp * beta);
    if constexpr (PAIR) otq = -(mq * beta);
  }
  float sp0 = 0.f, sp1 = 0.f, sq0 = 0.f, sq1 = 0.f, w0 = 0.f, w1 = 0.f, g = -INFINITY;
  float stp0 = 0.f, stp1 = 0.f, stq0 = 0.f, stq1 = 0.f;
#pragma unroll
  for (int e = 0; e < kElemsPerLane; ++e) {
    const bool odd = e & 1;
    const float xp = rp.at(e);
    const float ep = fast_exp2(__builtin_fmaf(xp, kL2E, op));
    if (odd) sp1 += ep; else sp0 += ep;
    if constexpr (MODE == 2) {
      const float etp = fast_exp2(__builtin_fmaf(xp, beta, otp));
      if (odd) stp1 += etp; else stp0 += etp;
    }
    if constexpr (PAIR) {
      const float xq = rq.at(e);
      const float eq = fast_exp2(__builtin_fmaf(xq, kL2E, oq));
      float diff = xq - xp;
      if constexpr (MASK) {
        if (col_lane + (e >> 3) * 512 + (e & 7) >= V) diff = 0.0f;
      }
      if (odd) {
        sq1 += eq;
        w1 = __builtin_fmaf(eq, diff, w1);
      } else {
        sq0 += eq;
        w0 = __builtin_fmaf(eq, diff, w0);
      }
      g = fmaxf(g, eq * diff);
      if constexpr (MODE == 2) {
        const float etq = fast_exp2(__builtin_fmaf(xq, beta, otq));
        if (odd) stq1 += etq; else stq0 += etq;
      }
    }
  }
  const float sp = wave_sum(sp0 + sp1);
  float stp = 0.f, sq = 0.f, stq = 0.f, w = 0.f;
  if constexpr (MODE == 2) stp = wave_sum(stp0 + stp1);
  if constexpr (PAIR) {
    sq = wave_sum(sq0 + sq1);
    w = wave_sum(w0 + w1);
    g = wave_max(g);
    if constexpr (MODE == 2) stq = wave_sum(stq0 + stq1);
  }
  int arg = 0;
  if constexpr (MODE == 1) {
    int best = 0x7fffffff;
#pragma unroll
    for (int e = kElemsPerLane - 1; e >= 0; --e)
      if (rp.at(e) == mp) best = static_cast<int>(col_lane + (e >> 3) * 512 + (e & 7));
    arg = wave_min_i(best);
  }
  if (lane == 0) {
    R.mp[s] = mp;
    R.sp[s] = sp;
    if constexpr (MODE == 2) R.stp[s] = stp;
    if constexpr (MODE == 1) R.ap[s] = arg;
    if constexpr (PAIR) {
      R.mq[s] = mq;
      R.sq[s] = sq;
      R.w[s] = w;
      R.g[s] = g;
      if constexpr (MODE == 2) R.stq[s] = stq;
    }
  }
}

// Streams the wave's slices (s = wave, wave + 4, ...) of the row (pair).
// Full bf16 slices of 16-byte-aligned rows: packed, next slice prefetched while the
// current one is reduced.  The ragged last slice and every other case: fp32, masked.
template <int DT, bool VEC, bool PAIR, int MODE>
__device__ __forceinline__ void stream_row(const void* prow, const void* qrow, float beta, int V,
                                           int n_slices, int wave, int lane, SliceRecs& R) {
  const int n_full = V / kSlice;
  int s = wave;
  if constexpr (DT == 0 && VEC && !SV_ROWS_PREFETCH) {
    const uint16_t* P = static_cast<const uint16_t*>(prow) + lane * 8;
    const uint16_t* Q = static_cast<const uint16_t*>(qrow) + lane * 8;
    for (; s < n_full; s += kRowWaves) {
      PackedRow ap, aq;
      ap.load(P + static_cast<int64_t>(s) * kSlice);
      if constexpr (PAIR) aq.load(Q + static_cast<int64_t>(s) * kSlice);
      slice_stats<PAIR, MODE, false>(ap, aq, beta, s, static_cast<int64_t>(s) * kSlice + lane * 8,
                                     V, lane, R);
    }
  }
  if constexpr (DT == 0 && VEC && SV_ROWS_PREFETCH) {
    const uint16_t* P = static_cast<const uint16_t*>(prow) + lane * 8;
    const uint16_t* Q = static_cast<const uint16_t*>(qrow) + lane * 8;
    PackedRow ap, aq, bp, bq;
    if (s < n_full) {
      ap.load(P + static_cast<int64_t>(s) * kSlice);
      if constexpr (PAIR) aq.load(Q + static_cast<int64_t>(s) * kSlice);
    }
    while (s < n_full) {
      const int s2 = s + kRowWaves;
      if (s2 < n_full) {
        bp.load(P + static_cast<int64_t>(s2) * kSlice);
        if constexpr (PAIR) bq.load(Q + static_cast<int64_t>(s2) * kSlice);
      }
      slice_stats<PAIR, MODE, false>(ap, aq, beta, s, static_cast<int64_t>(s) * kSlice + lane * 8,
                                     V, lane, R);
      if (s2 >= n_full) {
        s = s2;
        break;
      }
      const int s3 = s2 + kRowWaves;
      if (s3 < n_full) {
        ap.load(P + static_cast<int64_t>(s3) * kSlice);
        if constexpr (PAIR) aq.load(Q + static_cast<int64_t>(s3) * kSlice);
      }
      slice_stats<PAIR, MODE, false>(bp, bq, beta, s2,
                                     static_cast<int64_t>(s2) * kSlice + lane * 8, V, lane, R);
      s = s3;
    }
  }
  for (; s < n_slices; s += kRowWaves) {  // every slice not handled above
    const int64_t col_lane = static_cast<int64_t>(s) * kSlice + lane * 8;
    FloatRow fp, fq;
    fp.template load<DT, VEC>(prow, col_lane, V);
    if constexpr (PAIR) fq.template load<DT, VEC>(qrow, col_lane, V);
    slice_stats<PAIR, MODE, true>(fp, fq, beta, s, col_lane, V, lane, R);
  }
}

// ----------------------------------------------------------------------------- block helpers
// Fixed-order reductions over the 256-thread workgroup: wave butterfly, then the four
// wave results in order.  `red` holds kRowWaves doubles.
__device__ __forceinline__ double block_sum_d(double v, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_d(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) r += red[w];
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_max_f(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_max_f(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kRowWaves; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ int block_min_i(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_min_int(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int r = red[0];
#pragma unroll
  for (int w = 1; w < kRowWaves; ++w) r = min(r, red[w]);
  __syncthreads();
  return r;
}

// log2 normaliser of the row from the slice records (m[], S[]) at scale `scale`:
// K + log2(sum_s S_s 2^(fp32(m_s scale) - K)), K = fp32(M scale).
__device__ __forceinline__ double row_lz(const float* m, const float* S, float M, float scale,
                                         int n_slices, double* red) {
  const float K = M * scale;
  double acc = 0.0;
  for (int s = threadIdx.x; s < n_slices; s += kRowThreads)
    acc += static_cast<double>(S[s]) * exp2(static_cast<double>(m[s] * scale) - static_cast<double>(K));
  return static_cast<double>(K) + log2(block_sum_d(acc, red));
}

template <int DT>
__device__ __forceinline__ float logit_at(const void* row, int64_t col) {
  if constexpr (DT == 0) return bf16_at(static_cast<const uint16_t*>(row) + col);
  else return static_cast<const float*>(row)[col];
}

// Clipped reverse-KL of the row pair from its records; slices whose bound may reach
// delta are re-read and summed entry by entry (each by one wave).
template <int DT>
__device__ __forceinline__ double row_clipped_rkl(const void* prow, const void* qrow, int V, int n_slices,
                                  double LZp, double LZq, float delta, const SliceRecs& R,
                                  double* contrib, int* failed, int* s_nfail, double* red) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const double c2 = LZp - LZq;
  const double c2pos = c2 > 0.0 ? c2 : 0.0;
  if (tid == 0) *s_nfail = 0;
  __syncthreads();
  for (int s = tid; s < n_slices; s += kRowThreads) {
    const double scale = kLn2 * exp2(static_cast<double>(R.mq[s] * kL2E) - LZq);
    const double bound = scale * (static_cast<double>(kL2E) * R.g[s] + c2pos * 1.0001);
    contrib[s] = scale * (static_cast<double>(kL2E) * R.w[s] + c2 * R.sq[s]);
    if (!(bound * 1.0001 < static_cast<double>(delta))) failed[atomicAdd(s_nfail, 1)] = s;
  }
  __syncthreads();
  const int nfail = *s_nfail;
  const float c2f = static_cast<float>(c2);
  for (int f = wave; f < nfail; f += kRowWaves) {
    const int s = failed[f];
    float part = 0.0f;
#pragma unroll
    for (int c = 0; c < kGroups; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t col = static_cast<int64_t>(s) * kSlice + c * 512 + lane * 8 + e;
        if (col < V) {
          const float lq = logit_at<DT>(qrow, col);
          const float lp = logit_at<DT>(prow, col);
          const float q = fast_exp2(static_cast<float>(static_cast<double>(lq) * kL2E - LZq));
          const float term = q * static_cast<float>(kLn2) * __builtin_fmaf(lq - lp, kL2E, c2f);
          part += fminf(term, delta);
        }
      }
    }
    const double direct = wave_sum_d(static_cast<double>(part));
    if (lane == 0) contrib[s] = direct;
  }
  __syncthreads();
  double acc = 0.0;
  for (int s = tid; s < n_slices; s += kRowThreads) acc += contrib[s];
  return block_sum_d(acc, red);
}

// ----------------------------------------------------------------------------- kernel
struct RowCtx {
  int64_t t, d;  // target row, draft row (-1: bonus row)
  int64_t b;     // request (-1: clipped reverse-KL only)
  int mode;      // 0: T = 1, 1: greedy, 2: other T
  float beta;
  int row_flags;
};

template <int DT, bool VEC, bool PAIR, int MODE>
__device__ __forceinline__ void rowpair_body(const RowPairArgs& a, const RowCtx& ctx, SliceRecs& R, double* contrib,
                             int* failed, int* s_nfail, double* red_d, float* red_f, int* red_i,
                             int x, float lpx, float lqx) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int V = a.V;
  const int n_slices = static_cast<int>(a.n_slices);
  const void* prow = static_cast<const char*>(a.target) + ctx.t * a.ld_t * (DT == 0 ? 2 : 4);
  const void* qrow = static_cast<const char*>(a.draft) + (PAIR ? ctx.d : 0) * a.ld_d * (DT == 0 ? 2 : 4);

  stream_row<DT, VEC, PAIR, MODE>(prow, qrow, ctx.beta, V, n_slices, wave, lane, R);
  __syncthreads();

  // target row: normalisers at T = 1 and T_b, argmax
  float m = -INFINITY;
  for (int s = tid; s < n_slices; s += kRowThreads) m = fmaxf(m, R.mp[s]);
  const float Mp = block_max_f(m, red_f);
  const double LZ1p = row_lz(R.mp, R.sp, Mp, kL2E, n_slices, red_d);
  const double LZTp = (MODE == 2) ? row_lz(R.mp, R.stp, Mp, ctx.beta, n_slices, red_d) : LZ1p;
  int argp = 0;
  if constexpr (MODE == 1) {
    int best = 0x7fffffff;
    for (int s = tid; s < n_slices; s += kRowThreads)
      if (R.mp[s] == Mp) best = min(best, R.ap[s]);
    argp = block_min_i(best, red_i);
  }
  const float scale_T = (MODE == 2) ? ctx.beta : kL2E;
  if (tid == 0 && ctx.b >= 0) {
    const float KT = Mp * scale_T;
    a.t_off[ctx.t] = -KT;
    a.t_lz[ctx.t] = static_cast<float>(LZTp - static_cast<double>(KT));
    a.t_beta[ctx.t] = scale_T;
    a.t_arg[ctx.t] = argp;
    a.row_flags[ctx.t] = ctx.row_flags;
  }
  if constexpr (!PAIR) return;

  // draft row
  m = -INFINITY;
  for (int s = tid; s < n_slices; s += kRowThreads) m = fmaxf(m, R.mq[s]);
  const float Mq = block_max_f(m, red_f);
  const double LZ1q = row_lz(R.mq, R.sq, Mq, kL2E, n_slices, red_d);
  const double LZTq = (MODE == 2) ? row_lz(R.mq, R.stq, Mq, ctx.beta, n_slices, red_d) : LZ1q;
  if (a.rkl_out) {
    const double Rk = row_clipped_rkl<DT>(prow, qrow, V, n_slices, LZ1p, LZ1q, a.delta, R, contrib,
                                          failed, s_nfail, red_d);
    if (tid == 0) a.rkl_out[ctx.d] = static_cast<float>(Rk);
  }
  if (tid == 0 && ctx.b >= 0) {
    const float KT = Mq * scale_T;
    a.d_off[ctx.d] = -KT;
    a.d_lz[ctx.d] = static_cast<float>(LZTq - static_cast<double>(KT));
    int accept = 0;
    if (ctx.row_flags == 0) {  // the request's own flags are combined by the sampler
      const double Lp = static_cast<double>(lpx) * scale_T - LZTp;  // log2 p_T(x)
      const double Lq = static_cast<double>(lqx) * scale_T - LZTq;  // log2 q_T(x)
      if constexpr (MODE == 1) {
        accept = (x == argp) ? 1 : 0;
      } else {
        const double ratio = fmin(1.0, exp2(Lp - Lq));
        accept = (static_cast<double>(a.uniforms[ctx.t]) < ratio) ? 1 : 0;
      }
      if (a.p_at) a.p_at[ctx.d] = static_cast<float>(exp2(Lp));
      if (a.q_at) a.q_at[ctx.d] = static_cast<float>(exp2(Lq));
    } else {
      if (a.p_at) store_nan(a.p_at + ctx.d);
      if (a.q_at) store_nan(a.q_at + ctx.d);
    }
    a.acc[ctx.d] = accept;
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kRowThreads) __attribute__((amdgpu_waves_per_eu(SV_ROWS_WAVES_PER_EU)))
void sv_rowpair_kernel(RowPairArgs a) {
  __shared__ SliceRecs R;
  __shared__ double contrib[kMaxSlices];
  __shared__ int failed[kMaxSlices];
  __shared__ int s_nfail;
  __shared__ double red_d[kRowWaves];
  __shared__ float red_f[kRowWaves];
  __shared__ int red_i[kRowWaves];
  __shared__ int s_req, s_off, s_t, s_void, s_x;
  __shared__ float s_lpx, s_lqx;
  const int tid = threadIdx.x;
  const int64_t unit = blockIdx.x;

  RowCtx ctx;
  if (a.rkl_only) {  // unit = draft row, paired with target row p_row_index[unit]
    ctx.d = unit;
    ctx.t = a.p_row_index ? a.p_row_index[unit] : unit;
    ctx.b = -1;
    ctx.mode = 0;
    ctx.beta = kL2E;
    ctx.row_flags = 0;
    if (ctx.t < 0 || ctx.t >= a.n_target_rows) {
      if (tid == 0) {
        store_nan(a.rkl_out + unit);
        a.row_flags[unit] = 2;  // SV_DEV_ROWS_MISMATCH
      }
      return;
    }
    if (tid == 0) a.row_flags[unit] = 0;
    rowpair_body<DT, VEC, true, 0>(a, ctx, R, contrib, failed, &s_nfail, red_d, red_f, red_i, 0,
                                   0.0f, 0.0f);
    return;
  }

  // ---- verification: units 0 .. n_d-1 are the draft rows (each with its target row),
  // units n_d .. n_d+B-1 the bonus rows; the half-size bonus units run last and fill
  // the tail of the grid.
  if (a.desc) {  // large batch: descriptors and offsets from sv_plan
    if (a.glob[0]) {
      if (tid == 0 && unit < a.n_d) {
        if (a.rkl_out) store_nan(a.rkl_out + unit);
        if (a.p_at) store_nan(a.p_at + unit);
        if (a.q_at) store_nan(a.q_at + unit);
      }
      return;
    }
    if (tid == 0) {
      const RowDesc rd = a.desc[unit];
      s_req = rd.b;
      s_off = a.off_t[rd.b];
      s_t = rd.t;
    }
    __syncthreads();
  } else {  // every workgroup scans k itself (B <= kInlinePlanMaxB, 8 requests per thread)
    if (tid == 0) {
      s_void = 0;
      s_req = -1;
    }
    __syncthreads();
    int kk[kInlinePerThread];
    int tot = 0, bad = 0;
#pragma unroll
    for (int e = 0; e < kInlinePerThread; ++e) {
      const int64_t j = static_cast<int64_t>(tid) * kInlinePerThread + e;
      int v = 0;
      if (j < a.B) {
        v = a.k[j];
        if (v < 1 || v > a.k_max) {
          bad = 1;
          v = 0;
        }
        v += 1;  // target rows of the request
      }
      kk[e] = v;
      tot += v;
    }
    // exclusive scan of the per-thread totals (fixed order)
    const int lane = tid & 63, wave = tid >> 6;
    int incl = tot;
#pragma unroll
    for (int dd = 1; dd < 64; dd <<= 1) {
      const int o = __shfl_up(incl, dd, 64);
      if (lane >= dd) incl += o;
    }
    if (lane == 63) red_i[wave] = incl;
    if (bad) atomicOr(&s_void, 1);
    __syncthreads();
    int base = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) {
      if (w < wave) base += red_i[w];
      all += red_i[w];
    }
    // units 0 .. n_d-1 are the draft rows in packed order, then the B bonus rows
    int off = base + incl - tot;
#pragma unroll
    for (int e = 0; e < kInlinePerThread; ++e) {
      const int64_t j = static_cast<int64_t>(tid) * kInlinePerThread + e;
      const int64_t doff = off - j;  // first draft row of request j
      if (kk[e] > 0) {
        if (unit < a.n_d && unit >= doff && unit < doff + kk[e] - 1) {
          s_req = static_cast<int>(j);
          s_off = off;
          s_t = off + (unit - doff);
        } else if (unit >= a.n_d && unit - a.n_d == j) {
          s_req = static_cast<int>(j);
          s_off = off;
          s_t = off + kk[e] - 1;
        }
      }
      off += kk[e];
    }
    if (tid == 0 && !s_void && static_cast<int64_t>(all) != a.n_d + a.B) atomicOr(&s_void, 2);
    __syncthreads();
    const int vd = s_void;
    if (unit == 0 && tid == 0) {
      a.glob[0] = vd ? 1 : 0;
      *a.device_status = vd ? ((vd & 1) ? 1 : 2) : 0;
    }
    if (vd) {
      if (tid == 0 && unit < a.n_d) {
        if (a.rkl_out) store_nan(a.rkl_out + unit);
        if (a.p_at) store_nan(a.p_at + unit);
        if (a.q_at) store_nan(a.q_at + unit);
      }
      return;
    }
  }
  if (s_req < 0) return;  // unreachable when the layout is valid
  const int64_t b = s_req;
  const int64_t off = s_off;
  const int kb = a.k[b];
  ctx.t = s_t;
  const int i = static_cast<int>(ctx.t - off);
  ctx.b = b;
  ctx.d = (i < kb) ? (off - b + i) : -1;
  const float T = a.temperature ? a.temperature[b] : 1.0f;
  int flags = 0;
  ctx.mode = 0;
  ctx.beta = kL2E;
  if (!temperature_ok(T)) {
    flags |= 8;
  } else if (T == 0.0f) {
    ctx.mode = 1;
  } else if (T != 1.0f) {
    ctx.mode = 2;
    ctx.beta = kL2E / T;
  }
  if (!uniform_ok(a.uniforms[ctx.t])) flags |= 16;
  if (i == 0 && tid == 0 && !a.desc) a.off_t[b] = static_cast<int32_t>(off);
  // the draft token and the two logits at it, fetched before the stream starts
  if (tid == 0) {
    s_x = -1;
    s_lpx = 0.0f;
    s_lqx = 0.0f;
    if (ctx.d >= 0) {
      const int32_t x = a.tokens[ctx.d];
      if (x < 0 || x >= a.V) {
        flags |= 4;
      } else {
        s_x = x;
        s_lpx = logit_at<DT>(static_cast<const char*>(a.target) + ctx.t * a.ld_t * (DT == 0 ? 2 : 4), x);
        s_lqx = logit_at<DT>(static_cast<const char*>(a.draft) + ctx.d * a.ld_d * (DT == 0 ? 2 : 4), x);
      }
    }
  }
  ctx.row_flags = flags;  // token bit is only known to thread 0; thread 0 writes the flags
  __syncthreads();
  const int x = s_x;
  const float lpx = s_lpx, lqx = s_lqx;
  if (ctx.d >= 0) {
    if (ctx.mode == 0) rowpair_body<DT, VEC, true, 0>(a, ctx, R, contrib, failed, &s_nfail, red_d, red_f, red_i, x, lpx, lqx);
    if (ctx.mode == 1) rowpair_body<DT, VEC, true, 1>(a, ctx, R, contrib, failed, &s_nfail, red_d, red_f, red_i, x, lpx, lqx);
    if (ctx.mode == 2) rowpair_body<DT, VEC, true, 2>(a, ctx, R, contrib, failed, &s_nfail, red_d, red_f, red_i, x, lpx, lqx);
  } else {
    if (ctx.mode == 0) rowpair_body<DT, VEC, false, 0>(a, ctx, R, contrib, failed, &s_nfail, red_d, red_f, red_i, x, lpx, lqx);
    if (ctx.mode == 1) rowpair_body<DT, VEC, false, 1>(a, ctx, R, contrib, failed, &s_nfail, red_d, red_f, red_i, x, lpx, lqx);
    if (ctx.mode == 2) rowpair_body<DT, VEC, false, 2>(a, ctx, R, contrib, failed, &s_nfail, red_d, red_f, red_i, x, lpx, lqx);
  }
}

// ----------------------------------------------------------------------------- launch
hipError_t launch_rowpair(int dtype, bool vec, const RowPairArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.n_units));
  if (a.n_units == 0) return hipSuccess;
  if (dtype == 0) {
    if (vec) hipLaunchKernelGGL((sv_rowpair_kernel<0, true>), grid, dim3(kRowThreads), 0, st, a);
    else hipLaunchKernelGGL((sv_rowpair_kernel<0, false>), grid, dim3(kRowThreads), 0, st, a);
  } else {
    if (vec) hipLaunchKernelGGL((sv_rowpair_kernel<1, true>), grid, dim3(kRowThreads), 0, st, a);
    else hipLaunchKernelGGL((sv_rowpair_kernel<1, false>), grid, dim3(kRowThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace sv
