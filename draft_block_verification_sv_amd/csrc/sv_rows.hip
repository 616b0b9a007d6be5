// The streaming pass of the verification path (gfx950 / MI355X): every target and
// draft logit is read from HBM exactly once and reduced to per-slice statistics.
//
// One wavefront handles one (row, slice) unit: a slice is 64 lanes x kElemsPerLane
// columns of a target row and, for rows i < k_b, of the draft row it pairs with.  The
// lane issues all of its 16-byte loads first, then:
//   m      = max over the slice (wave butterfly), the exp2 offset K = fp32(m * L2E);
//   S      = sum 2^(l * L2E - K)                          (softmax sum at T = 1);
//   S_T    = sum 2^(l * beta - fp32(m * beta))            (rows with T_b not in {0, 1});
//   arg    = first column attaining m                     (greedy rows, target only);
//   W, G   = sum / max of E_y (l_q - l_p), E_y = 2^(l_q * L2E - K_q)   (draft rows):
// the two quantities that let the clipped reverse-KL (AdaFlash paper, Section 3.1
// equation) be finished without a second pass over HBM (see sv_finalize).
//
// This translation unit is built with IEEE mode off and NaN-free arithmetic assumed:
// logits are finite by the library's contract and nothing here tests for NaN, and it
// spares the max reductions the NaN-quieting instructions IEEE mode requires for
// values assembled from bf16 bit patterns.
#include <float.h>
#include <math.h>

#include "sv_device.h"
#include "sv_layout.h"
#include "sv_launch.h"

namespace sv {

// =========================================================================== rows
#ifndef SV_ROWS_PACKED
#define SV_ROWS_PACKED 1
#endif
#ifndef SV_ROWS_NT
#define SV_ROWS_NT 1
#endif

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// One 16-byte load (optionally with the nontemporal hint: every byte is read once).
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

// Loads the lane's kElemsPerLane elements of one row slice as fp32 (groups of 8
// consecutive columns, 512 columns apart).  Columns >= V read as -inf.
template <int DT, bool VEC, bool FULL>
__device__ __forceinline__ void load_slice(const void* base, int64_t row_off, int64_t col_lane,
                                           int V, float (&x)[kElemsPerLane]) {
  if constexpr (DT == 0) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + row_off;
#pragma unroll
    for (int c = 0; c < kGroups; ++c) {
      const int64_t col = col_lane + c * 512;
      if (VEC && (FULL || col + 8 <= V)) {
        const uint4 r = stream_load(reinterpret_cast<const uint4*>(p + col));
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
        for (int e = 0; e < 8; ++e) x[c * 8 + e] = (col + e < V) ? bf16_at(p + col + e) : -INFINITY;
      }
    }
  } else {
    const float* p = static_cast<const float*>(base) + row_off;
#pragma unroll
    for (int c = 0; c < kGroups; ++c) {
      const int64_t col = col_lane + c * 512;
      if (VEC && (FULL || col + 8 <= V)) {
        const float4 r0 = stream_load(reinterpret_cast<const float4*>(p + col));
        const float4 r1 = stream_load(reinterpret_cast<const float4*>(p + col + 4));
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
        for (int e = 0; e < 8; ++e) x[c * 8 + e] = (col + e < V) ? p[col + e] : -INFINITY;
      }
    }
  }
}

// Row data of one lane for one slice.  Full bf16 slices stay packed (two elements per
// register) and are unpacked where used; everything else is held as fp32.
template <bool PACKED>
struct LaneRow;
template <>
struct LaneRow<true> {
  uint32_t w[kElemsPerLane / 2];
  __device__ __forceinline__ float at(int e) const {
    return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
  }
  // Max of the lane's elements.  The high element of each word is maxed on the raw
  // 32-bit pattern read as fp32 (its low 16 bits only perturb the value inside the
  // high element's bf16 ulp, which never changes the order of distinct bf16 values)
  // and masked at the end; the low elements are unpacked.
  __device__ __forceinline__ float max() const {
    float mh = __uint_as_float(w[0]), ml = bf16_lo(w[0]);
#pragma unroll
    for (int i = 1; i < kElemsPerLane / 2; ++i) {
      mh = fmaxf(mh, __uint_as_float(w[i]));
      ml = fmaxf(ml, bf16_lo(w[i]));
    }
    return fmaxf(bf16_hi(__float_as_uint(mh)), ml);
  }
};
template <>
struct LaneRow<false> {
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
};

template <int DT, bool VEC, bool FULL, bool PACKED>
__device__ __forceinline__ void load_lane_row(const void* base, int64_t row_off, int64_t col_lane,
                                              int V, LaneRow<PACKED>& r) {
  if constexpr (PACKED) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + row_off + col_lane;
#pragma unroll
    for (int c = 0; c < kGroups; ++c) {
      const uint4 v = stream_load(reinterpret_cast<const uint4*>(p + c * 512));
      r.w[c * 4 + 0] = v.x;
      r.w[c * 4 + 1] = v.y;
      r.w[c * 4 + 2] = v.z;
      r.w[c * 4 + 3] = v.w;
    }
  } else {
    load_slice<DT, VEC, FULL>(base, row_off, col_lane, V, r.x);
  }
}

// Statistics of one (row pair | bonus row) slice, written by lane 0 to record `rec`.
template <int DT, bool VEC, bool FULL, bool PAIR, int MODE>
__device__ __forceinline__ void slice_stats(const RowsArgs& a, int64_t t, int64_t d, float beta,
                                            int64_t s, int lane, int64_t rec) {
  constexpr bool PACKED = SV_ROWS_PACKED && DT == 0 && VEC && FULL;
  const int64_t col_lane = s * kSlice + lane * 8;
  LaneRow<PACKED> rp, rq;
  load_lane_row<DT, VEC, FULL, PACKED>(a.target, t * a.ld_t, col_lane, a.V, rp);
  if constexpr (PAIR) load_lane_row<DT, VEC, FULL, PACKED>(a.draft, d * a.ld_d, col_lane, a.V, rq);

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
      if constexpr (!FULL) {
        const int64_t col = col_lane + (e >> 3) * 512 + (e & 7);
        if (col >= a.V) diff = 0.0f;
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
    a.part.mp[rec] = mp;
    a.part.sp[rec] = sp;
    if constexpr (MODE == 2) a.part.stp[rec] = stp;
    if constexpr (MODE == 1) a.part.ap[rec] = arg;
    if constexpr (PAIR) {
      a.part.mq[rec] = mq;
      a.part.sq[rec] = sq;
      a.part.w[rec] = w;
      a.part.g[rec] = g;
      if constexpr (MODE == 2) a.part.stq[rec] = stq;
    }
  }
}

// Mode dispatch.  Independent `if`s rather than an if/else chain: the chain made the
// compiler merge the variants' live ranges and allocate half again as many VGPRs.
template <int DT, bool VEC, bool FULL>
__device__ __forceinline__ void slice_dispatch(const RowsArgs& a, int64_t t, int64_t d, int mode,
                                               float beta, int64_t s, int lane, int64_t rec) {
  if (d >= 0) {
    if (mode == 0) slice_stats<DT, VEC, FULL, true, 0>(a, t, d, beta, s, lane, rec);
    if (mode == 1) slice_stats<DT, VEC, FULL, true, 1>(a, t, d, beta, s, lane, rec);
    if (mode == 2) slice_stats<DT, VEC, FULL, true, 2>(a, t, d, beta, s, lane, rec);
  } else {
    if (mode == 0) slice_stats<DT, VEC, FULL, false, 0>(a, t, d, beta, s, lane, rec);
    if (mode == 1) slice_stats<DT, VEC, FULL, false, 1>(a, t, d, beta, s, lane, rec);
    if (mode == 2) slice_stats<DT, VEC, FULL, false, 2>(a, t, d, beta, s, lane, rec);
  }
}

#ifndef SV_ROWS_WAVES_PER_EU
#define SV_ROWS_WAVES_PER_EU 1
#endif

template <int DT, bool VEC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SV_ROWS_WAVES_PER_EU)))
void sv_rows_kernel(RowsArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = static_cast<int64_t>(blockIdx.x) * kRowsWavesPerBlock + wave;
  if (wave_id >= a.n_waves) return;
  const uint32_t uw = static_cast<uint32_t>(wave_id);
  const int64_t unit = uw / static_cast<uint32_t>(a.n_slices);
  const int64_t s = uw - static_cast<uint32_t>(unit) * static_cast<uint32_t>(a.n_slices);
  if (!a.desc && wave_id == 0 && lane == 0) *a.device_status = 0;
  int64_t t, d;
  int mode;
  float beta;
  if (a.desc) {  // verification: unit = target row
    if (a.glob[0]) return;
    const RowDesc rd = a.desc[unit];
    t = unit;
    d = rd.d;
    mode = rd.mode;
    beta = rd.beta;
  } else {  // clipped reverse-KL only: unit = draft row
    d = unit;
    t = a.p_row_index ? a.p_row_index[unit] : unit;
    if (t < 0 || t >= a.n_target_rows) return;
    mode = 0;
    beta = kL2E;
  }
  const int64_t rec = unit * a.n_slices + s;
  if ((s + 1) * kSlice <= a.V) slice_dispatch<DT, VEC, true>(a, t, d, mode, beta, s, lane, rec);
  else slice_dispatch<DT, VEC, false>(a, t, d, mode, beta, s, lane, rec);
}

// =========================================================================== launch
template <int DT, bool VEC>
static hipError_t launch_rows_t(const RowsArgs& a, hipStream_t st) {
  const int64_t blocks = (a.n_waves + kRowsWavesPerBlock - 1) / kRowsWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((sv_rows_kernel<DT, VEC>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

hipError_t launch_rows(int dtype, bool vec, const RowsArgs& a, hipStream_t st) {
  if (dtype == 0) return vec ? launch_rows_t<0, true>(a, st) : launch_rows_t<0, false>(a, st);
  return vec ? launch_rows_t<1, true>(a, st) : launch_rows_t<1, false>(a, st);
}

}  // namespace sv
