// Re-reading one lane's columns of a row pair after the streaming pass, shared by the streaming
// kernel (clipped terms near the clip) and the draw kernel (exact sums of heavy lanes).
//
// Lane t < kRowThreads of a row streamed by one 256-thread workgroup owns, in each slice
// s = t / 64 + 4 j, kGroups groups of 8 consecutive columns (slice s, group g: columns
// s kSlice + g 512 + (t % 64) 8 ...).  A split row's parts fold their four waves into 64 lanes:
// lane kRowThreads + l owns those groups of thread l in every slice.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_device.h"
#include "sv_layout.h"

namespace sv {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resources: stride 0, byte-addressed, 32-bit data format word.
constexpr int kBufWord3 = 0x00020000;

// Some lanes have their columns read again after the stream: a lane's pieces (8 consecutive
// columns each: piece j is group j % kGroups of the lane's (j / kGroups)-th slice) are cut into
// lane_blocks(src) blocks of consecutive pieces, each read by one wave; piece j of a block goes
// to thread (j - first) % 64, two pieces in flight per thread, every load issued before any
// arithmetic.  A folded lane (four times the columns of a streaming lane) is read by four
// waves, one block each, so that it costs a wave no more than a streaming lane.  f sees the
// block's columns in a fixed order per thread; the wave's sums then combine in a fixed tree,
// and the blocks in block order, so the results do not depend on which lanes were listed or
// in what order.
// The 8 logits of one piece as raw words: a bf16 piece is one 16-byte word, an fp32 piece two.
// VEC rows are read through a bounds-checked buffer (a piece that is not valid, or the part of
// one past V, reads zeros); other rows column by column with the column clamped into the row.
template <int DT, bool VEC>
struct Piece {
  u32x4_t w[DT == 0 ? 1 : 2];
  __device__ __forceinline__ void load(const void* row, __amdgpu_buffer_rsrc_t rs, int64_t col0,
                                       bool ok, int V) {
    constexpr int es = DT == 0 ? 2 : 4;
    if constexpr (VEC) {
      const int off = ok ? static_cast<int>(col0) * es : V * es;
      w[0] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
      if constexpr (DT == 1) w[DT] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0);
    } else {
      int64_t c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) c[e] = ok ? (col0 + e < V ? col0 + e : V - 1) : 0;
      if constexpr (DT == 0) {
        const uint16_t* r = static_cast<const uint16_t*>(row);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[0][e] = static_cast<uint32_t>(r[c[2 * e]]) | (static_cast<uint32_t>(r[c[2 * e + 1]]) << 16);
      } else {
        const uint32_t* r = static_cast<const uint32_t*>(row);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[0][e] = r[c[e]];
          w[DT][e] = r[c[e + 4]];
        }
      }
    }
  }
  __device__ __forceinline__ float at(int e) const {
    if constexpr (DT == 0) return (e & 1) ? bf16_hi(w[0][e >> 1]) : bf16_lo(w[0][e >> 1]);
    else return __uint_as_float(e < 4 ? w[0][e] : w[DT][e - 4]);
  }
};

// for_lane_columns_all: f(l_p, l_q, valid) for every column slot of the lane's pieces, valid
// or not (an invalid slot holds zeros, or a clamped column's logits), with no branch around f:
// f masks by `valid` itself.  for_lane_columns: f(l_p, l_q) for the valid columns only.
__device__ __forceinline__ int lane_blocks(int src) { return src >= kRowThreads ? kRowWaves : 1; }

template <int DT, bool VEC, class F>
__device__ __forceinline__ void for_lane_columns_all(const void* prow, const void* qrow, int V,
                                                     int n_slices, int src, int block, int lane,
                                                     F&& f) {
  constexpr int es = DT == 0 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t RQ =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(qrow), 0, V * es, kBufWord3);
  const __amdgpu_buffer_rsrc_t RP =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(prow), 0, V * es, kBufWord3);
  const bool folded = src >= kRowThreads;
  const int sw = folded ? 0 : src >> 6, sl = src & 63, ss = folded ? 1 : kRowWaves;
  // the lane's slices are sw, sw + ss, ... < n_slices: kGroups pieces each
  const int n_pieces = ((n_slices - sw + ss - 1) / ss) * kGroups;
  const int per = (n_pieces + lane_blocks(src) - 1) / lane_blocks(src);
  const int jb = block * per, je = min(n_pieces, jb + per);
  for (int j0 = jb; j0 < je; j0 += 2 * 64) {
    Piece<DT, VEC> pq[2], pp[2];
    int64_t col[2];
    bool ok[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = j0 + u * 64 + lane;
      const int slice = sw + (j / kGroups) * ss;  // < n_slices whenever j < je
      col[u] = static_cast<int64_t>(slice) * kSlice + (j % kGroups) * 512 + sl * 8;
      ok[u] = j < je && col[u] < V;
      pq[u].load(qrow, RQ, col[u], ok[u], V);
      pp[u].load(prow, RP, col[u], ok[u], V);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) f(pp[u].at(e), pq[u].at(e), ok[u] && col[u] + e < V);
  }
}

template <int DT, bool VEC, class F>
__device__ __forceinline__ void for_lane_columns(const void* prow, const void* qrow, int V,
                                                 int n_slices, int src, int block, int lane, F&& f) {
  for_lane_columns_all<DT, VEC>(prow, qrow, V, n_slices, src, block, lane, [&](float lp, float lq, bool valid) {
    if (valid) f(lp, lq);
  });
}

// The fp64 sums of one block of a lane against the lane's offsets kp, kq (a wave; every thread
// gets the sums): S_p = sum 2^(l_p L2E - kp), S_q = sum E_q, E_q = 2^(l_q L2E - kq),
// W = sum E_q (l_q - l_p).
struct LaneSums {
  double sp, sq, w;
};
template <int DT, bool VEC>
__device__ __forceinline__ LaneSums exact_lane_sums(const void* prow, const void* qrow, int V,
                                                    int n_slices, int src, int block, int lane,
                                                    double kp, double kq) {
  LaneSums r{0.0, 0.0, 0.0};
  for_lane_columns_all<DT, VEC>(prow, qrow, V, n_slices, src, block, lane, [&](float lp, float lq, bool valid) {
    const double eq = exp2_bulk(static_cast<double>(lq) * static_cast<double>(kL2E) - kq);
    const double ep = exp2_bulk(static_cast<double>(lp) * static_cast<double>(kL2E) - kp);
    r.sp += valid ? ep : 0.0;
    r.sq += valid ? eq : 0.0;
    r.w += valid ? eq * (static_cast<double>(lq) - static_cast<double>(lp)) : 0.0;
  });
  r.sp = wave_sum_d(r.sp);
  r.sq = wave_sum_d(r.sq);
  r.w = wave_sum_d(r.w);
  return r;
}

}  // namespace sv
