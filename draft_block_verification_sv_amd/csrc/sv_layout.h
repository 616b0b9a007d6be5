// Work decomposition constants and the caller-workspace layout, shared by the
// host API and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sv {

// The streaming kernel gives one wavefront one slice of one row (pair): 64 lanes x
// kElemsPerLane elements, in groups of 8 consecutive columns 512 columns apart.  At
// 32 elements a bf16 slice of a row pair is 8 KiB, read with eight 16-byte loads per
// lane, all issued before any arithmetic.
#ifndef SV_ELEMS_PER_LANE
#define SV_ELEMS_PER_LANE 32
#endif
constexpr int kElemsPerLane = SV_ELEMS_PER_LANE;
static_assert(kElemsPerLane % 8 == 0 && kElemsPerLane >= 8, "groups of 8 columns per lane");
constexpr int kGroups = kElemsPerLane / 8;
constexpr int kSlice = 64 * kElemsPerLane;
constexpr int kRowsWavesPerBlock = 4;       // 256-thread workgroups
// The sampler gives one 256-thread workgroup 2048 columns (8 per thread).
constexpr int kChunk = 2048;
constexpr int kSampleThreads = 256;
constexpr int kFinWavesPerBlock = 4;

inline int64_t n_slices_for(int64_t V) { return (V + kSlice - 1) / kSlice; }
inline int64_t n_chunks_for(int64_t V) { return (V + kChunk - 1) / kChunk; }

// Per target row, filled by the plan kernel.
struct RowDesc {
  int32_t d;     // paired draft row, or -1 for the bonus row
  int32_t b;     // request
  int32_t mode;  // 0: T = 1, 1: greedy (T = 0), 2: any other T
  float beta;    // log2(e) / T in fp32 (log2(e) for modes 0 and 1)
};

// Per (unit, slice) partial statistics written by the streaming kernel (SoA).
// For a row with slice maximum m, the sums are taken relative to the fp32 offset
// -(m * kL2E) (or -(m * beta)) that the kernel used, so a reader can rebuild the
// exact shift.
struct Partials {
  float* mp;    // max of the target slice
  float* sp;    // sum exp2(l_p * kL2E - m_p * kL2E)
  float* stp;   // sum exp2(l_p * beta - m_p * beta)           (mode 2 only)
  int32_t* ap;  // first column attaining m_p                  (mode 1 only)
  float* mq;    // max of the draft slice
  float* sq;    // sum E_y, E_y = exp2(l_q * kL2E - m_q * kL2E)
  float* stq;   // sum exp2(l_q * beta - m_q * beta)           (mode 2 only)
  float* w;     // sum E_y * (l_q - l_p)
  float* g;     // max E_y * (l_q - l_p)
};

// Device pointers carved out of the caller's workspace.
struct Workspace {
  int32_t* glob;       // [4]: [0] call void (bad lengths / row count)
  int32_t* off_t;      // [B + 1] first target row of each request
  int32_t* req_flags;  // [B] SV_DEV_* bits of each request
  RowDesc* desc;       // [n_t]
  Partials part;       // [n_units * n_slices] each
  float* t_off;        // [n_t] -(M * beta) for the sampler's temperature
  float* t_lz;         // [n_t] log2 normaliser relative to that offset
  int32_t* t_arg;      // [n_t] argmax (lowest id)
  float* d_off;        // [n_d]
  float* d_lz;         // [n_d]
  int32_t* acc;        // [n_d] acceptance flag
  double* chunk_r;     // [B * n_chunks] sampler mass per chunk
  double* chunk_p;     // [B * n_chunks] p_T mass per chunk (zero-residual fallback)
};

struct Dims {
  int64_t B, n_t, n_d, V, n_units, n_slices, n_chunks;
};

// Lays out the regions (each 256-byte aligned) and returns the total byte count.
// With base == nullptr only the size is computed.
inline size_t carve(const Dims& d, Workspace* ws, char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~size_t(255);
    return p;
  };
  Workspace w{};
  const size_t np = static_cast<size_t>(d.n_units * d.n_slices);
  w.glob = reinterpret_cast<int32_t*>(take(4 * sizeof(int32_t)));
  w.off_t = reinterpret_cast<int32_t*>(take((d.B + 1) * sizeof(int32_t)));
  w.req_flags = reinterpret_cast<int32_t*>(take(d.B * sizeof(int32_t)));
  w.desc = reinterpret_cast<RowDesc*>(take(d.n_t * sizeof(RowDesc)));
  w.part.mp = reinterpret_cast<float*>(take(np * 4));
  w.part.sp = reinterpret_cast<float*>(take(np * 4));
  w.part.stp = reinterpret_cast<float*>(take(np * 4));
  w.part.ap = reinterpret_cast<int32_t*>(take(np * 4));
  w.part.mq = reinterpret_cast<float*>(take(np * 4));
  w.part.sq = reinterpret_cast<float*>(take(np * 4));
  w.part.stq = reinterpret_cast<float*>(take(np * 4));
  w.part.w = reinterpret_cast<float*>(take(np * 4));
  w.part.g = reinterpret_cast<float*>(take(np * 4));
  w.t_off = reinterpret_cast<float*>(take(d.n_t * 4));
  w.t_lz = reinterpret_cast<float*>(take(d.n_t * 4));
  w.t_arg = reinterpret_cast<int32_t*>(take(d.n_t * 4));
  w.d_off = reinterpret_cast<float*>(take(d.n_d * 4));
  w.d_lz = reinterpret_cast<float*>(take(d.n_d * 4));
  w.acc = reinterpret_cast<int32_t*>(take(d.n_d * 4));
  w.chunk_r = reinterpret_cast<double*>(take(d.B * d.n_chunks * 8));
  w.chunk_p = reinterpret_cast<double*>(take(d.B * d.n_chunks * 8));
  if (ws) *ws = w;
  return off;
}

}  // namespace sv
