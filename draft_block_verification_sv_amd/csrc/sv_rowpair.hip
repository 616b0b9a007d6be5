// The streaming pass of the verification path on gfx950 (MI355X), fused with the
// per-row finalize.
//
// One 256-thread workgroup owns one target row t and, when t scores a draft
// (position i < k_b), the draft row d it pairs with.  Its four wavefronts take slices of
// 64 lanes x kElemsPerLane columns round-robin, each wave loading its next slice (16-byte
// bounds-checked buffer loads) while it reduces the current one, so every logit is read
// from HBM exactly once.  Each lane keeps, over its own columns, statistics against
// whole-number exp2 offsets k (log2 units) set from its first slice:
//   S   = sum 2^(l L2E - k)                  softmax sums at T = 1 (target and draft);
//   S_T = sum 2^(l beta - k_T)               rows with T_b not in {0, 1};
//   W   = sum 2^(l_q L2E - k_q) (l_q - l_p)  and D = max (l_q - l_p)   (row pairs);
//   the running maxima, and for greedy rows the first argmax of the target row.
// The workgroup then finishes the row from the lane records (256, or 64 folded ones for rows
// split into many parts, below), in fixed order:
//   log2 normalisers LZ = K + log2(sum_l S_l 2^(k_l - K)), fp64;
//   the clipped reverse-KL R = sum_y min(delta, q log(q/p)) at T = 1 (AdaFlash paper,
//     Section 3.1 equation; Appendix B.1 for the temperature): per lane, with c2 = LZp - LZq,
//       sum of t_y over its columns  = ln2 2^(k_q - LZq) (L2E W + c2 S_q)     exactly, and
//       every t_y <= ln2 2^(k_q - LZq) S_q max(0, L2E D + c2);
//     a lane whose bound stays below delta contributes its exact unclipped sum, the columns
//     of any other lane are re-read and summed entry by entry;
//   the acceptance test u < min(1, p_T(x)/q_T(x)) (paper, Section 2.1), or for T = 0
//     the argmax match (DFlash notes, Section 5.2, worked example #4);
//   the offsets the sampler needs to rebuild p_T and q_T of this row.
// Launches of few rows split each row over several workgroups (PHASE 1), which hand their
// lane records to the part of the row that arrives last; that part folds them and finishes the
// row.  Rows split into many parts fold each part's four waves lane by lane first, into 64 lane
// records (lane l: the columns of thread l of every wave, in every slice), and are finished
// from those 64 lanes.
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
#include "sv_lanes.h"
#include "sv_layout.h"
#include "sv_launch.h"

namespace sv {

// Work-item and workgroup ids straight from the hardware registers: this translation unit
// is built with IEEE mode off, and the runtime's accessor functions (built with it on) are
// then not inlined; the calls would cost the kernel registers.
__device__ __forceinline__ int thread_index() {
  return static_cast<int>(__builtin_amdgcn_workitem_id_x());
}
__device__ __forceinline__ int64_t block_index() {
  return static_cast<int64_t>(__builtin_amdgcn_workgroup_id_x());
}

constexpr uint32_t kNaNBits = 0x7fc00000u;
constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0): every load and store of the wave done
// The bounds-checked loads of the streaming loop stream (nontemporal) like the plain ones.
constexpr int kBufAux = 2;

__device__ __forceinline__ void store_nan(float* p) { *reinterpret_cast<uint32_t*>(p) = kNaNBits; }

// Uniform valid iff in [0, 1) (-0 allowed); decided on the bits.
__device__ __forceinline__ bool uniform_ok(float u) {
  const uint32_t b = __float_as_uint(u);
  return b < 0x3f800000u || b == 0x80000000u;
}
// Temperature valid iff +-0 (greedy) or finite and at least kMinTemperature = 2^-10.  The
// stream forms exponents as fma(l, log2(e) / T, -k) with whole-number fp32 offsets k, and the
// draw rebuilds p_T from the fp32 offset -round(LZ_T); both are exact only while
// |l| log2(e) / T stays below 2^24, i.e. |l| < 11360 at the minimum temperature.  Below it,
// greedy decoding (T = 0) is the limit the caller wants.
__device__ __forceinline__ bool temperature_ok(float T) {
  const uint32_t b = __float_as_uint(T);
  return (b & 0x7fffffffu) == 0u || (b >= 0x3a800000u && b < 0x7f800000u);
}

// One 16-byte streaming load (nontemporal: every byte is read once).
template <class T>
__device__ __forceinline__ T stream_load(const T* p) {
  static_assert(sizeof(T) == 16, "16-byte loads");
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
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
  // Running maxima across slices: raw words (high elements, masked at the end) into mh,
  // low elements into ml.
  // Written as chains of three-input maxima (one v_max3_f32 per two elements).
  __device__ __forceinline__ void fold_max(float& mh, float& ml) const {
#pragma unroll
    for (int i = 0; i < kElemsPerLane / 2; i += 2) {
      mh = fmaxf(fmaxf(mh, __uint_as_float(w[i])), __uint_as_float(w[i + 1]));
      ml = fmaxf(fmaxf(ml, bf16_lo(w[i])), bf16_lo(w[i + 1]));
    }
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
  // Bounds-checked form: byte offset off of the lane's first column inside the buffer r;
  // words past the buffer's end read as zero and touch no memory.
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int off) {
#pragma unroll
    for (int c = 0; c < kGroups; ++c) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off + c * 1024, 0, kBufAux);
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
  __device__ __forceinline__ void fold_max(float& mh, float& ml) const {
    (void)mh;
#pragma unroll
    for (int j = 0; j < kElemsPerLane; j += 2) ml = fmaxf(fmaxf(ml, x[j]), x[j + 1]);
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

// ----------------------------------------------------------------------------- lane statistics
// Each lane keeps running statistics over its own columns of the row (pair), against
// exp2 offsets that are whole numbers (log2 units): a change of offset then rescales the
// sums exactly, and no cross-lane work is needed until the row is done.
constexpr float kOverflow = 18446744073709551616.0f;  // 2^64

struct LaneAcc {
  float kp, kq, ktp, ktq;      // offsets: T = 1 for p and q; T_b (rows with T_b not in {0, 1})
  double sp, sq, stp, stq, w;  // sums of 2^(l L2E - k), of 2^(l beta - kt), of E_q (l_q - l_p)
  float dmax;                  // max of l_q - l_p
  float xmax;                  // max of E_q (l_q - l_p), E_q = 2^(l_q L2E - kq) as in w
  float mhp, mlp, mhq, mlq;    // running maxima of l_p and l_q (see fold_max)
  float amax;                  // greedy rows: the lane's largest target logit ...
  int aidx;                    // ... and its first column
};

// What a part of a split row hands to the finalize, per lane: the offsets and sums after the
// top correction, the largest l_q - l_p and E_q (l_q - l_p), and the greedy argmax (the running
// maxima have no use once the sums are corrected).
struct LaneRec {
  float kp, kq, ktp, ktq;
  double sp, sq, stp, stq, w;
  float dmax, amax;
  int aidx;
  float xmax;
};
static_assert(sizeof(LaneRec) <= kLaneRecBytes, "lane records must fit their workspace slots");

__device__ __forceinline__ LaneRec lane_record(const LaneAcc& A) {
  LaneRec R;
  R.kp = A.kp;
  R.kq = A.kq;
  R.ktp = A.ktp;
  R.ktq = A.ktq;
  R.sp = A.sp;
  R.sq = A.sq;
  R.stp = A.stp;
  R.stq = A.stq;
  R.w = A.w;
  R.dmax = A.dmax;
  R.amax = A.amax;
  R.aidx = A.aidx;
  R.xmax = A.xmax;
  return R;
}

// Records of split rows, one per thread of a part, or when the launch folds (a.folded) one per
// thread of wave 0, into which the part folds its four waves lane by lane (thread l of every
// wave reads the same column offsets of its slices, so folded lane l of a split row covers
// columns l 8 .. l 8 + 7 of each 512-column group of every slice).  Laid out word-major: word i
// of lane l of a part at words[i * lanes + l], so that each store and load of a wave covers
// 512 contiguous bytes.  The records are read back within the launch, so they are written and
// read as 64-bit words with device-scope atomics, which go to and come from the coherence
// point shared by every XCD instead of this XCD's L2.
// A record moves only the words its row uses: (kp, kq), S_p, then for row pairs S_q, W and
// (D, max E_q (l_q - l_p)); (amax, aidx) for greedy rows; (kt_p, kt_q), S_T,p and for pairs
// S_T,q for rows with T_b not in {0, 1}.  The fields it leaves out read back as a cleared lane
// holds them.  A part's slot keeps room for every word (kRecWords per lane).
static_assert(sizeof(LaneRec) <= kLaneRecBytes && kFoldLanes == 64, "one folded record per thread of a wave");
constexpr int kRecWords = static_cast<int>((sizeof(LaneRec) + 7) / 8);
constexpr int kFoldMaxParts = 16;  // parts a split row may have (row_split gives at most 16)
constexpr int kFoldRecs = 8;       // records one thread of the finalize folds, at most
static_assert(kFoldMaxParts / kRowWaves <= kFoldRecs && kFoldMinSplit - 1 <= kFoldRecs, "finalize folds");
template <bool PAIR, int MODE>
constexpr int rec_words() {
  return (PAIR ? 5 : 2) + (MODE == 1 ? 1 : 0) + (MODE == 2 ? (PAIR ? 3 : 2) : 0);
}
static_assert(rec_words<true, 2>() <= kRecWords, "a record fits its slot");
__device__ __forceinline__ uint64_t two_words(float lo, float hi) {
  return static_cast<uint64_t>(__float_as_uint(lo)) | (static_cast<uint64_t>(__float_as_uint(hi)) << 32);
}
__device__ __forceinline__ float lo_float(uint64_t w) { return __uint_as_float(static_cast<uint32_t>(w)); }
__device__ __forceinline__ float hi_float(uint64_t w) { return __uint_as_float(static_cast<uint32_t>(w >> 32)); }
__device__ __forceinline__ uint64_t dword(double d) { return static_cast<uint64_t>(__double_as_longlong(d)); }
__device__ __forceinline__ double dval(uint64_t w) { return __longlong_as_double(static_cast<long long>(w)); }
template <bool PAIR, int MODE>
__device__ __forceinline__ void pack_record(const LaneRec& r, uint64_t (&w)[rec_words<PAIR, MODE>()]) {
  int i = 0;
  w[i++] = two_words(r.kp, r.kq);
  w[i++] = dword(r.sp);
  if constexpr (PAIR) {
    w[i++] = dword(r.sq);
    w[i++] = dword(r.w);
    w[i++] = two_words(r.dmax, r.xmax);
  }
  if constexpr (MODE == 1) w[i++] = two_words(r.amax, __int_as_float(r.aidx));
  if constexpr (MODE == 2) {
    w[i++] = two_words(r.ktp, r.ktq);
    w[i++] = dword(r.stp);
    if constexpr (PAIR) w[i++] = dword(r.stq);
  }
}
template <bool PAIR, int MODE>
__device__ __forceinline__ LaneRec unpack_record(const uint64_t (&w)[rec_words<PAIR, MODE>()]) {
  LaneRec r;
  r.ktp = r.ktq = 0.0f;
  r.sq = r.w = r.stp = r.stq = 0.0;
  r.dmax = r.xmax = r.amax = -INFINITY;
  r.aidx = 0x7fffffff;
  int i = 0;
  r.kp = lo_float(w[i]);
  r.kq = hi_float(w[i++]);
  r.sp = dval(w[i++]);
  if constexpr (PAIR) {
    r.sq = dval(w[i++]);
    r.w = dval(w[i++]);
    r.dmax = lo_float(w[i]);
    r.xmax = hi_float(w[i++]);
  }
  if constexpr (MODE == 1) {
    r.amax = lo_float(w[i]);
    r.aidx = __float_as_int(hi_float(w[i++]));
  }
  if constexpr (MODE == 2) {
    r.ktp = lo_float(w[i]);
    r.ktq = hi_float(w[i++]);
    r.stp = dval(w[i++]);
    if constexpr (PAIR) r.stq = dval(w[i++]);
  }
  return r;
}
template <bool PAIR, int MODE>
__device__ __forceinline__ void store_record(uint64_t* part_words, int l, int lanes, const LaneRec& r) {
  uint64_t w[rec_words<PAIR, MODE>()];
  pack_record<PAIR, MODE>(r, w);
#pragma unroll
  for (int i = 0; i < rec_words<PAIR, MODE>(); ++i)
    __hip_atomic_store(part_words + i * lanes + l, w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <bool PAIR, int MODE>
__device__ __forceinline__ LaneRec load_record(const uint64_t* part_words, int l, int lanes) {
  uint64_t w[rec_words<PAIR, MODE>()];
#pragma unroll
  for (int i = 0; i < rec_words<PAIR, MODE>(); ++i)
    w[i] = __hip_atomic_load(const_cast<uint64_t*>(part_words + i * lanes + l), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  return unpack_record<PAIR, MODE>(w);
}
// Part p's records of row (pair) unit.
__device__ __forceinline__ uint64_t* part_records(const RowPairArgs& a, int64_t unit, int p) {
  return static_cast<uint64_t*>(a.rec) + (unit * a.split + p) * kRecWords * rec_lanes(a.folded);
}

// The finalize of a split row, the records folded in part order with all loads issued at once.
// Unfolded records: thread t folds its lane's records of every part.  Folded: thread (q, l)
// folds lane l of a quarter of the parts (parts q per .. q per + per - 1, per = ceil(split /
// 4)), then wave 0 folds the quarters in order and lacc holds the row's 64 lanes, the other 192
// empty.
struct PartFold {
  LaneRec R[kFoldRecs];
  __device__ __forceinline__ void range(const RowPairArgs& a, int tid, int& p0, int& per) const {
    per = a.folded ? (a.split + kRowWaves - 1) / kRowWaves : a.split;
    p0 = a.folded ? (tid >> 6) * per : 0;
  }
  template <bool PAIR, int MODE>
  __device__ __forceinline__ void load(const RowPairArgs& a, int64_t unit, int tid) {
    int p0, per;
    range(a, tid, p0, per);
    const int lanes = rec_lanes(a.folded), l = a.folded ? (tid & 63) : tid;
#pragma unroll
    for (int u = 0; u < kFoldRecs; ++u)
      if (u < per && p0 + u < a.split)
        R[u] = load_record<PAIR, MODE>(part_records(a, unit, p0 + u), l, lanes);
  }
  __device__ __forceinline__ void fold(const RowPairArgs& a, int tid, LaneAcc* lacc) const;
};

// Arrival flags of a row's parts: part p of a row sets word p of the row's kFoldMaxParts flag
// words to the launch's epoch once its records are complete at the coherence point, waits for
// that store to complete there, then reads every part's flag.  Of two parts, the one that sets
// its flag later sees the other's, so the part that arrives last sees every flag set (others
// may too, and then finish the row as well, with the same results).  A flag word holding
// anything but the epoch (the row's flags of an earlier launch, which had its own epoch, or
// whatever the memory held) counts as not arrived.  A part that finds every flag set clears
// them: all parts have set theirs by then, so they stay cleared, and a replay of a captured
// launch, which carries the same epoch, starts from cleared flags.

__device__ __forceinline__ void lane_clear(LaneAcc& A) {
  A.kp = A.kq = A.ktp = A.ktq = 0.0f;
  A.sp = A.sq = A.stp = A.stq = A.w = 0.0;
  A.dmax = A.xmax = -INFINITY;
  A.mhp = A.mlp = A.mhq = A.mlq = -INFINITY;
  A.amax = -INFINITY;
  A.aidx = 0x7fffffff;
}

// Whole-number offset for a lane whose largest value is m at scale `scale`: every
// exponent of that lane's slice is then <= 0.  A lane holding padding only keeps 0.
__device__ __forceinline__ float offset_for(float m, float scale) {
  const float k = ceilf(m * scale);
  return k > -INFINITY ? k : 0.0f;
}

template <bool PAIR, int MODE, class Row>
__device__ __forceinline__ void lane_init(const Row& rp, const Row& rq, float beta, LaneAcc& A) {
  const float mp = rp.max();
  A.kp = offset_for(mp, kL2E);
  if constexpr (MODE == 2) A.ktp = offset_for(mp, beta);
  if constexpr (PAIR) {
    const float mq = rq.max();
    A.kq = offset_for(mq, kL2E);
    if constexpr (MODE == 2) A.ktq = offset_for(mq, beta);
  }
}

// The row values as fresh registers: keeps the compiler from hoisting the rare offset
// raise (and the maxima it needs) out of its branch.
template <class Row>
__device__ __forceinline__ Row opaque(const Row& r) {
  Row o = r;
  uint32_t* w = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
  for (int i = 0; i < static_cast<int>(sizeof(Row) / 4); ++i) asm volatile("" : "+v"(w[i]));
  return o;
}

// Raises the offsets to cover the slice's maxima; sums scale by exact powers of two.
__device__ __forceinline__ void raise_offset(float& k, double& s, float m, float scale) {
  const float kn = fmaxf(k, offset_for(m, scale));
  s = ldexp(s, static_cast<int>(k - kn));
  k = kn;
}

template <bool PAIR, int MODE, class Row>
__device__ __forceinline__ void lane_rebase(const Row& rp_in, const Row& rq_in, float beta,
                                            LaneAcc& A) {
  const Row rp = opaque(rp_in);
  const float mp = rp.max();
  raise_offset(A.kp, A.sp, mp, kL2E);
  if constexpr (MODE == 2) raise_offset(A.ktp, A.stp, mp, beta);
  if constexpr (PAIR) {
    const Row rq = opaque(rq_in);
    const float mq = rq.max();
    const float kn = fmaxf(A.kq, offset_for(mq, kL2E));
    const int sh = static_cast<int>(A.kq - kn);
    A.sq = ldexp(A.sq, sh);
    A.w = ldexp(A.w, sh);
    A.xmax = ldexpf(A.xmax, sh);
    A.kq = kn;
    if constexpr (MODE == 2) raise_offset(A.ktq, A.stq, mq, beta);
  }
}

// One slice's partial sums against the lane's current offsets.
struct SlicePart {
  float sp, sq, stp, stq, w, dm, xm;
  bool ok;  // every partial sum below 2^64
};

template <bool PAIR, int MODE, bool MASK, class Row>
__device__ __forceinline__ SlicePart slice_partials(const Row& rp, const Row& rq, float beta,
                                                    int64_t col_lane, int V, const LaneAcc& A) {
  const float op = -A.kp, oq = -A.kq, otp = -A.ktp, otq = -A.ktq;
  // Two chains per sum, each started from its first term (no add of zero); the maxima of
  // l_q - l_p and of E_q (l_q - l_p) as chains of three-input maxima.
  float sp0, sp1, sq0, sq1, w0, w1, stp0, stp1, stq0, stq1, dm0, dm1, xm0, xm1;
  auto acc = [](float& s, float v, bool first) { s = first ? v : s + v; };
#pragma unroll
  for (int e = 0; e < kElemsPerLane; e += 2) {
    const bool first = (e == 0);
    float t[2], x[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float xp = rp.at(e + h);
      const float ep = fast_exp2(__builtin_fmaf(xp, kL2E, op));
      acc(h ? sp1 : sp0, ep, first);
      if constexpr (MODE == 2) {
        const float etp = fast_exp2(__builtin_fmaf(xp, beta, otp));
        acc(h ? stp1 : stp0, etp, first);
      }
      if constexpr (PAIR) {
        const float xq = rq.at(e + h);
        const float eq = fast_exp2(__builtin_fmaf(xq, kL2E, oq));
        float diff = xq - xp;
        if constexpr (MASK) {
          const int ee = e + h;
          if (col_lane + (ee >> 3) * 512 + (ee & 7) >= V) diff = 0.0f;
        }
        float& sq = h ? sq1 : sq0;
        float& w = h ? w1 : w0;
        acc(sq, eq, first);
        w = first ? eq * diff : __builtin_fmaf(eq, diff, w);
        t[h] = diff;
        x[h] = eq * diff;
        if constexpr (MODE == 2) {
          const float etq = fast_exp2(__builtin_fmaf(xq, beta, otq));
          acc(h ? stq1 : stq0, etq, first);
        }
      }
    }
    if constexpr (PAIR) {
      float& dm = (e & 2) ? dm1 : dm0;
      dm = (e < 4) ? fmaxf(t[0], t[1]) : fmaxf(fmaxf(dm, t[0]), t[1]);
      float& xm = (e & 2) ? xm1 : xm0;
      xm = (e < 4) ? fmaxf(x[0], x[1]) : fmaxf(fmaxf(xm, x[0]), x[1]);
    }
  }
  SlicePart P;
  P.sp = sp0 + sp1;
  P.ok = P.sp < kOverflow;
  P.stp = P.sq = P.stq = P.w = 0.f;
  P.dm = P.xm = -INFINITY;
  if constexpr (MODE == 2) {
    P.stp = stp0 + stp1;
    P.ok = P.ok && P.stp < kOverflow;
  }
  if constexpr (PAIR) {
    P.sq = sq0 + sq1;
    P.w = w0 + w1;
    P.dm = fmaxf(dm0, dm1);
    P.xm = fmaxf(xm0, xm1);
    P.ok = P.ok && P.sq < kOverflow;
    if constexpr (MODE == 2) {
      P.stq = stq0 + stq1;
      P.ok = P.ok && P.stq < kOverflow;
    }
  }
  return P;
}

// Adds one slice of the lane's columns to its statistics.  col_lane: column of the lane's
// first element.  MASK: columns >= V are padding (-inf) whose difference term is zeroed.
// A slice whose partial sum reaches 2^64 (values far above the lane's offset) raises the
// offsets and is summed again; the partial sums are otherwise added in fp64.
template <bool PAIR, int MODE, bool MASK, class Row>
__device__ __forceinline__ void slice_accumulate(const Row& rp, const Row& rq, float beta,
                                                 int64_t col_lane, int V, LaneAcc& A) {
  if constexpr (MODE == 1) {
    const float m = rp.max();
    if (m > A.amax) {
      int best = 0;
#pragma unroll
      for (int e = kElemsPerLane - 1; e >= 0; --e)
        if (rp.at(e) == m) best = e;
      A.amax = m;
      A.aidx = static_cast<int>(col_lane + (best >> 3) * 512 + (best & 7));
    }
  }
  rp.fold_max(A.mhp, A.mlp);
  if constexpr (PAIR) rq.fold_max(A.mhq, A.mlq);
  SlicePart P = slice_partials<PAIR, MODE, MASK>(rp, rq, beta, col_lane, V, A);
  if (!P.ok) {  // rare: raise the offsets, sum the slice again from fresh registers
    lane_rebase<PAIR, MODE>(rp, rq, beta, A);
    P = slice_partials<PAIR, MODE, MASK>(opaque(rp), opaque(rq), beta, col_lane, V, A);
  }
  A.sp += static_cast<double>(P.sp);
  if constexpr (MODE == 2) A.stp += static_cast<double>(P.stp);
  if constexpr (PAIR) {
    A.sq += static_cast<double>(P.sq);
    A.w += static_cast<double>(P.w);
    A.dmax = fmaxf(A.dmax, P.dm);
    A.xmax = fmaxf(A.xmax, P.xm);
    if constexpr (MODE == 2) A.stq += static_cast<double>(P.stq);
  }
}

// Streams the wave's slices s = first, first + step, ... of the row (pair) into the lane's
// statistics (first = the wave and step = 4 when one workgroup takes the whole row).  Full
// bf16 slices of 16-byte-aligned rows: packed, next slice prefetched while the current one is
// reduced.  The ragged last slice and every other case: fp32, masked.  The lane's first slice
// sets its offsets from that slice's maxima.
template <int DT, bool VEC, bool PAIR, int MODE>
__device__ __forceinline__ void stream_row(const void* prow, const void* qrow, float beta, int V,
                                           int n_slices, int first, int step, int lane, LaneAcc& A) {
  const int n_full = V / kSlice;
  int s = first;
  bool fresh = true;
  if constexpr (DT == 0 && VEC) {
    // The row's full slices as bounds-checked buffers: the prefetch of a slice past the
    // last one reads zeros without touching memory, so every prefetch is issued without a
    // branch and the wait before a slice's arithmetic covers that slice's loads alone (a
    // load issued under a branch makes the wait at the join count it as well).
    const int full_bytes = n_full * kSlice * 2;
    const __amdgpu_buffer_rsrc_t RP =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(prow), 0, full_bytes, kBufWord3);
    const __amdgpu_buffer_rsrc_t RQ =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(qrow), 0, PAIR ? full_bytes : 0, kBufWord3);
    const int lane_off = lane * 16;
    PackedRow ap, aq, bp, bq;
    auto load_pair = [&](PackedRow& rp, PackedRow& rq, int sl) {
      rp.load(RP, lane_off + sl * (kSlice * 2));
      if constexpr (PAIR) rq.load(RQ, lane_off + sl * (kSlice * 2));
    };
    if (s < n_full) {
      load_pair(ap, aq, s);
      lane_init<PAIR, MODE>(ap, aq, beta, A);
      fresh = false;
      while (true) {
        load_pair(bp, bq, s + step);
        slice_accumulate<PAIR, MODE, false>(ap, aq, beta,
                                            static_cast<int64_t>(s) * kSlice + lane * 8, V, A);
        if (s + step >= n_full) {
          s += step;
          break;
        }
        load_pair(ap, aq, s + 2 * step);
        slice_accumulate<PAIR, MODE, false>(bp, bq, beta,
                                            static_cast<int64_t>(s + step) * kSlice + lane * 8,
                                            V, A);
        s += 2 * step;
        if (s >= n_full) break;
      }
    }
  }
  for (; s < n_slices; s += step) {  // every slice not handled above
    const int64_t col_lane = static_cast<int64_t>(s) * kSlice + lane * 8;
    FloatRow fp, fq;
    fp.template load<DT, VEC>(prow, col_lane, V);
    if constexpr (PAIR) fq.template load<DT, VEC>(qrow, col_lane, V);
    if (fresh) {
      lane_init<PAIR, MODE>(fp, fq, beta, A);
      fresh = false;
    }
    slice_accumulate<PAIR, MODE, true>(fp, fq, beta, col_lane, V, A);
  }
}

// Folds the record R of the same lane position over another part of the row into A.  Sums
// against whole-number offsets combine exactly up to rounding: both are rescaled to the larger
// offset of the two that carry mass (a record without mass keeps no offset).  Applied to a
// lane's parts in part order, so the result does not depend on which part finished first.
__device__ __forceinline__ void fold_sum(float& kA, double& sA, float kR, double sR) {
  if (!(sR > 0.0)) return;
  if (sA > 0.0) {
    const float K = fmaxf(kA, kR);
    sA = ldexp(sA, static_cast<int>(kA - K)) + ldexp(sR, static_cast<int>(kR - K));
    kA = K;
  } else {
    kA = kR;
    sA = sR;
  }
}

__device__ __forceinline__ void lane_merge(LaneAcc& A, const LaneRec& R) {
  fold_sum(A.kp, A.sp, R.kp, R.sp);
  fold_sum(A.ktp, A.stp, R.ktp, R.stp);
  fold_sum(A.ktq, A.stq, R.ktq, R.stq);
  if (R.sq > 0.0) {  // W shares the offset of S_q
    if (A.sq > 0.0) {
      const float K = fmaxf(A.kq, R.kq);
      const int ha = static_cast<int>(A.kq - K), hr = static_cast<int>(R.kq - K);
      A.sq = ldexp(A.sq, ha) + ldexp(R.sq, hr);
      A.w = ldexp(A.w, ha) + ldexp(R.w, hr);
      A.xmax = fmaxf(ldexpf(A.xmax, ha), ldexpf(R.xmax, hr));
      A.kq = K;
    } else {
      A.kq = R.kq;
      A.sq = R.sq;
      A.w = R.w;
      A.xmax = R.xmax;
    }
  }
  A.dmax = fmaxf(A.dmax, R.dmax);
  if (R.amax > A.amax || (R.amax == A.amax && R.aidx < A.aidx)) {
    A.amax = R.amax;
    A.aidx = R.aidx;
  }
}

__device__ __forceinline__ void PartFold::fold(const RowPairArgs& a, int tid, LaneAcc* lacc) const {
  int p0, per;
  range(a, tid, p0, per);
  LaneAcc F;
  lane_clear(F);
#pragma unroll
  for (int u = 0; u < kFoldRecs; ++u)
    if (u < per && p0 + u < a.split) lane_merge(F, R[u]);
  lacc[tid] = F;
  if (!a.folded) return;
  __syncthreads();
  if (tid < kFoldLanes) {
#pragma unroll
    for (int q = 1; q < kRowWaves; ++q) lane_merge(F, lane_record(lacc[q * kFoldLanes + tid]));
    lacc[tid] = F;
  }
  __syncthreads();  // wave 0 has read every quarter
  if (tid >= kFoldLanes) lane_clear(lacc[tid]);
}

// ----------------------------------------------------------------------------- block helpers
// Fixed-order reductions over the 256-thread workgroup: wave butterfly, then the four
// wave results in order.  `red` holds kRowWaves doubles.
__device__ __forceinline__ double block_sum_d(double v, double* red) {
  const int lane = thread_index() & 63, wave = thread_index() >> 6;
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
  const int lane = thread_index() & 63, wave = thread_index() >> 6;
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
  const int lane = thread_index() & 63, wave = thread_index() >> 6;
  v = wave_min_int(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int r = red[0];
#pragma unroll
  for (int w = 1; w < kRowWaves; ++w) r = min(r, red[w]);
  __syncthreads();
  return r;
}

// The lane's largest logit from its running maxima.
__device__ __forceinline__ float lane_max(float mh, float ml) {
  return fmaxf(bf16_hi(__float_as_uint(mh)), ml);
}

// The lane's largest element entered its sum as the fp32 exponential of a rounded
// exponent (up to one unit in the last place off).  In rows dominated by one token that
// error moves the normaliser, and through it the reverse-KL, by more than the rest of the
// row's rounding; the lane sum is corrected to carry that element's exact value.  The
// same fma and exp2 as the stream reproduce the value that was added.
__device__ __forceinline__ void correct_top(double& S, float M, float scale, float k) {
  if (S > 0.0 && M > -INFINITY) {
    const float added = fast_exp2(__builtin_fmaf(M, scale, -k));
    const double exact = exp2_d(static_cast<double>(M) * static_cast<double>(scale) -
                              static_cast<double>(k));
    S += exact - static_cast<double>(added);
  }
}

// Fixed-order reductions of N values per thread over the workgroup with one pair of barriers:
// value j is summed, or with bit j of MAX set, maximised.  red: N * kRowWaves doubles.
template <int N, unsigned MAX>
__device__ __forceinline__ void block_reduce(double (&v)[N], double* red) {
  const int lane = thread_index() & 63, wave = thread_index() >> 6;
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = ((MAX >> j) & 1u) ? wave_max_d(v[j]) : wave_sum_d(v[j]);
  if (lane == 0)
#pragma unroll
    for (int j = 0; j < N; ++j) red[j * kRowWaves + wave] = v[j];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < N; ++j) {
    double r = red[j * kRowWaves];
#pragma unroll
    for (int w = 1; w < kRowWaves; ++w)
      r = ((MAX >> j) & 1u) ? fmax(r, red[j * kRowWaves + w]) : r + red[j * kRowWaves + w];
    v[j] = r;
  }
  __syncthreads();
}

// The log2 normalisers of N (offset, sum) pairs of every lane at once:
// LZ_j = K_j + log2(sum_l S_jl 2^(k_jl - K_j)), K_j the largest offset of a lane with mass (the
// scaling by 2^(k_jl - K_j) is exact).
// With ARG, also the row's first argmax from every lane's (largest value, its column): the
// largest value in the first round, the lowest column holding it in the second.
template <int N, bool ARG>
__device__ __forceinline__ void lanes_lz_n(const float (&k)[N], const double (&S)[N], double (&LZ)[N],
                                           float (&K)[N], float amax, int aidx, int* argmax,
                                           double* red) {
  constexpr int NA = N + (ARG ? 1 : 0);
  double m[NA];
#pragma unroll
  for (int j = 0; j < N; ++j) m[j] = S[j] > 0.0 ? static_cast<double>(k[j]) : -INFINITY;
  if constexpr (ARG) m[N] = static_cast<double>(amax);
  block_reduce<NA, (1u << NA) - 1u>(m, red);
  double v[NA];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    K[j] = static_cast<float>(m[j]);
    v[j] = S[j] > 0.0 ? ldexp(S[j], static_cast<int>(k[j] - K[j])) : 0.0;
  }
  // lowest column among the maxima, as the largest of -column
  if constexpr (ARG) v[N] = (static_cast<double>(amax) == m[N]) ? -static_cast<double>(aidx) : -2147483647.0;
  block_reduce<NA, ARG ? (1u << N) : 0u>(v, red);
#pragma unroll
  for (int j = 0; j < N; ++j) LZ[j] = static_cast<double>(K[j]) + log2_d(v[j]);
  if constexpr (ARG) *argmax = static_cast<int>(-v[N]);
}


template <int DT>
__device__ __forceinline__ float logit_at(const void* row, int64_t col) {
  if constexpr (DT == 0) return bf16_at(static_cast<const uint16_t*>(row) + col);
  else return static_cast<const float*>(row)[col];
}

// A value the whole workgroup shares, moved to scalar registers (a buffer resource needs one).
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Lists the lanes whose flag is set (order of arrival; users combine per lane, so the order
// does not matter) and returns how many there are.
__device__ __forceinline__ int list_lanes(bool flag, int* list, int* s_n) {
  if (thread_index() == 0) *s_n = 0;
  __syncthreads();
  if (flag) list[atomicAdd(s_n, 1)] = thread_index();
  __syncthreads();
  return *s_n;
}

// The workgroup's LDS: the lane records, per-lane re-read results, the list of re-read
// lanes and the block reductions' slots.
struct Scratch {
  LaneAcc* lacc;
  double* direct;
  double* direct_x;
  double* direct_u0;
  int* failed;
  int* s_nfail;
  int* s_nheavy;  // a counter of its own: the heavy list is read while the next one starts
  int* s_last;    // split rows: this part found every part of the row arrived
  double* red_d;
  float* red_f;
  int* red_i;
  double* red_v;  // kRowWaves * kRowSums
};
constexpr int kRowSums = 6;  // values of the widest block reduction (lanes_lz_n: 5)

// Clipped reverse-KL of the row pair.  With Q = 2^(k_q - LZq) S_q, the q-mass of a lane's
// columns, and c2 = LZp - LZq, those columns contribute exactly
//   sum t_y = ln2 2^(k_q - LZq) (L2E W + c2 S_q),
// and since t_y = ln2 q_y (L2E (l_q - l_p)_y + c2), none of them exceeds
// ln2 Q max(0, L2E D + c2), D the lane's largest l_q - l_p, nor
// ln2 2^(k_q - LZq) (L2E max(0, X) + max(0, c2) S_q), X the lane's largest E_q (l_q - l_p).
// A lane whose smaller bound may reach delta (fail) has its columns re-read and summed entry
// by entry; the others take the closed form.
struct LaneClosed {
  double closed, mass;  // ln2-scaled closed form, q-mass
  bool fail;
};
__device__ __forceinline__ LaneClosed lane_closed(const LaneAcc& A, double LZp, double LZq,
                                                  float delta) {
  LaneClosed out{0.0, 0.0, false};
  if (!(A.sq > 0.0)) return out;
  const double c2 = LZp - LZq;
  const double scale = kLn2 * exp2_d(static_cast<double>(A.kq) - LZq);
  out.closed = scale * (static_cast<double>(kL2E) * A.w + c2 * A.sq);
  out.mass = scale * A.sq / kLn2;
  // Two bounds on the lane's largest term t_y = scale E_y (L2E d_y + c2), d_y = l_q - l_p,
  // both from max over y of a sum <= the sum of the maxima: its q-mass times the largest
  // slope, and L2E max_y E_y d_y + max(c2, 0) S_q (every E_y >= 0, so no E_y exceeds S_q;
  // the lane's offset need not cover its later slices).  The lane's sum is closed-form when
  // the smaller one stays below delta.
  const double slope = static_cast<double>(kL2E) * A.dmax + c2;
  const double by_mass = scale * A.sq * (slope > 0.0 ? slope : 0.0);
  const double by_peak = scale * (static_cast<double>(kL2E) * fmax(static_cast<double>(A.xmax), 0.0) +
                                  (c2 > 0.0 ? c2 : 0.0) * A.sq);
  const double bound = fmin(by_mass, by_peak);
  out.fail = !(bound * 1.0001 < static_cast<double>(delta));
  return out;
}

// A lower bound on the row's sum_y |min(delta, t_y)| from one lane: |sum t_y| for a closed-form
// lane, and for a lane near the clip the sum of its negative terms, at least -sum t_y.
__device__ __forceinline__ double lane_l1_lower(const LaneClosed& L) {
  return L.fail ? fmax(0.0, -L.closed) : fabs(L.closed);
}

// Exact sums of the lanes that carry the row's mass.  The stream's lane sums come from fp32
// exponentials (one unit in the last place each) and fp32 partial sums of 16 elements, a
// relative error of up to ~2.4e-7 of the lane's mass.  Through the normalisers that moves the
// clipped reverse-KL by up to ~2.4e-7 (P + Q) (P, Q the lane's shares of the two rows), and
// through its closed form, where L2E W and c2 S_q may be two large terms that cancel to a small
// one, by up to ~2.4e-7 ln2 mag, mag = 2^(k_q - LZq) (L2E |W| + |c2| S_q).  Against the
// accuracy the path is built to, 1e-5 max(|R|, L1) with L1 = sum_y |min(delta, t_y)|, a lane is
// heavy when its share of that error exceeds an eighth of 1e-5 times a lower bound on L1 (the
// sum of lane_l1_lower over the row), or when it holds more than half of either row's mass, or
// more than 1/32 of it with a closed form that cancels by a factor above 64.  A lane whose two
// rows are equal bit for bit (W = 0, same sums and offsets) rounds the same way in both, and
// moves R only through c2: its share is 2 * 2.4e-7 ln2 mag.  Heavy lanes are summed again from
// the logits in fp64 (exponentials exact to ~1e-15), against the same offsets, and their S_p,
// S_q and W replaced.  In verification the draw launch does this for rows with at most
// kFixLanes heavy lanes (RklFix); otherwise the finalize does it here.
constexpr double kLaneSumErr = 2.4e-7;
struct HeavyParts {
  bool by_mass;  // the mass and cancellation rules
  double err;    // the lane's share of the error, against 1e-5 L1 / 8
};
__device__ __forceinline__ HeavyParts heavy_parts(const LaneAcc& A, double LZp, double LZq) {
  const double P = A.sp > 0.0 ? exp2_d(static_cast<double>(A.kp) - LZp) * A.sp : 0.0;
  double Q = 0.0, closed = 0.0, mag = 0.0;
  if (A.sq > 0.0) {
    const double s = exp2_d(static_cast<double>(A.kq) - LZq);
    const double c2 = LZp - LZq;
    Q = s * A.sq;
    closed = s * (static_cast<double>(kL2E) * A.w + c2 * A.sq);
    mag = s * (static_cast<double>(kL2E) * fabs(A.w) + fabs(c2) * A.sq);
  }
  const double big = fmax(P, Q);
  const bool same = A.w == 0.0 && A.sp == A.sq && A.kp == A.kq;
  HeavyParts h;
  h.by_mass = big > 0.5 || (big > 1.0 / 32.0 && mag > 64.0 * fabs(closed));
  h.err = kLaneSumErr * (same ? 2.0 * kLn2 * mag : P + Q + kLn2 * mag);  // 0 without mass
  return h;
}
__device__ __forceinline__ double heavy_threshold(double L1lo) { return 1e-5 * L1lo * 0.125; }
__device__ __forceinline__ bool is_heavy(const HeavyParts& h, double thr) {
  return h.by_mass || h.err > thr;
}

// The n listed heavy lanes (sc.failed) summed again; their records in lacc are replaced.  Lane
// t's columns are those of lane t + col_base as the re-reading helpers number lanes (col_base =
// kRowThreads on split rows, whose lanes are the parts' folded ones).  A streaming lane is read
// by one wave, the lanes spread over the waves; a folded lane by every wave, one block each,
// whose sums meet in the direct arrays (block q of lane t at q kFoldLanes + t) and add up in
// block order.
template <int DT, bool VEC>
__device__ __forceinline__ void exact_heavy_sums(const void* prow, const void* qrow, int V,
                                                 int n_slices, LaneAcc* lacc, const Scratch& sc,
                                                 int n, int col_base) {
  const int tid = thread_index(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = lane_blocks(col_base);
  for (int it = wave; it < n * nb; it += kRowWaves) {
    const int f = it / nb, q = it - f * nb;
    const int src = sc.failed[f];
    const LaneSums e = exact_lane_sums<DT, VEC>(prow, qrow, V, n_slices, src + col_base, q, lane,
                                                static_cast<double>(lacc[src].kp),
                                                static_cast<double>(lacc[src].kq));
    if (lane == 0) {
      if (nb == 1) {
        lacc[src].sp = e.sp;
        lacc[src].sq = e.sq;
        lacc[src].w = e.w;
      } else {
        sc.direct[q * kFoldLanes + src] = e.sp;
        sc.direct_x[q * kFoldLanes + src] = e.sq;
        sc.direct_u0[q * kFoldLanes + src] = e.w;
      }
    }
  }
  __syncthreads();
  if (nb > 1) {
    for (int f = tid; f < n; f += kRowThreads) {
      const int src = sc.failed[f];
      double sp = 0.0, sq = 0.0, w = 0.0;
      for (int q = 0; q < nb; ++q) {
        sp += sc.direct[q * kFoldLanes + src];
        sq += sc.direct_x[q * kFoldLanes + src];
        w += sc.direct_u0[q * kFoldLanes + src];
      }
      lacc[src].sp = sp;
      lacc[src].sq = sq;
      lacc[src].w = w;
    }
    __syncthreads();
  }
}

// The row's clipped reverse-KL, lane by lane (lane_closed): closed form, or for a lane near the
// clip its columns re-read and summed entry by entry, q_y from an fp32 exponential, the log
// ratio L2E (l_q - l_p) + c2 and the sums in fp64.
// Per thread: its lane's closed form and q-mass, and whether it was re-read; the re-read lanes'
// sums are in LDS on return: direct = sum_y min(t_y, delta).  With SG, also
// direct_x = sum_y 1[t_y < delta] (t_y + q_y) = sum_y q_y g_y, the row statistic of the OPD
// gradient (g_y = 1[t_y < delta] (ln q_y - ln p_y + 1)), whose closed form on a passing lane is
// the lane's closed form plus Q.  With FIX instead, direct_x = sum over the unclipped terms and
// direct_u0 = their q-mass, from which the draw launch moves the lane's sum to new normalisers.
// Lane t's columns: as for exact_heavy_sums.
template <int DT, bool VEC, bool SG, bool FIX>
__device__ __forceinline__ LaneClosed lanes_clipped_rkl(const void* prow, const void* qrow, int V,
                                                       int n_slices, double LZp, double LZq,
                                                       float delta, const LaneAcc& A,
                                                       const Scratch& sc, int col_base) {
  static_assert(!(SG && FIX), "one use of the extra per-lane sums at a time");
  const int tid = thread_index(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const double c2 = LZp - LZq;
  const LaneClosed out = lane_closed(A, LZp, LZq, delta);
  const int nfail = list_lanes(out.fail, sc.failed, sc.s_nfail);
  if (nfail > 0) {
    const double dd = static_cast<double>(delta);
    const int nb = lane_blocks(col_base);  // blocks meet as in exact_heavy_sums
    for (int it = wave; it < nfail * nb; it += kRowWaves) {
      const int f = it / nb, q = it - f * nb;
      const int src = sc.failed[f], slot = q * kFoldLanes + src;
      double part = 0.0, xpart = 0.0, u0 = 0.0;
      for_lane_columns<DT, VEC>(prow, qrow, V, n_slices, src + col_base, q, lane, [&](float lp, float lq) {
        const double a = static_cast<double>(lq) * static_cast<double>(kL2E);
        const double q = static_cast<double>(fast_exp2(static_cast<float>(a - LZq)));
        const double term =
            q * kLn2 * ((static_cast<double>(lq) - static_cast<double>(lp)) * static_cast<double>(kL2E) + c2);
        part += fmin(term, dd);
        if constexpr (SG) xpart += term < dd ? term + q : 0.0;
        if constexpr (FIX) {
          xpart += term < dd ? term : 0.0;
          u0 += term < dd ? q : 0.0;
        }
      });
      part = wave_sum_d(part);
      if (lane == 0) sc.direct[slot] = part;
      if constexpr (SG || FIX) {
        xpart = wave_sum_d(xpart);
        if (lane == 0) sc.direct_x[slot] = xpart;
      }
      if constexpr (FIX) {
        u0 = wave_sum_d(u0);
        if (lane == 0) sc.direct_u0[slot] = u0;
      }
    }
    __syncthreads();
    if (nb > 1) {
      for (int f = tid; f < nfail; f += kRowThreads) {
        const int src = sc.failed[f];
        double part = 0.0, xpart = 0.0, u0 = 0.0;
        for (int q = 0; q < nb; ++q) {
          part += sc.direct[q * kFoldLanes + src];
          if constexpr (SG || FIX) xpart += sc.direct_x[q * kFoldLanes + src];
          if constexpr (FIX) u0 += sc.direct_u0[q * kFoldLanes + src];
        }
        sc.direct[src] = part;
        if constexpr (SG || FIX) sc.direct_x[src] = xpart;
        if constexpr (FIX) sc.direct_u0[src] = u0;
      }
      __syncthreads();
    }
  }
  return out;
}

// Offsets the sampler uses to rebuild a row's p_T: p_T(y) = 2^(fma(l_y, beta, off) - lz)
// with off = -round(LZ), so the exponent stays small wherever p_T is not negligible.
__device__ __forceinline__ void draw_offsets(double LZ, float* off, float* lz) {
  const double K = rint(LZ);
  *off = static_cast<float>(-K);
  *lz = static_cast<float>(LZ - K);
}

// ----------------------------------------------------------------------------- kernel
struct RowCtx {
  int64_t unit;  // the row (pair) this workgroup works on
  int part;      // which part of it, when rows are split over several workgroups
  int64_t t, d;  // target row, draft row (-1: bonus row)
  int64_t b;     // request (-1: clipped reverse-KL only)
  int pos;       // position of the target row in its request (verification)
  int mode;      // 0: T = 1, 1: greedy, 2: other T
  float beta;
  int row_flags;
};

template <int DT, bool VEC, int PHASE, bool PAIR, int MODE>
__device__ __forceinline__ void rowpair_body(const RowPairArgs& a, const RowCtx& ctx,
                                             const Scratch& sc, int xr) {
  LaneAcc* lacc = sc.lacc;
  double* red_d = sc.red_d;
  float* red_f = sc.red_f;
  const int tid = thread_index(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int V = a.V;
  const int n_slices = static_cast<int>(a.n_slices);
  const void* prow = static_cast<const char*>(a.target) + ctx.t * a.ld_t * (DT == 0 ? 2 : 4);
  const void* qrow = static_cast<const char*>(a.draft) + (PAIR ? ctx.d : 0) * a.ld_d * (DT == 0 ? 2 : 4);

  // The uniform and the two logits at the draft token, for thread 0's acceptance test at the
  // end, are loaded before the row is streamed: issued at the finalize they waited behind the
  // streaming traffic of the other workgroups, at the end of every row.  Every thread issues the
  // same three buffer loads, at offsets kept in bounds and with no branch around them (a load
  // under a branch is waited for where the branch closes), so nothing waits for them before
  // their use.  Buffers of zero length (no uniforms, an invalid token, a bonus row) read as 0
  // and touch no memory.
  const bool x_ok = PAIR && xr >= 0 && xr < V;
  uint32_t u_bits = 0, lp_bits = 0, lq_bits = 0;
  {
    // a zero the compiler cannot see through: with it the loaded values are per-lane to the
    // compiler, which then leaves them in vector registers instead of waiting for them at once
    // to move them to scalar ones
    int vzero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
    constexpr int es = DT == 0 ? 2 : 4;
    const __amdgpu_buffer_rsrc_t RU = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.uniforms), 0, a.uniforms ? static_cast<int>(a.n_units * 4) : 0, kBufWord3);
    u_bits = __builtin_amdgcn_raw_buffer_load_b32(RU, static_cast<int>(ctx.t * 4) + vzero, 0, 0);
    const int xoff = (x_ok ? xr : 0) * es + vzero;
    const __amdgpu_buffer_rsrc_t RPX = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(uniform_u64(reinterpret_cast<uint64_t>(prow))), 0, x_ok ? V * es : 0, kBufWord3);
    const __amdgpu_buffer_rsrc_t RQX = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(uniform_u64(reinterpret_cast<uint64_t>(qrow))), 0, x_ok ? V * es : 0, kBufWord3);
    if constexpr (DT == 0) {
      lp_bits = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(RPX, xoff, 0, 0)) << 16;
      lq_bits = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(RQX, xoff, 0, 0)) << 16;
    } else {
      lp_bits = __builtin_amdgcn_raw_buffer_load_b32(RPX, xoff, 0, 0);
      lq_bits = __builtin_amdgcn_raw_buffer_load_b32(RQX, xoff, 0, 0);
    }
  }

  {  // stream the row (pair), or this workgroup's part of it
    LaneAcc L;
    lane_clear(L);
    constexpr bool PART = PHASE == 1;
    const int first = (PART ? ctx.part * kRowWaves : 0) + wave;
    const int step = kRowWaves * (PART ? a.split : 1);
    stream_row<DT, VEC, PAIR, MODE>(prow, qrow, ctx.beta, V, n_slices, first, step, lane, L);
    const float Mp = lane_max(L.mhp, L.mlp);
    correct_top(L.sp, Mp, kL2E, L.kp);
    if constexpr (MODE == 2) correct_top(L.stp, Mp, ctx.beta, L.ktp);
    if constexpr (PAIR) {
      const float Mq = lane_max(L.mhq, L.mlq);
      correct_top(L.sq, Mq, kL2E, L.kq);
      if constexpr (MODE == 2) correct_top(L.stq, Mq, ctx.beta, L.ktq);
    }
    lacc[tid] = L;  // the finalize reads the record back as it needs it
    if constexpr (PART) {
      // A part stores its lane records (folded: wave 0 folds the four waves' lanes first) at
      // the coherence point shared by every XCD; once every wave's are complete there wave 0
      // sets the part's arrival flag and reads the row's.  A part that finds every flag set
      // reads the records back from the coherence point, folds them and finishes the row; the
      // others are done.
      uint64_t* mine = part_records(a, ctx.unit, ctx.part);
      if (a.folded) {
        __syncthreads();
        if (wave == 0) {
#pragma unroll
          for (int q = 1; q < kRowWaves; ++q) lane_merge(L, lane_record(lacc[q * kFoldLanes + lane]));
          store_record<PAIR, MODE>(mine, lane, kFoldLanes, lane_record(L));
        }
      } else {
        store_record<PAIR, MODE>(mine, tid, kRowThreads, lane_record(L));
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      if (wave == 0) {
        uint32_t* flags = a.flags + ctx.unit * kFoldMaxParts;
        if (lane == 0) __hip_atomic_store(flags + ctx.part, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        const uint32_t e = lane < a.split
                               ? __hip_atomic_load(flags + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                               : a.epoch;
        const int all = __all(e == a.epoch);
        // every part has set its flag: back to 0, so that a replay of this launch with the
        // same epoch (a captured graph) starts from cleared flags
        if (all && lane < a.split)
          __hip_atomic_store(flags + lane, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) *sc.s_last = all ? 1 : 0;
      }
      __syncthreads();
      if (!*sc.s_last) return;
      PartFold pf;
      pf.load<PAIR, MODE>(a, ctx.unit, tid);
      pf.fold(a, tid, lacc);
    }
  }
  // (a split row's records were folded into lacc above, by the part that arrived last)
  const LaneAcc& A = lacc[tid];
  const int col_base = (PHASE != 0 && a.folded) ? kRowThreads : 0;  // how the lanes' columns are numbered

  // thread 0: the uniform's and the draft token's range checks
  auto input_flags = [&]() {
    int f = ctx.row_flags;
    if (!uniform_ok(__uint_as_float(u_bits))) f |= 16;  // SV_DEV_BAD_UNIFORM
    if (PAIR && !x_ok) f |= 4;                          // SV_DEV_BAD_TOKEN
    return f;
  };

  // Normalisers at T = 1 and T_b of the target row (and the draft row), with the target's first
  // argmax on greedy rows, in two rounds of block reductions.
  constexpr int NZ = (PAIR ? 2 : 1) * (MODE == 2 ? 2 : 1);
  float kz[NZ], Kz[NZ];
  double sz[NZ], LZ[NZ];
  kz[0] = A.kp;
  sz[0] = A.sp;
  if constexpr (PAIR) {
    kz[1] = A.kq;
    sz[1] = A.sq;
  }
  if constexpr (MODE == 2) {
    kz[NZ / 2] = A.ktp;
    sz[NZ / 2] = A.stp;
    if constexpr (PAIR) {
      kz[3] = A.ktq;
      sz[3] = A.stq;
    }
  }
  int argp = 0;
  lanes_lz_n<NZ, MODE == 1>(kz, sz, LZ, Kz, A.amax, A.aidx, &argp, sc.red_v);
  double LZ1p = LZ[0];
  const double LZTp0 = (MODE == 2) ? LZ[NZ / 2] : LZ1p;
  const float Kp_ref = Kz[0];
  const float scale_T = (MODE == 2) ? ctx.beta : kL2E;
  RowOut* slot = ctx.b >= 0 ? a.rowout + ctx.b * a.kmax1 + ctx.pos : nullptr;
  if constexpr (!PAIR) {  // a bonus row: its offsets and flags for the draw
    if (tid == 0 && ctx.b >= 0) {
      draw_offsets(LZTp0, &slot->offp, &slot->lzp);
      slot->beta = scale_T;
      slot->targ = argp;
      slot->flags = input_flags();
    }
    return;
  }

  // draft row
  double LZ1q = LZ[PAIR ? 1 : 0];
  const float Kq_ref = Kz[PAIR ? 1 : 0];
  const double LZTq = (MODE == 2) ? LZ[NZ - 1] : LZ1q;
  double Rsg = 0.0;
  bool rkl_done = false;
  bool heavy = false;
  int n_heavy = 0, heavy_at = -1;
  if (a.rkl_out) {
    // One round decides the row: R over the closed-form lanes, a lower bound on L1, the lanes
    // near the clip and the heavy lanes.  Most rows have neither and are done here.
    const LaneClosed L0 = lane_closed(A, LZ1p, LZ1q, a.delta);
    const HeavyParts hp = heavy_parts(A, LZ1p, LZ1q);
    double v[6];
    v[0] = L0.fail ? 0.0 : L0.closed;
    v[1] = lane_l1_lower(L0);
    v[2] = L0.fail ? 0.0 : L0.closed + L0.mass;
    v[3] = L0.fail ? 1.0 : 0.0;
    v[4] = hp.by_mass ? 1.0 : 0.0;
    v[5] = hp.err;
    block_reduce<6, 1u << 5>(v, sc.red_v);
    const double thr = heavy_threshold(v[1]);
    if (v[3] == 0.0 && v[4] == 0.0 && !(v[5] > thr)) {
      rkl_done = true;
      Rsg = v[2];
      if (tid == 0) {
        a.rkl_out[ctx.d] = static_cast<float>(v[0]);
        if (a.fix) a.fix[ctx.d].n = 0;
      }
    } else {
      heavy = is_heavy(hp, thr);
      n_heavy = list_lanes(heavy, sc.failed, sc.s_nheavy);
      if (a.fix && !a.stats && n_heavy <= kFixLanes) {
        // left to the draw launch: each heavy thread notes its place in the list
        if (heavy)
          for (int j = 0; j < n_heavy; ++j)
            if (sc.failed[j] == tid) heavy_at = j;
      } else if (n_heavy > 0) {
        exact_heavy_sums<DT, VEC>(prow, qrow, V, n_slices, lacc, sc, n_heavy, col_base);
        const float k2[2] = {A.kp, A.kq};  // A reads the replaced sums back
        const double s2[2] = {A.sp, A.sq};
        double lz2[2];
        float K2[2];
        lanes_lz_n<2, false>(k2, s2, lz2, K2, 0.0f, 0, nullptr, sc.red_v);
        LZ1p = lz2[0];
        LZ1q = lz2[1];
        n_heavy = 0;
      }
    }
  }
  const double LZTp = (MODE == 2) ? LZTp0 : LZ1p;
  const double LZTqf = (MODE == 2) ? LZTq : LZ1q;
  if (tid == 0 && ctx.b >= 0) {
    draw_offsets(LZTp, &slot->offp, &slot->lzp);
    slot->beta = scale_T;
    slot->targ = argp;
  }
  if (a.rkl_out && !rkl_done) {
    if (MODE == 1 && a.stats) {
      const LaneClosed L = lanes_clipped_rkl<DT, VEC, true, false>(prow, qrow, V, n_slices, LZ1p, LZ1q,
                                                                   a.delta, A, sc, col_base);
      double v[2] = {L.fail ? sc.direct[tid] : L.closed, L.fail ? sc.direct_x[tid] : L.closed + L.mass};
      block_reduce<2, 0u>(v, sc.red_v);
      Rsg = v[1];
      if (tid == 0) a.rkl_out[ctx.d] = static_cast<float>(v[0]);
    } else if (n_heavy == 0) {
      const LaneClosed L = lanes_clipped_rkl<DT, VEC, false, false>(prow, qrow, V, n_slices, LZ1p, LZ1q,
                                                                    a.delta, A, sc, col_base);
      const double R = block_sum_d(L.fail ? sc.direct[tid] : L.closed, red_d);
      if (tid == 0) {
        a.rkl_out[ctx.d] = static_cast<float>(R);
        if (a.fix) a.fix[ctx.d].n = 0;
      }
    } else {
      // Provisional R, and the record the draw launch finishes it from: the heavy lanes that
      // take the closed form (H) are summed apart; every other lane's part, its unclipped
      // terms and their q-mass let the launch move it to the exact normalisers.
      const LaneClosed L = lanes_clipped_rkl<DT, VEC, false, true>(prow, qrow, V, n_slices, LZ1p, LZ1q,
                                                                   a.delta, A, sc, col_base);
      const bool H = heavy && !L.fail;
      double v[kRowSums];
      v[0] = H ? 0.0 : (L.fail ? sc.direct[tid] : L.closed);
      v[1] = H ? L.closed : 0.0;
      v[2] = H ? 0.0 : (L.fail ? sc.direct_x[tid] : L.closed);
      v[3] = H ? 0.0 : (L.fail ? sc.direct_u0[tid] : L.mass);
      v[4] = (heavy || !(A.sp > 0.0)) ? 0.0 : ldexp(A.sp, static_cast<int>(A.kp - Kp_ref));
      v[5] = (heavy || !(A.sq > 0.0)) ? 0.0 : ldexp(A.sq, static_cast<int>(A.kq - Kq_ref));
      block_reduce<kRowSums, 0u>(v, sc.red_v);
      RklFix* fx = a.fix + ctx.d;
      if (heavy_at >= 0) {
        RklFixLane h;
        h.lane = tid + col_base;
        h.direct = L.fail ? 1 : 0;
        h.kp = A.kp;
        h.kq = A.kq;
        fx->h[heavy_at] = h;
      }
      if (tid == 0) {
        fx->r_rest = v[0];
        fx->u1 = v[2];
        fx->u0 = v[3];
        fx->lzp = LZ1p;
        fx->lzq = LZ1q;
        fx->sp_rest = v[4];
        fx->sq_rest = v[5];
        fx->kp_ref = Kp_ref;
        fx->kq_ref = Kq_ref;
        fx->n = n_heavy;
        fx->t_row = static_cast<int32_t>(ctx.t);
        a.rkl_out[ctx.d] = static_cast<float>(v[0] + v[1]);
      }
    }
  }
  if (MODE == 1 && a.stats && a.rkl_out && tid == 0) {
    RowStats st;
    st.lzp = LZ1p;
    st.lzq = LZ1q;
    st.sg = Rsg;
    st.top1 = argp;
    st.pad = 0;
    a.stats[ctx.d] = st;
  }
  if constexpr (MODE == 1) {
    // hard-label cross-entropy against the target's top-1 (AdaFlash paper, Section 3.1):
    // -ln q(x*) = -ln2 (l_q(x*) L2E - LZq), temperature 1
    if (a.hard_out && tid == 0) {
      const double lq = static_cast<double>(logit_at<DT>(qrow, argp));
      a.hard_out[ctx.d] = static_cast<float>(-kLn2 * (lq * static_cast<double>(kL2E) - LZ1q));
      if (a.top1_out) a.top1_out[ctx.d] = argp;
    }
  }
  if (tid == 0 && ctx.b >= 0) {
    draw_offsets(LZTqf, &slot->offq, &slot->lzq);
    const int row_flags = input_flags();
    slot->flags = row_flags;
    int accept = 0;
    if (row_flags == 0) {  // the request's own flags are combined by the sampler
      const double Lp = static_cast<double>(__uint_as_float(lp_bits)) * scale_T - LZTp;  // log2 p_T(x)
      const double Lq = static_cast<double>(__uint_as_float(lq_bits)) * scale_T - LZTqf;  // log2 q_T(x)
      if constexpr (MODE == 1) {
        accept = (xr == argp) ? 1 : 0;
      } else {
        const double ratio = fmin(1.0, exp2_d(Lp - Lq));
        accept = (static_cast<double>(__uint_as_float(u_bits)) < ratio) ? 1 : 0;
      }
      if (a.p_at) a.p_at[ctx.d] = static_cast<float>(exp2_d(Lp));
      if (a.q_at) a.q_at[ctx.d] = static_cast<float>(exp2_d(Lq));
    } else {
      if (a.p_at) store_nan(a.p_at + ctx.d);
      if (a.q_at) store_nan(a.q_at + ctx.d);
    }
    slot->acc = accept;
  }
}

// Verification layout: which target row a workgroup owns.  Units 0 .. n_d-1 are the draft
// rows (each with its target row), units n_d .. n_d+B-1 the bonus rows; the half-size bonus
// units run last and fill the tail of the grid.  Large batches read the plan's descriptors;
// otherwise every workgroup scans k itself (8 requests per thread), and unit 0 publishes the
// call's validity.  Returns false when the workgroup has nothing more to do (a void call,
// whose outputs it has written).  WITH_T: s_T receives the request's temperature (1 without
// a temperature array), read in the same round of loads as the lengths.
template <bool WITH_T>
__device__ __forceinline__ bool resolve_unit(const RowPairArgs& a, int64_t unit, int tid,
                                             int* red_i, int& s_req, int& s_off, int& s_t,
                                             int& s_void, float* s_T = nullptr) {
  if (a.desc) {  // large batch: descriptors and offsets from sv_plan
    if (a.glob[0]) {
      if (tid == 0 && unit < a.n_d) {
        if (a.fix) a.fix[unit].n = 0;
        if (a.rkl_out) store_nan(a.rkl_out + unit);
        if (a.p_at) store_nan(a.p_at + unit);
        if (a.q_at) store_nan(a.q_at + unit);
      }
      return false;
    }
    if (tid == 0) {
      const RowDesc rd = a.desc[unit];
      s_req = rd.b;
      s_off = a.off_t[rd.b];
      s_t = rd.t;
      if constexpr (WITH_T) *s_T = a.temperature ? a.temperature[rd.b] : 1.0f;
    }
    __syncthreads();
  } else {  // every workgroup scans k itself (B <= kInlinePlanMaxB, 8 requests per thread)
    if (tid == 0) {
      s_void = 0;
      s_req = -1;
    }
    __syncthreads();
    int kk[kInlinePerThread];
    float tt[kInlinePerThread];
    int tot = 0, bad = 0;
#pragma unroll
    for (int e = 0; e < kInlinePerThread; ++e) {
      const int64_t j = static_cast<int64_t>(tid) * kInlinePerThread + e;
      int v = 0;
      tt[e] = 1.0f;
      if (j < a.B) {
        if (WITH_T && a.temperature) tt[e] = a.temperature[j];
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
          if constexpr (WITH_T) *s_T = tt[e];
        } else if (unit >= a.n_d && unit - a.n_d == j) {
          s_req = static_cast<int>(j);
          s_off = off;
          s_t = off + kk[e] - 1;
          if constexpr (WITH_T) *s_T = tt[e];
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
        if (a.fix) a.fix[unit].n = 0;
        if (a.rkl_out) store_nan(a.rkl_out + unit);
        if (a.p_at) store_nan(a.p_at + unit);
        if (a.q_at) store_nan(a.q_at + unit);
      }
      return false;
    }
  }
  return s_req >= 0;  // false only when the layout is invalid, which the scan reports
}

// PHASE 0: one workgroup streams and finishes a row (pair).  PHASE 1: workgroup blockIdx
// streams part blockIdx % split of row (pair) blockIdx / split and stores its lane records;
// the part of the row that arrives last folds them and finishes the row.
template <int DT, bool VEC, int PHASE>
__global__ __launch_bounds__(kRowThreads) __attribute__((amdgpu_waves_per_eu(1)))
void sv_rowpair_kernel(RowPairArgs a) {
  __shared__ LaneAcc lacc[kRowThreads];
  __shared__ double direct[kRowThreads];
  __shared__ double direct_x[kRowThreads];
  __shared__ double direct_u0[kRowThreads];
  __shared__ int failed[kRowThreads];
  __shared__ int s_nfail, s_nheavy, s_last;
  __shared__ double red_d[kRowWaves];
  __shared__ float red_f[kRowWaves];
  __shared__ int red_i[kRowWaves];
  __shared__ double red_v[kRowWaves * kRowSums];
  __shared__ int s_req, s_off, s_t, s_void;
  __shared__ float s_T;
  const Scratch sc{lacc, direct, direct_x, direct_u0, failed, &s_nfail, &s_nheavy, &s_last, red_d, red_f, red_i, red_v};
  const int tid = thread_index();
  const int64_t blk = block_index();
  const int64_t unit = PHASE == 1 ? blk / a.split : blk;

  RowCtx ctx;
  ctx.unit = unit;
  ctx.part = PHASE == 1 ? static_cast<int>(blk - unit * a.split) : 0;
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
        if (a.hard_out) store_nan(a.hard_out + unit);
        if (a.top1_out) a.top1_out[unit] = -1;
        a.row_flags[unit] = 2;  // SV_DEV_ROWS_MISMATCH
      }
      return;
    }
    if (tid == 0) a.row_flags[unit] = 0;
    if (a.hard_out) {  // with the hard-label cross-entropy: track the target row's argmax
      ctx.mode = 1;
      rowpair_body<DT, VEC, PHASE, true, 1>(a, ctx, sc, -1);
    } else {
      rowpair_body<DT, VEC, PHASE, true, 0>(a, ctx, sc, -1);
    }
    return;
  }

  // the draft token (draft units 0 .. n_d-1 are the draft rows in packed order), the same for
  // every thread, is fetched with the lengths and temperatures; it is checked, and the logits
  // at it are fetched, once the row has been streamed
  int32_t xr = -1;
  if (unit < a.n_d) xr = a.tokens[unit];
  if (!resolve_unit<true>(a, unit, tid, red_i, s_req, s_off, s_t, s_void, &s_T)) return;
  const int64_t b = s_req;
  const int64_t off = s_off;
  ctx.t = s_t;
  const int i = static_cast<int>(ctx.t - off);
  ctx.b = b;
  ctx.pos = i;
  ctx.d = unit < a.n_d ? unit : -1;
  const float T = s_T;
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
  if (i == 0 && tid == 0 && !a.desc) {
    a.off_t[b] = static_cast<int32_t>(off);
    if (a.arrive) a.arrive[b] = 0;  // the draw kernel counts its workgroups from zero
  }
  ctx.row_flags = flags;  // thread 0 adds the token and uniform bits after the stream
  if (ctx.d >= 0) {
    if (ctx.mode == 0) rowpair_body<DT, VEC, PHASE, true, 0>(a, ctx, sc, xr);
    if (ctx.mode == 1) rowpair_body<DT, VEC, PHASE, true, 1>(a, ctx, sc, xr);
    if (ctx.mode == 2) rowpair_body<DT, VEC, PHASE, true, 2>(a, ctx, sc, xr);
  } else {
    if (ctx.mode == 0) rowpair_body<DT, VEC, PHASE, false, 0>(a, ctx, sc, xr);
    if (ctx.mode == 1) rowpair_body<DT, VEC, PHASE, false, 1>(a, ctx, sc, xr);
    if (ctx.mode == 2) rowpair_body<DT, VEC, PHASE, false, 2>(a, ctx, sc, xr);
  }
}

// ----------------------------------------------------------------------------- greedy
// Greedy verification (every T_b = 0; the paper's default decoding, Appendix B.1): only the
// target rows' first argmax is needed (DFlash notes, Section 5.2, worked example #4), so one
// workgroup streams one target row and nothing else.  Per lane, the running maximum and the
// slice where it first appeared; the lanes holding the row maximum then look again at that one
// slice for the first column.  Writes the argmax, the acceptance flag x_i == argmax (draft-position
// rows) and the row's token flag; the pick kernel then scans and emits.
template <int DT, bool VEC>
__device__ __forceinline__ void stream_max(const void* prow, int V, int n_slices, int wave,
                                           int lane, float& best, int& best_s) {
  const int n_full = V / kSlice;
  int s = wave;
  if constexpr (DT == 0 && VEC) {
    // Four slices in flight through bounds-checked buffer loads (past the row's last full
    // slice they read zeros without touching memory).  Every round takes four slices and
    // refills four, with one exit at the bottom: a slice past the row counts as -inf through a
    // select, so no load sits under a branch and no wait has to cover a refill.  Each refill
    // is pinned where it stands (the compiler would otherwise sink it next to its use).
    const __amdgpu_buffer_rsrc_t RP = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(prow), 0, n_full * kSlice * 2, kBufWord3);
    const int lane_off = lane * 16;
    auto at = [&](int sl) { return lane_off + sl * (kSlice * 2); };
    auto pin = [] { asm volatile("" ::: "memory"); };
    auto take = [&](const PackedRow& r, int sl) {
      const float m = sl < n_full ? r.max() : -INFINITY;
      if (m > best) {
        best = m;
        best_s = sl;
      }
    };
    PackedRow r0, r1, r2, r3;
    if (s < n_full) {
      r0.load(RP, at(s));
      r1.load(RP, at(s + kRowWaves));
      r2.load(RP, at(s + 2 * kRowWaves));
      r3.load(RP, at(s + 3 * kRowWaves));
      do {
        take(r0, s);
        r0.load(RP, at(s + 4 * kRowWaves));
        pin();
        take(r1, s + kRowWaves);
        r1.load(RP, at(s + 5 * kRowWaves));
        pin();
        take(r2, s + 2 * kRowWaves);
        r2.load(RP, at(s + 6 * kRowWaves));
        pin();
        take(r3, s + 3 * kRowWaves);
        r3.load(RP, at(s + 7 * kRowWaves));
        pin();
        s += 4 * kRowWaves;
      } while (s < n_full);
      // s is now the first slice index of this wave past the full slices
      s = n_full + ((wave - n_full) % kRowWaves + kRowWaves) % kRowWaves;
    }
  }
  for (; s < n_slices; s += kRowWaves) {
    FloatRow f;
    f.template load<DT, VEC>(prow, static_cast<int64_t>(s) * kSlice + lane * 8, V);
    const float m = f.max();
    if (m > best) {
      best = m;
      best_s = s;
    }
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kRowThreads) void sv_greedy_kernel(RowPairArgs a) {
  __shared__ float red_f[kRowWaves];
  __shared__ int red_i[kRowWaves];
  __shared__ int s_req, s_off, s_t, s_void;
  const int tid = thread_index(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t unit = block_index();
  if (!resolve_unit<false>(a, unit, tid, red_i, s_req, s_off, s_t, s_void)) return;
  const int64_t b = s_req, off = s_off, t = s_t;
  const int kb = a.k[b];
  const int i = static_cast<int>(t - off);
  const int64_t d = (i < kb) ? (off - b + i) : -1;
  if (i == 0 && tid == 0 && !a.desc) {
    a.off_t[b] = static_cast<int32_t>(off);
    if (a.arrive) a.arrive[b] = 0;  // the draw kernel counts its workgroups from zero
  }
  const void* prow = static_cast<const char*>(a.target) + t * a.ld_t * (DT == 0 ? 2 : 4);

  float best = -INFINITY;
  int best_s = -1;
  stream_max<DT, VEC>(prow, a.V, static_cast<int>(a.n_slices), wave, lane, best, best_s);
  const float Mx = block_max_f(best, red_f);
  int col = 0x7fffffff;
  if (best == Mx && best_s >= 0) {  // first column of the maximum inside that slice
    FloatRow f;
    f.template load<DT, VEC>(prow, static_cast<int64_t>(best_s) * kSlice + lane * 8, a.V);
#pragma unroll
    for (int e = kElemsPerLane - 1; e >= 0; --e)
      if (f.at(e) == Mx) col = best_s * kSlice + (e >> 3) * 512 + lane * 8 + (e & 7);
  }
  const int argp = block_min_i(col, red_i);
  if (tid == 0) {
    RowOut* slot = a.rowout + b * a.kmax1 + i;
    slot->targ = argp;
    int flags = 0;
    if (d >= 0) {
      const int32_t x = a.tokens[d];
      if (x < 0 || x >= a.V) flags |= 4;  // SV_DEV_BAD_TOKEN
      slot->acc = (flags == 0 && x == argp) ? 1 : 0;
    }
    slot->flags = flags;
  }
}

hipError_t launch_greedy(int dtype, bool vec, const RowPairArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.n_units));
  if (a.n_units == 0) return hipSuccess;
  if (dtype == 0) {
    if (vec) hipLaunchKernelGGL((sv_greedy_kernel<0, true>), grid, dim3(kRowThreads), 0, st, a);
    else hipLaunchKernelGGL((sv_greedy_kernel<0, false>), grid, dim3(kRowThreads), 0, st, a);
  } else {
    if (vec) hipLaunchKernelGGL((sv_greedy_kernel<1, true>), grid, dim3(kRowThreads), 0, st, a);
    else hipLaunchKernelGGL((sv_greedy_kernel<1, false>), grid, dim3(kRowThreads), 0, st, a);
  }
  return hipGetLastError();
}

// First argmax (lowest id among the maxima) of every row: one workgroup per row, the greedy
// stream, then the lanes holding the row maximum look at that one slice again.
template <int DT, bool VEC>
__global__ __launch_bounds__(kRowThreads) void sv_row_argmax_kernel(ArgmaxArgs a) {
  __shared__ float red_f[kRowWaves];
  __shared__ int red_i[kRowWaves];
  const int tid = thread_index(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t = block_index();
  const void* prow = static_cast<const char*>(a.target) + t * a.ld_t * (DT == 0 ? 2 : 4);
  float best = -INFINITY;
  int best_s = -1;
  stream_max<DT, VEC>(prow, a.V, static_cast<int>(a.n_slices), wave, lane, best, best_s);
  const float Mx = block_max_f(best, red_f);
  int col = 0x7fffffff;
  if (best == Mx && best_s >= 0) {
    FloatRow f;
    f.template load<DT, VEC>(prow, static_cast<int64_t>(best_s) * kSlice + lane * 8, a.V);
#pragma unroll
    for (int e = kElemsPerLane - 1; e >= 0; --e)
      if (f.at(e) == Mx) col = best_s * kSlice + (e >> 3) * 512 + lane * 8 + (e & 7);
  }
  const int arg = block_min_i(col, red_i);
  if (tid == 0) {
    a.arg[t] = arg;
    if (t == 0 && a.zero_status) *a.zero_status = 0;
  }
}

hipError_t launch_row_argmax(int dtype, bool vec, const ArgmaxArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.n_rows));
  if (a.n_rows == 0) return hipSuccess;
  if (dtype == 0) {
    if (vec) hipLaunchKernelGGL((sv_row_argmax_kernel<0, true>), grid, dim3(kRowThreads), 0, st, a);
    else hipLaunchKernelGGL((sv_row_argmax_kernel<0, false>), grid, dim3(kRowThreads), 0, st, a);
  } else {
    if (vec) hipLaunchKernelGGL((sv_row_argmax_kernel<1, true>), grid, dim3(kRowThreads), 0, st, a);
    else hipLaunchKernelGGL((sv_row_argmax_kernel<1, false>), grid, dim3(kRowThreads), 0, st, a);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- launch
hipError_t launch_rowpair(int dtype, bool vec, const RowPairArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.n_units * (a.phase == 1 ? a.split : 1)));
  if (a.n_units == 0) return hipSuccess;
  if (a.phase < 0 || a.phase > 1 ||
      (a.phase == 1 && (a.split < 2 || a.split > kFoldMaxParts || !a.rec || !a.flags || a.epoch == 0)))
    return hipErrorInvalidValue;
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(kRowThreads), 0, st, a); };
  auto by_phase = [&](auto k0, auto k1) {
    if (a.phase == 0) go(k0);
    else go(k1);
  };
  if (dtype == 0) {
    if (vec) by_phase(sv_rowpair_kernel<0, true, 0>, sv_rowpair_kernel<0, true, 1>);
    else by_phase(sv_rowpair_kernel<0, false, 0>, sv_rowpair_kernel<0, false, 1>);
  } else {
    if (vec) by_phase(sv_rowpair_kernel<1, true, 0>, sv_rowpair_kernel<1, true, 1>);
    else by_phase(sv_rowpair_kernel<1, false, 0>, sv_rowpair_kernel<1, false, 1>);
  }
  return hipGetLastError();
}

}  // namespace sv
