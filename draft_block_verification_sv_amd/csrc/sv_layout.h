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
constexpr int kElemsPerLane = 16;
static_assert(kElemsPerLane % 8 == 0 && kElemsPerLane >= 8, "groups of 8 columns per lane");
constexpr int kGroups = kElemsPerLane / 8;
constexpr int kSlice = 64 * kElemsPerLane;
// The streaming kernel: one 256-thread workgroup (4 waves) per target row (and the
// draft row it pairs with); per-slice records live in LDS, so a row has at most
// kMaxSlices slices (V <= 524288 at 16 elements per lane).
constexpr int kRowWaves = 4;
constexpr int kRowThreads = 64 * kRowWaves;
constexpr int kMaxSlices = 512;
// Up to kInlinePlanMaxB requests every workgroup scans k itself; beyond, sv_plan
// writes per-row descriptors first.
constexpr int kInlinePerThread = 8;
constexpr int kInlinePlanMaxB = kRowThreads * kInlinePerThread;
// The draw works on chunks of kChunk columns (one wave, kChunkGroups groups of 8 per
// lane).  sv_draw: 256-thread workgroups of kMassChunksPerBlock chunks each, so a request's
// row is spread over ceil(n_chunks / kMassChunksPerBlock) workgroups; the last of them to
// finish scans the request's chunk masses with one wave (V <= kMaxChunks * kChunk).
constexpr int kChunkGroups = 4;
constexpr int kChunk = 64 * 8 * kChunkGroups;
constexpr int kMassWaves = 4;
constexpr int kMassThreads = 64 * kMassWaves;
constexpr int kMassChunksPerBlock = 2 * kMassWaves;
constexpr int kMaxChunks = 1024;

inline int64_t n_slices_for(int64_t V) { return (V + kSlice - 1) / kSlice; }

// Small launches split each row (pair) over several streaming workgroups, which store their
// lane records (at most kLaneRecBytes each) for the finalize: one per thread, or when a row has
// at least kFoldMinSplit parts, kFoldLanes, the part's four waves folded lane by lane.  Only
// launches of at most kSplitMaxUnits rows split (with more, one workgroup per row already
// covers most of the chip and the records and their fold cost more than they save); they take
// at most kSplitTarget streaming workgroups (two per CU, which the split kernel's registers
// allow at once: a launch that needs a second round of workgroups is slower), with at most 16
// parts per row, at least two slices per wave and at most kSplitSlots record sets in all.
constexpr int64_t kSplitTarget = 512;
constexpr int64_t kSplitMaxUnits = 128;
constexpr int64_t kSplitSlots = 1024;
constexpr size_t kLaneRecBytes = 72;
constexpr int kFoldLanes = 64;
constexpr int kFoldMinSplit = 9;
constexpr int rec_lanes(bool folded) { return folded ? kFoldLanes : kRowThreads; }
inline int row_split(int64_t n_units, int64_t n_slices) {
  if (n_units < 1 || n_units > kSplitMaxUnits) return 1;
  int64_t P = kSplitTarget / n_units;
  if (P > 16) P = 16;
  if (P > n_slices / 8) P = n_slices / 8;
  if (P > kSplitSlots / n_units) P = kSplitSlots / n_units;
  return P >= 2 ? static_cast<int>(P) : 1;
}
// Record sets to reserve for launches of at least min_units and at most max_units rows: the
// most any such launch splits into.
inline int64_t split_slots(int64_t min_units, int64_t max_units, int64_t n_slices) {
  int64_t most = 0;
  for (int64_t n = min_units < 1 ? 1 : min_units; n <= max_units && n <= kSplitMaxUnits; ++n) {
    const int P = row_split(n, n_slices);
    if (P > 1 && n * P > most) most = n * P;
  }
  return most;
}
inline int64_t n_chunks_for(int64_t V) { return (V + kChunk - 1) / kChunk; }
inline int64_t mass_blocks_for(int64_t n_chunks) {
  return (n_chunks + kMassChunksPerBlock - 1) / kMassChunksPerBlock;
}

// Per streaming unit, filled by the plan kernel (large batches only): units 0 .. n_d-1
// are the draft rows, units n_d .. n_d+B-1 the bonus rows.
struct RowDesc {
  int32_t t;  // target row
  int32_t b;  // request
};

// What the draw needs of one position i of request b, at slot b (k_max + 1) + i, so that the
// draw reads a request's positions without first reading where its rows start.  Written by the
// streaming pass (or the greedy stream) for i = 0 .. k_b.
struct RowOut {
  int32_t flags;  // SV_DEV_* bits found on the position's rows
  int32_t acc;    // draft i accepted (i < k_b)
  float beta;     // exp2 scale of the target row's temperature (log2(e) / T_b)
  float offp;     // -round(LZ) of p_T: p_T(y) = 2^(fma(l_y, beta, offp) - lzp)
  float lzp;
  float offq;     // likewise for q_T of draft row i (i < k_b)
  float lzq;
  int32_t targ;   // first argmax of the target row
};
static_assert(sizeof(RowOut) == 32, "two 16-byte loads per slot");

// Per draft row, from the OPD forward pass for the gradient pass: both log2 normalisers,
// sum_y q_y g_y (g_y = 1[t_y < delta] (ln q_y - ln p_y + 1)) and the target's top-1.
struct RowStats {
  double lzp, lzq, sg;
  int32_t top1;
  int32_t pad;
};

// Verification with the clipped reverse-KL: a draft row whose heavy lanes (lanes holding much
// of a row's mass, whose fp32 sums the streaming pass does not trust for the reverse-KL) number
// at most kFixLanes is finished by the draw launch.  The streaming pass writes its provisional
// reverse-KL and this record (n = 0 for every other row); the draw launch sums the heavy lanes
// again in fp64, forms the normalisers with them and moves R to them.  Sums are in log2 units
// as in the streaming pass.  The draw reads a record as kFixDwords 32-bit words, one per lane.
constexpr int kFixLanes = 8;
struct RklFixLane {
  int32_t lane;    // thread of the streaming workgroup that owned the lane
  int32_t direct;  // 1: the lane was summed term by term (near the clip); only its sums move
  float kp, kq;    // the lane's exp2 offsets
};
struct RklFix {
  double r_rest;            // R over every lane but the heavy closed-form ones
  double u1, u0;            // over those lanes: unclipped terms, and their q-mass
  double lzp, lzq;          // the normalisers the streaming pass used
  double sp_rest, sq_rest;  // the other lanes' sums scaled to 2^kp_ref and 2^kq_ref
  float kp_ref, kq_ref;     // the normalisers' reference offsets (largest lane offsets)
  int32_t n;       // heavy lanes recorded (0: R is final; nothing else is set then)
  int32_t t_row;   // the draft row's target row
  RklFixLane h[kFixLanes];
};
constexpr int kFixDwords = static_cast<int>(sizeof(RklFix) / 4);
static_assert(sizeof(RklFix) % 8 == 0 && kFixDwords <= 64, "one word per lane of a wave");
static_assert(offsetof(RklFix, kp_ref) == 56 && offsetof(RklFix, n) == 64 && offsetof(RklFix, t_row) == 68 &&
              offsetof(RklFix, h) == 72 && sizeof(RklFixLane) == 16, "word offsets the draw reads");

// Device pointers carved out of the caller's workspace.
struct Workspace {
  int32_t* glob;       // [4]: [0] call void (bad lengths / row count)
  int32_t* off_t;      // [B + 1] first target row of each request
  RowDesc* desc;       // [n_t] per unit (batches larger than kInlinePlanMaxB)
  int32_t* row_flags;  // [n_units] SV_DEV_* bits found on each row (reverse-KL calls)
  RowOut* rowout;      // [B * kmax1] per position, for the draw (verification calls)
  double* chunk_mass;  // [B * n_chunks] draw mass of each chunk of each request's draw row
  int32_t* arrive;     // [B] draw workgroups of each request done (zeroed by the streaming pass)
  void* rec;           // [rec_slots * kRowThreads] lane records of split rows
  RowStats* stats;     // [n_grad] OPD gradient: per-row forward statistics
  float* coef;         // [2 n_grad] OPD gradient: (alpha / k_b, (1 - alpha) / k_b) per row
  RklFix* fix;         // [n_d] verification: heavy lanes left to the draw launch per draft row
  uint32_t* flags;     // [n_units * 16] arrival flags of the parts of split rows
};

struct Dims {
  int64_t B, n_t, n_d, V, n_units, n_slices, n_chunks;
  int64_t kmax1;   // positions per request slot block: k_max + 1 (verification), else 0
  int64_t n_grad;  // rows of the OPD gradient pass (0 otherwise)
  int64_t rec_slots;  // record sets for split rows (0: launches of this size never split)
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
  w.glob = reinterpret_cast<int32_t*>(take(4 * sizeof(int32_t)));
  w.off_t = reinterpret_cast<int32_t*>(take((d.B + 1) * sizeof(int32_t)));
  w.desc = reinterpret_cast<RowDesc*>(take(d.n_t * sizeof(RowDesc)));
  w.row_flags = reinterpret_cast<int32_t*>(take(d.n_units * 4));
  w.rowout = reinterpret_cast<RowOut*>(take(static_cast<size_t>(d.B * d.kmax1) * sizeof(RowOut)));
  w.chunk_mass = reinterpret_cast<double*>(take(d.B * d.n_chunks * sizeof(double)));
  w.arrive = reinterpret_cast<int32_t*>(take(d.B * sizeof(int32_t)));
  w.rec = take(static_cast<size_t>(d.rec_slots) * kRowThreads * kLaneRecBytes);
  w.stats = reinterpret_cast<RowStats*>(take(d.n_grad * sizeof(RowStats)));
  w.coef = reinterpret_cast<float*>(take(d.n_grad * 2 * sizeof(float)));
  w.fix = reinterpret_cast<RklFix*>(take(d.n_d * sizeof(RklFix)));
  w.flags = reinterpret_cast<uint32_t*>(take(d.rec_slots > 0 ? d.n_units * 16 * sizeof(uint32_t) : 0));
  if (ws) *ws = w;
  return off;
}

}  // namespace sv
