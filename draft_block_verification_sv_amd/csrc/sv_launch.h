// Kernel argument blocks and the internal (C++) launch functions the C ABI calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_layout.h"

namespace sv {

struct PlanArgs {
  int64_t B;
  int32_t k_max;
  int64_t n_d;
  const int32_t* k;
  Workspace ws;
  int32_t* device_status;
};

struct RowPairArgs {
  const void* target;
  const void* draft;
  int64_t ld_t, ld_d;
  int32_t V;
  int64_t n_slices;
  int64_t n_units;  // workgroups: target rows (verification) or draft rows (rKL only)
  // verification
  int64_t B;
  int32_t k_max;
  int64_t n_d;
  const int32_t* k;
  const int32_t* tokens;
  const float* uniforms;
  const float* temperature;  // nullable
  const RowDesc* desc;       // nullptr: every workgroup scans k itself
  int32_t* glob;
  int32_t* off_t;
  // clipped reverse-KL only
  bool rkl_only;
  const int32_t* p_row_index;  // nullable = identity
  int64_t n_target_rows;
  // outputs
  float delta;
  float* rkl_out;  // nullable in verification
  float* hard_out;    // rKL only, nullable: -ln q(x*), x* the target row's first argmax
  int32_t* top1_out;  // rKL only, nullable: x*
  RowStats* stats;    // rKL only, nullable: statistics for the OPD gradient pass
  float* p_at;     // nullable
  float* q_at;     // nullable
  int32_t* device_status;
  int32_t* row_flags;  // reverse-KL calls: per draft row
  RowOut* rowout;      // verification: per (request, position), for the draw
  int32_t kmax1;       // k_max + 1: slots per request in rowout
  int32_t* arrive;  // nullable: per-request draw counters, zeroed here for the draw kernel
  // Rows split over several workgroups (small launches): phase 0 streams and finalizes each
  // row (pair) in one workgroup; phase 1 streams part `blockIdx % split` of row (pair)
  // `blockIdx / split`, stores its lane records in rec and sets its arrival flag (the launch's
  // nonzero epoch); the part that finds every part of its row arrived folds the row's records
  // and finalizes it.
  int32_t phase;
  int32_t split;
  void* rec;       // [n_units * split * rec_lanes(folded)] lane records
  int32_t folded;  // parts fold their four waves: kFoldLanes records a part, else kRowThreads
  uint32_t* flags;  // [n_units * 16]
  uint32_t epoch;
  // verification with the reverse-KL, nullable: rows whose heavy lanes the draw launch sums
  RklFix* fix;  // [n_d]
};

struct SampleArgs {
  const void* target;
  const void* draft;
  int64_t ld_t, ld_d;
  int32_t V;
  int64_t n_chunks;
  int64_t B;
  int64_t n_t;
  const int32_t* glob;
  const int32_t* off_t;
  const int32_t* k;
  const float* temperature;
  const int32_t* tokens;
  const float* uniforms;
  const RowOut* rowout;  // [B * kmax1] per (request, position)
  int32_t kmax1;
  double* chunk_mass;   // [B * n_chunks]: each draw workgroup's chunk masses
  int32_t* arrive;      // [B]: draw workgroups of the request done; the last one picks
  bool force_greedy;    // every request greedy (sv_verify_block_greedy): T_b = 0
  int32_t mass_blocks;  // draw workgroups per request
  int32_t* accept_len;
  int32_t* out_tokens;
  float* p_at;
  float* q_at;
  int32_t* device_status;
  // the reverse-KL rows the streaming pass left to this launch (nullable)
  float* rkl_out;
  const RklFix* fix;
  int64_t n_slices;  // the streaming pass's slices per row (lane geometry of the records)
  // with the reverse-KL, n_d: the workgroups after the B * mass_blocks drawing ones, one per
  // draft row, that finish the rows the streaming pass left to this launch (0: none)
  int64_t fix_rows;
};

hipError_t launch_plan(const PlanArgs& a, hipStream_t st);
hipError_t launch_rowpair(int dtype, bool vec, const RowPairArgs& a, hipStream_t st);
hipError_t launch_opd_reduce(const int32_t* k, int64_t B, int64_t n_rows, const float* rkl,
                             const float* hard, float alpha, const int32_t* row_flags,
                             float* opd_out, float* coef, int32_t* device_status, hipStream_t st);

// The gradient pass of the OPD loss: one workgroup per draft row.
struct GradArgs {
  const void* target;
  const void* draft;
  int64_t ld_t, ld_d, ld_g;
  int32_t V;
  int64_t n_rows, n_target_rows;
  const int32_t* p_row_index;  // nullable = identity
  float delta;
  const RowStats* stats;
  const float* coef;  // NaN for a void call (bad lengths): the gradient is NaN
  void* grad;         // [n_rows, ld_g] of the gradient dtype
};
hipError_t launch_opd_grad(int dtype, int grad_dtype, bool vec, const GradArgs& a, hipStream_t st);

// The adaptive length head.
struct HeadArgs {
  int64_t B;
  int32_t k;       // positions per request
  int32_t H, Hf;   // hidden size (multiple of 32), features
  const void* h;   // bf16 [B * k, ld_h]
  int64_t ld_h;
  const void* W1;  // bf16 [Hf, ld_w]
  int64_t ld_w;
  const float* b1;  // [Hf] or null
  const float* w2;  // [Hf]
  float b2, gamma;
  int32_t R;        // 16-row blocks per request: ceil(k / 16)
  int64_t NB;       // blocks in all: B R
  int32_t S;        // K-chunks of the split-K projection
  float* partial;   // workspace [S][NB * 16][Hf]: the chunks' partial sums of W1 h^T
  int32_t* ticket;  // workspace: pooling workgroups done (zeroed by the projection kernel)
  float* a_hat;     // [B]
  int32_t* k_hat;   // [B]
  int32_t* off_t;   // [B + 1] or null
};
constexpr int64_t kHeadSplitTarget = 512;  // workgroups the projection's K split aims for
// Blocks per workgroup and features per workgroup of the projection.
constexpr int kHeadBlocks = 4;
constexpr int kHeadTileN = 256;
constexpr int kHeadMaxSplit = 8;  // K-chunks at most
// The split of the projection for a head call: K-chunks so that the grid has about
// kHeadSplitTarget workgroups (at most kHeadMaxSplit chunks, at least one K step of 32
// each).
inline HeadArgs head_split(int64_t B, int32_t k, int32_t H, int32_t Hf) {
  HeadArgs a{};
  a.B = B;
  a.k = k;
  a.H = H;
  a.Hf = Hf;
  a.R = (k + 15) / 16;
  a.NB = B * a.R;
  const int64_t tiles = ((a.NB + kHeadBlocks - 1) / kHeadBlocks) * ((Hf + kHeadTileN - 1) / kHeadTileN);
  int64_t S = (kHeadSplitTarget + tiles - 1) / tiles;
  S = S < 1 ? 1 : (S > kHeadMaxSplit ? kHeadMaxSplit : S);
  if (S > H / 32) S = H / 32;
  a.S = static_cast<int32_t>(S);
  return a;
}
inline size_t head_partial_bytes(const HeadArgs& a) {
  return static_cast<size_t>(a.S) * static_cast<size_t>(a.NB) * 16 * static_cast<size_t>(a.Hf) * sizeof(float);
}
// Workspace: the partial sums, then (256-byte aligned) the pooling ticket.
inline size_t head_ticket_offset(const HeadArgs& a) { return (head_partial_bytes(a) + 255) & ~size_t(255); }
inline size_t head_workspace_bytes(const HeadArgs& a) { return head_ticket_offset(a) + 256; }
hipError_t launch_head(const HeadArgs& a, hipStream_t st);
hipError_t launch_head_pool(const HeadArgs& a, hipStream_t st);
hipError_t launch_len_loss(int64_t B, const float* a_hat, const int32_t* accept_len,
                           const int32_t* k_hat, float* loss, float* dloss, hipStream_t st);
hipError_t launch_status(const int32_t* row_flags, int64_t n, int32_t* device_status, hipStream_t st);
hipError_t launch_greedy(int dtype, bool vec, const RowPairArgs& a, hipStream_t st);
hipError_t launch_draw(int dtype, bool vec, const SampleArgs& a, hipStream_t st);

// Lookup of a prepared successor block after verification.
struct BranchArgs {
  int64_t B;
  int32_t k_max, n_branch;
  int64_t n_tokens;
  const int32_t* k;
  const int32_t* accept_len;
  const int32_t* out_tokens;
  const int32_t* branch_pos;  // [B, n_branch]
  const int32_t* branch_tok;  // [B, n_branch]
  int32_t* hit;               // [B]
};
hipError_t launch_branch(const BranchArgs& a, hipStream_t st);

// Greedy tree verification: the argmax of every target row, then the walk.
struct ArgmaxArgs {
  const void* target;
  int64_t ld_t;
  int32_t V;
  int64_t n_slices;
  int64_t n_rows;
  int32_t* arg;            // [n_rows]
  int32_t* zero_status;    // nullable: set to 0 by the first workgroup (for a later kernel)
};
hipError_t launch_row_argmax(int dtype, bool vec, const ArgmaxArgs& a, hipStream_t st);
struct TreeArgs {
  int64_t B;
  int32_t max_nodes;
  int32_t V;
  int64_t n_nodes_total;
  const int32_t* n_nodes;
  const int32_t* parent;
  const int32_t* tokens;
  const int32_t* arg;  // argmax of every target row
  int32_t* accept_len;
  int32_t* out_tokens;
  int32_t* out_nodes;  // nullable
  int32_t* device_status;
};
hipError_t launch_tree_walk(const TreeArgs& a, hipStream_t st);

// Diagnostics: a plain read of n_words 16-byte words; out receives kReadProbeBlocks words.
constexpr int kReadProbeBlocks = 1024;
hipError_t launch_read_probe(const void* data, int64_t n_words, uint32_t* out, hipStream_t st);

}  // namespace sv
