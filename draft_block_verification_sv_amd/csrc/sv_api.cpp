// C ABI of libspecverify: argument validation, workspace carving and the launch
// sequence.  Everything host-checkable is checked before the first HIP call, so an
// invalid call returns its status without touching the device or the runtime.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/specverify.h"
#include "sv_launch.h"

namespace {

using sv::Dims;
using sv::Workspace;

constexpr int kNumKernels = 22;
const char* const kKernelNames[kNumKernels] = {
    "sv_plan",        "sv_rowpair",      "sv_draw",
    "sv_rkl_rowpair", "sv_rkl_status",   "sv_opd_rowpair", "sv_opd_status",
    "sv_opd_reduce",  "sv_grad_rowpair", "sv_grad_reduce", "sv_opd_grad",
    "sv_greedy_plan", "sv_greedy",       "sv_greedy_pick", "sv_head_feat",
    "sv_head_pool",   "sv_len_loss",
    "sv_branch",      "sv_tree_argmax",  "sv_tree_walk",    "sv_rowpair_split",
    "sv_read_probe"};
enum {
  K_PLAN,
  K_ROWPAIR,
  K_DRAW,
  K_RKL_ROWPAIR,
  K_RKL_STATUS,
  K_OPD_ROWPAIR,
  K_OPD_STATUS,
  K_OPD_REDUCE,
  K_GRAD_ROWPAIR,
  K_GRAD_REDUCE,
  K_GRAD,
  K_GREEDY_PLAN,
  K_GREEDY,
  K_GREEDY_PICK,
  K_HEAD_FEAT,
  K_HEAD_POOL,
  K_LEN_LOSS,
  K_BRANCH,
  K_TREE_ARGMAX,
  K_TREE_WALK,
  K_ROWPAIR_SPLIT,
  K_READ_PROBE
};

// ------------------------------------------------------------------ profiling
// An opt-in diagnostic: while it is on, every launch is bracketed by a pair of HIP events on
// the call's stream, and the pairs are folded into per-kernel totals when they are read.  While
// it is off (the default) a launch reads one atomic flag and touches nothing else, so calls on
// different streams never contend on the host.
struct ProfRec {
  int kernel;
  hipEvent_t start, stop;
};
struct Profiler {
  std::atomic<bool> on{false};
  std::mutex mu;  // guards everything below; taken only while profiling is on or being read
  std::vector<ProfRec> pending;
  std::vector<hipEvent_t> pool;
  int64_t launches[kNumKernels] = {};
  double total_ms[kNumKernels] = {};
};
Profiler& prof() {
  static Profiler p;
  return p;
}

// Callers hold p.mu.
hipEvent_t take_event() {
  Profiler& p = prof();
  if (!p.pool.empty()) {
    hipEvent_t e = p.pool.back();
    p.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
void give_event(hipEvent_t e) {
  if (e) prof().pool.push_back(e);
}

// Waits for pending event pairs and folds them into the per-kernel totals (callers hold p.mu).
hipError_t drain_pending() {
  Profiler& p = prof();
  hipError_t first = hipSuccess;
  for (const ProfRec& r : p.pending) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e == hipSuccess) {
      p.launches[r.kernel] += 1;
      p.total_ms[r.kernel] += ms;
    } else if (first == hipSuccess) {
      first = e;
    }
    p.pool.push_back(r.start);
    p.pool.push_back(r.stop);
  }
  p.pending.clear();
  return first;
}

template <class F>
hipError_t timed(int kernel, hipStream_t st, F&& launch) {
  Profiler& p = prof();
  if (!p.on.load(std::memory_order_relaxed)) return launch();
  std::lock_guard<std::mutex> lock(p.mu);
  hipEvent_t a = take_event(), b = take_event();
  hipError_t e = (a && b) ? hipEventRecord(a, st) : hipErrorOutOfMemory;
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(b, st);
  if (e != hipSuccess) {  // the events go back to the pool; the launch error is the result
    give_event(a);
    give_event(b);
    return e;
  }
  p.pending.push_back({kernel, a, b});
  return hipSuccess;
}

// ------------------------------------------------------------------ helpers
bool dtype_ok(int32_t dtype) { return dtype == SV_BF16 || dtype == SV_F32; }
int64_t esize(int32_t dtype) { return dtype == SV_BF16 ? 2 : 4; }

bool vec_ok(int32_t dtype, int64_t ld, const void* base) {
  const int64_t per16 = 16 / esize(dtype);
  return (ld % per16) == 0 && (reinterpret_cast<uintptr_t>(base) % 16) == 0;
}

Dims verify_dims(int64_t B, int64_t k_max, int64_t V) {
  Dims d{};
  d.B = B;
  d.n_t = B * (k_max + 1);
  d.n_d = B * k_max;
  d.V = V;
  d.n_units = d.n_t;
  d.kmax1 = k_max + 1;
  d.n_slices = sv::n_slices_for(V);
  d.n_chunks = sv::n_chunks_for(V);
  d.rec_slots = sv::split_slots(2 * B, d.n_t, d.n_slices);  // a call has between 2B and B (k_max + 1) rows
  return d;
}

Dims rkl_dims(int64_t n_rows, int64_t V, bool with_grad = false) {
  Dims d{};
  d.n_grad = with_grad ? n_rows : 0;
  d.B = 1;
  d.n_t = 0;
  d.n_d = 0;
  d.V = V;
  d.n_units = n_rows;
  d.n_slices = sv::n_slices_for(V);
  d.n_chunks = 0;
  d.rec_slots = sv::split_slots(n_rows, n_rows, d.n_slices);
  return d;
}

bool shape_ok(int64_t V, int64_t ld_t, int64_t ld_d) {
  return V >= 1 && V <= SV_MAX_VOCAB && sv::n_slices_for(V) <= sv::kMaxSlices &&
         sv::n_chunks_for(V) <= sv::kMaxChunks && ld_t >= V && ld_d >= V;
}

}  // namespace

namespace {

// Epochs of the launches that fold split rows: distinct for 2^32 launches in the process, never
// 0, and spread over all 32 bits by an invertible mix, so that a flag word left in the
// workspace by other use (small integers, floats) matches the epoch of a launch only by chance.
uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{0};
  while (true) {
    uint32_t x = counter.fetch_add(1, std::memory_order_relaxed) + 1;
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    if (x != 0) return x;
  }
}

// A workspace that lacks room for the lane records of split rows but holds everything else
// (one sized for a larger call, say) is used without them: the call then streams each row in
// one workgroup.
bool fit_workspace(const void* workspace, size_t bytes, Dims& dm) {
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % 256) != 0) return false;
  if (bytes >= sv::carve(dm, nullptr, nullptr)) return true;
  dm.rec_slots = 0;
  return bytes >= sv::carve(dm, nullptr, nullptr);
}

// The streaming pass over n_units rows (pairs): one launch, each row streamed by one workgroup,
// or for small launches by several (the part of a row that arrives last finishes it).
hipError_t run_rowpair(int dtype, bool vec, sv::RowPairArgs ra, const Workspace& ws, int64_t rec_slots,
                       hipStream_t st, int k_whole) {
  const int P = rec_slots > 0 ? sv::row_split(ra.n_units, ra.n_slices) : 1;
  const bool split = P >= 2 && ra.n_units * P <= rec_slots;
  ra.folded = split && P >= sv::kFoldMinSplit ? 1 : 0;
  if (!split) {
    ra.phase = 0;
    ra.split = 1;
    return timed(k_whole, st, [&] { return sv::launch_rowpair(dtype, vec, ra, st); });
  }
  ra.phase = 1;
  ra.split = P;
  ra.rec = ws.rec;
  ra.flags = ws.flags;
  ra.epoch = next_epoch();
  return timed(K_ROWPAIR_SPLIT, st, [&] { return sv::launch_rowpair(dtype, vec, ra, st); });
}

// The clipped reverse-KL of n_rows row pairs, and with hard_out the hard-label
// cross-entropy against each target row's top-1: sv_clipped_rkl and sv_opd_loss.
sv_status rkl_rows(int32_t dtype, int64_t n_rows, int64_t n_target_rows, int64_t V,
                   int64_t ld_target, int64_t ld_draft, const void* target_logits,
                   const void* draft_logits, const int32_t* p_row_index, float delta,
                   float* rkl_out, float* hard_out, int32_t* top1_out, int32_t* device_status,
                   void* workspace, size_t workspace_bytes, hipStream_t st, int k_rowpair,
                   int k_status, Workspace* ws_out, bool with_grad = false) {
  if (!dtype_ok(dtype)) return SV_ERR_DTYPE;
  if (n_rows < 1 || n_target_rows < 1 || !shape_ok(V, ld_target, ld_draft)) return SV_ERR_SHAPE;
  if (!p_row_index && n_target_rows < n_rows) return SV_ERR_SHAPE;
  if (n_rows >= (int64_t(1) << 31)) return SV_ERR_SHAPE;
  Dims dm = rkl_dims(n_rows, V, with_grad);
  if (!target_logits || !draft_logits || !rkl_out || !device_status) return SV_ERR_NULL;
  if (!(std::isfinite(delta) && delta > 0.0f)) return SV_ERR_VALUE;
  if (!fit_workspace(workspace, workspace_bytes, dm)) return SV_ERR_WORKSPACE;

  Workspace ws{};
  sv::carve(dm, &ws, static_cast<char*>(workspace));
  const bool vec = vec_ok(dtype, ld_target, target_logits) && vec_ok(dtype, ld_draft, draft_logits);

  sv::RowPairArgs ra{};
  ra.target = target_logits;
  ra.draft = draft_logits;
  ra.ld_t = ld_target;
  ra.ld_d = ld_draft;
  ra.V = static_cast<int32_t>(V);
  ra.n_slices = dm.n_slices;
  ra.n_units = n_rows;
  ra.rkl_only = true;
  ra.p_row_index = p_row_index;
  ra.n_target_rows = n_target_rows;
  ra.delta = delta;
  ra.rkl_out = rkl_out;
  ra.hard_out = hard_out;
  ra.top1_out = top1_out;
  ra.stats = with_grad ? ws.stats : nullptr;
  ra.device_status = device_status;
  ra.row_flags = ws.row_flags;
  if (run_rowpair(dtype, vec, ra, ws, dm.rec_slots, st, k_rowpair) != hipSuccess) return SV_ERR_HIP;
  if (ws_out) {  // the caller folds the row flags into its own final kernel
    *ws_out = ws;
    return SV_OK;
  }
  if (timed(k_status, st,
            [&] { return sv::launch_status(ws.row_flags, n_rows, device_status, st); }) !=
      hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

}  // namespace

extern "C" {

const char* sv_version(void) { return "libspecverify 0.1.0 (gfx950)"; }

const char* sv_status_string(sv_status s) {
  switch (s) {
    case SV_OK: return "ok";
    case SV_ERR_NULL: return "a required pointer is NULL";
    case SV_ERR_SHAPE: return "shape out of range (B, k_max, V, ld or row count)";
    case SV_ERR_DTYPE: return "unknown dtype (expected SV_BF16 or SV_F32)";
    case SV_ERR_VALUE: return "delta must be finite and > 0 when the reverse-KL is requested";
    case SV_ERR_WORKSPACE: return "workspace missing, not 256-byte aligned, or too small";
    case SV_ERR_HIP: return "HIP runtime error or kernel launch failure";
    case SV_ERR_SCRATCH: return "the call needs more scratch than the library's fixed 16 MiB buffer holds";
    default: return "unknown status";
  }
}

size_t sv_workspace_size(int32_t B, int32_t k_max, int64_t V, int32_t dtype) {
  if (!dtype_ok(dtype) || B < 1 || B > SV_MAX_BATCH || k_max < 1 || k_max > SV_MAX_K ||
      !shape_ok(V, V, V))
    return 0;
  return sv::carve(verify_dims(B, k_max, V), nullptr, nullptr);
}

size_t sv_rkl_workspace_size(int64_t n_rows, int64_t V, int32_t dtype) {
  if (!dtype_ok(dtype) || n_rows < 1 || n_rows >= (int64_t(1) << 31) || !shape_ok(V, V, V))
    return 0;
  return sv::carve(rkl_dims(n_rows, V), nullptr, nullptr);
}

sv_status sv_verify_block(int32_t dtype, int32_t B, int32_t k_max, int64_t V, int64_t ld_target,
                          int64_t ld_draft, int64_t n_draft_rows, const void* target_logits,
                          const void* draft_logits, const int32_t* k, const int32_t* draft_tokens,
                          const float* uniforms, const float* temperature, float delta,
                          int32_t* accept_len, int32_t* out_tokens, float* rkl_out,
                          float* p_at_draft, float* q_at_draft, int32_t* device_status,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return SV_ERR_DTYPE;
  if (B < 1 || B > SV_MAX_BATCH || k_max < 1 || k_max > SV_MAX_K || !shape_ok(V, ld_target, ld_draft))
    return SV_ERR_SHAPE;
  if (n_draft_rows < B || n_draft_rows > static_cast<int64_t>(B) * k_max) return SV_ERR_SHAPE;
  Dims dm = verify_dims(B, k_max, V);
  if (!target_logits || !draft_logits || !k || !draft_tokens || !uniforms || !accept_len ||
      !out_tokens || !device_status)
    return SV_ERR_NULL;
  if (rkl_out && !(std::isfinite(delta) && delta > 0.0f)) return SV_ERR_VALUE;
  if (!fit_workspace(workspace, workspace_bytes, dm)) return SV_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  Workspace ws{};
  sv::carve(dm, &ws, static_cast<char*>(workspace));
  const int64_t n_d = n_draft_rows, n_t = n_draft_rows + B;
  const bool vec = vec_ok(dtype, ld_target, target_logits) && vec_ok(dtype, ld_draft, draft_logits);
  const int64_t n_slices = dm.n_slices, n_chunks = dm.n_chunks;

  const bool inline_plan = B <= sv::kInlinePlanMaxB;
  if (!inline_plan) {
    sv::PlanArgs pa{};
    pa.B = B;
    pa.k_max = k_max;
    pa.n_d = n_d;
    pa.k = k;
    pa.ws = ws;
    pa.device_status = device_status;
    if (timed(K_PLAN, st, [&] { return sv::launch_plan(pa, st); }) != hipSuccess) return SV_ERR_HIP;
  }

  sv::RowPairArgs ra{};
  ra.target = target_logits;
  ra.draft = draft_logits;
  ra.ld_t = ld_target;
  ra.ld_d = ld_draft;
  ra.V = static_cast<int32_t>(V);
  ra.n_slices = n_slices;
  ra.n_units = n_t;
  ra.B = B;
  ra.k_max = k_max;
  ra.n_d = n_d;
  ra.k = k;
  ra.tokens = draft_tokens;
  ra.uniforms = uniforms;
  ra.temperature = temperature;
  ra.desc = inline_plan ? nullptr : ws.desc;
  ra.glob = ws.glob;
  ra.off_t = ws.off_t;
  ra.rkl_only = false;
  ra.delta = delta;
  ra.rkl_out = rkl_out;
  ra.p_at = p_at_draft;
  ra.q_at = q_at_draft;
  ra.device_status = device_status;
  ra.rowout = ws.rowout;
  ra.kmax1 = k_max + 1;
  ra.arrive = ws.arrive;
  if (rkl_out) ra.fix = ws.fix;  // heavy lanes of the reverse-KL rows are summed by the draw launch
  if (run_rowpair(dtype, vec, ra, ws, dm.rec_slots, st, K_ROWPAIR) != hipSuccess) return SV_ERR_HIP;

  sv::SampleArgs sa{};
  sa.target = target_logits;
  sa.draft = draft_logits;
  sa.ld_t = ld_target;
  sa.ld_d = ld_draft;
  sa.V = static_cast<int32_t>(V);
  sa.n_chunks = n_chunks;
  sa.B = B;
  sa.n_t = n_t;
  sa.glob = ws.glob;
  sa.off_t = ws.off_t;
  sa.k = k;
  sa.temperature = temperature;
  sa.tokens = draft_tokens;
  sa.uniforms = uniforms;
  sa.rowout = ws.rowout;
  sa.kmax1 = k_max + 1;
  sa.chunk_mass = ws.chunk_mass;
  sa.arrive = ws.arrive;
  sa.mass_blocks = static_cast<int32_t>(sv::mass_blocks_for(n_chunks));
  sa.accept_len = accept_len;
  sa.out_tokens = out_tokens;
  sa.p_at = p_at_draft;
  sa.q_at = q_at_draft;
  sa.device_status = device_status;
  sa.rkl_out = rkl_out;
  sa.fix = ws.fix;
  sa.n_slices = n_slices;
  sa.fix_rows = rkl_out ? n_d : 0;
  if (timed(K_DRAW, st, [&] { return sv::launch_draw(dtype, vec, sa, st); }) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}


sv_status sv_opd_loss(int32_t dtype, int32_t B, int64_t n_rows, int64_t n_target_rows, int64_t V,
                      int64_t ld_target, int64_t ld_draft, const void* target_logits,
                      const void* draft_logits, const int32_t* p_row_index, const int32_t* k,
                      float delta, float alpha, float* rkl_out, float* hard_ce_out,
                      int32_t* top1_out, float* opd_out, int32_t* device_status, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!hard_ce_out) return SV_ERR_NULL;
  if (opd_out && (!k || B < 1 || B > SV_MAX_BATCH)) return k ? SV_ERR_SHAPE : SV_ERR_NULL;
  if (!(std::isfinite(alpha) && alpha >= 0.0f && alpha <= 1.0f)) return SV_ERR_VALUE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Workspace ws{};
  const sv_status s = rkl_rows(dtype, n_rows, n_target_rows, V, ld_target, ld_draft, target_logits,
                               draft_logits, p_row_index, delta, rkl_out, hard_ce_out, top1_out,
                               device_status, workspace, workspace_bytes, st, K_OPD_ROWPAIR,
                               K_OPD_STATUS, opd_out ? &ws : nullptr);
  if (s != SV_OK || !opd_out) return s;
  if (timed(K_OPD_REDUCE, st, [&] {
        return sv::launch_opd_reduce(k, B, n_rows, rkl_out, hard_ce_out, alpha, ws.row_flags,
                                     opd_out, nullptr, device_status, st);
      }) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

size_t sv_opd_grad_workspace_size(int64_t n_rows, int64_t V, int32_t dtype) {
  if (!dtype_ok(dtype) || n_rows < 1 || n_rows >= (int64_t(1) << 31) || !shape_ok(V, V, V)) return 0;
  return sv::carve(rkl_dims(n_rows, V, true), nullptr, nullptr);
}

sv_status sv_opd_loss_grad(int32_t dtype, int32_t B, int64_t n_rows, int64_t n_target_rows,
                           int64_t V, int64_t ld_target, int64_t ld_draft,
                           const void* target_logits, const void* draft_logits,
                           const int32_t* p_row_index, const int32_t* k, float delta, float alpha,
                           float* rkl_out, float* hard_ce_out, int32_t* top1_out, float* opd_out,
                           int32_t grad_dtype, int64_t ld_grad, void* grad_out,
                           int32_t* device_status, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (!hard_ce_out || !k || !grad_out) return SV_ERR_NULL;
  if (B < 1 || B > SV_MAX_BATCH || ld_grad < V) return SV_ERR_SHAPE;
  if (!dtype_ok(grad_dtype)) return SV_ERR_DTYPE;
  if (!(std::isfinite(alpha) && alpha >= 0.0f && alpha <= 1.0f)) return SV_ERR_VALUE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Workspace ws{};
  const sv_status s = rkl_rows(dtype, n_rows, n_target_rows, V, ld_target, ld_draft, target_logits,
                               draft_logits, p_row_index, delta, rkl_out, hard_ce_out, top1_out,
                               device_status, workspace, workspace_bytes, st, K_GRAD_ROWPAIR,
                               K_OPD_STATUS, &ws, true);
  if (s != SV_OK) return s;
  if (timed(K_GRAD_REDUCE, st, [&] {
        return sv::launch_opd_reduce(k, B, n_rows, rkl_out, hard_ce_out, alpha, ws.row_flags,
                                     opd_out, ws.coef, device_status, st);
      }) != hipSuccess)
    return SV_ERR_HIP;
  sv::GradArgs ga{};
  ga.target = target_logits;
  ga.draft = draft_logits;
  ga.ld_t = ld_target;
  ga.ld_d = ld_draft;
  ga.ld_g = ld_grad;
  ga.V = static_cast<int32_t>(V);
  ga.n_rows = n_rows;
  ga.n_target_rows = n_target_rows;
  ga.p_row_index = p_row_index;
  ga.delta = delta;
  ga.stats = ws.stats;
  ga.coef = ws.coef;
  ga.grad = grad_out;
  const bool vec = vec_ok(dtype, ld_target, target_logits) &&
                   vec_ok(dtype, ld_draft, draft_logits) && vec_ok(grad_dtype, ld_grad, grad_out);
  if (timed(K_GRAD, st, [&] { return sv::launch_opd_grad(dtype, grad_dtype, vec, ga, st); }) !=
      hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

sv_status sv_verify_block_greedy(int32_t dtype, int32_t B, int32_t k_max, int64_t V,
                                 int64_t ld_target, int64_t n_draft_rows,
                                 const void* target_logits, const int32_t* k,
                                 const int32_t* draft_tokens, int32_t* accept_len,
                                 int32_t* out_tokens, int32_t* device_status, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return SV_ERR_DTYPE;
  if (B < 1 || B > SV_MAX_BATCH || k_max < 1 || k_max > SV_MAX_K || !shape_ok(V, ld_target, V))
    return SV_ERR_SHAPE;
  if (n_draft_rows < B || n_draft_rows > static_cast<int64_t>(B) * k_max) return SV_ERR_SHAPE;
  Dims dm = verify_dims(B, k_max, V);
  if (!target_logits || !k || !draft_tokens || !accept_len || !out_tokens || !device_status)
    return SV_ERR_NULL;
  dm.rec_slots = 0;  // the greedy stream never splits rows
  if (!fit_workspace(workspace, workspace_bytes, dm)) return SV_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  Workspace ws{};
  sv::carve(dm, &ws, static_cast<char*>(workspace));
  const int64_t n_d = n_draft_rows, n_t = n_draft_rows + B;
  const bool vec = vec_ok(dtype, ld_target, target_logits);
  const bool inline_plan = B <= sv::kInlinePlanMaxB;
  if (!inline_plan) {
    sv::PlanArgs pa{};
    pa.B = B;
    pa.k_max = k_max;
    pa.n_d = n_d;
    pa.k = k;
    pa.ws = ws;
    pa.device_status = device_status;
    if (timed(K_GREEDY_PLAN, st, [&] { return sv::launch_plan(pa, st); }) != hipSuccess)
      return SV_ERR_HIP;
  }
  sv::RowPairArgs ra{};
  ra.target = target_logits;
  ra.ld_t = ld_target;
  ra.V = static_cast<int32_t>(V);
  ra.n_slices = dm.n_slices;
  ra.n_units = n_t;
  ra.B = B;
  ra.k_max = k_max;
  ra.n_d = n_d;
  ra.k = k;
  ra.tokens = draft_tokens;
  ra.desc = inline_plan ? nullptr : ws.desc;
  ra.glob = ws.glob;
  ra.off_t = ws.off_t;
  ra.device_status = device_status;
  ra.rowout = ws.rowout;
  ra.kmax1 = k_max + 1;
  if (timed(K_GREEDY, st, [&] { return sv::launch_greedy(dtype, vec, ra, st); }) != hipSuccess)
    return SV_ERR_HIP;

  sv::SampleArgs sa{};
  sa.target = target_logits;
  sa.ld_t = ld_target;
  sa.V = static_cast<int32_t>(V);
  sa.n_chunks = dm.n_chunks;
  sa.B = B;
  sa.n_t = n_t;
  sa.glob = ws.glob;
  sa.off_t = ws.off_t;
  sa.k = k;
  sa.tokens = draft_tokens;
  sa.rowout = ws.rowout;
  sa.kmax1 = k_max + 1;
  sa.chunk_mass = ws.chunk_mass;
  sa.arrive = ws.arrive;
  sa.force_greedy = true;
  sa.mass_blocks = 1;  // greedy: one workgroup per request emits, no masses are drawn
  sa.accept_len = accept_len;
  sa.out_tokens = out_tokens;
  sa.device_status = device_status;
  if (timed(K_GREEDY_PICK, st, [&] { return sv::launch_draw(dtype, vec, sa, st); }) !=
      hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

namespace {
bool head_shape_ok(int32_t B, int32_t k, int32_t H, int32_t H_feat) {
  return B >= 1 && B <= SV_MAX_BATCH && k >= 1 && k <= SV_MAX_K && H >= 32 && H % 32 == 0 &&
         H_feat >= 1 && H_feat <= SV_MAX_HEAD_FEATURES;
}
}  // namespace

size_t sv_length_head_workspace_size(int32_t B, int32_t k, int32_t H, int32_t H_feat) {
  if (!head_shape_ok(B, k, H, H_feat)) return 0;
  return sv::head_workspace_bytes(sv::head_split(B, k, H, H_feat));
}

sv_status sv_length_head(int32_t B, int32_t k, int32_t H, int32_t H_feat, const void* h,
                         int64_t ld_h, const void* W1, int64_t ld_w, const float* b1,
                         const float* w2, float b2, float gamma, float* a_hat, int32_t* k_hat,
                         int32_t* off_t, void* workspace, size_t workspace_bytes, void* stream) {
  if (!head_shape_ok(B, k, H, H_feat) || ld_h < H || ld_w < H || ld_h % 8 != 0 || ld_w % 8 != 0)
    return SV_ERR_SHAPE;
  if (!h || !W1 || !w2 || !a_hat || !k_hat) return SV_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(h) % 16) != 0 || (reinterpret_cast<uintptr_t>(W1) % 16) != 0)
    return SV_ERR_SHAPE;
  if (!(std::isfinite(gamma) && gamma > 0.0f) || !std::isfinite(b2)) return SV_ERR_VALUE;
  const size_t need = sv_length_head_workspace_size(B, k, H, H_feat);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % 256) != 0 || workspace_bytes < need)
    return SV_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  sv::HeadArgs ha = sv::head_split(B, k, H, H_feat);
  ha.h = h;
  ha.ld_h = ld_h;
  ha.W1 = W1;
  ha.ld_w = ld_w;
  ha.b1 = b1;
  ha.w2 = w2;
  ha.b2 = b2;
  ha.gamma = gamma;
  ha.partial = static_cast<float*>(workspace);
  ha.ticket = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + sv::head_ticket_offset(ha));
  ha.a_hat = a_hat;
  ha.k_hat = k_hat;
  ha.off_t = off_t;
  if (timed(K_HEAD_FEAT, st, [&] { return sv::launch_head(ha, st); }) != hipSuccess)
    return SV_ERR_HIP;
  if (timed(K_HEAD_POOL, st, [&] { return sv::launch_head_pool(ha, st); }) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

size_t sv_tree_workspace_size(int32_t B, int64_t n_nodes_total) {
  if (B < 1 || B > SV_MAX_BATCH || n_nodes_total < B ||
      n_nodes_total > static_cast<int64_t>(B) * SV_MAX_TREE_NODES)
    return 0;
  return ((static_cast<size_t>(n_nodes_total + B) * sizeof(int32_t)) + 255) & ~size_t(255);
}

sv_status sv_verify_tree_greedy(int32_t dtype, int32_t B, int32_t max_nodes, int64_t V,
                                int64_t ld_target, int64_t n_nodes_total,
                                const void* target_logits, const int32_t* n_nodes,
                                const int32_t* parent, const int32_t* tree_tokens,
                                int32_t* accept_len, int32_t* out_tokens, int32_t* out_nodes,
                                int32_t* device_status, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (!dtype_ok(dtype)) return SV_ERR_DTYPE;
  if (B < 1 || B > SV_MAX_BATCH || max_nodes < 1 || max_nodes > SV_MAX_TREE_NODES ||
      !shape_ok(V, ld_target, ld_target) || n_nodes_total < B ||
      n_nodes_total > static_cast<int64_t>(B) * max_nodes)
    return SV_ERR_SHAPE;
  if (!target_logits || !n_nodes || !parent || !tree_tokens || !accept_len || !out_tokens ||
      !device_status)
    return SV_ERR_NULL;
  const size_t need = sv_tree_workspace_size(B, n_nodes_total);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % 256) != 0 || workspace_bytes < need)
    return SV_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* arg = static_cast<int32_t*>(workspace);
  sv::ArgmaxArgs am{};
  am.target = target_logits;
  am.ld_t = ld_target;
  am.V = static_cast<int32_t>(V);
  am.n_slices = sv::n_slices_for(V);
  am.n_rows = n_nodes_total + B;
  am.arg = arg;
  am.zero_status = device_status;
  const bool vec = vec_ok(dtype, ld_target, target_logits);
  if (timed(K_TREE_ARGMAX, st, [&] { return sv::launch_row_argmax(dtype, vec, am, st); }) !=
      hipSuccess)
    return SV_ERR_HIP;
  sv::TreeArgs ta{};
  ta.B = B;
  ta.max_nodes = max_nodes;
  ta.V = static_cast<int32_t>(V);
  ta.n_nodes_total = n_nodes_total;
  ta.n_nodes = n_nodes;
  ta.parent = parent;
  ta.tokens = tree_tokens;
  ta.arg = arg;
  ta.accept_len = accept_len;
  ta.out_tokens = out_tokens;
  ta.out_nodes = out_nodes;
  ta.device_status = device_status;
  if (timed(K_TREE_WALK, st, [&] { return sv::launch_tree_walk(ta, st); }) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

sv_status sv_branch_lookup(int32_t B, int32_t k_max, int32_t n_branch, int64_t n_tokens,
                           const int32_t* k, const int32_t* accept_len, const int32_t* out_tokens,
                           const int32_t* branch_pos, const int32_t* branch_tok, int32_t* hit,
                           void* stream) {
  if (B < 1 || B > SV_MAX_BATCH || k_max < 1 || k_max > SV_MAX_K || n_branch < 1 ||
      n_branch > SV_MAX_BRANCHES || n_tokens < 1)
    return SV_ERR_SHAPE;
  if (!k || !accept_len || !out_tokens || !branch_pos || !branch_tok || !hit) return SV_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  sv::BranchArgs a{};
  a.B = B;
  a.k_max = k_max;
  a.n_branch = n_branch;
  a.n_tokens = n_tokens;
  a.k = k;
  a.accept_len = accept_len;
  a.out_tokens = out_tokens;
  a.branch_pos = branch_pos;
  a.branch_tok = branch_tok;
  a.hit = hit;
  if (timed(K_BRANCH, st, [&] { return sv::launch_branch(a, st); }) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

sv_status sv_length_loss(int32_t B, const float* a_hat, const int32_t* accept_len,
                         const int32_t* k_hat, float* loss, float* dloss, void* stream) {
  if (B < 1 || B > SV_MAX_BATCH) return SV_ERR_SHAPE;
  if (!a_hat || !accept_len || !k_hat || !loss) return SV_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (timed(K_LEN_LOSS, st, [&] {
        return sv::launch_len_loss(B, a_hat, accept_len, k_hat, loss, dloss, st);
      }) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

sv_status sv_clipped_rkl(int32_t dtype, int64_t n_rows, int64_t n_target_rows, int64_t V,
                         int64_t ld_target, int64_t ld_draft, const void* target_logits,
                         const void* draft_logits, const int32_t* p_row_index, float delta,
                         float* rkl_out, int32_t* device_status, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return rkl_rows(dtype, n_rows, n_target_rows, V, ld_target, ld_draft, target_logits,
                  draft_logits, p_row_index, delta, rkl_out, nullptr, nullptr, device_status,
                  workspace, workspace_bytes, static_cast<hipStream_t>(stream), K_RKL_ROWPAIR,
                  K_RKL_STATUS, nullptr);
}

sv_status sv_read_probe(const void* data, int64_t bytes, uint32_t* out, void* stream) {
  if (!data || !out) return SV_ERR_NULL;
  if (bytes <= 0 || bytes % 16 != 0) return SV_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(data) % 16 != 0) return SV_ERR_VALUE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return timed(K_READ_PROBE, st, [&] { return sv::launch_read_probe(data, bytes / 16, out, st); }) ==
                 hipSuccess
             ? SV_OK
             : SV_ERR_HIP;
}

sv_status sv_profile_enable(int32_t on) {
  prof().on.store(on != 0, std::memory_order_relaxed);
  return SV_OK;
}

sv_status sv_profile_reset(void) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> lock(p.mu);
  const hipError_t e = drain_pending();
  for (int i = 0; i < kNumKernels; ++i) {
    p.launches[i] = 0;
    p.total_ms[i] = 0.0;
  }
  return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

int32_t sv_profile_count(void) { return kNumKernels; }

sv_status sv_profile_get(int32_t index, char* name, size_t name_len, int64_t* launches,
                         double* total_ms) {
  if (index < 0 || index >= kNumKernels) return SV_ERR_SHAPE;
  Profiler& p = prof();
  std::lock_guard<std::mutex> lock(p.mu);
  const hipError_t e = drain_pending();
  if (name && name_len) {
    std::strncpy(name, kKernelNames[index], name_len - 1);
    name[name_len - 1] = '\0';
  }
  if (launches) *launches = p.launches[index];
  if (total_ms) *total_ms = p.total_ms[index];
  return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // extern "C"
