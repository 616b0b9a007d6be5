/*
 * libspecverify -- batched verification of a one-pass diffusion draft block,
 * with the fused entry-wise clipped reverse-KL, for AMD Instinct MI355X (gfx950).
 *
 * Plain C ABI: device pointers, sizes, one stream handle.  No C++ or framework
 * types cross this boundary and no exception escapes it.
 *
 * What is computed (cited by page title and section):
 *   - "AdaFlash: Adaptive Speculative Decoding via On-Policy Distilled Diffusion
 *     Drafters" (arXiv 2607.19223), Section 2.1: each draft token x_i is accepted
 *     with probability min(1, p(x_i)/q(x_i)); tokens up to the first rejection are
 *     kept; at the rejection a corrected token is drawn from the residual.
 *   - AdaFlash reading notes (zhongzhuzhou.org), basic recipe step 4: the residual
 *     is max(0, p - q), normalised.
 *   - DFlash notes (zhangshuibai.github.io), Section 3.1 step 6: when every draft
 *     is accepted the target emits one bonus token, so a round emits a_b + 1
 *     tokens; Section 5.2: the drafter's per-position marginals play q.
 *   - AdaFlash paper, Section 3.2: per-request verification length k_b in
 *     [1, k_max]; Section 3.3: the batch is packed to total length sum_b k_b.
 *   - AdaFlash paper, Section 3.1 (equation of the clipped reverse-KL) and
 *     Appendix B.1 (reverse-KL temperature 1):
 *         R_i = sum_y min(delta, q_i(y) log(q_i(y) / p_i(y))).
 *
 * Conventions where the pages leave a choice open:
 *   - accept iff u < min(1, p_T(x)/q_T(x)) (equality rejects);
 *   - uniforms slot k_b of a request drives its single final-token draw;
 *   - the final token is the smallest id y with prefix mass(0..y) > u * Z,
 *     Z the total mass, ids in ascending order (zero-mass ids are never drawn);
 *   - a residual of zero total mass (possible only through rounding) falls
 *     back to p_T of the same row;
 *   - temperature T_b = 0 is greedy: accept iff x_i == argmax of target row i,
 *     final token = argmax of the target row at a_b; ties go to the lowest id;
 *   - the clipped reverse-KL always uses temperature 1 and is reported for every
 *     draft row, accepted or not; min applies per entry, so R_i may be negative.
 *
 * Packed layout (request b has k_b drafts; off_t[b] = sum_{c<b} (k_c + 1)):
 *   target row off_t[b] + i, i = 0..k_b: row i < k_b scores draft i, row k_b is the
 *                                          bonus row;
 *   draft  row off_t[b] - b + i, i < k_b;
 *   draft_tokens and the reported per-draft outputs follow the draft rows;
 *   uniforms and out_tokens follow the target rows.
 * Logits are row-major with leading dimensions ld_target / ld_draft (elements,
 * >= V); only columns [0, V) are read.
 *
 * Streams and memory: every pointer argument except where stated is a device
 * pointer owned by the caller.  Calls are asynchronous on `stream` (a
 * hipStream_t; NULL = the null stream) and never synchronise the device.  The
 * library allocates nothing per call; scratch lives in the caller's workspace,
 * which a call may overwrite and which must not be shared by calls that can run
 * concurrently.  Results are bitwise deterministic for identical inputs.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sv_status;

/* Host-side status codes, returned synchronously before anything is enqueued. */
enum {
  SV_OK = 0,
  SV_ERR_NULL = 1,      /* a required pointer is NULL                                  */
  SV_ERR_SHAPE = 2,     /* B, V, ld, k_max or a row count out of range                 */
  SV_ERR_DTYPE = 3,     /* dtype is not SV_BF16 / SV_F32                               */
  SV_ERR_VALUE = 4,     /* delta not finite or <= 0 while the rKL is requested         */
  SV_ERR_WORKSPACE = 5, /* workspace NULL, misaligned (256 B) or smaller than required */
  SV_ERR_HIP = 6,       /* a HIP runtime call or kernel launch failed                  */
  SV_ERR_SCRATCH = 7    /* sv_verify_block_noalloc: the call needs more scratch than the
                           library's fixed buffer (SV_NOALLOC_SCRATCH_BYTES) holds       */
};

/* Logit element types. */
enum { SV_BF16 = 0, SV_F32 = 1 };

/* Bits written to *device_status by a call (0 = every request was valid). */
enum {
  SV_DEV_BAD_LENGTH = 1,       /* some k_b outside [1, k_max]: the whole call is void     */
  SV_DEV_ROWS_MISMATCH = 2,    /* sum_b k_b != n_draft_rows: the whole call is void       */
  SV_DEV_BAD_TOKEN = 4,        /* a draft token outside [0, V)                            */
  SV_DEV_BAD_TEMPERATURE = 8,  /* a T_b negative, not finite, or in (0, 2^-10)           */
  SV_DEV_BAD_UNIFORM = 16,     /* a uniform outside [0, 1) or NaN                         */
  SV_DEV_BAD_PARENT = 32       /* a tree node whose parent is not an earlier node or -1   */
};

/* Limits checked on the host. */
#define SV_MAX_K 64          /* k_max <= 64                                  */
#define SV_MAX_BATCH 65536   /* B <= 65536                                   */
#define SV_MAX_VOCAB (1 << 19) /* 524288 */
#define SV_MAX_HEAD_FEATURES 4096 /* H' of the length head */
#define SV_MAX_BRANCHES 4096 /* prepared successor blocks per request */
#define SV_MAX_TREE_NODES 1024 /* draft-tree nodes per request */

/* Bytes of workspace sv_verify_block needs for B requests of at most k_max drafts
 * over a vocabulary of V entries of the given dtype; 0 if the shape is invalid.  For calls
 * of at most 128 rows this includes lane records that let several workgroups stream each
 * row; a workspace without room for them but large enough otherwise (one sized for a larger
 * batch, say) is accepted, and the call then streams each row in one workgroup. */
size_t sv_workspace_size(int32_t B, int32_t k_max, int64_t V, int32_t dtype);

/*
 * sv_verify_block: verify B packed draft blocks.
 *
 *   dtype           SV_BF16 or SV_F32, the element type of both logit arrays.
 *   B, k_max        requests in the batch; upper bound on every k_b (1..SV_MAX_K).
 *   V               vocabulary size (columns read per row).
 *   ld_target/ld_draft  row strides in elements (>= V).
 *   n_draft_rows    sum_b k_b, as packed by the caller (the host knows it from the
 *                   shapes it allocated; the device checks it against k).
 *   target_logits   [n_draft_rows + B, ld_target]
 *   draft_logits    [n_draft_rows, ld_draft]
 *   k               int32[B], k_b in [1, k_max]
 *   draft_tokens    int32[n_draft_rows], ids in [0, V)
 *   uniforms        float[n_draft_rows + B] in [0, 1): slot i < k_b of a request is the
 *                   acceptance uniform of draft i, slot k_b drives the final token.
 *   temperature     float[B], T_b = 0 (greedy) or 2^-10 <= T_b < inf, or NULL for all 1.0.
 *                   Positive temperatures below 2^-10 are flagged SV_DEV_BAD_TEMPERATURE:
 *                   the fp32 exponent offsets are exact only while |l| log2(e) / T_b < 2^24.
 *   delta           clip threshold of the reverse-KL (finite, > 0 when rkl_out != NULL).
 * Outputs (device):
 *   accept_len      int32[B]: a_b, the accepted drafts (0..k_b); -1 for an invalid request.
 *   out_tokens      int32[n_draft_rows + B], per target row: the a_b accepted drafts, then
 *                   the final token (residual resample or bonus), then -1.
 *   rkl_out         float[n_draft_rows] clipped reverse-KL per draft row, or NULL to skip.
 *   p_at_draft      float[n_draft_rows] p_T(x_i) (temperature-1 value for greedy
 *                   requests), or NULL.
 *   q_at_draft      float[n_draft_rows] q_T(x_i), likewise, or NULL.
 *   device_status   int32[1]: OR of SV_DEV_* bits found by this call (required).
 *   workspace       device scratch of >= sv_workspace_size(B, k_max, V, dtype) bytes,
 *                   256-byte aligned.
 *   stream          hipStream_t to enqueue on (NULL = null stream).
 *
 * Errors: host-checkable problems return SV_ERR_* and enqueue nothing.  Data-dependent
 * problems never stop the device: an invalid request gets accept_len = -1, out_tokens
 * = -1 and NaN probabilities (its rKL values are still computed); a void call (bad k or
 * row count) writes -1 / NaN everywhere.  A failed launch returns SV_ERR_HIP.
 */
sv_status sv_verify_block(int32_t dtype, int32_t B, int32_t k_max, int64_t V, int64_t ld_target,
                          int64_t ld_draft, int64_t n_draft_rows, const void* target_logits,
                          const void* draft_logits, const int32_t* k, const int32_t* draft_tokens,
                          const float* uniforms, const float* temperature, float delta,
                          int32_t* accept_len, int32_t* out_tokens, float* rkl_out,
                          float* p_at_draft, float* q_at_draft, int32_t* device_status,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * sv_verify_block_noalloc: sv_verify_block for callers that cannot allocate device memory
 * around the call (code under stream capture, tight serving loops, harnesses that forbid
 * allocation).  The same arguments and outputs as sv_verify_block, without the workspace: the
 * call uses the library's own scratch, a fixed device array of SV_NOALLOC_SCRATCH_BYTES (16 MiB)
 * that each GPU the library runs on holds until the process ends.  Nothing is allocated per
 * call (the array's address on a device is looked up once, on the first call there).
 *
 * Limit: calls whose workspace (sv_workspace_size) exceeds the buffer run like a caller
 * workspace sized for a larger batch (each row streamed by one workgroup); calls that need
 * more than the buffer even then return SV_ERR_SCRATCH and enqueue nothing.  At V = 151936
 * and k_max = 15 that is beyond about 12000 requests (B = 128 needs 0.2 MiB).
 * Concurrency: every call on one GPU shares that GPU's buffer, and each call overwrites it;
 * calls that overlap on one GPU (several streams or host threads) race and must be serialised
 * by the caller.  Errors otherwise as sv_verify_block.
 */
#define SV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
sv_status sv_verify_block_noalloc(int32_t dtype, int32_t B, int32_t k_max, int64_t V,
                                  int64_t ld_target, int64_t ld_draft, int64_t n_draft_rows,
                                  const void* target_logits, const void* draft_logits,
                                  const int32_t* k, const int32_t* draft_tokens,
                                  const float* uniforms, const float* temperature, float delta,
                                  int32_t* accept_len, int32_t* out_tokens, float* rkl_out,
                                  float* p_at_draft, float* q_at_draft, int32_t* device_status,
                                  void* stream);

/*
 * sv_verify_block_greedy: sv_verify_block for a batch whose every request decodes greedily
 * (T_b = 0; the AdaFlash paper's default decoding, Appendix B.1).  A draft is accepted iff it
 * equals the argmax of its target row, and the final token is the argmax of target row a_b
 * (DFlash notes, Section 5.2, worked example #4); ties go to the lowest id.  Only the target
 * rows are read, with no exponentials, so no draft logits, uniforms, temperatures or
 * probability outputs appear.
 *
 *   dtype, B, k_max, V, ld_target, n_draft_rows, target_logits, k, draft_tokens   as
 *                   sv_verify_block.
 * Outputs: accept_len int32[B], out_tokens int32[n_draft_rows + B], device_status int32[1],
 *   with sv_verify_block's meaning (SV_DEV_BAD_TOKEN for a token outside [0, V): that
 *   request gets -1; bad lengths or a row-count mismatch void the call).
 * Workspace: sv_workspace_size(B, k_max, V, dtype) bytes, 256-byte aligned.
 */
sv_status sv_verify_block_greedy(int32_t dtype, int32_t B, int32_t k_max, int64_t V,
                                 int64_t ld_target, int64_t n_draft_rows,
                                 const void* target_logits, const int32_t* k,
                                 const int32_t* draft_tokens, int32_t* accept_len,
                                 int32_t* out_tokens, int32_t* device_status, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Bytes of workspace sv_clipped_rkl needs for n_rows row pairs; 0 if invalid.  As with
 * sv_workspace_size, the lane records of split rows (n_rows <= 128) are optional. */
size_t sv_rkl_workspace_size(int64_t n_rows, int64_t V, int32_t dtype);

/*
 * sv_clipped_rkl: the clipped reverse-KL alone (AdaFlash paper, Section 3.1), for an
 * on-policy-distillation reader of the same logits.
 *
 *   n_rows          draft rows to score.
 *   target_logits   [n_target_rows, ld_target]; draft_logits [n_rows, ld_draft].
 *   p_row_index     int32[n_rows]: target row paired with draft row r, or NULL for r.
 *                   Entries must lie in [0, n_target_rows).
 *   n_target_rows   rows in target_logits (bounds p_row_index).
 *   delta           finite, > 0.
 *   rkl_out         float[n_rows].
 *   device_status   int32[1]: SV_DEV_ROWS_MISMATCH if some p_row_index entry is out of
 *                   range (that row's output is NaN).
 */
sv_status sv_clipped_rkl(int32_t dtype, int64_t n_rows, int64_t n_target_rows, int64_t V,
                         int64_t ld_target, int64_t ld_draft, const void* target_logits,
                         const void* draft_logits, const int32_t* p_row_index, float delta,
                         float* rkl_out, int32_t* device_status, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * sv_opd_loss: the on-policy-distillation loss of the AdaFlash paper, Section 3.1 (mixture
 * OPD loss with reverse-KL, entry-wise divergence clipping; Appendix B.1: temperature 1),
 * read from the same logits in one pass over each row pair:
 *     x*_r   = first argmax of target row p_row_index[r]   (the target's top-1 token)
 *     hard_r = -ln q_r(x*_r)                                (hard-label cross-entropy)
 *     R_r    = sum_y min(delta, q_r(y) ln(q_r(y) / p(y)))   (as sv_clipped_rkl)
 *     opd_b  = alpha mean_r hard_r + (1 - alpha) mean_r R_r over request b's k_b rows.
 *
 *   B, k            requests and their draft-row counts (int32[B], device, k_b in [1, 64]);
 *                   the draft rows are packed request by request, sum_b k_b = n_rows.  Needed
 *                   only with opd_out (else pass NULL and any B).
 *   p_row_index, n_target_rows, V, ld_*, logits, delta   as sv_clipped_rkl.
 *   alpha           mixing coefficient in [0, 1].
 * Outputs (device): rkl_out float[n_rows] and hard_ce_out float[n_rows] (both required),
 *   top1_out int32[n_rows] (x*, or NULL), opd_out float[B] (or NULL), device_status int32[1]:
 *   SV_DEV_ROWS_MISMATCH for a p_row_index entry out of range (that row's outputs are NaN) or
 *   sum_b k_b != n_rows, SV_DEV_BAD_LENGTH for a k_b outside [1, 64] (opd_out is then NaN).
 * Workspace: sv_rkl_workspace_size(n_rows, V, dtype) bytes, 256-byte aligned.
 * Errors as sv_clipped_rkl; alpha outside [0, 1] is SV_ERR_VALUE.
 */
sv_status sv_opd_loss(int32_t dtype, int32_t B, int64_t n_rows, int64_t n_target_rows, int64_t V,
                      int64_t ld_target, int64_t ld_draft, const void* target_logits,
                      const void* draft_logits, const int32_t* p_row_index, const int32_t* k,
                      float delta, float alpha, float* rkl_out, float* hard_ce_out,
                      int32_t* top1_out, float* opd_out, int32_t* device_status, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Bytes of workspace sv_opd_loss_grad needs for n_rows row pairs; 0 if invalid. */
size_t sv_opd_grad_workspace_size(int64_t n_rows, int64_t V, int32_t dtype);

/*
 * sv_opd_loss_grad: everything sv_opd_loss computes, plus the gradient of each request's
 * l_OPD with respect to its drafter logits, the signal on-policy distillation trains the
 * drafter with (AdaFlash paper, Section 3.1: the clip exists to bound the gradients of a few
 * high-divergence entries).  For draft row r of request b, column z:
 *     grad[r, z] = alpha/k_b (q_z - 1[z = x*_r]) + (1 - alpha)/k_b q_z (g_z - sum_y q_y g_y),
 *     g_y = 1[t_y < delta] (ln q_y - ln p_y + 1),  t_y = q_y ln(q_y / p_y),
 * temperature 1; where an entry sits exactly on the clip (t = delta) the clipped side's
 * derivative, 0, is taken.  Two passes over each row pair: the forward (sv_opd_loss's kernel,
 * which also keeps per-row statistics in the workspace) and the gradient pass, which reads the
 * pair again and writes the gradient row once.
 *
 *   k               int32[B] (required): draft rows per request, packed, sum = n_rows.
 *   grad_dtype      SV_BF16 (rounded to nearest even) or SV_F32.
 *   ld_grad         row stride of grad_out in elements (>= V); columns [V, ld_grad) untouched.
 *   grad_out        device [n_rows, ld_grad] of grad_dtype; must not overlap any input.
 *   other arguments as sv_opd_loss (opd_out and top1_out may be NULL).
 * A request set with bad lengths (SV_DEV_BAD_LENGTH / SV_DEV_ROWS_MISMATCH from k) gets NaN
 * gradients everywhere; a row whose p_row_index entry is out of range gets a NaN row.
 * Workspace: sv_opd_grad_workspace_size(n_rows, V, dtype) bytes, 256-byte aligned.
 */
sv_status sv_opd_loss_grad(int32_t dtype, int32_t B, int64_t n_rows, int64_t n_target_rows,
                           int64_t V, int64_t ld_target, int64_t ld_draft,
                           const void* target_logits, const void* draft_logits,
                           const int32_t* p_row_index, const int32_t* k, float delta, float alpha,
                           float* rkl_out, float* hard_ce_out, int32_t* top1_out, float* opd_out,
                           int32_t grad_dtype, int64_t ld_grad, void* grad_out,
                           int32_t* device_status, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Bytes of workspace sv_length_head needs for this shape (the projection's split-K partial
 * sums); 0 if the shape is invalid. */
size_t sv_length_head_workspace_size(int32_t B, int32_t k, int32_t H, int32_t H_feat);

/*
 * sv_length_head: the adaptive length head of the AdaFlash paper, Section 3.2, and the packed
 * layout of the verification batch it implies (Section 3.3):
 *     a_hat_b = sigmoid(w2 . (1/k) sum_i SiLU(W1 h_{b,i} + b1) + b2)
 *     k_hat_b = clamp(floor(a_hat_b gamma k), 1, k)          (gamma scales a_hat before the floor)
 *     off_t[b] = sum_{c<b} (k_hat_c + 1), off_t[B] = sum_b (k_hat_b + 1)
 * The projection runs on the matrix cores in bf16 with fp32 accumulation.
 *
 *   B, k            requests; positions of each request's draft block (1..SV_MAX_K).
 *   H, H_feat       hidden size (a multiple of 32), features H' (1..SV_MAX_HEAD_FEATURES).
 *   h               bf16 [B * k, ld_h]: request b's positions are rows b k .. b k + k - 1.
 *   W1              bf16 [H_feat, ld_w] (row n projects onto feature n); b1 float[H_feat] or
 *                   NULL (no bias); w2 float[H_feat]; b2, gamma (> 0) scalars.
 *   ld_h, ld_w      row strides in elements, >= H and multiples of 8; h and W1 16-byte aligned.
 * Outputs (device): a_hat float[B], k_hat int32[B], off_t int32[B + 1] (or NULL).
 * Workspace: sv_length_head_workspace_size(B, k, H, H_feat) bytes, 256-byte aligned.
 */
sv_status sv_length_head(int32_t B, int32_t k, int32_t H, int32_t H_feat, const void* h,
                         int64_t ld_h, const void* W1, int64_t ld_w, const float* b1,
                         const float* w2, float b2, float gamma, float* a_hat, int32_t* k_hat,
                         int32_t* off_t, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sv_length_loss: the length head's online loss (AdaFlash paper, Section 3.2, "Online Update"):
 * l_b = (a_hat_b - a*_b)^2 with a*_b = accept_len_b / k_hat_b, the fraction of the verified
 * drafts that were accepted, and dloss_b = 2 (a_hat_b - a*_b) (or NULL).  A request whose
 * accept_len is -1 (invalid) or outside [0, k_hat_b] gets NaN.  All pointers are device [B].
 */
sv_status sv_length_loss(int32_t B, const float* a_hat, const int32_t* accept_len,
                         const int32_t* k_hat, float* loss, float* dloss, void* stream);

/*
 * sv_branch_lookup: which prepared successor block each request can reuse after verification
 * (review page "D3D: Decoupled Diffusion Drafting for Asynchronous Speculative Decoding",
 * Methodology, inference paragraph: while the target verifies, a drafter pass prepares blocks
 * for selected rejection positions and the full-acceptance case; a verified prefix that
 * matches a prepared branch is a cache hit and reuses it).
 * A branch is keyed by the verification outcome that fixes the next prefix: the accept length
 * (0..k_b; k_b = every draft accepted) and the token emitted after the accepted drafts (the
 * residual draw, the greedy replacement or the bonus token); a key token of -1 matches any.
 * hit[b] is the first branch j, in list order, with branch_pos[b, j] == accept_len[b] and
 * branch_tok[b, j] in {that token, -1}; -1 for a miss.
 *
 *   B, k_max        requests; upper bound on every k_b (1..SV_MAX_K).
 *   n_branch        keys per request (1..SV_MAX_BRANCHES), row-major [B, n_branch] arrays.
 *   n_tokens        length of out_tokens, sum_b (k_b + 1).
 *   k, accept_len   int32 [B]: the lengths and accept lengths of the verification call.
 *   out_tokens      int32 [n_tokens]: its packed output (request b at rows
 *                   sum_{c<b} (k_c + 1) .. + k_b).
 *   branch_pos, branch_tok   int32 [B, n_branch]: the prepared keys.
 *   hit             int32 [B] (out).
 * All pointers are device memory owned by the caller; nothing is allocated.  A request whose
 * k_b or accept length is out of range (e.g. -1 from an invalid verification), or whose row
 * falls past n_tokens, gets -1.  Shape and NULL errors return synchronously; otherwise the work
 * is enqueued on `stream`.
 */
sv_status sv_branch_lookup(int32_t B, int32_t k_max, int32_t n_branch, int64_t n_tokens,
                           const int32_t* k, const int32_t* accept_len, const int32_t* out_tokens,
                           const int32_t* branch_pos, const int32_t* branch_tok, int32_t* hit,
                           void* stream);

/* Bytes of workspace sv_verify_tree_greedy needs; 0 if invalid. */
size_t sv_tree_workspace_size(int32_t B, int64_t n_nodes_total);

/*
 * sv_verify_tree_greedy: greedy (temperature 0) verification of one draft tree per request in
 * one pass over the target rows (DFlash notes, Section 5.1: EAGLE-2/3 propose a dynamic draft
 * tree and verify it with one target pass; Section 5.2, worked example #4: greedy verification
 * accepts a draft iff it equals the target argmax at its prefix; AdaFlash paper, Appendix B.1:
 * greedy decoding is the default).
 * Node j of request b holds a drafted token and its parent: -1 (the root, i.e. the verified
 * anchor) or an earlier node of the same request.  The target scores the root and every node:
 * request b's target rows are root, node 0, ..., node n_b - 1.  From the root, the walk moves to
 * the lowest-index child whose token is the argmax (lowest id on ties) of the current node's
 * row; it stops at a node none of whose children matches and emits that node's argmax after
 * the accepted path.  A chain (parent j - 1) is exactly sv_verify_block_greedy.
 *
 *   dtype           SV_BF16 or SV_F32.
 *   B, max_nodes    requests; upper bound on every n_b (1..SV_MAX_TREE_NODES).
 *   V, ld_target    vocabulary; row stride in elements (>= V).
 *   n_nodes_total   sum_b n_b.
 *   target_logits   [n_nodes_total + B, ld_target]: request b's n_b + 1 rows start at row
 *                   sum_{c<b} (n_c + 1).
 *   n_nodes         int32 [B]: n_b.
 *   parent, tree_tokens   int32 [n_nodes_total]: request b's nodes start at sum_{c<b} n_c.
 * Outputs (device):
 *   accept_len      int32 [B]: accepted path length, -1 for an invalid request or a void call.
 *   out_tokens      int32 [n_nodes_total + B], following the target rows: the path's tokens,
 *                   the final token, then -1.
 *   out_nodes       int32 [n_nodes_total] or NULL, following the nodes: the accepted node
 *                   indices in path order (what a KV cache commits), then -1.
 *   device_status   int32 [1]: SV_DEV_BAD_LENGTH / SV_DEV_ROWS_MISMATCH (n_b out of range, or
 *                   the n_b do not sum to n_nodes_total: the call is void), SV_DEV_BAD_TOKEN,
 *                   SV_DEV_BAD_PARENT (that request is invalid).
 * Workspace: sv_tree_workspace_size(B, n_nodes_total) bytes, 256-byte aligned.  All pointers are
 * device memory owned by the caller; nothing is allocated.  Host-checkable errors return
 * synchronously; the work is enqueued on `stream`.
 */
sv_status sv_verify_tree_greedy(int32_t dtype, int32_t B, int32_t max_nodes, int64_t V,
                                int64_t ld_target, int64_t n_nodes_total,
                                const void* target_logits, const int32_t* n_nodes,
                                const int32_t* parent, const int32_t* tree_tokens,
                                int32_t* accept_len, int32_t* out_tokens, int32_t* out_nodes,
                                int32_t* device_status, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Static text for a status code. */
const char* sv_status_string(sv_status s);

/* Library version string. */
const char* sv_version(void);

/*
 * Kernel timing (diagnostics).  When enabled, every kernel the library launches is
 * bracketed by HIP events on the call's stream; sv_profile_get waits for those events
 * and reports, per kernel name, the number of launches and their summed duration.
 * Process-wide state, not thread-safe; off by default.
 */
sv_status sv_profile_enable(int32_t on);
sv_status sv_profile_reset(void);
int32_t sv_profile_count(void);
sv_status sv_profile_get(int32_t index, char* name, size_t name_len, int64_t* launches,
                         double* total_ms);

/*
 * Read ceiling (diagnostics).  A plain read of `bytes` bytes at `data` (device memory, 16-byte
 * aligned, bytes a positive multiple of 16) on `stream`, folding the words with xor into
 * out[0 .. SV_READ_PROBE_WORDS) (device memory owned by the caller).  It measures what a
 * kernel that only streams bytes in reaches on this part: each of 1024 workgroups reads its
 * contiguous share front to back with 16-byte nontemporal loads, the fastest of the read
 * patterns measured.  The streaming kernels' achieved bandwidth is compared with it as well as
 * with the published HBM peak.  Its duration is reported as "sv_read_probe" by the
 * kernel timing above.  Errors: SV_ERR_NULL, SV_ERR_SHAPE (size), SV_ERR_VALUE (alignment),
 * SV_ERR_HIP; nothing is enqueued on an error.
 */
#define SV_READ_PROBE_WORDS 1024
sv_status sv_read_probe(const void* data, int64_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
