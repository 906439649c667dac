/*
 * treeverify -- draft-tree verification for EAGLE-style speculative decoding on
 * AMD MI355X (gfx950).  C ABI of the library libtreeverify.so.
 *
 * Pages the operations follow (cited by title and section):
 *   [EAGLE]    "EAGLE" study notes on EAGLE-1/2/3 (s1mplewind astro-blog): sections
 *              "1. EAGLE pipeline / Draft Model", "3. Verify", "Well-Calibrated Draft
 *              Model", "Expansion of tree", "Reranking Nodes".
 *   [EAGLE-3]  "What is EAGLE-3 and how does it differ from standard speculative
 *              decoding?" (aivaro.ru Q&A): section 3 (tree attention term) and
 *              section 4, step 4 "Accepting the sequence".
 *   [EAGLE-4]  "Technical analysis of EAGLE-4" (dev48.org translation): section
 *              "EAGLE-4 verification trees and the harness".
 *
 * Conventions shared by every call
 *   - A draft tree holds at most TV_MAX_NODES = 64 nodes, the root included.  Node 0
 *     is the root: the token the target emitted last, queried in this pass but not
 *     yet in the KV cache.  parent[0] == -1 and 0 <= parent[i] < i for i >= 1.
 *   - Per-sequence arrays are [B][n_max] row-major with 1 <= n_max <= 64; entries at
 *     or beyond n_nodes[b] are padding.
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except where a
 *     comment says host.  The library allocates nothing and keeps no state between
 *     calls: workspaces are caller-owned and sized by the *_workspace_size queries.
 *   - Every call validates its host-side arguments first and returns an error
 *     status without touching the device when they are wrong.  Otherwise it only
 *     enqueues kernels on `stream` (asynchronous; no host synchronisation) and
 *     returns TV_OK, or TV_ERR_HIP if the launch itself failed.
 *   - Errors found in device data are reported per sequence in seq_status[b] (when
 *     the pointer is not NULL) with the TV_SEQ_* codes below; the outputs of that
 *     sequence are then zeros / -1 and the other sequences are unaffected.  No
 *     kernel reads or writes outside the buffers described, whatever the data.
 *   - Calls on one stream are ordered; calls that share output or workspace
 *     buffers must not run concurrently on different streams.
 */
#ifndef TREEVERIFY_H
#define TREEVERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TV_ABI_VERSION 3
#define TV_MAX_NODES 64

typedef enum {
  TV_OK = 0,
  TV_ERR_NULL = 1,         /* a required pointer is NULL */
  TV_ERR_SHAPE = 2,        /* a size argument is out of range or inconsistent */
  TV_ERR_DTYPE = 3,        /* unknown tv_dtype */
  TV_ERR_UNSUPPORTED = 4,  /* valid request the library does not implement (e.g. head_dim) */
  TV_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than the size query returns */
  TV_ERR_HIP = 6           /* the HIP runtime reported an error when launching */
} tv_status;

typedef enum { TV_F32 = 0, TV_BF16 = 1 } tv_dtype;

/* per-sequence device status codes written to seq_status[b] */
#define TV_SEQ_OK 0
#define TV_SEQ_BAD_PARENT 1   /* parent[0] != -1, or parent[i] < -1, or parent[i] >= i */
#define TV_SEQ_SECOND_ROOT 2  /* parent[i] == -1 for some i >= 1 */
#define TV_SEQ_BAD_N 3        /* n_nodes (or the kept count m) outside [1, n_max] */
#define TV_SEQ_NONFINITE 4    /* a draft-logit row holds NaN or +-Inf */
#define TV_SEQ_BAD_PREFIX 5   /* prefix_offsets[b] < 0, or offsets[b+1] - offsets[b] outside [0, max_prefix_len] */
#define TV_SEQ_BAD_STATE 6    /* expansion step called out of order for this workspace */

int tv_abi_version(void);
const char* tv_status_string(tv_status s);

/*
 * tree_build -- structure of each draft tree.
 * [EAGLE] "1. EAGLE pipeline / Draft Model": the draft is a tree of depth m holding
 * more than m tokens.  [EAGLE-4] "verification trees": a node may see the prefix,
 * its ancestors and itself; this call turns the parent array into that visibility.
 *
 *   parent     int32 [B][n_max]   in
 *   n_nodes    int32 [B]          in   nodes per tree, root included
 *   prefix_len int32 [B]          in   nullable (then 0)
 *   anc        uint64 [B][n_max]  out  bit j of anc[b][i] set iff node j lies on the
 *                                      path root -> i (root and i included)
 *   depth      int32 [B][n_max]   out  parent steps from i to the root
 *   pos        int32 [B][n_max]   out  nullable; prefix_len + depth, the position the
 *                                      caller encodes node i at
 *   seq_status int32 [B]          out  nullable; TV_SEQ_BAD_PARENT / SECOND_ROOT /
 *                                      BAD_N, the first offending node deciding
 * Padding entries and failed sequences hold anc 0, depth -1, pos -1.
 */
tv_status tree_build(int B, int n_max, const int32_t* parent, const int32_t* n_nodes,
                     const int32_t* prefix_len, uint64_t* anc, int32_t* depth, int32_t* pos,
                     int32_t* seq_status, hipStream_t stream);

/*
 * tree_expand_rerank -- one level of EAGLE-2 dynamic tree construction.
 * [EAGLE] "Well-Calibrated Draft Model": a draft token's confidence is the softmax of
 * the draft logits.  "Expansion of tree": a node's value is the product of the
 * confidences on its root path; the top-k are kept.  "Reranking Nodes": the m nodes
 * of largest value over everything generated form the tree that is verified.
 *
 * Call once per level, step = 1 .. max_steps, in order, with the same workspace
 * (step 1 resets it).  Per sequence, the frontier of a level is a list of k nodes
 * ranked best first; at step 1 it is the root alone.
 *   logits fp32 [B][rows][vocab], rows = 1 at step 1 and k after; row r holds the
 *          draft logits of the frontier node of rank r.
 * For every row: lse = log-sum-exp of the row, computed in float64 from the max and
 * rounded once to float32; the k tokens of largest logit (ties to the lower id)
 * become children with score = fl32(parent score + fl32(logit - lse)), the summed
 * log-confidence (log of the value).  Children are numbered in creation order
 * (row, then top-k rank).  The next frontier is the k best children of this level
 * by (score descending, creation ascending).
 * When final_m > 0 (the last level, or any level whose tree the caller may keep, as
 * with the per-level stop of tree_draft_continue), the whole pool of children so far
 * is reranked: the m - 1 best by the same order are kept with the root (m =
 * m_per_seq[b] if that pointer is given, else final_m), and written root first, then
 * by (depth, creation), with parents remapped to output indices (a later level may
 * still follow on the same workspace):
 *   parent int32 [B][n_max], token int32 [B][n_max] (token[b][0] = root_token[b]),
 *   score fp32 [B][n_max] (root 0), n_nodes int32 [B]; padding -1 / -1 / 0.
 * budget_log float32 [64] (device, nullable; last level only) is a verify budget
 * ([EAGLE-4] "verification trees and the harness": candidates are added while the
 * gain in cumulative probability per unit of measured verification cost stays above
 * a threshold): of the m - 1 kept, best first, candidate j (1-based) stays when its
 * score exceeds budget_log[j], and the first one that does not ends the run (the
 * kept set stays ancestor-closed).  tree_budget_thresholds derives it from a cost
 * table.
 * frontier_token int32 [B][k] (nullable) receives the tokens of the new frontier by
 * rank at every step, for the caller's next draft pass.
 * Limits: 1 <= k <= 16, k <= vocab <= 1048576, max_steps >= 1, k + (max_steps-1)*k*k <= 4096,
 * 1 <= n_max <= 64, 0 <= final_m <= n_max.  root_token may be NULL unless final_m > 0.
 * Device errors: TV_SEQ_NONFINITE (sticky for later steps), TV_SEQ_BAD_N (m), and
 * TV_SEQ_BAD_STATE (step > 1 without the previous step on this workspace).
 */
size_t tree_expand_workspace_size(int B, int k, int max_steps);
tv_status tree_expand_rerank(void* ws, size_t ws_bytes, int B, int k, int max_steps, int step,
                             int vocab, const float* logits, int final_m, const int32_t* m_per_seq,
                             const float* budget_log, const int32_t* root_token, int n_max,
                             int32_t* parent, int32_t* token, float* score, int32_t* n_nodes,
                             int32_t* frontier_token, int32_t* seq_status, hipStream_t stream);

/*
 * tree_draft_continue -- the harness's per-level stop.  [EAGLE-4] "verification trees
 * and the harness": at each draft level the gain in cumulative probability per unit
 * of measured marginal verification cost decides whether the tree is drafted
 * further.  Call after tree_expand_rerank of any level, on the same workspace and
 * with the same k and max_steps.  For sequence b, let c be the best child created by
 * the latest level (its frontier node of rank 0) and p its place in the whole pool
 * ranked best first by (score descending, creation ascending):
 *   more[b] = 1 when p <= m_b - 1 and every place j = 1..p passes the verify budget
 *             (its score > budget_log[j]; no budget when budget_log is NULL), i.e. c
 *             would be kept by the final rerank if drafting stopped now;
 *   more[b] = 0 otherwise, and for a failed sequence or m_b < 2.
 * A deeper node scores no better than its parent and ranks after it, so once more[b]
 * is 0 no later level adds a node to the reranked tree: the caller may stop drafting
 * that sequence (or keep drafting it with the batch) without changing its tree.
 *   m_b = m_per_seq[b] (device, nullable) else m; budget_log float32 [64] device,
 *   nullable, as for tree_expand_rerank; more int32 [B] device out.
 * Errors: TV_ERR_NULL (more), TV_ERR_SHAPE (B, k, max_steps, m outside 0..64, or
 * m < 1 without m_per_seq), TV_ERR_WORKSPACE (ws NULL or smaller than
 * tree_expand_workspace_size(B, k, max_steps)).
 */
tv_status tree_draft_continue(const void* ws, size_t ws_bytes, int B, int k, int max_steps, int m,
                              const int32_t* m_per_seq, const float* budget_log, int32_t* more,
                              hipStream_t stream);

/*
 * tree_candidate_logits -- the draft model's low-rank candidate head.  [EAGLE-4]
 * "EAGLE-4 architecture": a low-rank candidate head first scores the vocabulary in a
 * smaller representation, then computes full logits only for the selected candidates.
 * For every draft row i (h bf16 [rows][d], e.g. one row per frontier node):
 *   z      = A h_i                          A  bf16 [r][d]    (float32 result)
 *   s_v    = Bm[v] . z      for every v     Bm bf16 [vocab][r]
 *   cand_i = the C tokens of largest s (ties to the lower id), best first
 *   logits[i][v] = W[v] . h_i for v in cand_i, s_v elsewhere    W bf16 [vocab][d]
 * Each dot product is a float64 sum of the exact products, rounded once to float32.
 * The rows feed tree_expand_rerank unchanged (their log-sum-exp, top-k and scores).
 * Outputs: logits fp32 [rows][vocab], cand int32 [rows][C].  All device pointers,
 * 16-byte aligned inputs; ws: tree_candidate_workspace_size(rows, r, vocab) bytes (z in
 * float64, rows padded to whole groups of 16, then one uint32 score maximum per row and
 * group of 16 or 32 tokens), no initialisation needed.
 * Limits: d % 8 == 0, r % 32 == 0, 32 <= r <= 512, 1 <= C <= 256, C <= vocab.
 * Errors: TV_ERR_NULL, TV_ERR_SHAPE, TV_ERR_UNSUPPORTED (alignment), TV_ERR_WORKSPACE.
 */
size_t tree_candidate_workspace_size(int rows, int r, int vocab);
tv_status tree_candidate_logits(int rows, int d, int r, int vocab, int C, const void* h,
                                const void* A, const void* Bm, const void* W, float* logits,
                                int32_t* cand, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * tree_cost_lookup -- the verification cost at one (batch, context) from a calibrated
 * table (HOST pointers, no device work).  [EAGLE-4] "verification trees and the
 * harness": a one-time calibration records verification latency against batch size,
 * context length and candidate count, and the harness reads its costs from it.
 *   batch [n_batch], context [n_context], nodes [n_nodes_pts]: ascending grid axes
 *              (batch and context >= 1; node counts in 1..64)
 *   cost_us    [n_batch][n_context][n_nodes_pts]: measured microseconds (> 0, finite)
 *              of one tree_verify_attn call at each grid point
 *   B, L       the caller's batch and context length; n_max <= 64
 *   cost_out   [n_max] out: cost_out[N-1] = the latency with N nodes per tree: log
 *              latency bilinear in (log batch, log context) (exact for power laws),
 *              latency linear in N, the nearest grid value outside the grid, and
 *              never falling as N grows
 * Feeds tree_budget_thresholds.  Errors: TV_ERR_NULL, TV_ERR_SHAPE (empty or
 * non-ascending axes, sizes out of range, a latency that is not positive and finite).
 */
tv_status tree_cost_lookup(const int32_t* batch, int n_batch, const int32_t* context,
                           int n_context, const int32_t* nodes, int n_nodes_pts,
                           const float* cost_us, int B, int L, int n_max, float* cost_out);

/*
 * tree_budget_thresholds -- the per-place bars of the verify budget (HOST pointers,
 * no device work).  [EAGLE-4] "verification trees and the harness": a calibrated cost
 * table (verification latency against batch, context length and candidate count)
 * and a threshold on the gain in cumulative probability per marginal cost.  A
 * candidate's value is exp(score), the product of the confidences on its path.
 *   cost_us    [n_max] host: latency of one tree_verify_attn call with N = 1..n_max
 *              nodes per tree (cost_us[N-1]) at the caller's batch and context length
 *   threshold  accepted tokens per microsecond a candidate must bring
 *   budget_log [64] host out: budget_log[j] = log(threshold * (cost_us[j] -
 *              cost_us[j-1])) for 1 <= j < n_max (candidate j makes the tree j + 1
 *              nodes); -inf where that marginal cost is <= 0 or threshold <= 0, and for
 *              j = 0 and j >= n_max
 */
tv_status tree_budget_thresholds(const float* cost_us, int n_max, float threshold,
                                 float* budget_log);

/*
 * tree_verify_attn -- tree-masked attention of one target layer over all draft nodes.
 * [EAGLE-4] "verification trees": each token attends to the shared prefix, its
 * ancestors and itself; siblings and other branches stay hidden.  [EAGLE] "3. Verify"
 * and [EAGLE-3] section 3: all branches are checked in one target forward pass.
 *
 * For sequence b, query head h, node i < n_nodes[b], with g = h / (Hq / Hkv):
 *   out[b][i][h] = sum_j softmax_j(scale * q . k_j) v_j over the keys
 *   j in { prefix 0 .. L_b-1 of kv head g } U { tree nodes j with bit j of anc[b][i] }
 *   lse[b][i][h] = natural-log log-sum-exp of those scores (nullable output).
 * Layouts (element type per dt; all contiguous, row-major):
 *   q              [B][n_max][Hq][D]
 *   k_tree, v_tree [B][n_max][Hkv][D]   K/V of the tree nodes from this pass
 *   k_prefix, v_prefix [total][Hkv][D]  cached prefix, sequences packed back to back:
 *                  sequence b owns rows prefix_offsets[b] .. prefix_offsets[b+1]-1
 *   prefix_offsets int64 [B+1]          L_b = offsets[b+1] - offsets[b] <= max_prefix_len;
 *                  offsets[b] >= 0 and offsets[b+1] <= the rows of k_prefix / v_prefix
 *                  (the caller's contract: the library cannot see the buffer's size; a
 *                  negative offset or length, or a length past max_prefix_len, fails
 *                  that sequence with TV_SEQ_BAD_PREFIX and nothing is read for it)
 *   n_nodes int32 [B], anc uint64 [B][n_max] (from tree_build)
 *   out            [B][n_max][Hq][D]    rows of padding nodes and failed sequences are 0
 *   lse fp32       [B][n_max][Hq]       nullable; 0 where out is 0
 * scale <= 0 selects 1/sqrt(D).  Supported: dt = TV_BF16 with D in {64, 128}
 * (fp32 accumulation, bf16 output, round to nearest even) and dt = TV_F32 with
 * D % 4 == 0 and D <= 256.  k_prefix / v_prefix may be NULL when max_prefix_len == 0.
 * ws: caller workspace of tree_verify_attn_workspace_size(...) bytes for the partial
 * results of sequences whose prefix spans several key chunks (may be NULL when that
 * size is 0; no initialisation needed).  Calls sharing a workspace must not overlap.
 * Device errors: TV_SEQ_BAD_N, TV_SEQ_BAD_PREFIX in seq_status (nullable).
 */
size_t tree_verify_attn_workspace_size(tv_dtype dt, int B, int n_max, int Hq, int Hkv, int D,
                                       int max_prefix_len);
/*
 * tree_verify_attn_plan -- the launch plan tree_verify_attn takes for these sizes (host
 * only, no device call), for tests and diagnostics.  plan[8] (host, out):
 *   plan[0] waves per workgroup      plan[1] row groups (waves splitting the rows)
 *   plan[2] key splits (waves splitting each stage's keys)
 *   plan[3] 32-row tiles per wave    plan[4] rows (node x query head of one KV head)
 *           per workgroup            plan[5] keys per chunk
 *   plan[6] key chunks               plan[7] workgroups launched (after padding)
 * Returns TV_ERR_SHAPE / TV_ERR_UNSUPPORTED for sizes tree_verify_attn rejects, and
 * TV_ERR_DTYPE for TV_F32 (one workgroup per output row, no plan).
 */
tv_status tree_verify_attn_plan(tv_dtype dt, int B, int n_max, int Hq, int Hkv, int D,
                                int max_prefix_len, int32_t* plan);
tv_status tree_verify_attn(tv_dtype dt, int B, int Hq, int Hkv, int D, int n_max,
                           int max_prefix_len, float scale, const void* q, const void* k_tree,
                           const void* v_tree, const void* k_prefix, const void* v_prefix,
                           const int64_t* prefix_offsets, const int32_t* n_nodes,
                           const uint64_t* anc, void* out, float* lse, void* ws, size_t ws_bytes,
                           int32_t* seq_status, hipStream_t stream);

/*
 * tree_verify_attn_noalloc -- tree_verify_attn for callers that cannot allocate: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same arguments, results and kernels as tree_verify_attn, without ws / ws_bytes: the
 * chunk partials go to a fixed 128 MiB device array of the library (one per GPU, held
 * until the process ends; it needs no initialisation).  Nothing is allocated or freed.
 * Returns TV_ERR_WORKSPACE when the partials of these sizes exceed 128 MiB
 * (tree_verify_attn_workspace_size(...) > 134217728), TV_ERR_HIP if the array's device
 * address cannot be read.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (concurrent streams, or host threads) race and must be ordered by
 * the caller.
 */
tv_status tree_verify_attn_noalloc(tv_dtype dt, int B, int Hq, int Hkv, int D, int n_max,
                                   int max_prefix_len, float scale, const void* q,
                                   const void* k_tree, const void* v_tree, const void* k_prefix,
                                   const void* v_prefix, const int64_t* prefix_offsets,
                                   const int32_t* n_nodes, const uint64_t* anc, void* out,
                                   float* lse, int32_t* seq_status, hipStream_t stream);

/*
 * tree_accept -- greedy acceptance of the longest matching path.
 * [EAGLE] "Well-Calibrated Draft Model": under greedy decoding a draft token is
 * accepted when it is the target's most likely token.  [EAGLE-3] section 4 step 4:
 * the target keeps the longest prefix of the tree whose tokens all pass.  [EAGLE-4]
 * "verification trees": after the accepted path, generation continues with the
 * target's own token.
 *
 *   parent, depth int32 [B][n_max], anc uint64 [B][n_max], n_nodes int32 [B]
 *                  (a tree that tree_build accepted)
 *   token          int32 [B][n_max]  draft token of each node (token[b][0] is the root's)
 *   target_next    int32 [B][n_max]  the target's greedy token after node i
 *   accept_len     int32 [B]  out    depth of the chosen node (accepted draft tokens)
 *   best_node      int32 [B]  out    the deepest node whose root path all passes
 *                                    (node j >= 1 passes iff token[j] ==
 *                                    target_next[parent[j]]); ties to the lowest index
 *   bonus_token    int32 [B]  out    target_next[best_node]
 *   path           int32 [B][n_max] out, nullable: the chosen path without the root in
 *                                    index order, -1 padded
 * Sequences with n_nodes outside [1, n_max], or whose anc[b][0] != 1 (a tree
 * tree_build rejected), get -1 in every output.
 */
tv_status tree_accept(int B, int n_max, const int32_t* parent, const int32_t* depth,
                      const uint64_t* anc, const int32_t* n_nodes, const int32_t* token,
                      const int32_t* target_next, int32_t* accept_len, int32_t* best_node,
                      int32_t* bonus_token, int32_t* path, hipStream_t stream);

/*
 * tree_accept_stochastic -- rejection-sampling acceptance over the tree.
 * [EAGLE] "Well-Calibrated Draft Model": under random sampling a draft token x is
 * accepted with rate min(1, P_target(x) / P_draft(x)).  [EAGLE-3] section 4 steps 3-4:
 * a rejected token gives way to the target's own token, sampled from a corrected
 * distribution; the longest passing prefix of the tree is kept.  [EAGLE-4]
 * "verification trees and the harness": rejection sampling leaves the output
 * distribution unchanged.  The pages give the one-candidate rule only; for a tree:
 * from the root, the current node u's children are tried in index order.  With r
 * the target weights (p_target[u] at first) and S their float64 sum, child c with
 * token x passes when u_accept[c] * S * q_draft[u][x] < r[x] (float64, left to right;
 * with q == 0: when r[x] > 0) and becomes the current node; a failing child turns r
 * into max(r - fl32(S) * q_draft[u], 0) (float32 product, then difference).  When
 * no child passes, the bonus token is the first v whose float64 running sum of r
 * exceeds u_bonus * S (the last v with r > 0 if rounding leaves none).
 *
 *   parent, anc, n_nodes, token  as for tree_accept (a tree tree_build accepted)
 *   p_target   float32 [B][n_max][vocab]  target's next-token distribution after
 *                                        node i's root path
 *   q_draft    float32 [B][n_max][vocab]  draft's distribution that proposed node
 *                                        i's children
 *   u_accept   float32 [B][n_max]  uniform in [0,1) used when node i is a candidate
 *   u_bonus    float32 [B]         uniform in [0,1) for the bonus token
 *   accept_len, best_node, bonus_token int32 [B], path int32 [B][n_max] (nullable):
 *                 as for tree_accept
 *   ws, ws_bytes   workspace of at least tree_accept_stochastic_workspace_size(B, n_max,
 *                  vocab) bytes, 16-byte aligned, device memory; nullable
 * vocab >= 1.  With a workspace (and a size query above 0) each sequence's vocabulary
 * is cut into slices, one workgroup each, that keep their slice of r and of the draft
 * row on chip and exchange their float64 totals through the workspace after every
 * change of r; the workgroups of one call must all be resident at once (the slices are
 * sized so that B times their number stays within the device's compute units), and a
 * sequence whose exchange waits past a bound (work of other streams holding the compute
 * units) gets -1 in every output.  The workspace needs no initial contents; calls that
 * share one must be ordered.  Without a workspace (ws NULL) one workgroup per sequence
 * walks the tree: up to 36864 tokens with r in LDS; past that r is recomputed from
 * p_target and q_draft on every pass over the vocabulary (same bits), so each rejection
 * streams two rows instead of one.  Tokens outside [0, vocab) fail.  Sums in float64
 * depend on their order in the last bits (the slices add their totals in slice order):
 * a decision within ~1e-15 (relative) of its threshold may differ from a sequential
 * evaluation.
 * Errors: TV_ERR_NULL, TV_ERR_SHAPE, TV_ERR_WORKSPACE (ws given but smaller than the
 * query or misaligned), TV_ERR_HIP.
 */
size_t tree_accept_stochastic_workspace_size(int B, int n_max, int vocab);
tv_status tree_accept_stochastic(int B, int n_max, int vocab, const int32_t* parent,
                                 const uint64_t* anc, const int32_t* n_nodes,
                                 const int32_t* token, const float* p_target,
                                 const float* q_draft, const float* u_accept,
                                 const float* u_bonus, int32_t* accept_len, int32_t* best_node,
                                 int32_t* bonus_token, int32_t* path, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * tree_kv_compact -- the accepted continuation's K/V into the KV cache.
 * [EAGLE-4] "verification trees and the harness": after verification the harness
 * keeps the accepted continuation, frees the rejected KV-cache entries and starts
 * the next round.  The continuation is the root (node 0, the target's last token:
 * queried in this pass, not yet cached) and the accepted path, root to leaf.
 *
 *   dt             TV_BF16 or TV_F32 (the element type of all four K/V buffers)
 *   k_tree, v_tree [B][n_max][Hkv][D]  per-node K/V of this pass (tree_verify_attn's
 *                                     k_tree / v_tree)
 *   path           int32 [B][n_max]   tree_accept's path (accepted nodes without the
 *                                     root, in index order = root-to-leaf order)
 *   accept_len     int32 [B]          tree_accept's accept_len; < 0 copies nothing
 *   k_dst, v_dst   [dst_rows][Hkv][D] destination rows (e.g. the cache after each
 *                                     sequence's prefix), caller-owned
 *   dst_row        int64 [B]          destination row of sequence b's root; rows
 *                                     dst_row[b] .. dst_row[b] + accept_len[b] are
 *                                     written: row 0 <- node 0, row j <- path[j-1]
 *   dst_rows       host int64         rows in k_dst / v_dst; rows outside
 *                                     [0, dst_rows) and path entries outside
 *                                     [0, n_max) are skipped
 * No other destination row is touched.  Rows of different sequences must not
 * overlap (they are written concurrently).  Needs Hkv*D*element size a multiple of
 * 16 bytes and 16-byte aligned buffers (else TV_ERR_UNSUPPORTED).
 */
tv_status tree_kv_compact(tv_dtype dt, int B, int n_max, int Hkv, int D, const void* k_tree,
                          const void* v_tree, const int32_t* path, const int32_t* accept_len,
                          void* k_dst, void* v_dst, const int64_t* dst_row, int64_t dst_rows,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TREEVERIFY_H */
