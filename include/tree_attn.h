/*
 * tree_attn.h - C ABI of the MI355X (gfx950) tree-packed attention library.
 *
 * Branching token sequences that share prefixes are merged into one prefix
 * tree and laid out in depth-first (preorder) order, every tree token once
 * ("Tree Training", §3.1 Eq. 8; the "Trie packing" page, Step 1; the Claw-R1
 * "Prefix Tree Merge" page, section 1). Each packed token attends only to its
 * ancestors and itself ("Trie packing" Step 2; "Tree Training" §3.2, Attention
 * Mask), and takes RoPE at its depth on its own path ("Trie packing" Step 1;
 * "Tree Training" §3.2 Eq. 9). In preorder the descendants of token j are
 * exactly the packed indices in (j, subtree_end[j]), so the mask is the O(T)
 * rule: key j is visible to query i  iff  j <= i < subtree_end[j].
 *
 * Conventions for every entry point
 *   - Return value: TA_OK (0) or a negative TA_E* code. No C++ exception
 *     crosses this boundary. tree_attn_last_error() returns a thread-local
 *     message for the last failure on the calling thread.
 *   - All arguments are validated on the host before any HIP call; a rejected
 *     call touches no memory and launches nothing.
 *   - Nothing is allocated and nothing is freed: every buffer is owned by the
 *     caller. Device entry points are asynchronous on `stream` (a hipStream_t
 *     passed as void*, NULL = the default stream) and do not synchronize.
 *   - Device tensors are contiguous and token-major: q, o, dout, dq are
 *     [T][Hq][d]; k, v, dk, dv are [T][Hkv][d]; lse is [Hq][T] float32.
 *     Query head h uses kv head h / (Hq / Hkv).
 *   - The library keeps no state besides the thread-local error string, the
 *     opt-in, process-wide kernel timing table (tree_attn_profile_*; while it
 *     is enabled the library creates HIP events inside its calls) and the
 *     per-device entry table of tree_logprob_noalloc: calls on different
 *     streams with separate workspaces may run concurrently (calls of
 *     tree_logprob_noalloc that overlap on one device may not).
 */
#ifndef TREE_ATTN_H
#define TREE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  TA_OK = 0,
  TA_EINVAL = -1,       /* bad argument: null pointer, bad size or offsets */
  TA_ECAPACITY = -2,    /* an output capacity is too small; sizes reported */
  TA_EUNSUPPORTED = -3, /* valid but unsupported shape (e.g. head dim) */
  TA_EHIP = -4          /* a HIP runtime call or kernel launch failed */
};

typedef enum { TA_BF16 = 0, TA_F32 = 1 } ta_dtype;

/* Backward flags.
 * TA_REUSE_PREP: the workspace still holds what the matching forward put
 *   there for the same q, k, pos, subtree_end, T, heads, d and rope_theta
 *   (and cached rows), so the RoPE and tile-plan pass is skipped.
 * TA_ACCUMULATE_PAST (tree_attn_gw_bwd only): add the cached rows' gradients
 *   to dk_past / dv_past instead of overwriting them. */
enum { TA_REUSE_PREP = 1, TA_ACCUMULATE_PAST = 2 };

/* Thread-local text of the last error ("" if none). Never NULL. */
const char* tree_attn_last_error(void);

/* ------------------------------------------------------------------------
 * tree_pack  (HOST)
 *
 * Packs token sequences into DFS-serialized prefix trees, one tree per group.
 * Follows the "Trie packing" page (shared prefixes, depth positions), "Tree
 * Training" §3.1 (Eq. 2-4: g_t paths through t, weight g_t / K; Eq. 8: DFS
 * serialization; Eq. 9: positions) and the "Prefix Tree Merge" page, section
 * 1 (insert, compress single-child chains, preorder ranges).
 *
 * Readings fixed here: children are visited in first-insertion order; a new
 * node (chunk) starts at a tree root, below a fork, and after a token where
 * an input sequence ends; K is the number of input sequences of the group and
 * g the number of input sequences containing the token; groups become trees
 * in order of first appearance; positions restart at 0 in each tree; all
 * ends are exclusive.
 *
 * Inputs (host memory, caller-owned, read only):
 *   tokens        [seq_offsets[n_seqs]] token ids, any int32 value
 *   seq_offsets   [n_seqs + 1] int64, seq_offsets[0] == 0, strictly
 *                 increasing (an empty sequence is TA_EINVAL)
 *   n_seqs        >= 1
 *   group_of_seq  [n_seqs] group label per sequence, or NULL (one tree)
 *   cap_T         capacity of the per-token outputs (T <= seq_offsets[n_seqs])
 *   cap_nodes     capacity of the per-node outputs (n_nodes <= T)
 * Outputs (host memory, caller-owned; any may be NULL to skip it):
 *   packed_ids [T]  token id;    pos [T] depth on its path;
 *   subtree_end [T] one past its last descendant;  parent [T] (-1 at a root);
 *   path_count [T]  g;  weight [T] float32 g / K (IEEE round-to-nearest);
 *   occ_map [seq_offsets[n_seqs]]  packed index of every input token;
 *   node_start, node_end (exclusive), node_parent (-1 at a root),
 *   node_subtree_end  [n_nodes];
 *   tree_start [n_trees + 1] (capacity n_seqs + 1 always suffices);
 *   sizes  T, n_nodes, n_trees (always filled when non-NULL and the inputs
 *          are valid, also on TA_ECAPACITY).
 * Errors: TA_EINVAL (bad inputs), TA_ECAPACITY (cap_T < T or
 * cap_nodes < n_nodes; nothing but `sizes` is written).
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t T;
  int32_t n_nodes;
  int32_t n_trees;
} ta_pack_sizes;

int tree_pack(const int32_t* tokens, const int64_t* seq_offsets, int32_t n_seqs,
              const int32_t* group_of_seq, int32_t cap_T, int32_t cap_nodes,
              int32_t* packed_ids, int32_t* pos, int32_t* subtree_end, int32_t* parent,
              int32_t* path_count, float* weight, int32_t* occ_map,
              int32_t* node_start, int32_t* node_end, int32_t* node_parent,
              int32_t* node_subtree_end, int32_t* tree_start, ta_pack_sizes* sizes);

/* ------------------------------------------------------------------------
 * Tree-masked attention (DEVICE)
 *
 * Forward ("Trie packing" Step 3: S = Q K^T / sqrt(d) + M_tree, M_tree = 0
 * where visible, -inf elsewhere; "Tree Training" §3.2):
 *   q'_i = R(pos_i) q_i,  k'_j = R(pos_j) k_j        (RoPE, rotate-half)
 *   S_ij = scale * q'_i . k'_j   for visible pairs  (j <= i < subtree_end[j])
 *   o_i  = sum_j softmax_j(S_ij) v_j;  lse_i = ln sum_j exp(S_ij)
 * RoPE: angle(p, k) = p * rope_theta^(-2k/d) rotates dims (k, k + d/2);
 * rope_theta == 0 disables RoPE. scale <= 0 selects 1/sqrt(d).
 *
 * Backward (the "Trie packing" page, "Same chain rule", Step 3: ordinary
 * attention backward, masked edges contribute nothing; a shared key / value
 * row collects the gradients of all its descendants):
 *   dv_j = sum_i P_ij do_i;  dS_ij = P_ij (do_i . v_j - do_i . o_i)
 *   dq_i = R(pos_i)^T scale sum_j dS_ij k'_j;  dk_j = R(pos_j)^T scale sum_i dS_ij q'_i
 * with dk and dv summed over the query heads of a kv group. All gradient
 * accumulation is float32 ("Tree Training" App. B.5); dq, dk, dv are written
 * once, in the tensor dtype. The result is bitwise reproducible.
 *
 * dt: TA_BF16 or TA_F32 for q, k, v, o, dout, dq, dk, dv (TA_F32 inputs are
 * rounded to bf16 for the matrix products; accumulation stays float32).
 * q, k, v, o, dout must be 16-byte aligned (they are read with 16-byte
 * vector loads; else TA_EINVAL).
 * d must be 16, 64 or 128 (else TA_EUNSUPPORTED). 1 <= T <= 2^22,
 * Hq % Hkv == 0, Hq <= 256.
 * pos, subtree_end: device int32 [T] as produced by tree_pack (a forest of
 * trees is fine; subtree ends must satisfy i < subtree_end[i] <= T). Only
 * the device sees these values: a subtree end outside (i, T] is clamped into
 * that range (so no access leaves the buffers and every row sees at least
 * itself) and sets TA_STATUS_SUBTREE_END in the workspace status word; the
 * outputs are then those of the clamped mask.
 * workspace: device memory of at least tree_attn_workspace_bytes(...) bytes,
 * 256-byte aligned; contents are scratch between calls except under
 * TA_REUSE_PREP and the status word at its start (see
 * tree_attn_workspace_status). The size is O(T (Hq + Hkv) d) plus, with
 * with_bwd, a fixed 64 x Hkv x max(d, 32) KiB of float32 partial sums
 * for key tiles whose dK/dV work is split over several workgroups (64 MB at
 * Hkv = 8, d = 128).
 * Errors: TA_EINVAL, TA_EUNSUPPORTED, TA_EHIP (launch failure).
 * ---------------------------------------------------------------------- */
size_t tree_attn_workspace_bytes(int32_t T, int32_t Hq, int32_t Hkv, int32_t d, int32_t with_bwd);

int tree_attn_fwd(const void* q, const void* k, const void* v, ta_dtype dt,
                  int32_t T, int32_t Hq, int32_t Hkv, int32_t d,
                  const int32_t* pos, const int32_t* subtree_end,
                  float softmax_scale, float rope_theta,
                  void* o, float* lse, void* workspace, size_t ws_bytes, void* stream);

int tree_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, ta_dtype dt, int32_t T, int32_t Hq, int32_t Hkv, int32_t d,
                  const int32_t* pos, const int32_t* subtree_end,
                  float softmax_scale, float rope_theta, int32_t flags,
                  void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * tree_attn_workspace_status  (HOST, reads device memory)
 *
 * Data errors that only the device can see (the conventions of the C ABI:
 * arguments are validated on the host, metadata values are not). Every prep
 * pass (tree_attn_fwd, tree_attn_gw_fwd, and a backward without
 * TA_REUSE_PREP) clears the int32 status word at the start of its workspace
 * and sets bits in it; the word then stays as it is until the next prep pass
 * on that workspace. This call enqueues a copy of the word to *status (host
 * memory) on `stream` and waits for the stream.
 *   TA_STATUS_SUBTREE_END  some subtree_end[i] was outside (i, T] and clamped
 * Errors: TA_EINVAL (NULL pointer), TA_EHIP.
 * ---------------------------------------------------------------------- */
enum { TA_STATUS_SUBTREE_END = 1 };

int tree_attn_workspace_status(const void* workspace, int32_t* status, void* stream);

/* ------------------------------------------------------------------------
 * tree_attn_plan_counts  (HOST, reads device memory)
 *
 * The tile plan the device built in `workspace` during the last prep pass,
 * per 128-row query tile: nonempty[t] = key tiles of 64 the forward and dQ
 * passes visit for query tile t (tiles the plan skips hold no visible pair),
 * full[t] = those among them whose every pair is visible (no masking). The
 * classification is the one tree_tile_stats counts on the host, at BQ = 128,
 * BK = 64. T, past_len, Hq, Hkv, d: as given to the call that filled the
 * workspace (past_len = 0 for tree_attn_fwd); n_qtiles must equal
 * ceil((ceil(past_len / 128) * 128 + T) / 256) * 2. Query tiles of cached rows
 * and of padding report 0. Copies on `stream` into host memory and waits.
 * Errors: TA_EINVAL (shape, size, NULL), TA_EHIP.
 * ---------------------------------------------------------------------- */
int tree_attn_plan_counts(const void* workspace, size_t ws_bytes, int32_t T, int32_t past_len, int32_t Hq,
                          int32_t Hkv, int32_t d, int32_t n_qtiles, int32_t* nonempty, int32_t* full,
                          void* stream);

/* ------------------------------------------------------------------------
 * Tree-masked attention across a partition boundary (DEVICE)
 *
 * "Tree Training" §3.3 and App. B.2-B.5: a tree too large for one pass is
 * split at node boundaries; a child partition does not re-run its
 * ancestors but attends to the parent partition's cached, already rotated
 * keys and values (the "gateway", App. B.2). Its attention mask (Eq. 14) is
 *   cached row j:  0 if past_visible[j] else -inf  (the ancestor bias of
 *                  Eq. 15-16, the same for every query of the partition)
 *   own row j:     the ordinary tree mask of the partition's packed subtree
 * Own tokens take RoPE at pos_offset + pos[i] (Eq. 17: the depth of the
 * cut node's last token + 1). The gradients of the cached rows come out in
 * float32 (Eq. 18) and, with TA_ACCUMULATE_PAST, are added to what the
 * previous child partitions of the same cut node left there.
 *
 * Arguments as for tree_attn_fwd / tree_attn_bwd (q, k, v, o, dout, dq, dk,
 * dv, lse hold the T own tokens; pos and subtree_end are the partition's own
 * packing), plus:
 * k_past, v_past: device [past_len][Hkv][d] in dtype dt; k_past already
 *   rotated (RoPE at the parent's positions), v_past as is; 16-byte aligned.
 * past_visible: device uint8 [past_len], 1 = bias 0, 0 = bias -inf.
 * past_len: >= 0 (0 gives plain tree attention); T + past_len <= 2^22 - 128.
 * pos_offset: >= 0.
 * dk_past, dv_past: device float32 [past_len][Hkv][d]; dk_past is the
 *   gradient with respect to the rotated k_past (tree_attn_gw_relay takes
 *   it back through the parent's RoPE); rows the bias masks get 0.
 * tree_attn_gw_export builds k_past / v_past from the parent's tensors.
 * workspace: >= tree_attn_gw_workspace_bytes(T, past_len, ...) bytes.
 * Errors: TA_EINVAL, TA_EUNSUPPORTED, TA_EHIP. No allocation; asynchronous
 * on `stream`; bitwise reproducible for a fixed TA_ACCUMULATE_PAST order.
 * ---------------------------------------------------------------------- */
size_t tree_attn_gw_workspace_bytes(int32_t T, int32_t past_len, int32_t Hq, int32_t Hkv, int32_t d,
                                    int32_t with_bwd);

int tree_attn_gw_fwd(const void* q, const void* k, const void* v, ta_dtype dt,
                     int32_t T, int32_t Hq, int32_t Hkv, int32_t d,
                     const int32_t* pos, const int32_t* subtree_end, int32_t pos_offset,
                     const void* k_past, const void* v_past, const uint8_t* past_visible, int32_t past_len,
                     float softmax_scale, float rope_theta,
                     void* o, float* lse, void* workspace, size_t ws_bytes, void* stream);

int tree_attn_gw_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, ta_dtype dt, int32_t T, int32_t Hq, int32_t Hkv, int32_t d,
                     const int32_t* pos, const int32_t* subtree_end, int32_t pos_offset,
                     const void* k_past, const void* v_past, const uint8_t* past_visible, int32_t past_len,
                     float softmax_scale, float rope_theta, int32_t flags,
                     void* dq, void* dk, void* dv, float* dk_past, float* dv_past,
                     void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * tree_attn_gw_export / tree_attn_gw_relay  (DEVICE)
 *
 * The two hand-overs across a partition boundary ("Tree Training" App. B.2:
 * the parent's keys after RoPE and its values are cached for the child
 * partitions; App. B.5: the gradients of the cached rows, kept in float32,
 * flow back into the parent's gradients, summed over its children, Eq. 18).
 * They act on the tensors of one partition (the parent, or any ancestor
 * partition that holds part of a gateway): k, v, dk, dv [T][Hkv][d] in dt,
 * pos [T] its own depth positions, pos_offset its own offset (0 for a
 * partition of tree roots), so token j sits at position pos_offset + pos[j].
 * rows: device int32 [n_rows], the partition's own token indices that make
 * up cached rows r = 0 .. n_rows - 1 (for a gateway spread over several
 * ancestor partitions, call once per partition on the matching slice of
 * k_past / v_past / dk_past / dv_past).
 *
 * export: k_past[r] = R(pos_offset + pos[rows[r]]) k[rows[r]] (rotated in
 *   float32 exactly as the attention prep rotates its keys, then stored in
 *   dt), v_past[r] = v[rows[r]]; k_past, v_past [n_rows][Hkv][d] in dt. A row
 *   index outside [0, T) exports zeros.
 * relay: dk[rows[r]] += R(...)^T dk_past[r], dv[rows[r]] += dv_past[r], with
 *   dk_past, dv_past float32 [n_rows][Hkv][d] as tree_attn_gw_bwd returns
 *   them; each sum is formed in float32 and rounded once to dt. Run it after
 *   the partition's own tree_attn_bwd / tree_attn_gw_bwd (which overwrite dk,
 *   dv). rows must be distinct (calls that overlap on one stream and rows are
 *   ordered; duplicated rows within one call race). A row outside [0, T) is
 *   skipped.
 * Asynchronous on `stream`; no allocation. 16-byte alignment is not needed.
 * Errors: TA_EINVAL (NULL, sizes, dtype, negative theta or offset),
 * TA_EUNSUPPORTED (d not in {16, 64, 128}), TA_EHIP.
 * ---------------------------------------------------------------------- */
int tree_attn_gw_export(const void* k, const void* v, ta_dtype dt, int32_t T, int32_t Hkv, int32_t d,
                        const int32_t* pos, int32_t pos_offset, float rope_theta, const int32_t* rows,
                        int32_t n_rows, void* k_past, void* v_past, void* stream);

int tree_attn_gw_relay(const float* dk_past, const float* dv_past, const int32_t* rows, int32_t n_rows,
                       ta_dtype dt, int32_t T, int32_t Hkv, int32_t d, const int32_t* pos, int32_t pos_offset,
                       float rope_theta, void* dk, void* dv, void* stream);

/* ------------------------------------------------------------------------
 * tree_logprob  (DEVICE)
 *
 * Per-occurrence log-probabilities gathered from shared logit rows, weighted
 * loss, and the gradient scatter-added into the shared rows (the "Trie
 * packing" page, "Share logits, preserve every prediction" and "Combine
 * gradients at the shared logits"; "Tree Training" §3.1 Eq. 4 and §3.2 Loss
 * Weights):
 *   lse_r   = ln sum_v exp z[r, v]
 *   logp_m  = z[src_m, tgt_m] - lse[src_m]
 *   loss    = -sum_m w_m logp_m
 *   dlogits[r, :] = grad_scale * sum_{m: src_m = r} w_m (softmax(z_r) - e_{tgt_m})
 * Rows no entry references get dlogits = 0.
 *
 * logits [R][V] (dt TA_BF16 or TA_F32), row-major, device.
 * src_row, target: device int32 [M]; weight: device float32 [M].
 * logp [M] float32 (required). row_lse [R] float32 or NULL. loss: device
 * float32 scalar or NULL. dlogits [R][V] in dt, or NULL for forward only.
 * An entry with src_row outside [0, R) or target outside [0, V) gets
 * logp = NaN, contributes NaN to loss, and nothing to dlogits.
 * The loss and dlogits are summed in a fixed order: bitwise reproducible.
 * workspace: >= tree_logprob_workspace_bytes(R, M) bytes, 256-byte aligned.
 * Limits: 1 <= R < 2^31, 1 <= V < 2^31, 0 <= M < 2^31 - 1.
 * Errors: TA_EINVAL, TA_EHIP.
 * ---------------------------------------------------------------------- */
size_t tree_logprob_workspace_bytes(int64_t R, int64_t M);

int tree_logprob(const void* logits, ta_dtype dt, int64_t R, int64_t V,
                 const int32_t* src_row, const int32_t* target, const float* weight, int64_t M,
                 float* logp, float* row_lse, float* loss,
                 void* dlogits, float grad_scale,
                 void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * tree_logprob_noalloc  (DEVICE)
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): exactly
 * tree_logprob, with the same arguments and results, minus the workspace.
 * Its entry table lives in a fixed 16 MiB device array inside the library,
 * one per device for the life of the process, so a call needs
 * tree_logprob_workspace_bytes(R, M) <= 16 MiB (about R + M <= 1.3 million);
 * larger calls return TA_ECAPACITY without touching the device. The array's
 * address is resolved on the first call on each device (the device of
 * `stream`); later calls make no runtime call besides their launches and
 * allocate nothing. Every call on a device shares that device's array:
 * calls that overlap on one device (other streams, other threads) race and
 * must be ordered by the caller. Each call clears what it needs zeroed.
 * Errors: those of tree_logprob, TA_ECAPACITY, TA_EHIP.
 * ---------------------------------------------------------------------- */
int tree_logprob_noalloc(const void* logits, ta_dtype dt, int64_t R, int64_t V,
                         const int32_t* src_row, const int32_t* target, const float* weight, int64_t M,
                         float* logp, float* row_lse, float* loss,
                         void* dlogits, float grad_scale, void* stream);

/* ------------------------------------------------------------------------
 * tree_logprob_ppo  (DEVICE)
 *
 * Per-occurrence clipped policy loss on shared logit rows. The "Trie
 * packing" page (its PPO/GRPO paragraph) keeps, for every prediction
 * occurrence, its own advantage, old log-probability, clipping, mask and
 * weight, and warns against averaging advantages before the nonlinear loss;
 * "Tree Training" §3.1 gives the RL per-token objective -A_t log p. The
 * clipping rule, which the pages do not spell out, is the PPO clipped
 * surrogate:
 *   logp_m  as tree_logprob
 *   r_m     = exp(logp_m - old_logp_m)
 *   l_m     = -min(r_m A_m, clip(r_m, 1 - eps_low, 1 + eps_high) A_m)
 *   loss    = sum_m w_m mask_m l_m
 *   c_m     = -dloss/dlogp_m = w_m mask_m A_m r_m if r_m A_m <= clip(r_m) A_m, else 0
 *   dlogits[r, :] = grad_scale * sum_{m: src_m = r} c_m (softmax(z_r) - e_{tgt_m})
 * advantage, old_logp: device float32 [M]; mask: device uint8 [M] or NULL
 * (all on); a masked entry still gets logp but adds nothing to loss or
 * dlogits. eps_low, eps_high >= 0 (INFINITY: no clipping on that side).
 * Other arguments, layouts, limits and the workspace are those of
 * tree_logprob (same tree_logprob_workspace_bytes); an invalid entry gets
 * logp = NaN and, unless masked, makes the loss NaN. Bitwise reproducible.
 * Errors: TA_EINVAL (also for a negative or NaN eps), TA_EHIP.
 * ---------------------------------------------------------------------- */
int tree_logprob_ppo(const void* logits, ta_dtype dt, int64_t R, int64_t V,
                     const int32_t* src_row, const int32_t* target, const float* weight,
                     const float* advantage, const float* old_logp, const uint8_t* mask, int64_t M,
                     float eps_low, float eps_high,
                     float* logp, float* row_lse, float* loss,
                     void* dlogits, float grad_scale,
                     void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * tree_tile_stats  (HOST)
 *
 * Counts of (query-tile, key-tile) pairs under the tile classification the
 * kernels use, from a host copy of subtree_end. Tiles are BQ rows x BK keys;
 * key columns past T are padding that is never visible; only causal tiles
 * (first key <= last real row) are counted. With i0/i1 the first/one-past-
 * last real row and j0/j1 = j0 + BK the key range of a tile:
 *   empty   max(subtree_end over its keys) <= i0
 *   full    j1 - 1 <= i0 and min(subtree_end over its keys, padding = 0) >= i1
 *   partial otherwise
 * An empty tile holds no visible pair and a full tile only visible pairs.
 * Errors: TA_EINVAL.
 * ---------------------------------------------------------------------- */
int tree_tile_stats(const int32_t* subtree_end, int32_t T, int32_t BQ, int32_t BK,
                    int64_t* full, int64_t* partial, int64_t* empty, int64_t* causal);

/* ------------------------------------------------------------------------
 * tree_partition  (HOST)
 *
 * Partition plan for a tree that does not fit one pass ("Tree Training"
 * §3.3, Partitioning): cuts only at node boundaries; every partition has
 * exactly one parent partition (or none), so a backward pass keeps one
 * root-to-leaf chain of partition graphs alive; each partition holds at most
 * `capacity` tokens; the number of partitions is kept small. The pages leave
 * the algorithm to a general solver; this planner:
 *   1. cuts the tree into the fewest connected pieces of <= capacity tokens
 *      (bottom-up; while a node's residual, its length plus its attached
 *      children's residuals, exceeds capacity, the child with the largest
 *      residual -- ties: the earlier child -- is cut off);
 *   2. packs pieces cut from the same node (or tree roots), which share every
 *      ancestor, into shared partitions, first-fit decreasing by tokens
 *      (ties: preorder); tree roots first, then, for the partitions in
 *      creation order, the groups hanging from their nodes in preorder.
 * Inputs: the tree_pack chunk table (node_start, node_end exclusive,
 * node_parent; preorder). Outputs (host, caller-owned, n_nodes entries each
 * suffice): node_part[n] = partition of node n; part_tokens[p];
 * part_parent[p] (-1 for a partition of tree roots); part_cut[p] = the node
 * its pieces hang from (-1 for tree roots); *n_parts.
 * A child partition runs through tree_attn_gw_* with one gateway: the cached
 * rows of the cut node's last token and its ancestors (all visible), at
 * pos_offset = that token's depth + 1.
 * Errors: TA_EINVAL (a node longer than capacity, a parent not before its
 * node, an empty node, NULL arguments).
 * ---------------------------------------------------------------------- */
int tree_partition(const int32_t* node_start, const int32_t* node_end, const int32_t* node_parent,
                   int32_t n_nodes, int64_t capacity,
                   int32_t* node_part, int32_t* part_tokens, int32_t* part_parent, int32_t* part_cut,
                   int32_t* n_parts);

/* ------------------------------------------------------------------------
 * tree_conv_fwd / tree_conv_bwd  (DEVICE)
 *
 * Tree-correct depthwise causal conv1d ("Tree Training" §3.2, SSM Layers,
 * Eq. 11; App. A.3). In the DFS layout the tokens just before a child chunk
 * belong to a sibling branch, so every token's window is taken along its own
 * ancestor chain, as an independent per-branch pass would see it:
 *   a_t = bias + sum_{n=0}^{K-1} weight[:, K-1-n] * x_{anc_n(t)}
 *   y_t = SiLU(a_t) (activation = 1) or a_t (activation = 0)
 * anc_0(t) = t, anc_{n+1}(t) = parent[anc_n(t)]; terms past a root are zero.
 * x, y, dy, dx: device [T][C] in dt (TA_BF16 or TA_F32), 16-byte aligned;
 * weight: device float32 [C][K]; bias: device float32 [C] or NULL.
 * parent, pos, subtree_end: device int32 [T] from tree_pack. Only the device
 * reads them: a parent not in [-1, t) is read as -1 (no parent), a subtree
 * end outside (t, T] is clamped into it and a descendant at depth <= the
 * token's own is skipped, so malformed metadata gives meaningless values but
 * no access outside [0, T) and no endless walk.
 * Backward: dx in dt; dweight float32 [C][K]; dbias float32 [C] or NULL.
 * Gradients are summed in a fixed order (bitwise reproducible). The backward
 * gathers each token's descendants at most K-1 levels down from the
 * preorder range (t, subtree_end[t]) and pos; g = dy * act'(a) passes
 * between its passes in dt (dweight and dbias use it in float32).
 * Limits: T >= 1 (backward: T < 2^28), C a positive multiple of 8, 1 <= K <= 8.
 * workspace (backward): >= tree_conv_workspace_bytes(T, C, K) bytes, 256-byte
 * aligned. Errors: TA_EINVAL, TA_EHIP.
 * ---------------------------------------------------------------------- */
int tree_conv_fwd(const void* x, ta_dtype dt, int32_t T, int32_t C, int32_t K,
                  const float* weight, const float* bias, const int32_t* parent, int32_t activation,
                  void* y, void* stream);

size_t tree_conv_workspace_bytes(int32_t T, int32_t C, int32_t K);

int tree_conv_bwd(const void* x, const void* dy, ta_dtype dt, int32_t T, int32_t C, int32_t K,
                  const float* weight, const float* bias, const int32_t* parent, const int32_t* pos,
                  const int32_t* subtree_end, int32_t activation,
                  void* dx, float* dweight, float* dbias,
                  void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * tree_gdn_plan  (HOST)
 *
 * Chunk schedule for tree_gdn_fwd ("Tree Training" §3.2, SSM Layers, Eq. 10:
 * each tree node's segment starts from its parent node's end state; App.
 * A.2). Every node of the tree_pack chunk table (node_start, node_end
 * exclusive, node_parent; nodes in preorder, contiguous from 0) is cut into
 * chunks of at most `chunk` tokens (1..64). A chunk's parent is the previous
 * chunk of its node or the last chunk of the parent node (-1 at a root). A
 * chain is a maximal run of chunks each of whose parent is the chunk before
 * it; a chain's level is 0 at a root, else one more than the level of the
 * chain holding its parent chunk.
 * plan: host int32, `cap` entries; NULL or too small -> TA_ECAPACITY with
 * sizes filled in. Layout: header [n_chunks, n_chains, n_levels, chunk, T,
 * 0, 0, 0], chunk_start[n_chunks], chunk_len[n_chunks],
 * chunk_parent[n_chunks], chain_begin[n_chains + 1], chains by level
 * [n_chains], level_off[n_levels + 1], child_off[n_chunks + 1],
 * child_chains[n_chains] (the chains starting under chunk c, increasing).
 * Errors: TA_EINVAL (non-contiguous nodes, bad parent, chunk out of range),
 * TA_ECAPACITY.
 * ---------------------------------------------------------------------- */
typedef struct { int32_t n_chunks, n_chains, n_levels, plan_ints; } ta_gdn_plan_sizes;

int tree_gdn_plan(const int32_t* node_start, const int32_t* node_end, const int32_t* node_parent,
                  int32_t n_nodes, int32_t chunk, int32_t* plan, int32_t cap, ta_gdn_plan_sizes* sizes);

/* ------------------------------------------------------------------------
 * tree_gdn_fwd  (DEVICE)
 *
 * Gated delta rule with the recurrent state routed along the tree ("Tree
 * Training" §3.2, Eq. 10; App. A.2): per v-head, with alpha_t = exp(g_t),
 *   h_t = alpha_t (I - beta_t k_t k_t^T) h_{parent(t)} + beta_t k_t v_t^T,
 *   h = 0 before a root,  o_t = h_t^T q_t,
 * which equals running every root-to-leaf branch on its own. q/k head of
 * v-head j is j / (Hv / H); q and k are used as given (normalisation and
 * scaling are the caller's). Computed in chunks of the plan: WY form inside
 * a chunk, bf16 matrix products with float32 accumulation, the state carried
 * in float32 from chunk to chunk.
 * q, k: device [T][H][dk]; v, o: device [T][Hv][dv], dt TA_BF16 or TA_F32
 * (float inputs are rounded to bf16 for the products), 16-byte aligned.
 * g (log decay, <= 0 expected), beta: device float32 [T][Hv].
 * plan: device copy of the tree_gdn_plan blob; plan_host: the same blob in
 * host memory (its header and level table drive the launches).
 * dk, dv in {64, 128}; Hv a multiple of H.
 * workspace: >= tree_gdn_workspace_bytes(H, Hv, dk, dv, n_chunks) bytes,
 * 256-byte aligned; a workspace of tree_gdn_bwd_workspace_bytes serves as
 * well and is what a later tree_gdn_bwd of this call needs (the forward
 * leaves its chunk states and WY factors there). Asynchronous on `stream`;
 * one launch per chain level.
 * Errors: TA_EINVAL, TA_EUNSUPPORTED (dk, dv), TA_EHIP.
 * ---------------------------------------------------------------------- */
size_t tree_gdn_workspace_bytes(int32_t H, int32_t Hv, int32_t dk, int32_t dv, int32_t n_chunks);

int tree_gdn_fwd(const void* q, const void* k, const void* v, ta_dtype dt,
                 const float* g, const float* beta, int32_t T, int32_t H, int32_t Hv, int32_t dk, int32_t dv,
                 const int32_t* plan, const int32_t* plan_host, void* o,
                 void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * tree_gdn_bwd  (DEVICE)
 *
 * Gradients of sum(dout * o) for tree_gdn_fwd ("Tree Training" §3.2, Eq.
 * 10; App. A.2 gives the forward, which training differentiates): dq, dk
 * (summed over the v-heads that read each q/k head), dv, dg, dbeta. A
 * chunk's start state is its parent chunk's end state, so the gradient of a
 * chunk's end state is the sum of the start-state gradients of its child
 * chunks (siblings share one state and add their gradients, in increasing
 * chain order). Computed per chunk in reverse WY form: a parallel pass forms
 * the chunk-local terms, a reverse state pass (levels deepest first, each
 * chain from its last chunk back) carries the state gradient in float32, and
 * two parallel passes form the input gradients with bf16 matrix products and
 * float32 accumulation. Every sum is taken in a fixed order (bitwise
 * reproducible).
 * q, k, v, g, beta, plan, plan_host, T, H, Hv, dk, dv, dt: exactly as given
 * to the tree_gdn_fwd call whose outputs are differentiated.
 * dout: device [T][Hv][dv] in dt. dq, dk_out: device [T][H][dk] in dt;
 * dv_out: device [T][Hv][dv] in dt; dg, dbeta: device float32 [T][Hv]. All
 * 16-byte aligned, none overlapping another.
 * workspace: >= tree_gdn_bwd_workspace_bytes(H, Hv, dk, dv, n_chunks,
 * n_chains) bytes, 256-byte aligned, and the one that tree_gdn_fwd call
 * filled (its first tree_gdn_workspace_bytes bytes hold the forward's
 * chunk states and WY factors, which are read, not recomputed), unchanged
 * since. Asynchronous on `stream`.
 * Errors: TA_EINVAL, TA_EUNSUPPORTED (dk, dv), TA_EHIP.
 * ---------------------------------------------------------------------- */
size_t tree_gdn_bwd_workspace_bytes(int32_t H, int32_t Hv, int32_t dk, int32_t dv, int32_t n_chunks,
                                    int32_t n_chains);

int tree_gdn_bwd(const void* q, const void* k, const void* v, ta_dtype dt,
                 const float* g, const float* beta, const void* dout,
                 int32_t T, int32_t H, int32_t Hv, int32_t dk, int32_t dv,
                 const int32_t* plan, const int32_t* plan_host,
                 void* dq, void* dk_out, void* dv_out, float* dg, float* dbeta,
                 void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Kernel timing (HOST control; for benchmarks and tracing)
 *
 * tree_attn_profile_enable(1) clears the table and starts bracketing every
 * kernel group the library launches (RoPE prep, tile plan, forward, row
 * dots, dQ, dK/dV, log-prob CSR / rows / loss) with HIP events on the
 * caller's stream; (0) stops. tree_attn_profile_read(idx, ...) waits for the
 * recorded events and returns the idx-th kernel group's name, total time in
 * milliseconds and launch count (TA_EINVAL past the last entry). The table
 * is process-wide and guarded by a mutex; timings of calls that overlap on
 * several streams are not meaningful.
 * ---------------------------------------------------------------------- */
int tree_attn_profile_enable(int32_t on);
int tree_attn_profile_read(int32_t idx, char* name, int32_t name_cap, double* total_ms, int64_t* count);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H */
