/*
 * libmfdtree -- the mixture draft tree (Multi-Future Drafting) hot path on
 * MI355X (gfx950), behind a plain C ABI.
 *
 * What the calls compute, in the order a decoding round runs them:
 *
 *   mfd_logsoftmax_topk    per (tree, mode, position) row of drafter logits:
 *                          the log-normaliser and the k best tokens.
 *   mfd_mixture_threshold  the common cut-off: the B-th best best-mode score
 *                          over all prefixes, counting each prefix once.
 *   mfd_tree_build         the prefixes that reach the cut-off, merged into
 *                          one deduplicated tree with ties broken, laid out.
 *   mfd_mixture_tree       the two calls above from one search, in one launch.
 *   mfd_tree_mask          ancestor mask and position ids for verification.
 *   mfd_verify_walk        the verification walk over the target's per-node
 *                          logits: accepted length tau and the bonus token.
 *
 * Sources: the model card "MFD drafter for Qwen3.5-4B (1.42M prompts)"
 * (summary paragraph: K modes draft in one pass, the tree keeps the B
 * prefixes with the highest best-mode log-probability, the target verifies
 * it in one pass, standard tree verification keeps decoding lossless;
 * "Model": block of 16, 15 drafted positions; "Usage": tree_budget = B,
 * block_size - 1 = L, temperature = T) and the project page "Multi-Future
 * Drafting: Mixture Block Drafters for Tree-Verified Speculative Decoding"
 * ("In one minute": the B-th best score is the common cut-off, each mode
 * keeps the prefixes that reach it, a prefix produced by several modes
 * becomes one node; "How it works" step 1: a prefix's probability under a
 * mode is the product of that mode's per-position probabilities; step 3:
 * best-mode scoring, the union of
 * the per-mode trees, one verification pass; Figure 2: one distribution per
 * position per mode, tau counts the bonus token).
 *
 * Conventions for every call
 *   - Pointers named as device pointers are device memory on the current HIP
 *     device, contiguous, row-major, caller-owned.  The library allocates
 *     nothing and keeps no state between calls; calls on different streams
 *     are independent when their workspaces differ.
 *   - Every call is asynchronous on `stream` (0 = the null stream).
 *   - A return value other than MFD_OK means the call's outputs were not
 *     written: MFD_ERR_INVALID_ARG, MFD_ERR_DTYPE and MFD_ERR_WORKSPACE are
 *     found before any launch; after MFD_ERR_DEVICE, kernels of the call that
 *     were launched before the refused one may have written its workspace.
 *     A thread-local message is available from mfd_last_error().
 *   - Data-dependent problems are reported per tree in an optional device
 *     array `status` [N] (int32, bit flags OR-ed in; the caller zeroes it):
 *       MFD_TREE_NONFINITE        a NaN or +inf drafter logit in the tree
 *       MFD_TREE_CAPACITY         the tree exceeded a working capacity (see
 *                                 mfd_tree_build); that tree's outputs are
 *                                 not valid
 *       MFD_TREE_BAD_TEMPERATURE  temperature < 0 or not finite
 *       MFD_TREE_BAD_MODES        a per-tree mode count outside [1, K]
 *                                 (the *_modes calls; it is clamped)
 *   - Shapes: N trees, K modes, L drafted positions, V vocabulary, B budget
 *     (drafted nodes; the root is extra, so trees have B+1 rows), k = number
 *     of ranked candidates kept per row (use k = min(B, V)).
 *   - Scores are natural-log probabilities in fp64.
 *
 * Limits: 1 <= K <= 32, 1 <= L <= 32, 1 <= V < 2^20, 0 <= B <= 16383,
 *         1 <= k <= min(V, 2048); the tree calls also need K*k <= 16384.
 */
#ifndef MFDTREE_H
#define MFDTREE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enumerations are passed as int.  A C caller may pass any int value (a
 * value that is not an enumerator is rejected with an error); in C++ the
 * types therefore have int as their fixed underlying type, so every int is
 * a value of the type there too (without it, only the enumerators' range
 * would be). */
#ifdef __cplusplus
#define MFD_ENUM_BASE : int
#else
#define MFD_ENUM_BASE
#endif

typedef enum mfd_status MFD_ENUM_BASE {
  MFD_OK = 0,
  MFD_ERR_INVALID_ARG = 1, /* a size, pointer or flag is out of range */
  MFD_ERR_DTYPE = 2,       /* unsupported element type */
  MFD_ERR_WORKSPACE = 3,   /* workspace missing or smaller than mfd_workspace_size */
  MFD_ERR_DEVICE = 4       /* the HIP runtime refused a launch or query */
} mfd_status;

typedef enum mfd_dtype MFD_ENUM_BASE { MFD_BF16 = 0, MFD_F32 = 1 } mfd_dtype;

typedef enum mfd_op MFD_ENUM_BASE {
  MFD_OP_LOGSOFTMAX_TOPK = 0,
  MFD_OP_MIXTURE_THRESHOLD = 1,
  MFD_OP_TREE_BUILD = 2,
  MFD_OP_TREE_MASK = 3,
  MFD_OP_VERIFY_WALK = 4,
  MFD_OP_COVERED_MASS = 5,
  MFD_OP_LMHEAD_TOPK = 6,
  MFD_OP_MIXTURE_TREE = 7
} mfd_op;

#define MFD_TREE_NONFINITE 1
#define MFD_TREE_CAPACITY 2
#define MFD_TREE_BAD_TEMPERATURE 4
#define MFD_TREE_BAD_MODES 8

/* Message for the last failed call on this host thread ("" if none). */
const char* mfd_last_error(void);

/* Library version string. */
const char* mfd_version(void);

/* Bytes of device workspace the call `op` needs for these shapes (0 if none).
 * Arguments a call does not use are ignored.  Returns MFD_ERR_INVALID_ARG for
 * shapes outside the limits.  MFD_OP_VERIFY_WALK uses N, L (outside [1, 32]:
 * sized for L = 32), V (the target's vocabulary) and B (trees of B + 1 rows):
 * the size includes the arrays of the walk's speculative pass (see
 * mfd_verify_walk); with B < 0 or V < 1 it is the smaller size without them. */
mfd_status mfd_workspace_size(mfd_op op, int N, int K, int L, int V, int B, size_t* bytes);

/*
 * Per-(mode, position) log-softmax and top-k ("In one minute" and Figure 2:
 * each mode gives one distribution per position; step 3: the best-first
 * searches take each position's candidates from most to least probable).
 *
 *   logits    device [N, K, L, V], bf16 (MFD_BF16) or fp32 (MFD_F32), read once.
 *             Row r = (n, K, L) flattened; must be aligned to the element size.
 *   lse       device [N, K, L] fp64 out: log sum_v exp(logits[r, v]); -inf for
 *             a row of only -inf.  Never below the row's largest logit (as the
 *             exact value never is), so no log-probability is positive.
 *   topk_id   device [N, K, L, k] int32 out: token ids by logit descending,
 *             equal logits by id ascending (-0.0 and +0.0 are equal).
 *   topk_raw  device [N, K, L, k] fp32 out: the logit of each listed token,
 *             exactly (bf16 widened to fp32).
 *   topk_logp device [N, K, L, k] fp32 out or NULL: topk_raw - lse rounded to fp32.
 *   status    device [N] int32 or NULL: MFD_TREE_NONFINITE is OR-ed in for a
 *             tree with a NaN or +inf logit (its outputs are then unspecified).
 *   ws        unused (may be NULL; mfd_workspace_size reports 0).
 */
mfd_status mfd_logsoftmax_topk(const void* logits, mfd_dtype dtype, int N, int K, int L, int V, int k,
                               double* lse, int32_t* topk_id, float* topk_raw, float* topk_logp,
                               int32_t* status, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The same pass over a reduced drafting vocabulary (project page, "In a
 * serving engine": the drafter drafts over the target's 64K most frequent
 * tokens and the target verifies over the full vocabulary).  The logits cover
 * the V drafting tokens only; each listed token is reported by its id in the
 * full vocabulary of V_full tokens, so the tree and the walk work in target
 * ids.
 *
 *   vocab_map device [V] int32: full-vocabulary id of drafting token j, in
 *             strictly increasing order (the subset sorted by id), each in
 *             [0, V_full).  Ties between equal logits then break by full id
 *             exactly as in mfd_logsoftmax_topk over full-vocabulary logits
 *             that are -inf outside the subset.  Not checked on the device; a
 *             map out of order gives an unspecified tie order.
 *   V_full    size of the full vocabulary, V <= V_full < 2^20.
 *   Other arguments as for mfd_logsoftmax_topk; topk_id holds full ids.
 */
mfd_status mfd_logsoftmax_topk_mapped(const void* logits, mfd_dtype dtype, int N, int K, int L, int V,
                                      const int32_t* vocab_map, int V_full, int k, double* lse,
                                      int32_t* topk_id, float* topk_raw, float* topk_logp, int32_t* status,
                                      hipStream_t stream);

/*
 * The common cut-off ("In one minute": the B-th best score over all modes is
 * one cut-off shared by every mode; step 3: every prefix is scored by its best
 * mode).  A prefix t = (t_1..t_d), 1 <= d <= L, scores
 *     s_k(t) = (sum_{i<=d} raw_k(i, t_i)) - (sum_{i<=d} lse[k, i])
 * under mode k (both sums fp64, accumulated from i = 1 upward; an lse below
 * its row's first listed logit is taken as that logit, so that a prefix
 * never outscores its parent), and
 * S(t) = max_k s_k(t).  A mode scores only prefixes whose every token is among
 * its k listed candidates at that position (with k = min(B, V) this changes
 * nothing among the B best); -inf candidates never count.  Prefixes are
 * counted once however many modes reach them.
 *
 *   inputs    outputs of mfd_logsoftmax_topk for the same N, K, L, k.
 *   cutoff    device [N] fp64 out: S of the n_select-th best prefix
 *             (+inf when n_select is 0).
 *   n_select  device [N] int32 out: min(B, number of prefixes with finite S).
 *   per_mode_kept device [N, K] int32 out or NULL: number of prefixes with
 *             s_k >= cutoff under each mode ("each mode keeps the prefixes of
 *             its block that reach it").
 *   status    device [N] int32 or NULL: MFD_TREE_CAPACITY when a level of the
 *             search needs more than the working capacity.
 *   ws        device workspace of at least mfd_workspace_size(MFD_OP_MIXTURE_THRESHOLD).
 */
mfd_status mfd_mixture_threshold(const int32_t* topk_id, const float* topk_raw, const double* lse,
                                 int N, int K, int L, int k, int B,
                                 double* cutoff, int32_t* n_select, int32_t* per_mode_kept,
                                 int32_t* status, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The tree (project page, "In one minute": a prefix kept by several modes
 * becomes a single node; step 3: the B best prefixes over all modes form one
 * tree, the union of the per-mode trees).  Selects, among prefixes
 * with S >= cutoff, the first n_select in the order (S descending, best mode
 * ascending, token ids lexicographically ascending with a proper prefix first);
 * the best mode of a prefix is the lowest mode attaining S.  The selection is
 * prefix-closed.  Layout: row 0 is the root (anchor token, depth 0, parent -1,
 * score 0, best mode -1); rows 1..n_select are the selected prefixes sorted by
 * (depth, token sequence), so parent[i] < i and siblings are in token order.
 * Rows n_nodes..B are -1 (score -inf).
 *
 *   cutoff, n_select  device [N], normally from mfd_mixture_threshold.  Any
 *             cutoff at or below the true n_select-th score gives the same tree.
 *   anchor_token      device [N] int32: the committed token at the root.
 *   node_token, parent, depth, best_mode  device [N, B+1] int32 out.
 *   score     device [N, B+1] fp64 out: S of each node.
 *   n_nodes   device [N] int32 out: n_select + 1.
 *   status    device [N] int32 or NULL: MFD_TREE_CAPACITY if the prefixes
 *             reaching the cut-off exceed the working capacity, or more than
 *             2 C / (1 + L) prefixes tie exactly at the n_select-th score, with
 *             C = the next power of two of max(2 K k, 2 (B + 1), 2048), at most
 *             16384; that tree's rows are then not valid.
 *   ws        device workspace of at least mfd_workspace_size(MFD_OP_TREE_BUILD).
 */
mfd_status mfd_tree_build(const int32_t* topk_id, const float* topk_raw, const double* lse,
                          const double* cutoff, const int32_t* n_select, const int32_t* anchor_token,
                          int N, int K, int L, int k, int B,
                          int32_t* node_token, int32_t* parent, int32_t* depth, double* score,
                          int32_t* best_mode, int32_t* n_nodes, int32_t* status,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The cut-off and the tree together (project page, step 3: the union of the
 * per-mode trees is what one merged best-first search produces): the outputs
 * of mfd_mixture_threshold (cutoff, n_select, per_mode_kept) and of
 * mfd_tree_build at that cut-off (node_token .. n_nodes), bit for bit, from a
 * single search in one launch.  The search that finds the cut-off has by then
 * built every prefix that reaches it, with its best-mode score and best mode,
 * so the tree is laid out from those nodes instead of being searched for again.
 * Arguments, layouts, status flags and capacities as for the two calls; the
 * workspace is theirs (mfd_workspace_size with MFD_OP_MIXTURE_TREE, the same
 * size).  mfd_mixture_tree_modes: the same over the first K_n = modes[n] modes
 * of tree n (see the *_modes calls below).
 */
mfd_status mfd_mixture_tree(const int32_t* topk_id, const float* topk_raw, const double* lse,
                            const int32_t* anchor_token, int N, int K, int L, int k, int B,
                            double* cutoff, int32_t* n_select, int32_t* per_mode_kept,
                            int32_t* node_token, int32_t* parent, int32_t* depth, double* score,
                            int32_t* best_mode, int32_t* n_nodes, int32_t* status,
                            void* ws, size_t ws_bytes, hipStream_t stream);

mfd_status mfd_mixture_tree_modes(const int32_t* topk_id, const float* topk_raw, const double* lse,
                                  const int32_t* anchor_token, int N, int K, int L, int k, int B,
                                  const int32_t* modes, double* cutoff, int32_t* n_select,
                                  int32_t* per_mode_kept, int32_t* node_token, int32_t* parent,
                                  int32_t* depth, double* score, int32_t* best_mode, int32_t* n_nodes,
                                  int32_t* status, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Per-request mode count inside one batched launch (project page, "In a
 * serving engine": the MFD-D configuration runs the same drafter through a
 * single-mode default path once three or more requests are in flight, and is
 * the fastest option at every batch size of Figure 5).  Tree n is built from
 * its first K_n = modes[n] futures only; with K_n = 1 it is the single-future
 * (product) tree of that one mode.  The buffers keep the [N, K, L, ...]
 * layout of the calls above, so requests of any mode count share one launch.
 *
 *   modes     device [N] int32: K_n, in [1, K].  A value outside is clamped to
 *             it; the threshold and build calls then OR MFD_TREE_BAD_MODES into
 *             status (if not NULL).
 *
 * mfd_logsoftmax_topk_modes: as mfd_logsoftmax_topk, except that the rows of
 *   modes m >= K_n are neither read nor written (their lse, topk_* entries keep
 *   whatever the caller left there; the logits need not be computed).
 * mfd_mixture_threshold_modes, mfd_tree_build_modes: as mfd_mixture_threshold
 *   and mfd_tree_build over the first K_n modes of tree n; they read no row of
 *   a mode m >= K_n.  per_mode_kept is 0 for those modes.  The workspace is that
 *   of the full-K call (mfd_workspace_size with K).
 */
mfd_status mfd_logsoftmax_topk_modes(const void* logits, mfd_dtype dtype, int N, int K, int L, int V,
                                     const int32_t* modes, int k, double* lse, int32_t* topk_id,
                                     float* topk_raw, float* topk_logp, int32_t* status, hipStream_t stream);

mfd_status mfd_mixture_threshold_modes(const int32_t* topk_id, const float* topk_raw, const double* lse,
                                       int N, int K, int L, int k, int B, const int32_t* modes,
                                       double* cutoff, int32_t* n_select, int32_t* per_mode_kept,
                                       int32_t* status, void* ws, size_t ws_bytes, hipStream_t stream);

mfd_status mfd_tree_build_modes(const int32_t* topk_id, const float* topk_raw, const double* lse,
                                const double* cutoff, const int32_t* n_select, const int32_t* anchor_token,
                                int N, int K, int L, int k, int B, const int32_t* modes,
                                int32_t* node_token, int32_t* parent, int32_t* depth, double* score,
                                int32_t* best_mode, int32_t* n_nodes, int32_t* status,
                                void* ws, size_t ws_bytes, hipStream_t stream);

typedef enum mfd_head_layout MFD_ENUM_BASE { MFD_HEAD_ROWS = 0, MFD_HEAD_PACKED = 1 } mfd_head_layout;

/*
 * Packed LM head for the fused calls (a one-time re-layout of the weights,
 * for callers who stream the same head every round).  Rows are padded with
 * zeros to a multiple of 256 and cut into blocks of 64 rows x 32 columns;
 * block (vb, s) (rows 64 vb.., columns 32 s..) is stored contiguously at
 * element ((vb * D / 32) + s) * 2048, row-major inside the block.
 *
 *   mfd_lmhead_packed_size: bytes of the packed head, ceil(V / 256) * 256 * D * 2.
 *   weight  device [V, D] bf16, 16-byte aligned; packed: device, 16-byte
 *           aligned, at least mfd_lmhead_packed_size bytes, caller-owned.
 *   Errors: MFD_ERR_INVALID_ARG for V or D outside the fused call's limits,
 *           NULL or misaligned pointers, or a small packed buffer.
 */
mfd_status mfd_lmhead_packed_size(int V, int D, size_t* bytes);
mfd_status mfd_lmhead_pack_weight(const void* weight, int V, int D, void* packed, size_t packed_bytes,
                                  hipStream_t stream);

/*
 * Fused LM head + per-(mode, position) log-softmax and top-k.  The drafter
 * uses its target's LM head at run time (model card "MFD drafter for
 * Qwen3.5-4B", "Model" and "Parameters"), and the pages' interface runs the
 * tree step with fused_logits=True (same card, "Usage").  The logits
 * x[r, v] = sum_d hidden[r, d] * weight[v, d] are formed on the matrix cores
 * (bf16 products, exact; fp32 accumulation) and reduced in the same pass, so
 * the [N, K, L, V] logits are never written.  Outputs are those of
 * mfd_logsoftmax_topk over x.
 *
 *   hidden    device [N, K, L, D] bf16: the drafter's final hidden states, row
 *             r = (n, k, i); 16-byte aligned.
 *   weight    device bf16, 16-byte aligned: the LM head.  layout MFD_HEAD_ROWS:
 *             [V, D], one row per token.  layout MFD_HEAD_PACKED: the same head
 *             re-laid out once by mfd_lmhead_pack_weight, so every 64-row x
 *             32-column block a tile reads per step is one contiguous 4 KB
 *             run.  Results are identical for both layouts.
 *   D         hidden width, a multiple of 64 in [64, 16384]; N*K*L*D and V*D
 *             must be below 2^31.
 *   lse, topk_id, topk_raw, topk_logp: as for mfd_logsoftmax_topk; topk_raw
 *             is the fp32 logit as accumulated (ties break by token id).
 *   status    device [N] int32 or NULL: MFD_TREE_NONFINITE for a tree with a
 *             non-finite logit; MFD_TREE_CAPACITY for a tree with a row whose
 *             candidate list overflowed the workspace (rows whose logits pile
 *             up at one value, e.g. all equal).  That row's topk_id is -1 and
 *             topk_raw -inf; its lse is valid.  Such a tree can be redone
 *             unfused (write the logits, call mfd_logsoftmax_topk).
 *   ws        device workspace of at least mfd_workspace_size(MFD_OP_LMHEAD_TOPK,
 *             N, K, L, V, k) bytes (B = k there), 256-byte aligned.  Its
 *             contents on entry do not matter.
 *
 * Errors (nothing launched): MFD_ERR_INVALID_ARG for shapes outside the limits
 * above, k outside [1, min(V, 2048)], NULL or misaligned pointers;
 * MFD_ERR_WORKSPACE for a missing, small or misaligned workspace.
 */
mfd_status mfd_lmhead_logsoftmax_topk(const void* hidden, const void* weight, mfd_head_layout layout, int N,
                                      int K, int L, int D, int V, int k, double* lse, int32_t* topk_id,
                                      float* topk_raw, float* topk_logp, int32_t* status, void* ws,
                                      size_t ws_bytes, hipStream_t stream);

/*
 * The fused call over a reduced drafting vocabulary (project page, "In a
 * serving engine": drafting over the target's 64K most frequent tokens,
 * verification over the full vocabulary).  `weight` holds the LM-head rows
 * of the V drafting tokens only, in increasing order of their full ids
 * vocab_map[0..V); each listed token is reported by its full id, and equal
 * logits break ties by full id.  The workspace is that of
 * mfd_lmhead_logsoftmax_topk with this V.
 *
 *   vocab_map device [V] int32, strictly increasing, each in [0, V_full).
 *   V_full    size of the full vocabulary, V <= V_full < 2^20.
 *   Other arguments as for mfd_lmhead_logsoftmax_topk.
 */
mfd_status mfd_lmhead_logsoftmax_topk_mapped(const void* hidden, const void* weight, mfd_head_layout layout,
                                             const int32_t* vocab_map, int V_full, int N, int K, int L, int D, int V,
                                             int k, double* lse, int32_t* topk_id, float* topk_raw,
                                             float* topk_logp, int32_t* status, void* ws, size_t ws_bytes,
                                             hipStream_t stream);

/*
 * Tree-verification inputs (model card summary: the target checks the whole
 * tree in one pass with standard tree verification).  Row i of the mask has
 * bit j set iff node j is node i or one of its ancestors (the root included).
 *
 *   parent, depth  device [N, Bp1] int32, n_nodes device [N] int32 (from mfd_tree_build).
 *   pos_base  device [N] int64: position id of the root.
 *   mask_words device [N, Bp1, W] uint64 out, W = ceil(Bp1 / 64); column j is
 *             bit (j % 64) of word j / 64.  Rows and columns >= n_nodes are 0.
 *   position_ids device [N, Bp1] int64 out: pos_base + depth; -1 for rows >= n_nodes.
 *   dense_mask device [N, Bp1, Bp1] uint8 out or NULL: the same mask, one byte per entry.
 */
mfd_status mfd_tree_mask(const int32_t* parent, const int32_t* depth, const int32_t* n_nodes,
                         const int64_t* pos_base, int N, int Bp1,
                         uint64_t* mask_words, int64_t* position_ids, uint8_t* dense_mask,
                         hipStream_t stream);

/*
 * Verification walk (model card summary and project page Figure 2: the target
 * keeps the future it takes; accepted drafted tokens plus one bonus token).
 * From the root u = 0: the target's token at u is t* = argmax_v R[u, v] at
 * T = 0 (equal logits to the lower id), or at T > 0 the Gumbel-max sample
 *     t* = argmax_v ( fp64(R[u, v]) / fp64(T) + g_v ),  g_v = -log(-log(U_v)),
 *     U_v = (w_v + 1/2) * 2^-32,
 *     w_v = word (v mod 4) of Philox4x32-10(counter = (v div 4, depth(u), 0, 0),
 *                                           key = (seed[n] mod 2^32, seed[n] div 2^32))
 * (Salmon et al., "Parallel random numbers: as easy as 1, 2, 3", SC'11).  The
 * kernel ranks fp32 estimates of these values first and evaluates the exact
 * fp64 ones only for elements within the estimates' error bound of the best,
 * so the winner is that of the fp64 values.
 * If u has a child with token t*, the walk moves there and repeats; else it
 * stops with tau = depth(u) + 1.
 *
 *   target_logits device [N, Bp1, V] bf16 or fp32: the target's logits at each
 *             node (only the rows on the walked path are read).
 *   node_token, parent, depth, n_nodes  the tree (from mfd_tree_build).
 *   temperature device [N] fp32; seed device [N] uint64.
 *   tau       device [N] int32 out (1..L+1; 0 with MFD_TREE_BAD_TEMPERATURE).
 *   out_tokens device [N, L+1] int32 out: accepted drafted tokens then the
 *             bonus token; -1 after.
 *   path_nodes device [N, L+1] int32 out: rows visited, root first; -1 after.
 *   status    device [N] int32 or NULL: MFD_TREE_BAD_TEMPERATURE; MFD_TREE_CAPACITY
 *             if the call gave up waiting for work to finish (a bounded wait,
 *             seconds long, that never runs out in a correct run; tau is then 0).
 *   ws        device workspace, 8-byte aligned, of at least
 *             mfd_workspace_size(MFD_OP_VERIFY_WALK, N, .., L, V, B) bytes
 *             with B < 0 (per tree: its first round, and a result slot and
 *             flag per round and slice; set up by the call itself, so it
 *             needs no clearing).  With the size for the trees' B and the
 *             target's V it also holds the speculative pass's arrays.
 * Each visited row is cut into slices, one per workgroup of the tree's
 * group; each slice's result goes to a slot of its own round, and every
 * workgroup of the group merges the round from the slots itself.  A
 * workgroup that sees no progress for a while computes a missing slice
 * (results are the same whoever computes them), so none depends on another
 * being resident (an ordinary launch: any number of processes may walk on
 * one GPU).  Calls on one stream are ordered; calls that overlap must not
 * share `ws`.
 * Speculative pass: the token chosen at a node depends only on that node's
 * row, T, the seed and its depth.  When the workspace holds the pass's arrays
 * and the rows are few enough (every node's row up to 160 MiB per launch,
 * else the rows of nodes that have a child up to 400 MiB), those rows are
 * reduced first, in parallel over all workgroups, and each tree is walked
 * along the chosen tokens at once; the walk proper then reads at most the
 * last node's row.  The outputs are the same bit for bit either way.
 */
mfd_status mfd_verify_walk(const void* target_logits, mfd_dtype dtype, int N, int Bp1, int V, int L,
                           const int32_t* node_token, const int32_t* parent, const int32_t* depth,
                           const int32_t* n_nodes, const float* temperature, const uint64_t* seed,
                           int32_t* tau, int32_t* out_tokens, int32_t* path_nodes, int32_t* status,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * mfd_verify_walk without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The call itself allocates nothing (no
 * hipMalloc, hipFree or allocating library routine).  The walk's workspace
 * is a built-in 16 MiB device array of the library, one copy per GPU, held
 * until the process ends; its address on a device is looked up on the first
 * call made with that device current.  Same arguments, outputs and errors as
 * mfd_verify_walk, plus:
 *   - N is at most the number of trees whose walk workspace
 *     (mfd_workspace_size(MFD_OP_VERIFY_WALK, N, 0, L, 0, -1)) fits 16 MiB:
 *     511 at L = 15, 248 at L = 32; a larger N returns MFD_ERR_WORKSPACE
 *     before any launch.
 *   - The call clears what must start at zero itself; the array keeps the
 *     last call's contents otherwise.
 *   - The speculative pass of mfd_verify_walk runs when its arrays fit in
 *     what the walk proper leaves of the 16 MiB (same outputs either way).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap on
 *     a GPU (different streams, or other threads, without ordering between
 *     them) race and give wrong results.  Calls on one stream are ordered.
 */
mfd_status mfd_verify_walk_noalloc(const void* target_logits, mfd_dtype dtype, int N, int Bp1, int V, int L,
                                   const int32_t* node_token, const int32_t* parent, const int32_t* depth,
                                   const int32_t* n_nodes, const float* temperature, const uint64_t* seed,
                                   int32_t* tau, int32_t* out_tokens, int32_t* path_nodes, int32_t* status,
                                   hipStream_t stream);

/*
 * Covered target mass of each tree (project page, "Abstract": under tree
 * verification the expected number of accepted drafted tokens is the
 * probability mass the tree covers).  For tree n at temperature T = T[n]:
 *     mass[n] = sum over drafted nodes v of  prod over the edges (u -> w) on
 *               the path root .. v of  p_T(token(w) | row u),
 *     p_T(t | u) = exp(R[u, t] / T) / sum_v exp(R[u, v] / T)      (T > 0),
 *     p_0(t | u) = 1 if t is the lowest-id argmax of R[u, :], else 0.
 * At T = 0 the mass is the greedy walk's number of accepted drafted tokens.
 *
 *   target_logits device [N, Bp1, V] bf16 or fp32: the rows of the nodes that
 *             have a child are read (twice at T > 0, once at T = 0).
 *   node_token, parent, n_nodes  the tree (any node order; a parent outside
 *             the tree, or a token outside [0, V), makes the mass NaN).
 *   temperature device [N] fp32; T < 0 or not finite gives NaN and
 *             MFD_TREE_BAD_TEMPERATURE in status (if not NULL).
 *   mass      device [N] fp64 out.
 *   ws        device workspace of mfd_workspace_size(MFD_OP_COVERED_MASS, N,
 *             0, 0, 0, Bp1 - 1) bytes (per-node normalisers).
 * N is at most 65535.  Row probabilities use fp32 exponentials summed in fp64
 * (relative error about 1e-7 per edge).
 */
mfd_status mfd_covered_mass(const void* target_logits, mfd_dtype dtype, int N, int Bp1, int V,
                            const int32_t* node_token, const int32_t* parent, const int32_t* n_nodes,
                            const float* temperature, double* mass, int32_t* status, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * Chimeras of each tree relative to two futures (project page, "TL;DR" and
 * "Abstract": prefixes stitched together from different futures, which the
 * target never produces).  count[n] = number of drafted nodes whose token at
 * every depth d is future_a[n][d-1] or future_b[n][d-1] while their path is a
 * prefix of neither future.
 *
 *   node_token, parent, depth, n_nodes  the tree (depth d in [1, L] for drafted
 *             nodes; a node whose path leaves the tree or [1, L] is not counted).
 *   future_a, future_b  device [N, L] int32.
 *   count     device [N] int32 out.
 */
mfd_status mfd_chimera_count(const int32_t* node_token, const int32_t* parent, const int32_t* depth,
                             const int32_t* n_nodes, int N, int Bp1, int L, const int32_t* future_a,
                             const int32_t* future_b, int32_t* count, hipStream_t stream);

/*
 * Measurement reference, not a step of the method: reads `bytes` bytes of
 * device memory once (16-byte nontemporal loads spread over every compute
 * unit) and XORs every 32-bit word into *sink.  Its rate is the HBM read rate
 * that a pass reading its input exactly once can reach on this device, the
 * achievable ceiling for mfd_logsoftmax_topk beside the nominal peak.
 *
 *   buf    device, 16-byte aligned (may be NULL when bytes is 0).
 *   bytes  a multiple of 16; MFD_ERR_INVALID_ARG otherwise.
 *   sink   device [1] uint32, caller-initialised: *sink ^= XOR of all words.
 */
mfd_status mfd_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MFDTREE_H */
