/*
 * libspecverify -- the verification step of tree speculative decoding on one
 * AMD Instinct MI355X (gfx950).
 *
 * One verify step is four calls, issued in this order on one HIP stream:
 *
 *   sv_build_tree_mask  parent array -> ancestor bitsets, depths, path rows
 *   sv_tree_attention   ancestor-masked GQA attention of the draft-tree query
 *                       tokens over a contiguous or paged KV prefix
 *   sv_accept           greedy argmax matching, full-distribution rejection
 *                       sampling with the residual normalize(max(0, p - q)),
 *                       deterministic (top-K) drafts or threshold acceptance,
 *                       plus the bonus token (it can also run the commit)
 *   sv_kv_commit        copy the accepted branch's KV rows into the cache
 *
 * Around the step: sv_outcome_lookup and sv_saguaro_reweight (speculative
 * speculative decoding) and sv_draft_subset_logits (drafters on a vocabulary
 * subset).
 *
 * Sources (web pages, cited by title and section):
 *  [EP]  "EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on Ascend
 *        NPUs" (gist.science summary), technical summary sec. 2 Metodologia:
 *        branchable KV cache, commit by length or by path indices; shifted
 *        indexing with a dummy root row 0 in place of the -1 sentinel;
 *        ancestor index tables; range, acyclicity and depth checks before the
 *        fused kernels; tree attention mask (a token sees itself and its
 *        ancestors only).
 *  [PX]  "Accelerating Sonar Through Speculation" (Perplexity), sections
 *        "Decodificacion Especulativa", "Objetivo-Borrador", "EAGLE",
 *        "Inferencia con Decodificacion Especulativa": n drafted tokens give
 *        up to n+1 emitted tokens; the longest acceptable sequence is kept;
 *        acceptance compares full draft and target distributions; the target
 *        logits after the accepted sequence give a bonus token; the accepted
 *        count forces a GPU->CPU sync unless device work consumes it.
 *  [SSD] "Speculative Speculative Decoding" (gist.science summary), sec. 3B
 *        (residual probability mass), sec. 5 (exact output distribution).
 *
 * Conventions shared by every call
 *  - Tree node i in [0, N) owns row r = i + 1.  Row 0 is the root: the last
 *    committed token, whose KV is already in the prefix and whose target and
 *    draft logits are row 0 of the logits tensors ([EP] sec. 2 dummy row).
 *    parents[i] = -1 means "child of the root"; no call ever forms a negative
 *    index from it.
 *  - All pointers are device pointers unless stated; the caller owns every
 *    buffer.  The library allocates nothing, never synchronises the stream
 *    and never copies to the host: calls only enqueue kernels on `stream`
 *    (a hipStream_t, or NULL for the null stream).  It is stateless and
 *    reentrant.
 *  - Argument and shape problems are returned synchronously as a non-zero
 *    sv_status and nothing is enqueued.  Data-dependent problems (a malformed
 *    tree, a token id out of range, a ghost block table entry, capacity) are
 *    written as per-sequence codes into a caller-provided device `status`
 *    array; kernels then clamp the offending index to the ghost row / slot 0
 *    and never dereference a negative or out-of-range index.
 *  - Limits: 1 <= N <= 256, 1 <= max_depth <= 16, head_dim in {64, 128},
 *    Hq % Hkv == 0 with Hq/Hkv <= 16, block_size 16, V >= 1.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sv_status;
#define SV_OK 0
#define SV_ERR_INVALID_ARGUMENT 1
#define SV_ERR_UNSUPPORTED 2
#define SV_ERR_BAD_TREE 3          /* SV_FLAG_VALIDATE: a sequence's device status is non-zero (read back by the call) */
#define SV_ERR_HIP 4
#define SV_ERR_SCRATCH_LIMIT 5     /* sv_accept_noalloc: the call needs more than SV_ACCEPT_SCRATCH_BYTES */

/* element types */
#define SV_F32 0
#define SV_BF16 1

/* acceptance modes */
#define SV_GREEDY 0
#define SV_STOCHASTIC 1
#define SV_TOPK_DRAFT 2
#define SV_THRESHOLD 3

/* call flags.  SV_FLAG_VALIDATE selects the reference mode of [EP] sec. 2
 * ("Metodologia": a reference mode with invariant checks next to the fast
 * fused path): the call additionally checks its inputs, waits for the stream,
 * reads the per-sequence status back and returns SV_ERR_BAD_TREE when any
 * sequence reports a non-zero code.  It synchronises the stream (so it is
 * rejected with SV_ERR_INVALID_ARGUMENT while the stream is being captured).
 * Without it (performance mode) a call only enqueues work. */
#define SV_FLAG_VALIDATE 1u
/* SV_FLAG_ROW_LIST (sv_accept only): greedy batches of at least 512 logits rows whose B*(N+1)
 * rows fit 4352, and threshold batches (mode 3), resolve every row that has a usable child --
 * greedy: the batch's needed rows streamed as one list; threshold: the statistics of every such
 * row, then one walk per sequence -- instead of following each sequence's accepted (passing)
 * paths row by row (which reads only those paths' rows and the stop row, and which the call
 * picks by itself when the rows would be many bytes).  The results are the same; other calls
 * ignore the flag. */
#define SV_FLAG_ROW_LIST 2u

/* commit modes ([EP] sec. 2: length-based or path-index-based commit) */
#define SV_COMMIT_PATH 0
#define SV_COMMIT_LENGTH 1

/* per-sequence device status codes */
#define SV_SEQ_OK 0
#define SV_SEQ_PARENT_RANGE 1   /* a parent index outside [-1, N), or accept data out of range */
#define SV_SEQ_CYCLE 2          /* a node reaches itself by following parents */
#define SV_SEQ_DEPTH 3          /* a root path longer than max_depth */
#define SV_SEQ_TOKEN 4          /* a draft token id outside [0, V) */
#define SV_SEQ_BLOCK 5          /* a needed block-table entry is 0 (ghost) or outside the pool */
#define SV_SEQ_CAPACITY 6       /* prefix_len (+ accepted rows) exceeds the cache capacity */
#define SV_SEQ_TIMEOUT 7        /* sv_accept: a bounded wait between cooperating work-groups expired */
#define SV_SEQ_NONFINITE 8      /* sv_accept: a logits row holds NaN or +Inf, or no finite entry */

/*
 * sv_build_tree_mask -- tree tensorisation ([EP] sec. 2, "Semantica de
 * Tensores de Arbol Segura").
 *   parents   [B, N] int32, values in {-1} U [0, N); any order (need not be
 *             topologically sorted).
 *   anc_bits  [B, N, W] uint64, W = ceil(N/64): bit j of node i is set iff j
 *             lies on the root path of i (i itself included) -- the tree
 *             attention mask of [EP] sec. 2.
 *   depth     [B, N] int32: number of nodes on the root path of i (1 for a
 *             child of the root); 0 marks an invalid node.
 *   path_rows [B, N+1, max_depth] int32 or NULL: row r = i+1 lists the rows of
 *             the root path of node i, root-most first, padded with the ghost
 *             row 0; row 0 is all 0 (ancestor index tables, [EP] sec. 2).
 *   status    [B] int32: 0, or the smallest code among the sequence's nodes.
 * Checks per node while walking up (in this order): parent in [-1, N) (code
 * 1), parent not already on the walk (code 2), path length <= max_depth
 * (code 3).  The walk stops at the first failing check, so a cycle longer
 * than max_depth reports code 3.  An invalid node gets anc_bits = {i}, depth
 * 0 and an all-ghost path row; valid nodes are unaffected by invalid ones.
 * flags: 0, or SV_FLAG_VALIDATE (wait, read status back, SV_ERR_BAD_TREE for
 * a malformed tree in any sequence).
 */
sv_status sv_build_tree_mask(const int32_t* parents, int32_t B, int32_t N, int32_t max_depth,
                             uint64_t* anc_bits, int32_t* depth, int32_t* path_rows, int32_t* status,
                             uint32_t flags, void* stream);

/*
 * sv_tree_attention -- ancestor-masked GQA attention of the tree's query
 * tokens ([EP] sec. 2, "Ejecucion del Maestro con Mascara de Arbol
 * Fusionada").  For batch b, query head h, KV head g = h / (Hq/Hkv), node i:
 *     keys   = prefix positions j in [0, prefix_len[b])  (cache)
 *              then tree nodes t with bit t of anc_bits[b,i] (k_tree row t+1)
 *     out[b,i,h,:] = sum_j softmax_j(scale * q.k_j) v_j
 * Layouts (element type `dtype` for q, caches, tree KV and out):
 *     q        [B, N, Hq, D]
 *     k_cache, v_cache: contiguous [B, Hkv, Lcap, D], or paged
 *              [num_blocks, Hkv, block_size, D] with block_table [B, max_blocks]
 *              (block 0 is the ghost block and is never a valid entry)
 *     k_tree, v_tree [B, Hkv, N+1, D]: the tree tokens' K/V, row 0 = ghost
 *              (never read as a key)
 *     anc_bits [B, N, ceil(N/64)] from sv_build_tree_mask
 *     prefix_len [B] int32 (device)
 *     out      [B, N, Hq, D]
 * Scale: the caller passes it (1/sqrt(D) for standard attention); no rotary
 * embedding, soft-capping or bias is applied inside.
 * workspace: device scratch of at least sv_tree_attention_workspace(args)
 * bytes (may be 0), 256-byte aligned.
 * status (nullable) [B]: 5 if a needed block-table entry is 0 or >=
 * num_blocks (read as the ghost block), 6 if prefix_len is outside
 * [0, capacity] (clamped).
 * tree_in_cache (0 or 1): 1 keeps the tree tokens' K/V inside the cache
 *   itself, as the speculative region after the prefix ([EP] sec. 2: the
 *   committed prefix and the per-branch speculative state of one cache, then
 *   committed in place).  Node t's key is then cache position prefix_len[b] + t
 *   (through the block table when paged), k_tree / v_tree are not read (may be
 *   NULL), the capacity left for the prefix is capacity - N (status 6 and a
 *   clamped prefix beyond it), the blocks of positions [0, prefix_len + N) are
 *   the needed ones, and capacity >= N is required (else
 *   SV_ERR_INVALID_ARGUMENT).
 */
typedef struct sv_attn_args {
  int32_t B, N, Hq, Hkv, D, dtype;
  float scale;
  int32_t paged;                  /* 0 contiguous, 1 paged */
  int32_t Lcap;                   /* contiguous capacity per sequence */
  int32_t block_size, max_blocks, num_blocks;  /* paged geometry */
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const void* k_tree;
  const void* v_tree;
  const int32_t* block_table;
  const int32_t* prefix_len;
  const uint64_t* anc_bits;
  void* out;
  void* workspace;
  size_t workspace_bytes;
  int32_t* status;
  int32_t tree_in_cache;
} sv_attn_args;
size_t sv_tree_attention_workspace(const sv_attn_args* args);
sv_status sv_tree_attention(const sv_attn_args* args, void* stream);

/*
 * sv_accept -- speculative acceptance and the bonus token ([PX], [SSD]).
 * Inputs:
 *   parents [B,N], tokens [B,N] int32 (draft token of node i), anc_bits and
 *   depth from sv_build_tree_mask (modes 0, 1 and 2 may pass both as NULL:
 *   the kernel then derives each node's depth from parents by the same rule
 *   -- the node count of its root path when that path reaches -1 through
 *   in-range parents within max_depth nodes, else 0 -- and the call does not
 *   wait for the mask; mode 3 returns SV_ERR_INVALID_ARGUMENT for a NULL
 *   one); target_logits [B, N+1, V] (row r = the
 *   target's next-token logits after row r's token, row 0 = the root);
 *   draft_logits [B, N+1, V] (mode 1 only; row r = the drafter's logits
 *   its children were drawn from); u_accept, u_sample [B, N+1] float
 *   uniforms in [0,1) (modes 1 and 2).
 * A node is usable when its depth is > 0 and its token lies in [0, V).
 * Greedy (mode 0): a_r = argmax of target row r over the stored values, the
 *   lowest id on ties.  Node i matches when tokens[i] == a_{parents[i]+1};
 *   it is accepted when every node of its root path is usable and matches.
 *   The stop node is the deepest accepted node (lowest index on ties), or
 *   the root when none; A = its depth; bonus = a_{stop row}.
 * Stochastic (mode 1), p_r = softmax(target row r / T), q_r = softmax(draft
 *   row r / T), exponentials in fp32 and sums over V in fp64:
 *   start at row 0 with p_cur = p_0; test the usable children c of the
 *   current row in ascending index, with x = tokens[c]: accept iff
 *   u_accept[c+1] < p_cur(x)/q_r(x) (q_r(x) = 0 accepts); on accept move to
 *   row c+1 with p_cur = p_{c+1}; on reject replace p_cur by
 *   normalize(max(0, p_cur - q_r)).  When no child is accepted the walk stops
 *   at the current row and the bonus is the smallest v whose ascending-id
 *   cumulative mass of p_cur exceeds u_sample[stop row] times its total.
 * Top-K drafts (mode 2): the drafter proposed every child deterministically
 *   (its top candidates, [PX] "Objetivo-Borrador" and "EAGLE"), so its
 *   proposal for child c is the point mass at x = tokens[c]; draft_logits is
 *   not read (may be NULL).  The walk is mode 1's with that proposal: accept
 *   iff u_accept[c+1] < p_cur(x); a rejection sets p_cur(x) to 0 and
 *   renormalises (sampling without replacement), so a token repeated among
 *   siblings is never accepted twice.  p(x) is taken from the row statistics
 *   with no second pass over the row; the bonus is drawn from p_r with the
 *   rejected tokens removed, as in mode 1 (if rounding leaves that residual
 *   without mass, from p_r itself).
 * Threshold (mode 3, [PX] "Decodificacion Especulativa": every prefix of the
 *   candidates is scored with a probability and the longest one above an
 *   acceptance threshold is kept, plus one target token): the score of node i
 *   is the product over its root path of p_{parent row}(token), p_r =
 *   softmax(target row r / T) (fp32 exponentials, fp64 sums and products);
 *   node i is accepted when every node of its path is usable and its score is
 *   >= threshold (0 <= threshold <= 1, else SV_ERR_INVALID_ARGUMENT); the stop
 *   node is the deepest accepted node (lowest index on ties), or the root; the
 *   bonus is the argmax of the stop row (lowest id on ties).  draft_logits,
 *   u_accept and u_sample are not read (may be NULL).
 * Outputs (device, int32): accept_len [B] (A), accept_rows [B, max_depth]
 *   (rows of the accepted path, root-most first, ghost-0 padded), out_tokens
 *   [B, max_depth+1] (accepted tokens then the bonus, 0 padded), num_out [B]
 *   (A+1), stop_row [B], status [B] (4 if some token id is out of range; 8
 *   if the walk reached a row whose statistics are not finite, see below).
 * Non-finite logits.  Modes 1 and 2 check every row they resolve: a row whose
 *   softmax normaliser is not a finite positive number (a NaN or +Inf logit,
 *   or no finite entry; -Inf entries alone are probability 0 and allowed)
 *   accepts no child and gives bonus 0, and a walk that stops there reports
 *   status 8.  With SV_FLAG_VALIDATE (flags) every row of target_logits (and
 *   of draft_logits in mode 1) is scanned after the acceptance: a row with a
 *   NaN or +Inf entry, or with no finite entry, sets status 8 for its
 *   sequence unless an earlier code is set; the call then waits for the
 *   stream and returns SV_ERR_BAD_TREE if any status is non-zero.
 * workspace: at least sv_accept_workspace(args) bytes, 256-byte aligned,
 *   zero-filled by the caller before its first use; every call leaves it
 *   zeroed again.  Calls that overlap in time must not share a workspace.
 *   The work-groups that share one logits row wait for each other with a
 *   bounded spin; if one never arrives (the device could not hold the whole
 *   persistent grid at once) the wait expires and every sequence of the call
 *   reports status 7 instead of hanging.
 */
typedef struct sv_accept_args {
  int32_t B, N, V, max_depth, logits_dtype, mode;
  float temperature;
  const int32_t* parents;
  const int32_t* tokens;
  const uint64_t* anc_bits;
  const int32_t* depth;
  const void* target_logits;
  const void* draft_logits;
  const float* u_accept;
  const float* u_sample;
  int32_t* accept_len;
  int32_t* accept_rows;
  int32_t* out_tokens;
  int32_t* num_out;
  int32_t* stop_row;
  int32_t* status;
  void* workspace;
  size_t workspace_bytes;
  float threshold;  /* mode 3 only */
  /* nullable: the acceptance kernel also commits each sequence's accepted path, as
   * sv_kv_commit(commit) would after it (same checks and outputs), from the work-group that
   * found the path -- one launch less.  Its B, N and max_depth must equal these; only a
   * single layer with the tree rows in their own tensor (else SV_ERR_UNSUPPORTED); the
   * struct is read at call time.  The commit writes cache positions >= prefix_len only, but it
   * writes new_len, so new_len must not alias prefix_len while anything that reads prefix_len
   * (sv_tree_attention) may still run beside it. */
  const struct sv_commit_args* commit;
  uint32_t flags;   /* 0, or SV_FLAG_VALIDATE and/or SV_FLAG_ROW_LIST */
} sv_accept_args;
size_t sv_accept_workspace(const sv_accept_args* args);
sv_status sv_accept(const sv_accept_args* args, void* stream);

/*
 * sv_accept_noalloc -- sv_accept for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments and outputs as sv_accept, but
 * args->workspace and args->workspace_bytes are ignored and the workspace is
 * a library-owned device array of SV_ACCEPT_SCRATCH_BYTES (4 MiB) per GPU,
 * kept until the process ends.  Nothing is allocated by the call: no hipMalloc,
 * hipFree or allocating library routine.  The first call on a device looks up
 * the array's address (hipGetSymbolAddress) and enqueues one clearing kernel on
 * `stream` before the acceptance kernels; later calls enqueue only those.
 * Calls whose workspace (sv_accept_workspace) would exceed the array return
 * SV_ERR_SCRATCH_LIMIT and enqueue nothing.  Every call on one GPU shares the
 * array and leaves it zeroed: calls that overlap in time on one GPU (several
 * streams, several host threads) race and must be serialised by the caller.
 */
#define SV_ACCEPT_SCRATCH_BYTES (4u << 20)
sv_status sv_accept_noalloc(const sv_accept_args* args, void* stream);

/*
 * sv_kv_commit -- append the accepted branch's KV to the cache ([EP] sec. 2,
 * "Gestion de Cache KV Ramificada").  For sequence b with L = prefix_len[b]
 * and A = accept_len[b], for k < A the tree row src_k (accept_rows[b,k] in
 * path mode, k+1 in length mode) of k_tree / v_tree is copied, for every KV
 * head, to position L + k: contiguous slot L + k of [B, Hkv, Lcap, D], or
 * paged slot block_table[b][(L+k)/bs]*bs + (L+k)%bs of [num_blocks, Hkv, bs,
 * D].  committed_slots [B, max_depth] receives the slots (0 for k >= A) and
 * new_len [B] = L + A (new_len may alias prefix_len).
 * Before any write, every k < A is checked in order; the first failure sets
 * status[b] (1: A outside [0, max_depth] or a source row outside [1, N];
 * 5: ghost or out-of-pool block; 6: beyond capacity) and then nothing of that
 * sequence is written: new_len = L, committed_slots all 0.
 * Element size follows dtype (SV_F32 4 bytes, SV_BF16 2 bytes).
 *
 * tree_in_cache (0 or 1): the tree rows live in the cache at positions L + t
 *   (node t, as in sv_tree_attention); k_tree / v_tree are not read (may be
 *   NULL).  The commit is then an in-place compaction of the accepted path:
 *   position L + k receives what position L + src_k - 1 held before the call
 *   (every source row is read before any row is written, so the order of the
 *   path does not matter), and a row already in place (src_k - 1 == k, e.g.
 *   every row in length mode) is not moved at all ([EP] sec. 2: the path-index
 *   commit avoids needless memory moves).  Checks add: L + N within the
 *   capacity (6) and valid blocks for the source positions (5).  The blocks of
 *   positions [L, L + N) must belong to this sequence alone.
 * num_layers (>= 1; 0 is read as 1): commits that many layers in one launch.
 *   Layer l's caches start cache_layer_stride elements after layer l-1's (both
 *   k_cache and v_cache), its tree rows tree_layer_stride elements after layer
 *   l-1's; every layer shares prefix_len, the accepted rows and the block
 *   table, so the checks, new_len, committed_slots and status are those of one
 *   layer.  Strides of 0 with num_layers > 1 are rejected.
 */
typedef struct sv_commit_args {
  int32_t B, N, Hkv, D, dtype, max_depth, commit_mode;
  int32_t paged, Lcap, block_size, max_blocks, num_blocks;
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;
  const void* k_tree;
  const void* v_tree;
  const int32_t* prefix_len;
  const int32_t* accept_len;
  const int32_t* accept_rows;
  int32_t* new_len;
  int32_t* committed_slots;
  int32_t* status;
  int32_t tree_in_cache;
  int32_t num_layers;
  int64_t cache_layer_stride;
  int64_t tree_layer_stride;
} sv_commit_args;
sv_status sv_kv_commit(const sv_commit_args* args, void* stream);

/*
 * sv_verify_step -- the whole verification step in one launch: the tree
 * tensorisation, sv_tree_attention, sv_accept and (when accept->commit is set)
 * the commit of the accepted path, with the same inputs, outputs and results as
 * those calls in sequence ([EP] sec. 2: the tree mask fused into the target's
 * execution; [EP] sec. 4: mask construction and tensorisation overhead, with
 * verification and cache commit dominating; [PX] "Inferencia con
 * Decodificacion Especulativa": the accepted count stays on the device).  A
 * step of separate calls is a chain of dependent launches whose gaps dominate
 * at small batches; one launch removes them.
 *   attn:   the attention arguments; attn->anc_bits is not read (each node's
 *           ancestor set is derived from accept->parents inside the launch, by
 *           the rule of sv_build_tree_mask); attn->workspace is not used.
 *   accept: the acceptance arguments (modes 0, 1 and 2); accept->anc_bits and
 *           accept->depth are not read; accept->workspace is not used;
 *           accept->commit as for sv_accept.  flags must be 0 (the reference
 *           mode runs the separate calls).
 *   anc_bits, depth, mask_status (and path_rows, nullable): when set, the
 *           mask outputs of sv_build_tree_mask are written too (all three, or
 *           none of them; NULL skips that work).
 *   workspace: at least sv_verify_step_workspace(args) bytes, 256-byte aligned,
 *           zero-filled before its first use; every call leaves its counters
 *           zeroed again (the attention's split partials in it hold data).
 * Requirements (else SV_ERR_UNSUPPORTED, nothing enqueued): bf16 attention
 * (head_dim 64 or 128), bf16 logits whose rows start on 16 bytes (V a multiple
 * of 8), equal B and N in both argument blocks, and no commit when the tree
 * rows are in the cache (that commit moves rows the attention reads).
 * attn->status additionally reports 7 if a wait inside the launch expired.
 */
typedef struct sv_step_args {
  const sv_attn_args* attn;
  const sv_accept_args* accept;
  uint64_t* anc_bits;     /* optional mask outputs [B, N, W] */
  int32_t* depth;         /* [B, N] */
  int32_t* path_rows;     /* [B, N+1, max_depth], nullable */
  int32_t* mask_status;   /* [B] */
  void* workspace;
  size_t workspace_bytes;
} sv_step_args;
size_t sv_verify_step_workspace(const sv_step_args* args);
sv_status sv_verify_step(const sv_step_args* args, void* stream);

/*
 * sv_outcome_lookup -- outcome lookup of speculative speculative decoding
 * ([SSD] sec. 2: while the target verifies, the drafter prepares speculations
 * for the likely verification outcomes -- how many tokens are accepted and
 * which bonus token is drawn; a hit sends the prepared tokens to the next
 * verification at once, a miss falls back to synchronous drafting).
 * The outcome of sequence b is (stop_row[b], bonus) with bonus =
 * out_tokens[b, num_out[b] - 1], all three from sv_accept; the stop row names
 * the accepted path (on a chain it equals the accepted length).  Prepared
 * outcome k < min(n_keys[b], K) of sequence b is (key_row[b,k], key_token[b,k]).
 *   hit [B]:        1 when some prepared outcome equals the real one, else 0
 *   branch [B]:     k + 1 for the lowest such k, else 0 (the ghost entry, so
 *                   no -1 is ever produced)
 *   next_tokens [B, P] (nullable): prepared[b, k, :] on a hit, zeros on a miss
 *                   (prepared [B, K, P] is then required when P > 0)
 *   n_hits [1] (nullable): number of sequences that hit (e.g. to pick the
 *                   fallback drafter by how many sequences miss, [SSD] sec. 3C)
 * num_out outside [1, max_depth + 1] is a miss.  All arrays int32, device.
 */
typedef struct sv_outcome_args {
  int32_t B, K, P, max_depth;
  const int32_t* stop_row;
  const int32_t* out_tokens;
  const int32_t* num_out;
  const int32_t* key_row;
  const int32_t* key_token;
  const int32_t* n_keys;
  const int32_t* prepared;
  int32_t* hit;
  int32_t* branch;
  int32_t* next_tokens;
  int32_t* n_hits;
} sv_outcome_args;
sv_status sv_outcome_lookup(const sv_outcome_args* args, void* stream);

/*
 * sv_saguaro_reweight -- Saguaro sampling's draft reweighting ([SSD] sec. 3B:
 * lowering the draft probability of tokens already in the speculation cache
 * raises the residual mass on them, so the bonus token more often lands in the
 * cache).  In place on draft_logits [B, R, V] (dtype SV_F32 or SV_BF16): for
 * every distinct token v in [0, V) of cache_tokens[b, r, 0 .. C-1] (int32,
 * device), draft_logits[b, r, v] += shift, added in fp32 and rounded to the
 * logits' type (bf16: nearest even).  Entries outside [0, V) and repeats are
 * ignored.  shift = T ln(rho) multiplies those tokens' unnormalised
 * probabilities by rho at temperature T.  The drafter must sample from the
 * same reweighted logits that sv_accept then receives as draft_logits; the
 * acceptance rule keeps the output distribution exact for any draft
 * distribution.  A non-finite shift is SV_ERR_INVALID_ARGUMENT.
 */
sv_status sv_saguaro_reweight(void* draft_logits, int32_t B, int32_t R, int32_t V, int32_t dtype,
                              const int32_t* cache_tokens, int32_t C, float shift, void* stream);

/*
 * sv_draft_subset_logits -- draft logits over a vocabulary subset, laid out
 * over the target vocabulary ([EP] sec. 3, item 5: the drafter's vocabulary is
 * a cached subset of the target's; acceptance compares full distributions,
 * [PX] "Objetivo-Borrador").  sub_logits [B, R, Vd] are the drafter's logits
 * over its Vd subset entries; t2d [V] int32 maps target id v to j + 1 when v is
 * subset entry j and to 0 when v is not in the subset (values outside [0, Vd]
 * count as 0, so no negative or out-of-range index is ever read).
 * full_logits [B, R, V] (output, same dtype): sub_logits[b, r, t2d[v] - 1], or
 * -inf (probability 0) for ids outside the subset.  The result is the
 * draft_logits of sv_accept: a drafted token outside the subset never occurs,
 * and the residual max(0, p - q) carries the target's mass on those ids.
 * dtype SV_F32 or SV_BF16.  full_logits must not overlap sub_logits.
 */
sv_status sv_draft_subset_logits(const void* sub_logits, int32_t B, int32_t R, int32_t Vd, const int32_t* t2d,
                                 int32_t V, int32_t dtype, void* full_logits, void* stream);

/* Human-readable name of an sv_status (static string). */
const char* sv_status_string(sv_status s);

/* Library version, major*10000 + minor*100 + patch. */
int32_t sv_version(void);

#ifdef __cplusplus
}
#endif
#endif
