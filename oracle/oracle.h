/*
 * CPU oracle for the verification step of tree speculative decoding.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, scalar fp64 statement of
 * what the verification step computes.  It is used by the test-suite, by the
 * smoke check and by the benchmark's CPU-baseline leg; nothing on the product
 * path links or calls it.  It shares no source with the GPU library.
 *
 * Sources (web pages, cited by title and section):
 *  [EP]  "EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on Ascend
 *        NPUs" (gist.science summary), technical summary section 2
 *        (Metodologia): branchable KV cache with length / path-index commit;
 *        shifted indexing with a dummy row 0 for the root instead of -1;
 *        ancestor index tables; range, acyclicity and depth checks; the tree
 *        attention mask that lets a token see only itself and its ancestors.
 *  [PX]  "Accelerating Sonar Through Speculation" (Perplexity), sections
 *        "Decodificacion Especulativa", "Objetivo-Borrador" and "EAGLE":
 *        n drafted tokens give up to n+1 emitted tokens; the longest
 *        acceptable sequence is kept; acceptance compares the full draft and
 *        target distributions; the target logits after the accepted sequence
 *        give one extra (bonus) token.
 *  [SSD] "Speculative Speculative Decoding" (gist.science summary), sections 3B
 *        and 5: residual probability mass, exactness of the output distribution.
 *
 * Index conventions: node i in [0,N) owns row r = i+1; row 0 is the root
 * (the dummy row of [EP] sec. 2).  parents[i] = -1 means "child of the root".
 *
 * Per-sequence status codes (shared meaning with the GPU library, not code):
 *  0 ok, 1 parent out of range, 2 cycle, 3 depth > max_depth,
 *  4 token id outside [0,V), 5 needed block-table entry is the ghost block 0
 *  or outside the pool, 6 capacity exceeded.
 */
#ifndef SV_ORACLE_H
#define SV_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Tree tensorisation ([EP] sec. 2, "Semantica de Tensores de Arbol Segura").
 * parents [B,N]; outputs anc_bits [B,N,W] (W = ceil(N/64)), depth [B,N],
 * path_rows [B,N+1,max_depth] (nullable), status [B].  Returns 0, or -1 on bad
 * sizes. */
int orc_build_tree_mask(const int32_t* parents, int32_t B, int32_t N, int32_t max_depth,
                        uint64_t* anc_bits, int32_t* depth, int32_t* path_rows, int32_t* status);

/* Ancestor-masked GQA tree attention ([EP] sec. 2, "Ejecucion del Maestro con
 * Mascara de Arbol Fusionada"), fp64 throughout.
 * dtype 0 = fp32, 1 = bf16 (uint16 bit patterns) for q / caches / tree KV.
 * Output is fp64: out[n_sel][D] for the selected (b, node, q-head) triples, or
 * out[B][N][Hq][D] when sel == NULL. */
typedef struct {
  int32_t B, N, Hq, Hkv, D, dtype;
  double scale;
  int32_t paged, Lcap, block_size, max_blocks, num_blocks;
  const void* q;          /* [B,N,Hq,D] */
  const void* k_cache;    /* contiguous [B,Hkv,Lcap,D] | paged [num_blocks,Hkv,bs,D] */
  const void* v_cache;
  const void* k_tree;     /* [B,Hkv,N+1,D], row 0 is the ghost row */
  const void* v_tree;
  const int32_t* block_table; /* [B,max_blocks] */
  const int32_t* prefix_len;  /* [B] */
  const int32_t* parents;     /* [B,N] */
  int32_t max_depth;
  const int64_t* sel;         /* flat (b*N + i)*Hq + h, or NULL for all */
  int64_t n_sel;
  double* out;
  /* 1: the tree rows live in the cache itself, node t at position prefix_len + t
   * ([EP] sec. 2: prefix and speculative state of one branchable cache); the
   * prefix may then fill only capacity - N positions, k_tree / v_tree unused */
  int32_t tree_in_cache;
} orc_attn_args;
int orc_tree_attention(const orc_attn_args* a);

/* Speculative acceptance ([PX], [SSD]); mode 0 greedy, 1 stochastic, 2 stochastic
 * with deterministic (top-K) drafts: the drafter's proposal for each child is the
 * point mass at the child's token ([PX] "Objetivo-Borrador": the drafter takes
 * its top token at each stage; "EAGLE": the top-K candidates of each node), so
 * the walk is mode 1's with q = that point mass, and draft_logits is not read.
 * logits dtype 0 = fp32, 1 = bf16.  target/draft logits [B,N+1,V];
 * u_accept, u_sample [B,N+1] (modes 1 and 2).
 * Outputs: accept_len [B], accept_rows [B,max_depth], out_tokens [B,max_depth+1],
 * num_out [B], stop_row [B], status [B], flagged [B] (stochastic: a draw was
 * within 1e-6 of its threshold). */
typedef struct {
  int32_t B, N, V, max_depth, logits_dtype, mode;  /* mode 3: threshold acceptance, see below */
  double temperature;
  const int32_t* parents;
  const int32_t* tokens;
  const void* target_logits;
  const void* draft_logits;
  const float* u_accept;
  const float* u_sample;
  int32_t *accept_len, *accept_rows, *out_tokens, *num_out, *stop_row, *status, *flagged;
  /* mode 3, threshold acceptance ([PX] "Decodificacion Especulativa": every
   * prefix of the candidates gets a probability and the longest one above an
   * acceptance threshold is kept; the target adds one token): the score of node
   * i is the product over its root path of p_{parent row}(token), p =
   * softmax(target row / T); a node is accepted when every node of its path is
   * usable and scores >= threshold; stop at the deepest accepted node (lowest
   * index on ties); bonus = argmax of the stop row (lowest id on ties).
   * flagged: some path score lies within a relative 1e-5 of the threshold. */
  double threshold;
} orc_accept_args;
int orc_accept(const orc_accept_args* a);

/* Commit of the accepted branch's KV ([EP] sec. 2, "Gestion de Cache KV
 * Ramificada").  commit_mode 0 = path-index (rows accept_rows[b][k]),
 * 1 = length (rows 1..A, chains only).  elem_bytes 2 or 4.  The caches are
 * updated in place; new_len [B], committed_slots [B,max_depth], status [B]. */
typedef struct {
  int32_t B, N, Hkv, D, elem_bytes, max_depth, commit_mode;
  int32_t paged, Lcap, block_size, max_blocks, num_blocks;
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;
  const void* k_tree;
  const void* v_tree;
  const int32_t* prefix_len;
  const int32_t* accept_len;
  const int32_t* accept_rows;
  int32_t *new_len, *committed_slots, *status;
  /* 1: tree rows in the cache at positions L + t; the commit makes position L + k
   * hold what position L + src_k - 1 held before the call (in-place compaction of
   * the accepted path, [EP] sec. 2) */
  int32_t tree_in_cache;
  /* layers committed by one call (0 is read as 1): layer l of the caches starts
   * cache_layer_stride elements after layer l-1, its tree rows tree_layer_stride
   * elements after; every layer shares lengths, accepted rows and block table */
  int32_t num_layers;
  int64_t cache_layer_stride, tree_layer_stride;
} orc_commit_args;
int orc_kv_commit(const orc_commit_args* a);

/* Outcome lookup of speculative speculative decoding ([SSD] sec. 2: the
 * drafter prepares speculations for likely verification outcomes -- how many
 * tokens are accepted and which bonus token is drawn; when verification ends
 * the outcome either hits that cache, and the prepared tokens go straight to
 * the next verification, or misses and a fallback runs).  The outcome of
 * sequence b is (stop_row[b], bonus = out_tokens[b, num_out[b] - 1]): the stop
 * row names the accepted path (for a chain it is the accepted length).
 * Prepared outcome k < min(n_keys[b], K) is (key_row[b,k], key_token[b,k]).
 * hit[b] = 1 and branch[b] = k + 1 for the lowest matching k; else hit 0 and
 * branch 0 (the ghost entry: no -1).  next_tokens[b] (nullable, [B,P]) =
 * prepared[b,k,:] on a hit, zeros on a miss; n_hits[0] (nullable) = number of
 * hits.  num_out outside [1, max_depth+1] is a miss. */
int orc_outcome_lookup(int32_t B, int32_t K, int32_t P, int32_t max_depth, const int32_t* stop_row,
                       const int32_t* out_tokens, const int32_t* num_out, const int32_t* key_row,
                       const int32_t* key_token, const int32_t* n_keys, const int32_t* prepared, int32_t* hit,
                       int32_t* branch, int32_t* next_tokens, int32_t* n_hits);

/* Saguaro sampling ([SSD] sec. 3B): the drafter lowers the probability of the
 * tokens already in the speculation cache, which raises the residual mass on
 * them and so the chance that the bonus token lands in the cache.  Stated on
 * logits: every distinct token v in [0, V) of cache_tokens[b, r, 0..C-1] gets
 * draft_logits[b, r, v] += shift (shift = T ln(rho) for a factor rho on the
 * probabilities), added in fp32 and rounded to the logits' type (bf16: nearest
 * even); other entries of the list are ignored.  dtype 0 fp32, 1 bf16.  In place. */
int orc_saguaro_reweight(void* draft_logits, int32_t B, int32_t R, int32_t V, int32_t dtype,
                         const int32_t* cache_tokens, int32_t C, float shift);

/* Draft vocabulary subset ([EP] sec. 3, item 5: the drafter's vocabulary is a
 * cached subset of the target's, trading speed for quality).  The drafter's
 * logits sub [B,R,Vd] cover the subset; acceptance needs the draft distribution
 * over the target vocabulary, where ids outside the subset have probability 0.
 * t2d [V] maps target id v to j + 1 when v is subset entry j, 0 when v is not
 * in the subset (values outside [0, Vd] count as 0).  full[b,r,v] =
 * sub[b,r,t2d[v]-1], or -inf (probability 0) when absent.  dtype 0 fp32, 1 bf16. */
int orc_draft_subset_logits(const void* sub, int32_t B, int32_t R, int32_t Vd, const int32_t* t2d, int32_t V,
                            int32_t dtype, void* full);

#ifdef __cplusplus
}
#endif
#endif
