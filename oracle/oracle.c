/*
 * CPU oracle for tree speculative-decoding verification -- TEST INFRASTRUCTURE.
 *
 * Plain scalar C, fp64 arithmetic, no blocking, fusion or reordering beyond
 * what each definition states.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg call it.  See oracle.h for the cited pages.
 *
 * Build: gcc -O2 -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static double bf16_bits_to_double(uint16_t h) {
  uint32_t x = (uint32_t)h << 16;
  float f;
  memcpy(&f, &x, 4);
  return (double)f;
}

static double load_elem(const void* base, int dtype, int64_t idx) {
  if (dtype == 0) return (double)((const float*)base)[idx];
  return bf16_bits_to_double(((const uint16_t*)base)[idx]);
}

/*
 * Walk from node i up to the root ([EP] sec. 2: ancestor tables and the
 * range / acyclicity / depth checks).  On success returns 0 and writes the
 * root-first path (path[0] is the depth-1 ancestor, path[len-1] = i).
 * Checks at each step, in this order: the parent index lies in [-1, N)
 * (code 1); -1 ends the walk; a parent already on the walk is a cycle
 * (code 2); taking it would make the path longer than max_depth (code 3).
 */
static int walk_to_root(const int32_t* par, int32_t N, int32_t max_depth, int32_t i, int32_t* path, int32_t* len) {
  int32_t up[64];
  int32_t count = 0;
  up[count++] = i;
  int32_t cur = i;
  for (;;) {
    int32_t p = par[cur];
    if (p < -1 || p >= N) return 1;
    if (p == -1) break;
    for (int32_t k = 0; k < count; ++k)
      if (up[k] == p) return 2;
    if (count + 1 > max_depth) return 3;
    up[count++] = p;
    cur = p;
  }
  for (int32_t k = 0; k < count; ++k) path[k] = up[count - 1 - k];
  *len = count;
  return 0;
}

int orc_build_tree_mask(const int32_t* parents, int32_t B, int32_t N, int32_t max_depth,
                        uint64_t* anc_bits, int32_t* depth, int32_t* path_rows, int32_t* status) {
  if (B < 0 || N < 1 || max_depth < 1 || max_depth > 64) return -1;
  const int32_t W = (N + 63) / 64;
  int32_t path[64];
  for (int32_t b = 0; b < B; ++b) {
    const int32_t* par = parents + (int64_t)b * N;
    int32_t worst = 0;
    if (path_rows) /* row 0 is the root's dummy row: all ghost */
      for (int32_t k = 0; k < max_depth; ++k) path_rows[((int64_t)b * (N + 1) + 0) * max_depth + k] = 0;
    for (int32_t i = 0; i < N; ++i) {
      uint64_t* bits = anc_bits + ((int64_t)b * N + i) * W;
      for (int32_t w = 0; w < W; ++w) bits[w] = 0;
      int32_t* prow = path_rows ? path_rows + ((int64_t)b * (N + 1) + (i + 1)) * max_depth : NULL;
      if (prow)
        for (int32_t k = 0; k < max_depth; ++k) prow[k] = 0;
      int32_t len = 0;
      int code = walk_to_root(par, N, max_depth, i, path, &len);
      if (code == 0) {
        for (int32_t k = 0; k < len; ++k) {
          bits[path[k] / 64] |= 1ull << (path[k] % 64);
          if (prow) prow[k] = path[k] + 1; /* shifted index: node t lives in row t+1 */
        }
        depth[(int64_t)b * N + i] = len;
      } else {
        /* an invalid node sees only itself and has no path */
        bits[i / 64] |= 1ull << (i % 64);
        depth[(int64_t)b * N + i] = 0;
        if (worst == 0 || code < worst) worst = code;
      }
    }
    status[b] = worst;
  }
  return 0;
}

/* --------------------------------------------------------------- attention */
/* Element offset of logical position j of sequence b, KV head g, in a cache that
 * is contiguous [B,Hkv,Lcap,D] or paged [num_blocks,Hkv,bs,D] (an entry outside
 * the pool reads the ghost block 0). */
static int64_t attn_cache_offset(const orc_attn_args* a, int32_t b, int32_t g, int64_t j) {
  if (a->paged) {
    int32_t id = a->block_table[(int64_t)b * a->max_blocks + j / a->block_size];
    if (id < 0 || id >= a->num_blocks) id = 0;
    return (((int64_t)id * a->Hkv + g) * a->block_size + j % a->block_size) * a->D;
  }
  return (((int64_t)b * a->Hkv + g) * a->Lcap + j) * a->D;
}

int orc_tree_attention(const orc_attn_args* a) {
  if (a->B < 1 || a->N < 1 || a->Hkv < 1 || a->Hq % a->Hkv != 0 || a->D < 1) return -1;
  const int32_t N = a->N, Hq = a->Hq, Hkv = a->Hkv, D = a->D, G = a->Hq / a->Hkv;
  const int64_t n_out = a->sel ? a->n_sel : (int64_t)a->B * N * Hq;
  int32_t path[64];
  for (int64_t o = 0; o < n_out; ++o) {
    const int64_t flat = a->sel ? a->sel[o] : o;
    const int32_t h = (int32_t)(flat % Hq);
    const int32_t i = (int32_t)((flat / Hq) % N);
    const int32_t b = (int32_t)(flat / ((int64_t)Hq * N));
    const int32_t g = h / G;
    /* tree keys: anc*(i), root-first; an invalid node sees only itself */
    int32_t len = 0;
    if (walk_to_root(a->parents + (int64_t)b * N, N, a->max_depth, i, path, &len) != 0) {
      path[0] = i;
      len = 1;
    }
    int32_t cap = a->paged ? a->max_blocks * a->block_size : a->Lcap;
    if (a->tree_in_cache) cap -= N; /* the speculative region follows the prefix */
    int32_t L = a->prefix_len[b];
    if (L < 0) L = 0;
    if (L > cap) L = cap;
    const int64_t nkeys = (int64_t)L + len;
    double* s = (double*)malloc(sizeof(double) * (size_t)nkeys);
    const int64_t qoff = (((int64_t)b * N + i) * Hq + h) * D;
    /* scores: prefix positions ascending, then ancestors by depth */
    for (int64_t j = 0; j < nkeys; ++j) {
      int64_t koff;
      const void* kb;
      if (j < L) {
        if (a->paged) {
          int32_t id = a->block_table[(int64_t)b * a->max_blocks + j / a->block_size];
          if (id < 0 || id >= a->num_blocks) id = 0;
          koff = (((int64_t)id * Hkv + g) * a->block_size + j % a->block_size) * D;
        } else {
          koff = (((int64_t)b * Hkv + g) * a->Lcap + j) * D;
        }
        kb = a->k_cache;
      } else if (a->tree_in_cache) {
        koff = attn_cache_offset(a, b, g, (int64_t)L + path[j - L]);
        kb = a->k_cache;
      } else {
        int32_t t = path[j - L];
        koff = (((int64_t)b * Hkv + g) * (N + 1) + (t + 1)) * D;
        kb = a->k_tree;
      }
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d) dot += load_elem(a->q, a->dtype, qoff + d) * load_elem(kb, a->dtype, koff + d);
      s[j] = a->scale * dot;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < nkeys; ++j)
      if (s[j] > m) m = s[j];
    double Z = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
      s[j] = exp(s[j] - m);
      Z += s[j];
    }
    double* out = a->out + o * D;
    for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
      int64_t voff;
      const void* vb;
      if (j < L) {
        if (a->paged) {
          int32_t id = a->block_table[(int64_t)b * a->max_blocks + j / a->block_size];
          if (id < 0 || id >= a->num_blocks) id = 0;
          voff = (((int64_t)id * Hkv + g) * a->block_size + j % a->block_size) * D;
        } else {
          voff = (((int64_t)b * Hkv + g) * a->Lcap + j) * D;
        }
        vb = a->v_cache;
      } else if (a->tree_in_cache) {
        voff = attn_cache_offset(a, b, g, (int64_t)L + path[j - L]);
        vb = a->v_cache;
      } else {
        int32_t t = path[j - L];
        voff = (((int64_t)b * Hkv + g) * (N + 1) + (t + 1)) * D;
        vb = a->v_tree;
      }
      const double w = s[j] / Z;
      for (int32_t d = 0; d < D; ++d) out[d] += w * load_elem(vb, a->dtype, voff + d);
    }
    free(s);
  }
  return 0;
}

/* --------------------------------------------------------------- acceptance */
/* softmax(l/T) of one logits row, fp64 */
static void softmax_row(const void* logits, int dtype, int64_t row_off, int32_t V, double T, double* out) {
  double m = -INFINITY;
  for (int32_t v = 0; v < V; ++v) {
    double l = load_elem(logits, dtype, row_off + v);
    if (l > m) m = l;
  }
  double Z = 0.0;
  for (int32_t v = 0; v < V; ++v) {
    out[v] = exp((load_elem(logits, dtype, row_off + v) - m) / T);
    Z += out[v];
  }
  for (int32_t v = 0; v < V; ++v) out[v] /= Z;
}

int orc_accept(const orc_accept_args* a) {
  const int32_t B = a->B, N = a->N, V = a->V, Dm = a->max_depth;
  if (B < 0 || N < 1 || V < 1 || Dm < 1 || Dm > 64 || a->mode < 0 || a->mode > 3) return -1;
  if (a->mode == 3 && !(a->threshold >= 0.0 && a->threshold <= 1.0)) return -1;
  if (a->mode != 0 && !(a->temperature > 0.0)) return -1;
  const double EPS = 1e-6;
  int32_t* valid = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  int32_t* depth = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  int32_t* usable = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  int32_t* amax = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N + 1));
  double* pcur = (double*)malloc(sizeof(double) * (size_t)V);
  double* q = (double*)malloc(sizeof(double) * (size_t)V);
  int32_t path[64];
  for (int32_t b = 0; b < B; ++b) {
    const int32_t* par = a->parents + (int64_t)b * N;
    const int32_t* tok = a->tokens + (int64_t)b * N;
    int32_t st = 0;
    for (int32_t i = 0; i < N; ++i) {
      int32_t len = 0;
      valid[i] = walk_to_root(par, N, Dm, i, path, &len) == 0;
      depth[i] = valid[i] ? len : 0;
      int tok_ok = tok[i] >= 0 && tok[i] < V;
      if (!tok_ok) st = 4;
      usable[i] = valid[i] && tok_ok;
    }
    int32_t A = 0, stop_node = -1, bonus = 0, flagged = 0;
    int32_t acc_path[64];
    if (a->mode == 0) {
      /* greedy: argmax of every row over the stored values, lowest id on ties */
      for (int32_t r = 0; r <= N; ++r) {
        const int64_t off = ((int64_t)b * (N + 1) + r) * V;
        double best = -INFINITY;
        int32_t arg = 0;
        for (int32_t v = 0; v < V; ++v) {
          double l = load_elem(a->target_logits, a->logits_dtype, off + v);
          if (l > best) { best = l; arg = v; }
        }
        amax[r] = arg;
      }
      /* accepted nodes: every node on the root path matches its parent row's argmax;
         stop at the deepest accepted node, ties to the lowest index */
      for (int32_t i = 0; i < N; ++i) {
        if (!usable[i]) continue;
        int32_t len = 0;
        walk_to_root(par, N, Dm, i, path, &len);
        int ok = 1;
        for (int32_t k = 0; k < len && ok; ++k) {
          int32_t t = path[k];
          if (!usable[t] || tok[t] != amax[par[t] + 1]) ok = 0;
        }
        if (ok && len > A) {
          A = len;
          stop_node = i;
        }
      }
      if (stop_node >= 0) {
        int32_t len = 0;
        walk_to_root(par, N, Dm, stop_node, acc_path, &len);
      }
      bonus = amax[stop_node + 1];
    } else if (a->mode == 3) {
      /* threshold: p of each usable child's token under its parent row's softmax(l/T) */
      const double T = a->temperature, tau = a->threshold;
      double* pchild = (double*)malloc(sizeof(double) * (size_t)N);
      for (int32_t r = 0; r <= N; ++r) {
        int32_t has = 0;
        for (int32_t c = 0; c < N; ++c) has |= usable[c] && par[c] + 1 == r;
        if (!has) continue;
        softmax_row(a->target_logits, a->logits_dtype, ((int64_t)b * (N + 1) + r) * V, V, T, pcur);
        for (int32_t c = 0; c < N; ++c)
          if (usable[c] && par[c] + 1 == r) pchild[c] = pcur[tok[c]];
      }
      /* a prefix is accepted when each of its own prefixes scores at least the threshold */
      for (int32_t i = 0; i < N; ++i) {
        if (!usable[i]) continue;
        int32_t len = 0;
        walk_to_root(par, N, Dm, i, path, &len);
        int ok = 1;
        double score = 1.0;
        for (int32_t k = 0; k < len && ok; ++k) {
          const int32_t t = path[k];
          if (!usable[t]) { ok = 0; break; }
          score *= pchild[t];
          if (fabs(score - tau) <= 1e-5 * tau) flagged = 1;
          if (score < tau) ok = 0;
        }
        if (ok && len > A) {
          A = len;
          stop_node = i;
        }
      }
      if (stop_node >= 0) {
        int32_t len = 0;
        walk_to_root(par, N, Dm, stop_node, acc_path, &len);
      }
      free(pchild);
      /* bonus: the target's own choice after the accepted prefix, argmax of the stop row */
      const int64_t off = ((int64_t)b * (N + 1) + (stop_node + 1)) * V;
      double best = -INFINITY;
      for (int32_t v = 0; v < V; ++v) {
        double l = load_elem(a->target_logits, a->logits_dtype, off + v);
        if (l > best) { best = l; bonus = v; }
      }
    } else {
      /* stochastic: multi-round rejection walk from the root row.  q is the draft
         distribution of the current row (mode 1) or the point mass at the tested
         child's token (mode 2, deterministic drafts) */
      const double T = a->temperature;
      int32_t r = 0;
      softmax_row(a->target_logits, a->logits_dtype, ((int64_t)b * (N + 1) + 0) * V, V, T, pcur);
      if (a->mode == 2)
        for (int32_t v = 0; v < V; ++v) q[v] = 0.0;
      for (;;) {
        if (a->mode == 1) softmax_row(a->draft_logits, a->logits_dtype, ((int64_t)b * (N + 1) + r) * V, V, T, q);
        int32_t moved = 0;
        for (int32_t c = 0; c < N; ++c) {
          if (!usable[c] || par[c] + 1 != r) continue;
          const int32_t x = tok[c];
          if (a->mode == 2) q[x] = 1.0;
          const double u = (double)a->u_accept[(int64_t)b * (N + 1) + (c + 1)];
          const double ratio = q[x] > 0.0 ? pcur[x] / q[x] : INFINITY;
          if (fabs(u - ratio) < EPS) flagged = 1;
          if (u < ratio) {
            if (a->mode == 2) q[x] = 0.0;
            acc_path[A++] = c;
            r = c + 1;
            softmax_row(a->target_logits, a->logits_dtype, ((int64_t)b * (N + 1) + r) * V, V, T, pcur);
            moved = 1;
            break;
          }
          /* rejected: the current distribution becomes normalize(max(0, p_cur - q)) */
          double W = 0.0;
          for (int32_t v = 0; v < V; ++v) W += fmax(0.0, pcur[v] - q[v]);
          if (W > 0.0) {
            for (int32_t v = 0; v < V; ++v) pcur[v] = fmax(0.0, pcur[v] - q[v]) / W;
          } else {
            flagged = 1; /* only reachable through rounding: keep p_cur */
          }
          if (a->mode == 2) q[x] = 0.0;
        }
        if (!moved) break;
      }
      stop_node = r - 1;
      /* bonus: smallest v whose ascending-id cumulative mass exceeds u_s * total */
      const double us = (double)a->u_sample[(int64_t)b * (N + 1) + r];
      double tot = 0.0;
      for (int32_t v = 0; v < V; ++v) tot += pcur[v];
      const double thr = us * tot;
      double C = 0.0, Cprev = 0.0;
      bonus = V - 1;
      for (int32_t v = 0; v < V; ++v) {
        Cprev = C;
        C += pcur[v];
        if (C > thr) { bonus = v; break; }
      }
      if (fabs(us - Cprev / tot) < EPS || fabs(us - C / tot) < EPS) flagged = 1;
    }
    a->accept_len[b] = A;
    for (int32_t k = 0; k < Dm; ++k) a->accept_rows[(int64_t)b * Dm + k] = k < A ? acc_path[k] + 1 : 0;
    for (int32_t k = 0; k <= Dm; ++k) {
      int32_t t = 0;
      if (k < A) t = tok[acc_path[k]];
      else if (k == A) t = bonus;
      a->out_tokens[(int64_t)b * (Dm + 1) + k] = t;
    }
    a->num_out[b] = A + 1;
    a->stop_row[b] = stop_node + 1;
    a->status[b] = st;
    if (a->flagged) a->flagged[b] = flagged;
  }
  free(valid);
  free(depth);
  free(usable);
  free(amax);
  free(pcur);
  free(q);
  return 0;
}

/* --------------------------------------------------------------- KV commit */
/* Slot of logical position pos of sequence b: 0 and *slot, or a status code
 * (6 beyond the capacity, 5 a ghost or out-of-pool block). */
static int commit_slot(const orc_commit_args* a, int32_t b, int64_t pos, int64_t* slot) {
  if (a->paged) {
    const int64_t blk = pos / a->block_size;
    if (blk >= a->max_blocks) return 6;
    const int32_t id = a->block_table[(int64_t)b * a->max_blocks + blk];
    if (id < 1 || id >= a->num_blocks) return 5;
    *slot = (int64_t)id * a->block_size + pos % a->block_size;
  } else {
    if (pos >= a->Lcap) return 6;
    *slot = pos;
  }
  return 0;
}

/* Row offset (in rows of D elements) of slot `slot`, KV head h, sequence b, in one layer's cache. */
static int64_t commit_cache_row(const orc_commit_args* a, int32_t b, int32_t h, int64_t slot) {
  if (a->paged) return (slot / a->block_size * a->Hkv + h) * a->block_size + slot % a->block_size;
  return ((int64_t)b * a->Hkv + h) * a->Lcap + slot;
}

/*
 * [EP] sec. 2, branchable KV cache: the accepted path's K/V rows become the
 * cache entries at positions L, L+1, ..., L+A-1 (by path index, or the first A
 * tree rows in length mode).  Checks per sequence, in order: L >= 0 and
 * 0 <= A <= max_depth (1); with cache-resident tree rows L + N within the
 * capacity (6); then for k = 0 .. A-1: the source row lies in [1, N] (1), the
 * destination position has a slot (6 / 5), and with cache-resident tree rows
 * so does the source position L + src - 1 (5).  A failing sequence is left
 * untouched.  With cache-resident rows every source row is read (into a copy)
 * before any destination is written: position L + k receives the old contents
 * of position L + src_k - 1.
 */
int orc_kv_commit(const orc_commit_args* a) {
  const int32_t B = a->B, N = a->N, Hkv = a->Hkv, D = a->D, Dm = a->max_depth, eb = a->elem_bytes;
  if (B < 0 || N < 1 || Dm < 1 || Dm > 64 || (eb != 2 && eb != 4)) return -1;
  const int32_t layers = a->num_layers < 1 ? 1 : a->num_layers;
  const size_t row_bytes = (size_t)D * eb;
  const int64_t cap = a->paged ? (int64_t)a->max_blocks * a->block_size : a->Lcap;
  char* copy = (char*)malloc(row_bytes * 2 * 64 * (size_t)Hkv);
  for (int32_t b = 0; b < B; ++b) {
    const int32_t L = a->prefix_len[b];
    const int32_t A = a->accept_len[b];
    int32_t code = 0;
    if (L < 0 || A < 0 || A > Dm) code = 1;
    else if (a->tree_in_cache && (int64_t)L + N > cap) code = 6;
    int64_t slot[64], src_slot[64];
    int32_t src[64];
    for (int32_t k = 0; k < A && code == 0; ++k) {
      src[k] = a->commit_mode == 0 ? a->accept_rows[(int64_t)b * Dm + k] : k + 1;
      if (src[k] < 1 || src[k] > N) { code = 1; break; }
      code = commit_slot(a, b, (int64_t)L + k, &slot[k]);
      if (code == 0 && a->tree_in_cache) code = commit_slot(a, b, (int64_t)L + src[k] - 1, &src_slot[k]);
    }
    a->status[b] = code;
    for (int32_t k = 0; k < Dm; ++k) a->committed_slots[(int64_t)b * Dm + k] = 0;
    if (code != 0) {
      a->new_len[b] = L;
      continue;
    }
    for (int32_t l = 0; l < layers; ++l) {
      char* kc = (char*)a->k_cache + (size_t)(l * a->cache_layer_stride) * eb;
      char* vc = (char*)a->v_cache + (size_t)(l * a->cache_layer_stride) * eb;
      if (a->tree_in_cache) {
        /* read every source row first, then write */
        for (int32_t k = 0; k < A; ++k)
          for (int32_t h = 0; h < Hkv; ++h) {
            const int64_t s_row = commit_cache_row(a, b, h, src_slot[k]);
            memcpy(copy + ((size_t)(k * Hkv + h) * 2 + 0) * row_bytes, kc + s_row * row_bytes, row_bytes);
            memcpy(copy + ((size_t)(k * Hkv + h) * 2 + 1) * row_bytes, vc + s_row * row_bytes, row_bytes);
          }
        for (int32_t k = 0; k < A; ++k)
          for (int32_t h = 0; h < Hkv; ++h) {
            const int64_t d_row = commit_cache_row(a, b, h, slot[k]);
            memcpy(kc + d_row * row_bytes, copy + ((size_t)(k * Hkv + h) * 2 + 0) * row_bytes, row_bytes);
            memcpy(vc + d_row * row_bytes, copy + ((size_t)(k * Hkv + h) * 2 + 1) * row_bytes, row_bytes);
          }
      } else {
        const char* kt = (const char*)a->k_tree + (size_t)(l * a->tree_layer_stride) * eb;
        const char* vt = (const char*)a->v_tree + (size_t)(l * a->tree_layer_stride) * eb;
        for (int32_t k = 0; k < A; ++k)
          for (int32_t h = 0; h < Hkv; ++h) {
            const int64_t s_row = ((int64_t)b * Hkv + h) * (N + 1) + src[k];
            const int64_t d_row = commit_cache_row(a, b, h, slot[k]);
            memcpy(kc + d_row * row_bytes, kt + s_row * row_bytes, row_bytes);
            memcpy(vc + d_row * row_bytes, vt + s_row * row_bytes, row_bytes);
          }
      }
    }
    for (int32_t k = 0; k < A; ++k) a->committed_slots[(int64_t)b * Dm + k] = (int32_t)slot[k];
    a->new_len[b] = L + A;
  }
  free(copy);
  return 0;
}

/* ------------------------------------------------------- SSD outcome lookup */
int orc_outcome_lookup(int32_t B, int32_t K, int32_t P, int32_t max_depth, const int32_t* stop_row,
                       const int32_t* out_tokens, const int32_t* num_out, const int32_t* key_row,
                       const int32_t* key_token, const int32_t* n_keys, const int32_t* prepared, int32_t* hit,
                       int32_t* branch, int32_t* next_tokens, int32_t* n_hits) {
  if (B < 0 || K < 1 || P < 0 || max_depth < 1) return -1;
  int32_t hits = 0;
  for (int32_t b = 0; b < B; ++b) {
    int32_t found = -1;
    const int32_t n = num_out[b];
    if (n >= 1 && n <= max_depth + 1) {
      const int32_t row = stop_row[b];
      const int32_t bonus = out_tokens[(int64_t)b * (max_depth + 1) + (n - 1)];
      int32_t nk = n_keys[b];
      if (nk > K) nk = K;
      for (int32_t k = 0; k < nk; ++k)
        if (key_row[(int64_t)b * K + k] == row && key_token[(int64_t)b * K + k] == bonus) {
          found = k;
          break;
        }
    }
    hit[b] = found >= 0;
    branch[b] = found + 1;
    hits += found >= 0;
    if (next_tokens)
      for (int32_t j = 0; j < P; ++j)
        next_tokens[(int64_t)b * P + j] = found >= 0 ? prepared[((int64_t)b * K + found) * P + j] : 0;
  }
  if (n_hits) n_hits[0] = hits;
  return 0;
}

/* ------------------------------------------------------- Saguaro reweighting */
static uint16_t float_to_bf16_rne(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  x += 0x7fffu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}

int orc_saguaro_reweight(void* draft_logits, int32_t B, int32_t R, int32_t V, int32_t dtype,
                         const int32_t* cache_tokens, int32_t C, float shift) {
  if (B < 0 || R < 1 || V < 1 || C < 0 || (dtype != 0 && dtype != 1)) return -1;
  for (int32_t b = 0; b < B; ++b)
    for (int32_t r = 0; r < R; ++r) {
      const int32_t* list = cache_tokens + ((int64_t)b * R + r) * C;
      for (int32_t c = 0; c < C; ++c) {
        const int32_t v = list[c];
        if (v < 0 || v >= V) continue;
        int dup = 0;
        for (int32_t e = 0; e < c; ++e) dup |= list[e] == v;
        if (dup) continue; /* each distinct token once */
        const int64_t idx = ((int64_t)b * R + r) * V + v;
        if (dtype == 0) {
          float* l = (float*)draft_logits;
          l[idx] = l[idx] + shift;
        } else {
          uint16_t* l = (uint16_t*)draft_logits;
          const float cur = (float)bf16_bits_to_double(l[idx]);
          l[idx] = float_to_bf16_rne(cur + shift);
        }
      }
    }
  return 0;
}

/* ------------------------------------------------------- draft vocabulary subset */
int orc_draft_subset_logits(const void* sub, int32_t B, int32_t R, int32_t Vd, const int32_t* t2d, int32_t V,
                            int32_t dtype, void* full) {
  if (B < 0 || R < 1 || Vd < 1 || V < 1 || (dtype != 0 && dtype != 1)) return -1;
  for (int64_t row = 0; row < (int64_t)B * R; ++row)
    for (int32_t v = 0; v < V; ++v) {
      const int32_t j = t2d[v];
      const int present = j >= 1 && j <= Vd;
      if (dtype == 0) {
        ((float*)full)[row * V + v] = present ? ((const float*)sub)[row * Vd + (j - 1)] : -INFINITY;
      } else {
        ((uint16_t*)full)[row * V + v] = present ? ((const uint16_t*)sub)[row * Vd + (j - 1)] : (uint16_t)0xFF80u;
      }
    }
  return 0;
}
