// Threshold acceptance (sv_accept mode SV_THRESHOLD).
//
// "Accelerating Sonar Through Speculation" (Perplexity), section
// "Decodificacion Especulativa": every prefix of the draft candidates is
// scored with a probability and the longest prefix above an acceptance
// threshold is kept; the target supplies one more token after it.  The score
// of a prefix is the product over its tokens of the target probability
// p_r(x) = softmax(l_r / T)(x) at the token's parent row r; a node is
// accepted when every prefix of its root path scores at least the threshold
// (all factors are <= 1, so this is its own score); the stop node is the
// deepest accepted node (lowest index on ties); the extra token is the argmax
// of the stop row (lowest id on ties).
//
//  k_thr_rows<T, AL>  one work-group per (row, part) of the rows with a usable
//                     child (others exit after one scan of the parent array);
//                     a part is a contiguous run of the row (one part per row
//                     for large batches, up to 8 for small ones), streamed
//                     with 8 16-byte loads per thread in flight; each
//                     thread keeps a running maximum with its lowest id and
//                     sum_v exp((l_v - m) / T) (fp32 exponentials, fp64 sums,
//                     rescaled when its maximum moves); one block reduction
//                     gives the part's (max, id, sum).  About a thousand
//                     work-groups in all: work-group dispatch, not HBM, limits
//                     grids of tens of thousands.
//  k_thr_walk<T, AL>  one work-group per sequence: forms p_r(x) for every
//                     usable node from its logit and its parent row's
//                     statistics, scores every root path, picks the stop node,
//                     takes the bonus from the stop row's statistics (or scans
//                     a leaf stop row itself, 8 loads per thread in flight),
//                     writes the outputs and zeroes the sequence's statistics.
#include <float.h>
#include <math.h>

#include "sv_commit_dev.h"

namespace {

constexpr int TR_THREADS = 256;   // walk kernel
constexpr int RW_THREADS = 512;   // row kernel and the walk's row scan
constexpr int TR_BATCH = 8;       // 16-byte loads in flight per thread

template <typename T> constexpr int tr_epc() { return 16 / (int)sizeof(T); }  // entries per 16-byte chunk

struct ThrPartial {
  float m;      // row maximum of the stored logits
  int32_t arg;  // lowest id holding it
  double z;     // sum over the row of exp((l - m) / T)
};

// Order-preserving key of (value, id): larger value first, then the lower id.
__device__ __forceinline__ uint64_t argmax_key(float v, int id) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0x7fffffff - id);
}
__device__ __forceinline__ int key_id(uint64_t k) { return 0x7fffffff - (int)(uint32_t)k; }
__device__ __forceinline__ float key_val(uint64_t k) {
  uint32_t u = (uint32_t)(k >> 32);
  u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t y = __shfl_xor(x, o);
    x = y > x ? y : x;
  }
  return x;
}
__device__ __forceinline__ double wave_sum_f64(double x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <typename T>
__device__ __forceinline__ float logit(const T* row, int64_t v) {
  return load_as_f32<T>(row, v);
}

// Entry e of a 16-byte chunk as float.
template <typename T>
__device__ __forceinline__ float chunk_entry(const uint4& w, int e) {
  const uint32_t u = e / (tr_epc<T>() / 4) == 0 ? w.x : (e / (tr_epc<T>() / 4) == 1 ? w.y : (e / (tr_epc<T>() / 4) == 2 ? w.z : w.w));
  if constexpr (sizeof(T) == 2) return bf16_bits_to_f32((uint16_t)(u >> (16 * (e % 2))));
  else return __uint_as_float(u);
}

// Chunk c of a row (entries c*EPC ..): a 16-byte load when whole and aligned, else entry
// by entry with -inf past V (the -inf bit pattern of T).
template <typename T, bool AL>
__device__ __forceinline__ uint4 load_chunk(const T* row, int V, int c) {
  constexpr int EPC = tr_epc<T>();
  const int v0 = c * EPC;
  if (AL && v0 + EPC <= V) return *(const uint4*)(row + v0);
  uint32_t u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (sizeof(T) == 2) {
      const uint32_t lo = v0 + 2 * i < V ? (uint32_t)((const uint16_t*)row)[v0 + 2 * i] : 0xFF80u;
      const uint32_t hi = v0 + 2 * i + 1 < V ? (uint32_t)((const uint16_t*)row)[v0 + 2 * i + 1] : 0xFF80u;
      u[i] = lo | (hi << 16);
    } else {
      u[i] = v0 + i < V ? __float_as_uint(((const float*)row)[v0 + i]) : 0xFF800000u;
    }
  }
  return make_uint4(u[0], u[1], u[2], u[3]);
}

// Row r of sequence b has a usable child (depth > 0 and a token in [0, V)).
__device__ bool row_needed(const sv_accept_args& a, int b, int r) {
  int found = 0;
  for (int i = threadIdx.x; i < a.N; i += blockDim.x) {
    const int64_t o = (int64_t)b * a.N + i;
    const int tok = a.tokens[o];
    if (a.parents[o] + 1 == r && a.depth[o] > 0 && tok >= 0 && tok < a.V) found = 1;
  }
  return __syncthreads_or(found) != 0;
}

// Block-wide max of 64-bit keys (s_key: one slot per wave).
template <int NT>
__device__ __forceinline__ uint64_t block_max_key(uint64_t k, uint64_t* s_key) {
  k = wave_max_u64(k);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_key[threadIdx.x >> 6] = k;
  __syncthreads();
  uint64_t best = s_key[0];
  for (int i = 1; i < NT / 64; ++i) best = s_key[i] > best ? s_key[i] : best;
  return best;
}

// Argmax (lowest id on ties) of one whole row by the work-group's NT threads.
template <typename T, bool AL, int NT>
__device__ int row_argmax(const T* row, int V, uint64_t* s_key) {
  constexpr int EPC = tr_epc<T>();
  const int chunks = (V + EPC - 1) / EPC;
  const int t = threadIdx.x;
  uint64_t best = 0ull;
  for (int base = 0; base < chunks; base += TR_BATCH * NT) {
    uint4 w[TR_BATCH];
#pragma unroll
    for (int k = 0; k < TR_BATCH; ++k) {
      const int c = base + k * NT + t;
      w[k] = c < chunks ? load_chunk<T, AL>(row, V, c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < TR_BATCH; ++k) {
      const int c = base + k * NT + t;
      if (c >= chunks) continue;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const int v = c * EPC + e;
        const float x = chunk_entry<T>(w[k], e);
        if (v < V && x == x) {  // a NaN is never the maximum (as in a scan that takes only larger entries)
          const uint64_t kk = argmax_key(x, v);
          best = kk > best ? kk : best;
        }
      }
    }
  }
  const uint64_t k = block_max_key<NT>(best, s_key);
  return k == 0ull ? 0 : key_id(k);  // no entry but NaN: id 0
}

template <typename T, bool AL>
__global__ void __launch_bounds__(RW_THREADS) k_thr_rows(sv_accept_args a, int S, ThrPartial* part) {
  constexpr int EPC = tr_epc<T>();
  __shared__ uint64_t s_key[RW_THREADS / 64];
  __shared__ double s_z[RW_THREADS / 64];
  const int64_t rowid = blockIdx.x / S;  // b * (N + 1) + r
  const int s = blockIdx.x % S;          // part of the row: a contiguous run of its chunks
  const int b = (int)(rowid / (a.N + 1)), r = (int)(rowid % (a.N + 1));
  if (!row_needed(a, b, r)) return;
  const int t = threadIdx.x;
  const int V = a.V;
  const T* row = (const T*)a.target_logits + rowid * V;
  const int chunks = (V + EPC - 1) / EPC;
  const int per = (chunks + S - 1) / S;
  const int c0 = s * per, c1 = min(chunks, c0 + per);
  const float c2 = 1.4426950408889634f / a.temperature;
  float m = -INFINITY;
  int id = 0x7fffffff;
  double z = 0.0;
  for (int base = c0; base < c1; base += TR_BATCH * RW_THREADS) {
    uint4 w[TR_BATCH];
#pragma unroll
    for (int k = 0; k < TR_BATCH; ++k) {
      const int c = base + k * RW_THREADS + t;
      w[k] = c < c1 ? load_chunk<T, AL>(row, V, c) : make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
    }
    if constexpr (sizeof(T) == 4) {  // the fill above is the bf16 pattern; make it fp32 -inf
#pragma unroll
      for (int k = 0; k < TR_BATCH; ++k)
        if (base + k * RW_THREADS + t >= c1) w[k] = make_uint4(0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u);
    }
    // batch maximum with its lowest id (chunks and entries in ascending id order)
    float bm = -INFINITY;
    int bid = 0x7fffffff;
#pragma unroll
    for (int k = 0; k < TR_BATCH; ++k)
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const float x = chunk_entry<T>(w[k], e);
        if (x > bm) { bm = x; bid = (base + k * RW_THREADS + t) * EPC + e; }
      }
    if (bm > m) {  // the running sum follows the new maximum
      if (m != -INFINITY) z *= (double)exp2f((m - bm) * c2);
      m = bm;
      id = bid;
    }
    if (m != -INFINITY) {
      float zb = 0.f;
      double zd = 0.0;
#pragma unroll
      for (int k = 0; k < TR_BATCH; ++k) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) zb += exp2f((chunk_entry<T>(w[k], e) - m) * c2);
        zd += (double)zb;  // fp32 sums of one chunk, fp64 across chunks
        zb = 0.f;
      }
      z += zd;
    }
  }
  const uint64_t best = block_max_key<RW_THREADS>(m == -INFINITY ? 0ull : argmax_key(m, id), s_key);
  const float M = key_val(best);
  double zt = m == -INFINITY ? 0.0 : z * (double)exp2f((m - M) * c2);
  zt = wave_sum_f64(zt);
  if ((t & 63) == 0) s_z[t >> 6] = zt;
  __syncthreads();
  if (t == 0) {
    double tot = 0.0;
    for (int i = 0; i < RW_THREADS / 64; ++i) tot += s_z[i];
    ThrPartial p;
    p.m = best == 0ull ? -INFINITY : M;  // a part past the end of a short row holds no entry
    p.arg = key_id(best);
    p.z = tot;
    part[rowid * S + s] = p;
  }
}

template <typename T, bool AL>
__global__ void __launch_bounds__(RW_THREADS) k_thr_walk(sv_accept_args a, int S, ThrPartial* part,
                                                          sv_commit_args cm, int32_t has_cm) {
  constexpr int NT = RW_THREADS;
  __shared__ int32_t s_par[SV_MAX_N], s_tok[SV_MAX_N];
  __shared__ uint8_t s_use[SV_MAX_N], s_stats[SV_MAX_N + 1];
  __shared__ double s_p[SV_MAX_N];
  __shared__ uint64_t s_key[NT / 64];
  __shared__ int s_bad, s_A;
  __shared__ int32_t s_path[SV_MAX_DEPTH];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int N = a.N, V = a.V, Dm = a.max_depth;
  const double temp = a.temperature;
  if (t == 0) s_bad = 0;
  for (int i = t; i <= N; i += NT) s_stats[i] = 0;
  __syncthreads();
  for (int i = t; i < N; i += NT) {
    const int64_t o = (int64_t)b * N + i;
    const int par = a.parents[o], tok = a.tokens[o], dep = a.depth[o];
    const bool tok_ok = tok >= 0 && tok < V;
    if (!tok_ok) s_bad = 1;
    const bool use = dep > 0 && tok_ok;  // depth > 0 implies a parent in [-1, N)
    s_par[i] = use ? par : -1;
    s_tok[i] = use ? tok : 0;
    s_use[i] = use;
    if (use) s_stats[par + 1] = 1;  // every writer stores the same value
  }
  __syncthreads();
  const ThrPartial* pb = part + (int64_t)b * (N + 1) * S;
  // p_r(x) of every usable node from its parent row's statistics (parts merged in fp64)
  for (int i = t; i < N; i += NT) {
    if (!s_use[i]) continue;
    const int r = s_par[i] + 1;
    const ThrPartial* pr = pb + (int64_t)r * S;
    float m = -INFINITY;
    for (int q = 0; q < S; ++q) m = fmaxf(m, pr[q].m);
    double z = 0.0;
    for (int q = 0; q < S; ++q)
      if (pr[q].m != -INFINITY) z += pr[q].z * exp(((double)pr[q].m - (double)m) / temp);
    const float l = logit<T>((const T*)a.target_logits + ((int64_t)b * (N + 1) + r) * V, s_tok[i]);
    s_p[i] = exp(((double)l - (double)m) / temp) / z;
  }
  __syncthreads();
  // a node is accepted when its whole root path is usable and its score reaches the threshold
  uint64_t key = 0ull;
  for (int i = t; i < N; i += NT) {
    if (!s_use[i]) continue;
    double score = 1.0;
    bool ok = true;
    int cur = i, len = 0;
    while (cur >= 0 && len <= Dm) {
      if (!s_use[cur]) { ok = false; break; }
      score *= s_p[cur];
      cur = s_par[cur];
      ++len;
    }
    if (ok && cur < 0 && score >= (double)a.threshold) {
      const uint64_t k = ((uint64_t)len << 32) | (uint32_t)(0x7fffffff - i);  // deeper, then lower index
      key = k > key ? k : key;
    }
  }
  const uint64_t best = block_max_key<NT>(key, s_key);
  const int stop = best == 0ull ? -1 : key_id(best);
  const int srow = stop + 1;
  // bonus: argmax of the stop row, from its statistics or by a scan of the (leaf) row
  int bonus;
  if (s_stats[srow]) {  // parts in ascending id order: the strictly larger maximum, else the earlier part
    const ThrPartial* pr = pb + (int64_t)srow * S;
    uint64_t bk = 0ull;
    for (int q = 0; q < S; ++q)
      if (pr[q].m != -INFINITY) {
        const uint64_t k = argmax_key(pr[q].m, pr[q].arg);
        bk = k > bk ? k : bk;
      }
    bonus = bk == 0ull ? 0 : key_id(bk);  // every entry -inf or NaN: id 0
  } else {
    bonus = row_argmax<T, AL, NT>((const T*)a.target_logits + ((int64_t)b * (N + 1) + srow) * V, V, s_key);
  }
  // outputs: the stop node's root path, root-most first
  if (t == 0) {
    int pathn[SV_MAX_DEPTH];
    int A = 0;
    for (int cur = stop; cur >= 0 && A < SV_MAX_DEPTH; cur = s_par[cur]) pathn[A++] = cur;
    for (int k = 0; k < A; ++k) s_path[k] = pathn[A - 1 - k];
    s_A = A;
    for (int k = 0; k < Dm; ++k) a.accept_rows[(int64_t)b * Dm + k] = k < A ? pathn[A - 1 - k] + 1 : 0;
    for (int k = 0; k <= Dm; ++k)
      a.out_tokens[(int64_t)b * (Dm + 1) + k] = k < A ? s_tok[pathn[A - 1 - k]] : (k == A ? bonus : 0);
    a.accept_len[b] = A;
    a.num_out[b] = A + 1;
    a.stop_row[b] = srow;
    a.status[b] = s_bad ? SV_SEQ_TOKEN : 0;
  }
  __syncthreads();
  if (has_cm) svc::walker_commit(cm, b, s_A, s_path);  // the accepted path into the cache
  // leave the workspace zeroed for the next call
  ThrPartial* pw = part + (int64_t)b * (N + 1) * S;
  const ThrPartial zero = {0.f, 0, 0.0};
  for (int i = t; i < (N + 1) * S; i += NT) pw[i] = zero;
}

}  // namespace

// Parts per row: about a thousand work-groups in all (one part per row for large batches, up to
// 8 parts of a row for small ones, where one work-group per row would leave most CUs idle).
int thr_parts(const sv_accept_args& a) {
  const int64_t rows = (int64_t)a.B * (a.N + 1);
  int64_t S = (1024 + rows - 1) / rows;
  return (int)(S < 1 ? 1 : (S > 8 ? 8 : S));
}

size_t sv_threshold_workspace(const sv_accept_args& a) {
  return ((size_t)a.B * (a.N + 1) * thr_parts(a) * sizeof(ThrPartial) + 255) / 256 * 256;
}

sv_status sv_threshold_launch(const sv_accept_args& a, const sv_commit_args& cm, int32_t has_cm, hipStream_t st) {
  if (!(a.threshold >= 0.f && a.threshold <= 1.f)) return SV_ERR_INVALID_ARGUMENT;
  if (a.workspace_bytes < sv_threshold_workspace(a)) return SV_ERR_INVALID_ARGUMENT;
  const bool bf = a.logits_dtype == SV_BF16;
  const int S = thr_parts(a);
  const int64_t rows = (int64_t)a.B * (a.N + 1);
  if (rows * S > 0x7fffffff) return SV_ERR_UNSUPPORTED;
  ThrPartial* part = (ThrPartial*)a.workspace;
  const size_t esz = bf ? 2 : 4;
  const bool al = ((size_t)a.V * esz) % 16 == 0 && ((uintptr_t)a.target_logits % 16) == 0;
#define SV_THR(T, AL)                                                                                   \
  do {                                                                                                  \
    hipLaunchKernelGGL((k_thr_rows<T, AL>), dim3((unsigned)(rows * S)), dim3(RW_THREADS), 0, st, a, S, part); \
    hipLaunchKernelGGL((k_thr_walk<T, AL>), dim3((unsigned)a.B), dim3(RW_THREADS), 0, st, a, S, part, cm,     \
                       has_cm);                                                                                \
  } while (0)
  if (bf) {
    if (al) SV_THR(uint16_t, true); else SV_THR(uint16_t, false);
  } else {
    if (al) SV_THR(float, true); else SV_THR(float, false);
  }
#undef SV_THR
  return sv_launch_status();
}
