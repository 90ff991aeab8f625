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
//  k_thr_rows<T, AL>  one work-group per (row, vocabulary slice) of the rows
//                     that have a usable child: slice maximum with its lowest
//                     id, and sum_v exp((l_v - m_slice) / T) (fp32 exponentials,
//                     fp64 sums), one 16-byte partial per slice.  Other rows
//                     exit at once, so each needed row is read from HBM once.
//  k_thr_walk<T, AL>  one work-group per sequence: merges the partials of each
//                     needed row, forms p_r(x) for every usable node from its
//                     logit, scores every root path, picks the stop node,
//                     takes the bonus from the stop row's partials (or scans a
//                     leaf stop row itself), writes the outputs and zeroes the
//                     sequence's partials again.
#include <float.h>
#include <math.h>

#include "sv_common.h"

namespace {

constexpr int TR_THREADS = 256;
constexpr int TR_PIECES = 8;  // 16-byte pieces per thread and slice

template <typename T> constexpr int tr_epp() { return 16 / (int)sizeof(T); }
template <typename T> constexpr int tr_slice() { return TR_THREADS * TR_PIECES * tr_epp<T>(); }

struct ThrPartial {
  float m;      // slice maximum of the stored logits
  int32_t arg;  // lowest id holding it
  double z;     // sum over the slice of exp((l - m) / T)
};

// Order-preserving key of (value, id): larger value first, then the lower id.
__device__ __forceinline__ uint64_t argmax_key(float v, int id) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0x7fffffff - id);
}
__device__ __forceinline__ int key_id(uint64_t k) { return 0x7fffffff - (int)(uint32_t)k; }

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

// Thread t's TR_PIECES * EPP logits of slice s (ids ascending within the thread), -inf past V.
template <typename T, bool AL>
__device__ __forceinline__ void load_slice(const T* row, int V, int s, float (&x)[TR_PIECES * tr_epp<T>()]) {
  constexpr int EPP = tr_epp<T>();
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < TR_PIECES; ++k) {
    const int v0 = s * tr_slice<T>() + (k * TR_THREADS + t) * EPP;
    if (AL && v0 + EPP <= V) {
      const uint4 w = *(const uint4*)(row + v0);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < EPP; ++e) {
        if constexpr (sizeof(T) == 2)
          x[k * EPP + e] = bf16_bits_to_f32((uint16_t)(u[e / 2] >> (16 * (e % 2))));
        else
          x[k * EPP + e] = __uint_as_float(u[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPP; ++e) x[k * EPP + e] = v0 + e < V ? logit<T>(row, v0 + e) : -INFINITY;
    }
  }
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

template <typename T, bool AL>
__global__ void __launch_bounds__(TR_THREADS) k_thr_rows(sv_accept_args a, int S, ThrPartial* part) {
  constexpr int E = TR_PIECES * tr_epp<T>();
  __shared__ uint64_t s_key[TR_THREADS / 64];
  __shared__ double s_z[TR_THREADS / 64];
  const int s = blockIdx.x % S;
  const int64_t rowid = blockIdx.x / S;  // b * (N + 1) + r
  const int b = (int)(rowid / (a.N + 1)), r = (int)(rowid % (a.N + 1));
  if (!row_needed(a, b, r)) return;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const T* row = (const T*)a.target_logits + rowid * a.V;
  float x[E];
  load_slice<T, AL>(row, a.V, s, x);
  // slice maximum, lowest id first (each thread scans its ids in ascending order)
  float m = -INFINITY;
  int id = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const int v = s * tr_slice<T>() + ((k / tr_epp<T>()) * TR_THREADS + t) * tr_epp<T>() + k % tr_epp<T>();
    if (x[k] > m) { m = x[k]; id = v; }
  }
  uint64_t key = m == -INFINITY ? 0ull : argmax_key(m, id);
  key = wave_max_u64(key);
  if (lane == 0) s_key[w] = key;
  __syncthreads();
  uint64_t best = s_key[0];
  for (int i = 1; i < TR_THREADS / 64; ++i) best = s_key[i] > best ? s_key[i] : best;
  // the slice maximum back from its key
  uint32_t u = (uint32_t)(best >> 32);
  u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
  const float ms = __uint_as_float(u);
  const float c = 1.4426950408889634f / a.temperature;
  double z = 0.0;
#pragma unroll
  for (int k = 0; k < E; ++k) z += (double)exp2f((x[k] - ms) * c);  // exp2(-inf) = 0 past V
  z = wave_sum_f64(z);
  if (lane == 0) s_z[w] = z;
  __syncthreads();
  if (t == 0) {
    double zt = 0.0;
    for (int i = 0; i < TR_THREADS / 64; ++i) zt += s_z[i];
    ThrPartial p;
    p.m = ms;
    p.arg = key_id(best);
    p.z = zt;
    part[rowid * S + s] = p;
  }
}

template <typename T, bool AL>
__global__ void __launch_bounds__(TR_THREADS) k_thr_walk(sv_accept_args a, int S, ThrPartial* part) {
  __shared__ int32_t s_par[SV_MAX_N], s_tok[SV_MAX_N];
  __shared__ uint8_t s_use[SV_MAX_N], s_stats[SV_MAX_N + 1];
  __shared__ double s_p[SV_MAX_N];
  __shared__ uint64_t s_key[TR_THREADS / 64];
  __shared__ int s_bad, s_stop;
  const int b = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int N = a.N, V = a.V, Dm = a.max_depth;
  const double temp = a.temperature;
  if (t == 0) s_bad = 0;
  for (int i = t; i <= N; i += TR_THREADS) s_stats[i] = 0;
  __syncthreads();
  for (int i = t; i < N; i += TR_THREADS) {
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
  // p_r(x) of every usable node from its parent row's merged statistics
  for (int i = t; i < N; i += TR_THREADS) {
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
  for (int i = t; i < N; i += TR_THREADS) {
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
  key = wave_max_u64(key);
  if (lane == 0) s_key[w] = key;
  __syncthreads();
  if (t == 0) {
    uint64_t best = 0ull;
    for (int i = 0; i < TR_THREADS / 64; ++i) best = s_key[i] > best ? s_key[i] : best;
    s_stop = best == 0ull ? -1 : key_id(best);
  }
  __syncthreads();
  const int stop = s_stop;
  const int srow = stop + 1;
  // bonus: argmax of the stop row, from its partials or by a scan of the row
  int bonus;
  if (s_stats[srow]) {
    const ThrPartial* pr = pb + (int64_t)srow * S;
    uint64_t bk = 0ull;
    for (int q = 0; q < S; ++q)
      if (pr[q].m != -INFINITY) {
        const uint64_t k = argmax_key(pr[q].m, pr[q].arg);
        bk = k > bk ? k : bk;
      }
    bonus = key_id(bk);
  } else {
    const T* row = (const T*)a.target_logits + ((int64_t)b * (N + 1) + srow) * V;
    uint64_t bk = 0ull;
    const int nsl = (V + tr_slice<T>() - 1) / tr_slice<T>();
    for (int s = 0; s < nsl; ++s) {
      float x[TR_PIECES * tr_epp<T>()];
      load_slice<T, AL>(row, V, s, x);
#pragma unroll
      for (int k = 0; k < TR_PIECES * tr_epp<T>(); ++k) {
        const int v = s * tr_slice<T>() + ((k / tr_epp<T>()) * TR_THREADS + t) * tr_epp<T>() + k % tr_epp<T>();
        if (v < V) {
          const uint64_t kk = argmax_key(x[k], v);
          bk = kk > bk ? kk : bk;
        }
      }
    }
    bk = wave_max_u64(bk);
    __syncthreads();
    if (lane == 0) s_key[w] = bk;
    __syncthreads();
    uint64_t best = s_key[0];
    for (int i = 1; i < TR_THREADS / 64; ++i) best = s_key[i] > best ? s_key[i] : best;
    bonus = key_id(best);
  }
  // outputs: the stop node's root path, root-most first
  if (t == 0) {
    int pathn[SV_MAX_DEPTH];
    int A = 0;
    for (int cur = stop; cur >= 0 && A < SV_MAX_DEPTH; cur = s_par[cur]) pathn[A++] = cur;
    for (int k = 0; k < Dm; ++k) a.accept_rows[(int64_t)b * Dm + k] = k < A ? pathn[A - 1 - k] + 1 : 0;
    for (int k = 0; k <= Dm; ++k)
      a.out_tokens[(int64_t)b * (Dm + 1) + k] = k < A ? s_tok[pathn[A - 1 - k]] : (k == A ? bonus : 0);
    a.accept_len[b] = A;
    a.num_out[b] = A + 1;
    a.stop_row[b] = srow;
    a.status[b] = s_bad ? SV_SEQ_TOKEN : 0;
  }
  // leave the workspace zeroed for the next call
  __syncthreads();
  ThrPartial* pw = part + (int64_t)b * (N + 1) * S;
  const ThrPartial zero = {0.f, 0, 0.0};
  for (int i = t; i < (N + 1) * S; i += TR_THREADS) pw[i] = zero;
}

}  // namespace

size_t sv_threshold_workspace(const sv_accept_args& a) {
  const int slice = a.logits_dtype == SV_BF16 ? tr_slice<uint16_t>() : tr_slice<float>();
  const size_t S = (size_t)((a.V + slice - 1) / slice);
  return ((size_t)a.B * (a.N + 1) * S * sizeof(ThrPartial) + 255) / 256 * 256;
}

sv_status sv_threshold_launch(const sv_accept_args& a, hipStream_t st) {
  if (!(a.threshold >= 0.f && a.threshold <= 1.f)) return SV_ERR_INVALID_ARGUMENT;
  if (a.workspace_bytes < sv_threshold_workspace(a)) return SV_ERR_INVALID_ARGUMENT;
  const bool bf = a.logits_dtype == SV_BF16;
  const int slice = bf ? tr_slice<uint16_t>() : tr_slice<float>();
  const int S = (a.V + slice - 1) / slice;
  const int64_t blocks = (int64_t)a.B * (a.N + 1) * S;
  if (blocks > 0x7fffffff) return SV_ERR_UNSUPPORTED;
  ThrPartial* part = (ThrPartial*)a.workspace;
  const size_t esz = bf ? 2 : 4;
  const bool al = ((size_t)a.V * esz) % 16 == 0 && ((uintptr_t)a.target_logits % 16) == 0;
#define SV_THR(T, AL)                                                                              \
  do {                                                                                             \
    hipLaunchKernelGGL((k_thr_rows<T, AL>), dim3((unsigned)blocks), dim3(TR_THREADS), 0, st, a, S, part); \
    hipLaunchKernelGGL((k_thr_walk<T, AL>), dim3((unsigned)a.B), dim3(TR_THREADS), 0, st, a, S, part);   \
  } while (0)
  if (bf) {
    if (al) SV_THR(uint16_t, true); else SV_THR(uint16_t, false);
  } else {
    if (al) SV_THR(float, true); else SV_THR(float, false);
  }
#undef SV_THR
  return sv_launch_status();
}
