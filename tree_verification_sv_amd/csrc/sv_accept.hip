// Speculative acceptance and the bonus token.
//
// "Accelerating Sonar Through Speculation" (Perplexity), sections
// "Decodificacion Especulativa" and "EAGLE": the longest acceptable draft
// sequence is kept, and the target logits after it yield one extra token, so
// n drafted tokens emit up to n+1; section "Objetivo-Borrador": acceptance
// compares the full draft and target distributions; section "Inferencia con
// Decodificacion Especulativa": the accepted count stays on the device here,
// so no host sync is needed.  "Speculative Speculative Decoding", sec. 3B:
// after a rejection the residual mass max(0, p - q) carries the next draw.
//
// Two kernels:
//  1. row pass, grid (slice, row, sequence): for every row that has a usable
//     child (and the root row), one pass over a vocabulary slice gives
//     (max, argmax) of the target logits (greedy) or (max, sum exp) of the
//     target and draft logits (stochastic).  Rows without children are skipped.
//  2. walk, one work-group per sequence: merges the slice partials, then
//     greedy: match bitset and ancestor test over the anc_bits rows;
//     stochastic: the rejection walk.  A rejection at row r with residual
//     coefficient c turns the current distribution into max(0, p - c' q)
//     normalised, c' = c + (previous normaliser); each such step is one
//     block-wide pass over row r (L2 resident).  The bonus token is drawn by
//     an inverse-CDF scan in ascending id order.
#include <float.h>

#include "sv_common.h"

namespace {

constexpr int RP_THREADS = 256;
constexpr int RP_EPT = 32;                      // elements per thread per slice
constexpr int RP_SLICE = RP_THREADS * RP_EPT;   // 8192 vocabulary entries per slice
constexpr int WK_THREADS = 1024;

struct RowPart {
  float pm;     // max of the target row slice
  int32_t parg; // argmax (greedy)
  double pz;    // sum exp((l - pm)/T) (stochastic)
  float qm;     // max of the draft row slice
  int32_t pad;
  double qz;
};
static_assert(sizeof(RowPart) == 32, "RowPart layout");

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) { return load_as_f32<T>(p, i); }

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ double wave_sum(double x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
// (value, index): larger value wins, lower index on equal values
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o);
    int oi = __shfl_xor(i, o);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}

template <int NT>
__device__ float block_max(float x, float* sm) {
  x = wave_max(x);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) sm[w] = x;
  __syncthreads();
  float r = sm[0];
  for (int k = 1; k < NT / 64; ++k) r = fmaxf(r, sm[k]);
  return r;
}
template <int NT>
__device__ double block_sum(double x, double* sm) {
  x = wave_sum(x);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) sm[w] = x;
  __syncthreads();
  double r = 0.0;
  for (int k = 0; k < NT / 64; ++k) r += sm[k];
  return r;
}
template <int NT>
__device__ void block_argmax(float& v, int& i, float* smv, int* smi) {
  wave_argmax(v, i);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) { smv[w] = v; smi[w] = i; }
  __syncthreads();
  v = smv[0];
  i = smi[0];
  for (int k = 1; k < NT / 64; ++k)
    if (smv[k] > v || (smv[k] == v && smi[k] < i)) { v = smv[k]; i = smi[k]; }
}

__device__ __forceinline__ bool node_usable(const sv_accept_args& a, int b, int c) {
  const int32_t tok = a.tokens[(int64_t)b * a.N + c];
  return a.depth[(int64_t)b * a.N + c] > 0 && tok >= 0 && tok < a.V;
}

// ---------------------------------------------------------------- row pass
template <typename T>
__global__ void __launch_bounds__(RP_THREADS) k_row_pass(sv_accept_args a, int32_t S, RowPart* __restrict__ parts) {
  __shared__ float smf[RP_THREADS / 64];
  __shared__ int smi[RP_THREADS / 64];
  __shared__ double smd[RP_THREADS / 64];
  // flat grid: slice fastest, then row, then sequence
  const int64_t bid = blockIdx.x;
  const int s = (int)(bid % S);
  const int r = (int)((bid / S) % (a.N + 1));
  const int b = (int)(bid / ((int64_t)S * (a.N + 1)));
  const int t = threadIdx.x;
  // is row r needed?  (root row, or a row with at least one usable child)
  bool mine = false;
  for (int c = t; c < a.N; c += RP_THREADS)
    mine |= (a.parents[(int64_t)b * a.N + c] + 1 == r) && node_usable(a, b, c);
  const bool needed = (r == 0) || __syncthreads_or(mine);
  if (!needed) return;

  const int64_t row = (int64_t)b * (a.N + 1) + r;
  const T* tp = (const T*)a.target_logits + row * a.V;
  const int v0 = s * RP_SLICE;
  RowPart out;
  out.pad = 0;
  if (a.mode == SV_GREEDY) {
    float best = -FLT_MAX;
    int arg = 0x7fffffff;
#pragma unroll 8
    for (int k = 0; k < RP_EPT; ++k) {
      const int v = v0 + k * RP_THREADS + t;
      if (v < a.V) {
        const float x = ld(tp, v);
        if (x > best) { best = x; arg = v; }  // ascending v per thread: first max kept
      }
    }
    block_argmax<RP_THREADS>(best, arg, smf, smi);
    out.pm = best;
    out.parg = arg;
    out.pz = 0.0;
    out.qm = 0.f;
    out.qz = 0.0;
  } else {
    const T* qp = (const T*)a.draft_logits + row * a.V;
    const float invT = 1.0f / a.temperature;
    float xp[RP_EPT], xq[RP_EPT];
    float mp = -FLT_MAX, mq = -FLT_MAX;
#pragma unroll
    for (int k = 0; k < RP_EPT; ++k) {
      const int v = v0 + k * RP_THREADS + t;
      xp[k] = v < a.V ? ld(tp, v) : -FLT_MAX;
      xq[k] = v < a.V ? ld(qp, v) : -FLT_MAX;
      mp = fmaxf(mp, xp[k]);
      mq = fmaxf(mq, xq[k]);
    }
    mp = block_max<RP_THREADS>(mp, smf);
    mq = block_max<RP_THREADS>(mq, smf);
    double zp = 0.0, zq = 0.0;
#pragma unroll
    for (int k = 0; k < RP_EPT; ++k) {
      const int v = v0 + k * RP_THREADS + t;
      if (v < a.V) {
        zp += (double)expf((xp[k] - mp) * invT);
        zq += (double)expf((xq[k] - mq) * invT);
      }
    }
    zp = block_sum<RP_THREADS>(zp, smd);
    zq = block_sum<RP_THREADS>(zq, smd);
    out.pm = mp;
    out.parg = 0;
    out.pz = zp;
    out.qm = mq;
    out.qz = zq;
  }
  if (t == 0) parts[row * S + s] = out;
}

// ---------------------------------------------------------------- walk
struct WalkShared {
  float red_f[WK_THREADS / 64];
  int red_i[WK_THREADS / 64];
  double red_d[WK_THREADS / 64];
  double scan[WK_THREADS];
  int32_t usable[SV_MAX_N];
  int32_t nchild[SV_MAX_N + 1];
  int32_t amax[SV_MAX_N + 1];
  float pm[SV_MAX_N + 1], qm[SV_MAX_N + 1];
  double pz[SV_MAX_N + 1], qz[SV_MAX_N + 1];
  uint64_t match[SV_MAX_W];
  int32_t path[SV_MAX_DEPTH];
  int32_t bad_token;
  int32_t first_hit;
};

// p_r(v) for the current row as fp32 exponential over an fp64 normaliser
template <typename T>
__device__ __forceinline__ double prob(const T* row, int v, float m, double z, float invT) {
  return (double)expf((ld(row, v) - m) * invT) / z;
}

// Block-wide argmax (lowest id on ties) of one row.
template <typename T>
__device__ int row_argmax(const T* row, int V, WalkShared& sh) {
  float best = -FLT_MAX;
  int arg = 0x7fffffff;
  for (int v = threadIdx.x; v < V; v += WK_THREADS) {
    const float x = ld(row, v);
    if (x > best) { best = x; arg = v; }
  }
  block_argmax<WK_THREADS>(best, arg, sh.red_f, sh.red_i);
  return arg;
}

// Block-wide (max, sum exp) of one row.
template <typename T>
__device__ void row_stats(const T* row, int V, float invT, float& m, double& z, WalkShared& sh) {
  float mx = -FLT_MAX;
  for (int v = threadIdx.x; v < V; v += WK_THREADS) mx = fmaxf(mx, ld(row, v));
  mx = block_max<WK_THREADS>(mx, sh.red_f);
  double s = 0.0;
  for (int v = threadIdx.x; v < V; v += WK_THREADS) s += (double)expf((ld(row, v) - mx) * invT);
  z = block_sum<WK_THREADS>(s, sh.red_d);
  m = mx;
}

// residual weight max(0, p(v) - c q(v)); with c == 0 it is p(v) and q is not read
template <typename T>
__device__ __forceinline__ double resid(const T* prow, const T* qrow, int v, float pm, double pz, float qm, double qz,
                                        float invT, double c) {
  const double p = prob(prow, v, pm, pz, invT);
  if (c == 0.0) return p;
  const double q = prob(qrow, v, qm, qz, invT);
  return fmax(0.0, p - c * q);
}

template <typename T>
__global__ void __launch_bounds__(WK_THREADS) k_walk(sv_accept_args a, int32_t S, const RowPart* __restrict__ parts) {
  __shared__ WalkShared sh;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int N = a.N, V = a.V, Dm = a.max_depth;
  const int W = (N + 63) / 64;
  const int32_t* par = a.parents + (int64_t)b * N;
  const int32_t* tok = a.tokens + (int64_t)b * N;
  const T* tgt = (const T*)a.target_logits + (int64_t)b * (N + 1) * V;
  const T* drf = a.mode == SV_STOCHASTIC ? (const T*)a.draft_logits + (int64_t)b * (N + 1) * V : nullptr;
  const float invT = a.mode == SV_STOCHASTIC ? 1.0f / a.temperature : 1.0f;

  if (t == 0) sh.bad_token = 0;
  if (t <= N) sh.nchild[t] = 0;
  if (t < SV_MAX_W) sh.match[t] = 0;
  __syncthreads();
  if (t < N) {
    const int32_t x = tok[t];
    const bool ok = x >= 0 && x < V;
    if (!ok) atomicOr(&sh.bad_token, 1);
    const bool u = ok && a.depth[(int64_t)b * N + t] > 0;
    sh.usable[t] = u;
    if (u) {
      const int pr = par[t] + 1;  // depth > 0 guarantees par[t] in [-1, N)
      atomicAdd(&sh.nchild[pr], 1);
    }
  }
  __syncthreads();
  // merge slice partials of the rows the row pass computed
  if (t <= N) {
    const bool needed = (t == 0) || sh.nchild[t] > 0;
    sh.amax[t] = -1;
    if (needed) {
      const RowPart* pp = parts + ((int64_t)b * (N + 1) + t) * S;
      if (a.mode == SV_GREEDY) {
        float bv = pp[0].pm;
        int bi = pp[0].parg;
        for (int s = 1; s < S; ++s)
          if (pp[s].pm > bv || (pp[s].pm == bv && pp[s].parg < bi)) { bv = pp[s].pm; bi = pp[s].parg; }
        sh.amax[t] = bi;
      } else {
        float mp = pp[0].pm, mq = pp[0].qm;
        for (int s = 1; s < S; ++s) { mp = fmaxf(mp, pp[s].pm); mq = fmaxf(mq, pp[s].qm); }
        double zp = 0.0, zq = 0.0;
        for (int s = 0; s < S; ++s) {
          zp += pp[s].pz * exp((double)(pp[s].pm - mp) * (double)invT);
          zq += pp[s].qz * exp((double)(pp[s].qm - mq) * (double)invT);
        }
        sh.pm[t] = mp;
        sh.pz[t] = zp;
        sh.qm[t] = mq;
        sh.qz[t] = zq;
      }
    }
  }
  __syncthreads();

  int A = 0, stop_row = 0, bonus = 0;
  if (a.mode == SV_GREEDY) {
    if (t < N && sh.usable[t] && tok[t] == sh.amax[par[t] + 1]) atomicOr((unsigned long long*)&sh.match[t >> 6], 1ull << (t & 63));
    __syncthreads();
    // accepted: every node on the root path is usable and matches (anc_bits lists the path)
    int key = -1;
    if (t < N && sh.usable[t]) {
      const uint64_t* arow = a.anc_bits + ((int64_t)b * N + t) * W;
      bool ok = true;
      for (int w = 0; w < W; ++w) ok &= (arow[w] & ~sh.match[w]) == 0;
      if (ok) key = (a.depth[(int64_t)b * N + t] << 9) | (511 - t);  // deepest, then lowest index
    }
    // block max of key
    {
      float kv = (float)key;
      int ki = key;
      block_argmax<WK_THREADS>(kv, ki, sh.red_f, sh.red_i);
      key = (int)kv;
    }
    if (key >= 0) {
      A = key >> 9;
      const int stop = 511 - (key & 511);
      stop_row = stop + 1;
      if (t == 0) {
        int node = stop;
        for (int k = A - 1; k >= 0; --k) {
          sh.path[k] = node;
          node = par[node];
        }
      }
    }
    int am = sh.amax[stop_row];
    if (am < 0) am = row_argmax<T>(tgt + (int64_t)stop_row * V, V, sh);  // leaf stop row
    bonus = am;
  } else {
    // ---------------- stochastic rejection walk
    int r = 0;
    double c = 0.0, Dn = 1.0;
    // root row statistics are always present
    for (;;) {
      const T* prow = tgt + (int64_t)r * V;
      const T* qrow = drf + (int64_t)r * V;
      if (r > 0 && sh.nchild[r] == 0) {
        // a leaf row is only visited as the stop row: its target statistics are computed here
        float m;
        double z;
        row_stats<T>(prow, V, invT, m, z, sh);
        if (t == 0) { sh.pm[r] = m; sh.pz[r] = z; }
        __syncthreads();
        break;
      }
      const float pm = sh.pm[r], qm = sh.qm[r];
      const double pz = sh.pz[r], qz = sh.qz[r];
      int moved = 0;
      for (int cnode = 0; cnode < N; ++cnode) {
        if (!sh.usable[cnode] || par[cnode] + 1 != r) continue;  // uniform across the block
        const int x = tok[cnode];
        const double px = prob(prow, x, pm, pz, invT);
        const double qx = prob(qrow, x, qm, qz, invT);
        const double cur = fmax(0.0, px - c * qx) / Dn;
        const double u = (double)a.u_accept[(int64_t)b * (N + 1) + cnode + 1];
        const bool acc = qx > 0.0 ? (u < cur / qx) : true;
        if (acc) {
          if (t == 0) sh.path[A] = cnode;
          ++A;
          r = cnode + 1;
          c = 0.0;
          Dn = 1.0;
          moved = 1;
          break;
        }
        // rejection: new residual coefficient and its normaliser (one pass over row r)
        const double cn = c + Dn;
        double s = 0.0;
        for (int v = t; v < V; v += WK_THREADS) {
          const double p = prob(prow, v, pm, pz, invT);
          const double q = prob(qrow, v, qm, qz, invT);
          s += fmax(0.0, p - cn * q);
        }
        s = block_sum<WK_THREADS>(s, sh.red_d);
        if (s > 0.0) { c = cn; Dn = s; }  // s == 0 only through rounding: keep the previous residual
      }
      __syncthreads();
      if (!moved) break;
    }
    stop_row = r;
    // bonus: inverse CDF of the residual weights in ascending id order
    const T* prow = tgt + (int64_t)r * V;
    const T* qrow = drf + (int64_t)r * V;
    const float pm = sh.pm[r], qm = (c != 0.0) ? sh.qm[r] : 0.f;
    const double pz = sh.pz[r], qz = (c != 0.0) ? sh.qz[r] : 1.0;
    const int CH = (V + WK_THREADS - 1) / WK_THREADS;
    const int lo = t * CH, hi = min(V, lo + CH);
    double mysum = 0.0;
    for (int v = lo; v < hi; ++v) mysum += resid(prow, qrow, v, pm, pz, qm, qz, invT, c);
    // inclusive scan over threads (Hillis-Steele in LDS, fixed order)
    sh.scan[t] = mysum;
    __syncthreads();
    for (int off = 1; off < WK_THREADS; off <<= 1) {
      const double add = t >= off ? sh.scan[t - off] : 0.0;
      __syncthreads();
      sh.scan[t] += add;
      __syncthreads();
    }
    const double total = sh.scan[WK_THREADS - 1];
    const double thr = (double)a.u_sample[(int64_t)b * (N + 1) + r] * total;
    if (t == 0) sh.first_hit = 0x7fffffff;
    __syncthreads();
    if (sh.scan[t] > thr) atomicMin(&sh.first_hit, t);
    __syncthreads();
    const int owner = sh.first_hit;
    if (t == (owner == 0x7fffffff ? WK_THREADS - 1 : owner)) {
      double run = t > 0 ? sh.scan[t - 1] : 0.0;
      int pick = -1, last_pos = -1;
      for (int v = lo; v < hi; ++v) {
        const double w = resid(prow, qrow, v, pm, pz, qm, qz, invT, c);
        if (w > 0.0) last_pos = v;
        run += w;
        if (run > thr) { pick = v; break; }
      }
      if (pick < 0) pick = last_pos >= 0 ? last_pos : (hi > lo ? hi - 1 : V - 1);
      sh.first_hit = pick;
    }
    __syncthreads();
    bonus = sh.first_hit;
  }

  __syncthreads();
  if (t == 0) {
    a.accept_len[b] = A;
    a.num_out[b] = A + 1;
    a.stop_row[b] = stop_row;
    a.status[b] = sh.bad_token ? SV_SEQ_TOKEN : 0;
  }
  if (t < Dm) a.accept_rows[(int64_t)b * Dm + t] = t < A ? sh.path[t] + 1 : 0;
  if (t <= Dm) a.out_tokens[(int64_t)b * (Dm + 1) + t] = t < A ? tok[sh.path[t]] : (t == A ? bonus : 0);
}

}  // namespace

static int32_t accept_slices(const sv_accept_args& a) { return (a.V + RP_SLICE - 1) / RP_SLICE; }

extern "C" size_t sv_accept_workspace(const sv_accept_args* args) {
  if (!args || args->B < 1 || args->N < 1 || args->V < 1) return 0;
  return (size_t)args->B * (args->N + 1) * accept_slices(*args) * sizeof(RowPart);
}

extern "C" sv_status sv_accept(const sv_accept_args* args, void* stream) {
  if (!args) return SV_ERR_INVALID_ARGUMENT;
  const sv_accept_args& a = *args;
  if (a.B < 0 || a.N < 1 || a.N > SV_MAX_N || a.V < 1 || a.max_depth < 1 || a.max_depth > SV_MAX_DEPTH)
    return SV_ERR_INVALID_ARGUMENT;
  if (a.mode != SV_GREEDY && a.mode != SV_STOCHASTIC) return SV_ERR_INVALID_ARGUMENT;
  if (a.logits_dtype != SV_F32 && a.logits_dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
  if (a.B == 0) return SV_OK;
  if (!a.parents || !a.tokens || !a.anc_bits || !a.depth || !a.target_logits || !a.accept_len || !a.accept_rows ||
      !a.out_tokens || !a.num_out || !a.stop_row || !a.status || !a.workspace)
    return SV_ERR_INVALID_ARGUMENT;
  if (a.mode == SV_STOCHASTIC && (!a.draft_logits || !a.u_accept || !a.u_sample || !(a.temperature > 0.f)))
    return SV_ERR_INVALID_ARGUMENT;
  if (a.workspace_bytes < sv_accept_workspace(&a)) return SV_ERR_INVALID_ARGUMENT;
  if ((uintptr_t)a.workspace % 256) return SV_ERR_INVALID_ARGUMENT;
  const int32_t S = accept_slices(a);
  RowPart* parts = (RowPart*)a.workspace;
  hipStream_t st = (hipStream_t)stream;
  const int64_t nblocks = (int64_t)S * (a.N + 1) * a.B;
  if (nblocks > 0x7fffffff) return SV_ERR_UNSUPPORTED;
  dim3 g1((unsigned)nblocks);
  if (a.logits_dtype == SV_BF16) {
    hipLaunchKernelGGL(k_row_pass<uint16_t>, g1, dim3(RP_THREADS), 0, st, a, S, parts);
    hipLaunchKernelGGL(k_walk<uint16_t>, dim3(a.B), dim3(WK_THREADS), 0, st, a, S, parts);
  } else {
    hipLaunchKernelGGL(k_row_pass<float>, g1, dim3(RP_THREADS), 0, st, a, S, parts);
    hipLaunchKernelGGL(k_walk<float>, dim3(a.B), dim3(WK_THREADS), 0, st, a, S, parts);
  }
  return sv_launch_status();
}
