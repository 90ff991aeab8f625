// Speculative acceptance and the bonus token.
//
// "Accelerating Sonar Through Speculation" (Perplexity), sections
// "Decodificacion Especulativa" and "EAGLE": the longest acceptable draft
// sequence is kept and the target logits after it yield one extra token, so
// n drafted tokens emit up to n+1; section "Objetivo-Borrador": acceptance
// compares the full draft and target distributions; section "Inferencia con
// Decodificacion Especulativa": the accepted count stays on the device here,
// so no host sync is needed.  "Speculative Speculative Decoding", sec. 3B:
// after a rejection the residual mass max(0, p - q) carries the next draw.
//
// Row decomposition.  At row r (distributions p = p_r, q = q_r) the children
// are tested in ascending index.  After k rejections the current distribution
// is max(0, p - c_k q) / S(c_k), with S(c) = sum_v max(0, p(v) - c q(v)),
// c_0 = 0, S(c_0) = 1 and c_k = c_{k-1} + S(c_{k-1}): one rejection maps
// max(0, p - c q)/S(c) to max(0, p - (c + S(c)) q)/S(c + S(c)).  The walk only
// stops at a row after every child was rejected, so both the first accepted
// child of a row and the bonus token drawn if the walk stops there depend on
// that row alone.  Every row is therefore resolved independently and in
// parallel, and the walk is a pointer chase over the per-row results.
//
// One persistent kernel.  Groups of G work-groups share one row; each keeps a
// 16384-entry vocabulary slice in registers (exponentials computed once) and
// the group exchanges per-slice partials through device-scope barriers.
// Greedy rows need one pass (slice max / argmax, lowest id on ties).  The
// group that completes the last row of a sequence performs its walk.  Rows
// resolved: greedy -- the root row and rows with a usable child (a leaf stop
// row's argmax is taken by the walker); stochastic -- the root row and the
// rows of all usable nodes (leaf rows only read the target logits).
#include <float.h>
#include <math.h>

#include "sv_common.h"

namespace {

constexpr int AC_THREADS = 256;
constexpr int AC_CT = 64;                      // vocabulary entries per thread
constexpr int AC_SLICE = AC_THREADS * AC_CT;   // 16384 entries per work-group
constexpr int AC_MAX_RESIDENT = 4096;          // cap on persistent work-groups
constexpr uint32_t AC_SPIN_LIMIT = 1u << 20;   // bounded wait at a group barrier (polls)
constexpr int SEQ_COOP_TIMEOUT = 7;            // status: a group barrier timed out

struct Xchg {       // one work-group's partial for the current row
  float pm, qm;     // slice maxima
  double pz, qz;    // slice sums of exp((l - m)/T)
  double s[2];      // slice residual sums, alternating between rejection steps
  double cdf;       // slice total of the final residual
  float av;         // greedy slice maximum
  int32_t ai;       // greedy slice argmax
};
static_assert(sizeof(Xchg) == 56, "Xchg layout");

struct RowRes {     // resolved row
  int32_t child;    // first accepted child node, -1 when all rejected (stochastic)
  int32_t token;    // bonus token if the walk stops here (stochastic) / argmax (greedy)
};

struct AccWs {      // workspace views
  uint32_t* bar;    // [AC_MAX_RESIDENT] group barrier counters
  uint32_t* gexit;  // [AC_MAX_RESIDENT] group exit counters
  uint32_t* seqdone;// [B] rows resolved per sequence
  uint32_t* err;    // [0] barrier timeout flag, [1] work-groups exited
  RowRes* res;      // [B, N+1]
  Xchg* xg;         // [AC_MAX_RESIDENT][2]: (group * G + rank) * 2 + row parity
};

template <typename T>
__device__ __forceinline__ float ldf(const T* p, int64_t i) { return load_as_f32<T>(p, i); }

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_maxf(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ double wave_sumd(double x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(i, o);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}

struct Red {
  float f[AC_THREADS / 64];
  double d[AC_THREADS / 64];
  int i[AC_THREADS / 64];
  double scan[AC_THREADS];
};

__device__ float block_max(float x, Red& r) {
  x = wave_maxf(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.f[threadIdx.x >> 6] = x;
  __syncthreads();
  float m = r.f[0];
  for (int k = 1; k < AC_THREADS / 64; ++k) m = fmaxf(m, r.f[k]);
  return m;
}
__device__ double block_sum(double x, Red& r) {
  x = wave_sumd(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.d[threadIdx.x >> 6] = x;
  __syncthreads();
  double s = 0.0;
  for (int k = 0; k < AC_THREADS / 64; ++k) s += r.d[k];
  return s;
}
__device__ void block_argmax(float& v, int& i, Red& r) {
  wave_argmax(v, i);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { r.f[threadIdx.x >> 6] = v; r.i[threadIdx.x >> 6] = i; }
  __syncthreads();
  v = r.f[0];
  i = r.i[0];
  for (int k = 1; k < AC_THREADS / 64; ++k)
    if (r.f[k] > v || (r.f[k] == v && r.i[k] < i)) { v = r.f[k]; i = r.i[k]; }
}

// ---------------------------------------------------------------- cross-work-group messages
// Values crossing work-groups are written with relaxed device-scope atomic
// stores and read with relaxed device-scope atomic loads (both coherent at
// device scope); a writer waits for its stores to complete (s_waitcnt) before
// it bumps the counter a reader polls.  This message-passing order needs no
// cache write-back or invalidation.
#define AGENT __HIP_MEMORY_SCOPE_AGENT
__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, AGENT); }
__device__ __forceinline__ void st_u64(uint64_t* p, uint64_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, AGENT); }
__device__ __forceinline__ uint32_t ld_u32(uint32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, AGENT); }
__device__ __forceinline__ uint64_t ld_u64(uint64_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, AGENT); }
__device__ __forceinline__ uint32_t add_u32(uint32_t* p, uint32_t v) { return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, AGENT); }
__device__ __forceinline__ void st_f(float* p, float v) { st_u32((uint32_t*)p, __float_as_uint(v)); }
__device__ __forceinline__ float ld_f(float* p) { return __uint_as_float(ld_u32((uint32_t*)p)); }
__device__ __forceinline__ void st_d(double* p, double v) { st_u64((uint64_t*)p, __double_as_longlong(v)); }
__device__ __forceinline__ double ld_d(double* p) { return __longlong_as_double(ld_u64((uint64_t*)p)); }
__device__ __forceinline__ void st_i(int32_t* p, int32_t v) { st_u32((uint32_t*)p, (uint32_t)v); }
__device__ __forceinline__ int32_t ld_i(int32_t* p) { return (int32_t)ld_u32((uint32_t*)p); }
// wait until this thread's memory operations have completed
__device__ __forceinline__ void mem_complete() {
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
}

// Arrive-and-wait among the G work-groups of a group; `target` = (barrier
// sequence number) * G, identical across the group.  Thread 0 of each
// work-group wrote this step's exchange values.  The wait is bounded: on
// timeout the error flag is raised, and once it is raised no work-group waits
// any more, so every wave exits promptly (results then carry status 7).
__device__ void group_barrier(uint32_t* bar, uint32_t target, uint32_t* err, int G) {
  __syncthreads();
  if (G > 1 && threadIdx.x == 0) {
    mem_complete();
    add_u32(bar, 1u);
    uint32_t spins = 0;
    while (ld_u32(bar) < target) {
      if ((++spins & 63) == 0 && (spins > AC_SPIN_LIMIT || ld_u32(err) != 0)) {
        st_u32(err, 1u);
        break;
      }
    }
    asm volatile("" ::: "memory");
  }
  __syncthreads();
}

struct SeqInfo {    // per-sequence facts every work-group derives the same way
  int32_t par[SV_MAX_N];
  int32_t usable[SV_MAX_N];
  int32_t nkids[SV_MAX_N + 1];
  int32_t kids[SV_MAX_N];     // usable children of the current row, ascending
  int32_t wcount[AC_THREADS / 64];
  int32_t wlive[AC_THREADS / 64];
  int32_t K;                  // number of usable children of the current row
  int32_t nlive;              // rows this sequence resolves
  int32_t bad_token;
  int32_t path[SV_MAX_DEPTH];
  int32_t flag;
};

// per-sequence facts: usable nodes, child counts per row, live-row count (one node per thread)
__device__ void seq_load(const sv_accept_args& a, int b, SeqInfo& si) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int N = a.N;
  for (int x = t; x <= N; x += AC_THREADS) si.nkids[x] = 0;
  if (t == 0) si.bad_token = 0;
  __syncthreads();
  bool u = false;
  if (t < N) {
    const int32_t tok = a.tokens[(int64_t)b * N + t];
    const bool ok = tok >= 0 && tok < a.V;
    if (!ok) atomicOr(&si.bad_token, 1);
    const int pr = a.parents[(int64_t)b * N + t];
    u = ok && a.depth[(int64_t)b * N + t] > 0 && pr >= -1 && pr < N;
    si.par[t] = pr;
    if (u) atomicAdd(&si.nkids[pr + 1], 1);
  }
  if (t < SV_MAX_N) si.usable[t] = u;
  __syncthreads();
  // live rows: greedy -- rows with a usable child; stochastic -- rows of usable nodes
  const bool live = a.mode == SV_GREEDY ? (t >= 1 && t <= N && si.nkids[t] > 0) : u;
  const uint64_t lm = __ballot(live);
  if (lane == 0) si.wlive[wv] = __popcll(lm);
  __syncthreads();
  if (t == 0) {
    int nl = 0;
    for (int k = 0; k < AC_THREADS / 64; ++k) nl += si.wlive[k];
    si.nlive = nl + 1;  // + the root row
  }
  __syncthreads();
}

// usable children of row r in ascending index, from the cached sequence facts
__device__ void row_kids(int N, int r, SeqInfo& si) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const bool kid = t < N && si.usable[t] && si.par[t] + 1 == r;
  const uint64_t m = __ballot(kid);
  if (lane == 0) si.wcount[wv] = __popcll(m);
  __syncthreads();
  int off = 0, K = 0;
  for (int k = 0; k < AC_THREADS / 64; ++k) {
    if (k < wv) off += si.wcount[k];
    K += si.wcount[k];
  }
  if (kid) si.kids[off + __popcll(m & ((1ull << lane) - 1ull))] = t;
  if (t == 0) si.K = K;
  __syncthreads();
}

__device__ __forceinline__ bool row_live(const sv_accept_args& a, const SeqInfo& si, int r) {
  if (r == 0) return true;
  return a.mode == SV_GREEDY ? si.nkids[r] > 0 : si.usable[r - 1] != 0;
}

// AC_CT contiguous logits starting at v (entries >= V read as -FLT_MAX)
template <typename T>
__device__ __forceinline__ void load_chunk(const T* row, int v, int V, float (&x)[AC_CT]) {
  constexpr int PER16 = 16 / sizeof(T);
  if (v + AC_CT <= V && ((uintptr_t)(row + v) % 16) == 0) {
#pragma unroll
    for (int k = 0; k < AC_CT / PER16; ++k) {
      const uint4 w = *(const uint4*)(row + v + k * PER16);
      if (sizeof(T) == 2) {
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          x[k * 8 + 2 * h] = __uint_as_float(ww[h] << 16);
          x[k * 8 + 2 * h + 1] = __uint_as_float(ww[h] & 0xffff0000u);
        }
      } else {
        x[k * 4 + 0] = __uint_as_float(w.x);
        x[k * 4 + 1] = __uint_as_float(w.y);
        x[k * 4 + 2] = __uint_as_float(w.z);
        x[k * 4 + 3] = __uint_as_float(w.w);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < AC_CT; ++e) x[e] = v + e < V ? ldf(row, v + e) : -FLT_MAX;
  }
}

// p(x) of one entry against the row's global max / normaliser
template <typename T>
__device__ __forceinline__ double prob_at(const T* row, int x, float m, double z, float invT) {
  return (double)expf((ldf(row, x) - m) * invT) / z;
}

// ---------------------------------------------------------------- the kernel
constexpr int AC_MAXG = 64;  // work-groups per row group (vocabulary up to 1M entries)
constexpr int AC_PAD = AC_CT + 8;  // LDS entries per thread: the padding keeps 16-byte reads conflict-free

template <typename T> __device__ __forceinline__ T lowest_of();
template <> __device__ __forceinline__ float lowest_of<float>() { return -FLT_MAX; }
template <> __device__ __forceinline__ uint16_t lowest_of<uint16_t>() { return 0xff7f; }  // bf16 -3.39e38
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
// the 16 bytes of w as PER16 = 16/sizeof(T) floats
template <typename T> __device__ __forceinline__ void unpack16(const uint4& w, float (&x)[16 / sizeof(T)]);
template <> __device__ __forceinline__ void unpack16<uint16_t>(const uint4& w, float (&x)[8]) {
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    x[2 * h] = __uint_as_float(ww[h] << 16);
    x[2 * h + 1] = __uint_as_float(ww[h] & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ void unpack16<float>(const uint4& w, float (&x)[4]) {
  x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y); x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
}
// 8 consecutive LDS entries as floats
__device__ __forceinline__ void lds8(const uint16_t* p, float (&x)[8]) {
  const uint4 w = *(const uint4*)p;
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    x[2 * h] = __uint_as_float(ww[h] << 16);
    x[2 * h + 1] = __uint_as_float(ww[h] & 0xffff0000u);
  }
}
__device__ __forceinline__ void lds8(const float* p, float (&x)[8]) {
  const float4 a0 = *(const float4*)p, a1 = *(const float4*)(p + 4);
  x[0] = a0.x; x[1] = a0.y; x[2] = a0.z; x[3] = a0.w;
  x[4] = a1.x; x[5] = a1.y; x[6] = a1.z; x[7] = a1.w;
}

// 8 contiguous logits starting at v (entries >= V read as -FLT_MAX)
template <typename T>
__device__ __forceinline__ void load8(const T* row, int v, int V, float (&x)[8]) {
  if (v + 8 <= V && ((uintptr_t)(row + v) % 16) == 0) {
    if (sizeof(T) == 2) {
      const uint4 w = *(const uint4*)(row + v);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        x[2 * h] = __uint_as_float(ww[h] << 16);
        x[2 * h + 1] = __uint_as_float(ww[h] & 0xffff0000u);
      }
    } else {
      const float4 a0 = *(const float4*)(row + v);
      const float4 a1 = *(const float4*)(row + v + 4);
      x[0] = a0.x; x[1] = a0.y; x[2] = a0.z; x[3] = a0.w;
      x[4] = a1.x; x[5] = a1.y; x[6] = a1.z; x[7] = a1.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = v + e < V ? ldf(row, v + e) : -FLT_MAX;
  }
}

template <typename T, int MODE>
__global__ void __launch_bounds__(AC_THREADS, 2) k_accept(sv_accept_args a, int32_t G, AccWs ws) {
  __shared__ Red red;
  __shared__ SeqInfo si;
  __shared__ int32_t s_last, s_hit;
  __shared__ uint64_t s_match[SV_MAX_W];
  __shared__ float xs_f0[AC_MAXG], xs_f1[AC_MAXG];   // group partials copied in by thread 0
  __shared__ double xs_d0[AC_MAXG], xs_d1[AC_MAXG];
  __shared__ int32_t xs_i[AC_MAXG];
  __shared__ __attribute__((aligned(16))) T lds_p[AC_THREADS * AC_PAD];
  __shared__ __attribute__((aligned(16))) T lds_q[AC_THREADS * AC_PAD];
  const int t = threadIdx.x;
  // work-groups are dispatched round-robin over the 8 XCDs; the members of a
  // group share an XCD (the grid size is a multiple of 8 * G)
  const int NG = gridDim.x / G;
  const int xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
  const int grp = (idx / G) * 8 + xcd;
  const int rank = idx % G;
  const int N = a.N, V = a.V;
  const float invT = MODE == SV_STOCHASTIC ? 1.0f / a.temperature : 1.0f;
  const float l2T = invT * 1.4426950408889634f;  // bulk exponentials as exp2((x - m) * log2(e) / T)
  uint32_t* bar = ws.bar + grp;
  uint32_t nbar = 0;
  auto gsync = [&]() { ++nbar; group_barrier(bar, nbar * (uint32_t)G, ws.err, G); };
  // exchange slots of this group, double-buffered by the parity of the row count:
  // a work-group can run at most one row ahead of the slowest member of its group
  auto slot = [&](int k, int par) -> Xchg* { return ws.xg + ((int64_t)grp * G + k) * 2 + par; };

  const int64_t items = (int64_t)a.B * (N + 1);
  int nrows = 0;
  int cached_b = -1;

  for (int64_t item = grp; item < items; item += NG) {
    // per-lane offsets are recomputed each row from an opaque lane index instead of
    // being hoisted out of the loop (hoisted, they exceed the register budget and spill)
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    // this work-group's slice of the vocabulary; thread t owns AC_CT contiguous entries
    const int v0 = rank * AC_SLICE + t * AC_CT;
    const int b = (int)(item / (N + 1));
    const int r = (int)(item % (N + 1));
    if (b != cached_b) {  // rows of one sequence reuse its facts
      seq_load(a, b, si);
      cached_b = b;
    }
    if (!row_live(a, si, r)) continue;  // uniform across the group
    row_kids(N, r, si);
    const int par = nrows++ & 1;
    const T* prow = (const T*)a.target_logits + ((int64_t)b * (N + 1) + r) * V;
    const T* qrow = MODE == SV_STOCHASTIC ? (const T*)a.draft_logits + ((int64_t)b * (N + 1) + r) * V : nullptr;
    int done_by_me = 0;  // this work-group wrote the row result

    if constexpr (MODE == SV_GREEDY) {
      float best = -FLT_MAX;
      int arg = 0x7fffffff;
      {
        constexpr int PER16 = 16 / sizeof(T);
        constexpr int NLD = AC_CT / PER16;
        const bool fast = v0 + AC_CT <= V && ((uintptr_t)(prow + v0) % 16) == 0;
        if (fast) {
          uint4 rp[NLD];
#pragma unroll
          for (int k = 0; k < NLD; ++k) rp[k] = *(const uint4*)(prow + v0 + k * PER16);  // all loads first
#pragma unroll
          for (int k = 0; k < NLD; ++k) {
            float x[PER16];
            unpack16<T>(rp[k], x);
#pragma unroll
            for (int e = 0; e < PER16; ++e)  // ascending ids: the first maximum is kept
              if (x[e] > best) { best = x[e]; arg = v0 + k * PER16 + e; }
          }
        } else {
          for (int e = 0; e < AC_CT; ++e) {
            const int v = v0 + e;
            if (v < V) {
              const float x = ldf(prow, v);
              if (x > best) { best = x; arg = v; }
            }
          }
        }
      }
      block_argmax(best, arg, red);
      if (t == 0) { st_f(&slot(rank, par)->av, best); st_i(&slot(rank, par)->ai, arg); }
      gsync();
      if (rank == 0) {
        if (t == 0) {
          float bv = ld_f(&slot(0, par)->av);
          int bi = ld_i(&slot(0, par)->ai);
          for (int k = 1; k < G; ++k) {
            const float kv = ld_f(&slot(k, par)->av);
            const int ki = ld_i(&slot(k, par)->ai);
            if (kv > bv || (kv == bv && ki < bi)) { bv = kv; bi = ki; }
          }
          st_i(&ws.res[item].child, -1);
          st_i(&ws.res[item].token, bi);
        }
        done_by_me = 1;
      }
    } else {
      // ---- stochastic: the slice's raw logits stay in LDS (thread t's AC_CT entries at
      // sp[t * AC_PAD ...], padded for conflict-free 16-byte reads); every pass recomputes
      // the exponentials exp2((x - m) * log2(e) / T) from them, which keeps LDS small
      // enough for two work-groups per CU
      const int K = __builtin_amdgcn_readfirstlane(si.K);
      const bool need_q = K > 0;
      T* sp = (T*)lds_p + t * AC_PAD;
      T* sq = (T*)lds_q + t * AC_PAD;
      float mp = -FLT_MAX, mq = -FLT_MAX;
      {
        // coalesced global -> LDS copy: piece q = k * AC_THREADS + t covers entries
        // [q * PER16, (q + 1) * PER16) of the slice, owned by thread (q * PER16) / AC_CT
        constexpr int PER16 = 16 / sizeof(T);
        constexpr int NLD = AC_CT / PER16;
        const int s0 = rank * AC_SLICE;
        const bool rowal = ((uintptr_t)prow % 16) == 0 && ((uintptr_t)qrow % 16) == 0;
        // one tensor at a time keeps at most NLD 16-byte loads in flight per thread
        auto copy = [&](const T* src, T* lds, float& m) {
#pragma unroll
          for (int k = 0; k < NLD; ++k) {
            const int q = k * AC_THREADS + t;
            const int e0 = q * PER16;  // entry inside the slice
            T* d = lds + (e0 / AC_CT) * AC_PAD + (e0 % AC_CT);
            const int v = s0 + e0;
            if (rowal && v + PER16 <= V) {
              const uint4 w = *(const uint4*)(src + v);
              float x[PER16];
              unpack16<T>(w, x);
#pragma unroll
              for (int e = 0; e < PER16; ++e) m = fmaxf(m, x[e]);
              *(uint4*)d = w;
            } else {
              for (int e = 0; e < PER16; ++e) {  // ragged tail: entries past V hold the lowest value
                const T xv = v + e < V ? src[v + e] : lowest_of<T>();
                m = fmaxf(m, to_f32(xv));
                d[e] = xv;
              }
            }
          }
        };
        copy(prow, (T*)lds_p, mp);
        if (need_q) copy(qrow, (T*)lds_q, mq);
      }
      mp = block_max(mp, red);  // also orders the LDS copies before the passes below
      mq = block_max(mq, red);
      const float op = mp * l2T, oq = mq * l2T;  // exp2(x * l2T - o): one FMA per entry
      double zp = 0.0, zq = 0.0;
      for (int k = 0; k < AC_CT; k += 8) {
        float x[8], g = 0.f;  // fp32 partial of 8 entries, fp64 across partials
        lds8(sp + k, x);
        for (int e = 0; e < 8; ++e) g += __builtin_amdgcn_exp2f(fmaf(x[e], l2T, -op));
        zp += (double)g;
        if (need_q) {
          lds8(sq + k, x);
          g = 0.f;
          for (int e = 0; e < 8; ++e) g += __builtin_amdgcn_exp2f(fmaf(x[e], l2T, -oq));
          zq += (double)g;
        }
      }
      zp = block_sum(zp, red);
      zq = block_sum(zq, red);
      if (t == 0) {
        Xchg* x = slot(rank, par);
        st_f(&x->pm, mp); st_d(&x->pz, zp); st_f(&x->qm, mq); st_d(&x->qz, zq);
      }
      gsync();
      if (t < G) {
        Xchg* x = slot(t, par);
        xs_f0[t] = ld_f(&x->pm); xs_d0[t] = ld_d(&x->pz); xs_f1[t] = ld_f(&x->qm); xs_d1[t] = ld_d(&x->qz);
      }
      __syncthreads();
      // global statistics, merged in rank order by every work-group alike
      float Mp = xs_f0[0], Mq = xs_f1[0];
      for (int k = 1; k < G; ++k) { Mp = fmaxf(Mp, xs_f0[k]); Mq = fmaxf(Mq, xs_f1[k]); }
      double Zp = 0.0, Zq = 0.0;
      for (int k = 0; k < G; ++k) {
        Zp += xs_d0[k] * exp2((double)(xs_f0[k] - Mp) * (double)l2T);
        if (need_q) Zq += xs_d1[k] * exp2((double)(xs_f1[k] - Mq) * (double)l2T);
      }
      const double fp = exp2((double)(mp - Mp) * (double)l2T) / Zp;  // p(v) = ep(v) * fp on this slice
      const double fq = need_q ? exp2((double)(mq - Mq) * (double)l2T) / Zq : 0.0;
      // residual weights on this slice in units of fp: max(0, ep - kappa eq), with
      // ep = exp2(x_p * l2T - op), eq = exp2(x_q * l2T - oq)
      auto slice_sum = [&](float kappa) -> double {
        double acc = 0.0;
        for (int k = 0; k < AC_CT; k += 8) {
          float x[8], y[8], g = 0.f;  // fp32 partial of 8 entries, fp64 across partials
          lds8(sp + k, x);
          if (kappa == 0.f) {
            for (int e = 0; e < 8; ++e) g += __builtin_amdgcn_exp2f(fmaf(x[e], l2T, -op));
          } else {
            lds8(sq + k, y);
            for (int e = 0; e < 8; ++e)
              g += fmaxf(fmaf(-kappa, __builtin_amdgcn_exp2f(fmaf(y[e], l2T, -oq)),
                              __builtin_amdgcn_exp2f(fmaf(x[e], l2T, -op))), 0.f);
          }
          acc += (double)g;
        }
        return acc;
      };
      // ---- accept tests along the residual chain
      double c = 0.0, Dn = 1.0, c_prev = 0.0;
      int accepted = -1;
      for (int j = 0; j < K; ++j) {
        const int kid = si.kids[j];
        const int x = a.tokens[(int64_t)b * N + kid];
        const double px = prob_at(prow, x, Mp, Zp, invT);
        const double qx = prob_at(qrow, x, Mq, Zq, invT);
        const double cur = fmax(0.0, px - c * qx) / Dn;
        const double u = (double)a.u_accept[(int64_t)b * (N + 1) + kid + 1];
        if (qx > 0.0 ? (u < cur / qx) : true) { accepted = kid; break; }
        // rejection: next residual coefficient; its normaliser is needed only for a later test,
        // after the last child the bonus scan below computes it as its total
        const double cn = c + Dn;
        if (j == K - 1) { c_prev = c; c = cn; break; }
        // max(0, p - cn q) = fp * max(0, ep - kappa eq) on this slice, kappa = cn fq / fp
        const float kappa = (float)(cn * fq / fp);
        double sl = block_sum(slice_sum(kappa), red) * fp;
        if (t == 0) st_d(&slot(rank, par)->s[j & 1], sl);
        gsync();
        if (t < G) xs_d0[t] = ld_d(&slot(t, par)->s[j & 1]);
        __syncthreads();
        double S = 0.0;
        for (int k = 0; k < G; ++k) S += xs_d0[k];
        __syncthreads();
        if (S > 0.0) { c = cn; Dn = S; }  // S == 0 only through rounding: keep the residual
      }
      if (accepted >= 0) {
        if (rank == 0) {
          if (t == 0) { st_i(&ws.res[item].child, accepted); st_i(&ws.res[item].token, -1); }
          done_by_me = 1;
        }
      } else {
        // ---- bonus: smallest v whose ascending cumulative residual exceeds u * total.
        // A residual of total 0 (reachable only through rounding) falls back to the previous one.
        const double us = (double)a.u_sample[(int64_t)b * (N + 1) + r];
        for (int attempt = 0; attempt < 2; ++attempt) {
          // residual weights on this slice in units of fp: max(0, ep - kappa eq), kappa = c fq / fp
          const float kappa = c == 0.0 ? 0.f : (float)(c * fq / fp);
          red.scan[t] = slice_sum(kappa);
          __syncthreads();
          for (int off = 1; off < AC_THREADS; off <<= 1) {  // inclusive scan, fixed order
            const double add = t >= off ? red.scan[t - off] : 0.0;
            __syncthreads();
            red.scan[t] += add;
            __syncthreads();
          }
          if (t == 0) st_d(&slot(rank, par)->s[attempt], red.scan[AC_THREADS - 1] * fp);
          gsync();
          if (t < G) xs_d1[t] = ld_d(&slot(t, par)->s[attempt]);
          __syncthreads();
          double before = 0.0, total = 0.0;
          for (int k = 0; k < G; ++k) {
            if (k < rank) before += xs_d1[k];
            total += xs_d1[k];
          }
          if (!(total > 0.0) && attempt == 0 && c != 0.0) {  // uniform: retry with the previous residual
            c = c_prev;
            __syncthreads();
            continue;
          }
          // the slice whose inclusive prefix first exceeds the threshold draws the token
          const double thr = us * total;
          int owner = G - 1;
          {
            double pre = 0.0;
            for (int k = 0; k < G; ++k) {
              pre += xs_d1[k];
              if (pre > thr) { owner = k; break; }
            }
          }
          if (rank == owner) {
            if (t == 0) s_hit = 0x7fffffff;
            __syncthreads();
            const double lthr = (thr - before) / fp;  // threshold in this slice's units
            if (red.scan[t] > lthr) atomicMin(&s_hit, t);
            __syncthreads();
            const int hit = s_hit == 0x7fffffff ? AC_THREADS - 1 : s_hit;
            if (t == hit) {
              double run = t > 0 ? red.scan[t - 1] : 0.0;
              int pick = -1, last_pos = -1;
              for (int e = 0; e < AC_CT; ++e) {
                const int v = v0 + e;
                const float ep1 = __builtin_amdgcn_exp2f(fmaf(to_f32(sp[e]), l2T, -op));
                const float w = kappa == 0.f ? ep1
                                             : fmaxf(fmaf(-kappa, __builtin_amdgcn_exp2f(fmaf(to_f32(sq[e]), l2T, -oq)), ep1), 0.f);
                if (v < V && w > 0.f) last_pos = v;
                run += (double)w;
                if (pick < 0 && v < V && run > lthr) pick = v;
              }
              if (pick < 0) pick = last_pos >= 0 ? last_pos : min(v0 + AC_CT, V) - 1;
              st_i(&ws.res[item].child, -1);
              st_i(&ws.res[item].token, pick);
              mem_complete();
            }
            done_by_me = 1;
          }
          break;
        }
      }
    }

    // ---- the work-group that wrote the row result counts it; the last row of a sequence walks
    if (done_by_me) {
      __syncthreads();
      if (t == 0) {
        mem_complete();
        const uint32_t old = add_u32(&ws.seqdone[b], 1u);
        s_last = old + 1 == (uint32_t)si.nlive;
      }
      __syncthreads();
      if (s_last) {
        // ----------------------------------------------------- walk of sequence b
        int A = 0, stop_row = 0, bonus = 0;
        RowRes* rr = ws.res + (int64_t)b * (N + 1);
        if constexpr (MODE == SV_GREEDY) {
          // match[i]: token equals its parent row's argmax; accepted: the whole root path matches
          if (t < SV_MAX_W) s_match[t] = 0;
          __syncthreads();
          if (t < N && si.usable[t] && a.tokens[(int64_t)b * N + t] == ld_i(&rr[si.par[t] + 1].token))
            atomicOr((unsigned long long*)&s_match[t >> 6], 1ull << (t & 63));
          __syncthreads();
          const int W = (N + 63) / 64;
          int key = -1;
          if (t < N && si.usable[t]) {
            const uint64_t* arow = a.anc_bits + ((int64_t)b * N + t) * W;
            bool ok = true;
            for (int w = 0; w < W; ++w) ok &= (arow[w] & ~s_match[w]) == 0;
            if (ok) key = (a.depth[(int64_t)b * N + t] << 9) | (511 - t);  // deepest, then lowest index
          }
          {
            float kv = (float)key;
            int ki = key;
            block_argmax(kv, ki, red);
            key = (int)kv;
          }
          if (key >= 0) {
            A = key >> 9;
            const int stop = 511 - (key & 511);
            stop_row = stop + 1;
            if (t == 0) {
              int node = stop;
              for (int k = A - 1; k >= 0; --k) { si.path[k] = node; node = si.par[node]; }
            }
          }
          if (row_live(a, si, stop_row)) {
            if (t == 0) s_hit = ld_i(&rr[stop_row].token);
            __syncthreads();
            bonus = s_hit;
          } else {
            // leaf stop row: argmax by this work-group
            const T* srow = (const T*)a.target_logits + ((int64_t)b * (N + 1) + stop_row) * V;
            float best = -FLT_MAX;
            int arg = 0x7fffffff;
            for (int v = t; v < V; v += AC_THREADS) {
              const float x = ldf(srow, v);
              if (x > best) { best = x; arg = v; }
            }
            block_argmax(best, arg, red);
            bonus = arg;
          }
        } else {
          if (t == 0) {
            int row = 0, n = 0;
            for (;;) {
              const int ch = ld_i(&rr[row].child);
              if (ch < 0 || n >= SV_MAX_DEPTH) break;
              si.path[n++] = ch;
              row = ch + 1;
            }
            si.flag = (n << 16) | row;  // A and the stop row
            s_hit = ld_i(&rr[row].token);
          }
          __syncthreads();
          A = si.flag >> 16;
          stop_row = si.flag & 0xffff;
          bonus = s_hit;
        }
        __syncthreads();
        const int Dm = a.max_depth;
        if (t == 0) {
          a.accept_len[b] = A;
          a.num_out[b] = A + 1;
          a.stop_row[b] = stop_row;
          a.status[b] = ld_u32(ws.err) ? SEQ_COOP_TIMEOUT : (si.bad_token ? SV_SEQ_TOKEN : 0);
          st_u32(&ws.seqdone[b], 0u);  // every row of b has been counted: ready for the next call
        }
        if (t < Dm) a.accept_rows[(int64_t)b * Dm + t] = t < A ? si.path[t] + 1 : 0;
        if (t <= Dm) a.out_tokens[(int64_t)b * (Dm + 1) + t] = t < A ? a.tokens[(int64_t)b * N + si.path[t]] : (t == A ? bonus : 0);
      }
    }
    __syncthreads();
  }

  // ---- leave every counter zeroed for the next call
  if (t == 0) {
    mem_complete();
    if (G > 1) {
      const uint32_t old = add_u32(ws.gexit + grp, 1u);
      if (old + 1 == (uint32_t)G) {  // every member of the group passed its last barrier
        st_u32(bar, 0u);
        st_u32(ws.gexit + grp, 0u);
      }
    }
    const uint32_t done = add_u32(ws.err + 1, 1u);
    if (done + 1 == gridDim.x) {  // the whole grid has finished: clear the timeout flag
      st_u32(ws.err, 0u);
      st_u32(ws.err + 1, 0u);
    }
  }
}

// occupancy-based size of the persistent grid (per device, cached)
template <typename T, int MODE>
int occupancy_of() {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_accept<T, MODE>, AC_THREADS, 0) != hipSuccess) per_cu = 1;
  return per_cu;
}

int resident_groups(int G, int dtype_bf16, int mode) {
  static int cached[64][2][2] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int& c = cached[dev][dtype_bf16][mode];
  if (c == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 1;
    const int per_cu = dtype_bf16 ? (mode ? occupancy_of<uint16_t, SV_STOCHASTIC>() : occupancy_of<uint16_t, SV_GREEDY>())
                                  : (mode ? occupancy_of<float, SV_STOCHASTIC>() : occupancy_of<float, SV_GREEDY>());
    c = cus * (per_cu > 0 ? per_cu : 1);
    if (c < 1) c = 1;
    if (c > AC_MAX_RESIDENT) c = AC_MAX_RESIDENT;
  }
  return c / G;
}

struct WsLayout {
  size_t bar, gexit, seqdone, err, res, xg, total;
};
WsLayout ws_layout(const sv_accept_args& a) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  WsLayout l{};
  size_t o = 0;
  l.bar = o; o = up(o + AC_MAX_RESIDENT * 4);
  l.gexit = o; o = up(o + AC_MAX_RESIDENT * 4);
  l.seqdone = o; o = up(o + (size_t)a.B * 4);
  l.err = o; o = up(o + 8);
  l.res = o; o = up(o + (size_t)a.B * (a.N + 1) * sizeof(RowRes));
  l.xg = o; o = up(o + (size_t)AC_MAX_RESIDENT * 2 * sizeof(Xchg));
  l.total = o;
  return l;
}

int groups_G(const sv_accept_args& a) {
  const int G = (a.V + AC_SLICE - 1) / AC_SLICE;
  return G < 1 ? 1 : G;
}

}  // namespace

extern "C" size_t sv_accept_workspace(const sv_accept_args* args) {
  if (!args || args->B < 1 || args->N < 1 || args->V < 1) return 0;
  return ws_layout(*args).total;
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
  const WsLayout l = ws_layout(a);
  if (a.workspace_bytes < l.total || ((uintptr_t)a.workspace % 256)) return SV_ERR_INVALID_ARGUMENT;
  const int G = groups_G(a);
  if (G > AC_MAXG) return SV_ERR_UNSUPPORTED;
  const int bf = a.logits_dtype == SV_BF16;
  int NG = resident_groups(G, bf, a.mode == SV_STOCHASTIC);
  const int64_t items = (int64_t)a.B * (a.N + 1);
  if (NG > items) NG = (int)((items + 7) / 8 * 8);
  NG = NG / 8 * 8;  // groups are placed per XCD
  if (NG < 8) return SV_ERR_UNSUPPORTED;  // the groups do not fit on the device at once
  char* base = (char*)a.workspace;
  AccWs ws;
  ws.bar = (uint32_t*)(base + l.bar);
  ws.gexit = (uint32_t*)(base + l.gexit);
  ws.seqdone = (uint32_t*)(base + l.seqdone);
  ws.err = (uint32_t*)(base + l.err);
  ws.res = (RowRes*)(base + l.res);
  ws.xg = (Xchg*)(base + l.xg);
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)(NG * G));
  if (bf) {
    if (a.mode == SV_STOCHASTIC) hipLaunchKernelGGL((k_accept<uint16_t, SV_STOCHASTIC>), grid, dim3(AC_THREADS), 0, st, a, G, ws);
    else hipLaunchKernelGGL((k_accept<uint16_t, SV_GREEDY>), grid, dim3(AC_THREADS), 0, st, a, G, ws);
  } else {
    if (a.mode == SV_STOCHASTIC) hipLaunchKernelGGL((k_accept<float, SV_STOCHASTIC>), grid, dim3(AC_THREADS), 0, st, a, G, ws);
    else hipLaunchKernelGGL((k_accept<float, SV_GREEDY>), grid, dim3(AC_THREADS), 0, st, a, G, ws);
  }
  return sv_launch_status();
}
