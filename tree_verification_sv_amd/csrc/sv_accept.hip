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
// Work decomposition.  A group of G work-groups resolves one row; each owns a
// 16384-entry slice of the vocabulary.  Thread t owns the 16-byte pieces
// k * 256 + t (k = 0 .. 64 / (16 / sizeof(T)) - 1) of its slice, so every load
// instruction of a wave reads 1 KB of consecutive logits.  The exponentials
// are computed once into registers; each later pass over the row (a
// rejection's residual sum, the bonus scan) is a few register operations per
// entry.  Members of a group trade per-slice partials through tagged 64-bit
// words (tag and payload in one atomic word, so a reader that sees the tag
// also sees the value).  Greedy rows need one pass (slice max / argmax, lowest
// id on ties).  The group that completes the last row of a sequence performs
// its walk.  Rows resolved: greedy -- the root row and rows with a usable
// child (a leaf stop row's argmax is taken by the walker); stochastic -- the
// root row and the rows of all usable nodes (leaf rows only read the target
// logits); the work-groups of other rows exit at once.
//
// Forward progress.  Work-groups are dispatched in index order, round-robin
// over the 8 XCDs; the members of a group are consecutive in their XCD's
// dispatch order (block indices x, x + 8, ..., x + 8 (G - 1)), and a member
// only ever waits for members of its own group.  Every group ahead of the
// oldest unfinished one has finished, so that group is resident or next in
// line: no group waits for a work-group that cannot start.  The waits are
// bounded all the same (status SV_SEQ_TIMEOUT).
#include <float.h>
#include <math.h>

#include "sv_common.h"

namespace {

constexpr int AC_THREADS = 256;
constexpr int AC_NW = AC_THREADS / 64;         // waves per work-group
constexpr int AC_CT = 64;                      // vocabulary entries per thread
constexpr int AC_SLICE = AC_THREADS * AC_CT;   // 16384 entries per work-group
constexpr int AC_MAXG = 64;                    // work-groups per row group (vocabulary up to 1M entries)
constexpr int AC_XW = 8;                       // tagged words per exchange slot
constexpr uint32_t AC_SPIN_LIMIT = 1u << 20;   // bounded wait for a group partner (polls)

struct XSlot {      // one work-group's partials for one exchange: (tag << 32) | payload
  uint64_t w[AC_XW];
};

struct RowRes {     // resolved row
  int32_t child;    // first accepted child node, -1 when all rejected (stochastic)
  int32_t token;    // bonus token if the walk stops here (stochastic) / argmax (greedy)
};

struct AccWs {      // workspace views
  uint32_t* gexit;  // [groups] group exit counters
  uint32_t* seqdone;// [B] rows resolved per sequence
  uint32_t* err;    // [0] wait-timeout flag, [1] work-groups exited
  RowRes* res;      // [B, N+1]
  XSlot* xs;        // [groups * G * 2]: (group * G + rank) * 2 + exchange parity
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
// inclusive prefix sum over the 64 lanes of a wave, ascending lane order
__device__ __forceinline__ double wave_scand(double x, int lane) {
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

struct Red {
  float f[AC_NW];
  double d[AC_NW];
  int i[AC_NW];
  double scan1[AC_THREADS];  // exclusive prefixes of the bonus scan, one per thread
};
// LDS index of slice-local entry i in the bonus staging buffer: a stride of 68
// floats per 64 entries keeps the 16-byte reads of consecutive threads on
// distinct banks
__host__ __device__ constexpr int wpad(int i) { return i + (i / AC_CT) * 4; }

__device__ __forceinline__ float block_max(float x, Red& r) {
  x = wave_maxf(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.f[threadIdx.x >> 6] = x;
  __syncthreads();
  float m = r.f[0];
  for (int k = 1; k < AC_NW; ++k) m = fmaxf(m, r.f[k]);
  return m;
}
__device__ __forceinline__ double block_sum(double x, Red& r) {
  x = wave_sumd(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.d[threadIdx.x >> 6] = x;
  __syncthreads();
  double s = 0.0;
  for (int k = 0; k < AC_NW; ++k) s += r.d[k];
  return s;
}
__device__ __forceinline__ void block_argmax(float& v, int& i, Red& r) {
  wave_argmax(v, i);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { r.f[threadIdx.x >> 6] = v; r.i[threadIdx.x >> 6] = i; }
  __syncthreads();
  v = r.f[0];
  i = r.i[0];
  for (int k = 1; k < AC_NW; ++k)
    if (r.f[k] > v || (r.f[k] == v && r.i[k] < i)) { v = r.f[k]; i = r.i[k]; }
}

// ---------------------------------------------------------------- cross-work-group messages
// Values crossing work-groups are written with relaxed device-scope atomic
// stores and read with relaxed device-scope atomic loads (both coherent at
// device scope).  Exchange words carry their tag in the same 64-bit word as
// the payload.  Row results are published before the per-sequence counter:
// the writer waits for its stores to complete (s_waitcnt) and then bumps the
// counter.  Neither order needs a cache write-back or invalidation.
#define AGENT __HIP_MEMORY_SCOPE_AGENT
__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, AGENT); }
__device__ __forceinline__ void st_u64(uint64_t* p, uint64_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, AGENT); }
__device__ __forceinline__ uint32_t ld_u32(uint32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, AGENT); }
__device__ __forceinline__ uint64_t ld_u64(uint64_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, AGENT); }
__device__ __forceinline__ uint32_t add_u32(uint32_t* p, uint32_t v) { return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, AGENT); }
__device__ __forceinline__ void st_i(int32_t* p, int32_t v) { st_u32((uint32_t*)p, (uint32_t)v); }
__device__ __forceinline__ int32_t ld_i(int32_t* p) { return (int32_t)ld_u32((uint32_t*)p); }
// wait until this thread's memory operations have completed
__device__ __forceinline__ void mem_complete() {
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ uint32_t dlo(double x) { return (uint32_t)__double_as_longlong(x); }
__device__ __forceinline__ uint32_t dhi(double x) { return (uint32_t)((uint64_t)__double_as_longlong(x) >> 32); }
__device__ __forceinline__ double dof(uint32_t lo, uint32_t hi) {
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Exchange number `tag` (>= 1, the same on every member) of a group: this
// work-group publishes the nw words w0..w5 (identical in all its threads) and
// collects every member's words into xv[rank][word].  Slots alternate by tag
// parity: a member can only reach exchange tag+2 after every member has
// published tag+1, that is after every member has collected exchange tag.
// The wait is bounded: on timeout the error flag is raised, and once it is
// raised no thread waits any more, so every wave exits (results then carry
// status SV_SEQ_TIMEOUT).
__device__ __forceinline__ void exchange(XSlot* gs, int G, int rank, uint32_t tag, int nw, uint32_t (*xv)[AC_XW],
                                         uint32_t* err, uint32_t w0, uint32_t w1, uint32_t w2 = 0, uint32_t w3 = 0,
                                         uint32_t w4 = 0, uint32_t w5 = 0) {
  const int t = threadIdx.x;
  const int par = tag & 1;
  if (t < nw) {
    const uint32_t w = t == 0 ? w0 : t == 1 ? w1 : t == 2 ? w2 : t == 3 ? w3 : t == 4 ? w4 : w5;
    st_u64(&gs[rank * 2 + par].w[t], ((uint64_t)tag << 32) | w);
  }
  for (int q = t; q < G * nw; q += AC_THREADS) {
    const int k = q / nw, i = q - k * nw;
    uint64_t* p = &gs[k * 2 + par].w[i];
    uint64_t v = ld_u64(p);
    uint32_t spins = 0;
    while ((uint32_t)(v >> 32) != tag) {
      if ((++spins & 63) == 0 && (spins > AC_SPIN_LIMIT || ld_u32(err) != 0)) {
        st_u32(err, 1u);
        break;
      }
      v = ld_u64(p);
    }
    xv[k][i] = (uint32_t)v;
  }
  __syncthreads();
}

struct SeqInfo {    // per-sequence facts every work-group derives the same way
  int32_t par[SV_MAX_N];
  int32_t usable[SV_MAX_N];
  int32_t nkids[SV_MAX_N + 1];
  int32_t kids[SV_MAX_N];     // usable children of the current row, ascending
  int32_t wcount[AC_NW];
  int32_t wlive[AC_NW];
  int32_t K;                  // number of usable children of the current row
  int32_t nlive;              // rows this sequence resolves
  int32_t bad_token;
  int32_t path[SV_MAX_DEPTH];
  int32_t flag;
};

// per-sequence facts: usable nodes, child counts per row, live-row count (one node per thread)
__device__ __forceinline__ void seq_load(const sv_accept_args& a, int b, SeqInfo& si) {
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
    for (int k = 0; k < AC_NW; ++k) nl += si.wlive[k];
    si.nlive = nl + 1;  // + the root row
  }
  __syncthreads();
}

// usable children of row r in ascending index, from the sequence facts
__device__ __forceinline__ void row_kids(int N, int r, SeqInfo& si) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const bool kid = t < N && si.usable[t] && si.par[t] + 1 == r;
  const uint64_t m = __ballot(kid);
  if (lane == 0) si.wcount[wv] = __popcll(m);
  __syncthreads();
  int off = 0, K = 0;
  for (int k = 0; k < AC_NW; ++k) {
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

// ---------------------------------------------------------------- slice loads
template <typename T> struct Piece {
  static constexpr int E = 16 / sizeof(T);  // entries per 16-byte piece
  static constexpr int NK = AC_CT / E;      // pieces per thread
};
template <typename T> __device__ __forceinline__ T lowest_of();
template <> __device__ __forceinline__ float lowest_of<float>() { return -FLT_MAX; }
template <> __device__ __forceinline__ uint16_t lowest_of<uint16_t>() { return 0xff7f; }  // bf16 -3.39e38
__device__ __forceinline__ uint32_t bits_of(float x) { return __float_as_uint(x); }
__device__ __forceinline__ uint32_t bits_of(uint16_t x) { return (uint32_t)x; }
// the 16 bytes of w as E = 16/sizeof(T) floats
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
// hide the register values from the optimiser, so that values derived from
// them are recomputed where they are used rather than kept alive in between
template <int NK>
__device__ __forceinline__ void opaque(uint4 (&raw)[NK]) {
#pragma unroll
  for (int k = 0; k < NK; ++k) asm volatile("" : "+v"(raw[k].x), "+v"(raw[k].y), "+v"(raw[k].z), "+v"(raw[k].w));
}
// first entry of piece k of thread t in a slice starting at s0
template <typename T>
__device__ __forceinline__ int piece_v(int s0, int k, int t) { return s0 + (k * AC_THREADS + t) * Piece<T>::E; }

// Thread t's pieces of one logits row.  `aligned`: the row starts on 16 bytes
// and V * sizeof(T) is a multiple of 16, so each piece lies wholly inside or
// wholly past the row; the loads then go through a buffer resource sized to
// the row, which returns zeros for pieces past V.  Otherwise entries are
// loaded one by one and entries past V read as the lowest value.  Callers
// treat pieces starting at or past V as absent.
template <typename T>
__device__ __forceinline__ void load_pieces(const T* row, int s0, int V, bool aligned, int t,
                                            uint4 (&raw)[Piece<T>::NK]) {
  constexpr int E = Piece<T>::E;
  if (aligned) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)row, 0, V * (int)sizeof(T), 0x00020000);
    const int vo = (s0 + t * E) * (int)sizeof(T);
#pragma unroll
    for (int k = 0; k < Piece<T>::NK; ++k)
      raw[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, k * AC_THREADS * 16, 0));
  } else {
#pragma unroll
    for (int k = 0; k < Piece<T>::NK; ++k) {
      const int v = piece_v<T>(s0, k, t);
      uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const T x = v + e < V ? row[v + e] : lowest_of<T>();
        wd[e * sizeof(T) / 4] |= bits_of(x) << (8 * ((e * sizeof(T)) % 4));
      }
      raw[k] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
  }
}

// ---------------------------------------------------------------- the kernel
template <typename T, int MODE>
__global__ void __launch_bounds__(AC_THREADS, 2) k_accept(sv_accept_args a, int32_t G, AccWs ws) {
  constexpr int E = Piece<T>::E, NK = Piece<T>::NK;
  __shared__ Red red;
  __shared__ SeqInfo si;
  __shared__ int32_t s_last, s_hit, s_first, s_lpos;
  __shared__ uint64_t s_match[SV_MAX_W];
  __shared__ uint32_t xv[AC_MAXG][AC_XW];                          // collected group partials
  __shared__ float s_lp[SV_MAX_N], s_lq[SV_MAX_N], s_u[SV_MAX_N];  // per child: logits at its token, u_accept
  __shared__ float s_us;                                            // u_sample of the row
  // bonus weights of the slice in id order, 4 floats of padding after every 64 entries
  __shared__ __attribute__((aligned(16))) float s_w[MODE == SV_STOCHASTIC ? wpad(AC_SLICE) : 4];
  // work-groups are dispatched round-robin over the 8 XCDs; the members of a
  // group share an XCD (the grid size is a multiple of 8 * G)
  const int t = threadIdx.x, lane = t & 63;
  const int xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
  const int grp = (idx / G) * 8 + xcd;
  const int rank = idx % G;
  const int N = a.N, V = a.V;
  const float invT = MODE == SV_STOCHASTIC ? 1.0f / a.temperature : 1.0f;
  const float l2T = invT * 1.4426950408889634f;  // bulk exponentials as exp2((x - m) * log2(e) / T)
  XSlot* gslots = ws.xs + (int64_t)grp * G * 2;
  uint32_t xtag = 0;  // exchanges of this group so far (identical on every member)
  const int64_t item = grp;
  const int s0 = rank * AC_SLICE;  // this work-group's slice of the vocabulary

  if (item < (int64_t)a.B * (N + 1)) {
    const int b = (int)(item / (N + 1));
    const int r = (int)(item % (N + 1));
    const T* prow = (const T*)a.target_logits + ((int64_t)b * (N + 1) + r) * V;
    const T* qrow = MODE == SV_STOCHASTIC ? (const T*)a.draft_logits + ((int64_t)b * (N + 1) + r) * V : nullptr;
    const bool aligned = ((size_t)V * sizeof(T)) % 16 == 0 && ((uintptr_t)prow % 16) == 0 &&
                         (MODE == SV_GREEDY || ((uintptr_t)qrow % 16) == 0);
    // stochastic: nearly every row is resolved, so the target slice is fetched before the
    // sequence facts that confirm it is needed (its latency overlaps them)
    uint4 rp[NK];
    if constexpr (MODE == SV_STOCHASTIC) load_pieces<T>(prow, s0, V, aligned, t, rp);
    seq_load(a, b, si);
    if (row_live(a, si, r)) {  // uniform across the group
      row_kids(N, r, si);
      int done_by_me = 0;  // this work-group wrote the row result

      if constexpr (MODE == SV_GREEDY) {
        float best = -FLT_MAX;
        int arg = 0x7fffffff;
        {
          load_pieces<T>(prow, s0, V, aligned, t, rp);
#pragma unroll
          for (int k = 0; k < NK; ++k) {
            float x[E];
            unpack16<T>(rp[k], x);
            const int v = piece_v<T>(s0, k, t);
#pragma unroll
            for (int e = 0; e < E; ++e)  // a thread visits its entries in ascending id
              if (v + e < V && x[e] > best) { best = x[e]; arg = v + e; }
          }
        }
        block_argmax(best, arg, red);
        exchange(gslots, G, rank, ++xtag, 2, xv, ws.err, __float_as_uint(best), (uint32_t)arg);
        if (rank == 0) {
          if (t == 0) {
            float bv = __uint_as_float(xv[0][0]);
            int bi = (int)xv[0][1];
            for (int k = 1; k < G; ++k) {
              const float kv = __uint_as_float(xv[k][0]);
              const int ki = (int)xv[k][1];
              if (kv > bv || (kv == bv && ki < bi)) { bv = kv; bi = ki; }
            }
            st_i(&ws.res[item].child, -1);
            st_i(&ws.res[item].token, bi);
          }
          done_by_me = 1;
        }
      } else {
        const int K = __builtin_amdgcn_readfirstlane(si.K);
        const bool need_q = K > 0;
        // ---- children's logits at their tokens and their uniforms, fetched alongside the slice
        if (t < K) {
          const int kid = si.kids[t];
          const int x = a.tokens[(int64_t)b * N + kid];  // usable: x in [0, V)
          s_lp[t] = ldf(prow, x);
          s_lq[t] = ldf(qrow, x);
          s_u[t] = a.u_accept[(int64_t)b * (N + 1) + kid + 1];
        }
        if (t == AC_THREADS - 1) s_us = a.u_sample[(int64_t)b * (N + 1) + r];
        // ---- the slice: raw logits -> slice maxima -> exponentials kept in registers
        float ep[AC_CT], eq[AC_CT];
        float mp = -FLT_MAX, mq = -FLT_MAX;
        double zp = 0.0, zq = 0.0;
        {
          uint4 rq[NK];
          if (need_q) load_pieces<T>(qrow, s0, V, aligned, t, rq);
#pragma unroll
          for (int k = 0; k < NK; ++k) {
            float x[E];
            unpack16<T>(rp[k], x);
#pragma unroll
            for (int e = 0; e < E; ++e) mp = piece_v<T>(s0, k, t) < V ? fmaxf(mp, x[e]) : mp;
          }
          mp = block_max(mp, red);
          opaque(rp);  // unpack again below instead of keeping the unpacked floats alive
          const float op = mp * l2T;  // exp2(x * l2T - op): one FMA per entry
          const bool whole = s0 + AC_SLICE <= V;  // uniform: no entry of the slice lies past V
          auto expo = [&](const uint4 (&raw)[NK], float o, float (&ex)[AC_CT], double& z) {
            if (whole) {
#pragma unroll
              for (int k = 0; k < NK; ++k) {
                float x[E], g = 0.f;  // fp32 partial of one piece, fp64 across pieces
                unpack16<T>(raw[k], x);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                  ex[k * E + e] = __builtin_amdgcn_exp2f(fmaf(x[e], l2T, -o));
                  g += ex[k * E + e];
                }
                z += (double)g;
              }
            } else {
#pragma unroll
              for (int k = 0; k < NK; ++k) {
                float x[E], g = 0.f;
                unpack16<T>(raw[k], x);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                  ex[k * E + e] = piece_v<T>(s0, k, t) < V ? __builtin_amdgcn_exp2f(fmaf(x[e], l2T, -o)) : 0.f;
                  g += ex[k * E + e];
                }
                z += (double)g;
              }
            }
          };
          expo(rp, op, ep, zp);
          if (need_q) {
#pragma unroll
            for (int k = 0; k < NK; ++k) {
              float x[E];
              unpack16<T>(rq[k], x);
#pragma unroll
              for (int e = 0; e < E; ++e) mq = piece_v<T>(s0, k, t) < V ? fmaxf(mq, x[e]) : mq;
            }
            mq = block_max(mq, red);
            opaque(rq);
            expo(rq, mq * l2T, eq, zq);
          } else {
#pragma unroll
            for (int i = 0; i < AC_CT; ++i) eq[i] = 0.f;
          }
        }
        zp = block_sum(zp, red);
        zq = block_sum(zq, red);
        exchange(gslots, G, rank, ++xtag, 6, xv, ws.err, __float_as_uint(mp), __float_as_uint(mq), dlo(zp), dhi(zp),
                 dlo(zq), dhi(zq));
        // global statistics: lane k of every wave takes member k's partials (G <= 64); the
        // butterfly reductions give every lane, wave and member the same values
        double Zp, Zq, fp, fq;
        float Mp, Mq;
        {
          const bool on = lane < G;
          const int k = on ? lane : 0;
          const float mpk = on ? __uint_as_float(xv[k][0]) : -FLT_MAX;
          const float mqk = on ? __uint_as_float(xv[k][1]) : -FLT_MAX;
          Mp = wave_maxf(mpk);
          Mq = wave_maxf(mqk);
          const double sp = on ? exp2((double)(mpk - Mp) * (double)l2T) : 0.0;  // member k's scale
          const double sq = on && need_q ? exp2((double)(mqk - Mq) * (double)l2T) : 0.0;
          Zp = wave_sumd(on ? dof(xv[k][2], xv[k][3]) * sp : 0.0);
          Zq = wave_sumd(on && need_q ? dof(xv[k][4], xv[k][5]) * sq : 0.0);
          fp = __shfl(sp, rank) / Zp;                   // p(v) = ep(v) * fp on this slice
          fq = need_q ? __shfl(sq, rank) / Zq : 0.0;
        }
        // residual weight of one entry in units of fp: max(0, ep - kappa eq); kappa = 0 is p itself
        auto wgt = [&](int i, float kappa) -> float {
          return kappa == 0.f ? ep[i] : fmaxf(fmaf(-kappa, eq[i], ep[i]), 0.f);
        };
        auto slice_sum = [&](float kappa) -> double {
          double acc = 0.0;
#pragma unroll
          for (int k = 0; k < NK; ++k) {
            float g = 0.f;  // fp32 partial of one piece, fp64 across pieces
#pragma unroll
            for (int e = 0; e < E; ++e) g += wgt(k * E + e, kappa);
            acc += (double)g;
          }
          return acc;
        };
        // ---- accept tests along the residual chain
        double c = 0.0, Dn = 1.0, c_prev = 0.0;
        int accepted = -1;
        for (int j = 0; j < K; ++j) {
          const double px = (double)expf((s_lp[j] - Mp) * invT) / Zp;
          const double qx = (double)expf((s_lq[j] - Mq) * invT) / Zq;
          const double cur = fmax(0.0, px - c * qx) / Dn;
          const double u = (double)s_u[j];
          if (qx > 0.0 ? (u < cur / qx) : true) { accepted = si.kids[j]; break; }
          // rejection: next residual coefficient; its normaliser is needed only for a later test,
          // after the last child the bonus scan below computes it as its total
          const double cn = c + Dn;
          if (j == K - 1) { c_prev = c; c = cn; break; }
          // max(0, p - cn q) = fp * max(0, ep - kappa eq) on this slice, kappa = cn fq / fp
          const float kappa = (float)(cn * fq / fp);
          const double sl = block_sum(slice_sum(kappa), red) * fp;
          exchange(gslots, G, rank, ++xtag, 2, xv, ws.err, dlo(sl), dhi(sl));
          double S = 0.0;
          for (int k = 0; k < G; ++k) S += dof(xv[k][0], xv[k][1]);
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
          // The slice's weights are staged in LDS in id order; thread t then scans the 64
          // consecutive entries [64 t, 64 t + 64) (fp32 partials of 8 entries, fp64 above).
          const int wv = t >> 6;
          const double us = (double)s_us;
          for (int attempt = 0; attempt < 2; ++attempt) {
            const float kappa = c == 0.0 ? 0.f : (float)(c * fq / fp);
#pragma unroll
            for (int k = 0; k < NK; ++k) {
              const int i0 = (k * AC_THREADS + t) * E;  // slice-local id of the piece
              float* dst = s_w + wpad(i0);
#pragma unroll
              for (int e = 0; e < E; e += 4)
                *(float4*)(dst + e) = make_float4(wgt(k * E + e, kappa), wgt(k * E + e + 1, kappa),
                                                  wgt(k * E + e + 2, kappa), wgt(k * E + e + 3, kappa));
            }
            __syncthreads();
            const float* mine = s_w + wpad(t * AC_CT);
            double tsum = 0.0;
#pragma unroll
            for (int j = 0; j < AC_CT; j += 8) {
              const float4 x0 = *(const float4*)(mine + j), x1 = *(const float4*)(mine + j + 4);
              tsum += (double)(((((((x0.x + x0.y) + x0.z) + x0.w) + x1.x) + x1.y) + x1.z) + x1.w);
            }
            double incl = wave_scand(tsum, lane);
            if (lane == 63) red.d[wv] = incl;
            __syncthreads();
            double col = 0.0;
            for (int w2 = 0; w2 < AC_NW; ++w2) {
              if (w2 < wv) incl += red.d[w2];
              col += red.d[w2];
            }
            const double sl = col * fp;
            exchange(gslots, G, rank, ++xtag, 2, xv, ws.err, dlo(sl), dhi(sl));
            double before = 0.0, total = 0.0;
            for (int k = 0; k < G; ++k) {
              const double s = dof(xv[k][0], xv[k][1]);
              if (k < rank) before += s;
              total += s;
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
                pre += dof(xv[k][0], xv[k][1]);
                if (pre > thr) { owner = k; break; }
              }
            }
            if (rank == owner) {
              const double lthr = (thr - before) / fp;  // threshold in this slice's units
              if (t == 0) { s_first = 0x7fffffff; s_lpos = -1; }
              __syncthreads();
              {  // the first thread whose inclusive prefix exceeds the threshold: one atomic per wave
                const uint64_t over = __ballot(incl > lthr);
                if (over && lane == 0) atomicMin(&s_first, wv * 64 + __ffsll((long long)over) - 1);
              }
              red.scan1[t] = incl - tsum;  // exclusive prefix of each thread
              __syncthreads();
              const int h = s_first;
              if (h != 0x7fffffff) {
                if (wv == 0) {  // one wave searches thread h's 64 entries, lane e = entry e
                  const float w = s_w[wpad(h * AC_CT) + lane];
                  const double run = red.scan1[h] + wave_scand((double)w, lane);
                  const uint64_t hit = __ballot(w > 0.f && run > lthr);
                  const uint64_t pos = __ballot(w > 0.f);
                  int pick;
                  if (hit) pick = s0 + h * AC_CT + __ffsll((long long)hit) - 1;
                  else if (pos) pick = s0 + h * AC_CT + 63 - __clzll((long long)pos);
                  else pick = min(s0 + h * AC_CT + AC_CT, V) - 1;
                  if (lane == 0) {
                    st_i(&ws.res[item].child, -1);
                    st_i(&ws.res[item].token, pick);
                  }
                }
              } else {  // rounding left the threshold unreached: the highest id with a positive weight
                int lp = -1;
                for (int j = 0; j < AC_CT; ++j) lp = mine[j] > 0.f ? s0 + t * AC_CT + j : lp;
                for (int o = 32; o > 0; o >>= 1) lp = max(lp, __shfl_xor(lp, o));
                if (lane == 0) atomicMax(&s_lpos, lp);
                __syncthreads();
                if (t == 0) {
                  const int pick = s_lpos >= 0 ? s_lpos : min(s0 + AC_SLICE, V) - 1;
                  st_i(&ws.res[item].child, -1);
                  st_i(&ws.res[item].token, pick);
                }
              }
              done_by_me = 1;
            }
            break;
          }
        }
      }

      // ---- the work-group that wrote the row result counts it; the last row of a sequence walks
      if (done_by_me) {
        mem_complete();  // this thread's row-result stores (if any) have completed
        __syncthreads();
        if (t == 0) {
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
            {  // wave w holds nodes 64 w .. 64 w + 63: its ballot is bitset word w
              const uint64_t mb =
                  __ballot(t < N && si.usable[t] && a.tokens[(int64_t)b * N + t] == ld_i(&rr[si.par[t] + 1].token));
              if (lane == 0 && (t >> 6) < SV_MAX_W) s_match[t >> 6] = mb;
            }
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
            a.status[b] = ld_u32(ws.err) ? SV_SEQ_TIMEOUT : (si.bad_token ? SV_SEQ_TOKEN : 0);
            st_u32(&ws.seqdone[b], 0u);  // every row of b has been counted: ready for the next call
          }
          if (t < Dm) a.accept_rows[(int64_t)b * Dm + t] = t < A ? si.path[t] + 1 : 0;
          if (t <= Dm)
            a.out_tokens[(int64_t)b * (Dm + 1) + t] = t < A ? a.tokens[(int64_t)b * N + si.path[t]] : (t == A ? bonus : 0);
        }
      }
    }
  }

  // ---- leave every counter and exchange slot zeroed for the next call
  __syncthreads();
  if (t == 0) {
    mem_complete();
    int last = 1;
    if (G > 1) {
      const uint32_t old = add_u32(ws.gexit + grp, 1u);
      last = old + 1 == (uint32_t)G;  // every member of the group passed its last exchange
      if (last) st_u32(ws.gexit + grp, 0u);
    }
    s_last = last;
  }
  __syncthreads();
  if (s_last && xtag > 0)
    for (int i = t; i < G * 2 * AC_XW; i += AC_THREADS) st_u64(&gslots[i / AC_XW].w[i % AC_XW], 0ull);
  mem_complete();
  __syncthreads();
  if (t == 0) {
    const uint32_t done = add_u32(ws.err + 1, 1u);
    if (done + 1 == gridDim.x) {  // the whole grid has finished: clear the timeout flag
      st_u32(ws.err, 0u);
      st_u32(ws.err + 1, 0u);
    }
  }
}

int groups_G(const sv_accept_args& a) {
  const int G = (a.V + AC_SLICE - 1) / AC_SLICE;
  return G < 1 ? 1 : G;
}
// one group per row, rounded up to a whole number of groups per XCD
int64_t num_groups(const sv_accept_args& a) { return ((int64_t)a.B * (a.N + 1) + 7) / 8 * 8; }

struct WsLayout {
  size_t gexit, seqdone, err, res, xs, total;
};
WsLayout ws_layout(const sv_accept_args& a) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t NG = (size_t)num_groups(a), G = (size_t)groups_G(a);
  WsLayout l{};
  size_t o = 0;
  l.gexit = o; o = up(o + NG * 4);
  l.seqdone = o; o = up(o + (size_t)a.B * 4);
  l.err = o; o = up(o + 8);
  l.res = o; o = up(o + (size_t)a.B * (a.N + 1) * sizeof(RowRes));
  l.xs = o; o = up(o + NG * G * 2 * sizeof(XSlot));
  l.total = o;
  return l;
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
  const int64_t blocks = num_groups(a) * G;
  if (blocks > 0x7fffffff) return SV_ERR_UNSUPPORTED;
  char* base = (char*)a.workspace;
  AccWs ws;
  ws.gexit = (uint32_t*)(base + l.gexit);
  ws.seqdone = (uint32_t*)(base + l.seqdone);
  ws.err = (uint32_t*)(base + l.err);
  ws.res = (RowRes*)(base + l.res);
  ws.xs = (XSlot*)(base + l.xs);
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)blocks);
  if (a.logits_dtype == SV_BF16) {
    if (a.mode == SV_STOCHASTIC) hipLaunchKernelGGL((k_accept<uint16_t, SV_STOCHASTIC>), grid, dim3(AC_THREADS), 0, st, a, G, ws);
    else hipLaunchKernelGGL((k_accept<uint16_t, SV_GREEDY>), grid, dim3(AC_THREADS), 0, st, a, G, ws);
  } else {
    if (a.mode == SV_STOCHASTIC) hipLaunchKernelGGL((k_accept<float, SV_STOCHASTIC>), grid, dim3(AC_THREADS), 0, st, a, G, ws);
    else hipLaunchKernelGGL((k_accept<float, SV_GREEDY>), grid, dim3(AC_THREADS), 0, st, a, G, ws);
  }
  return sv_launch_status();
}
