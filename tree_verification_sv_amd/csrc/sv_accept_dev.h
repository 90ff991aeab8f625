// Device code of the speculative acceptance (the row resolution, its exchanges and walks),
// shared by the acceptance kernel and the one-launch verification step.  The method, the row
// decomposition and the protocol between work-groups are described in sv_accept.hip.
#pragma once
#include <float.h>
#include <math.h>

#include <type_traits>

#include "sv_commit_dev.h"

namespace {

// threads per work-group: 512 for greedy rows (half the work-groups of 256-thread ones,
// fewer to dispatch); stochastic and top-K rows take 256 (smaller barriers and bonus scans,
// and the residual staging fits two work-groups per compute unit) except for batches of
// wide trees (N >= AC_WIDE_N, where the walk cancels most rows) with at least AC_WIDE_ROWS
// rows, where 512 (half the work-groups, one per compute unit for the 155 KB of LDS) measured
// faster on MI355X: 256-node trees at batch 16 (4112 rows) 3.38 -> 2.93 ms per step, at batch
// 8 even; 60-node trees were slower with 512 at every batch (batch 64, 3904 rows: 1.11 ->
// 1.18 ms; batch 1: 13%), and so were 768-row chains.  Rows that do not start on 16 bytes
// (`aligned` false) take 256 in these modes: their element-wise loads need more registers
// than a 512-thread work-group has.
constexpr int AC_WIDE_ROWS = 2048;
constexpr int AC_WIDE_N = 128;
int acc_threads(const sv_accept_args& a, bool aligned) {
  if (a.mode == SV_GREEDY) return 512;
  return aligned && a.N >= AC_WIDE_N && (int64_t)a.B * (a.N + 1) >= AC_WIDE_ROWS ? 512 : 256;
}
constexpr int AC_NWMAX = 8;                    // waves per work-group at most
// vocabulary entries per thread: 8 pieces of 16 bytes (64 bf16 / 32 fp32 logits), so a
// work-group's slice is 8 * 16 bytes per thread
template <typename T> constexpr int ac_ct() { return 8 * (16 / (int)sizeof(T)); }
template <typename T, int TH> constexpr int ac_slice() { return TH * ac_ct<T>(); }
constexpr int AC_MAXG = 64;                    // work-groups per row group (vocabulary up to 1M entries)
constexpr int AC_BLIST = 4352;                 // greedy batch streams: rows of the batch at most
constexpr int AC_LEAFROW = 1 << 30;            // greedy batch streams: a stream entry that is a leaf stop row
constexpr int AC_XW = 8;                       // tagged words per exchange slot
constexpr int AC_XV = 6;                       // words an exchange carries at most
constexpr uint32_t AC_SPIN_LIMIT = 1u << 20;   // bounded wait for a group partner (polls)

struct XSlot {      // one work-group's partials for one exchange: (tag << 32) | payload
  uint64_t w[AC_XW];
};

// A resolved row, one 64-bit word (0 = not resolved in this call): bit 63 set, bit 62 set
// when the row's statistics are not finite (AC_RES_BAD), bits 32..61 the first accepted
// child node + 1 (0 when all children were rejected), bits 0..31 the bonus token if the walk
// stops here (stochastic) / the argmax (greedy).
constexpr uint64_t AC_RES_BAD = 1ull << 62;
__device__ __forceinline__ uint64_t res_word(int child, int token) {
  return (1ull << 63) | ((uint64_t)(uint32_t)(child + 1) << 32) | (uint32_t)token;
}
__device__ __forceinline__ bool res_ready(uint64_t v) { return (v >> 63) != 0; }
__device__ __forceinline__ bool res_bad(uint64_t v) { return (v & AC_RES_BAD) != 0; }
__device__ __forceinline__ int res_child(uint64_t v) { return (int)((v >> 32) & 0x3fffffffu) - 1; }
__device__ __forceinline__ int res_token(uint64_t v) { return (int)(uint32_t)v; }
// Greedy argmax scans start from (-inf, no id) and take an entry only when it is larger, so a
// row without an entry above -inf (every entry -inf or NaN) ends with no id: its argmax is then
// id 0, the lowest id of an all-equal row.
constexpr int AC_NO_ID = 0x7fffffff;
__device__ __forceinline__ int greedy_token(int arg) { return arg == AC_NO_ID ? 0 : arg; }
constexpr uint32_t AC_FRONT_BUSY = 0xffffffffu;  // the walk's frontier is claimed by a work-group

struct AccWs {        // workspace views
  uint32_t* gexit;    // [groups] group exit counters
  uint32_t* seqdone;  // [B] rows resolved per sequence (greedy)
  uint32_t* err;      // [0] wait-timeout flag, [1] work-groups exited, [2] greedy batch streams: rows taken
  uint64_t* res;      // [B, N+1] resolved rows
  uint32_t* frontier; // [B] stochastic walk: the first row of the path not yet resolved
  uint32_t* cancel;   // [B] stochastic walk finished: remaining rows are not needed
  uint32_t* seqexit;  // [B] stochastic: work-groups of the sequence that have exited
  XSlot* xs;          // [groups * G * 2]: (group * G + rank) * 2 + exchange parity
};

template <typename T>
__device__ __forceinline__ float ldf(const T* p, int64_t i) { return load_as_f32<T>(p, i); }
// raw bits of one logit, and their value (split so that the conversion can be placed late)
template <typename T> __device__ __forceinline__ uint32_t ldraw(const T* p, int64_t i);
template <> __device__ __forceinline__ uint32_t ldraw<float>(const float* p, int64_t i) { return __float_as_uint(p[i]); }
template <> __device__ __forceinline__ uint32_t ldraw<uint16_t>(const uint16_t* p, int64_t i) { return p[i]; }
template <typename T> __device__ __forceinline__ float rawf(uint32_t b) {
  return sizeof(T) == 2 ? __uint_as_float(b << 16) : __uint_as_float(b);
}

// ---------------------------------------------------------------- reductions
// Cross-lane steps use DPP moves (a few cycles each) instead of LDS permutes.
// Within a 16-lane row: quad permutations and the row mirrors for butterflies,
// row shifts for the scan; across rows: lane reads for reductions and the row
// broadcasts of lanes 15 and 31 for the scan.  Results are identical in every
// lane, and the order of operations is fixed, so every work-group that reduces
// the same values gets the same bits.
enum : int {
  DPP_XOR1 = 0xB1,         // quad_perm [1, 0, 3, 2]
  DPP_XOR2 = 0x4E,         // quad_perm [2, 3, 0, 1]
  DPP_ROW_SHR1 = 0x111,    // row_shr:n = 0x110 + n
  DPP_ROW_MIRROR = 0x140,
  DPP_ROW_HALF_MIRROR = 0x141,
  DPP_ROW_BCAST15 = 0x142,
  DPP_ROW_BCAST31 = 0x143,
};
template <int CTRL, int ROWS = 0xf, bool BC = true>
__device__ __forceinline__ uint32_t dpp32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xf, BC);
}
template <int CTRL, int ROWS = 0xf, bool BC = true>
__device__ __forceinline__ float dppf(float x) { return __uint_as_float(dpp32<CTRL, ROWS, BC>(__float_as_uint(x))); }
template <int CTRL, int ROWS = 0xf, bool BC = true>
__device__ __forceinline__ double dppd(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint64_t lo = dpp32<CTRL, ROWS, BC>((uint32_t)b), hi = dpp32<CTRL, ROWS, BC>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)((hi << 32) | lo));
}
__device__ __forceinline__ float lanef(float x, int l) { return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), l)); }
__device__ __forceinline__ double laned(double x, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((uint32_t)b, l);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)((hi << 32) | lo));
}
__device__ __forceinline__ float wave_maxf(float x) {
  x = fmaxf(x, dppf<DPP_XOR1>(x));
  x = fmaxf(x, dppf<DPP_XOR2>(x));
  x = fmaxf(x, dppf<DPP_ROW_HALF_MIRROR>(x));
  x = fmaxf(x, dppf<DPP_ROW_MIRROR>(x));  // every lane of a row holds the row's maximum
  return fmaxf(fmaxf(lanef(x, 0), lanef(x, 16)), fmaxf(lanef(x, 32), lanef(x, 48)));
}
__device__ __forceinline__ double wave_sumd(double x) {
  x += dppd<DPP_XOR1>(x);
  x += dppd<DPP_XOR2>(x);
  x += dppd<DPP_ROW_HALF_MIRROR>(x);
  x += dppd<DPP_ROW_MIRROR>(x);  // every lane of a row holds the row's sum
  return (laned(x, 0) + laned(x, 16)) + (laned(x, 32) + laned(x, 48));
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
  (void)lane;
  x += dppd<DPP_ROW_SHR1 + 0>(x);  // shifted-in lanes read 0
  x += dppd<DPP_ROW_SHR1 + 1>(x);
  x += dppd<DPP_ROW_SHR1 + 3>(x);
  x += dppd<DPP_ROW_SHR1 + 7>(x);  // inclusive scan within each row of 16
  x += dppd<DPP_ROW_BCAST15, 0xa, false>(x);  // rows 1, 3 add lane 15 of the row before
  x += dppd<DPP_ROW_BCAST31, 0xc, false>(x);  // rows 2, 3 add lane 31
  return x;
}

struct Red {
  float f[AC_NWMAX];
  double d[AC_NWMAX], d2[AC_NWMAX];
  int i[AC_NWMAX];
};

template <int TH>
__device__ __forceinline__ float block_max(float x, Red& r) {
  x = wave_maxf(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.f[threadIdx.x >> 6] = x;
  __syncthreads();
  float m = r.f[0];
  for (int k = 1; k < TH / 64; ++k) m = fmaxf(m, r.f[k]);
  return m;
}
template <int TH>
__device__ __forceinline__ double block_sum(double x, Red& r) {
  x = wave_sumd(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.d[threadIdx.x >> 6] = x;
  __syncthreads();
  double s = 0.0;
  for (int k = 0; k < TH / 64; ++k) s += r.d[k];
  return s;
}
// two block sums with one pair of barriers
template <int TH>
__device__ __forceinline__ void block_sum2(double& x, double& y, Red& r) {
  x = wave_sumd(x);
  y = wave_sumd(y);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    r.d[threadIdx.x >> 6] = x;
    r.d2[threadIdx.x >> 6] = y;
  }
  __syncthreads();
  double s = 0.0, s2 = 0.0;
  for (int k = 0; k < TH / 64; ++k) {
    s += r.d[k];
    s2 += r.d2[k];
  }
  x = s;
  y = s2;
}
template <int TH>
__device__ __forceinline__ void block_argmax(float& v, int& i, Red& r) {
  wave_argmax(v, i);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { r.f[threadIdx.x >> 6] = v; r.i[threadIdx.x >> 6] = i; }
  __syncthreads();
  v = r.f[0];
  i = r.i[0];
  for (int k = 1; k < TH / 64; ++k)
    if (r.f[k] > v || (r.f[k] == v && r.i[k] < i)) { v = r.f[k]; i = r.i[k]; }
}

// ---------------------------------------------------------------- cross-work-group messages
// Values crossing work-groups are written with relaxed device-scope atomic
// stores and read with relaxed device-scope atomic loads (both coherent at
// device scope: on gfx950 they bypass the per-XCD caches that are not
// coherent with each other).  Exchange words carry their tag in the same
// 64-bit word as the payload.  Row results are published before the
// per-sequence counter: the writer waits for its stores to complete
// (s_waitcnt) and then bumps the counter; the reader issues its loads of the
// results only after the counter value it depends on has returned.  Neither
// order needs a cache write-back or invalidation, because no plain
// (non-atomic) store carries data between work-groups.  Device-scope
// release/acquire on these counters was measured and rejected: a release
// writes back the XCD's whole L2 and an acquire invalidates it, which evicts
// the logits rows other work-groups are streaming (the 60-node bf16 tree step
// went from 33 to 60 us, the 64x32 greedy acceptance from 84 to 188 us).
#define AGENT __HIP_MEMORY_SCOPE_AGENT
__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, AGENT); }
__device__ __forceinline__ void st_u64(uint64_t* p, uint64_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, AGENT); }
__device__ __forceinline__ uint32_t ld_u32(uint32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, AGENT); }
__device__ __forceinline__ uint64_t ld_u64(uint64_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, AGENT); }
__device__ __forceinline__ uint32_t add_u32(uint32_t* p, uint32_t v) { return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, AGENT); }
__device__ __forceinline__ bool cas_u32(uint32_t* p, uint32_t expect, uint32_t v) {
  return __hip_atomic_compare_exchange_strong(p, &expect, v, __ATOMIC_RELAXED, __ATOMIC_RELAXED, AGENT);
}
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
// cancel (nullable): the sequence's walk-finished flag.  It is read once per
// exchange (alongside the polls) and while waiting; once it is seen set, the
// work-group's sticky flag *xc is set and the exchange returns true (the row's
// result is no longer needed; a member that waits for a member that has left
// sees the flag too).
template <int TH>
__device__ __forceinline__ bool exchange(XSlot* gs, int G, int rank, uint32_t tag, int nw, uint32_t (*xv)[AC_XV],
                                         uint32_t* err, uint32_t* cancel, int* xc, uint32_t w0, uint32_t w1,
                                         uint32_t w2 = 0, uint32_t w3 = 0, uint32_t w4 = 0, uint32_t w5 = 0) {
  const int t = threadIdx.x;
  const int par = tag & 1;
  if (t < nw) {
    const uint32_t w = t == 0 ? w0 : t == 1 ? w1 : t == 2 ? w2 : t == 3 ? w3 : t == 4 ? w4 : w5;
    st_u64(&gs[rank * 2 + par].w[t], ((uint64_t)tag << 32) | w);
  }
  const uint32_t c0 = (cancel && t == 0) ? ld_u32(cancel) : 0u;  // overlaps the polls below
  for (int q = t; q < G * nw; q += TH) {
    const int k = q / nw, i = q - k * nw;
    uint64_t* p = &gs[k * 2 + par].w[i];
    uint64_t v = ld_u64(p);
    uint32_t spins = 0;
    while ((uint32_t)(v >> 32) != tag) {
      ++spins;
      if ((spins & 63) == 0 && (spins > AC_SPIN_LIMIT || ld_u32(err) != 0)) {
        st_u32(err, 1u);
        break;
      }
      // every fourth poll also reads the cancel flag; both loads are in flight together
      const bool chk = cancel != nullptr && (spins & 3) == 0;
      v = ld_u64(p);
      const uint32_t cv = chk ? ld_u32(cancel) : 0u;
      if (cv != 0u) {
        *xc = 1;
        break;
      }
    }
    xv[k][i] = (uint32_t)v;
  }
  if (c0) *xc = 1;
  __syncthreads();
  return *xc != 0;
}

struct SeqInfo {    // per-sequence facts every work-group derives the same way
  int32_t tok[SV_MAX_N];
  int16_t par[SV_MAX_N];
  uint8_t usable[SV_MAX_N];
  int8_t dep[SV_MAX_N];          // nodes on the root path (0: invalid node)
  uint8_t haskid[SV_MAX_N + 1];  // row has a usable child
  int16_t kids[SV_MAX_N];     // usable children of the current row, ascending
  int32_t wcount[AC_NWMAX];
  int32_t wlive[AC_NWMAX];
  int32_t K;                  // number of usable children of the current row
  int32_t nlive;              // rows this sequence resolves
  int32_t bad_token;
  int32_t path[SV_MAX_DEPTH];
  int32_t flag;
};

// per-sequence facts: usable nodes, rows with children, live-row count (one node per thread).
// The loads are issued by seq_fetch ahead of the slice loads, so that waiting for them does
// not wait for the slice.
struct SeqRaw {
  int32_t tok, par, dep;
};
__device__ __forceinline__ SeqRaw seq_fetch(const sv_accept_args& a, int b) {
  SeqRaw r{0, -2, 0};
  const int t = threadIdx.x;
  if (t < a.N) {
    const int64_t i = (int64_t)b * a.N + t;
    r.tok = a.tokens[i];
    r.par = a.parents[i];
    // without a depth array the load takes the parents (the value is then unused): an
    // unconditional load keeps the kernel free of scratch
    r.dep = (a.depth ? a.depth : a.parents)[i];
  }
  return r;
}
template <int TH>
__device__ __forceinline__ void seq_facts(const sv_accept_args& a, const SeqRaw& sr, SeqInfo& si) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int N = a.N;
  for (int x = t; x <= N; x += TH) si.haskid[x] = 0;
  if (t == 0) si.bad_token = 0;
  __syncthreads();
  bool u = false;
  if (t < N) {
    // an out-of-range parent is staged as -2 (only usable nodes' parents are read later)
    si.par[t] = (int16_t)(sr.par >= -1 && sr.par < N ? sr.par : -2);
    si.tok[t] = sr.tok;
  }
  int dep = sr.dep;
  if (!a.depth) {  // uniform: no depth array, derive it from the staged parents
    // the rule of the tree mask: the number of nodes on the root path when the walk reaches
    // parent -1 through in-range parents within max_depth nodes, else 0 (a cycle never
    // reaches -1, so it ends on the depth limit)
    __syncthreads();
    dep = 0;
    if (t < N) {
      int cur = t, cnt = 1;
#pragma unroll 1
      for (int s = 0; s < SV_MAX_DEPTH; ++s) {  // at most max_depth - 1 <= 15 steps up
        const int p = si.par[cur];
        if (p == -1) { dep = cnt; break; }
        if (p < 0 || cnt >= a.max_depth) break;
        ++cnt;
        cur = p;
      }
    }
  }
  if (t < N) {  // the thread's own staged values (no barrier needed to read them back)
    const int pr = si.par[t], tok = si.tok[t];
    const bool ok = tok >= 0 && tok < a.V;
    if (!ok) si.bad_token = 1;  // every writer stores the same value
    u = ok && dep > 0 && pr != -2;
    if (u) si.haskid[pr + 1] = 1;
    si.dep[t] = (int8_t)(u ? dep : 0);
  }
  if (t < SV_MAX_N) si.usable[t] = u;
  __syncthreads();
  // live rows: greedy -- rows with a usable child; stochastic -- rows of usable nodes
  const bool live = a.mode == SV_GREEDY ? (t >= 1 && t <= N && si.haskid[t]) : u;
  const uint64_t lm = __ballot(live);
  if (lane == 0) si.wlive[wv] = __popcll(lm);
  __syncthreads();
  if (t == 0) {
    int nl = 0;
    for (int k = 0; k < TH / 64; ++k) nl += si.wlive[k];
    si.nlive = nl + 1;  // + the root row
  }
  __syncthreads();
}

// usable children of row r in ascending index, from the sequence facts
template <int TH>
__device__ __forceinline__ void row_kids(int N, int r, SeqInfo& si) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const bool kid = t < N && si.usable[t] && si.par[t] + 1 == r;
  const uint64_t m = __ballot(kid);
  if (lane == 0) si.wcount[wv] = __popcll(m);
  __syncthreads();
  int off = 0, K = 0;
  for (int k = 0; k < TH / 64; ++k) {
    if (k < wv) off += si.wcount[k];
    K += si.wcount[k];
  }
  if (kid) si.kids[off + __popcll(m & ((1ull << lane) - 1ull))] = t;
  if (t == 0) si.K = K;
  __syncthreads();
}

__device__ __forceinline__ bool row_live(const sv_accept_args& a, const SeqInfo& si, int r) {
  if (r == 0) return true;
  return a.mode == SV_GREEDY ? si.haskid[r] != 0 : si.usable[r - 1] != 0;
}

// Where a work-group sits among the acceptance work-groups of its launch.
struct AccRole {
  int bid;       // index among the acceptance work-groups of its launch (they start on a multiple of 8)
  int nblocks;   // acceptance work-groups of the launch
  int seq_wgs;   // acceptance work-groups per sequence
};

// ---------------------------------------------------------------- slice loads
template <typename T> struct Piece {
  static constexpr int E = 16 / sizeof(T);  // entries per 16-byte piece
  static constexpr int NK = ac_ct<T>() / E;  // pieces per thread
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
template <typename T, int TH>
__device__ __forceinline__ int piece_v(int s0, int k, int t) { return s0 + (k * TH + t) * Piece<T>::E; }

// Cache policy of the slice loads: non-temporal (nt).  Every logits byte is read once, so the
// lines are marked for early eviction and leave the caches to the data that is reused (the
// attention's query rows, the exchange words).  MI355X, one-launch 60-node tree step: 33.2 ->
// 32.2 us.
constexpr int AC_NT = 2;
// Thread t's pieces of one logits row.  `aligned`: the row starts on 16 bytes
// and V * sizeof(T) is a multiple of 16, so each piece lies wholly inside or
// wholly past the row; the loads then go through a buffer resource sized to
// the row, which returns zeros for pieces past V.  Otherwise entries are
// loaded one by one and entries past V read as the lowest value.  Callers
// treat pieces starting at or past V as absent.  `present` false (uniform):
// the row is not needed; aligned loads are still issued, against an empty
// range, so they return zeros without touching memory and the register
// assignment does not depend on the branch.
template <typename T, int TH>
__device__ __forceinline__ void load_pieces(const T* row, int s0, int V, bool aligned, int t,
                                            uint4 (&raw)[Piece<T>::NK], bool present = true) {
  constexpr int E = Piece<T>::E;
  if (aligned) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)row, 0, present ? V * (int)sizeof(T) : 0, 0x00020000);
    const int vo = (s0 + t * E) * (int)sizeof(T);
#pragma unroll
    for (int k = 0; k < Piece<T>::NK; ++k)
      raw[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, k * TH * 16, AC_NT));
  } else if (!present) {
#pragma unroll
    for (int k = 0; k < Piece<T>::NK; ++k) raw[k] = make_uint4(0u, 0u, 0u, 0u);
  } else {
#pragma unroll
    for (int k = 0; k < Piece<T>::NK; ++k) {
      const int v = piece_v<T, TH>(s0, k, t);
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

// This thread's argmax over a whole logits row (lowest id on ties), one TH-thread slice at a time
// with the next slice's loads in flight; a thread visits its entries in ascending id.
template <typename T, int TH>
__device__ __forceinline__ void argmax_row(const T* row, int V, bool aligned, int t, float& best, int& arg) {
  constexpr int E = Piece<T>::E, NK = Piece<T>::NK;
  const int ns = (V + ac_slice<T, TH>() - 1) / ac_slice<T, TH>();
  uint4 r0[NK], r1[NK];
  auto consume = [&](const uint4 (&raw)[NK], int gs) {
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      float x[E];
      unpack16<T>(raw[k], x);
      const int v = piece_v<T, TH>(gs * ac_slice<T, TH>(), k, t);
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (v + e < V && x[e] > best) { best = x[e]; arg = v + e; }
    }
  };
  load_pieces<T, TH>(row, 0, V, aligned, t, r0);
  for (int gs = 0; gs < ns; gs += 2) {
    if (gs + 1 < ns) load_pieces<T, TH>(row, (gs + 1) * ac_slice<T, TH>(), V, aligned, t, r1);
    consume(r0, gs);
    if (gs + 1 >= ns) break;
    if (gs + 2 < ns) load_pieces<T, TH>(row, (gs + 2) * ac_slice<T, TH>(), V, aligned, t, r0);
    consume(r1, gs + 1);
  }
}

// ---------------------------------------------------------------- a stop row without children
// A walk that accepts a node whose row has no usable child stops there, and the bonus is a draw
// from p = softmax(l / T) of that row alone: the smallest id whose ascending cumulative weight
// exp2((x - M) l2T) exceeds u times the row total (M the row maximum).  Such rows are resolved
// on demand by the walker's work-group: wave w streams the contiguous pieces of R rounds of 64
// pieces, so wave totals are the row's prefix sums in id order.  Pass 1 takes the maximum;
// pass 2 sums the fp32 piece weights in fp64 per wave and per batch of AC_LB rounds (kept in
// LDS); the wave holding the threshold re-reads the one batch that crosses it (now in the L2
// cache) and scans it round by round.  Returns the row-result word: token 0 with AC_RES_BAD
// when the row has no finite positive total, as a row resolved by its group reports.
// s_bs: LDS for NW * ceil(R / AC_LB) doubles (at most 512 for any V the acceptance accepts).
constexpr int AC_LB = 8;  // rounds per batch: loads in flight per lane
template <typename T, int TH>
__device__ __forceinline__ uint64_t leaf_bonus(const T* row, int V, bool aligned, float l2T, float u, Red& red, double* s_bs,
                               int32_t* s_pick) {
  constexpr int E = Piece<T>::E, NW = TH / 64;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int pieces = (V + E - 1) / E;
  const int R = ((pieces + 63) / 64 + NW - 1) / NW;  // rounds per wave
  const int NB = (R + AC_LB - 1) / AC_LB;            // batches per wave
  const int pw = wv * R * 64;                        // first piece of this wave
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)row, 0, aligned ? V * (int)sizeof(T) : 0, 0x00020000);
  auto load = [&](int pc) -> uint4 {  // piece pc (entries past V read as the lowest value)
    if (aligned) return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, pc * 16, 0, 0));
    uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int v = pc * E + e;
      const T x = v < V ? row[v] : lowest_of<T>();
      wd[e * sizeof(T) / 4] |= bits_of(x) << (8 * ((e * sizeof(T)) % 4));
    }
    return make_uint4(wd[0], wd[1], wd[2], wd[3]);
  };
  auto valid = [&](int j, int pc) { return j < R && pc < pieces; };  // round j of this wave
  // ---- pass 1: the maximum
  float mx = -FLT_MAX;
  for (int j0 = 0; j0 < R; j0 += AC_LB) {
    uint4 raw[AC_LB];
#pragma unroll
    for (int k = 0; k < AC_LB; ++k) raw[k] = load(pw + (j0 + k) * 64 + lane);
#pragma unroll
    for (int k = 0; k < AC_LB; ++k) {
      const int pc = pw + (j0 + k) * 64 + lane;
      float x[E];
      unpack16<T>(raw[k], x);
#pragma unroll
      for (int e = 0; e < E; ++e) mx = valid(j0 + k, pc) && pc * E + e < V ? fmaxf(mx, x[e]) : mx;
    }
  }
  const float M = block_max<TH>(mx, red);
  const float o = M * l2T;  // exp2(x * l2T - o): one FMA per entry
  auto weights = [&](const uint4& raw, int pc, bool on, float (&w)[E]) -> float {
    float x[E], g = 0.f;
    unpack16<T>(raw, x);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      w[e] = on && pc * E + e < V ? __builtin_amdgcn_exp2f(fmaf(x[e], l2T, -o)) : 0.f;
      g += w[e];
    }
    return g;
  };
  // ---- pass 2: batch and wave totals
  double wsum = 0.0;
  for (int j0 = 0, bi = 0; j0 < R; j0 += AC_LB, ++bi) {
    uint4 raw[AC_LB];
#pragma unroll
    for (int k = 0; k < AC_LB; ++k) raw[k] = load(pw + (j0 + k) * 64 + lane);
    double bs = 0.0;
#pragma unroll
    for (int k = 0; k < AC_LB; ++k) {
      const int pc = pw + (j0 + k) * 64 + lane;
      float w[E];
      bs += (double)weights(raw[k], pc, valid(j0 + k, pc), w);
    }
    bs = wave_sumd(bs);
    if (lane == 0) s_bs[wv * NB + bi] = bs;
    wsum += bs;
  }
  __syncthreads();
  if (lane == 0) red.d[wv] = wsum;
  __syncthreads();
  double Z = 0.0;
  for (int k = 0; k < NW; ++k) Z += red.d[k];
  if (!(Z > 0.0 && Z < (double)INFINITY)) return res_word(-1, 0) | AC_RES_BAD;  // uniform
  const double thr = (double)u * Z;
  // the wave, then the batch, whose inclusive prefix first exceeds the threshold (rounding that
  // leaves it unreached: the last one with a positive total)
  int ow = -1;
  double before = 0.0;
  {
    double run = 0.0;
    int lastw = 0;
    double lastb = 0.0;
    for (int k = 0; k < NW; ++k) {
      const double d = red.d[k];
      if (ow < 0 && d > 0.0 && run + d > thr) { ow = k; before = run; }
      if (d > 0.0) { lastw = k; lastb = run; }
      run += d;
    }
    if (ow < 0) { ow = lastw; before = lastb; }
  }
  if (t == 0) *s_pick = -1;
  __syncthreads();
  if (wv == ow) {
    // batch: lane i takes batch i's total (NB <= 64)
    const double bsl = lane < NB ? s_bs[ow * NB + lane] : 0.0;
    const double incl = wave_scand(bsl, lane) + before;
    const uint64_t over = __ballot(lane < NB && bsl > 0.0 && incl > thr);
    const uint64_t pos = __ballot(lane < NB && bsl > 0.0);
    const int bi = over ? __ffsll((long long)over) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
    double run = laned(incl - bsl, bi);  // cumulative weight before the batch
    const int j0 = bi * AC_LB;
    uint4 raw[AC_LB];
#pragma unroll
    for (int k = 0; k < AC_LB; ++k) raw[k] = load(pw + (j0 + k) * 64 + lane);
    bool found = false;  // uniform over the wave
    int lastpos = -1;
#pragma unroll
    for (int k = 0; k < AC_LB; ++k) {
      if (!found) {
        const int pc = pw + (j0 + k) * 64 + lane;
        float w[E];
        const float g = weights(raw[k], pc, valid(j0 + k, pc), w);
        int lp = -1;
#pragma unroll
        for (int e = 0; e < E; ++e) lp = w[e] > 0.f ? pc * E + e : lp;
        for (int s2 = 32; s2 > 0; s2 >>= 1) lp = max(lp, __shfl_xor(lp, s2));
        lastpos = max(lastpos, lp);
        const double ic = wave_scand((double)g, lane) + run;
        const uint64_t ov = __ballot(g > 0.f && ic > thr);
        if (ov) {  // lane h holds the crossing piece; it walks its E entries
          const int h = __ffsll((long long)ov) - 1;
          if (lane == h) {
            double r2 = ic - (double)g;
            int pick = -1, last = -1;
#pragma unroll
            for (int e = 0; e < E; ++e) {
              if (w[e] > 0.f) {
                last = pc * E + e;
                r2 += (double)w[e];
                if (pick < 0 && r2 > thr) pick = pc * E + e;
              }
            }
            *s_pick = pick >= 0 ? pick : last;
          }
          found = true;
        } else {
          run = laned(ic, 63);
        }
      }
    }
    if (!found && lane == 0) *s_pick = lastpos >= 0 ? lastpos : V - 1;
  }
  __syncthreads();
  return res_word(-1, *s_pick);
}

// ---------------------------------------------------------------- the kernel
// ALIGNED: every logits row starts on 16 bytes (decided on the host; a compile-time choice
// keeps the two load paths from meeting in one register assignment)

// The acceptance body's LDS.
template <typename T, int TH, bool STO>
struct AccShared {
  Red red;
  SeqInfo si;
  int32_t s_last, s_hit, s_first, s_lpos;
  uint64_t s_match[SV_MAX_W];
  uint32_t xv[AC_MAXG][AC_XV];                          // collected group partials
  float s_lp[SV_MAX_N], s_lq[SV_MAX_N], s_u[SV_MAX_N];  // per child: logits at its token, u_accept
  float s_us;                                           // u_sample of the row
  alignas(16) float s_g[STO ? Piece<T>::NK * TH : 4];   // bonus: per-piece sums [k][t] (a walker's leaf
                                                        // draw: batch totals, doubles)
  double s_col[Piece<T>::NK];                           // ... and their row totals
  int s_xc, s_claim, s_fin;  // walk finished (sticky); stochastic walk: claimed row, finisher
  int s_leaf;                // stochastic walk: a stop row without children, drawn by the walker
  int s_bad;                 // the stop row's statistics were not finite
  int s_to;                  // a bounded wait of this call expired: no commit, status 7
  uint64_t rr[STO ? SV_MAX_N + 1 : 1];  // stochastic walk: the sequence's row results
  int16_t rows[STO ? 1 : SV_MAX_N + 1];  // greedy row streams: the rows the walk needs, ascending
  uint8_t bflag[STO ? 1 : AC_BLIST];     // greedy batch streams: row of the batch needed
  uint16_t blist[STO ? 1 : AC_BLIST];    // ... the needed rows of the batch, ascending
  int32_t bscan[AC_NWMAX + 1];           // ... block scan
  uint16_t bseq[STO ? 1 : AC_BLIST / 2 + 1];  // ... first list position of each sequence
  int32_t ring[4];                       // ... this work-group's next rows (list positions or leaf rows)
  int32_t q_inj;                         // ... a leaf stop row waiting for a ring slot
  int32_t q_pend, q_ended;               // ... row j + D's entry when not from the counter; counter run out
  int32_t rowarg[STO ? 1 : SV_MAX_N + 1];  // greedy chains: argmax of each followed row
  double nscore[STO ? 1 : SV_MAX_N];       // threshold chains: score of each passing node
  int32_t q_head, q_tail;                  // ... rows to follow: S.rows[q_head .. q_tail)
};

// The greedy walk of sequence b, by the work-group that counted its last needed row: the
// accepted node is the deepest one (lowest index on ties) whose whole root path matches the
// parents' argmax; the bonus is the stop row's argmax (for a row without a usable child, which
// no work-group resolved, streamed here -- or, with DEFER, left to the caller, who gets the
// stream entry AC_LEAFROW | A << 13 | (batch row) back and writes the bonus token itself).
// Writes the outputs, clears the sequence's row results and counter for the next call, and
// commits the accepted path when asked to.  Returns -1 when nothing is left to the caller.
template <typename T, int TH, bool DEFER = false>
__device__ __forceinline__ int greedy_walk(const sv_accept_args& a, const AccWs& ws, const sv_commit_args& cm, int32_t has_cm,
                            int b, bool aligned, AccShared<T, TH, false>& S) {
  auto row_token = [](uint64_t v) { return res_token(v); };
  const int t = threadIdx.x, lane = t & 63;
  const int N = a.N, V = a.V;
  SeqInfo& si = S.si;
  Red& red = S.red;
  uint64_t* s_match = S.s_match;
  int32_t &s_hit = S.s_hit, &s_to = S.s_to;
  // ----------------------------------------------------- walk of sequence b
  if (t == 0) s_to = ld_u32(ws.err) != 0;  // read after the barriers below
  int A = 0, stop_row = 0, bonus = 0, left = -1;
  uint64_t* rr = ws.res + (int64_t)b * (N + 1);
  {
    // match[i]: token equals its parent row's argmax; accepted: the whole root path matches
    {  // wave w holds nodes 64 w .. 64 w + 63: its ballot is bitset word w
      const uint64_t mb =
          __ballot(t < N && si.usable[t] && a.tokens[(int64_t)b * N + t] == row_token(ld_u64(&rr[si.par[t] + 1])));
      if (lane == 0 && (t >> 6) < SV_MAX_W) s_match[t >> 6] = mb;
    }
    __syncthreads();
    int key = -1;
    if (t < N && si.usable[t]) {
      // up the root path of t (si.dep[t] nodes, all in range for a usable node): t is
      // accepted when every node on it matches
      const int dt = si.dep[t];
      bool ok = true;
      int cur = t;
      for (int st = 0; st < dt; ++st) {
        ok &= ((s_match[cur >> 6] >> (cur & 63)) & 1ull) != 0;
        cur = si.par[cur];
      }
      if (ok) key = (dt << 9) | (511 - t);  // deepest, then lowest index
    }
    {
      float kv = (float)key;
      int ki = key;
      block_argmax<TH>(kv, ki, red);
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
      if (t == 0) s_hit = row_token(ld_u64(&rr[stop_row]));
      __syncthreads();
      bonus = s_hit;
    } else if constexpr (DEFER) {
      left = AC_LEAFROW | (A << 13) | (b * (N + 1) + stop_row);
    } else {
      // leaf stop row: argmax by this work-group, one slice at a time with the next
      // slice's loads in flight (a thread visits its entries in ascending id)
      const T* srow = (const T*)a.target_logits + ((int64_t)b * (N + 1) + stop_row) * V;
      float best = -INFINITY;
      int arg = AC_NO_ID;
      argmax_row<T, TH>(srow, V, aligned, t, best, arg);
      block_argmax<TH>(best, arg, red);
      bonus = greedy_token(arg);
    }
  }
  __syncthreads();
  const int Dm = a.max_depth;
  if (t == 0) {
    a.accept_len[b] = A;
    a.num_out[b] = A + 1;
    a.stop_row[b] = stop_row;
    a.status[b] = s_to ? SV_SEQ_TIMEOUT : (si.bad_token ? SV_SEQ_TOKEN : 0);
    st_u32(&ws.seqdone[b], 0u);  // every row of b has been counted: ready for the next call
  }
  // every row result of b has been read: leave them cleared for the next call
  for (int x = t; x <= N; x += TH) st_u64(&rr[x], 0ull);
  if (t < Dm) a.accept_rows[(int64_t)b * Dm + t] = t < A ? si.path[t] + 1 : 0;
  if (t <= Dm && !(t == A && left >= 0)) {
    int tt = t;  // opaque copy: the lane's address is formed here, not held in registers across callers' loops
    asm volatile("" : "+v"(tt));
    a.out_tokens[(int64_t)b * (Dm + 1) + tt] = tt < A ? a.tokens[(int64_t)b * N + si.path[tt]] : (tt == A ? bonus : 0);
  }
  // the accepted path into the cache (nothing after a timeout: the path may be wrong)
  if (has_cm) svc::walker_commit(cm, b, s_to ? 0 : A, si.path);
  return left;
}

// Greedy batches whose B (N + 1) rows fit the LDS list: every work-group derives the batch's
// needed rows -- the root and the rows with a usable child, by the rule of the sequence facts --
// as one ascending list and streams whole rows of it: its first rows by its index, the rest taken
// from a device-wide counter, each early enough (two slices before it is needed, or two rows ahead for rows of fewer than three
// slices) that the counter's round trip hides behind the loads.  A
// work-group streams its rows' slices with the next slice's loads in flight across row
// boundaries, stores each row's argmax (lowest id on ties) as its result word and counts the
// row for its sequence; the work-group that counts a sequence's last needed row walks it at
// once, while the stream goes on, so the walks spread over the launch instead of piling up
// at its end.  A walk that stops on a row without children (never streamed) hands that row
// back: it joins the work-group's own stream, and its argmax becomes the bonus token.  No
// work-group waits for another; a timeout word already set when the launch starts is reported
// as status 7 by every walk and cleared by the last work-group.
template <typename T, bool ALIGNED, int TH>
__device__ __forceinline__ void greedy_batch_body(const sv_accept_args& a, const AccWs& ws, const sv_commit_args& cm,
                                                  int32_t has_cm, AccShared<T, TH, false>& S) {
  constexpr int E = Piece<T>::E, NK = Piece<T>::NK, NW = TH / 64;
  constexpr int SL = ac_slice<T, TH>();
  constexpr bool aligned = ALIGNED;
  constexpr int END = -1;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int N = a.N, V = a.V, B = a.B, R = N + 1, rows = B * R, BN = B * N, Dm = a.max_depth;
  uint32_t* const queue = ws.err + 2;  // list positions handed out by the counter so far
  Red& red = S.red;
  const int ns = (V + SL - 1) / SL;  // slices per row
  const int D = ns >= 3 ? 1 : 2;     // rows taken ahead of the one being streamed
  // work-group g starts on list positions g (and g + grid when D = 2); the counter hands out
  // the positions from D * grid on
  const uint32_t G = gridDim.x, first = (uint32_t)D * G;
  // ---- the needed rows of the batch
  for (int x = t; x < rows; x += TH) S.bflag[x] = x % R == 0;
  __syncthreads();
  constexpr int PU = 4;  // nodes per thread whose loads are issued together
  for (int n0 = 0; n0 < BN; n0 += TH * PU) {
    int pr[PU], tk[PU], dp[PU];
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      const int n = n0 + u * TH + t;
      pr[u] = n < BN ? a.parents[n] : -2;
      tk[u] = n < BN ? a.tokens[n] : -1;
      dp[u] = n < BN && a.depth ? a.depth[n] : 0;
    }
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      const int n = n0 + u * TH + t;
      if (n >= BN || pr[u] < -1 || pr[u] >= N || tk[u] < 0 || tk[u] >= V) continue;
      const int b = n / N;
      int dep = dp[u];
      if (!a.depth) {  // nodes on the root path within max_depth, through in-range parents
        int cur = n - b * N, cnt = 1;
        for (int st = 0; st < SV_MAX_DEPTH; ++st) {
          const int p = a.parents[(int64_t)b * N + cur];
          if (p == -1) { dep = cnt; break; }
          if (p < 0 || p >= N || cnt >= Dm) break;
          ++cnt;
          cur = p;
        }
      }
      if (dep > 0) S.bflag[b * R + pr[u] + 1] = 1;  // every writer stores the same value
    }
  }
  __syncthreads();
  // ascending list: thread t scans a contiguous chunk, a block scan places it
  const int C = (rows + TH - 1) / TH;
  const int x0 = min(rows, t * C), x1 = min(rows, x0 + C);
  int c = 0;
  for (int x = x0; x < x1; ++x) c += S.bflag[x];
  int incl = c;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) S.bscan[wv] = incl;
  __syncthreads();
  int pos = incl - c, total = 0;
  for (int k = 0; k < NW; ++k) {
    if (k < wv) pos += S.bscan[k];
    total += S.bscan[k];
  }
  for (int x = x0; x < x1; ++x)
    if (S.bflag[x]) S.blist[pos++] = (uint16_t)x;
  __syncthreads();
  // every sequence has its root row in the list: its rows are bseq[b] .. bseq[b + 1] - 1
  for (int p = t; p < total; p += TH) {
    const int b = S.blist[p] / R;
    if (p == 0 || S.blist[p - 1] / R != b) S.bseq[b] = (uint16_t)p;
  }
  if (t == 0) {
    S.bseq[B] = (uint16_t)total;
    S.ring[0] = blockIdx.x < (uint32_t)total ? (int)blockIdx.x : END;
    S.ring[1] = D == 2 && blockIdx.x + G < (uint32_t)total ? (int)(blockIdx.x + G) : END;
    S.q_ended = first >= (uint32_t)total;
    S.q_inj = END;
  }
  __syncthreads();
  // ---- this work-group's stream: rows j = 0, 1, ... (S.ring[j & 3]), ns slices each
  int e_cur = S.ring[0];
  if (e_cur == END) return;  // uniform
  const T* target = (const T*)a.target_logits;
  auto row_of = [&](int e) {
    return __builtin_amdgcn_readfirstlane((e & AC_LEAFROW) ? (e & 8191) : (int)S.blist[e]);
  };
  auto load_item = [&](int e, int s, uint4 (&r)[NK]) {
    load_pieces<T, TH>(target + (int64_t)row_of(e) * V, s * SL, V, aligned, t, r);
  };
  float best = -INFINITY;
  int arg = AC_NO_ID;
  int j = 0, s = 0;
  uint32_t taken = ~0u;  // (thread 0) the counter's answer for row j + D, ~0: none asked
  const int s_take = D == 1 ? ns - 3 : 0, s_put = D == 1 ? ns - 2 : ns - 1;
  // (thread 0) row j + D's entry into its ring slot, published by the next barrier
  auto put = [&]() {
    int e = S.q_pend;
    if (taken != ~0u) {
      e = taken < (uint32_t)total ? (int)taken : END;
      if (e == END) S.q_ended = 1;
    }
    S.ring[(j + D) & 3] = e;
  };
  auto step = [&](uint4 (&cur)[NK], uint4 (&nxt)[NK]) -> bool {
    if (s == s_take && t == 0) {  // row j + D: a handed-back leaf row first, else the counter
      taken = ~0u;
      S.q_pend = S.q_inj;
      if (S.q_inj != END) S.q_inj = END;
      else if (!S.q_ended) taken = first + add_u32(queue, 1u);  // its value is needed only at slice s_put
    }
    int e_nx = e_cur, s_nx = s + 1;
    if (s_nx == ns) {
      e_nx = S.ring[(j + 1) & 3];
      s_nx = 0;
    }
    if (e_nx != END) load_item(e_nx, s_nx, nxt);
    // this slice
    const int s0 = s * SL;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      float x[E];
      unpack16<T>(cur[k], x);
      const int v = piece_v<T, TH>(s0, k, t);
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (v + e < V && x[e] > best) { best = x[e]; arg = v + e; }
    }
    if (s_nx != 0) {
      if (D == 1 && s == s_put) {
        if (t == 0) put();
        __syncthreads();
      }
      ++s;
      return true;
    }
    // ---- the end of row j
    if (D == 2 && t == 0) put();  // published by the reduction's barriers
    block_argmax<TH>(best, arg, red);
    arg = greedy_token(arg);
    const int row = row_of(e_cur), b = row / R;
    if (e_cur & AC_LEAFROW) {  // a walk's leaf stop row: its argmax is the bonus token
      if (t == 0) a.out_tokens[(int64_t)b * (Dm + 1) + ((e_cur >> 13) & 31)] = arg;
    } else {
      if (t == 0) {
        st_u64(&ws.res[row], res_word(-1, arg));
        mem_complete();  // the result is visible before the count below
        const uint32_t need = (uint32_t)(S.bseq[b + 1] - S.bseq[b]);
        S.s_last = add_u32(&ws.seqdone[b], 1u) + 1 == need;
      }
      __syncthreads();
      if (S.s_last) {  // uniform: the sequence's last row, walk it now
        seq_facts<TH>(a, seq_fetch(a, b), S.si);
        const int left = greedy_walk<T, TH, true>(a, ws, cm, has_cm, b, aligned, S);
        if (left != END && t == 0) {  // the first ring slot still free, else the next take
          if (S.ring[(j + 1) & 3] == END) S.ring[(j + 1) & 3] = left;
          else if (D == 2 && S.ring[(j + 2) & 3] == END) S.ring[(j + 2) & 3] = left;
          else S.q_inj = left;
        }
        __syncthreads();
      }
    }
    best = -INFINITY;
    arg = AC_NO_ID;
    if (e_nx == END) {  // nothing was in flight: a walk may just have handed back a row
      e_nx = S.ring[(j + 1) & 3];
      if (e_nx == END) return false;
      load_item(e_nx, 0, nxt);
    }
    ++j;
    s = 0;
    e_cur = e_nx;
    return true;
  };
  uint4 r0[NK], r1[NK];
  load_item(e_cur, 0, r0);
  while (step(r0, r1) && step(r1, r0)) {
  }
}

// This thread's argmax (lowest id on ties) over the slices s0, s0 + step, ... of a logits row,
// with up to DEPTH slices in flight; a thread visits its entries in ascending id.  has_pre: the
// first slice's loads were issued already, into `pre`.
template <typename T, int TH, int DEPTH>
__device__ __forceinline__ void argmax_slices(const T* row, int V, bool aligned, int t, int s0, int step, float& best,
                                              int& arg, bool has_pre, const uint4 (&pre)[Piece<T>::NK]) {
  constexpr int E = Piece<T>::E, NK = Piece<T>::NK, SL = ac_slice<T, TH>();
  const int ns = (V + SL - 1) / SL;
  const int n = s0 < ns ? (ns - s0 + step - 1) / step : 0;  // slices of this work-group
  uint4 r[DEPTH][NK];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    if (d == 0 && has_pre) {
#pragma unroll
      for (int k = 0; k < NK; ++k) r[0][k] = pre[k];
    } else if (d < n) {
      load_pieces<T, TH>(row, (s0 + d * step) * SL, V, aligned, t, r[d]);
    }
  }
  for (int g = 0; g < n; g += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (g + d < n) {
        const int sv = (s0 + (g + d) * step) * SL;
#pragma unroll
        for (int k = 0; k < NK; ++k) {
          float x[E];
          unpack16<T>(r[d][k], x);
          const int v = piece_v<T, TH>(sv, k, t);
#pragma unroll
          for (int e = 0; e < E; ++e)
            if (v + e < V && x[e] > best) { best = x[e]; arg = v + e; }
        }
        if (g + d + DEPTH < n) load_pieces<T, TH>(row, (s0 + (g + d + DEPTH) * step) * SL, V, aligned, t, r[d]);
      }
    }
  }
}

// Greedy batches of at least AC_CHAIN_B sequences: a group of G work-groups per sequence
// follows the accepted path itself, row after row -- the root row's argmax names the children
// that match, their rows name theirs, and so on -- so it reads only the rows of nodes whose
// whole root path matches, plus the stop row for its bonus, rather than every row with a usable
// child.  All children that match one row (equal sibling tokens) are followed, breadth first,
// since the accepted node is the deepest match (lowest index on ties).  A CU streams only a few
// tens of GB/s by itself, so a row is split over the G members (slices rank, rank + G, ...,
// all in flight at once), whose (maximum, index) pairs meet in one exchange per row; every
// member then takes the same decisions.  Member 0 writes the outputs and commits the accepted
// path when asked to.  A timeout of an exchange, or a timeout word already set when the launch
// starts, is reported as status 7 (the word is cleared by the last work-group).
constexpr int AC_CHAIN_B = 16;
constexpr int AC_CHAIN_TH = 256;  // threads per chain work-group (512 / AC_CHAIN_TH work-groups per CU)
constexpr int AC_CHAIN_G = 8;     // members per sequence at most
// members per sequence: the batch's groups about fill the CUs (256 of them, each holding
// 512 / AC_CHAIN_TH members at once), each member holding a slice
inline int chain_G(const sv_accept_args& a) {
  const int64_t sl = (int64_t)AC_CHAIN_TH * (a.logits_dtype == SV_BF16 ? 64 : 32);  // entries per slice
  const int ns = (int)((a.V + sl - 1) / sl);
  const int64_t room = 256 * (512 / AC_CHAIN_TH);
  int g = 1;
  while (g * 2 <= AC_CHAIN_G && g * 2 <= ns && (int64_t)a.B * g * 2 <= room) g *= 2;
  return g;
}
template <typename T, bool ALIGNED, int TH>
__device__ __forceinline__ void greedy_chain_seq(const sv_accept_args& a, int b, int rank, int G, XSlot* gslots,
                                                 const AccWs& ws, const sv_commit_args& cm, int32_t has_cm,
                                                 AccShared<T, TH, false>& S) {
  constexpr bool aligned = ALIGNED;
  constexpr int CD = ALIGNED ? 4 : 1;  // slices in flight (rows off 16 bytes load entry by entry: a register each)
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int N = a.N, V = a.V, Dm = a.max_depth;
  SeqInfo& si = S.si;
  Red& red = S.red;
  const T* rows = (const T*)a.target_logits + (int64_t)b * (N + 1) * V;
  // the root row is read first in any case: its first slice's loads go out with the sequence's
  uint4 pre[Piece<T>::NK];
  const SeqRaw sr = seq_fetch(a, b);
  load_pieces<T, TH>(rows, rank * ac_slice<T, TH>(), V, aligned, t, pre, rank * ac_slice<T, TH>() < V);
  seq_facts<TH>(a, sr, si);
  for (int x = t; x < N; x += TH) S.bflag[x] = 0;  // node matched, and every node above it did
  if (t == 0) {
    S.s_xc = 0;
    S.rows[0] = 0;  // rows to follow: the root row first
    S.q_head = 0;
    S.q_tail = 1;
  }
  __syncthreads();
  uint32_t xtag = 0;  // exchanges so far (the same on every member)
  // the argmax of row r over the whole group (lowest id on ties), in every thread
  auto row_argmax = [&](int r) {
    float best = -INFINITY;
    int arg = AC_NO_ID;
    const T* row = rows + (int64_t)r * V;
    argmax_slices<T, TH, CD>(row, V, aligned, t, rank, G, best, arg, r == 0, pre);
    block_argmax<TH>(best, arg, red);
    if (G > 1) {
      exchange<TH>(gslots, G, rank, ++xtag, 2, S.xv, ws.err, nullptr, &S.s_xc, __float_as_uint(best), (uint32_t)arg);
      best = -INFINITY;
      arg = AC_NO_ID;
      for (int k = 0; k < G; ++k) {  // members hold disjoint slices: the larger value, then the lower id
        const float v = __uint_as_float(S.xv[k][0]);
        const int i = (int)S.xv[k][1];
        if (v > best || (v == best && i < arg)) { best = v; arg = i; }
      }
    }
    return greedy_token(arg);
  };
  int A = 0, stop_row = 0;
  bool settled = false;  // the accepted node is known
  for (;;) {
    const int h = S.q_head;
    if (h == S.q_tail) {  // uniform
      if (settled) break;
      settled = true;
      // the accepted node: the deepest match, lowest index on ties
      int key = -1;
      if (t < N && S.bflag[t]) key = (si.dep[t] << 9) | (511 - t);
      {
        float kv = (float)key;
        int ki = key;
        block_argmax<TH>(kv, ki, red);
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
      // a followed stop row's argmax is known; one without usable children is read last
      if (stop_row != 0 && !si.haskid[stop_row]) {
        if (t == 0) S.rows[S.q_tail++] = (int16_t)stop_row;
        __syncthreads();
      }
      continue;
    }
    const int r = S.rows[h];
    const int arg = row_argmax(r);
    // the usable children of row r whose token is its argmax; those with usable children of
    // their own are followed next (each row is queued at most once: a node has one parent)
    const bool m = t < N && si.usable[t] && si.par[t] + 1 == r && si.tok[t] == arg;
    if (m) S.bflag[t] = 1;
    const bool push = m && si.haskid[t + 1];
    const uint64_t pm = __ballot(push);
    if (lane == 0) si.wcount[wv] = __popcll(pm);
    __syncthreads();
    int off = S.q_tail, add = 0;
    for (int k = 0; k < TH / 64; ++k) {
      if (k < wv) off += si.wcount[k];
      add += si.wcount[k];
    }
    if (push) S.rows[off + __popcll(pm & ((1ull << lane) - 1ull))] = (int16_t)(t + 1);
    __syncthreads();  // every thread has read q_tail and the counts
    if (t == 0) {
      S.rowarg[r] = arg;
      S.q_head = h + 1;
      S.q_tail += add;
    }
    __syncthreads();
  }
  const int bonus = S.rowarg[stop_row];
  if (t == 0) S.s_to = ld_u32(ws.err) != 0;  // set before the launch, or by a wait of this call that expired
  __syncthreads();
  if (rank != 0) return;
  const bool to = S.s_to != 0;
  if (t == 0) {
    a.accept_len[b] = A;
    a.num_out[b] = A + 1;
    a.stop_row[b] = stop_row;
    a.status[b] = to ? SV_SEQ_TIMEOUT : (si.bad_token ? SV_SEQ_TOKEN : 0);
  }
  if (t < Dm) a.accept_rows[(int64_t)b * Dm + t] = t < A ? si.path[t] + 1 : 0;
  if (t <= Dm)
    a.out_tokens[(int64_t)b * (Dm + 1) + t] = t < A ? a.tokens[(int64_t)b * N + si.path[t]] : (t == A ? bonus : 0);
  // the accepted path into the cache (nothing after a timeout: the path may be wrong)
  if (has_cm) svc::walker_commit(cm, b, to ? 0 : A, si.path);
}

// Threshold acceptance (mode 3) over batches whose needed rows are many bytes: the group of a
// sequence follows the paths whose score stays at or above the threshold, row after row, as the
// greedy chains do.  A followed row's statistics -- its maximum with the lowest id holding it and
// Z = sum_v exp((l_v - m) / T) (fp32 exponentials, fp64 sums, rescaled when a thread's maximum
// moves) -- meet in one exchange; each usable child of the row gets p = exp((l - M) / T) / Z and
// the score of its parent times p, and the children at or above the threshold that have usable
// children of their own are followed next.  So only the rows of passing nodes, and the stop row
// for its bonus (its argmax, lowest id on ties), are read.
template <typename T, bool ALIGNED, int TH>
__device__ __forceinline__ void thr_chain_seq(const sv_accept_args& a, int b, int rank, int G, XSlot* gslots,
                                              const AccWs& ws, const sv_commit_args& cm, int32_t has_cm,
                                              AccShared<T, TH, false>& S) {
  constexpr bool aligned = ALIGNED;
  constexpr int E = Piece<T>::E, NK = Piece<T>::NK, SL = ac_slice<T, TH>();
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int N = a.N, V = a.V, Dm = a.max_depth;
  SeqInfo& si = S.si;
  Red& red = S.red;
  const float c2 = 1.4426950408889634f / a.temperature;  // exp((x - m) / T) = exp2((x - m) c2)
  const double temp = a.temperature;
  const T* rows = (const T*)a.target_logits + (int64_t)b * (N + 1) * V;
  seq_facts<TH>(a, seq_fetch(a, b), si);
  for (int x = t; x < N; x += TH) S.bflag[x] = 0;  // node at or above the threshold, and its path too
  if (t == 0) {
    S.s_xc = 0;
    S.rows[0] = 0;  // rows to follow: the root row first
    S.q_head = 0;
    S.q_tail = 1;
  }
  __syncthreads();
  uint32_t xtag = 0;  // exchanges so far (the same on every member)
  const int ns = (V + SL - 1) / SL;
  const int nmine = rank < ns ? (ns - rank + G - 1) / G : 0;  // slices rank, rank + G, ...
  // statistics of row r over the whole group, in every thread: M, the lowest id holding it, Z
  auto row_stats = [&](int r, float& M, int& ID, double& Z) {
    const T* row = rows + (int64_t)r * V;
    float m = -INFINITY;
    int id = AC_NO_ID;
    double z = 0.0;
    // two slices in flight (one for rows off 16 bytes, which load entry by entry)
    constexpr int TD = ALIGNED ? 2 : 1;
    uint4 raw[TD][NK];
    if (nmine > 0) load_pieces<T, TH>(row, rank * SL, V, aligned, t, raw[0]);
    for (int q = 0; q < nmine; q += TD) {
#pragma unroll
      for (int d = 0; d < TD; ++d) {
        if (q + d < nmine) {
          if (TD == 2 && q + d + 1 < nmine)
            load_pieces<T, TH>(row, (rank + (q + d + 1) * G) * SL, V, aligned, t, raw[(d + 1) % TD]);
          const int s0 = (rank + (q + d) * G) * SL;
          // this thread's entries of the slice (ascending ids): maximum and lowest id, then the
          // sum at that maximum, merged into the running pair
          float sm = -INFINITY;
          int sid = AC_NO_ID;
#pragma unroll
          for (int k = 0; k < NK; ++k) {
            float x[E];
            unpack16<T>(raw[d][k], x);
            const int v = piece_v<T, TH>(s0, k, t);
#pragma unroll
            for (int e = 0; e < E; ++e)
              if (v + e < V && x[e] > sm) { sm = x[e]; sid = v + e; }
          }
          if (sm != -INFINITY) {
            double zd = 0.0;
#pragma unroll
            for (int k = 0; k < NK; ++k) {
              float x[E], g = 0.f;
              unpack16<T>(raw[d][k], x);
              const int v = piece_v<T, TH>(s0, k, t);
#pragma unroll
              for (int e = 0; e < E; ++e)
                if (v + e < V) g += exp2f((x[e] - sm) * c2);
              zd += (double)g;
            }
            if (sm > m) {
              z = (m == -INFINITY ? 0.0 : z * (double)exp2f((m - sm) * c2)) + zd;
              m = sm;
              id = sid;
            } else {
              z += zd * (double)exp2f((sm - m) * c2);
            }
          }
          if (TD == 1 && q + 1 < nmine) load_pieces<T, TH>(row, (rank + (q + 1) * G) * SL, V, aligned, t, raw[0]);
        }
      }
    }
    // the work-group: maximum with the lowest id, sums rescaled to it
    float bm = m;
    int bid = id;
    block_argmax<TH>(bm, bid, red);
    const double zt = block_sum<TH>(m == -INFINITY ? 0.0 : z * (double)exp2f((m - bm) * c2), red);
    M = bm;
    ID = bid;
    Z = zt;
    if (G > 1) {
      exchange<TH>(gslots, G, rank, ++xtag, 4, S.xv, ws.err, nullptr, &S.s_xc, __float_as_uint(bm), (uint32_t)bid,
                   dlo(zt), dhi(zt));
      M = -INFINITY;
      ID = AC_NO_ID;
      for (int k = 0; k < G; ++k) {  // members hold disjoint slices: the larger value, then the lower id
        const float v = __uint_as_float(S.xv[k][0]);
        const int i = (int)S.xv[k][1];
        if (v > M || (v == M && i < ID)) { M = v; ID = i; }
      }
      Z = 0.0;
      for (int k = 0; k < G; ++k) {
        const float v = __uint_as_float(S.xv[k][0]);
        if (v != -INFINITY) Z += dof(S.xv[k][2], S.xv[k][3]) * exp(((double)v - (double)M) / temp);
      }
    }
    ID = greedy_token(ID);
  };
  int A = 0, stop_row = 0;
  bool settled = false;  // the accepted node is known
  for (;;) {
    const int h = S.q_head;
    if (h == S.q_tail) {  // uniform
      if (settled) break;
      settled = true;
      // the accepted node: the deepest node at or above the threshold, lowest index on ties
      int key = -1;
      if (t < N && S.bflag[t]) key = (si.dep[t] << 9) | (511 - t);
      {
        float kv = (float)key;
        int ki = key;
        block_argmax<TH>(kv, ki, red);
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
      // a followed stop row's argmax is known; one without usable children is read last
      if (stop_row != 0 && !si.haskid[stop_row]) {
        if (t == 0) S.rows[S.q_tail++] = (int16_t)stop_row;
        __syncthreads();
      }
      continue;
    }
    const int r = S.rows[h];
    row_kids<TH>(N, r, si);  // the usable children of row r, ascending
    const int K = si.K;
    float lc = 0.f;  // this thread's child's logit at its token
    if (t < K) lc = load_as_f32<T>(rows + (int64_t)r * V, si.tok[si.kids[t]]);
    float M;
    int ID;
    double Z;
    row_stats(r, M, ID, Z);
    const double sr = r == 0 ? 1.0 : S.nscore[r - 1];
    bool push = false;
    int c = 0;
    if (t < K) {
      c = si.kids[t];
      const double sc = sr * (exp(((double)lc - (double)M) / temp) / Z);
      if (sc >= (double)a.threshold) {
        S.nscore[c] = sc;
        S.bflag[c] = 1;
        push = si.haskid[c + 1] != 0;
      }
    }
    const uint64_t pm = __ballot(push);
    if (lane == 0) si.wcount[wv] = __popcll(pm);
    __syncthreads();
    int off = S.q_tail, add = 0;
    for (int k = 0; k < TH / 64; ++k) {
      if (k < wv) off += si.wcount[k];
      add += si.wcount[k];
    }
    if (push) S.rows[off + __popcll(pm & ((1ull << lane) - 1ull))] = (int16_t)(c + 1);
    __syncthreads();  // every thread has read q_tail and the counts
    if (t == 0) {
      S.rowarg[r] = ID;
      S.q_head = h + 1;
      S.q_tail += add;
    }
    __syncthreads();
  }
  const int bonus = S.rowarg[stop_row];
  if (t == 0) S.s_to = ld_u32(ws.err) != 0;  // set before the launch, or by a wait of this call that expired
  __syncthreads();
  if (rank != 0) return;
  const bool to = S.s_to != 0;
  if (t == 0) {
    a.accept_len[b] = A;
    a.num_out[b] = A + 1;
    a.stop_row[b] = stop_row;
    a.status[b] = to ? SV_SEQ_TIMEOUT : (si.bad_token ? SV_SEQ_TOKEN : 0);
  }
  if (t < Dm) a.accept_rows[(int64_t)b * Dm + t] = t < A ? si.path[t] + 1 : 0;
  if (t <= Dm)
    a.out_tokens[(int64_t)b * (Dm + 1) + t] = t < A ? a.tokens[(int64_t)b * N + si.path[t]] : (t == A ? bonus : 0);
  // the accepted path into the cache (nothing after a timeout: the path may be wrong)
  if (has_cm) svc::walker_commit(cm, b, to ? 0 : A, si.path);
}

// G: members per sequence of a chain (chain_G; the grid is chain_grid), unused for the list.
// THR: the chains of threshold acceptance (mode 3) instead of greedy ones.
template <typename T, bool ALIGNED, int TH, bool CHAIN, bool THR = false>
__device__ __forceinline__ void greedy_rows_body(const sv_accept_args& a, int G, const AccWs& ws, const sv_commit_args& cm,
                                                 int32_t has_cm, AccShared<T, TH, false>& S) {
  const int t = threadIdx.x;
  if constexpr (CHAIN) {
    // work-groups are dispatched round-robin over the 8 XCDs: the members of a sequence's group
    // are consecutive work-groups of one XCD
    const int bid = (int)blockIdx.x, xcd = bid % 8, idx = bid / 8;
    const int b = (idx / G) * 8 + xcd, rank = idx % G;
    if (b < a.B) {
      XSlot* gslots = ws.xs + (int64_t)b * G * 2;
      if constexpr (THR) thr_chain_seq<T, ALIGNED, TH>(a, b, rank, G, gslots, ws, cm, has_cm, S);
      else greedy_chain_seq<T, ALIGNED, TH>(a, b, rank, G, gslots, ws, cm, has_cm, S);
      if (G > 1) {  // the group's last member leaves its exchange slots and exit count zeroed
        mem_complete();
        __syncthreads();
        if (t == 0) S.s_last = add_u32(ws.gexit + b, 1u) + 1 == (uint32_t)G;
        __syncthreads();
        if (S.s_last) {
          for (int i = t; i < G * 2 * AC_XW; i += TH) st_u64(&gslots[i / AC_XW].w[i % AC_XW], 0ull);
          if (t == 0) st_u32(ws.gexit + b, 0u);
        }
      }
    }
  } else {
    greedy_batch_body<T, ALIGNED, TH>(a, ws, cm, has_cm, S);  // one list for the batch
  }
  // every work-group counts out; the last one leaves the timeout word and the counters zeroed
  mem_complete();
  __syncthreads();
  if (t == 0 && add_u32(ws.err + 1, 1u) + 1 == gridDim.x) {
    st_u32(ws.err, 0u);
    st_u32(ws.err + 1, 0u);
    st_u32(ws.err + 2, 0u);
  }
}
// The greedy form of a batch: chains when the list cannot hold the batch's rows, else (or with
// SV_FLAG_ROW_LIST) the list when it would read few bytes -- about half the batch's rows under
// 48 MB from AC_CHAIN_B sequences on, under 96 MB below -- and chains otherwise.  The bounds
// are where the two forms took about the same time on MI355X: a chain costs its longest path's
// rows one after another (a slice load and an exchange each), the list its bytes plus a few
// dependent steps at either end.
inline bool chain_pays(const sv_accept_args& a) {
  const double half = (double)a.B * (a.N + 1) / 2 * (double)a.V * (a.logits_dtype == SV_BF16 ? 2 : 4);
  return half >= (a.B >= AC_CHAIN_B ? 48.0 : 96.0) * (1 << 20);
}
inline bool rows_chain(const sv_accept_args& a) {
  if ((int64_t)a.B * (a.N + 1) > AC_BLIST) return true;
  if (a.flags & SV_FLAG_ROW_LIST) return false;
  return chain_pays(a);
}
// Threshold acceptance: chains by the same bound (rows on 16 bytes), else (or with
// SV_FLAG_ROW_LIST) the row statistics of every row with a usable child and one walk per
// sequence (sv_threshold.hip).
inline bool thr_chain(const sv_accept_args& a) { return !(a.flags & SV_FLAG_ROW_LIST) && chain_pays(a); }
// chains: whole groups of 8 sequences (one per XCD) of G members each
inline int64_t chain_grid(const sv_accept_args& a, int G) { return ((int64_t)a.B + 7) / 8 * 8 * G; }
static_assert(AC_BLIST <= 8192 && SV_MAX_DEPTH < 32, "leaf stream entries: batch row in 13 bits, depth in 5");
// one list over the batch: as many work-groups as the CUs hold at once (per_cu on each of the
// 256 CUs), fewer when the batch has fewer rows
inline int64_t rows_grid(const sv_accept_args& a, int per_cu) {
  const int64_t rows = (int64_t)a.B * (a.N + 1), wgs = 256 * per_cu;  // rows: an upper bound of the list's
  return rows < wgs ? rows : wgs;
}

// The resolution of one row slice by one work-group of a row group (see the file comment of
// sv_accept.hip), callable from any kernel whose work-groups have TH threads.  `role` places the
// work-group among the acceptance work-groups of its launch; S is its LDS.
// PREFETCH: the target slice is loaded before the sequence facts that say whether the row is
// needed (its latency then overlaps theirs); otherwise after them, and only for needed rows.
// Either choice gives the same results; prefetching pays where nearly every row is resolved.
// ROWMAJOR: stochastic wide trees take their rows row-major over the batch, and row groups of
// finished walks leave at their start (the separate acceptance launch; the one-launch step,
// which holds few rows, keeps sequence-major rows).
template <typename T, int MODE, bool ALIGNED, int TH, bool PREFETCH, bool ROWMAJOR = true>
__device__ __forceinline__ void accept_body(const sv_accept_args& a, int32_t G, const AccWs& ws,
                                            const sv_commit_args& cm, int32_t has_cm, const AccRole role,
                                            AccShared<T, TH, MODE != SV_GREEDY>& S) {
  constexpr int NW = TH / 64;
  // STO: a rejection walk (modes 1 and 2); TOPK: deterministic drafts (q = point mass per child)
  constexpr bool STO = MODE != SV_GREEDY, TOPK = MODE == SV_TOPK_DRAFT;
  constexpr int E = Piece<T>::E, NK = Piece<T>::NK;
  Red& red = S.red;
  SeqInfo& si = S.si;
  int32_t &s_last = S.s_last, &s_hit = S.s_hit, &s_first = S.s_first, &s_lpos = S.s_lpos;
  uint64_t* s_match = S.s_match;
  auto& xv = S.xv;  // collected group partials
  float *s_lp = S.s_lp, *s_lq = S.s_lq, *s_u = S.s_u;  // per child: logits at its token, u_accept
  float& s_us = S.s_us;                                 // u_sample of the row
  float* s_g = S.s_g;                                   // bonus: per-piece sums [k][t]
  double* s_col = S.s_col;                              // ... and their row totals
  int &s_xc = S.s_xc, &s_claim = S.s_claim, &s_fin = S.s_fin, &s_bad = S.s_bad, &s_to = S.s_to;
  // work-groups are dispatched round-robin over the 8 XCDs; the members of a
  // group share an XCD (each region of acceptance work-groups starts on a multiple of 8 and
  // holds a multiple of 8 * G of them)
  const int t = threadIdx.x, lane = t & 63;
  const int xcd = role.bid % 8, idx = role.bid / 8;
  const int grp = (idx / G) * 8 + xcd;  // the group within its region: the row it resolves
  const int rank = idx % G;
  const int N = a.N, V = a.V;
  const float invT = STO ? 1.0f / a.temperature : 1.0f;
  const float l2T = invT * 1.4426950408889634f;  // bulk exponentials as exp2((x - m) * log2(e) / T)
  const int64_t gslot = grp;  // exchange slots and exit counter of the group
  XSlot* gslots = ws.xs + gslot * G * 2;
  uint32_t xtag = 0;  // exchanges of this group so far (identical on every member)
  // the row this group resolves (index b (N + 1) + r).  Stochastic wide trees (ROWMAJOR) take
  // the rows row-major over the batch -- row r of every sequence before row r + 1 -- so that
  // the rows near the roots, where the walks run, resolve first; once a walk has finished, the
  // groups of its sequence's remaining rows leave at their start.  Elsewhere sequence-major.
  const bool wide = STO && N > 2 * a.max_depth;
  const int64_t nrows = (int64_t)a.B * (N + 1);
  const int64_t item =
      ROWMAJOR && wide && grp < nrows ? (int64_t)(grp % a.B) * (N + 1) + grp / a.B : (int64_t)grp;
  const int s0 = rank * ac_slice<T, TH>();  // this work-group's slice of the vocabulary
  if (t == 0) s_xc = 0;
  bool live_row = false;
  bool gone = false;  // (wide trees) the walk had finished when this work-group started
  if (item < (int64_t)a.B * (N + 1)) {
    // uniform, and kept in scalar registers so that the slice loads take a scalar resource
    const int b = __builtin_amdgcn_readfirstlane((int)(item / (N + 1)));
    const int r = __builtin_amdgcn_readfirstlane((int)(item % (N + 1)));
    const T* prow = (const T*)a.target_logits + ((int64_t)b * (N + 1) + r) * V;
    const T* qrow = MODE == SV_STOCHASTIC ? (const T*)a.draft_logits + ((int64_t)b * (N + 1) + r) * V : nullptr;
    constexpr bool aligned = ALIGNED;
    SeqRaw sr = seq_fetch(a, b);
    // stochastic, wide trees: the walk advances as rows resolve and ends the sequence's
    // remaining rows (below); without the prefetch, rows without a usable child are not
    // resolved here -- the walker draws the bonus of such a stop row itself (leaf_bonus).
    // Chains and narrow trees, where nearly every row is on the path, resolve every row and
    // walk once after the last one.
    const bool incr = wide;
    const bool wleaf = !PREFETCH && incr;  // stop rows without children: drawn by the walker
    uint32_t* cancel = incr ? &ws.cancel[b] : nullptr;
    uint32_t cx0 = 0u;  // the sequence's walk already finished (a late work-group)
    if (incr && t == 0) cx0 = ld_u32(cancel);
    // PREFETCH (chains and narrow trees, which resolve nearly every row): the target slice is
    // fetched before the sequence facts that confirm it is needed (its latency overlaps theirs;
    // the facts' own loads go first); otherwise after the facts, for the rows resolved
    uint4 rp[NK];
    if constexpr (STO && PREFETCH) load_pieces<T, TH>(prow, s0, V, aligned, t, rp);
    asm volatile("" : "+v"(sr.tok), "+v"(sr.par), "+v"(sr.dep), "+v"(cx0));  // nothing uses them before this point
    if (cx0) s_xc = 1;
    if (ROWMAJOR && incr) {  // uniform: a finished walk needs nothing more from this row
      __syncthreads();
      gone = s_xc != 0;
    }
    if (!gone) {
      seq_facts<TH>(a, sr, si);
      // the same on every member
      live_row = row_live(a, si, r) && (!wleaf || r == 0 || si.haskid[r] != 0);
    }
    if constexpr (STO && !PREFETCH) load_pieces<T, TH>(prow, s0, V, aligned, t, rp, live_row && !s_xc);
    if (live_row && !s_xc) {
      row_kids<TH>(N, r, si);
      int done_by_me = 0;  // this work-group wrote the row result

      if (MODE == SV_GREEDY && G == 1) {
        // greedy, one work-group per row (large batches): the whole row streams through the
        // work-group one slice at a time with the next slice's loads in flight; no exchange
        float best = -INFINITY;
        int arg = AC_NO_ID;
        argmax_row<T, TH>(prow, V, aligned, t, best, arg);
        block_argmax<TH>(best, arg, red);
        if (t == 0) st_u64(&ws.res[item], res_word(-1, greedy_token(arg)));
        done_by_me = 1;
      } else if constexpr (MODE == SV_GREEDY) {
        float best = -INFINITY;
        int arg = AC_NO_ID;
        {
          load_pieces<T, TH>(prow, s0, V, aligned, t, rp);
#pragma unroll
          for (int k = 0; k < NK; ++k) {
            float x[E];
            unpack16<T>(rp[k], x);
            const int v = piece_v<T, TH>(s0, k, t);
#pragma unroll
            for (int e = 0; e < E; ++e)  // a thread visits its entries in ascending id
              if (v + e < V && x[e] > best) { best = x[e]; arg = v + e; }
          }
        }
        block_argmax<TH>(best, arg, red);
        exchange<TH>(gslots, G, rank, ++xtag, 2, xv, ws.err, nullptr, &s_xc, __float_as_uint(best), (uint32_t)arg);
        if (rank == 0) {
          if (t < 64) {  // wave 0: lane k takes member k's best; the butterfly keeps the lowest id on ties
            float bv = lane < G ? __uint_as_float(xv[lane][0]) : -INFINITY;
            int bi = lane < G ? (int)xv[lane][1] : AC_NO_ID;
            wave_argmax(bv, bi);
            if (t == 0) st_u64(&ws.res[item], res_word(-1, greedy_token(bi)));
          }
          done_by_me = 1;
        }
      } else {
        // the row's resolution; returns early once the sequence's walk has finished
        [&]() {
        const int K = __builtin_amdgcn_readfirstlane(si.K);
        const bool need_q = !TOPK && K > 0;  // deterministic drafts read no draft logits
        // ---- the slice: raw logits -> slice maxima -> exponentials kept in registers
        float ep[ac_ct<T>()], eq[ac_ct<T>()];
        float mp = -FLT_MAX, mq = -FLT_MAX;
        double zp = 0.0, zq = 0.0;
        {
          uint4 rq[NK];
          if constexpr (!TOPK) load_pieces<T, TH>(qrow, s0, V, aligned, t, rq, need_q);
          // children's logits at their tokens and their uniforms: issued after the draft
          // slice (so that nothing waits for them before it is issued), stored to LDS once
          // both slices are in
          uint32_t c_lp = 0u, c_lq = 0u, c_u = 0u, c_us = 0u;
          if (t < K) {
            const int kid = si.kids[t];
            const int x = si.tok[kid];  // usable: x in [0, V)
            c_lp = ldraw(prow, x);
            if constexpr (!TOPK) c_lq = ldraw(qrow, x);
            c_u = __float_as_uint(a.u_accept[(int64_t)b * (N + 1) + kid + 1]);
          }
          if (t == TH - 1) c_us = __float_as_uint(a.u_sample[(int64_t)b * (N + 1) + r]);
#pragma unroll
          for (int k = 0; k < NK; ++k) {
            float x[E];
            unpack16<T>(rp[k], x);
#pragma unroll
            for (int e = 0; e < E; ++e) mp = piece_v<T, TH>(s0, k, t) < V ? fmaxf(mp, x[e]) : mp;
          }
          mp = block_max<TH>(mp, red);
          opaque(rp);  // unpack again below instead of keeping the unpacked floats alive
          const float op = mp * l2T;  // exp2(x * l2T - op): one FMA per entry
          const bool whole = s0 + ac_slice<T, TH>() <= V;  // uniform: no entry of the slice lies past V
          auto expo = [&](const uint4 (&raw)[NK], float o, float (&ex)[ac_ct<T>()], double& z) {
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
                  ex[k * E + e] = piece_v<T, TH>(s0, k, t) < V ? __builtin_amdgcn_exp2f(fmaf(x[e], l2T, -o)) : 0.f;
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
              for (int e = 0; e < E; ++e) mq = piece_v<T, TH>(s0, k, t) < V ? fmaxf(mq, x[e]) : mq;
            }
            mq = block_max<TH>(mq, red);
            opaque(rq);
            expo(rq, mq * l2T, eq, zq);
          } else {
#pragma unroll
            for (int i = 0; i < ac_ct<T>(); ++i) eq[i] = 0.f;
          }
          asm volatile("" : "+v"(c_lp), "+v"(c_lq), "+v"(c_u), "+v"(c_us));  // first use: here
          if (t < K) {
            s_lp[t] = rawf<T>(c_lp);
            if constexpr (TOPK) {  // s_lq holds 1 where the child repeats an earlier sibling's token
              const int x = si.tok[si.kids[t]];
              bool dup = false;
              for (int j = 0; j < t; ++j) dup |= si.tok[si.kids[j]] == x;
              s_lq[t] = dup ? 1.f : 0.f;
            } else {
              s_lq[t] = rawf<T>(c_lq);
            }
            s_u[t] = __uint_as_float(c_u);
          }
          if (t == TH - 1) s_us = __uint_as_float(c_us);
        }
        block_sum2<TH>(zp, zq, red);  // its barriers also publish the children's values
        if (exchange<TH>(gslots, G, rank, ++xtag, TOPK ? 4 : 6, xv, ws.err, cancel, &s_xc, __float_as_uint(mp),
                     __float_as_uint(mq), dlo(zp), dhi(zp), dlo(zq), dhi(zq)))
          return;
        // global statistics: lane k of every wave takes member k's partials (G <= 64); the
        // butterfly reductions give every lane, wave and member the same values
        double Zp, Zq, fp, fq, rq;  // rq = fq / fp: residual coefficients in this slice's units
        double iZp, iZq;            // 1 / Zp, 1 / Zq: the tests below multiply instead of dividing
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
          iZp = 1.0 / Zp;
          iZq = need_q ? 1.0 / Zq : 0.0;
          const double spr = __shfl(sp, rank), sqr = __shfl(sq, rank);
          fp = spr * iZp;  // p(v) = ep(v) * fp on this slice
          fq = need_q ? sqr * iZq : 0.0;
          rq = need_q && spr > 0.0 ? (sqr * Zp) / (spr * Zq) : 0.0;
        }
        // a row without a finite positive normaliser (a NaN or +Inf logit, or no finite entry)
        // accepts no child: the walk stops here with bonus 0 and the sequence reports status 8.
        // Every member holds the same totals, so all of them leave here together.
        if (!(Zp > 0.0 && Zp < (double)INFINITY) || (need_q && !(Zq > 0.0 && Zq < (double)INFINITY))) {
          if (rank == 0) {
            if (t == 0) st_u64(&ws.res[item], res_word(-1, 0) | AC_RES_BAD);
            done_by_me = 1;
          }
          return;
        }
        // residual weight of one entry in units of fp: max(0, ep - kappa eq) for kappa > 0
        auto wgt = [&](int i, float kappa) -> float { return fmaxf(fmaf(-kappa, eq[i], ep[i]), 0.f); };
        auto slice_sum = [&](float kappa) -> double {  // kappa > 0
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
        if constexpr (TOPK) {
          // child j's proposal is the point mass at its token x: the test is u < p_cur(x), and
          // a rejection zeroes x.  p_cur is p restricted to the tokens not rejected yet at this
          // row, renormalised by their mass `rem`; a repeated token has mass 0.  No exchange:
          // p(x) is known from the row statistics.
          double rem = 1.0;
          for (int j = 0; j < K; ++j) {
            const double px = (double)expf((s_lp[j] - Mp) * invT) * iZp;
            const bool dup = s_lq[j] != 0.f;
            if (!dup && (double)s_u[j] * rem < px) { accepted = si.kids[j]; break; }  // u < px / rem
            if (!dup && rem - px > 0.0) rem -= px;  // a residual without mass (rounding only) is kept
          }
          // the bonus below zeroes the children's tokens (c != 0) and, should rounding leave
          // that residual without mass, falls back to p itself (c_prev = 0)
          if (accepted < 0 && K > 0) c = 1.0;
        } else
        for (int j = 0; j < K; ++j) {
          const double px = (double)expf((s_lp[j] - Mp) * invT) * iZp;
          const double qx = (double)expf((s_lq[j] - Mq) * invT) * iZq;
          const double u = (double)s_u[j];
          // u < max(0, px - c qx) / (Dn qx), with Dn > 0
          if (qx > 0.0 ? (u * qx * Dn < fmax(0.0, px - c * qx)) : true) { accepted = si.kids[j]; break; }
          // rejection: next residual coefficient; its normaliser is needed only for a later test,
          // after the last child the bonus scan below computes it as its total
          const double cn = c + Dn;
          if (j == K - 1) { c_prev = c; c = cn; break; }
          // max(0, p - cn q) = fp * max(0, ep - kappa eq) on this slice, kappa = cn fq / fp
          const float kappa = (float)(cn * rq);
          const double sl = block_sum<TH>(slice_sum(kappa), red) * fp;
          if (exchange<TH>(gslots, G, rank, ++xtag, 2, xv, ws.err, cancel, &s_xc, dlo(sl), dhi(sl))) return;
          // lane k of every wave takes member k's sum (G <= 64): one LDS read and a DPP reduction
          const double S = wave_sumd(lane < G ? dof(xv[lane][0], xv[lane][1]) : 0.0);
          __syncthreads();
          if (S > 0.0) { c = cn; Dn = S; }  // S == 0 only through rounding: keep the residual
        }
        if (accepted >= 0) {
          if (rank == 0) {
            if (t == 0) st_u64(&ws.res[item], res_word(accepted, -1));
            done_by_me = 1;
          }
        } else {
          // ---- bonus: smallest v whose ascending cumulative residual exceeds u * total.
          // A residual of total 0 (reachable only through rounding) falls back to the previous one.
          // Ids ascend piece by piece: piece (k, t) holds the slice-local ids (k * TH + t) * E ..
          // + E - 1.  Every thread sums its pieces' weights from the exponentials in its
          // registers; piece-row totals give the coarse cumulative sum, one work-group scan over
          // the pieces of the row that crosses the threshold finds the piece, and the thread that
          // holds it walks its E entries, again from its registers.  Piece sums are fp32 over E
          // entries; every sum above that is fp64.
          const int wv = t >> 6;
          const double us = (double)s_us;
          for (int attempt = 0; attempt < 2; ++attempt) {
            // c == 0 (no rejection at this row): the weights are p itself
            const float kappa = TOPK || c == 0.0 ? 0.f : (float)(c * rq);
            // top-K drafts whose children were all rejected: the children's tokens get weight 0;
            // bit k * E + e of zm marks such a token among this thread's entries
            uint64_t zm = 0ull;
            if (TOPK && c != 0.0) {
              for (int j = 0; j < K; ++j) {
                const int x = si.tok[si.kids[j]] - s0;
                if (x < 0 || x >= ac_slice<T, TH>()) continue;
                const int pc = x / E;
                if (pc % TH == t) zm |= 1ull << ((pc / TH) * E + x % E);
              }
            }
            // weight of entry i of this thread (i a compile-time index into the registers)
            auto wz = [&](int i) -> float {
              const float w = kappa == 0.f ? ep[i] : wgt(i, kappa);
              return ((zm >> i) & 1ull) ? 0.f : w;
            };
#pragma unroll
            for (int k = 0; k < NK; ++k) {
              float g = 0.f;
#pragma unroll
              for (int e = 0; e < E; ++e) g += wz(k * E + e);
              s_g[k * TH + t] = g;
            }
            __syncthreads();
            for (int k = wv; k < NK; k += NW) {  // wave wv totals rows wv, wv + NW, ...
              double x = 0.0;
              for (int i = lane; i < TH; i += 64) x += (double)s_g[k * TH + i];
              x = wave_sumd(x);
              if (lane == 0) s_col[k] = x;
            }
            __syncthreads();
            double col = 0.0;
            for (int k = 0; k < NK; ++k) col += s_col[k];
            const double sl = col * fp;
            if (exchange<TH>(gslots, G, rank, ++xtag, 2, xv, ws.err, cancel, &s_xc, dlo(sl), dhi(sl))) return;
            // lane k holds member k's slice total; one inclusive scan gives every member the
            // same prefixes, total and owner
            const double sk = lane < G ? dof(xv[lane][0], xv[lane][1]) : 0.0;
            const double incl_k = wave_scand(sk, lane);
            const double total = laned(incl_k, G - 1);
            const double before = laned(incl_k - sk, rank);
            if (!(total > 0.0) && attempt == 0 && c != 0.0) {  // uniform: retry with the previous residual
              c = c_prev;
              __syncthreads();
              continue;
            }
            // the slice whose inclusive prefix first exceeds the threshold draws the token
            const double thr = us * total;
            int owner = G - 1;
            {
              const uint64_t over = __ballot(lane < G && incl_k > thr);
              if (over) owner = __ffsll((long long)over) - 1;
            }
            if (rank == owner) {
              const double lthr = (thr - before) / fp;  // threshold in this slice's units
              // the piece row whose cumulative total first exceeds it (uniform)
              int ks = -1;
              double below = 0.0;
              for (int k = 0; k < NK; ++k) {
                if (below + s_col[k] > lthr) { ks = k; break; }
                below += s_col[k];
              }
              int h = 0x7fffffff;
              double excl = 0.0;
              if (ks >= 0) {  // inclusive scan of row ks over the threads, in id order
                const float gk = s_g[ks * TH + t];
                double incl = wave_scand((double)gk, lane);
                if (lane == 63) red.d[wv] = incl;
                if (t == 0) s_first = 0x7fffffff;
                __syncthreads();
                for (int w2 = 0; w2 < wv; ++w2) incl += red.d[w2];
                incl += below;
                excl = incl - (double)gk;
                const uint64_t over = __ballot(incl > lthr);  // one atomic per wave
                if (over && lane == 0) atomicMin(&s_first, wv * 64 + __ffsll((long long)over) - 1);
                __syncthreads();
                h = s_first;
              }
              if (h != 0x7fffffff) {
                if (t == h) {  // walk the E entries of piece (ks, h)
                  float w[E];
#pragma unroll
                  for (int e = 0; e < E; ++e) w[e] = 0.f;
#pragma unroll
                  for (int k = 0; k < NK; ++k)
#pragma unroll
                    for (int e = 0; e < E; ++e) w[e] = k == ks ? wz(k * E + e) : w[e];
                  const int v0 = s0 + (ks * TH + t) * E;  // id of its first entry
                  double run = excl;
                  int pick = -1, lastpos = -1;
#pragma unroll
                  for (int e = 0; e < E; ++e) {
                    if (w[e] > 0.f) {
                      lastpos = v0 + e;
                      run += (double)w[e];
                      if (pick < 0 && run > lthr) pick = v0 + e;
                    }
                  }
                  if (pick < 0) pick = lastpos >= 0 ? lastpos : min(v0 + E, V) - 1;
                  st_u64(&ws.res[item], res_word(-1, pick));
                }
              } else {
                // rounding left the threshold unreached: the highest id with a positive weight
                // (in rows up to ks when a row was found, else in the whole slice)
                const int klim = ks >= 0 ? ks : NK - 1;
                int lp = -1;
#pragma unroll
                for (int k = 0; k < NK; ++k)
#pragma unroll
                  for (int e = 0; e < E; ++e)
                    lp = (k <= klim && wz(k * E + e) > 0.f) ? s0 + (k * TH + t) * E + e : lp;
                for (int o = 32; o > 0; o >>= 1) lp = max(lp, __shfl_xor(lp, o));
                if (t == 0) s_lpos = -1;
                __syncthreads();
                if (lane == 0) atomicMax(&s_lpos, lp);
                __syncthreads();
                if (t == 0) {
                  const int pick = s_lpos >= 0 ? s_lpos : min(s0 + ac_slice<T, TH>(), V) - 1;
                  st_u64(&ws.res[item], res_word(-1, pick));
                }
              }
              done_by_me = 1;
            }
            break;
          }
        }
        }();
      }

      // ---- stochastic: the walk advances as rows resolve.  frontier[b] is the first row of
      // the accepted path not yet resolved.  The work-group that publishes that row claims
      // the frontier (compare-and-swap to BUSY) and follows the path through the rows that
      // are already resolved; it either reaches the stop row (it then writes the outputs
      // and raises cancel[b], so the sequence's other rows stop) or moves the frontier to
      // the next unresolved row and checks that row once more, since its publisher may have
      // looked at the frontier before the move (each side completes its store before its
      // load, so at least one of them sees the other's).
      if (STO && done_by_me) {
        mem_complete();  // this thread's row-result store (if any) has completed
        __syncthreads();
        uint32_t* front = &ws.frontier[b];
        uint64_t* rr = ws.res + (int64_t)b * (N + 1);
        uint64_t* s_rr = S.rr;  // the sequence's row results
        if (t == 0) {
          s_fin = 0;
          S.s_leaf = -1;
          if (incr) {
            s_claim = cas_u32(front, (uint32_t)r, AC_FRONT_BUSY) ? r : -1;
          } else {  // the last row of the sequence to resolve walks
            s_claim = -1;
            s_fin = add_u32(&ws.seqdone[b], 1u) + 1 == (uint32_t)si.nlive;
            if (s_fin) st_u32(&ws.seqdone[b], 0u);  // every row of b has been counted
          }
        }
        __syncthreads();
        if (s_fin) {
          for (int x = t; x <= N; x += TH) s_rr[x] = ld_u64(&rr[x]);
          __syncthreads();
        }
        for (int guard = 0; s_claim >= 0 && guard <= N + 1; ++guard) {  // uniform
          for (int x = t; x <= N; x += TH) s_rr[x] = ld_u64(&rr[x]);
          __syncthreads();
          if (t == 0) {
            int row = s_claim, claim = -1;
            bool stop = false;
            for (int n = 0; n <= N + 1; ++n) {
              const uint64_t v = s_rr[row];
              if (!res_ready(v)) break;
              const int ch = res_child(v);
              if (ch < 0 || ch >= N) { stop = true; break; }
              row = ch + 1;
            }
            if (stop) {
              s_fin = 1;
            } else if (wleaf && row > 0 && !si.haskid[row]) {  // a stop row without children
              S.s_leaf = row;
              s_fin = 1;
            } else {
              st_u32(front, (uint32_t)row);
              mem_complete();
              if (res_ready(ld_u64(&rr[row])) && cas_u32(front, (uint32_t)row, AC_FRONT_BUSY)) claim = row;
            }
            s_claim = claim;
          }
          __syncthreads();
        }
        if (!PREFETCH && S.s_leaf >= 0) {  // uniform: its bonus is drawn here, from the target row alone
          const int lr = S.s_leaf;
          const uint64_t wd =
              leaf_bonus<T, TH>((const T*)a.target_logits + ((int64_t)b * (N + 1) + lr) * V, V, aligned, l2T,
                                a.u_sample[(int64_t)b * (N + 1) + lr], red, (double*)S.s_g, &s_first);
          if (t == 0) s_rr[lr] = wd;
          __syncthreads();
        }
        if (s_fin) {
          // the path from the root in the LDS copy: every row on it was resolved before the
          // frontier passed it (a stop row without children: drawn just above)
          if (t == 0) {
            int row = 0, n = 0;
            for (;;) {
              const int ch = res_child(s_rr[row]);
              if (ch < 0 || ch >= N || n >= SV_MAX_DEPTH) break;
              si.path[n++] = ch;
              row = ch + 1;
            }
            si.flag = (n << 16) | row;  // A and the stop row
            s_hit = res_token(s_rr[row]);
            s_bad = res_bad(s_rr[row]) ? 1 : 0;
            s_to = ld_u32(ws.err) != 0;
          }
          __syncthreads();
          const int A = si.flag >> 16, stop_row = si.flag & 0xffff, bonus = s_hit;
          const int Dm = a.max_depth;
          if (t == 0) {
            a.accept_len[b] = A;
            a.num_out[b] = A + 1;
            a.stop_row[b] = stop_row;
            a.status[b] = s_to ? SV_SEQ_TIMEOUT
                               : (si.bad_token ? SV_SEQ_TOKEN : (s_bad ? SV_SEQ_NONFINITE : 0));
          }
          if (t < Dm) a.accept_rows[(int64_t)b * Dm + t] = t < A ? si.path[t] + 1 : 0;
          if (t <= Dm)
            a.out_tokens[(int64_t)b * (Dm + 1) + t] = t < A ? si.tok[si.path[t]] : (t == A ? bonus : 0);
          // the accepted path into the cache (nothing after a timeout: the path may be wrong)
          if (has_cm) svc::walker_commit(cm, b, s_to ? 0 : A, si.path);
          if (incr && t == 0) st_u32(cancel, 1u);  // the sequence's remaining rows are not needed
          if (!incr)  // every row result of b has been read: leave them cleared for the next call
            for (int x = t; x <= N; x += TH) st_u64(&rr[x], 0ull);
        }
      }

      // ---- greedy: the work-group that wrote the row result counts it; the last row of a
      // sequence walks
      if constexpr (MODE == SV_GREEDY) {
        if (done_by_me) {
          mem_complete();  // this thread's row-result stores (if any) have completed
          __syncthreads();
          if (t == 0) {
            const uint32_t old = add_u32(&ws.seqdone[b], 1u);
            s_last = old + 1 == (uint32_t)si.nlive;
          }
          __syncthreads();
          if (s_last) greedy_walk<T, TH>(a, ws, cm, has_cm, b, aligned, S);
        }
      }
    }
  }

  // ---- leave every counter and exchange slot zeroed for the next call.  The three exit
  // counts (group, sequence, grid) are independent and go out together; the last arrival
  // at each clears what it guards.
  mem_complete();  // this work-group's stores (results, outputs) have completed
  __syncthreads();
  // (stochastic wide trees only: elsewhere the walker is the sequence's last reader of its
  // row results and clears them itself)
  const bool seq_item = MODE != SV_GREEDY && N > 2 * a.max_depth && item < (int64_t)a.B * (N + 1);
  const int bq = seq_item ? (int)(item / (N + 1)) : 0;
  if (t == 0) {
    const uint32_t og = G > 1 ? add_u32(ws.gexit + gslot, 1u) : 0u;
    const uint32_t os = seq_item ? add_u32(&ws.seqexit[bq], 1u) : 0u;
    const uint32_t oe = add_u32(ws.err + 1, 1u);
    s_last = G == 1 || og + 1 == (uint32_t)G;  // every member of the group passed its last exchange
    s_claim = seq_item && os + 1 == (uint32_t)role.seq_wgs;  // every work-group of the sequence left
    s_fin = oe + 1 == (uint32_t)role.nblocks;                // every acceptance work-group has finished
  }
  __syncthreads();
  // (a member that left early on a finished walk may have exchanged less than the others,
  // so the slots of every live row are cleared, and of every row a member left at its start)
  if (s_last && (xtag > 0 || live_row || gone))
    for (int i = t; i < G * 2 * AC_XW; i += TH) st_u64(&gslots[i / AC_XW].w[i % AC_XW], 0ull);
  if (s_claim) {  // stochastic: the sequence's row results, frontier, cancel flag and exit count
    for (int x = t; x <= N; x += TH) st_u64(&ws.res[(int64_t)bq * (N + 1) + x], 0ull);
    if (t == 0) {
      st_u32(&ws.frontier[bq], 0u);
      st_u32(&ws.cancel[bq], 0u);
      st_u32(&ws.seqexit[bq], 0u);
    }
  }
  // After a timeout some row may never have been published (members that stopped waiting can
  // disagree), so some walk may never have run: the last work-group of the grid reports status 7
  // for every sequence and clears every per-sequence word for the next call.  Every other
  // work-group has exited, so nothing reads these words any more.
  const bool timed_out = s_fin && ld_u32(ws.err) != 0;
  if (timed_out) {
    for (int x = t; x < a.B; x += TH) {
      st_i(&a.status[x], SV_SEQ_TIMEOUT);
      st_u32(&ws.seqdone[x], 0u);
      st_u32(&ws.frontier[x], 0u);
      st_u32(&ws.cancel[x], 0u);
      st_u32(&ws.seqexit[x], 0u);
    }
    for (int64_t x = t; x < (int64_t)a.B * (N + 1); x += TH) st_u64(&ws.res[x], 0ull);
  }
  __syncthreads();  // every thread has read the timeout word before it is cleared
  if (t == 0) {
    if (G > 1 && s_last) st_u32(ws.gexit + gslot, 0u);
    if (s_fin) {  // clear the timeout flag
      st_u32(ws.err, 0u);
      st_u32(ws.err + 1, 0u);
    }
  }
}

// ---------------------------------------------------------------- workspace (host side)
// Work-groups per row group for TH-thread work-groups.
int groups_G_th(const sv_accept_args& a, int TH) {
  const int slice = TH * (a.logits_dtype == SV_BF16 ? ac_ct<uint16_t>() : ac_ct<float>());
  const int G = (a.V + slice - 1) / slice;
  return G < 1 ? 1 : G;
}
int groups_G(const sv_accept_args& a, bool aligned) { return groups_G_th(a, acc_threads(a, aligned)); }
// Greedy batches of at least AC_STREAM_ROWS rows read each row they need with one work-group
// (no exchange: a chain per sequence, or the batch's needed rows as one list); smaller batches
// split a row over a group of G work-groups for parallelism.
constexpr int64_t AC_STREAM_ROWS = 512;
int launch_G(const sv_accept_args& a, int TH) {
  if (a.mode == SV_GREEDY && (int64_t)a.B * (a.N + 1) >= AC_STREAM_ROWS) return 1;
  return groups_G_th(a, TH);
}
// one group per row, rounded up to a whole number of groups per XCD
int64_t num_groups(const sv_accept_args& a) { return ((int64_t)a.B * (a.N + 1) + 7) / 8 * 8; }

struct WsLayout {
  size_t gexit, seqdone, err, res, frontier, cancel, seqexit, xs, total;
};
// regions: regions of row groups in the launch (each with its own exit counters and exchange slots)
WsLayout ws_layout_g(const sv_accept_args& a, int G, int regions) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t NG = (size_t)num_groups(a) * (size_t)regions;
  WsLayout l{};
  size_t o = 0;
  l.gexit = o; o = up(o + NG * 4);
  l.seqdone = o; o = up(o + (size_t)a.B * 4);
  l.err = o; o = up(o + 16);
  l.res = o; o = up(o + (size_t)a.B * (a.N + 1) * sizeof(uint64_t));
  l.frontier = o; o = up(o + (size_t)a.B * 4);
  l.cancel = o; o = up(o + (size_t)a.B * 4);
  l.seqexit = o; o = up(o + (size_t)a.B * 4);
  // (also the greedy chains' slots: AC_CHAIN_G members per sequence)
  const size_t nxs = std::max(NG * (size_t)G, (size_t)a.B * AC_CHAIN_G) * 2;
  l.xs = o; o = up(o + nxs * sizeof(XSlot));
  l.total = o;
  return l;
}
// sized for the larger of the two group sizes (the row alignment is known only at the launch)
WsLayout ws_layout(const sv_accept_args& a) { return ws_layout_g(a, groups_G(a, false), 1); }
AccWs ws_views(void* workspace, const WsLayout& l) {
  char* base = (char*)workspace;
  AccWs ws;
  ws.gexit = (uint32_t*)(base + l.gexit);
  ws.seqdone = (uint32_t*)(base + l.seqdone);
  ws.err = (uint32_t*)(base + l.err);
  ws.res = (uint64_t*)(base + l.res);
  ws.frontier = (uint32_t*)(base + l.frontier);
  ws.cancel = (uint32_t*)(base + l.cancel);
  ws.seqexit = (uint32_t*)(base + l.seqexit);
  ws.xs = (XSlot*)(base + l.xs);
  return ws;
}

}  // namespace
