// KV commit of the accepted branch.  "EAGLE-Pangu: Accelerator-Safe Tree
// Speculative Decoding on Ascend NPUs", technical summary sec. 2 (branchable
// KV cache): committed prefix and speculative state are kept apart, and the
// accepted path's new entries are committed by length or by path index; the
// path-index commit avoids memory moves that are not needed.
//
// The accepted length never leaves the device.  Every kernel below first
// checks all accepted positions of its sequence (nothing is written for a
// sequence that fails a check), then moves whole rows with 16-byte vector
// loads and stores.
//  k_kv_commit           one work-group per sequence, one layer, tree rows in
//                        their own tensor: checks, copies every KV head and
//                        writes new_len / committed_slots / status.
//  k_kv_commit_rows      one work-group per (sequence, run of layers), every KV
//                        head: the layer-batched commit and the in-place
//                        compaction of cache-resident tree rows.  One wave
//                        moves one (layer, head) plane: it loads all of the
//                        plane's source rows into registers and waits for them
//                        before writing any destination row, so a path in any
//                        node order compacts correctly; rows already in place
//                        are skipped.
//  k_kv_commit_finalize  one work-group per sequence, launched after
//                        k_kv_commit_rows: writes new_len / committed_slots /
//                        status (new_len may alias prefix_len, which every
//                        k_kv_commit_rows work-group has read by then).
#include "sv_commit_dev.h"

namespace {

struct CommitPlan {
  int32_t es;   // bytes per element
  int32_t cpr;  // 16-byte chunks per row
};

// Shared-memory result of the per-sequence checks.
struct CommitCheck {
  int32_t code, L, A;
  int64_t dst[SV_MAX_DEPTH];  // destination slot of accepted position k
  int64_t src[SV_MAX_DEPTH];  // source: tree row (separate tree rows) or cache slot (tree_in_cache)
};

using svc::cache_row;
using svc::capacity;
using svc::slot_of;

// Checks of one sequence, one thread per accepted position (all loads issued at once):
// L >= 0 and 0 <= A <= max_depth (1); with cache-resident tree rows L + N within the
// capacity (6); then per position k in order: source row in [1, N] (1), destination
// slot (6 capacity, 5 block), cache-resident source slot (5).  The first failing
// position decides the code, as a walk in position order would.
__device__ void commit_check(const sv_commit_args& a, int b, CommitCheck& c) {
  __shared__ int32_t s_code;
  const int t = threadIdx.x;
  const int Dm = a.max_depth;
  if (t == 0) s_code = 0x7fffffff;
  __syncthreads();
  const int32_t L0 = a.prefix_len[b];
  const int32_t A0 = a.accept_len[b];
  const bool seq_ok = L0 >= 0 && A0 >= 0 && A0 <= Dm;
  const bool fits = !a.tree_in_cache || (int64_t)L0 + a.N <= capacity(a);
  if (t == 0) {
    c.L = L0;
    c.A = A0;
    if (!seq_ok) s_code = SV_SEQ_PARENT_RANGE;
    else if (!fits) s_code = SV_SEQ_CAPACITY;
  }
  if (t < Dm && seq_ok && fits && t < A0) {
    const int k = t;
    const int32_t src = a.commit_mode == SV_COMMIT_PATH ? a.accept_rows[(int64_t)b * Dm + k] : k + 1;
    int32_t code = 0;
    int64_t dslot = 0, sslot = src;
    if (src < 1 || src > a.N) {
      code = SV_SEQ_PARENT_RANGE;
    } else {
      code = slot_of(a, b, (int64_t)L0 + k, &dslot);
      if (code == 0 && a.tree_in_cache) code = slot_of(a, b, (int64_t)L0 + src - 1, &sslot);
    }
    c.dst[k] = dslot;
    c.src[k] = sslot;
    if (code != 0) atomicMin(&s_code, (k << 4) | code);
  }
  __syncthreads();
  if (t == 0) c.code = s_code == 0x7fffffff ? 0 : (s_code & 15);
  __syncthreads();
}


__device__ void write_outputs(const sv_commit_args& a, int b, const CommitCheck& c) {
  const int t = threadIdx.x;
  const int Dm = a.max_depth;
  if (t < Dm) a.committed_slots[(int64_t)b * Dm + t] = (c.code == 0 && t < c.A) ? (int32_t)c.dst[t] : 0;
  if (t == 0) {
    a.status[b] = c.code;
    a.new_len[b] = c.code == 0 ? c.L + c.A : c.L;
  }
}

__global__ void __launch_bounds__(256) k_kv_commit(sv_commit_args a, CommitPlan p) {
  __shared__ CommitCheck c;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  commit_check(a, b, c);
  const int A = c.A;
  if (c.code == 0) {
    // A rows x Hkv heads x D elements for K and V, 16 bytes per move
    const int64_t total = (int64_t)A * a.Hkv * p.cpr;
    const int64_t row_bytes = (int64_t)a.D * p.es;
    for (int64_t x = t; x < total; x += blockDim.x) {
      const int ch = (int)(x % p.cpr);
      const int h = (int)((x / p.cpr) % a.Hkv);
      const int k = (int)(x / ((int64_t)p.cpr * a.Hkv));
      const int64_t src_row = ((int64_t)b * a.Hkv + h) * (a.N + 1) + c.src[k];
      const int64_t dst_row = cache_row(a, b, h, c.dst[k]);
      const uint4* ks = (const uint4*)((const char*)a.k_tree + src_row * row_bytes) + ch;
      const uint4* vs = (const uint4*)((const char*)a.v_tree + src_row * row_bytes) + ch;
      uint4* kd = (uint4*)((char*)a.k_cache + dst_row * row_bytes) + ch;
      uint4* vd = (uint4*)((char*)a.v_cache + dst_row * row_bytes) + ch;
      *kd = *ks;
      *vd = *vs;
    }
  }
  // prefix_len was read by commit_check before its barrier, so new_len may alias it
  write_outputs(a, b, c);
}

// Addresses of the layered commit: head h of a row sits hstride rows after head 0 (paged:
// within its block; contiguous: the next head's plane), so every chunk's address is a base
// row of its position k plus multiples of strides -- no 64-bit division per chunk.
struct CommitRows {
  int64_t src[SV_MAX_DEPTH], dst[SV_MAX_DEPTH];  // row of KV head 0 for accepted position k
};

__device__ void commit_rows(const sv_commit_args& a, int b, const CommitCheck& c, CommitRows& r) {
  const int t = threadIdx.x;
  if (t < c.A) {
    r.dst[t] = cache_row(a, b, 0, c.dst[t]);
    r.src[t] = a.tree_in_cache ? cache_row(a, b, 0, c.src[t]) : (int64_t)b * a.Hkv * (a.N + 1) + c.src[t];
  }
  __syncthreads();
}

// Chunk y of a (layer, head) unit: K or V, accepted position k, 16-byte chunk ch of the row.
struct UnitChunk {
  const char* src;
  char* dst;
  bool move;
};
__device__ __forceinline__ UnitChunk unit_chunk(const sv_commit_args& a, const CommitPlan& p, const CommitCheck& c,
                                                const CommitRows& r, int layer, int h, int y, int A) {
  const int64_t hstride = a.paged ? a.block_size : a.Lcap;
  const int64_t tstride = a.tree_in_cache ? hstride : (int64_t)(a.N + 1);
  const int64_t row_bytes = (int64_t)a.D * p.es;
  const int kv = y / (A * p.cpr), k = (y / p.cpr) % A, ch = y % p.cpr;
  UnitChunk u;
  u.move = !(a.tree_in_cache && c.src[k] == c.dst[k]);  // a row already in place stays
  const char* sb = a.tree_in_cache ? (const char*)(kv ? a.v_cache : a.k_cache) + layer * a.cache_layer_stride * p.es
                                   : (const char*)(kv ? a.v_tree : a.k_tree) + layer * a.tree_layer_stride * p.es;
  char* db = (char*)(kv ? a.v_cache : a.k_cache) + layer * a.cache_layer_stride * p.es;
  u.src = sb + (r.src[k] + h * tstride) * row_bytes + ch * 16;
  u.dst = db + (r.dst[k] + h * hstride) * row_bytes + ch * 16;
  return u;
}

// Small units (at most 64 * CM_CPL chunks: bf16 D 128 up to 8 accepted rows, D 64 up to 16):
// one work-group per (sequence, run of `lpw` layers); its four waves take batches of whole
// (layer, KV head) units in turn; every lane loads its chunks of the batch into registers,
// the wave waits for all of them, then stores.  Rows of one cache plane are only ever touched
// by the wave that owns the unit, so an in-place compaction never overwrites a row it still
// has to read, and waves never wait for each other.
constexpr int CM_THREADS = 256;
constexpr int CM_CPL = 4;  // chunks per lane per batch (more would spill the addresses)

__global__ void __launch_bounds__(CM_THREADS) k_kv_commit_rows(sv_commit_args a, CommitPlan p, int lpw, int layers) {
  __shared__ CommitCheck c;
  __shared__ CommitRows r;
  const int b = blockIdx.x;
  const int l0 = blockIdx.y * lpw;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  commit_check(a, b, c);
  if (c.code != 0) return;
  const int A = c.A;
  const int nl = min(lpw, layers - l0);
  if (A == 0 || nl <= 0) return;
  commit_rows(a, b, c, r);
  const int per_unit = A * p.cpr * 2;        // <= 64 * CM_CPL on this path
  const int upb = (64 * CM_CPL) / per_unit;  // whole units per wave batch (>= 1)
  const int units = nl * a.Hkv;
  for (int u0 = wv * upb; u0 < units; u0 += (CM_THREADS / 64) * upb) {
    const int nb = min(upb, units - u0) * per_unit;
    uint4 v[CM_CPL];
#pragma unroll
    for (int i = 0; i < CM_CPL; ++i) {
      const int x = lane + i * 64;
      if (x >= nb) continue;
      const int u = u0 + x / per_unit;
      const UnitChunk q = unit_chunk(a, p, c, r, l0 + u / a.Hkv, u % a.Hkv, x % per_unit, A);
      if (q.move) v[i] = *(const uint4*)q.src;
    }
    // every load of the batch's units has returned before any of their stores
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < CM_CPL; ++i) {
      const int x = lane + i * 64;
      if (x >= nb) continue;
      const int u = u0 + x / per_unit;
      const UnitChunk q = unit_chunk(a, p, c, r, l0 + u / a.Hkv, u % a.Hkv, x % per_unit, A);
      if (q.move) *(uint4*)q.dst = v[i];
    }
  }
}

// Large units (up to 1024 chunks): rounds of whole units staged in LDS; every source chunk of a
// round is in LDS before the barrier and written after it.
constexpr int STAGE_CHUNKS = 2048;

__global__ void __launch_bounds__(CM_THREADS) k_kv_commit_rows_lds(sv_commit_args a, CommitPlan p, int lpw,
                                                                   int layers) {
  __shared__ CommitCheck c;
  __shared__ CommitRows r;
  __shared__ uint4 stage[STAGE_CHUNKS];
  const int b = blockIdx.x;
  const int l0 = blockIdx.y * lpw;
  const int t = threadIdx.x;
  commit_check(a, b, c);
  if (c.code != 0) return;
  const int A = c.A;
  const int nl = min(lpw, layers - l0);
  if (A == 0 || nl <= 0) return;
  commit_rows(a, b, c, r);
  const int per_unit = A * p.cpr * 2;
  const int upr = STAGE_CHUNKS / per_unit;  // units per round (>= 2)
  const int units = nl * a.Hkv;
  for (int u0 = 0; u0 < units; u0 += upr) {
    const int n = min(upr, units - u0) * per_unit;
    for (int x = t; x < n; x += CM_THREADS) {
      const int u = u0 + x / per_unit;
      const UnitChunk q = unit_chunk(a, p, c, r, l0 + u / a.Hkv, u % a.Hkv, x % per_unit, A);
      if (q.move) stage[x] = *(const uint4*)q.src;
    }
    __syncthreads();
    for (int x = t; x < n; x += CM_THREADS) {
      const int u = u0 + x / per_unit;
      const UnitChunk q = unit_chunk(a, p, c, r, l0 + u / a.Hkv, u % a.Hkv, x % per_unit, A);
      if (q.move) *(uint4*)q.dst = stage[x];
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(64) k_kv_commit_finalize(sv_commit_args a) {
  __shared__ CommitCheck c;
  const int b = blockIdx.x;
  commit_check(a, b, c);
  write_outputs(a, b, c);
}

}  // namespace

extern "C" sv_status sv_kv_commit(const sv_commit_args* args, void* stream) {
  if (!args) return SV_ERR_INVALID_ARGUMENT;
  const sv_commit_args& a = *args;
  if (a.B < 0 || a.N < 1 || a.N > SV_MAX_N || a.Hkv < 1 || a.max_depth < 1 || a.max_depth > SV_MAX_DEPTH)
    return SV_ERR_INVALID_ARGUMENT;
  if (a.D != 64 && a.D != 128) return SV_ERR_UNSUPPORTED;
  if (a.dtype != SV_F32 && a.dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
  if (a.commit_mode != SV_COMMIT_PATH && a.commit_mode != SV_COMMIT_LENGTH) return SV_ERR_INVALID_ARGUMENT;
  if (a.tree_in_cache != 0 && a.tree_in_cache != 1) return SV_ERR_INVALID_ARGUMENT;
  if (a.num_layers < 0 || a.num_layers > 65535) return SV_ERR_INVALID_ARGUMENT;
  const int layers = a.num_layers == 0 ? 1 : a.num_layers;
  if (layers > 1 && (a.cache_layer_stride <= 0 || (!a.tree_in_cache && a.tree_layer_stride <= 0)))
    return SV_ERR_INVALID_ARGUMENT;
  if (a.B == 0) return SV_OK;
  if (!a.k_cache || !a.v_cache || (!a.tree_in_cache && (!a.k_tree || !a.v_tree)) || !a.prefix_len ||
      !a.accept_len || !a.new_len || !a.committed_slots || !a.status)
    return SV_ERR_INVALID_ARGUMENT;
  if (a.commit_mode == SV_COMMIT_PATH && !a.accept_rows) return SV_ERR_INVALID_ARGUMENT;
  if (a.paged) {
    if (a.block_size != 16 || a.max_blocks < 1 || a.num_blocks < 1 || !a.block_table) return SV_ERR_INVALID_ARGUMENT;
  } else if (a.Lcap < 1) {
    return SV_ERR_INVALID_ARGUMENT;
  }
  CommitPlan p;
  p.es = a.dtype == SV_F32 ? 4 : 2;
  p.cpr = a.D * p.es / 16;
  hipStream_t s = (hipStream_t)stream;
  if (layers == 1 && !a.tree_in_cache) {
    hipLaunchKernelGGL(k_kv_commit, dim3(a.B), dim3(256), 0, s, a, p);
  } else {
    // about a thousand work-groups: enough to fill the device, few enough that dispatch keeps up
    int lpw = (int)(((int64_t)a.B * layers + 1023) / 1024);
    if (lpw < 1) lpw = 1;
    const int runs = (layers + lpw - 1) / lpw;
    // the largest unit this call can have: max_depth accepted rows
    if (a.max_depth * p.cpr * 2 <= 64 * CM_CPL)
      hipLaunchKernelGGL(k_kv_commit_rows, dim3((unsigned)a.B, (unsigned)runs), dim3(CM_THREADS), 0, s, a, p, lpw, layers);
    else
      hipLaunchKernelGGL(k_kv_commit_rows_lds, dim3((unsigned)a.B, (unsigned)runs), dim3(CM_THREADS), 0, s, a, p, lpw,
                         layers);
    hipLaunchKernelGGL(k_kv_commit_finalize, dim3(a.B), dim3(64), 0, s, a);
  }
  return sv_launch_status();
}
