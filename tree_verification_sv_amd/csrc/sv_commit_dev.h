// Device helpers of the KV commit ("EAGLE-Pangu: Accelerator-Safe Tree
// Speculative Decoding on Ascend NPUs", technical summary sec. 2: the accepted
// path's entries are committed after the prefix, by length or by path index),
// shared by the commit kernels and by the acceptance walkers that commit the
// path they just found (sv_accept_args.commit).
#pragma once
#include "sv_common.h"

namespace svc {

__device__ __forceinline__ int64_t capacity(const sv_commit_args& a) {
  return a.paged ? (int64_t)a.max_blocks * a.block_size : (int64_t)a.Lcap;
}

// Logical position -> slot of sequence b (checked: 0 ok, else a status code).
__device__ __forceinline__ int32_t slot_of(const sv_commit_args& a, int b, int64_t pos, int64_t* slot) {
  if (a.paged) {
    const int64_t blk = pos / a.block_size;
    if (blk >= a.max_blocks) return SV_SEQ_CAPACITY;
    const int32_t id = a.block_table[(int64_t)b * a.max_blocks + blk];
    if (id < 1 || id >= a.num_blocks) return SV_SEQ_BLOCK;
    *slot = (int64_t)id * a.block_size + pos % a.block_size;
  } else {
    if (pos >= a.Lcap) return SV_SEQ_CAPACITY;
    *slot = pos;
  }
  return 0;
}

// Row index (in rows of D elements) of slot `slot`, KV head h, sequence b, within one layer's cache.
__device__ __forceinline__ int64_t cache_row(const sv_commit_args& a, int b, int h, int64_t slot) {
  if (a.paged) {
    const int64_t id = slot / a.block_size, off = slot % a.block_size;
    return (id * a.Hkv + h) * a.block_size + off;
  }
  return ((int64_t)b * a.Hkv + h) * a.Lcap + slot;
}

// Commit of sequence b's accepted path by the work-group that found it (every thread calls
// it; single layer, tree rows in their own tensor).  path[k] (LDS) is the node at depth k + 1
// of the path and A its length.  Same checks, outputs and "nothing written on error" as
// sv_kv_commit: L >= 0 and 0 <= A <= max_depth (1), source row in [1, N] (1), destination slot
// (6 capacity, 5 block), the first failing position deciding the code.
__device__ __forceinline__ void walker_commit(const sv_commit_args& c, int b, int A, const int32_t* path) {
  __shared__ int64_t wc_slot[SV_MAX_DEPTH];
  __shared__ int32_t wc_src[SV_MAX_DEPTH];
  __shared__ int32_t wc_code, wc_L;
  const int t = threadIdx.x;
  const int Dm = c.max_depth;
  if (t == 0) wc_code = 0x7fffffff;
  __syncthreads();
  const int32_t L0 = c.prefix_len[b];
  const bool seq_ok = L0 >= 0 && A >= 0 && A <= Dm;
  if (t == 0) {
    wc_L = L0;
    if (!seq_ok) wc_code = SV_SEQ_PARENT_RANGE;
  }
  if (seq_ok && t < A) {
    const int32_t src = c.commit_mode == SV_COMMIT_PATH ? path[t] + 1 : t + 1;
    int64_t slot = 0;
    const int32_t code = (src < 1 || src > c.N) ? SV_SEQ_PARENT_RANGE : slot_of(c, b, (int64_t)L0 + t, &slot);
    wc_slot[t] = slot;
    wc_src[t] = src;
    if (code != 0) atomicMin(&wc_code, (t << 4) | code);
  }
  __syncthreads();
  const int32_t code = wc_code == 0x7fffffff ? 0 : (wc_code & 15);
  if (t < Dm) c.committed_slots[(int64_t)b * Dm + t] = (code == 0 && t < A) ? (int32_t)wc_slot[t] : 0;
  if (t == 0) {
    c.status[b] = code;
    c.new_len[b] = code == 0 ? wc_L + A : wc_L;  // prefix_len was read before the barrier
  }
  if (code != 0) return;  // uniform
  const int es = c.dtype == SV_F32 ? 4 : 2;
  const int cpr = c.D * es / 16;
  const int64_t row_bytes = (int64_t)c.D * es;
  const int64_t total = (int64_t)A * c.Hkv * cpr;
  for (int64_t x = t; x < total; x += blockDim.x) {
    const int ch = (int)(x % cpr);
    const int h = (int)((x / cpr) % c.Hkv);
    const int k = (int)(x / ((int64_t)cpr * c.Hkv));
    const int64_t src_row = ((int64_t)b * c.Hkv + h) * (c.N + 1) + wc_src[k];
    const int64_t dst_row = cache_row(c, b, h, wc_slot[k]);
    *((uint4*)((char*)c.k_cache + dst_row * row_bytes) + ch) = *((const uint4*)((const char*)c.k_tree + src_row * row_bytes) + ch);
    *((uint4*)((char*)c.v_cache + dst_row * row_bytes) + ch) = *((const uint4*)((const char*)c.v_tree + src_row * row_bytes) + ch);
  }
}

// Host-side check that a commit can run inside an acceptance kernel.
inline sv_status walker_commit_ok(const sv_commit_args& c, int32_t B, int32_t N, int32_t max_depth) {
  if (c.B != B || c.N != N || c.max_depth != max_depth) return SV_ERR_INVALID_ARGUMENT;
  if (c.Hkv < 1 || (c.D != 64 && c.D != 128)) return SV_ERR_INVALID_ARGUMENT;
  if (c.dtype != SV_F32 && c.dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
  if (c.commit_mode != SV_COMMIT_PATH && c.commit_mode != SV_COMMIT_LENGTH) return SV_ERR_INVALID_ARGUMENT;
  if (c.tree_in_cache || c.num_layers > 1) return SV_ERR_UNSUPPORTED;  // those run as sv_kv_commit
  if (!c.k_cache || !c.v_cache || !c.k_tree || !c.v_tree || !c.prefix_len || !c.new_len || !c.committed_slots ||
      !c.status)
    return SV_ERR_INVALID_ARGUMENT;
  if (c.paged) {
    if (c.block_size != 16 || c.max_blocks < 1 || c.num_blocks < 1 || !c.block_table) return SV_ERR_INVALID_ARGUMENT;
  } else if (c.Lcap < 1) {
    return SV_ERR_INVALID_ARGUMENT;
  }
  return SV_OK;
}

}  // namespace svc
