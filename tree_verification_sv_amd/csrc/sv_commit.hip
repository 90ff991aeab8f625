// KV commit of the accepted branch.  "EAGLE-Pangu: Accelerator-Safe Tree
// Speculative Decoding on Ascend NPUs", technical summary sec. 2 (branchable
// KV cache): committed prefix and speculative state are kept apart, and the
// accepted path's new entries are appended, by length or by path index.
//
// The accepted length never leaves the device: one work-group per sequence
// reads accept_len / accept_rows / prefix_len, validates every slot first,
// then copies K and V rows of all KV heads with 16-byte vector moves.
#include "sv_common.h"

namespace {

__global__ void __launch_bounds__(256) k_kv_commit(sv_commit_args a, int32_t es) {
  __shared__ int32_t s_code, s_L, s_A;
  __shared__ int64_t s_slot[SV_MAX_DEPTH];
  __shared__ int32_t s_src[SV_MAX_DEPTH];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int Dm = a.max_depth;
  // validation, one thread per accepted position: every load is issued at once (the
  // block-table entry is the only one that depends on another load)
  if (t == 0) s_code = 0x7fffffff;
  __syncthreads();
  const int32_t L0 = a.prefix_len[b];
  const int32_t A0 = a.accept_len[b];
  if (t == 0) {
    s_L = L0;
    s_A = A0;
    if (L0 < 0 || A0 < 0 || A0 > Dm) atomicMin(&s_code, SV_SEQ_PARENT_RANGE);
  }
  if (t < Dm && L0 >= 0 && A0 >= 0 && A0 <= Dm && t < A0) {
    const int k = t;
    int32_t code = 0;
    const int32_t src = a.commit_mode == SV_COMMIT_PATH ? a.accept_rows[(int64_t)b * Dm + k] : k + 1;
    const int64_t pos = (int64_t)L0 + k;
    if (src < 1 || src > a.N) {
      code = SV_SEQ_PARENT_RANGE;
    } else if (a.paged) {
      const int64_t blk = pos / a.block_size;
      if (blk >= a.max_blocks) {
        code = SV_SEQ_CAPACITY;
      } else {
        const int32_t id = a.block_table[(int64_t)b * a.max_blocks + blk];
        if (id < 1 || id >= a.num_blocks) code = SV_SEQ_BLOCK;
        else s_slot[k] = (int64_t)id * a.block_size + pos % a.block_size;
      }
    } else {
      if (pos >= a.Lcap) code = SV_SEQ_CAPACITY;
      else s_slot[k] = pos;
    }
    s_src[k] = src;
    // the first failing position decides the code, as a walk in position order would
    if (code != 0) atomicMin(&s_code, (k << 4) | code);
  }
  __syncthreads();
  if (t == 0) s_code = s_code == 0x7fffffff ? 0 : (s_code & 15);
  __syncthreads();
  const int32_t code = s_code, L = s_L, A = s_A;
  if (t < Dm) a.committed_slots[(int64_t)b * Dm + t] = (code == 0 && t < A) ? (int32_t)s_slot[t] : 0;
  if (code != 0) {
    if (t == 0) {
      a.status[b] = code;
      a.new_len[b] = L;
    }
    return;
  }
  // copy A rows x Hkv heads x D elements for K and V, 16 bytes per move
  const int chunks_per_row = (a.D * es) / 16;
  const int64_t total = (int64_t)A * a.Hkv * chunks_per_row;
  for (int64_t c = t; c < total; c += blockDim.x) {
    const int ch = (int)(c % chunks_per_row);
    const int h = (int)((c / chunks_per_row) % a.Hkv);
    const int k = (int)(c / ((int64_t)chunks_per_row * a.Hkv));
    const int64_t src_row = ((int64_t)b * a.Hkv + h) * (a.N + 1) + s_src[k];
    int64_t dst_row;
    if (a.paged) {
      const int64_t id = s_slot[k] / a.block_size, off = s_slot[k] % a.block_size;
      dst_row = (id * a.Hkv + h) * a.block_size + off;
    } else {
      dst_row = ((int64_t)b * a.Hkv + h) * a.Lcap + s_slot[k];
    }
    const int64_t row_bytes = (int64_t)a.D * es;
    const uint4* ks = (const uint4*)((const char*)a.k_tree + src_row * row_bytes) + ch;
    const uint4* vs = (const uint4*)((const char*)a.v_tree + src_row * row_bytes) + ch;
    uint4* kd = (uint4*)((char*)a.k_cache + dst_row * row_bytes) + ch;
    uint4* vd = (uint4*)((char*)a.v_cache + dst_row * row_bytes) + ch;
    *kd = *ks;
    *vd = *vs;
  }
  if (t == 0) {
    a.status[b] = 0;
    a.new_len[b] = L + A;  // prefix_len was read before the barrier, so aliasing is safe
  }
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
  if (a.B == 0) return SV_OK;
  if (!a.k_cache || !a.v_cache || !a.k_tree || !a.v_tree || !a.prefix_len || !a.accept_len || !a.new_len ||
      !a.committed_slots || !a.status)
    return SV_ERR_INVALID_ARGUMENT;
  if (a.commit_mode == SV_COMMIT_PATH && !a.accept_rows) return SV_ERR_INVALID_ARGUMENT;
  if (a.paged) {
    if (a.block_size != 16 || a.max_blocks < 1 || a.num_blocks < 1 || !a.block_table) return SV_ERR_INVALID_ARGUMENT;
  } else if (a.Lcap < 1) {
    return SV_ERR_INVALID_ARGUMENT;
  }
  const int es = a.dtype == SV_F32 ? 4 : 2;
  hipLaunchKernelGGL(k_kv_commit, dim3(a.B), dim3(256), 0, (hipStream_t)stream, a, es);
  return sv_launch_status();
}
