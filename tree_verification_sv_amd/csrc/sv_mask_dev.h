// Tree tensorisation of one sequence by one work-group, shared by sv_build_tree_mask and the
// one-launch verification step.  "EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on
// Ascend NPUs", technical summary sec. 2: shifted indexing with a dummy root row 0 instead of
// the -1 sentinel, ancestor index tables, and range / acyclicity / depth checks.  Each thread
// owns one node and walks up at most max_depth (<= 16) steps, keeping the visited set as a
// 256-bit register bitset, which is both the cycle detector and the node's mask row.
#pragma once
#include "sv_common.h"

namespace {

__device__ __forceinline__ bool bit_get(const uint64_t (&w)[SV_MAX_W], int j) {
  const int q = j >> 6;
  const uint64_t m = 1ull << (j & 63);
  uint64_t x = q == 0 ? w[0] : q == 1 ? w[1] : q == 2 ? w[2] : w[3];
  return (x & m) != 0;
}

__device__ __forceinline__ void bit_set(uint64_t (&w)[SV_MAX_W], int j) {
  const int q = j >> 6;
  const uint64_t m = 1ull << (j & 63);
  if (q == 0) w[0] |= m;
  else if (q == 1) w[1] |= m;
  else if (q == 2) w[2] |= m;
  else w[3] |= m;
}

// Mask of sequence b by one work-group (one node per thread: at least N threads); spar: N ints of LDS, worst: one int of LDS.
__device__ __forceinline__ void mask_seq(const int32_t* __restrict__ parents, int32_t N, int32_t max_depth,
                                         int32_t W, uint64_t* __restrict__ anc_bits, int32_t* __restrict__ depth_out,
                                         int32_t* __restrict__ path_rows, int32_t* __restrict__ status, int b,
                                         int32_t* spar, int32_t* worst) {
  const int t = threadIdx.x;
  if (t == 0) *worst = 0x7fffffff;
  if (t < N) spar[t] = parents[(int64_t)b * N + t];
  __syncthreads();
  if (t < N) {
    uint64_t bits[SV_MAX_W] = {0, 0, 0, 0};
    bit_set(bits, t);
    int count = 1;
    int cur = t;
    int code = 0;
    // at most max_depth iterations: every iteration either exits or grows count
    for (int step = 0; step <= SV_MAX_DEPTH; ++step) {
      const int p = spar[cur];
      if (p < -1 || p >= N) { code = SV_SEQ_PARENT_RANGE; break; }
      if (p == -1) break;
      if (bit_get(bits, p)) { code = SV_SEQ_CYCLE; break; }
      if (count + 1 > max_depth) { code = SV_SEQ_DEPTH; break; }
      bit_set(bits, p);
      ++count;
      cur = p;
    }
    uint64_t* arow = anc_bits + ((int64_t)b * N + t) * W;
    int32_t* prow = path_rows ? path_rows + ((int64_t)b * (N + 1) + (t + 1)) * max_depth : nullptr;
    if (code == 0) {
#pragma unroll
      for (int w = 0; w < SV_MAX_W; ++w)  // constant indices keep the bitset in registers
        if (w < W) arow[w] = bits[w];
      depth_out[(int64_t)b * N + t] = count;
      if (prow) {
        // the walk from t visits depths count, count-1, ..., 1
        int node = t;
        for (int k = count - 1; k >= 0; --k) {
          prow[k] = node + 1;  // node `node` lives in row node+1
          node = spar[node];
        }
        for (int k = count; k < max_depth; ++k) prow[k] = 0;
      }
    } else {
      for (int w = 0; w < W; ++w) arow[w] = (w == (t >> 6)) ? (1ull << (t & 63)) : 0ull;
      depth_out[(int64_t)b * N + t] = 0;
      if (prow)
        for (int k = 0; k < max_depth; ++k) prow[k] = 0;
      atomicMin(worst, code);
    }
  }
  if (path_rows && t < max_depth) path_rows[((int64_t)b * (N + 1)) * max_depth + t] = 0;
  __syncthreads();
  if (t == 0) status[b] = *worst == 0x7fffffff ? 0 : *worst;
}

}  // namespace
