// Tree tensorisation: parent array -> ancestor bitsets, depths, path rows,
// per-sequence status.  "EAGLE-Pangu: Accelerator-Safe Tree Speculative
// Decoding on Ascend NPUs", technical summary sec. 2: shifted indexing with a
// dummy root row 0 instead of the -1 sentinel, ancestor index tables, and
// range / acyclicity / depth checks before the fused kernels run.
//
// One work-group per sequence, one thread per node (N <= 256).  The parent
// array is staged in LDS; each thread walks up at most max_depth (<= 16)
// steps, keeping the visited set as a 256-bit register bitset, which is both
// the cycle detector and the node's attention-mask row.
#include "sv_mask_dev.h"

namespace {

__global__ void __launch_bounds__(256) k_build_tree_mask(const int32_t* __restrict__ parents, int32_t N,
                                                          int32_t max_depth, int32_t W, uint64_t* __restrict__ anc_bits,
                                                          int32_t* __restrict__ depth_out,
                                                          int32_t* __restrict__ path_rows,
                                                          int32_t* __restrict__ status) {
  __shared__ int32_t spar[SV_MAX_N];
  __shared__ int32_t worst;
  mask_seq(parents, N, max_depth, W, anc_bits, depth_out, path_rows, status, blockIdx.x, spar, &worst);
}

}  // namespace

extern "C" sv_status sv_build_tree_mask(const int32_t* parents, int32_t B, int32_t N, int32_t max_depth,
                                        uint64_t* anc_bits, int32_t* depth, int32_t* path_rows, int32_t* status,
                                        uint32_t flags, void* stream) {
  if (B < 0 || N < 1 || N > SV_MAX_N || max_depth < 1 || max_depth > SV_MAX_DEPTH) return SV_ERR_INVALID_ARGUMENT;
  if (flags & ~(uint32_t)SV_FLAG_VALIDATE) return SV_ERR_INVALID_ARGUMENT;
  if (B == 0) return SV_OK;
  if (!parents || !anc_bits || !depth || !status) return SV_ERR_INVALID_ARGUMENT;
  hipStream_t st = (hipStream_t)stream;
  const bool validate = (flags & SV_FLAG_VALIDATE) != 0;
  if (validate) {
    const sv_status r = sv_validate_ready(st);
    if (r != SV_OK) return r;
  }
  const int W = (N + 63) / 64;
  hipLaunchKernelGGL(k_build_tree_mask, dim3(B), dim3(256), 0, st, parents, N, max_depth, W, anc_bits, depth,
                     path_rows, status);
  const sv_status ls = sv_launch_status();
  if (ls != SV_OK || !validate) return ls;
  return sv_validate_status(status, B, st);
}
