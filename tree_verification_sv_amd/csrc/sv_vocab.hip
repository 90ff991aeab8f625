// Draft vocabulary subset.  "EAGLE-Pangu: Accelerator-Safe Tree Speculative
// Decoding on Ascend NPUs", technical summary sec. 3, item 5: the drafter works
// on a cached subset of the vocabulary.  Acceptance compares full draft and
// target distributions ("Accelerating Sonar Through Speculation",
// "Objetivo-Borrador"), so the draft logits are laid out over the target
// vocabulary with -inf (probability 0) outside the subset.
//
// k_draft_subset<T, AL>: gather form, one thread per 16 bytes of output.  Each
// output entry v reads t2d[v] (j + 1, or 0 when v is not in the subset) and
// then the subset logit j of its row; writes are whole 16-byte stores, so every
// output row streams out coalesced, and no two threads write one entry.
#include <math.h>

#include "sv_common.h"

namespace {

template <typename T, bool AL>
__global__ void __launch_bounds__(256) k_draft_subset(const T* sub, int32_t Vd, const int32_t* t2d, int32_t V,
                                                      int64_t chunks_per_row, int64_t total, T* full) {
  constexpr int EPC = 16 / sizeof(T);  // entries per 16-byte chunk
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= total) return;  // the grid is rounded up to whole work-groups
  const int64_t row = g / chunks_per_row;
  const int v0 = (int)(g % chunks_per_row) * EPC;
  const T* srow = sub + row * Vd;
  T* frow = full + row * V;
  T vals[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    const int v = v0 + e;
    const int j = v < V ? t2d[v] : 0;
    if (j >= 1 && j <= Vd) {
      vals[e] = srow[j - 1];
    } else {
      if constexpr (sizeof(T) == 4) vals[e] = -INFINITY;
      else vals[e] = (T)0xFF80u;  // bf16 -inf
    }
  }
  if (AL && v0 + EPC <= V) {
    uint4 pk;
    __builtin_memcpy(&pk, vals, 16);
    *(uint4*)(frow + v0) = pk;
  } else {
#pragma unroll
    for (int e = 0; e < EPC; ++e)
      if (v0 + e < V) frow[v0 + e] = vals[e];
  }
}

}  // namespace

extern "C" sv_status sv_draft_subset_logits(const void* sub_logits, int32_t B, int32_t R, int32_t Vd,
                                            const int32_t* t2d, int32_t V, int32_t dtype, void* full_logits,
                                            void* stream) {
  if (B < 0 || R < 1 || Vd < 1 || V < 1) return SV_ERR_INVALID_ARGUMENT;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
  if (B == 0) return SV_OK;
  if (!sub_logits || !t2d || !full_logits) return SV_ERR_INVALID_ARGUMENT;
  const int esz = dtype == SV_F32 ? 4 : 2;
  const int epc = 16 / esz;
  const int64_t cpr = (V + epc - 1) / epc;
  const int64_t total = (int64_t)B * R * cpr;
  const int64_t grid = (total + 255) / 256;
  if (grid > 0x7fffffff) return SV_ERR_UNSUPPORTED;
  const bool al = ((int64_t)V * esz) % 16 == 0 && ((uintptr_t)full_logits % 16) == 0;
  hipStream_t s = (hipStream_t)stream;
#define SV_SUB(T, AL)                                                                                   \
  hipLaunchKernelGGL((k_draft_subset<T, AL>), dim3((unsigned)grid), dim3(256), 0, s, (const T*)sub_logits, Vd, \
                     t2d, V, cpr, total, (T*)full_logits)
  if (dtype == SV_F32) {
    if (al) SV_SUB(float, true); else SV_SUB(float, false);
  } else {
    if (al) SV_SUB(uint16_t, true); else SV_SUB(uint16_t, false);
  }
#undef SV_SUB
  return sv_launch_status();
}
