// Draft vocabulary subset.  "EAGLE-Pangu: Accelerator-Safe Tree Speculative
// Decoding on Ascend NPUs", technical summary sec. 3, item 5: the drafter works
// on a cached subset of the vocabulary.  Acceptance compares full draft and
// target distributions ("Accelerating Sonar Through Speculation",
// "Objetivo-Borrador"), so the draft logits are laid out over the target
// vocabulary with -inf (probability 0) outside the subset.
//
// k_draft_subset<T, AL>: gather form, 16 bytes of output per thread and pass of
// a grid-stride loop (4 passes' loads issued together).  Each output entry v
// reads t2d[v] (j + 1, or 0 when v is not in the subset) and then the subset
// logit j of its row; writes are whole 16-byte stores, so every output row
// streams out coalesced, and no two threads write one entry.
#include <math.h>

#include "sv_common.h"

namespace {

constexpr int DS_UNROLL = 4;  // chunks per thread per pass: their map and logit loads are issued together

template <typename T, bool AL>
__global__ void __launch_bounds__(256) k_draft_subset(const T* sub, int32_t Vd, const int32_t* t2d, int32_t V,
                                                      int64_t chunks_per_row, int64_t total, T* full) {
  constexpr int EPC = 16 / sizeof(T);  // entries per 16-byte chunk
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t g0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t gb = g0; gb < total; gb += stride * DS_UNROLL) {
    int j[DS_UNROLL][EPC];
#pragma unroll
    for (int u = 0; u < DS_UNROLL; ++u) {
      const int64_t g = gb + u * stride;
      const int v0 = (int)(g % chunks_per_row) * EPC;
#pragma unroll
      for (int e = 0; e < EPC; ++e) j[u][e] = (g < total && v0 + e < V) ? t2d[v0 + e] : 0;
    }
    T vals[DS_UNROLL][EPC];
#pragma unroll
    for (int u = 0; u < DS_UNROLL; ++u) {
      const int64_t row = (gb + u * stride) / chunks_per_row;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const int jj = j[u][e];
        if (jj >= 1 && jj <= Vd) {
          vals[u][e] = sub[row * Vd + (jj - 1)];
        } else {
          if constexpr (sizeof(T) == 4) vals[u][e] = -INFINITY;
          else vals[u][e] = (T)0xFF80u;  // bf16 -inf
        }
      }
    }
#pragma unroll
    for (int u = 0; u < DS_UNROLL; ++u) {
      const int64_t g = gb + u * stride;
      if (g >= total) break;
      const int64_t row = g / chunks_per_row;
      const int v0 = (int)(g % chunks_per_row) * EPC;
      T* frow = full + row * V;
      if (AL && v0 + EPC <= V) {
        uint4 pk;
        __builtin_memcpy(&pk, vals[u], 16);
        *(uint4*)(frow + v0) = pk;
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          if (v0 + e < V) frow[v0 + e] = vals[u][e];
      }
    }
  }
}

// LDS form, for subsets of at most 64 KB per row: the work-group first copies its row's
// subset logits into LDS with coalesced loads, then every output entry gathers from LDS
// instead of from scattered cache lines (a random map would otherwise make every lane of a
// gather touch its own line).  Work-group (row, part) writes chunks part, part + parts, ...
constexpr int DL_THREADS = 512;
constexpr int DL_MAX_BYTES = 64 * 1024;

template <typename T, bool AL>
__global__ void __launch_bounds__(DL_THREADS) k_draft_subset_lds(const T* sub, int32_t Vd, const int32_t* t2d,
                                                                 int32_t V, int parts, T* full) {
  constexpr int EPC = 16 / sizeof(T);
  extern __shared__ __align__(16) unsigned char dl_smem[];
  T* srow_l = (T*)dl_smem;
  const int64_t row = blockIdx.x / parts;
  const int part = blockIdx.x % parts;
  const int t = threadIdx.x;
  const T* srow = sub + row * Vd;
  // subset row -> LDS (16-byte pieces when the row is aligned, element by element otherwise)
  const bool sal = AL && ((uintptr_t)srow % 16) == 0;
  if (sal) {
    const int nv = Vd / EPC;
    for (int i = t; i < nv; i += DL_THREADS) ((uint4*)srow_l)[i] = ((const uint4*)srow)[i];
    for (int i = nv * EPC + t; i < Vd; i += DL_THREADS) srow_l[i] = srow[i];
  } else {
    for (int i = t; i < Vd; i += DL_THREADS) srow_l[i] = srow[i];
  }
  __syncthreads();
  T ninf;
  if constexpr (sizeof(T) == 4) ninf = -INFINITY;
  else ninf = (T)0xFF80u;  // bf16 -inf
  T* frow = full + row * V;
  const int chunks = (V + EPC - 1) / EPC;
  for (int c = part * DL_THREADS + t; c < chunks; c += parts * DL_THREADS) {
    const int v0 = c * EPC;
    int j[EPC];
    if (AL && v0 + EPC <= V) {  // the map entries of a chunk are 16-byte aligned (EPC is 4 or 8)
#pragma unroll
      for (int q = 0; q < EPC / 4; ++q) {
        const int4 m4 = ((const int4*)(t2d + v0))[q];
        j[4 * q] = m4.x;
        j[4 * q + 1] = m4.y;
        j[4 * q + 2] = m4.z;
        j[4 * q + 3] = m4.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) j[e] = v0 + e < V ? t2d[v0 + e] : 0;
    }
    T vals[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) vals[e] = (j[e] >= 1 && j[e] <= Vd) ? srow_l[j[e] - 1] : ninf;
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
  // a grid-stride loop over a few thousand work-groups: tens of thousands of one-chunk
  // work-groups would be limited by the work-group dispatch rate, not by HBM
  int64_t grid = (total + 256 * DS_UNROLL - 1) / (256 * DS_UNROLL);
  if (grid > 4096) grid = 4096;
  const bool al = ((int64_t)V * esz) % 16 == 0 && ((uintptr_t)full_logits % 16) == 0;
  hipStream_t s = (hipStream_t)stream;
  if ((int64_t)Vd * esz <= DL_MAX_BYTES) {
    // the map is read as 16-byte vectors on the aligned path, so it must be aligned too
    const bool al2 = al && ((uintptr_t)t2d % 16) == 0;
    const int64_t rows = (int64_t)B * R;
    int parts = (int)((1024 + rows - 1) / rows);  // about a thousand work-groups in all
    if (parts > 16) parts = 16;
    const int64_t grid2 = rows * parts;
    if (grid2 > 0x7fffffff) return SV_ERR_UNSUPPORTED;
    const size_t lds = (size_t)((Vd * esz + 15) / 16 * 16);
#define SV_SUBL(T, AL)                                                                                            hipLaunchKernelGGL((k_draft_subset_lds<T, AL>), dim3((unsigned)grid2), dim3(DL_THREADS), lds, s,                                 (const T*)sub_logits, Vd, t2d, V, parts, (T*)full_logits)
    if (dtype == SV_F32) {
      if (al2) SV_SUBL(float, true); else SV_SUBL(float, false);
    } else {
      if (al2) SV_SUBL(uint16_t, true); else SV_SUBL(uint16_t, false);
    }
#undef SV_SUBL
    return sv_launch_status();
  }
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
