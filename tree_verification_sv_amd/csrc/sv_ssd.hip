// Speculative speculative decoding around the verification step.
//
// "Speculative Speculative Decoding" (gist.science summary), sec. 2: while the
// target verifies, the drafter prepares speculations for the likely outcomes of
// that verification -- how many tokens are accepted and which bonus token is
// drawn; when verification ends, the real outcome either hits that cache (the
// prepared tokens go to the next verification at once) or misses (a fallback
// drafts synchronously).  Sec. 3B (Saguaro sampling): the drafter lowers the
// probability of tokens already in the cache, which moves residual mass onto
// them and makes a cached bonus token more likely.
//
//  k_outcome_lookup   one work-group; thread-per-sequence loop.  The outcome of
//                     sequence b is (stop_row[b], last emitted token); the
//                     first prepared outcome with that key wins.  Outputs stay
//                     on the device (no host round trip between verification
//                     and the next draft), branch k + 1 or the ghost 0.
//  k_saguaro_reweight one thread per (sequence, row, cache entry): adds the
//                     shift to the draft logit of each distinct listed token.
#include "sv_common.h"

namespace {

constexpr int OL_THREADS = 256;

__global__ void __launch_bounds__(OL_THREADS) k_outcome_lookup(sv_outcome_args a) {
  __shared__ int s_hits[OL_THREADS / 64];
  const int t = threadIdx.x;
  const int Dm = a.max_depth;
  int hits = 0;
  for (int b = t; b < a.B; b += OL_THREADS) {
    int found = -1;
    const int n = a.num_out[b];
    if (n >= 1 && n <= Dm + 1) {
      const int row = a.stop_row[b];
      const int bonus = a.out_tokens[(int64_t)b * (Dm + 1) + (n - 1)];
      int nk = a.n_keys[b];
      nk = nk < 0 ? 0 : (nk > a.K ? a.K : nk);
      const int32_t* kr = a.key_row + (int64_t)b * a.K;
      const int32_t* kt = a.key_token + (int64_t)b * a.K;
      for (int k = 0; k < nk; ++k)
        if (kr[k] == row && kt[k] == bonus) {
          found = k;
          break;
        }
    }
    a.hit[b] = found >= 0;
    a.branch[b] = found + 1;
    hits += found >= 0;
    if (a.next_tokens) {
      const int32_t* src = found >= 0 ? a.prepared + ((int64_t)b * a.K + found) * a.P : nullptr;
      for (int j = 0; j < a.P; ++j) a.next_tokens[(int64_t)b * a.P + j] = src ? src[j] : 0;
    }
  }
  if (a.n_hits) {
    for (int o = 32; o > 0; o >>= 1) hits += __shfl_xor(hits, o);
    if ((t & 63) == 0) s_hits[t >> 6] = hits;
    __syncthreads();
    if (t == 0) {
      int tot = 0;
      for (int i = 0; i < OL_THREADS / 64; ++i) tot += s_hits[i];
      a.n_hits[0] = tot;
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(256) k_saguaro_reweight(T* logits, int32_t B, int32_t R, int32_t V,
                                                          const int32_t* cache_tokens, int32_t C, float shift) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)B * R * C) return;
  const int64_t row = e / C;  // b * R + r
  const int c = (int)(e % C);
  const int32_t* list = cache_tokens + row * C;
  const int v = list[c];
  if (v < 0 || v >= V) return;
  for (int k = 0; k < c; ++k)
    if (list[k] == v) return;  // each distinct token once: the first listing owns it
  T* p = logits + row * V + v;
  if constexpr (sizeof(T) == 4) {
    *p = *p + shift;
  } else {
    *p = f32_to_bf16_bits(bf16_bits_to_f32(*p) + shift);
  }
}

}  // namespace

extern "C" sv_status sv_outcome_lookup(const sv_outcome_args* args, void* stream) {
  if (!args) return SV_ERR_INVALID_ARGUMENT;
  const sv_outcome_args& a = *args;
  if (a.B < 0 || a.K < 1 || a.P < 0 || a.max_depth < 1 || a.max_depth > SV_MAX_DEPTH) return SV_ERR_INVALID_ARGUMENT;
  if (a.B == 0) return SV_OK;
  if (!a.stop_row || !a.out_tokens || !a.num_out || !a.key_row || !a.key_token || !a.n_keys || !a.hit || !a.branch)
    return SV_ERR_INVALID_ARGUMENT;
  if (a.next_tokens && a.P > 0 && !a.prepared) return SV_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(k_outcome_lookup, dim3(1), dim3(OL_THREADS), 0, (hipStream_t)stream, a);
  return sv_launch_status();
}

extern "C" sv_status sv_saguaro_reweight(void* draft_logits, int32_t B, int32_t R, int32_t V, int32_t dtype,
                                         const int32_t* cache_tokens, int32_t C, float shift, void* stream) {
  if (B < 0 || R < 1 || V < 1 || C < 0) return SV_ERR_INVALID_ARGUMENT;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
  if (!(shift == shift) || shift == INFINITY || shift == -INFINITY) return SV_ERR_INVALID_ARGUMENT;
  if (B == 0 || C == 0) return SV_OK;
  if (!draft_logits || !cache_tokens) return SV_ERR_INVALID_ARGUMENT;
  const int64_t n = (int64_t)B * R * C;
  const int64_t grid = (n + 255) / 256;
  if (grid > 0x7fffffff) return SV_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == SV_F32)
    hipLaunchKernelGGL(k_saguaro_reweight<float>, dim3((unsigned)grid), dim3(256), 0, s, (float*)draft_logits, B, R, V,
                       cache_tokens, C, shift);
  else
    hipLaunchKernelGGL(k_saguaro_reweight<uint16_t>, dim3((unsigned)grid), dim3(256), 0, s, (uint16_t*)draft_logits,
                       B, R, V, cache_tokens, C, shift);
  return sv_launch_status();
}
