// Internal helpers shared by the libspecverify kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "specverify.h"

#define SV_MAX_N 256
#define SV_MAX_DEPTH 16
#define SV_MAX_W 4  // ceil(SV_MAX_N / 64)

typedef __bf16 sv_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 sv_bf16x2 __attribute__((ext_vector_type(2)));
typedef float sv_f32x16 __attribute__((ext_vector_type(16)));
typedef float sv_f32x4 __attribute__((ext_vector_type(4)));

// bf16 bit pattern -> float (exact)
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t x = __float_as_uint(f);
  x += 0x7fffu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }

// Translate a HIP launch error into an sv_status.
static inline sv_status sv_launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

// SV_FLAG_VALIDATE (reference mode): a synchronous call needs a stream that is not being
// captured into a graph.  Checked before anything is enqueued.
static inline sv_status sv_validate_ready(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) return SV_ERR_HIP;
  return cs == hipStreamCaptureStatusNone ? SV_OK : SV_ERR_INVALID_ARGUMENT;
}

// SV_FLAG_VALIDATE: wait for the stream and read the per-sequence status back;
// SV_ERR_BAD_TREE when some sequence reports a non-zero code.
static inline sv_status sv_validate_status(const int32_t* status, int32_t B, hipStream_t st) {
  std::vector<int32_t> h((size_t)B);
  if (hipMemcpyAsync(h.data(), status, (size_t)B * sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess)
    return SV_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return SV_ERR_HIP;
  for (int32_t b = 0; b < B; ++b)
    if (h[(size_t)b] != 0) return SV_ERR_BAD_TREE;
  return SV_OK;
}

// Wait until this wave's outstanding LDS operations have completed, so that
// lanes of the same wave can read what other lanes just wrote.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Argument checks of sv_tree_attention (sv_attention.hip).
sv_status sv_attn_validate(const sv_attn_args& a);

// Threshold acceptance (sv_threshold.hip): workspace bytes and launch of both kernels.
size_t sv_threshold_workspace(const sv_accept_args& a);
sv_status sv_threshold_launch(const sv_accept_args& a, const sv_commit_args& cm, int32_t has_cm, hipStream_t stream);
