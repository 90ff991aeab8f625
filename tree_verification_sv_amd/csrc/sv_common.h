// Internal helpers shared by the libspecverify kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Wait until this wave's outstanding LDS operations have completed, so that
// lanes of the same wave can read what other lanes just wrote.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Threshold acceptance (sv_threshold.hip): workspace bytes and launch of both kernels.
size_t sv_threshold_workspace(const sv_accept_args& a);
sv_status sv_threshold_launch(const sv_accept_args& a, const sv_commit_args& cm, int32_t has_cm, hipStream_t stream);
