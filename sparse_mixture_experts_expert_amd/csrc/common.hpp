// Shared device-side definitions of the OLMoE MoE library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/olmoe_moe.h"

namespace olmoe {

constexpr int D = OLMOE_D;  // hidden size
constexpr int F = OLMOE_F;  // expert width
constexpr int E = OLMOE_E;  // experts
constexpr int K = OLMOE_K;  // experts per token
constexpr int ROUTE_BLOCK = 16;  // tokens per routing block (one wavefront's share in the router)
// loss weights: load balancing ("OLMoE Guide", item 2) and router z-loss (item 3)
constexpr double LB_ALPHA = 0.01;
constexpr double Z_BETA = 0.001;

typedef uint16_t bf16_t;  // storage type of bfloat16 values
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// round to nearest even; inputs are finite
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// fp16 storage of the intermediates: round to nearest even, saturate at the
// largest finite fp16 so out-of-range activations stay finite
constexpr float F16_MAX = 65504.0f;
__device__ __forceinline__ uint16_t f32_to_f16_sat(float f) {
  const _Float16 h = static_cast<_Float16>(fminf(fmaxf(f, -F16_MAX), F16_MAX));
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_to_f32(uint16_t v) {
  return static_cast<float>(__builtin_bit_cast(_Float16, v));
}

// two fp32 values rounded to nearest even into one packed bf16 pair (gfx950 converts a pair in one
// instruction; NaN stays NaN)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
  return v;
}

// inclusive prefix sum across the 64 lanes of a wavefront
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    int o = __shfl_up(v, s, 64);
    if (lane >= s) v += o;
  }
  return v;
}

}  // namespace olmoe
