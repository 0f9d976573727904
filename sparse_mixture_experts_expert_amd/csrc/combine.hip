// Weighted combine of the OLMoE MoE layer and the residual-stack glue.
//
// combine: out[t] = sum_{j=0..7} p[t,j] * Y[inv[t,j]] (Y rows in fp16), the probability-weighted
// sum of the chosen experts' outputs ("OLMoE Guide: 64-Expert Fine-Grained Open
// MoE Architecture", item 1; "Mixture-of-experts LLMs from scratch with OLMoE",
// section 2, where each result is added back to its token, weighted).  Every
// token gathers its own 8 rows and sums them in slot order in fp32, so no two
// threads ever add into the same output: no atomics, reproducible bit for bit.
//
// rmsnorm / residual_add: the pre-norm residual block of the same page's
// section 3, h <- h + MoE(RMSNorm(h)) with h kept in fp32 and unit norm weight.
// The residual epilogue of combine fuses both into the layer: the fp32 sum goes
// straight into h (no bf16 rounding of the layer output) and the wave that owns
// the token's row then writes the next layer's input bf16(RMSNorm(h)), so the
// stack reads and writes h once per layer.
#include "common.hpp"
#include "kernels.hpp"

namespace olmoe {

namespace {

// residual variant: one wavefront per token, 64 lanes x 32 columns (four 16-byte chunks per lane)
constexpr int CMB_TOK_PER_WG = 4;

template <bool RESIDUAL>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int t = RESIDUAL ? blockIdx.x * CMB_TOK_PER_WG + (threadIdx.x >> 6) : blockIdx.x;
  if (t >= a.T) return;
  const int lane = threadIdx.x & 63;
  int pos[K];
  float p[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    pos[j] = a.inv[t * K + j];
    p[j] = a.probs[t * K + j];
  }
  constexpr int NC = D / (64 * 8);   // 16-byte output chunks per lane
  if constexpr (!RESIDUAL) {
    // the plain layer output needs no whole-row step: wavefront w of the token's workgroup takes
    // chunk w (four times the wavefronts in flight for the same loads and arithmetic)
    static_assert(NC == 4, "a token's four chunks on the four wavefronts of its workgroup");
    const int col = ((threadIdx.x >> 6) * 64 + lane) * 8;
    u32x4 v[K];
#pragma unroll
    for (int j = 0; j < K; ++j) v[j] = *reinterpret_cast<const u32x4*>(a.y + (size_t)pos[j] * D + col);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(p[j], f16_to_f32(static_cast<uint16_t>(v[j][i] & 0xFFFFu)), acc[2 * i]);
        acc[2 * i + 1] = fmaf(p[j], f16_to_f32(static_cast<uint16_t>(v[j][i] >> 16)), acc[2 * i + 1]);
      }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *reinterpret_cast<u32x4*>(a.out + (size_t)t * D + col) = o;
    return;
  }
  float acc[NC][8];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int col = (c * 64 + lane) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[c][i] = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(a.y + (size_t)pos[j] * D + col);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[c][2 * i] = fmaf(p[j], f16_to_f32(static_cast<uint16_t>(v[i] & 0xFFFFu)), acc[c][2 * i]);
        acc[c][2 * i + 1] = fmaf(p[j], f16_to_f32(static_cast<uint16_t>(v[i] >> 16)), acc[c][2 * i + 1]);
      }
    }
    if constexpr (!RESIDUAL) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[c][2 * i], acc[c][2 * i + 1]);
      *reinterpret_cast<u32x4*>(a.out + (size_t)t * D + col) = o;
    }
  }
  if constexpr (RESIDUAL) {
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float4* hp = reinterpret_cast<float4*>(a.h + (size_t)t * D + (c * 64 + lane) * 8);
      float4 u = hp[0], w = hp[1];
      u.x += acc[c][0]; u.y += acc[c][1]; u.z += acc[c][2]; u.w += acc[c][3];
      w.x += acc[c][4]; w.y += acc[c][5]; w.z += acc[c][6]; w.w += acc[c][7];
      hp[0] = u;
      hp[1] = w;
      acc[c][0] = u.x; acc[c][1] = u.y; acc[c][2] = u.z; acc[c][3] = u.w;
      acc[c][4] = w.x; acc[c][5] = w.y; acc[c][6] = w.z; acc[c][7] = w.w;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(acc[c][i], acc[c][i], ss);
    }
    if (a.x_next) {
      const float r = 1.0f / sqrtf(wave_sum(ss) / D + a.eps);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[c][2 * i] * r, acc[c][2 * i + 1] * r);
        *reinterpret_cast<u32x4*>(a.x_next + (size_t)t * D + (c * 64 + lane) * 8) = o;
      }
    }
  }
}

// one workgroup (256 threads x 8 values) per token
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h, float eps, int T,
                                                      bf16_t* __restrict__ xo) {
  __shared__ float part[4];
  const int t = blockIdx.x;
  const int c = threadIdx.x * 8;
  const float4 v0 = *reinterpret_cast<const float4*>(h + (size_t)t * D + c);
  const float4 v1 = *reinterpret_cast<const float4*>(h + (size_t)t * D + c + 4);
  float ss = v0.x * v0.x + v0.y * v0.y + v0.z * v0.z + v0.w * v0.w + v1.x * v1.x + v1.y * v1.y +
             v1.z * v1.z + v1.w * v1.w;
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float r = 1.0f / sqrtf(tot / D + eps);
  u32x4 o;
  o[0] = pack_bf16x2(v0.x * r, v0.y * r);
  o[1] = pack_bf16x2(v0.z * r, v0.w * r);
  o[2] = pack_bf16x2(v1.x * r, v1.y * r);
  o[3] = pack_bf16x2(v1.z * r, v1.w * r);
  *reinterpret_cast<u32x4*>(xo + (size_t)t * D + c) = o;
}

__global__ __launch_bounds__(256) void residual_add_kernel(float* __restrict__ h,
                                                           const bf16_t* __restrict__ y, long n8) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const u32x4 v = *reinterpret_cast<const u32x4*>(y + i * 8);
  float4* hp = reinterpret_cast<float4*>(h + i * 8);
  float4 a = hp[0], b = hp[1];
  a.x += __uint_as_float(v[0] << 16);
  a.y += __uint_as_float(v[0] & 0xFFFF0000u);
  a.z += __uint_as_float(v[1] << 16);
  a.w += __uint_as_float(v[1] & 0xFFFF0000u);
  b.x += __uint_as_float(v[2] << 16);
  b.y += __uint_as_float(v[2] & 0xFFFF0000u);
  b.z += __uint_as_float(v[3] << 16);
  b.w += __uint_as_float(v[3] & 0xFFFF0000u);
  hp[0] = a;
  hp[1] = b;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  if (a.h)
    hipLaunchKernelGGL(combine_kernel<true>, dim3((a.T + CMB_TOK_PER_WG - 1) / CMB_TOK_PER_WG), dim3(256), 0,
                       stream, a);
  else   // a workgroup per token
    hipLaunchKernelGGL(combine_kernel<false>, dim3(a.T), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* h, float eps, int T, uint16_t* x_out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, stream, h, eps, T, x_out);
  return hipGetLastError();
}

hipError_t launch_residual_add(float* h, const uint16_t* y, int T, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const long n8 = (long)T * D / 8;
  hipLaunchKernelGGL(residual_add_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, h,
                     y, n8);
  return hipGetLastError();
}

}  // namespace olmoe
