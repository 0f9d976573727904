// Router of the OLMoE MoE layer: logits = x W_router^T (2048 -> 64), the
// linear layer that scores all experts ("OLMoE Guide: 64-Expert Fine-Grained
// Open MoE Architecture", item 1 of Router Mechanics; "Mixture-of-experts LLMs
// from scratch with OLMoE", section 2), then softmax and top-8 (select_block in
// routing.hpp).
//
// The logits are produced in k-slice partials (16 slices up to 2048 tokens, 4
// above), each a (sum, compensation) pair whose fp64 sum the selection forms.
//
// Up to 2048 tokens: fp32 MFMA (16x16x4) straight from the fp32 router weights
// and the bf16 tokens.  One wavefront per (16 tokens, 16 experts, k-slice):
// a workgroup reads only an 8 KiB slice of W_router, so the router spreads over
// many CUs even for a handful of tokens (one workgroup pulling the whole router
// through one CU would be bound by that CU's load bandwidth).  Each lane loads
// 4 consecutive k of its row, and MFMA step s takes element s of every lane:
// the k-order inside a 16-k block is permuted identically for both operands,
// which leaves the dot product unchanged.
//
// Larger batches, where the router's MFMA work matters: bf16 matrix cores at
// one eighth of the fp32-MFMA cost.  Every fp32 weight w is split into three
// bf16 values hi + mid + lo == w exactly (8 + 8 + 8 significand bits cover
// fp32's 24), so x*w = x*hi + x*mid + x*lo with every product exact (x is
// bf16); the prep kernel writes the three planes once per call in MFMA
// fragment order (every wavefront load is one contiguous 1 KiB), and each
// wavefront reuses a weight fragment for 4 token sub-blocks.
//
// Both paths keep the summation error far below the 1e-5 logit window inside
// which two routings count as equally correct: each 64-wide k-chunk is summed
// into a fresh partial, and the partials are added to the running sum with
// Knuth's TwoSum, whose exact rounding error goes to a compensation term (the
// bf16 path sums the small mid and lo products in one plain accumulator).  A
// plain fp32 accumulator over k = 2048 drifts by ~2e-5 on rows scaled by 8;
// this scheme stays near 2e-6.
#include "common.hpp"
#include "kernels.hpp"
#include "routing.hpp"

namespace olmoe {

namespace {

constexpr int KQ = D / 4;        // k-range of one partial wavefront
constexpr int KSTEPS = D / 32;   // bf16 MFMA k-steps over a whole row

__device__ __forceinline__ void split3(float w, bf16_t& hi, bf16_t& mid, bf16_t& lo) {
  hi = f32_to_bf16(w);
  const float r1 = w - bf16_to_f32(hi);     // exact
  mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);   // exact, at most 8 significant bits
  lo = f32_to_bf16(r2);
}

// W_router fp32 [64,2048] -> planes[p][g][kstep][lane][8] with expert 16g + lane%16,
// k = 32*kstep + 8*(lane/16) + i: the B fragment of a 16x16x32 MFMA, one 16-byte
// chunk per lane
__global__ __launch_bounds__(256) void router_prep_kernel(const float* __restrict__ wr,
                                                          bf16_t* __restrict__ planes) {
  const int c = blockIdx.x * 256 + threadIdx.x;      // one 8-wide k chunk of one expert
  if (c >= E * D / 8) return;
  const int e = c / (D / 8), k = (c % (D / 8)) * 8;
  const float4 v0 = *reinterpret_cast<const float4*>(wr + e * D + k);
  const float4 v1 = *reinterpret_cast<const float4*>(wr + e * D + k + 4);
  const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  bf16_t h[8], m[8], l[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) split3(f[j], h[j], m[j], l[j]);
  const int g = e >> 4, lane = ((k & 31) >> 3) * 16 + (e & 15), ks = k >> 5;
  const size_t o = (((size_t)g * KSTEPS + ks) * 64 + lane) * 8;
  const size_t P = (size_t)E * D;
  u32x4 vh, vm, vl;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    vh[j] = h[2 * j] | (uint32_t(h[2 * j + 1]) << 16);
    vm[j] = m[2 * j] | (uint32_t(m[2 * j + 1]) << 16);
    vl[j] = l[2 * j] | (uint32_t(l[2 * j + 1]) << 16);
  }
  *reinterpret_cast<u32x4*>(planes + o) = vh;
  *reinterpret_cast<u32x4*>(planes + P + o) = vm;
  *reinterpret_cast<u32x4*>(planes + 2 * P + o) = vl;
}

__device__ __forceinline__ void twosum_into(f32x4& tot, f32x4& cmp, const f32x4& part) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float s0 = tot[i], p = part[i];
    const float t = s0 + p;
    const float b = t - s0;
    cmp[i] += (s0 - (t - b)) + (p - b);
    tot[i] = t;
  }
}

// fp32 path: partial[ks][t][e] for 16 tokens, 16 experts, one of KS k-slices.  Every load of
// the slice is issued before the first MFMA: with one wavefront per workgroup and a handful of
// workgroups per CU, a loop that waits on each load in turn is bound by memory latency.
template <int KS>
__global__ __launch_bounds__(64) void router_partial_f32_kernel(const bf16_t* __restrict__ x,
                                                                const float* __restrict__ wr, int T,
                                                                float2* __restrict__ partial) {
  constexpr int KW = D / KS;                 // k per slice
  constexpr int NB = KW / 16;                // 16-k blocks per slice
  static_assert(KW % 64 == 0, "TwoSum chunks of 64 k");
  const int lane = threadIdx.x;
  const int g = blockIdx.y & 3;              // expert group of 16
  const int ks = blockIdx.y >> 2;            // k-slice
  const int tok0 = blockIdx.x * 16;
  const int row = tok0 + (lane & 15);
  const bool aok = row < T;
  // lane (n, q) = (lane % 16, lane / 16) loads k = kb + 4q .. kb + 4q + 3 of its rows
  const float* bp = wr + (size_t)(g * 16 + (lane & 15)) * D + ks * KW + (lane >> 4) * 4;
  const bf16_t* ap = x + (size_t)(aok ? row : 0) * D + ks * KW + (lane >> 4) * 4;
  float4 b[NB];
  uint2 av[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    b[i] = *reinterpret_cast<const float4*>(bp + i * 16);
    av[i] = *reinterpret_cast<const uint2*>(ap + i * 16);
  }

  f32x4 part = {0.f, 0.f, 0.f, 0.f}, tot = part, cmp = part;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const uint2 a = aok ? av[i] : make_uint2(0u, 0u);
    part = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x << 16), b[i].x, part, 0, 0, 0);
    part = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x & 0xFFFF0000u), b[i].y, part, 0, 0, 0);
    part = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y << 16), b[i].z, part, 0, 0, 0);
    part = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y & 0xFFFF0000u), b[i].w, part, 0, 0, 0);
    if ((i & 3) == 3) {   // every 64 k: fold the chunk partial in with TwoSum
      twosum_into(tot, cmp, part);
      part = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // element i: token tok0 + (lane/16)*4 + i, expert 16g + lane%16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = tok0 + (lane >> 4) * 4 + i;
    if (t < T) partial[((size_t)ks * T + t) * E + g * 16 + (lane & 15)] = make_float2(tot[i], cmp[i]);
  }
}

// bf16x3 path: partial[kq][t][e] for TS x 16 tokens, 16 experts, one k-quarter
template <int TS>
__global__ __launch_bounds__(64) void router_partial_bf16x3_kernel(const bf16_t* __restrict__ x,
                                                                   const bf16_t* __restrict__ planes, int T,
                                                                   float2* __restrict__ partial) {
  const int lane = threadIdx.x;
  const int g = blockIdx.y & 3;              // expert group of 16
  const int kq = blockIdx.y >> 2;            // k-quarter
  const int tok0 = blockIdx.x * TS * 16;

  const bf16_t* bp = planes + (((size_t)g * KSTEPS + kq * (KQ / 32)) * 64 + lane) * 8;
  const bf16_t* ap[TS];
  bool aok[TS];
#pragma unroll
  for (int s = 0; s < TS; ++s) {
    const int row = tok0 + s * 16 + (lane & 15);
    aok[s] = row < T;
    ap[s] = x + (size_t)(aok[s] ? row : 0) * D + kq * KQ + (lane >> 4) * 8;
  }

  f32x4 acc_hi[TS], acc_lm[TS], tot[TS], cmp[TS];
#pragma unroll
  for (int s = 0; s < TS; ++s) acc_hi[s] = acc_lm[s] = tot[s] = cmp[s] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int ks = 0; ks < KQ / 32; ++ks) {
    const bf16x8 bh = *reinterpret_cast<const bf16x8*>(bp + ks * 512);
    const bf16x8 bm = *reinterpret_cast<const bf16x8*>(bp + (size_t)E * D + ks * 512);
    const bf16x8 bl = *reinterpret_cast<const bf16x8*>(bp + 2 * (size_t)E * D + ks * 512);
#pragma unroll
    for (int s = 0; s < TS; ++s) {
      bf16x8 a = *reinterpret_cast<const bf16x8*>(ap[s] + ks * 32);
      if (!aok[s]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = (__bf16)0.0f;
      }
      acc_lm[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc_lm[s], 0, 0, 0);
      acc_lm[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bm, acc_lm[s], 0, 0, 0);
      acc_hi[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc_hi[s], 0, 0, 0);
    }
    if (ks & 1) {   // every 64 k: fold the hi partial in with TwoSum
#pragma unroll
      for (int s = 0; s < TS; ++s) {
        twosum_into(tot[s], cmp[s], acc_hi[s]);
        acc_hi[s] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  // element i of sub-block s: token s*16 + (lane/16)*4 + i, expert 16g + lane%16
#pragma unroll
  for (int s = 0; s < TS; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = tok0 + s * 16 + (lane >> 4) * 4 + i;
      if (t < T)
        partial[((size_t)kq * T + t) * E + g * 16 + (lane & 15)] =
            make_float2(tot[s][i], cmp[s][i] + acc_lm[s][i]);
    }
}

template <int NS>
__global__ __launch_bounds__(256) void router_select_kernel(SelectArgs a) {
  __shared__ SelectLds L;
  select_block<NS>(a.partial, a.T, blockIdx.x, L, a.ids, a.probs, a.lrank, a.blk_counts, a.blk_psum,
                   a.blk_lse2, a.keep, a.renormalize, a.p_all, a.lse);
}

}  // namespace

hipError_t launch_router_partial(const RouterArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  if (a.T <= ROUTER_F32_TOKENS) {
    static_assert(router_slices(ROUTER_F32_TOKENS) == 16, "slices of the fp32 path");
    hipLaunchKernelGGL(router_partial_f32_kernel<16>, dim3((a.T + 15) / 16, 4 * 16), dim3(64), 0, stream, a.x,
                       a.wr, a.T, a.partial);
    return hipGetLastError();
  }
  static_assert(router_slices(ROUTER_F32_TOKENS + 1) == 4, "slices of the bf16x3 path");
  hipLaunchKernelGGL(router_prep_kernel, dim3(E * D / 8 / 256), dim3(256), 0, stream, a.wr, a.planes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int TS = 4;
  hipLaunchKernelGGL(router_partial_bf16x3_kernel<TS>, dim3((a.T + TS * 16 - 1) / (TS * 16), 16), dim3(64), 0,
                     stream, a.x, a.planes, a.T, a.partial);
  return hipGetLastError();
}

hipError_t launch_router_select(const SelectArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const int nblk = (a.T + ROUTE_BLOCK - 1) / ROUTE_BLOCK;
  if (router_slices(a.T) == 16)
    hipLaunchKernelGGL(router_select_kernel<16>, dim3(nblk), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(router_select_kernel<4>, dim3(nblk), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace olmoe
