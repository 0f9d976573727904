// Router of the OLMoE MoE layer: logits = x W_router^T (2048 -> 64), softmax over
// all 64 experts, top-8 ("OLMoE Guide: 64-Expert Fine-Grained Open MoE
// Architecture", item 1 of Router Mechanics; "Mixture-of-experts LLMs from
// scratch with OLMoE", section 2, softmax first then the k largest, no
// renormalisation).
//
// fp32 router on bf16 matrix cores: every fp32 weight w is split into three
// bf16 values hi + mid + lo == w exactly (8 + 8 + 8 significand bits cover
// fp32's 24), so x*w = x*hi + x*mid + x*lo with every product exact (x is
// bf16).  Three bf16 MFMAs per tile give the fp32 dot product at one eighth of
// the fp32-MFMA cost.  Summation error is kept far below the 1e-5 logit window
// inside which two routings count as equally correct: the hi products of each
// 64-wide k-chunk are summed into a fresh partial, and the partials are added
// to the running logit with Knuth's TwoSum, whose exact rounding error goes to
// a compensation term; the mid and lo products (2^-8 of the total and less)
// share one plain accumulator.  A plain fp32 accumulator over k = 2048 drifts
// by ~2e-5 on rows scaled by 8; this scheme stays near 2e-6.
//
// One wavefront owns 16 tokens (a routing block).  Lane e of the wavefront
// holds expert e's logit for one token at a time, so the softmax and the top-8
// are wavefront reductions over the 64 lanes; ties between equal logits go to
// the lowest lane, i.e. the lower expert id.  Lane e also counts how many of
// the block's tokens chose expert e, which gives each (token, slot) its rank
// inside the block for a stable dispatch.
#include "common.hpp"
#include "kernels.hpp"

namespace olmoe {

namespace {

constexpr int KC = 64;              // k-chunk of the router weights staged in LDS
constexpr int WSTRIDE = KC + 8;     // padded row (144 bytes): conflict-free 16-byte reads

__device__ __forceinline__ void split3(float w, bf16_t& hi, bf16_t& mid, bf16_t& lo) {
  hi = f32_to_bf16(w);
  const float r1 = w - bf16_to_f32(hi);
  mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);
  lo = f32_to_bf16(r2);
}

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void router_top8_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ wr, int T,
    int32_t* __restrict__ ids, float* __restrict__ probs, uint8_t* __restrict__ lrank,
    int32_t* __restrict__ blk_counts, float* __restrict__ blk_psum, float* __restrict__ blk_lse2) {
  constexpr int NT = WAVES * 64;
  constexpr int WCH = E * KC / 4 / NT;  // float4 chunks of a weight k-chunk per thread
  __shared__ __align__(16) bf16_t wsm[3][E * WSTRIDE];
  __shared__ float lsm[WAVES][ROUTE_BLOCK][E + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int blk = blockIdx.x * WAVES + w;   // routing block of this wavefront
  const int tok0 = blk * ROUTE_BLOCK;

  // A operand: lane holds token (lane % 16), k-group (lane / 16) of 8 values
  const int arow = tok0 + (lane & 15);
  const bool arow_ok = arow < T;
  const bf16_t* xrow = x + (size_t)(arow_ok ? arow : 0) * D + (lane >> 4) * 8;

  f32x4 acc_hi[4], acc_lm[4], tot[4], cmp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc_hi[i] = acc_lm[i] = tot[i] = cmp[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  float4 wreg[WCH];
  auto load_w = [&](int k0) {
#pragma unroll
    for (int q = 0; q < WCH; ++q) {
      const int c = tid + q * NT;
      const int row = c / (KC / 4), c4 = c % (KC / 4);
      wreg[q] = *reinterpret_cast<const float4*>(wr + (size_t)row * D + k0 + c4 * 4);
    }
  };
  auto store_w = [&]() {
#pragma unroll
    for (int q = 0; q < WCH; ++q) {
      const int c = tid + q * NT;
      const int row = c / (KC / 4), c4 = c % (KC / 4);
      const float v[4] = {wreg[q].x, wreg[q].y, wreg[q].z, wreg[q].w};
      bf16_t h[4], m[4], l[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) split3(v[i], h[i], m[i], l[i]);
      const int o = row * WSTRIDE + c4 * 4;
      *reinterpret_cast<uint2*>(&wsm[0][o]) = make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16));
      *reinterpret_cast<uint2*>(&wsm[1][o]) = make_uint2(m[0] | (uint32_t(m[1]) << 16), m[2] | (uint32_t(m[3]) << 16));
      *reinterpret_cast<uint2*>(&wsm[2][o]) = make_uint2(l[0] | (uint32_t(l[1]) << 16), l[2] | (uint32_t(l[3]) << 16));
    }
  };

  load_w(0);
  for (int k0 = 0; k0 < D; k0 += KC) {
    // this wavefront's x fragments for the chunk (two k-steps of 32)
    bf16x8 a[KC / 32];
#pragma unroll
    for (int s = 0; s < KC / 32; ++s) {
      if (arow_ok) {
        a[s] = *reinterpret_cast<const bf16x8*>(xrow + k0 + s * 32);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) a[s][i] = (__bf16)0.0f;
      }
    }
    __syncthreads();          // previous chunk fully consumed
    store_w();
    __syncthreads();
    if (k0 + KC < D) load_w(k0 + KC);   // in flight during the MFMAs
#pragma unroll
    for (int s = 0; s < KC / 32; ++s) {
#pragma unroll
      for (int eb = 0; eb < 4; ++eb) {
        const int o = (eb * 16 + (lane & 15)) * WSTRIDE + s * 32 + (lane >> 4) * 8;
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&wsm[0][o]);
        const bf16x8 bm = *reinterpret_cast<const bf16x8*>(&wsm[1][o]);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&wsm[2][o]);
        acc_lm[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], bl, acc_lm[eb], 0, 0, 0);
        acc_lm[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], bm, acc_lm[eb], 0, 0, 0);
        acc_hi[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], bh, acc_hi[eb], 0, 0, 0);
      }
    }
    // tot + cmp += chunk partial, with the rounding error of the add kept exactly (TwoSum)
#pragma unroll
    for (int eb = 0; eb < 4; ++eb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s0 = tot[eb][i], p = acc_hi[eb][i];
        const float t = s0 + p;
        const float bp = t - s0;
        const float err = (s0 - (t - bp)) + (p - bp);
        tot[eb][i] = t;
        cmp[eb][i] += err;
      }
      acc_hi[eb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // logit of token (lane/16)*4+i, expert eb*16 + lane%16
#pragma unroll
  for (int eb = 0; eb < 4; ++eb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lsm[w][(lane >> 4) * 4 + i][eb * 16 + (lane & 15)] = tot[eb][i] + (cmp[eb][i] + acc_lm[eb][i]);
  __syncthreads();

  if (tok0 >= T) return;
  int cnt = 0;          // tokens of this block that chose expert `lane` so far
  float psum = 0.f;     // sum of expert `lane`'s probabilities over the block
  float lse2 = 0.f;     // sum of lse^2 over the block
  const int ntok = min(ROUTE_BLOCK, T - tok0);
  for (int r = 0; r < ntok; ++r) {
    const int t = tok0 + r;
    const float v = lsm[w][r][lane];
    const float m = wave_max(v);
    const float ex = expf(v - m);          // v - m is exact (Sterbenz) near the top
    const float s = wave_sum(ex);
    const float lse = m + logf(s);
    const float p = ex / s;
    psum += p;
    lse2 += lse * lse;
    float cand = v;
    bool taken = false;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float mx = wave_max(taken ? -INFINITY : cand);
      uint64_t hit = __ballot(!taken && cand == mx);
      if (hit == 0) hit = __ballot(!taken);   // only NaN logits left: lowest free expert
      const int win = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      if (lane == win) {
        ids[t * K + j] = lane;
        probs[t * K + j] = p;
        lrank[t * K + j] = static_cast<uint8_t>(cnt);
        ++cnt;
        taken = true;
      }
    }
  }
  blk_counts[blk * E + lane] = cnt;
  blk_psum[blk * E + lane] = psum;
  if (lane == 0) blk_lse2[blk] = lse2;
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, hipStream_t stream) {
  const int nblk = (a.T + ROUTE_BLOCK - 1) / ROUTE_BLOCK;
  if (a.T > 1024) {
    const int grid = (nblk + 3) / 4;
    hipLaunchKernelGGL(router_top8_kernel<4>, dim3(grid), dim3(256), 0, stream, a.x, a.wr, a.T,
                       a.ids, a.probs, a.lrank, a.blk_counts, a.blk_psum, a.blk_lse2);
  } else {
    hipLaunchKernelGGL(router_top8_kernel<1>, dim3(nblk), dim3(64), 0, stream, a.x, a.wr, a.T,
                       a.ids, a.probs, a.lrank, a.blk_counts, a.blk_psum, a.blk_lse2);
  }
  return hipGetLastError();
}

}  // namespace olmoe
