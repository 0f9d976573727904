// Expert-choice routing of the OLMoE MoE layer: the experts pick their tokens
// instead of the tokens picking experts.  "OLMoE: Open Mixture-of-Experts
// Language Models", section 4.1.4, sets this scheme against token choice (it
// trains faster per device but was not adopted); the page gives no formulas, so
// the layer takes its plainest reading, built from the token-choice layer's own
// steps ("OLMoE Guide: 64-Expert Fine-Grained Open MoE Architecture", items 1-3):
//
//   p[t,e]   = the same 64-way softmax of the router logits (fp32)
//   C        = ceil(8T / 64): the 8T (token, expert) pairs of token choice,
//              shared equally by the experts
//   S_e      = the C tokens with the largest p[t,e]; equal values go to the
//              lower token id
//   out[t]   = sum over the experts e with t in S_e (ascending e) of
//              p[t,e] * Expert_e(x_t)     (a token may have 0..64 experts)
//   aux      = 0.01 * 64 * sum_e f_e P_e with f_e = C / (8T), P_e = mean_t p[t,e]
//   z        = 0.001 * mean_t lse_t^2
//
// Kernels: softmax (probabilities stored per expert row, so that the selection
// reads one contiguous column), choose (one workgroup per expert: the exact C-th
// largest value found four bits at a time on the float bits, then a stable
// compaction in token order), the grouped GEMMs of the token-choice path on the
// 64 equal row blocks, and a combine that walks each token's experts in
// ascending order.
#include "common.hpp"
#include "kernels.hpp"
#include "routing.hpp"

namespace olmoe {

namespace {

constexpr int EC_SM_TOK = 16;       // tokens per softmax workgroup

// Softmax over the 64 experts of 16 tokens per workgroup, in the token-choice router's lane
// layout: wave w holds tokens 4w..4w+3, lane (r, j) = (lane / 16, lane % 16) the logits of
// token 4w + r for experts 4j..4j+3, reduced over the 16 lanes of a DPP row.  The logit is
// the fp64 sum of the router's per-slice (sum, compensation) pairs rounded once to fp32, and
// p = exp(l - max) * (1 / sum), as in the token-choice router.  The 16x64 tile then goes out
// transposed, 16 consecutive tokens of each expert's row of pT per workgroup.
template <int NS>
__global__ __launch_bounds__(256) void ec_softmax_kernel(EcArgs a) {
  __shared__ float tile[EC_SM_TOK][E + 1];
  __shared__ float lse2[EC_SM_TOK];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane >> 4, j = lane & 15;
  const int rt = w * 4 + r;
  const int t0 = blockIdx.x * EC_SM_TOK;
  const int t = t0 + rt;
  const bool valid = t < a.T;
  float v[4];
  if (valid) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kq = 0; kq < NS; ++kq) {
      const f32x4* src = reinterpret_cast<const f32x4*>(a.partial + ((size_t)kq * a.T + t) * E + j * 4);
      const f32x4 x0 = src[0], x1 = src[1];
      acc[0] += (double)x0[0] + (double)x0[1];
      acc[1] += (double)x0[2] + (double)x0[3];
      acc[2] += (double)x1[0] + (double)x1[1];
      acc[3] += (double)x1[2] + (double)x1[3];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (float)acc[i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = 0.f;
  }
  const float m = row16_max(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = expf(v[i] - m);
  const float sum = row16_sum((p[0] + p[1]) + (p[2] + p[3]));
  const float rs = 1.0f / sum;
  const float lse = m + logf(sum);
#pragma unroll
  for (int i = 0; i < 4; ++i) tile[rt][j * 4 + i] = valid ? p[i] * rs : 0.f;
  if (j == 0) lse2[rt] = valid ? lse * lse : 0.f;
  if (valid) {
    if (j == 0) a.lse[t] = lse;
    *reinterpret_cast<int4*>(a.inv_ec + (size_t)t * E + j * 4) = make_int4(-1, -1, -1, -1);
    if (a.p_all) *reinterpret_cast<f32x4*>(a.p_all + (size_t)t * E + j * 4) = f32x4{p[0] * rs, p[1] * rs, p[2] * rs, p[3] * rs};
  }
  __syncthreads();
  const int e = tid >> 2, q = tid & 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tt = q * 4 + i;
    if (t0 + tt < a.T) a.pT[(size_t)e * a.T + t0 + tt] = tile[tt][e];
  }
  // per-block sums for the losses, in token order
  if (tid < E) {
    float ps = 0.f;
#pragma unroll
    for (int tt = 0; tt < EC_SM_TOK; ++tt) ps += tile[tt][tid];
    a.blk_psum[blockIdx.x * E + tid] = ps;
  } else if (tid == E) {
    float l2 = 0.f;
#pragma unroll
    for (int tt = 0; tt < EC_SM_TOK; ++tt) l2 += lse2[tt];
    a.blk_lse2[blockIdx.x] = l2;
  }
}

// Workgroup barrier for data exchanged through LDS only: waits for this wave's LDS operations,
// not for its global stores in flight (which __syncthreads would also drain)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// wavefront totals by DPP within each row of 16 lanes, then the four rows' lanes 0
__device__ __forceinline__ int wave_total(int v) {
  v += row16_partner<0>(v);
  v += row16_partner<1>(v);
  v += row16_partner<2>(v);
  v += row16_partner<3>(v);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const uint32_t o = static_cast<uint32_t>(st == 0 ? row16_partner<0>(static_cast<int>(v))
                                             : st == 1 ? row16_partner<1>(static_cast<int>(v))
                                             : st == 2 ? row16_partner<2>(static_cast<int>(v))
                                                       : row16_partner<3>(static_cast<int>(v)));
    v = min(v, o);
  }
  return min(min(static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 0)), static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 16))),
             min(static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 32)), static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 48))));
}

// One workgroup per expert e, NT threads; thread i holds p[t,e] of its VPT consecutive tokens
// t = i * VPT + v as raw bits.  For p >= 0 the unsigned order of the bits is the order of the
// values, so the C-th largest value, kth = the largest key k with at least C keys >= k, is found
// exactly one bit at a time: the bits above the highest bit in which the column's smallest and
// largest keys differ are common to all keys, and the search stops as soon as exactly C keys
// are >= the bits found so far (then those C are the selection and no tie remains).
// Otherwise the tokens above kth are all taken and, of the tokens equal to it, the lowest ids
// fill the remaining places.  A workgroup scan of the per-thread (greater, equal) counts gives
// each thread the place of its first token; the place of token t is (#greater before t) +
// min(#equal before t, places left), so the chosen tokens land in ascending order.
//
// Workgroup 64, when launched, computes the losses from the softmax kernel's block sums
// (fixed order), alongside the selection.
template <int NT, int VPT>
__global__ __launch_bounds__(NT) void ec_choose_kernel(EcArgs a) {
  constexpr int NW = NT / 64;
  __shared__ int red[2][NW];
  __shared__ uint32_t mm[2][NW];
  __shared__ int2 scan_lds[NW];
  __shared__ double dsum[NW][E + 1];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int T = a.T, C = a.C;
  if (e == 0 && tid == 0 && a.clip) *a.clip = 0;   // counted by the GEMMs after this launch
  if (e == E) {   // losses: wave s sums part s of the blocks, lane x for expert x
    const int nblk = (T + EC_SM_TOK - 1) / EC_SM_TOK;
    const int per = (nblk + NW - 1) / NW;
    const int b0 = min(nblk, w * per), b1 = min(nblk, b0 + per);
    double ps = 0.0, l2 = 0.0;
    for (int b = b0; b < b1; ++b) {
      ps += (double)a.blk_psum[b * E + lane];
      l2 += (double)a.blk_lse2[b];
    }
    dsum[w][lane] = ps;
    if (lane == 0) dsum[w][E] = l2;
    __syncthreads();
    if (w == 0) {
      double pe = 0.0, lz = 0.0;
      for (int i = 0; i < NW; ++i) {
        pe += dsum[i][lane];
        lz += dsum[i][E];
      }
      // aux = alpha E sum_e f_e P_e with f_e = C / (8T) and P_e = (column sum) / T
      const double term = T > 0 ? pe * ((double)C / (8.0 * T) / T) : 0.0;
      __builtin_amdgcn_wave_barrier();
      dsum[0][lane] = term;   // every lane of wave 0 has read its column above
      __builtin_amdgcn_wave_barrier();
      if (lane == 0) {
        double aux = 0.0;
        for (int x = 0; x < E; ++x) aux += dsum[0][x];
        if (a.aux_loss) a.aux_loss[0] = (float)(LB_ALPHA * E * aux);
        if (a.z_loss) a.z_loss[0] = T > 0 ? (float)(Z_BETA * lz / T) : 0.f;
      }
    }
    return;
  }
  if (T == 0) {   // no rows: zero offsets and tile counts (the backward's weight gradients read them)
    if (e == 0 && tid <= E) {
      a.offsets[tid] = 0;
      a.tile_prefix_gu[tid] = 0;
      a.tile_prefix_dn[tid] = 0;
    }
    return;
  }
  const float* col = a.pT + (size_t)e * T;
  const int tbase = tid * VPT;

  uint32_t key[VPT];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int t = tbase + v;
    key[v] = t < T ? __float_as_uint(col[t]) : 0u;   // t >= T: key 0, never counted (candidates >= 1)
  }
#pragma unroll
  for (int v = 0; v < VPT; ++v)
    if (tbase + v < T) {
      kmin = min(kmin, key[v]);
      kmax = max(kmax, key[v]);
    }
  // the column's range (max as the complement's min)
  kmin = wave_min_u32(kmin);
  kmax = ~wave_min_u32(~kmax);
  if (lane == 0) {
    mm[0][w] = kmin;
    mm[1][w] = kmax;
  }
  lds_barrier();
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    kmin = min(kmin, mm[0][i]);
    kmax = max(kmax, mm[1][i]);
  }
  uint32_t kth = kmin;
  int cge = T;   // keys >= kth
  int slot = 0;
  if (kmin != kmax) {
    const int top = 31 - __builtin_clz(kmin ^ kmax);   // highest differing bit
    kth = kmin & ~((2u << top) - 1u);                  // the common bits above it
    for (int b = top; b >= 0; --b) {
      const uint32_t cand = kth | (1u << b);
      int c = 0;
#pragma unroll
      for (int v = 0; v < VPT; ++v) c += key[v] >= cand ? 1 : 0;
      c = wave_total(c);
      if (lane == 0) red[slot][w] = c;
      lds_barrier();
      int tot = 0;
#pragma unroll
      for (int i = 0; i < NW; ++i) tot += red[slot][i];
      slot ^= 1;
      if (tot >= C) {
        kth = cand;
        cge = tot;
      }
      if (cge == C) break;
    }
  }
  // selection: keys > lo, then keys == lo (lowest ids first) while places are left
  uint32_t lo;
  int need;
  if (cge == C && kth > 0) {
    lo = kth - 1;
    need = 0;
  } else {
    lo = kth;
    int c = 0;
#pragma unroll
    for (int v = 0; v < VPT; ++v) c += key[v] > kth ? 1 : 0;
    c = wave_total(c);
    if (lane == 0) red[slot][w] = c;
    lds_barrier();
    int n_gt = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) n_gt += red[slot][i];
    need = C - n_gt;
  }

  int lgt = 0, leq = 0;
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    lgt += key[v] > lo ? 1 : 0;
    leq += (tbase + v < T && key[v] == lo) ? 1 : 0;
  }
  const int igt = wave_inclusive_scan(lgt), ieq = wave_inclusive_scan(leq);
  if (lane == 63) scan_lds[w] = make_int2(igt, ieq);
  lds_barrier();
  int gt_before = igt - lgt, eq_before = ieq - leq;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int2 c = scan_lds[i];
    gt_before += i < w ? c.x : 0;
    eq_before += i < w ? c.y : 0;
  }
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int t = tbase + v;
    const bool gt = key[v] > lo;
    const bool eq = t < T && key[v] == lo;
    if (gt || (eq && eq_before < need)) {
      const int row = e * C + gt_before + min(eq_before, need);
      const float p = __uint_as_float(key[v]);
      a.perm[row] = t;
      a.row_w[row] = p;
      a.inv_ec[(size_t)t * E + e] = row;
      if (a.choice_tokens) a.choice_tokens[row] = t;
      if (a.choice_probs) a.choice_probs[row] = p;
    }
    gt_before += gt ? 1 : 0;
    eq_before += eq ? 1 : 0;
  }

  // row blocks of C rows per expert: offsets, and the GEMM tile lists in near-equal parts
  // (multiples of 32 rows except the last) exactly as the token-choice tile lists
  if (e == 0 && tid <= E) a.offsets[tid] = tid * C;
  const int ngu = (C + a.bm_gu - 1) / a.bm_gu, ndn = (C + a.bm_dn - 1) / a.bm_dn;
  if (e == 0 && tid <= E) {
    a.tile_prefix_gu[tid] = tid * ngu;
    a.tile_prefix_dn[tid] = tid * ndn;
  }
  const int qgu = min(a.bm_gu, ((C + ngu - 1) / ngu + 31) & ~31);
  const int qdn = min(a.bm_dn, ((C + ndn - 1) / ndn + 31) & ~31);
  for (int i = tid; i < ngu; i += NT)
    a.tiles_gu[e * ngu + i] = make_int2(e * C + i * qgu, e | (min(qgu, C - i * qgu) << 8));
  for (int i = tid; i < ndn; i += NT)
    a.tiles_dn[e * ndn + i] = make_int2(e * C + i * qdn, e | (min(qdn, C - i * qdn) << 8));
}

// Per token: lane e of each wavefront holds the row of (t, e) or -1; the chosen experts are
// taken in ascending order, 8 rows per batch (a short batch repeats its first row with weight 0,
// which adds exactly nothing), each lane summing 8 columns in fp32.

__global__ __launch_bounds__(256) void ec_combine_kernel(EcArgs a) {
  // a workgroup per token, wavefront w on 512-column chunk w (four times the wavefronts in flight
  // of one wavefront per token, for the same loads and arithmetic)
  const int t = blockIdx.x;
  if (t >= a.T) return;
  const int lane = threadIdx.x & 63;
  const int chunk = threadIdx.x >> 6;
  static_assert(D / (64 * 8) == 4, "a token's four chunks on the four wavefronts of its workgroup");
  const int myrow = a.inv_ec[(size_t)t * E + lane];
  const float myw = myrow >= 0 ? a.row_w[myrow] : 0.f;
  uint64_t mask = __ballot(myrow >= 0);
  if (a.token_counts && chunk == 0 && lane == 0) a.token_counts[t] = __popcll(mask);
  const int col = (chunk * 64 + lane) * 8;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  while (mask) {
    int pos[8];
    float wt[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ej = mask ? __builtin_ctzll(mask) : -1;
      mask &= mask - 1;
      pos[j] = ej >= 0 ? __shfl(myrow, ej) : pos[0];
      wt[j] = ej >= 0 ? __shfl(myw, ej) : 0.f;
    }
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = *reinterpret_cast<const u32x4*>(a.y + (size_t)pos[j] * D + col);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wt[j], f16_to_f32(static_cast<uint16_t>(v[j][i] & 0xFFFFu)), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wt[j], f16_to_f32(static_cast<uint16_t>(v[j][i] >> 16)), acc[2 * i + 1]);
      }
  }
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
  *reinterpret_cast<u32x4*>(a.out + (size_t)t * D + col) = o;
}

}  // namespace

hipError_t launch_ec_softmax(const EcArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid((a.T + EC_SM_TOK - 1) / EC_SM_TOK);
  if (router_slices(a.T) == 16)
    hipLaunchKernelGGL(ec_softmax_kernel<16>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(ec_softmax_kernel<4>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_ec_choose(const EcArgs& a, hipStream_t stream) {
  const bool losses = a.aux_loss || a.z_loss;
  const dim3 grid(E + (losses ? 1 : 0));
  if (a.T <= 256)
    hipLaunchKernelGGL((ec_choose_kernel<256, 1>), grid, dim3(256), 0, stream, a);
  else if (a.T <= 256 * 4)
    hipLaunchKernelGGL((ec_choose_kernel<256, 4>), grid, dim3(256), 0, stream, a);
  else if (a.T <= 256 * 16)
    hipLaunchKernelGGL((ec_choose_kernel<256, 16>), grid, dim3(256), 0, stream, a);
  else if (a.T <= 256 * 64)
    hipLaunchKernelGGL((ec_choose_kernel<256, 64>), grid, dim3(256), 0, stream, a);
  else if (a.T <= 1024 * 64)   // keys partly spilled to scratch: the large-batch path is GEMM-bound
    hipLaunchKernelGGL((ec_choose_kernel<1024, 64>), grid, dim3(1024), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_ec_combine(const EcArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(ec_combine_kernel, dim3(a.T), dim3(256), 0, stream, a);
  return hipGetLastError();
}

static_assert(1024 * 64 == EC_MAX_TOKENS, "choose kernel covers every supported T");

}  // namespace olmoe
