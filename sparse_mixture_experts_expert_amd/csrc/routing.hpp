// Device-side building blocks of the routing stage shared by the routing
// kernels: the top-8 selection of one routing block, the dispatch scan and the
// stable permutation.  Sources of each step are cited at its function.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace olmoe {

// all-reduce over the 16 lanes of a DPP row: quad xor 1, quad xor 2, half-row
// mirror, row mirror (each step combines two disjoint groups, so after the 4
// steps every lane holds the combination of all 16)
template <int STEP>
__device__ __forceinline__ int row16_partner(int v) {
  constexpr int ctrl = STEP == 0 ? 0xB1 : STEP == 1 ? 0x4E : STEP == 2 ? 0x141 : 0x140;
  return __builtin_amdgcn_mov_dpp(v, ctrl, 0xF, 0xF, false);
}
template <int STEP>
__device__ __forceinline__ float row16_partner(float v) {
  return __int_as_float(row16_partner<STEP>(__float_as_int(v)));
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, row16_partner<0>(v));
  v = fmaxf(v, row16_partner<1>(v));
  v = fmaxf(v, row16_partner<2>(v));
  return fmaxf(v, row16_partner<3>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  // pairwise in a fixed pattern: identical on every lane of the row
  v += row16_partner<0>(v);
  v += row16_partner<1>(v);
  v += row16_partner<2>(v);
  return v + row16_partner<3>(v);
}
// (value, id) argmax: larger value wins, equal values -> lower id
template <int STEP>
__device__ __forceinline__ void argmax_step(float& bv, int& be) {
  const float ov = row16_partner<STEP>(bv);
  const int oe = row16_partner<STEP>(be);
  if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
}

struct SelectLds {
  uint8_t chosen[ROUTE_BLOCK][16];   // per token and 4-expert group: chosen bits
  float p[ROUTE_BLOCK][E + 1];       // softmax probabilities
  float lse2[ROUTE_BLOCK];
  uint8_t rank[ROUTE_BLOCK][E];      // rank of the token among the block's tokens of that expert
};

// Softmax over all 64 experts and top-8 of one 16-token routing block, by the
// 4 wavefronts of a workgroup ("OLMoE Guide: 64-Expert Fine-Grained Open MoE
// Architecture", item 1 of Router Mechanics; "Mixture-of-experts LLMs from
// scratch with OLMoE", section 2: softmax first, then the k largest, not
// renormalised).
//
// Router variants: experts outside `keep` get score -inf before the softmax
// (pruning, "... from scratch with OLMoE", section 5), and `renormalize`
// divides the 8 chosen weights by their sum (the renormalised router of that
// page's section 2).  The caller guarantees at least 8 kept experts.
//
// The logits are the fp64 sum of the NS k-slice (sum, compensation) pairs left
// by the partial kernel.  Wavefront w holds tokens 4w..4w+3; lane
// (r, j) = (lane / 16, lane % 16) holds token 4w + r's logits of experts
// 4j..4j+3, so each of the 8 selection rounds is a 4-element register argmax
// plus a 16-lane DPP all-reduce.  Ties: the lower expert id wins (ascending
// scan with strict > inside a lane, explicit id comparison across lanes).  The
// selection is made on the fp32 logits; probabilities are exp(l - max) / sum.
//
// Outputs per token: ids, probs and, per (token, slot), the rank of the token
// among the block's tokens of the same expert (for the stable dispatch); per
// block: expert counts, probability sums and the sum of lse^2 (fixed token
// order).  Called by all 256 threads of a workgroup (two barriers inside).
template <int NS>
__device__ __forceinline__ void select_block(const float2* __restrict__ partial, int T, int blk,
                                             SelectLds& L, int32_t* __restrict__ ids,
                                             float* __restrict__ probs, uint8_t* __restrict__ lrank,
                                             int32_t* __restrict__ blk_counts,
                                             float* __restrict__ blk_psum,
                                             float* __restrict__ blk_lse2, uint64_t keep,
                                             int renormalize, float* __restrict__ p_all = nullptr,
                                             float* __restrict__ lse_out = nullptr) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int r = lane >> 4, j = lane & 15;
  const int rt = w * 4 + r;                        // token within the block
  const int t = blk * ROUTE_BLOCK + rt;
  const bool valid = t < T;

  float v[4], p[4];
  if (valid) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kq = 0; kq < NS; ++kq) {
      const f32x4* src = reinterpret_cast<const f32x4*>(partial + ((size_t)kq * T + t) * E + j * 4);
      const f32x4 a = src[0], b = src[1];
      acc[0] += (double)a[0] + (double)a[1];
      acc[1] += (double)a[2] + (double)a[3];
      acc[2] += (double)b[0] + (double)b[1];
      acc[3] += (double)b[2] + (double)b[3];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (keep >> (j * 4 + i)) & 1u ? (float)acc[i] : -INFINITY;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = 0.f;
  }
  const float m = row16_max(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = expf(v[i] - m);   // v - m is exact (Sterbenz) near the top
  const float sum = row16_sum((p[0] + p[1]) + (p[2] + p[3]));
  const float lse = m + logf(sum);
  const float rs = 1.0f / sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] *= rs;

  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = v[i] != v[i] ? -INFINITY : v[i];   // NaN ranks last
  uint32_t taken = 0;
  int my_slot[4] = {-1, -1, -1, -1};
#pragma unroll
  for (int s = 0; s < K; ++s) {
    float bv = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (!((taken >> i) & 1u) && (bi < 0 || c[i] > bv)) { bv = c[i]; bi = i; }
    int be = bi < 0 ? 1 << 30 : j * 4 + bi;   // a lane with nothing left never wins
    if (bi < 0) bv = -INFINITY;
    argmax_step<0>(bv, be);
    argmax_step<1>(bv, be);
    argmax_step<2>(bv, be);
    argmax_step<3>(bv, be);
    if ((be >> 2) == j) {
      const int i = be & 3;
      taken |= 1u << i;
      my_slot[0] = i == 0 ? s : my_slot[0];
      my_slot[1] = i == 1 ? s : my_slot[1];
      my_slot[2] = i == 2 ? s : my_slot[2];
      my_slot[3] = i == 3 ? s : my_slot[3];
      if (valid) ids[t * K + s] = be;
    }
  }
  // weights of the chosen experts, optionally divided by their sum (fixed DPP order)
  float wsc = 1.0f;
  if (renormalize) {
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) q += (taken >> i) & 1u ? p[i] : 0.f;
    wsc = 1.0f / row16_sum(q);
  }
  if (valid) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (my_slot[i] >= 0) probs[t * K + my_slot[i]] = renormalize ? p[i] * wsc : p[i];
  }
  if (valid && p_all) *reinterpret_cast<f32x4*>(p_all + (size_t)t * E + j * 4) = f32x4{p[0], p[1], p[2], p[3]};
  if (valid && lse_out && j == 0) lse_out[t] = lse;
  L.chosen[rt][j] = valid ? static_cast<uint8_t>(taken) : 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) L.p[rt][j * 4 + i] = valid ? p[i] : 0.f;
  if (j == 0) L.lse2[rt] = valid ? lse * lse : 0.f;
  __syncthreads();
  // wavefront 0, lane e: ranks, count and probability sum of expert e, in token order
  if (w == 0) {
    int cnt = 0;
    float psum = 0.f, l2 = 0.f;
#pragma unroll
    for (int rr = 0; rr < ROUTE_BLOCK; ++rr) {
      L.rank[rr][lane] = static_cast<uint8_t>(cnt);
      cnt += (L.chosen[rr][lane >> 2] >> (lane & 3)) & 1;
      psum += L.p[rr][lane];
      l2 += L.lse2[rr];
    }
    if (blk * ROUTE_BLOCK < T) {
      blk_counts[blk * E + lane] = cnt;
      blk_psum[blk * E + lane] = psum;
      if (lane == 0) blk_lse2[blk] = l2;
    }
  }
  __syncthreads();
  if (valid) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (my_slot[i] >= 0) lrank[t * K + my_slot[i]] = L.rank[rt][j * 4 + i];
  }
}

constexpr int SCAN_SUB = 16;  // threads per expert in the scan

struct ScanLds {
  int sc[SCAN_SUB][E];
  double sp[SCAN_SUB][E];
  double sl2[16];
  int soff[E + 1];
  int tgu[E + 1], tdn[E + 1];   // row-tile prefixes
};

// write the row-tile list of one GEMM: tile t of expert e (tp[e] <= t < tp[e+1]) covers
// rows off[e] + (t - tp[e]) * q .. of that expert, q <= bm as below
__device__ __forceinline__ void fill_tiles(const int* tp, const int* off, int bm, int2* tiles) {
  const int n = tp[E];
  for (int t = threadIdx.x; t < n; t += blockDim.x) {
    int lo = 0, hi = E;
    while (hi - lo > 1) {   // last expert whose first tile is <= t (LDS only)
      const int mid = (lo + hi) >> 1;
      if (tp[mid] <= t) lo = mid; else hi = mid;
    }
    // the expert's c rows go to its ceil(c/bm) tiles in near-equal parts, each a multiple of
    // 32 rows (one MFMA fragment) except the last, so no tile is mostly padding
    const int c = off[lo + 1] - off[lo];
    const int n = tp[lo + 1] - tp[lo];
    const int q = min(bm, ((c + n - 1) / n + 31) & ~31);
    const int row0 = off[lo] + (t - tp[lo]) * q;
    const int rows = min(q, off[lo + 1] - row0);
    tiles[t] = make_int2(row0, lo | (rows << 8));
  }
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
  return v;
}

// Dispatch scan by 1024 threads: per-expert counts and their exclusive prefix
// (offsets), the first output row of every (routing block, expert) pair in
// block order, the row-tile lists of the grouped GEMMs, and the
// Switch load-balancing loss 0.01 * 64 * sum_e f_e P_e and router z-loss
// 0.001 * mean lse^2 ("OLMoE Guide", items 2 and 3).  Every sum runs in a
// fixed order, so the results are reproducible bit for bit.
__device__ __forceinline__ void scan_block(const ScanArgs& a, ScanLds& L) {
  const int tid = threadIdx.x;
  if (tid == 0 && a.clip) *a.clip = 0;   // the GEMMs after this launch count their clipped values
  const int e = tid & 63;
  const int s = tid >> 6;
  const int nblk = (a.T + ROUTE_BLOCK - 1) / ROUTE_BLOCK;
  const int per = (nblk + SCAN_SUB - 1) / SCAN_SUB;
  const int b0 = min(nblk, s * per), b1 = min(nblk, b0 + per);

  int c = 0;
  double ps = 0.0;
  // unrolled so that several blocks' loads are in flight before the first add (same order)
#pragma unroll 8
  for (int b = b0; b < b1; ++b) {
    c += a.blk_counts[b * E + e];
    ps += static_cast<double>(a.blk_psum[b * E + e]);
  }
  L.sc[s][e] = c;
  L.sp[s][e] = ps;
  double l2 = 0.0;
  for (int b = tid; b < nblk; b += 1024) l2 += static_cast<double>(a.blk_lse2[b]);
  l2 = wave_sum_f64(l2);
  if (e == 0) L.sl2[s] = l2;
  __syncthreads();

  if (tid < 64) {
    int run = 0;
    double P = 0.0;
    for (int q = 0; q < SCAN_SUB; ++q) {
      const int tmp = L.sc[q][e];
      L.sc[q][e] = run;
      run += tmp;
      P += L.sp[q][e];
    }
    const int total = run;
    const int incl = wave_inclusive_scan(total);
    L.soff[e] = incl - total;
    a.offsets[e] = incl - total;
    if (e == 63) {
      L.soff[E] = incl;
      a.offsets[E] = incl;
    }
    if (a.expert_counts) a.expert_counts[e] = total;

    const int tg = (total + a.bm_gu - 1) / a.bm_gu;
    const int ig = wave_inclusive_scan(tg);
    a.tile_prefix_gu[e] = ig - tg;
    L.tgu[e] = ig - tg;
    if (e == 63) a.tile_prefix_gu[E] = L.tgu[E] = ig;
    const int td = (total + a.bm_dn - 1) / a.bm_dn;
    const int id = wave_inclusive_scan(td);
    a.tile_prefix_dn[e] = id - td;
    L.tdn[e] = id - td;
    if (e == 63) a.tile_prefix_dn[E] = L.tdn[E] = id;

    const double f = a.T > 0 ? total / (8.0 * a.T) : 0.0;
    const double Pm = a.T > 0 ? P / a.T : 0.0;
    const double fp = wave_sum_f64(f * Pm);
    if (e == 0) {
      double z = 0.0;
      for (int q = 0; q < 16; ++q) z += L.sl2[q];
      if (a.aux_loss) a.aux_loss[0] = static_cast<float>(LB_ALPHA * E * fp);
      if (a.z_loss) a.z_loss[0] = a.T > 0 ? static_cast<float>(Z_BETA * z / a.T) : 0.f;
    }
  }
  __syncthreads();

  int base = L.soff[e] + L.sc[s][e];
#pragma unroll 8
  for (int b = b0; b < b1; ++b) {
    a.blk_base[b * E + e] = base;
    base += a.blk_counts[b * E + e];
  }
  fill_tiles(L.tgu, L.soff, a.bm_gu, a.tiles_gu);
  fill_tiles(L.tdn, L.soff, a.bm_dn, a.tiles_dn);
}

// Stable permutation of the (token, slot) pairs into expert-contiguous rows
// ("Mixture-of-experts LLMs from scratch with OLMoE", section 2: a stable sort
// of the pairs by expert): row = first row of (block, expert) + rank in block.
__device__ __forceinline__ void permute_range(const PermuteArgs& a, int i0, int stride) {
  for (int i = i0; i < a.T * K; i += stride) {
    const int t = i / K;
    const int e = a.ids[i];
    const int pos = a.blk_base[(t / ROUTE_BLOCK) * E + e] + a.lrank[i];
    a.perm[pos] = t;
    a.inv[i] = pos;
    if (a.row_w) a.row_w[pos] = a.probs[i];
  }
}

}  // namespace olmoe
