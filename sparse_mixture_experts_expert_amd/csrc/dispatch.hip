// Dropless dispatch of the OLMoE MoE layer: per-expert counts, prefix sums and a
// stable permutation of the (token, slot) pairs into expert-contiguous rows
// ("Mixture-of-experts LLMs from scratch with OLMoE", section 2, grouped
// dispatch: stable sort of the pairs by expert, then count), plus the
// load-balancing loss and router z-loss ("OLMoE Guide: 64-Expert Fine-Grained
// Open MoE Architecture", items 2 and 3).
//
// The router kernel already left, per routing block of 16 tokens, the count of
// each expert and the rank of every (token, slot) inside its block.  The scan
// turns the [nblk,64] block counts into the first output row of every
// (block, expert) pair, in block order, so tokens stay ascending inside each
// expert: the same order as a stable sort.  All sums run in a fixed order
// (no atomics), so the tables and losses are reproducible bit for bit.
#include "common.hpp"
#include "kernels.hpp"

namespace olmoe {

namespace {

constexpr int SCAN_SUB = 16;  // threads per expert in the scan

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
  return v;
}

__global__ __launch_bounds__(1024) void scan_kernel(ScanArgs a) {
  __shared__ int sc[SCAN_SUB][E];
  __shared__ double sp[SCAN_SUB][E];
  __shared__ double sl2[1024 / 64];
  __shared__ int soff[E + 1];

  const int tid = threadIdx.x;
  const int e = tid & 63;
  const int s = tid >> 6;
  const int lane = e;
  const int nblk = (a.T + ROUTE_BLOCK - 1) / ROUTE_BLOCK;
  const int per = (nblk + SCAN_SUB - 1) / SCAN_SUB;
  const int b0 = min(nblk, s * per), b1 = min(nblk, b0 + per);

  int c = 0;
  double ps = 0.0;
  for (int b = b0; b < b1; ++b) {
    c += a.blk_counts[b * E + e];
    ps += static_cast<double>(a.blk_psum[b * E + e]);
  }
  sc[s][e] = c;
  sp[s][e] = ps;
  double l2 = 0.0;
  for (int b = tid; b < nblk; b += 1024) l2 += static_cast<double>(a.blk_lse2[b]);
  l2 = wave_sum_f64(l2);
  if (lane == 0) sl2[s] = l2;
  __syncthreads();

  if (tid < 64) {
    int run = 0;
    double P = 0.0;
    for (int q = 0; q < SCAN_SUB; ++q) {
      const int tmp = sc[q][e];
      sc[q][e] = run;
      run += tmp;
      P += sp[q][e];
    }
    const int total = run;
    const int incl = wave_inclusive_scan(total);
    soff[e] = incl - total;
    a.offsets[e] = incl - total;
    if (e == 63) {
      soff[E] = incl;
      a.offsets[E] = incl;
    }
    if (a.expert_counts) a.expert_counts[e] = total;

    const int tg = (total + a.bm_gu - 1) / a.bm_gu;
    const int ig = wave_inclusive_scan(tg);
    a.tile_prefix_gu[e] = ig - tg;
    if (e == 63) a.tile_prefix_gu[E] = ig;
    const int td = (total + a.bm_dn - 1) / a.bm_dn;
    const int id = wave_inclusive_scan(td);
    a.tile_prefix_dn[e] = id - td;
    if (e == 63) a.tile_prefix_dn[E] = id;

    // Switch load-balancing loss: alpha * E * sum_e f_e * P_e
    const double f = a.T > 0 ? total / (8.0 * a.T) : 0.0;
    const double Pm = a.T > 0 ? P / a.T : 0.0;
    const double fp = wave_sum_f64(f * Pm);
    if (e == 0) {
      double z = 0.0;
      for (int q = 0; q < 1024 / 64; ++q) z += sl2[q];
      if (a.aux_loss) a.aux_loss[0] = static_cast<float>(0.01 * E * fp);
      if (a.z_loss) a.z_loss[0] = a.T > 0 ? static_cast<float>(0.001 * z / a.T) : 0.f;
    }
  }
  __syncthreads();

  int base = soff[e] + sc[s][e];
  for (int b = b0; b < b1; ++b) {
    a.blk_base[b * E + e] = base;
    base += a.blk_counts[b * E + e];
  }
}

__global__ __launch_bounds__(256) void permute_kernel(PermuteArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.T * K) return;
  const int t = i / K;
  const int e = a.ids[i];
  const int pos = a.blk_base[(t / ROUTE_BLOCK) * E + e] + a.lrank[i];
  a.perm[pos] = t;
  a.inv[i] = pos;
}

}  // namespace

hipError_t launch_scan(const ScanArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const int n = a.T * K;
  hipLaunchKernelGGL(permute_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace olmoe
