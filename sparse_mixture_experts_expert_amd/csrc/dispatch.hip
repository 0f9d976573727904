// Dropless dispatch of the OLMoE MoE layer: per-expert counts, prefix sums and a
// stable permutation of the (token, slot) pairs into expert-contiguous rows
// ("Mixture-of-experts LLMs from scratch with OLMoE", section 2, grouped
// dispatch: stable sort of the pairs by expert, then count), plus the
// load-balancing loss and router z-loss ("OLMoE Guide: 64-Expert Fine-Grained
// Open MoE Architecture", items 2 and 3).
//
// The router's selection left, per routing block of 16 tokens, the count of
// each expert and the rank of every (token, slot) inside its block.  The scan
// turns the [nblk,64] block counts into the first output row of every
// (block, expert) pair, in block order, so tokens stay ascending inside each
// expert: the same order as a stable sort.  No atomics anywhere.
//
// Up to 2048 tokens the scan and the permutation share one workgroup and one
// launch: at such sizes a launch costs more than the work in it.
#include "common.hpp"
#include "kernels.hpp"
#include "routing.hpp"

namespace olmoe {

namespace {

__global__ __launch_bounds__(1024) void scan_kernel(ScanArgs a) {
  __shared__ ScanLds L;
  scan_block(a, L);
}

__global__ __launch_bounds__(256) void permute_kernel(PermuteArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.T * K) return;
  permute_range(a, i, a.T * K);
}

__global__ __launch_bounds__(1024) void scan_permute_kernel(ScanArgs sa, PermuteArgs pa) {
  __shared__ ScanLds scl;
  scan_block(sa, scl);
  __syncthreads();
  permute_range(pa, threadIdx.x, 1024);
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

hipError_t launch_scan_permute(const ScanArgs& sa, const PermuteArgs& pa, hipStream_t stream) {
  hipLaunchKernelGGL(scan_permute_kernel, dim3(1), dim3(1024), 0, stream, sa, pa);
  return hipGetLastError();
}

}  // namespace olmoe
