// The non-GEMM steps of the backward pass of the OLMoE MoE layer (token choice, and the
// expert-choice form of the layer, whose routing weights are the same probabilities).
//
// With out[t] = sum_j w[t,j] Y[t,j] and w[t,j] = p[t, e_j] (the 64-way softmax
// probabilities, not renormalised: "Mixture-of-experts LLMs from scratch with
// OLMoE", section 2), the loss L = <dout, out> + g_aux * aux + g_z * z has
//   dL/dw[t,j]   = <dout[t], Y[t,j]> = <dout[t] W_down[e_j], H[t,j]>
//   dL/dp[t,e]   = dL/dw for the chosen e, plus g_aux * 0.01 * 64 * f_e / T from the
//                  load-balancing term (f_e, the routed share, is piecewise constant)
//   dL/dl[t,e]   = p (dL/dp - <p, dL/dp>)  +  g_z * 0.001 * 2 lse_t / T * p
// ("OLMoE Guide: 64-Expert Fine-Grained Open MoE Architecture", items 1-3), and
// through the router's linear layer dx += dl W_router, dW_router = dl^T x.
// Every sum runs in a fixed order (no atomics): results are reproducible.
#include "common.hpp"
#include "kernels.hpp"
#include "routing.hpp"

namespace olmoe {

namespace {

constexpr int WR_SPLIT_TOKENS = 32;    // tokens per load batch of the dW_router partial kernel
constexpr int WR_MAX_SPLITS = 32;      // dW_router partial sums at most (16: 80 + 6 us at 4096 tokens, 32: 48 + 10, 128: 46 + 33)

// the zero row and the dgrad row-tile list (the GEMMs read x and dout rows through perm)
__global__ __launch_bounds__(256) void bwd_prepare_kernel(BwdSmallArgs a, int bm) {
  const int tid = threadIdx.x;
  __shared__ int off[E + 1], tp[E + 1];
  reinterpret_cast<u32x4*>(a.zero)[tid] = u32x4{0u, 0u, 0u, 0u};   // 4 KiB
  if (tid <= E) off[tid] = a.offsets[tid];
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
      tp[e] = acc;
      acc += (off[e + 1] - off[e] + bm - 1) / bm;
    }
    tp[E] = acc;
  }
  __syncthreads();
  if (tid <= E) a.tp_bwd[tid] = tp[tid];
  fill_tiles(tp, off, bm, a.tiles_bwd);
}

// one wavefront per token: dL/dw for its 8 rows (expert choice: for the rows of the experts that
// took it, in ascending expert order), then dL/dlogits with lane = expert.  dL/dw of a row is
// <dout[t], Y row> = <dout[t] W_down, H row>, which the dH~ dgrad epilogue leaves as dot_parts
// partial sums per row: the expert outputs themselves are not needed.
template <bool EC>
__global__ __launch_bounds__(256) void bwd_router_kernel(BwdSmallArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int lane = threadIdx.x & 63;
  const size_t stride = a.rows ? a.rows : (size_t)K * a.T;
  // the sums for up to 8 rows (row < 0: none), the same on every lane: lane 8j+q adds parts
  // q, q+8 of row j, then the 8 lanes of a row add up in a fixed order
  auto dot_rows = [&](const int* rows, float* out) __attribute__((always_inline)) {
    const int jl = lane >> 3, q = lane & 7;
    int row = -1;
#pragma unroll
    for (int j = 0; j < K; ++j) row = j == jl ? rows[j] : row;
    float s = 0.f;
    if (row >= 0)
      for (int p = q; p < a.dot_parts; p += 8) s += a.rowdot[(size_t)p * stride + row];
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    s += __shfl_xor(s, 4, 64);
#pragma unroll
    for (int j = 0; j < K; ++j) out[j] = __shfl(s, j * 8, 64);
  };
  const float p = a.p_all[(size_t)t * E + lane];
  const float cnt = static_cast<float>(a.offsets[lane + 1] - a.offsets[lane]);
  const float Tf = static_cast<float>(a.T);
  float dp = a.g_aux * static_cast<float>(LB_ALPHA * E) * (cnt / (K * Tf)) / Tf;
  if constexpr (EC) {   // the experts that took the token, eight at a time in ascending order
    const int myrow = a.inv_ec[(size_t)t * E + lane];
    float dwl = 0.f;
    for (uint64_t m = __ballot(myrow >= 0); m;) {
      int rows[K], ej[K];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        ej[j] = m ? __builtin_ctzll(m) : -1;
        rows[j] = m ? __shfl(myrow, ej[j]) : -1;
        m &= m - 1;
      }
      float d[K];
      dot_rows(rows, d);
#pragma unroll
      for (int j = 0; j < K; ++j) dwl = lane == ej[j] ? d[j] : dwl;
    }
    dp += dwl;
  } else {
    int rows[K];
#pragma unroll
    for (int j = 0; j < K; ++j) rows[j] = a.inv[t * K + j];
    float dw[K];
    dot_rows(rows, dw);
#pragma unroll
    for (int j = 0; j < K; ++j) dp += a.ids[t * K + j] == lane ? dw[j] : 0.f;
  }
  const float s = wave_sum(p * dp);
  a.dlogits[(size_t)t * E + lane] =
      p * (dp - s) + a.g_z * static_cast<float>(Z_BETA) * 2.0f * a.lse[t] / Tf * p;
}

// dW_router partial sums, one per gridDim.y token range (whole batches of WR_SPLIT_TOKENS tokens,
// summed in token order): thread (2 columns, 16 experts).  A batch's dlogits go to LDS with one
// coalesced load per workgroup; the 16 experts are the same for the whole wavefront, so their
// values are broadcast reads.
constexpr int WR_COLS = 128;   // columns per workgroup (2 per thread)
__global__ __launch_bounds__(256) void bwd_wrouter_partial_kernel(BwdSmallArgs a) {
  __shared__ float sdl[WR_SPLIT_TOKENS][E];
  const int tid = threadIdx.x;
  const int col = blockIdx.x * WR_COLS + 2 * (tid & 63);
  const int e0 = __builtin_amdgcn_readfirstlane((tid >> 6) * 16);
  const int batches = (a.T + WR_SPLIT_TOKENS - 1) / WR_SPLIT_TOKENS;
  const int per = (batches + gridDim.y - 1) / gridDim.y * WR_SPLIT_TOKENS;   // tokens per range
  const int r0 = blockIdx.y * per;
  const int r1 = min(a.T, r0 + per);
  float acc0[16], acc1[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc0[i] = acc1[i] = 0.f;
  for (int t0 = r0; t0 < r1; t0 += WR_SPLIT_TOKENS) {
    const int nt = min(r1, t0 + WR_SPLIT_TOKENS) - t0;
    __syncthreads();   // the previous batch's dlogits are no longer read
    static_assert(WR_SPLIT_TOKENS * E == 256 * 8, "two float4 per thread");
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = (h * 256 + tid) * 4;   // float index in the batch: token i / 64, expert i % 64
      const int tk = i / E;
      *reinterpret_cast<f32x4*>(&sdl[tk][i % E]) =
          tk < nt ? *reinterpret_cast<const f32x4*>(a.dlogits + (size_t)(t0 + tk) * E + i % E) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    uint32_t xv[WR_SPLIT_TOKENS];
#pragma unroll
    for (int q = 0; q < WR_SPLIT_TOKENS; ++q)
      xv[q] = q < nt ? *reinterpret_cast<const uint32_t*>(a.x + (size_t)(t0 + q) * D + col) : 0u;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < WR_SPLIT_TOKENS; ++q) {
      if (q >= nt) break;   // tokens past the range are not added (sums in token order)
      const float x0 = __uint_as_float(xv[q] << 16), x1 = __uint_as_float(xv[q] & 0xFFFF0000u);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sdl[q][e0 + 4 * i4]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc0[4 * i4 + c] = fmaf(d4[c], x0, acc0[4 * i4 + c]);
          acc1[4 * i4 + c] = fmaf(d4[c], x1, acc1[4 * i4 + c]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float* o = a.dwr_part + ((size_t)blockIdx.y * E + e0 + i) * D + col;
    *reinterpret_cast<float2*>(o) = make_float2(acc0[i], acc1[i]);
  }
}

// dW_router: the partial sums added in range order (loads of eight ranges issued together)
__global__ __launch_bounds__(256) void bwd_wrouter_reduce_kernel(BwdSmallArgs a, int nsplit) {
  const int i = blockIdx.x * 256 + threadIdx.x;   // over 64 x 2048
  float s = 0.f;
  for (int sp0 = 0; sp0 < nsplit; sp0 += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = sp0 + k < nsplit ? a.dwr_part[(size_t)(sp0 + k) * E * D + i] : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (sp0 + k < nsplit) s += v[k];
  }
  a.dw_router[i] = s;
}

// dx for DX_TOK tokens and 256 columns per workgroup, one column per thread: dl W_router, then
// the token's 8 per-row input gradients in slot order (expert choice: the rows of the experts
// that took it, in ascending expert order)
constexpr int DX_TOK = 16;
template <bool EC>
__global__ __launch_bounds__(256) void bwd_dx_kernel(BwdSmallArgs a) {
  __shared__ float sdl[DX_TOK][E];
  __shared__ int srow[EC ? DX_TOK : 1][E];
  __shared__ int scnt[DX_TOK];
  const int t0 = blockIdx.x * DX_TOK;
  const int tid = threadIdx.x;
  for (int i = tid; i < DX_TOK * E; i += 256) {
    const int tk = i / E;
    sdl[tk][i % E] = t0 + tk < a.T ? a.dlogits[(size_t)(t0 + tk) * E + i % E] : 0.f;
  }
  if constexpr (EC) {   // wave w lists the rows of tokens w, w + 4, ... in ascending expert order
    const int lane = tid & 63;
    for (int tk = tid >> 6; tk < DX_TOK; tk += 4) {
      const int row = t0 + tk < a.T ? a.inv_ec[(size_t)(t0 + tk) * E + lane] : -1;
      const uint64_t m = __ballot(row >= 0);
      const int pos = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
      if (row >= 0) srow[tk][pos] = row;
      if (lane == 0) scnt[tk] = __popcll(m);
    }
  }
  const int col = blockIdx.y * 256 + tid;
  float wr[E];
#pragma unroll
  for (int e = 0; e < E; ++e) wr[e] = a.w_router[(size_t)e * D + col];
  __syncthreads();
  float acc[DX_TOK];
#pragma unroll
  for (int tk = 0; tk < DX_TOK; ++tk) acc[tk] = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e)
#pragma unroll
    for (int tk = 0; tk < DX_TOK; ++tk) acc[tk] = fmaf(sdl[tk][e], wr[e], acc[tk]);
#pragma unroll
  for (int tk = 0; tk < DX_TOK; ++tk) {
    const int t = t0 + tk;
    if (t >= a.T) break;
    if constexpr (EC) {   // a varying count of rows: loaded eight at a time, added in order
      const int n = scnt[tk];
      for (int j0 = 0; j0 < n; j0 += 8) {
        float r[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          r[jj] = j0 + jj < n ? a.dxr[(size_t)srow[tk][j0 + jj] * D + col] : 0.f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          if (j0 + jj < n) acc[tk] += r[jj];
      }
    } else {
      float r[K];
#pragma unroll
      for (int j = 0; j < K; ++j) r[j] = a.dxr[(size_t)a.inv[t * K + j] * D + col];
#pragma unroll
      for (int j = 0; j < K; ++j) acc[tk] += r[j];
    }
    a.dx[(size_t)t * D + col] = acc[tk];
  }
}

}  // namespace

int bwd_router_splits(int T) { return min(WR_MAX_SPLITS, (T + WR_SPLIT_TOKENS - 1) / WR_SPLIT_TOKENS); }

hipError_t launch_bwd_prepare(const BwdSmallArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_prepare_kernel, dim3(1), dim3(256), 0, stream, a,
                     bwd_tile_rows(a.rows ? a.rows / K : a.T));
  return hipGetLastError();
}

hipError_t launch_bwd_router(const BwdSmallArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  if (a.inv_ec)
    hipLaunchKernelGGL(bwd_router_kernel<true>, dim3((a.T + 3) / 4), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_router_kernel<false>, dim3((a.T + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_finish(const BwdSmallArgs& a, hipStream_t stream) {
  const int ns = bwd_router_splits(a.T);
  if (ns > 0) hipLaunchKernelGGL(bwd_wrouter_partial_kernel, dim3(D / WR_COLS, ns), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_wrouter_reduce_kernel, dim3(E * D / 256), dim3(256), 0, stream, a, ns);
  e = hipGetLastError();
  if (e != hipSuccess || a.T == 0) return e;
  const dim3 grid((a.T + DX_TOK - 1) / DX_TOK, D / 256);
  if (a.inv_ec)
    hipLaunchKernelGGL(bwd_dx_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_dx_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace olmoe
