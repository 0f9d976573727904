// Host-side launchers of the OLMoE MoE kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace olmoe {

struct RouterArgs {
  const uint16_t* x;      // bf16 [T,2048]
  const float* wr;        // fp32 [64,2048]
  int T;
  float2* partial;        // [S,T,64] per-k-slice (sum, compensation) of the logits (scratch)
  uint16_t* planes;       // bf16 [3,64,2048] exact split of wr in fragment order (scratch, T > 2048)
};
// router logits in router_slices(T) k-slice partials
constexpr int ROUTER_F32_TOKENS = 2048;   // up to here the fp32-MFMA router path
constexpr int router_slices(int T) { return T <= ROUTER_F32_TOKENS ? 16 : 4; }
hipError_t launch_router_partial(const RouterArgs& a, hipStream_t stream);

struct SelectArgs {
  const float2* partial;
  int T;
  int32_t* ids;           // [T,8]
  float* probs;           // [T,8]
  uint8_t* lrank;         // [T,8] rank of the token among its routing block's tokens of that expert
  int32_t* blk_counts;    // [nblk,64]
  float* blk_psum;        // [nblk,64]
  float* blk_lse2;        // [nblk]
  uint64_t keep;          // bit e set: expert e may be chosen (at least 8 bits set)
  int renormalize;        // nonzero: route_probs divided by their sum over the 8 slots
};
// softmax + top-8 per routing block (one launch, one workgroup per block)
hipError_t launch_router_select(const SelectArgs& a, hipStream_t stream);

constexpr int SMALL_TOKENS = 2048;   // up to here scan and permutation share one launch

struct ScanArgs {
  int T;
  const int32_t* blk_counts;
  const float* blk_psum;
  const float* blk_lse2;
  int32_t* blk_base;        // [nblk,64] first row of each (block, expert)
  int32_t* offsets;         // [65]
  int32_t* tile_prefix_gu;  // [65] prefix of gate/up row tiles per expert
  int2* tiles_gu;           // per gate/up row tile: (first row, expert | rows << 8)
  int bm_gu;
  int32_t* tile_prefix_dn;  // [65] prefix of down row tiles per expert
  int2* tiles_dn;
  int bm_dn;
  int32_t* expert_counts;   // [64] or null
  float* aux_loss;          // [1] or null
  float* z_loss;            // [1] or null
};
hipError_t launch_scan(const ScanArgs& a, hipStream_t stream);

struct PermuteArgs {
  int T;
  const int32_t* ids;
  const uint8_t* lrank;
  const int32_t* blk_base;
  int32_t* perm;            // [8T]
  int32_t* inv;             // [T,8]
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream);
// scan + permutation in one workgroup, for T <= SMALL_TOKENS
hipError_t launch_scan_permute(const ScanArgs& sa, const PermuteArgs& pa, hipStream_t stream);

// Grouped GEMM tile shapes, chosen from T (rows per expert ~ T/8).
struct GemmPlan {
  int bm_gu, bm_dn;         // row-tile heights of gate/up and down
  int variant;              // which compiled tile set
};
GemmPlan plan_gemm(int T);
int max_row_tiles(int T, int bm);
constexpr int MIN_TILE_ROWS = 32;   // smallest row tile of any plan (sizes the tile lists)
constexpr int LARGE_TOKENS = 2048;  // above this the grouped GEMMs use 256-row tiles

struct GemmArgs {
  int T;
  const uint16_t* x;        // bf16 [T,2048] (gate/up source)
  const uint16_t* w_gate;   // bf16 [64,1024,2048]
  const uint16_t* w_up;
  const uint16_t* w_down;   // bf16 [64,2048,1024]
  const int32_t* perm;
  const int32_t* offsets;
  const int32_t* tile_prefix_gu;   // [64] holds the tile count
  const int32_t* tile_prefix_dn;
  const int2* tiles_gu;
  const int2* tiles_dn;
  uint16_t* h;              // fp16 [8T,1024] SwiGLU activations, expert-contiguous rows
  uint16_t* y;              // fp16 [8T,2048] expert outputs, expert-contiguous rows
};
hipError_t launch_gateup(const GemmArgs& a, const GemmPlan& p, hipStream_t stream);
hipError_t launch_down(const GemmArgs& a, const GemmPlan& p, hipStream_t stream);

struct CombineArgs {
  int T;
  const uint16_t* y;
  const int32_t* inv;
  const float* probs;
  uint16_t* out;            // bf16 [T,2048]; unused when h is set
  float* h;                 // fp32 [T,2048] residual: h += layer output (fused residual epilogue)
  uint16_t* x_next;         // bf16 [T,2048] RMSNorm(h) after the update, or null
  float eps;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

hipError_t launch_rmsnorm(const float* h, float eps, int T, uint16_t* x_out, hipStream_t stream);
hipError_t launch_residual_add(float* h, const uint16_t* y, int T, hipStream_t stream);

}  // namespace olmoe
