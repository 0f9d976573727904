// Host-side launchers of the OLMoE MoE kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

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
  float* p_all = nullptr; // [T,64] all 64 probabilities, or null (backward pass)
  float* lse = nullptr;   // [T] log-sum-exp of the logits, or null (backward pass)
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
  int32_t* clip = nullptr;  // [1] count of clipped fp16 intermediates: zeroed here, before the GEMMs
};
hipError_t launch_scan(const ScanArgs& a, hipStream_t stream);

struct PermuteArgs {
  int T;
  const int32_t* ids;
  const uint8_t* lrank;
  const int32_t* blk_base;
  int32_t* perm;            // [8T]
  int32_t* inv;             // [T,8]
  const float* probs = nullptr;   // [T,8] routing weights, read when row_w is set
  float* row_w = nullptr;         // [8T] routing weight of each row, or null (backward pass)
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
  float* gu = nullptr;      // gate/up: also store fp32 G and U [8T, 2048] (backward recompute), or null
  int32_t* clip = nullptr;  // [1] += values of H and Y outside fp16's range (or NaN), stored clipped
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

// ---------------------------------------------------------------- expert choice

constexpr int EC_MAX_TOKENS = static_cast<int>(OLMOE_EC_MAX_TOKENS);
constexpr int ec_capacity(int T) { return (K * T + E - 1) / E; }   // ceil(8T / 64) tokens per expert

struct EcArgs {
  int T, C;
  const float2* partial;      // [S,T,64] router partials
  float* pT;                  // fp32 [64,T] probabilities, one row per expert
  float* lse;                 // fp32 [T]
  int32_t* inv_ec;            // [T,64] row holding (t, e), or -1
  int32_t* perm;              // [64C] token of each row (expert e owns rows e*C .. e*C+C-1)
  float* row_w;               // [64C] routing weight p[t,e] of each row
  float* blk_psum;            // [ceil(T/16),64] sum of p[t,e] over each 16-token block (token order)
  float* blk_lse2;            // [ceil(T/16)] sum of lse^2 over each block
  int32_t* offsets;           // [65] e*C
  int32_t* tile_prefix_gu;    // [65]; entry 64 holds the tile count
  int2* tiles_gu;
  int bm_gu;
  int32_t* tile_prefix_dn;
  int2* tiles_dn;
  int bm_dn;
  int32_t* choice_tokens;     // [64,C] or null
  float* choice_probs;        // [64,C] or null
  const uint16_t* y;          // fp16 [64C,2048] expert outputs
  uint16_t* out;              // bf16 [T,2048]
  int32_t* token_counts;      // [T] or null
  float* aux_loss;            // [1] or null
  float* z_loss;              // [1] or null
  float* p_all = nullptr;     // fp32 [T,64] probabilities by token (backward pass), or null
  int32_t* clip = nullptr;    // [1] count of clipped fp16 intermediates: zeroed by the selection
};
hipError_t launch_ec_softmax(const EcArgs& a, hipStream_t stream);   // p (transposed), lse, inv_ec = -1
// top-C per expert and the tile lists (one workgroup per expert), aux and z (one more)
hipError_t launch_ec_choose(const EcArgs& a, hipStream_t stream);
hipError_t launch_ec_combine(const EcArgs& a, hipStream_t stream);   // weighted sum per token

// ---------------------------------------------------------------- backward pass

// dgrad: rows of one expert (tile list) x output columns, K = 2048
struct BwdDgradArgs {
  const uint16_t* a;          // bf16 rows of 2048 (K-inner)
  const int32_t* a_rows;      // row -> source row of a (gather), or null (row itself)
  const uint16_t* b0;         // weights read as [k][n]: rows k < kb_split from b0, the rest from b1
  const uint16_t* b1;
  int ldb;                    // elements per weight row
  long b_stride;              // elements per expert
  int kb_split;
  const int32_t* tile_count;  // row tiles (first row, expert | rows << 8)
  const int2* tiles;
  // epilogue: dH~ -> dG, dU (bf16 [rows, 2048]) and w*H (bf16 [rows, 1024]), or plain fp32 rows
  const float* row_w;
  const float* gu;            // fp32 [rows, 2048]: G | U of the forward
  uint16_t* dgu;
  uint16_t* hw;
  float* out_f32;             // fp32 [rows, 2048]
  // dH~ epilogue: per row, partial sums of <dH~, H> = <dout, Y> over the columns of one workgroup
  // ([bwd_dot_parts(T), rowdot_stride], row index in expert order)
  float* rowdot = nullptr;
  int rowdot_stride = 0;
};
int bwd_tile_rows(int T);   // row tile height of the dgrad kernels for T tokens (rows 8T)
int bwd_dot_parts(int T);   // partial sums per row of the dH~ epilogue's <dout, Y>
constexpr int BWD_MAX_DOT_PARTS = 16;
hipError_t launch_dgrad(const BwdDgradArgs& a, int T, bool dh, hipStream_t stream);

// wgrad: per expert, out[m][n] = sum over the expert's rows r of a[r][m] * b[r][n]
struct BwdWgradArgs {
  const uint16_t* a;          // bf16 [rows, lda], expert-contiguous (or gathered through a_rows)
  int lda;
  const uint16_t* b;          // bf16 [rows, ldb] (or gathered through b_rows)
  int ldb;
  const int32_t* offsets;     // [65]
  const uint16_t* zero;       // at least 256 zero bytes (rows past an expert's count)
  int m_total, n_total;       // output rows / columns per expert
  void* out0;                 // rows m < m_split
  void* out1;                 // rows m >= m_split (at m - m_split)
  int m_split;
  long out_stride;            // elements per expert in out0 / out1
  // row -> source row of a / b (expert order -> token), or null (row itself); at most one of the
  // two, and the table must stay readable 64 entries past its last row
  const int32_t* a_rows = nullptr;
  const int32_t* b_rows = nullptr;
  bool out_bf16 = false;      // out0 / out1 hold bf16 (the fp32 sums rounded to nearest even), else fp32
};
hipError_t launch_wgrad(const BwdWgradArgs& a, hipStream_t stream);

struct BwdSmallArgs {
  int T;
  const uint16_t* x;          // bf16 [T,2048]
  const float* w_router;      // fp32 [64,2048]
  const int32_t* ids;         // [T,8]
  const float* p_all;         // [T,64]
  const float* lse;           // [T]
  const int32_t* offsets;     // [65]
  const int32_t* perm;        // [8T]
  const int32_t* inv;         // [T,8]
  const float* rowdot;        // [dot_parts, rows] partial sums of <dout[t], Y row> (dH~ dgrad epilogue)
  float g_aux, g_z;
  float* dlogits;             // fp32 [T,64]
  const float* dxr;           // fp32 [8T,2048] per-row input gradients
  float* dx;                  // fp32 [T,2048]
  float* dwr_part;            // fp32 [nsplit,64,2048]
  float* dw_router;           // fp32 [64,2048]
  uint16_t* zero;             // 4 KiB
  int32_t* tp_bwd;            // [65] row-tile prefix of the dgrad tile list
  int2* tiles_bwd;
  const int32_t* inv_ec = nullptr;   // expert choice: [T,64] row of (t, e) or -1 (replaces ids / inv)
  int rows = 0;                      // rows in expert order (0: 8T)
  int dot_parts = 0;                 // partial sums per row in rowdot (1 .. BWD_MAX_DOT_PARTS)
};
int bwd_router_splits(int T);
hipError_t launch_bwd_prepare(const BwdSmallArgs& a, hipStream_t stream);   // zero row, dgrad tile list
hipError_t launch_bwd_router(const BwdSmallArgs& a, hipStream_t stream);    // dw and dlogits
hipError_t launch_bwd_finish(const BwdSmallArgs& a, hipStream_t stream);    // dW_router and dx

hipError_t launch_rmsnorm(const float* h, float eps, int T, uint16_t* x_out, hipStream_t stream);
hipError_t launch_residual_add(float* h, const uint16_t* y, int T, hipStream_t stream);

}  // namespace olmoe
