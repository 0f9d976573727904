// Grouped expert GEMMs of the OLMoE MoE layer on MFMA (gfx950).
//
// Each expert is a SwiGLU network, (SiLU(x W_gate^T) * (x W_up^T)) W_down^T,
// with gate/up [1024,2048] and down [2048,1024] ("OLMoE Guide: 64-Expert
// Fine-Grained Open MoE Architecture", item 1 and its SwiGLUExpert module;
// "Mixture-of-experts LLMs from scratch with OLMoE", section 2, where every
// expert runs once on the rows routed to it and production kernels put all
// the groups into one grouped matrix multiplication).
//
// Work unit: (row tile of one expert, column tile).  Row tiles of all experts
// are numbered in expert order; the scan leaves a list of (first row, expert,
// rows) per tile, so a workgroup learns its work with a single load: no host
// round trip, no per-expert launch, no dependent chain of loads at start.
// The 1-D grid is sized from the upper bound on the tile count (workgroups
// past the real count return at once) and remapped so that consecutive units
// run on the same XCD and share its L2; units are ordered expert by expert,
// column tile by column tile (see unit_of).
//
// gate/up: A = x rows gathered through perm (never materialised), B = the gate
// rows and the up rows of the same output columns, so one workgroup holds both
// accumulators and applies SiLU(g)*u in fp32 before the single store of H.
// down: A = H rows (already expert-contiguous), B = W_down[e].
//
// Operand staging: an S-stage ring of LDS tiles, BK k wide, filled by direct
// global->LDS 16-byte loads (each lane supplies its own address, so the row
// gather costs nothing extra), issued a slice per MFMA k-step.  A wavefront's load covers 1 KiB: 1024/(2 BK)
// rows x 2 BK contiguous bytes, whole cache lines per row.  The 16-byte chunks
// land with the low 3 bits of their index XOR-swizzled by row, so the MFMA
// fragment reads (8 rows x 16 bytes per group of lanes) hit distinct banks.  One barrier per k-step,
// after waiting only for the loads of the stage about to be used: S-1 stages
// stay in flight while the MFMAs run.
//
// The intermediates H and Y are stored as fp16 (round to nearest even): same
// bytes as bf16 but 3 more significand bits, which keeps their rounding well
// below the output's own bf16 rounding.  A value outside fp16's range (or NaN)
// is stored clipped to +-65504 and counted in the workspace's clip counter, so
// the caller learns of it.  The down GEMM therefore runs on f16 MFMA; W_down's
// bf16 values are converted to fp16 after the LDS read, scaled by 16 on the way
// (exact) and the products scaled back by 1/16 in fp32 (exact): every weight
// with 2^-18 <= |w| < 4096 converts exactly, smaller ones round toward zero
// with an absolute error under 2^-28, larger ones saturate.
constexpr float W_DOWN_SCALE = 16.0f;
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

#define GPTR(p) ((const __attribute__((address_space(1))) void*)(p))
#define LPTR(p) ((__attribute__((address_space(3))) void*)(p))

namespace olmoe {

namespace {

// XOR key of the 16-byte chunks of tile row `row`: with 8 chunks per row (BK = 64) the low 3
// bits of the row; with 4 (BK = 32) rows 4 apart, so 16 consecutive rows cover 256 bytes once
template <int BK>
__device__ __forceinline__ int swz_key(int row) { return BK >= 64 ? (row & 7) : ((row >> 2) & 3); }
// element offset of 16-byte chunk `ch` of tile row `row` (rows of BK elements)
template <int BK>
__device__ __forceinline__ int swz(int row, int ch) { return row * BK + ((ch ^ swz_key<BK>(row)) << 3); }

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// wait until at most N of this thread's vector-memory operations are in flight,
// then workgroup barrier; the memory clobber keeps LDS reads below it
template <int N>
__device__ __forceinline__ void vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Work-unit order: expert by expert; inside an expert, groups of up to UNIT_GROUP row tiles, and
// inside a group column tile by column tile with the group's row tiles adjacent.  The units that
// share a weight tile (one expert, one column tile) then run together, and those that share token
// rows (one row tile) a few units apart, so both are fetched into an XCD's L2 about once instead
// of once per unit (19% fewer L2 misses for the 4096-token gate/up GEMM); the groups keep an
// expert with many row tiles from spreading one row tile's units over its whole range.
// tile_count points at entry E of the per-expert prefix of row tiles; u < tile count * n_blocks.
// The expert lookup is one load per lane and a ballot.
constexpr int UNIT_GROUP = 4;
__device__ __forceinline__ void unit_of(const int32_t* tile_count, int n_blocks, int u, int& tile, int& nt) {
  const int32_t* tp = tile_count - E;
  const int lane = threadIdx.x & 63;
  const int tpl = tp[lane];                                       // first row tile of expert `lane`
  const int e = __popcll(__ballot(tpl * n_blocks <= u)) - 1;      // last expert starting at or before u
  const int t0 = __builtin_amdgcn_readfirstlane(__shfl(tpl, e));
  const int t1 = e < E - 1 ? __builtin_amdgcn_readfirstlane(__shfl(tpl, e + 1)) : *tile_count;
  const int nte = t1 - t0;                                        // >= 1: u lies in expert e's units
  const int local = u - t0 * n_blocks;
  const int grp = local / (UNIT_GROUP * n_blocks);
  const int rows = min(UNIT_GROUP, nte - grp * UNIT_GROUP);       // row tiles in this group
  const int w = local - grp * UNIT_GROUP * n_blocks;
  nt = w / rows;
  tile = t0 + grp * UNIT_GROUP + (w - nt * rows);
}

template <int BM_, int BN_, int WM_, int WN_, bool GATEUP_, int STAGES_, int BK_ = 64, int ROT_ = 1, bool NTW_ = false,
          bool SAVE_GU_ = false>
struct Cfg {
  static constexpr bool SAVE_GU = SAVE_GU_;   // gate/up: also store the fp32 pre-activations G and U
  static constexpr int ROT = ROT_;   // rotate each work unit's starting k-step
  static constexpr bool NTW = NTW_;  // weight loads marked non-temporal (streamed once)
  static constexpr int BM = BM_;   // rows (tokens) per tile
  static constexpr int BN = BN_;   // output columns per tile
  static constexpr int BK = BK_;   // k per stage
  static constexpr int CPR = BK / 8;   // 16-byte chunks per tile row
  static constexpr int WM = WM_, WN = WN_;
  static constexpr bool GATEUP = GATEUP_;
  static constexpr int STAGES = STAGES_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int NW = WM * WN;
  static constexpr int G = GATEUP ? 2 : 1;        // accumulator sets (gate, up)
  using V = typename std::conditional<GATEUP, bf16x8, f16x8>::type;   // MFMA operand type
  static constexpr int NB = G * BN;               // B rows per tile
  static constexpr int ROWS = BM + NB;            // LDS rows per stage
  static constexpr int KD = GATEUP ? D : F;       // reduction length
  static constexpr int ND = GATEUP ? F : D;       // output row length
  static constexpr int KT = KD / BK;
  static constexpr int FM = BM / WM / 32;         // 32x32 fragments per wavefront
  static constexpr int FN = BN / WN / 32;
  static constexpr int RPL = 64 / CPR;            // tile rows per wavefront load
  static constexpr int IPS = ROWS * CPR / NT;     // LDS-DMA loads per thread per stage
  static constexpr int JA = BM / (RPL * NW);      // loads j < JA fill A rows, the rest B rows
  static_assert(BM % (RPL * NW) == 0, "each load fills A rows only or B rows only");
  static_assert(FM >= 1 && FN >= 1, "tile too small for the wave grid");
  static_assert((CPR == 4 || CPR == 8) && IPS * NT == ROWS * CPR && ROWS % (RPL * NW) == 0, "stage loading");
  static_assert(STAGES >= 2 && IPS * (STAGES - 2) <= 63, "vmcnt range");
  static_assert(ND % BN == 0 && KD % BK == 0, "tiles");
};

// wait for the stage about to be used; `remaining` = stages issued after it (0 .. STAGES-2)
template <class C, int R>
__device__ __forceinline__ void wait_stage(int remaining) {
  if constexpr (R == 0) {
    vm_barrier<0>();
  } else {
    if (remaining >= R) vm_barrier<R * C::IPS>();
    else wait_stage<C, R - 1>(remaining);
  }
}

template <class C>
__global__ __launch_bounds__(C::NT) void grouped_gemm_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ W0, const bf16_t* __restrict__ W1,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ tile_count, const int2* __restrict__ tiles,
    int n_blocks, bf16_t* __restrict__ Cout, float* __restrict__ gu, int32_t* __restrict__ clip) {
  constexpr int BK = C::BK;
  __shared__ __align__(16) bf16_t smem[C::STAGES][C::ROWS * BK];

  // XCD-aware remap over the real unit count (known only here, from the scan): those units are
  // spread evenly over the 8 XCDs (dispatch is round-robin over them), consecutive units on one
  // XCD; surplus workgroups of the worst-case grid exit at once.  A remap over the padded grid
  // would leave the last XCDs idle whenever the real count is well under the bound.
  const int nunits = *tile_count * n_blocks;
  const int nper = (nunits + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  const int logical = (blockIdx.x & 7) * nper + slot;
  if (slot >= nper || logical >= nunits) return;
  int tile, nt;
  unit_of(tile_count, n_blocks, logical, tile, nt);
  const int2 ti = tiles[tile];
  const int e = ti.y & 255;
  const int row0 = ti.x;
  const int valid = ti.y >> 8;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches below
  const int wm = wv / C::WN, wn = wv % C::WN;
  // fragment i of wave row wm covers tile rows (i * WM + wm) * 32 .. +32, so the fragments of a
  // partly filled tile spread over all waves (and SIMDs).  This wave's fragments past `valid`
  // (always a suffix) are skipped: nf, the count of the others, picks one of FM+1 copies of
  // the k-loop once, so no branch sits between the MFMAs of a loop.
  int nf = 0;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) nf += (i * C::WM + wm) * 32 < valid;

  // LDS-DMA sources: load j of wavefront wv fills stage rows (j*NW + wv)*RPL .. +RPL;
  // lane -> row + lane/CPR, slot lane%CPR, which holds chunk slot ^ swz_key(row)
  const bf16_t* gp[C::IPS];
  const int dummy = C::GATEUP ? perm[row0] : row0;   // any valid row for the tile's unused rows
#pragma unroll
  for (int j = 0; j < C::IPS; ++j) {
    const int r = (j * C::NW + wv) * C::RPL + lane / C::CPR;
    const int ch = (lane % C::CPR) ^ swz_key<C::BK>(r);
    const bf16_t* p;
    if (r < C::BM) {
      const int src = r < valid ? (C::GATEUP ? perm[row0 + r] : row0 + r) : dummy;
      p = A + (size_t)src * C::KD;
    } else {
      const int rb = r - C::BM;
      if constexpr (C::GATEUP) {
        const bf16_t* base = rb < C::BN ? W0 : W1;
        const int n = nt * C::BN + (rb < C::BN ? rb : rb - C::BN);
        p = base + ((size_t)e * F + n) * D;
      } else {
        p = W0 + ((size_t)e * D + nt * C::BN + rb) * F;
      }
    }
    gp[j] = p + ch * 8;
  }
  // work units start at different k-steps so that concurrently running ones spread their
  // requests over the memory channels (every tile row starts on a 4 KiB boundary); the
  // order is a function of the unit only, so results stay reproducible
  const int k0 = C::ROT ? (logical * 5) % C::KT : 0;
  // loads j0 .. j1-1 of stage kt into ring slot sl
  auto issue = [&](int kt, int sl, int j0, int j1) {
    int kr = kt + k0;
    kr = kr >= C::KT ? kr - C::KT : kr;
#pragma unroll
    for (int j = 0; j < C::IPS; ++j) {
      if (j < j0 || j >= j1) continue;
      const auto src = GPTR(gp[j] + kr * BK);
      const auto dst = LPTR(&smem[sl][(j * C::NW + wv) * C::RPL * BK]);
      if (C::NTW && j >= C::JA)
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 2);   // cache policy: non-temporal
      else
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    }
  };

  f32x16 acc[C::G][C::FM][C::FN];
#pragma unroll
  for (int g = 0; g < C::G; ++g)
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[g][i][j][v] = 0.f;

#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (s < C::KT) issue(s, s, 0, C::IPS);

  constexpr int NKK = BK / 16;   // MFMA k-steps per stage
  using V = typename C::V;
  // fragments of MFMA k-step kk of a stage: A rows of this wave's NF fragments, B of its columns
  auto load_frags = [&](auto nf_tag, const bf16_t* As, const bf16_t* Bs, int kk, V* af, V (*bfr)[C::FN])
      __attribute__((always_inline)) {
    constexpr int NF = decltype(nf_tag)::value;
    const int kc = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int r = (i * C::WM + wm) * 32 + (lane & 31);
      af[i] = *reinterpret_cast<const V*>(&As[swz<BK>(r, kc)]);
    }
#pragma unroll
    for (int g = 0; g < C::G; ++g)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int r = g * C::BN + wn * (C::BN / C::WN) + j * 32 + (lane & 31);
        u32x4 v = *reinterpret_cast<const u32x4*>(&Bs[swz<BK>(r, kc)]);
        if constexpr (!C::GATEUP) {   // bf16 -> fp16 of 16 w (exact for 2^-18 <= |w| < 4096)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(v[q] << 16) * W_DOWN_SCALE,
                                                      __uint_as_float(v[q] & 0xFFFF0000u) * W_DOWN_SCALE);
            v[q] = __builtin_bit_cast(uint32_t, h);
          }
        }
        bfr[g][j] = __builtin_bit_cast(V, v);
      }
  };
  auto mfmas = [&](auto nf_tag, const V* af, const V (*bfr)[C::FN]) __attribute__((always_inline)) {
    constexpr int NF = decltype(nf_tag)::value;
#pragma unroll
    for (int g = 0; g < C::G; ++g)
#pragma unroll
      for (int i = 0; i < NF; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          if constexpr (C::GATEUP)
            acc[g][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[g][j], acc[g][i][j], 0, 0, 0);
          else
            acc[g][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bfr[g][j], acc[g][i][j], 0, 0, 0);
        }
  };
  auto kloop = [&](auto nf_tag) __attribute__((always_inline)) {
    constexpr int NF = decltype(nf_tag)::value;
    for (int kt = 0; kt < C::KT; ++kt) {
      wait_stage<C, C::STAGES - 2>(min(C::STAGES - 2, C::KT - 1 - kt));
      const bool more = kt + C::STAGES - 1 < C::KT;
      const int next_slot = (kt + C::STAGES - 1) % C::STAGES;
      const bf16_t* As = smem[kt % C::STAGES];
      const bf16_t* Bs = As + C::BM * BK;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        // the next stage's loads go out a slice per MFMA k-step: issuing them all at once
        // stalls the wave on the memory queue before its MFMAs can start
        if (more) issue(kt + C::STAGES - 1, next_slot, kk * C::IPS / NKK, (kk + 1) * C::IPS / NKK);
        if constexpr (NF > 0) {
          V af[NF], bfr[C::G][C::FN];
          load_frags(nf_tag, As, Bs, kk, af, bfr);
          mfmas(nf_tag, af, bfr);
        }
      }
    }
  };
  static_assert(C::FM <= 4, "k-loop copies");
  if (nf >= C::FM) kloop(std::integral_constant<int, C::FM>{});
  else if (C::FM > 1 && nf == 1) kloop(std::integral_constant<int, (C::FM > 1 ? 1 : 0)>{});
  else if (C::FM > 2 && nf == 2) kloop(std::integral_constant<int, (C::FM > 2 ? 2 : 0)>{});
  else if (C::FM > 3 && nf == 3) kloop(std::integral_constant<int, (C::FM > 3 ? 3 : 0)>{});
  else kloop(std::integral_constant<int, 0>{});

  // C layout of a 32x32 fragment: lane holds column lane%32, rows (v/4)*8 + (lane/32)*4 + v%4
  int nclip = 0;
  if constexpr (!C::SAVE_GU && C::WM * 32 * C::BN * 4 <= C::STAGES * C::ROWS * BK * 2) {
    // the fp32 results go through the drained LDS ring one slice of fragment rows (WM*32 rows x BN
    // columns) at a time, so that each thread then stores 8 consecutive fp16 values of a row with one
    // 16-byte store instead of 2-byte stores spread over 16 rows (1% off the layer at 4096 and 16384
    // tokens, the same bits)
    constexpr int SR = C::WM * 32;           // rows per slice
    constexpr int CG = C::BN / 8;            // 8-column groups per row
    constexpr int RPP = C::NT / CG;          // rows per pass
    constexpr int PASSES = SR / RPP;
    static_assert(C::NT % CG == 0 && SR % RPP == 0, "slice mapping");
    float* S = reinterpret_cast<float*>(&smem[0][0]);
    const int cg = tid % CG, rsub = tid / CG;
    const int c0 = nt * C::BN + cg * 8;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      __syncthreads();   // the ring (or the previous slice) is no longer read
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float o;
          if constexpr (C::GATEUP) o = silu(acc[0][i][j][v]) * acc[1][i][j][v];
          else o = acc[0][i][j][v] * (1.0f / W_DOWN_SCALE);
          S[(wm * 32 + (lane >> 5) * 4 + (v >> 2) * 8 + (v & 3)) * C::BN + wn * (C::BN / C::WN) + j * 32 +
            (lane & 31)] = o;
        }
      __syncthreads();
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        const int rl = ps * RPP + rsub;
        const int r = i * SR + rl;
        if (r < valid) {
          const f32x4 d0 = *reinterpret_cast<const f32x4*>(&S[rl * C::BN + cg * 8]);
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(&S[rl * C::BN + cg * 8 + 4]);
          const float d[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
          u32x4 pk;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            nclip += !(fabsf(d[2 * q]) <= F16_MAX);   // out of range or NaN: stored clipped, counted
            nclip += !(fabsf(d[2 * q + 1]) <= F16_MAX);
            pk[q] = static_cast<uint32_t>(f32_to_f16_sat(d[2 * q])) |
                    (static_cast<uint32_t>(f32_to_f16_sat(d[2 * q + 1])) << 16);
          }
          *reinterpret_cast<u32x4*>(&Cout[(size_t)(row0 + r) * C::ND + c0]) = pk;
        }
      }
    }
  } else {
    // the fragments stored as they are (the tile configs whose slice does not fit the ring, and
    // the gate/up configs that also keep G and U)
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = (i * C::WM + wm) * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
          const int c = nt * C::BN + wn * (C::BN / C::WN) + j * 32 + (lane & 31);
          if (r < valid) {
            float o;
            if constexpr (C::GATEUP) o = silu(acc[0][i][j][v]) * acc[1][i][j][v];
            else o = acc[0][i][j][v] * (1.0f / W_DOWN_SCALE);
            nclip += !(fabsf(o) <= F16_MAX);   // out of range or NaN: stored clipped, counted
            Cout[(size_t)(row0 + r) * C::ND + c] = f32_to_f16_sat(o);
            if constexpr (C::SAVE_GU) {   // [rows, 2F]: G in columns 0..F-1, U in F..2F-1
              gu[(size_t)(row0 + r) * (2 * F) + c] = acc[0][i][j][v];
              gu[(size_t)(row0 + r) * (2 * F) + F + c] = acc[1][i][j][v];
            }
          }
        }
  }
  nclip = wave_sum_int(nclip);
  if (nclip && lane == 0 && clip) atomicAdd(clip, nclip);   // an integer count: order does not matter
}

// tile sets by batch size (rows per expert ~ T/8), chosen by measurement on MI355X.  Up to a
// few hundred tokens the layer is bound by streaming the weights once; marking the weight loads
// non-temporal keeps them from displacing the activation rows that every column tile re-reads.
// 8 waves (2 per SIMD) keep more loads in flight per CU at small batches and give more MFMA
// work per byte staged on the 256-row tiles of large batches.  The large gate/up tiles run
// three 32-k stages: the deeper prefetch beats the longer rows of two 64-k stages (328 against
// 390 us at 4096 tokens on random data); the down GEMM prefers 64-k stages, and a 2 x 4 wave
// grid (wave tiles of 128 rows x 64 columns): each W_down fragment, converted to fp16 after its
// LDS read, is then read by two waves instead of four (230 against 250 us at 4096 tokens).
using GuTiny = Cfg<32, 64, 1, 2, true, 4, 64, 1, true>;
using DnTiny = Cfg<32, 64, 1, 2, false, 4>;
using GuSmall = Cfg<64, 128, 2, 4, true, 2, 64, 1, true>;
using DnSmall = Cfg<64, 256, 2, 4, false, 2, 64, 1, true>;
// a few hundred tokens up to about a thousand: experts hold 60-130 rows, so 64-row tiles would
// stream most experts' weights twice and 256-row tiles leave most of each tile padding; 128-row
// tiles in the small tiles' streaming style (two 64-k stages, non-temporal weights, rotated start)
// stream each expert's weights about once (layer 0.183 against 0.206 ms at 416 tokens, 0.206
// against 0.236 at 768, 0.237 against 0.247 at 832, and 0.269 against 0.243 at 896, where the
// 256-row tiles take over; three 32-k stages instead were slower than both neighbours)
using GuMed = Cfg<128, 128, 2, 4, true, 2, 64, 1, true>;
using DnMed = Cfg<128, 256, 2, 4, false, 2, 64, 1, true>;
// and 192-row tiles in the same style for experts of 100-190 rows (0.220 against 0.246 ms at 896
// tokens, 0.228 against 0.253 at 1024; 0.277 against 0.272 at 1280, where the 256-row tiles win)
using GuMed192 = Cfg<192, 128, 2, 4, true, 2, 64, 1, true>;
using DnMed192 = Cfg<192, 256, 2, 4, false, 2, 64, 1, true>;
// 256-row tiles in that style still lead up to about 1500 tokens (0.255 against 0.273 ms at 1280,
// 0.281 against 0.290 at 1536), level at 1792, and behind the MFMA-tuned large tiles from 2048
using GuMed256 = Cfg<256, 128, 2, 4, true, 2, 64, 1, true>;
using DnMed256 = Cfg<256, 256, 2, 4, false, 2, 64, 1, true>;
// and 384-row streaming tiles (three 32-k stages on 4 x 2 waves to fit LDS) up to about 2500
// tokens: 0.339 against 0.379 ms at 1792, 0.364 against 0.389 at 2048, 0.383 against 0.400 at
// 2560; at 3072 (0.568 against 0.442) experts commonly outgrow one tile
using GuMed384 = Cfg<384, 128, 4, 2, true, 3, 32, 1, true>;
using DnMed384 = Cfg<384, 256, 4, 2, false, 3, 32, 1, true>;
using GuLarge = Cfg<256, 128, 4, 2, true, 3, 32, 0>;
using DnLarge = Cfg<256, 256, 2, 4, false, 2, 64, 0>;
// 64-row tiles stream an expert's weights once per tile, so they lose as soon as experts commonly
// hold more than 64 rows; the 128-row tiles likewise beyond about 128 rows
constexpr int SMALL_PLAN_TOKENS = 384;
constexpr int MEDIUM_PLAN_TOKENS = 832;
constexpr int MEDIUM192_PLAN_TOKENS = 1024;
constexpr int MEDIUM256_PLAN_TOKENS = 1536;
constexpr int MEDIUM384_PLAN_TOKENS = 2560;

template <class C>
hipError_t launch_cfg(const bf16_t* A, const bf16_t* W0, const bf16_t* W1, const GemmArgs& a,
                      const int32_t* tile_prefix, const int2* tiles, bf16_t* out, hipStream_t stream,
                      float* gu = nullptr) {
  const int max_tiles = max_row_tiles(a.T, C::BM);
  if (max_tiles == 0) return hipSuccess;
  const int n_blocks = C::ND / C::BN;
  const int grid = (max_tiles * n_blocks + 7) / 8 * 8;
  hipLaunchKernelGGL(grouped_gemm_kernel<C>, dim3(grid), dim3(C::NT), 0, stream, A, W0, W1, a.perm,
                     tile_prefix + E, tiles, n_blocks, out, gu, a.clip);
  return hipGetLastError();
}

// the gate/up config C with the pre-activations saved (the backward pass recomputes them)
template <class C>
using SavingGU = Cfg<C::BM, C::BN, C::WM, C::WN, true, C::STAGES, C::BK, C::ROT, C::NTW, true>;

}  // namespace

int max_row_tiles(int T, int bm) {
  // sum_e ceil(c_e / bm) with sum_e c_e = 8T and every c_e <= T
  const long long rows = 8LL * T;
  const long long a = (rows + (long long)E * (bm - 1)) / bm;
  const long long b = (long long)E * ((T + bm - 1) / bm);
  return static_cast<int>(a < b ? a : b);
}

GemmPlan plan_gemm(int T) {
  GemmPlan p;
  if (T <= 48) {
    p.variant = 0;
    p.bm_gu = GuTiny::BM;
    p.bm_dn = DnTiny::BM;
  } else if (T <= SMALL_PLAN_TOKENS) {
    p.variant = 1;
    p.bm_gu = GuSmall::BM;
    p.bm_dn = DnSmall::BM;
  } else if (T <= MEDIUM_PLAN_TOKENS) {
    p.variant = 3;
    p.bm_gu = GuMed::BM;
    p.bm_dn = DnMed::BM;
  } else if (T <= MEDIUM192_PLAN_TOKENS) {
    p.variant = 4;
    p.bm_gu = GuMed192::BM;
    p.bm_dn = DnMed192::BM;
  } else if (T <= MEDIUM256_PLAN_TOKENS) {
    p.variant = 5;
    p.bm_gu = GuMed256::BM;
    p.bm_dn = DnMed256::BM;
  } else if (T <= MEDIUM384_PLAN_TOKENS) {
    p.variant = 6;
    p.bm_gu = GuMed384::BM;
    p.bm_dn = DnMed384::BM;
  } else {
    p.variant = 2;
    p.bm_gu = GuLarge::BM;
    p.bm_dn = DnLarge::BM;
  }
  return p;
}

hipError_t launch_gateup(const GemmArgs& a, const GemmPlan& p, hipStream_t stream) {
  if (a.gu) {
    switch (p.variant) {
      case 0: return launch_cfg<SavingGU<GuTiny>>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.tiles_gu, a.h, stream, a.gu);
      case 1: return launch_cfg<SavingGU<GuSmall>>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.tiles_gu, a.h, stream, a.gu);
      case 3: return launch_cfg<SavingGU<GuMed>>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.tiles_gu, a.h, stream, a.gu);
      case 4: return launch_cfg<SavingGU<GuMed192>>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.tiles_gu, a.h, stream, a.gu);
      case 5: return launch_cfg<SavingGU<GuMed256>>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.tiles_gu, a.h, stream, a.gu);
      case 6: return launch_cfg<SavingGU<GuMed384>>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.tiles_gu, a.h, stream, a.gu);
      default: return launch_cfg<SavingGU<GuLarge>>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.tiles_gu, a.h, stream, a.gu);
    }
  }
  switch (p.variant) {
    case 0: return launch_cfg<GuTiny>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.tiles_gu, a.h, stream);
    case 1: return launch_cfg<GuSmall>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.tiles_gu, a.h, stream);
    case 3: return launch_cfg<GuMed>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.tiles_gu, a.h, stream);
    case 4: return launch_cfg<GuMed192>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.tiles_gu, a.h, stream);
    case 5: return launch_cfg<GuMed256>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.tiles_gu, a.h, stream);
    case 6: return launch_cfg<GuMed384>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.tiles_gu, a.h, stream);
    default: return launch_cfg<GuLarge>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.tiles_gu, a.h, stream);
  }
}

hipError_t launch_down(const GemmArgs& a, const GemmPlan& p, hipStream_t stream) {
  switch (p.variant) {
    case 0: return launch_cfg<DnTiny>(a.h, a.w_down, nullptr, a, a.tile_prefix_dn, a.tiles_dn, a.y, stream);
    case 1: return launch_cfg<DnSmall>(a.h, a.w_down, nullptr, a, a.tile_prefix_dn, a.tiles_dn, a.y, stream);
    case 3: return launch_cfg<DnMed>(a.h, a.w_down, nullptr, a, a.tile_prefix_dn, a.tiles_dn, a.y, stream);
    case 4: return launch_cfg<DnMed192>(a.h, a.w_down, nullptr, a, a.tile_prefix_dn, a.tiles_dn, a.y, stream);
    case 5: return launch_cfg<DnMed256>(a.h, a.w_down, nullptr, a, a.tile_prefix_dn, a.tiles_dn, a.y, stream);
    case 6: return launch_cfg<DnMed384>(a.h, a.w_down, nullptr, a, a.tile_prefix_dn, a.tiles_dn, a.y, stream);
    default: return launch_cfg<DnLarge>(a.h, a.w_down, nullptr, a, a.tile_prefix_dn, a.tiles_dn, a.y, stream);
  }
}

}  // namespace olmoe
