// Grouped expert GEMMs of the OLMoE MoE layer on bf16 MFMA (gfx950).
//
// Each expert is a SwiGLU network, (SiLU(x W_gate^T) * (x W_up^T)) W_down^T,
// with gate/up [1024,2048] and down [2048,1024] ("OLMoE Guide: 64-Expert
// Fine-Grained Open MoE Architecture", item 1 and its SwiGLUExpert module;
// "Mixture-of-experts LLMs from scratch with OLMoE", section 2, where every
// expert runs once on the rows routed to it and production kernels put all
// the groups into one grouped matrix multiplication).
//
// Work unit: (row tile of one expert, column tile).  Row tiles of all experts
// are numbered in expert order; the scan kernel leaves the per-expert prefix of
// that numbering, and each workgroup finds its expert by a binary search over
// the 65-entry prefix, so there is no host round trip and no per-expert launch.
// The grid is sized from the upper bound on the tile count; workgroups past the
// real count return at once.
//
// gate/up: A = x rows gathered through perm (never materialised), B = the gate
// rows and the up rows of the same output columns, so one workgroup holds both
// accumulators and applies SiLU(g)*u in fp32 before the single store of H.
// down: A = H rows (already expert-contiguous), B = W_down[e]; Y stored per row.
//
// The intermediates H and Y are stored as fp16 (round to nearest even,
// saturated at +-65504): same bytes as bf16 but 3 more significand bits, which
// keeps their rounding well below the output's own bf16 rounding.  The down
// GEMM therefore runs on f16 MFMA; W_down's bf16 values are converted to fp16
// while being staged into LDS, exactly for every weight in fp16's normal range
// (weights below 2^-14 in magnitude keep an absolute error under 2^-24).
//
// Both operands are staged through LDS in [row][64] bf16 tiles whose 16-byte
// chunks are XOR-swizzled by row, so the MFMA fragment reads (8 rows x 16 bytes
// per group of lanes) hit distinct banks; two LDS buffers let the next k-tile's
// global loads run during the current tile's MFMAs.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace olmoe {

namespace {

constexpr int BK = 64;

__device__ __forceinline__ int swz(int row, int ch) { return row * BK + ((ch ^ (row & 7)) << 3); }

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

template <int BM_, int BN_, int WM_, int WN_, bool GATEUP_>
struct Cfg {
  static constexpr int BM = BM_;   // rows (tokens) per tile
  static constexpr int BN = BN_;   // output columns per tile
  static constexpr int WM = WM_, WN = WN_;
  static constexpr bool GATEUP = GATEUP_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int G = GATEUP ? 2 : 1;        // accumulator sets (gate, up)
  using V = typename std::conditional<GATEUP, bf16x8, f16x8>::type;   // MFMA operand type
  static constexpr int NB = G * BN;               // B rows per tile
  static constexpr int KD = GATEUP ? D : F;       // reduction length
  static constexpr int ND = GATEUP ? F : D;       // output row length
  static constexpr int FM = BM / WM / 32;         // 32x32 fragments per wavefront
  static constexpr int FN = BN / WN / 32;
  static constexpr int ACH = BM * (BK / 8) / NT;  // 16-byte A chunks per thread per k-tile
  static constexpr int BCH = NB * (BK / 8) / NT;
  static_assert(FM >= 1 && FN >= 1, "tile too small for the wave grid");
  static_assert(ACH >= 1 && BCH >= 1 && ACH * NT == BM * 8 && BCH * NT == NB * 8, "chunking");
  static_assert(ND % BN == 0, "column tiles");
};

template <class C>
__global__ __launch_bounds__(C::NT) void grouped_gemm_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ W0, const bf16_t* __restrict__ W1,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_prefix, bf16_t* __restrict__ Cout) {
  __shared__ __align__(16) bf16_t smem[2][(C::BM + C::NB) * BK];

  const int tile = blockIdx.y;
  const int nt = blockIdx.x;
  if (tile >= tile_prefix[E]) return;
  int lo = 0, hi = E;
  while (hi - lo > 1) {   // last expert whose first tile is <= tile
    const int mid = (lo + hi) >> 1;
    if (tile_prefix[mid] <= tile) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int row0 = offsets[e] + (tile - tile_prefix[e]) * C::BM;
  const int valid = min(C::BM, offsets[e + 1] - row0);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv / C::WN, wn = wv % C::WN;
  const int ch = tid & 7;

  const bf16_t* asrc[C::ACH];
#pragma unroll
  for (int q = 0; q < C::ACH; ++q) {
    const int r = (tid >> 3) + q * (C::NT / 8);
    if (r < valid) {
      const int src = C::GATEUP ? perm[row0 + r] : row0 + r;
      asrc[q] = A + (size_t)src * C::KD + ch * 8;
    } else {
      asrc[q] = nullptr;
    }
  }
  const bf16_t* bsrc[C::BCH];
#pragma unroll
  for (int q = 0; q < C::BCH; ++q) {
    const int r = (tid >> 3) + q * (C::NT / 8);
    if (C::GATEUP) {
      const bf16_t* base = r < C::BN ? W0 : W1;
      const int n = nt * C::BN + (r < C::BN ? r : r - C::BN);
      bsrc[q] = base + ((size_t)e * F + n) * D + ch * 8;
    } else {
      bsrc[q] = W0 + ((size_t)e * D + nt * C::BN + r) * F + ch * 8;
    }
  }

  u32x4 ra[C::ACH], rb[C::BCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < C::ACH; ++q)
      ra[q] = asrc[q] ? *reinterpret_cast<const u32x4*>(asrc[q] + k0) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < C::BCH; ++q) rb[q] = *reinterpret_cast<const u32x4*>(bsrc[q] + k0);
  };
  auto sstore = [&](int buf) {
    bf16_t* As = smem[buf];
    bf16_t* Bs = smem[buf] + C::BM * BK;
#pragma unroll
    for (int q = 0; q < C::ACH; ++q) {
      const int r = (tid >> 3) + q * (C::NT / 8);
      *reinterpret_cast<u32x4*>(&As[swz(r, ch)]) = ra[q];
    }
#pragma unroll
    for (int q = 0; q < C::BCH; ++q) {
      const int r = (tid >> 3) + q * (C::NT / 8);
      u32x4 v = rb[q];
      if constexpr (!C::GATEUP) {   // bf16 -> fp16 (exact in fp16's normal range)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(v[i] << 16),
                                                      __uint_as_float(v[i] & 0xFFFF0000u));
          v[i] = __builtin_bit_cast(uint32_t, h);
        }
      }
      *reinterpret_cast<u32x4*>(&Bs[swz(r, ch)]) = v;
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

  constexpr int KT = C::KD / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
    const bf16_t* As = smem[buf];
    const bf16_t* Bs = smem[buf] + C::BM * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int kc = kk * 2 + (lane >> 5);
      using V = typename C::V;
      V af[C::FM], bfr[C::G][C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int r = wm * (C::BM / C::WM) + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const V*>(&As[swz(r, kc)]);
      }
#pragma unroll
      for (int g = 0; g < C::G; ++g)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int r = g * C::BN + wn * (C::BN / C::WN) + j * 32 + (lane & 31);
          bfr[g][j] = *reinterpret_cast<const V*>(&Bs[swz(r, kc)]);
        }
#pragma unroll
      for (int g = 0; g < C::G; ++g)
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            if constexpr (C::GATEUP)
              acc[g][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[g][j], acc[g][i][j], 0, 0, 0);
            else
              acc[g][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bfr[g][j], acc[g][i][j], 0, 0, 0);
          }
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  // C layout of a 32x32 fragment: lane holds column lane%32, rows (v/4)*8 + (lane/32)*4 + v%4
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * (C::BM / C::WM) + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        const int c = nt * C::BN + wn * (C::BN / C::WN) + j * 32 + (lane & 31);
        if (r < valid) {
          float o;
          if constexpr (C::GATEUP) o = silu(acc[0][i][j][v]) * acc[1][i][j][v];
          else o = acc[0][i][j][v];
          Cout[(size_t)(row0 + r) * C::ND + c] = f32_to_f16_sat(o);
        }
      }
}

// tile sets: 0 = small row tiles (decode-like batches), 1 = large row tiles
using GuSmall = Cfg<32, 64, 1, 2, true>;
using DnSmall = Cfg<32, 64, 1, 2, false>;
using GuLarge = Cfg<128, 64, 2, 2, true>;
using DnLarge = Cfg<128, 128, 2, 2, false>;

template <class C>
hipError_t launch_cfg(const bf16_t* A, const bf16_t* W0, const bf16_t* W1, const GemmArgs& a,
                      const int32_t* tile_prefix, bf16_t* out, hipStream_t stream) {
  const int tiles = max_row_tiles(a.T, C::BM);
  if (tiles == 0) return hipSuccess;
  dim3 grid(C::ND / C::BN, tiles);
  hipLaunchKernelGGL(grouped_gemm_kernel<C>, grid, dim3(C::NT), 0, stream, A, W0, W1, a.perm,
                     a.offsets, tile_prefix, out);
  return hipGetLastError();
}

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
  if (T <= 384) {
    p.variant = 0;
    p.bm_gu = GuSmall::BM;
    p.bm_dn = DnSmall::BM;
  } else {
    p.variant = 1;
    p.bm_gu = GuLarge::BM;
    p.bm_dn = DnLarge::BM;
  }
  return p;
}

hipError_t launch_gateup(const GemmArgs& a, const GemmPlan& p, hipStream_t stream) {
  if (p.variant == 0)
    return launch_cfg<GuSmall>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.h, stream);
  return launch_cfg<GuLarge>(a.x, a.w_gate, a.w_up, a, a.tile_prefix_gu, a.h, stream);
}

hipError_t launch_down(const GemmArgs& a, const GemmPlan& p, hipStream_t stream) {
  if (p.variant == 0)
    return launch_cfg<DnSmall>(a.h, a.w_down, nullptr, a, a.tile_prefix_dn, a.y, stream);
  return launch_cfg<DnLarge>(a.h, a.w_down, nullptr, a, a.tile_prefix_dn, a.y, stream);
}

}  // namespace olmoe
