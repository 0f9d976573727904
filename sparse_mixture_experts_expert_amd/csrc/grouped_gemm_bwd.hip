// Grouped GEMMs of the backward pass of the OLMoE MoE layer on MFMA (gfx950).
//
// The expert network is (SiLU(X W_gate^T) * (X W_up^T)) W_down^T ("OLMoE Guide:
// 64-Expert Fine-Grained Open MoE Architecture", item 1 and its SwiGLUExpert
// module); its gradients contract over the other index of each product:
//
//   dgrad (rows of one expert x output columns, K fixed):
//     dH~ = dOut_rows W_down[e]            A = upstream rows (gathered), B = W_down[e] as [d][f]
//     dX  = dG W_gate[e] + dU W_up[e]      A = [dG | dU] rows, B = W_gate[e] / W_up[e] as [f][d]
//   wgrad (one expert's weight tile, K = the expert's rows):
//     dW_down[e]       = dOut_rows^T (w H)
//     dW_gate/up[e]    = [dG | dU]^T X_rows
//
// The weights are read as stored, so the dgrad B operand and both wgrad operands
// have the reduction index as their outer (row) index.  Such tiles are staged
// in LDS as rows of k (LDS-DMA, 16-byte chunks XOR-swizzled by k & 3), and the
// MFMA fragments are read with gfx950's transposing LDS read: within a group of
// 16 lanes, lane p receives element p % 4 of the 8-byte pieces addressed by
// lanes p/4, p/4 + 4, p/4 + 8 and p/4 + 12, so pointing lane j at
// (k0 + j/4, n0 + 4 (j%4)) hands lane p column n0 + p at k0 .. k0+3.  Two such
// reads give the 8 consecutive k of a 32x32x16 operand.  Row-major (K-inner)
// A tiles use the forward kernel's layout and 16-byte reads.
//
// Pipelining, XCD remap and the per-workgroup choice of k-loop copy follow the
// forward grouped GEMM.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

#define GPTR(p) ((const __attribute__((address_space(1))) void*)(p))
#define LPTR(p) ((__attribute__((address_space(3))) void*)(p))

namespace olmoe {

namespace {

template <int N>
__device__ __forceinline__ void vm_barrier_b() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
template <int R, int IPS>
__device__ __forceinline__ void wait_stage_b(int remaining) {
  if constexpr (R == 0) {
    vm_barrier_b<0>();
  } else {
    if (remaining >= R) vm_barrier_b<R * IPS>();
    else wait_stage_b<R - 1, IPS>(remaining);
  }
}

// element offset of (k, col) in a K-outer tile of BW columns; col % 4 == 0 inside a chunk
template <int BW>
__device__ __forceinline__ int kout_off(int k, int col) {
  return k * BW + ((((col >> 3) ^ ((k & 3) << 1))) << 3) + (col & 7);
}
// element offset of chunk ch of row `row` in a K-inner tile of 64-element rows
__device__ __forceinline__ int kin_off(int row, int ch) { return row * 64 + ((ch ^ (row & 7)) << 3); }

// a table read through the constant address space: wave-uniform reads of it become scalar loads
using cint_ptr = const __attribute__((address_space(4))) int*;
__device__ __forceinline__ cint_ptr as_const(const int32_t* p) {
  return (cint_ptr)reinterpret_cast<uintptr_t>(p);
}

// LDS byte address (offset in the LDS aperture) of element e of a K-outer tile
__device__ __forceinline__ uint32_t lds_addr(const bf16_t* tile, int e) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const bf16_t*)(tile + e)));
}

// addresses of the two transposing reads that give the 32x32x16 operand of columns
// col0 .. col0+31 at k-step kk of a K-outer tile: 8 consecutive k of column col0 + lane%32
template <int BW>
__device__ __forceinline__ void frag_kout_addr(const bf16_t* tile, int kk, int col0, int lane, uint32_t& a_lo,
                                               uint32_t& a_hi) {
  const int krow = kk * 16 + (lane >> 5) * 8 + ((lane & 15) >> 2);
  const int col = col0 + ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  a_lo = lds_addr(tile, kout_off<BW>(krow, col));
  a_hi = lds_addr(tile, kout_off<BW>(krow + 4, col));
}

__device__ __forceinline__ bf16x8 frag_of(uint2 lo, uint2 hi) {
  const u32x4 v = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, v);
}

// Four transposing LDS reads, waited for inside the same block.  Written as assembly
// because the compiler, unable to tell these reads from the LDS-DMA writes still in flight
// (to other ring slots), would otherwise drain every outstanding load before each of them;
// the stage being read was already waited for at the top of its k-step.
__device__ __forceinline__ void tr_read4(uint2& r0, uint2& r1, uint2& r2, uint2& r3, uint32_t a0, uint32_t a1,
                                         uint32_t a2, uint32_t a3) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}

// two 32x32x16 operands (columns col0 and col1) of a K-outer tile
template <int BW>
__device__ __forceinline__ void frag_kout2(const bf16_t* tile, int kk, int col0, int col1, int lane, bf16x8& f0,
                                           bf16x8& f1) {
  uint32_t a0, a1, a2, a3;
  frag_kout_addr<BW>(tile, kk, col0, lane, a0, a1);
  frag_kout_addr<BW>(tile, kk, col1, lane, a2, a3);
  uint2 r0, r1, r2, r3;
  tr_read4(r0, r1, r2, r3, a0, a1, a2, a3);
  f0 = frag_of(r0, r1);
  f1 = frag_of(r2, r3);
}

__device__ __forceinline__ float sigmoidf(float g) { return 1.0f / (1.0f + __expf(-g)); }

constexpr int BK = 64;   // reduction rows per stage

// ----------------------------------------------------------------------------- dgrad

enum { EPI_DH = 0, EPI_F32 = 1 };

template <int BM_, int BN_, int WM_, int WN_, int STAGES_, int EPI_>
struct DCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_, EPI = EPI_;
  static constexpr int NW = WM * WN, NT = NW * 64;
  static constexpr int KD = 2 * F;                     // both dgrad products reduce over 2048
  static constexpr int ND = EPI == EPI_DH ? F : D;     // output columns
  static constexpr int KT = KD / BK;
  static constexpr int FM = BM / WM / 32, FN = BN / WN / 32;
  static constexpr int A_ELEMS = BM * BK, B_ELEMS = BK * BN;
  static constexpr int IPA = A_ELEMS / 8 / NT;         // 16-byte loads per thread per stage
  static constexpr int IPB = B_ELEMS / 8 / NT;
  static constexpr int IPS = IPA + IPB;
  static constexpr int CPB = BN / 8;                   // chunks per B row
  static constexpr int RPB = 64 / CPB;                 // B rows per wave load
  static_assert(FM >= 1 && FN >= 1 && IPA * NT * 8 == A_ELEMS && IPB * NT * 8 == B_ELEMS, "tiling");
  static_assert(CPB >= 8 && BM % (8 * NW) == 0 && BK % (RPB * NW) == 0, "stage loading");
  static_assert(STAGES >= 2 && IPS * (STAGES - 2) <= 63 && ND % BN == 0, "pipeline");
};

template <class C>
__global__ __launch_bounds__(C::NT) void dgrad_kernel(BwdDgradArgs a) {
  __shared__ __align__(16) bf16_t smem[C::STAGES][C::A_ELEMS + C::B_ELEMS];

  const int n_blocks = C::ND / C::BN;
  const int nunits = *a.tile_count * n_blocks;
  const int nper = (nunits + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  const int logical = (blockIdx.x & 7) * nper + slot;
  if (slot >= nper || logical >= nunits) return;
  const int tile = logical / n_blocks;
  const int nt = logical - tile * n_blocks;
  const int2 ti = a.tiles[tile];
  const int e = ti.y & 255;
  const int row0 = ti.x;
  const int valid = ti.y >> 8;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / C::WN, wn = wv % C::WN;
  int nf = 0;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) nf += (i * C::WM + wm) * 32 < valid;

  // A (K-inner rows): load j fills rows (j*NW + wv)*8 + lane/8, slot lane%8 <- chunk slot ^ (row & 7)
  const bf16_t* ga[C::IPA];
  const int dummy = a.a_rows ? a.a_rows[row0] : row0;
#pragma unroll
  for (int j = 0; j < C::IPA; ++j) {
    const int r = (j * C::NW + wv) * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ (r & 7);
    const int src = r < valid ? (a.a_rows ? a.a_rows[row0 + r] : row0 + r) : dummy;
    ga[j] = a.a + (size_t)src * C::KD + ch * 8;
  }
  // B (K-outer weight rows): load j fills k-rows (j*NW + wv)*RPB + lane/CPB, slot lane%CPB
  int gb[C::IPB];   // element offset inside a k-stage of the weight matrix
#pragma unroll
  for (int j = 0; j < C::IPB; ++j) {
    const int k = (j * C::NW + wv) * C::RPB + lane / C::CPB;
    const int ch = (lane % C::CPB) ^ ((k & 3) << 1);
    gb[j] = k * a.ldb + nt * C::BN + ch * 8;
  }
  auto issue = [&](int kt, int sl, int j0, int j1) {
    const int kg = kt * BK;
    const bf16_t* bbase = (kg < a.kb_split ? a.b0 + (size_t)kg * a.ldb : a.b1 + (size_t)(kg - a.kb_split) * a.ldb) +
                          (size_t)e * a.b_stride;
#pragma unroll
    for (int j = 0; j < C::IPS; ++j) {
      if (j < j0 || j >= j1) continue;
      if (j < C::IPA) {
        __builtin_amdgcn_global_load_lds(GPTR(ga[j] + kg), LPTR(&smem[sl][(j * C::NW + wv) * 8 * 64]), 16, 0, 0);
      } else {
        const int jb = j - C::IPA;
        __builtin_amdgcn_global_load_lds(GPTR(bbase + gb[jb]),
                                         LPTR(&smem[sl][C::A_ELEMS + (jb * C::NW + wv) * C::RPB * C::BN]), 16, 0, 0);
      }
    }
  };

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s) issue(s, s, 0, C::IPS);
  constexpr int NKK = BK / 16;
  auto kloop = [&](auto nf_tag) __attribute__((always_inline)) {
    constexpr int NF = decltype(nf_tag)::value;
    for (int kt = 0; kt < C::KT; ++kt) {
      wait_stage_b<C::STAGES - 2, C::IPS>(min(C::STAGES - 2, C::KT - 1 - kt));
      const bool more = kt + C::STAGES - 1 < C::KT;
      const int next_slot = (kt + C::STAGES - 1) % C::STAGES;
      const bf16_t* As = smem[kt % C::STAGES];
      const bf16_t* Bs = As + C::A_ELEMS;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (more) issue(kt + C::STAGES - 1, next_slot, kk * C::IPS / NKK, (kk + 1) * C::IPS / NKK);
        if constexpr (NF > 0) {
          bf16x8 af[NF], bfr[C::FN];
          const int kc = kk * 2 + (lane >> 5);
#pragma unroll
          for (int i = 0; i < NF; ++i)
            af[i] = *reinterpret_cast<const bf16x8*>(&As[kin_off((i * C::WM + wm) * 32 + (lane & 31), kc)]);
          static_assert(C::FN % 2 == 0, "B operands are read in pairs");
#pragma unroll
          for (int j = 0; j < C::FN; j += 2)
            frag_kout2<C::BN>(Bs, kk, wn * (C::BN / C::WN) + j * 32, wn * (C::BN / C::WN) + j * 32 + 32, lane,
                              bfr[j], bfr[j + 1]);
#pragma unroll
          for (int i = 0; i < NF; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  };
  if (nf >= C::FM) kloop(std::integral_constant<int, C::FM>{});
  else if (C::FM > 1 && nf == 1) kloop(std::integral_constant<int, (C::FM > 1 ? 1 : 0)>{});
  else if (C::FM > 2 && nf == 2) kloop(std::integral_constant<int, (C::FM > 2 ? 2 : 0)>{});
  else if (C::FM > 3 && nf == 3) kloop(std::integral_constant<int, (C::FM > 3 ? 3 : 0)>{});
  else kloop(std::integral_constant<int, 0>{});

  // The accumulators go through LDS one slice of fragment rows (WM*32 rows x BN columns, fp32) at
  // a time, so that each thread then takes 8 consecutive columns of a row: 16-byte loads and stores
  // instead of 4-byte ones spread over 16 rows per lane.
  //   dH~ epilogue: dH = w dH~; H = SiLU(G) U, so dG = dH U SiLU'(G), dU = dH SiLU(G); and the row
  //   sums of dH~ * H, whose total over all columns is <dout, Y> (dH~ = dout W_down), the routing
  //   weight's gradient without the expert outputs.
  //   fp32 epilogue: the rows as they are.
  constexpr int SR = C::WM * 32;           // rows per slice
  constexpr int CG = C::BN / 8;            // 8-column groups per row
  constexpr int RPP = C::NT / CG;          // rows per pass
  constexpr int PASSES = SR / RPP;
  static_assert(SR * C::BN * 4 <= C::STAGES * (C::A_ELEMS + C::B_ELEMS) * 2, "a slice fits the LDS ring");
  static_assert(C::NT % CG == 0 && SR % RPP == 0 && (CG & (CG - 1)) == 0 && CG <= 64, "slice mapping");
  float* S = reinterpret_cast<float*>(&smem[0][0]);
  const int cg = tid % CG, rsub = tid / CG;
  const int c0 = nt * C::BN + cg * 8;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    __syncthreads();   // the ring (or the previous slice) is no longer read
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        S[(wm * 32 + (lane >> 5) * 4 + (v >> 2) * 8 + (v & 3)) * C::BN + wn * (C::BN / C::WN) + j * 32 +
          (lane & 31)] = acc[i][j][v];
    __syncthreads();
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int rl = ps * RPP + rsub;
      const int r = i * SR + rl;
      const bool ok = r < valid;
      const size_t row = (size_t)row0 + (ok ? r : 0);   // padding rows read row0 and store nothing
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(&S[rl * C::BN + cg * 8]);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(&S[rl * C::BN + cg * 8 + 4]);
      if constexpr (C::EPI == EPI_DH) {
        const f32x4* gp = reinterpret_cast<const f32x4*>(a.gu + row * (2 * F) + c0);
        const f32x4* up = reinterpret_cast<const f32x4*>(a.gu + row * (2 * F) + F + c0);
        const f32x4 g0 = gp[0], g1 = gp[1], u0 = up[0], u1 = up[1];
        const float w = a.row_w[row];
        const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
        const float u[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
        const float d[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
        float dg[8], du[8], hw[8];
        float sum = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float sg = sigmoidf(g[k]);
          const float sl = g[k] * sg;
          const float h = sl * u[k];
          const float dh = w * d[k];
          dg[k] = dh * u[k] * (sg * (1.0f + g[k] * (1.0f - sg)));
          du[k] = dh * sl;
          hw[k] = w * h;
          sum = fmaf(d[k], h, sum);
        }
        if (ok) {
          const u32x4 pg = {cvt_bf16x2(dg[0], dg[1]), cvt_bf16x2(dg[2], dg[3]), cvt_bf16x2(dg[4], dg[5]),
                            cvt_bf16x2(dg[6], dg[7])};
          const u32x4 pu = {cvt_bf16x2(du[0], du[1]), cvt_bf16x2(du[2], du[3]), cvt_bf16x2(du[4], du[5]),
                            cvt_bf16x2(du[6], du[7])};
          const u32x4 ph = {cvt_bf16x2(hw[0], hw[1]), cvt_bf16x2(hw[2], hw[3]), cvt_bf16x2(hw[4], hw[5]),
                            cvt_bf16x2(hw[6], hw[7])};
          *reinterpret_cast<u32x4*>(a.dgu + row * (2 * F) + c0) = pg;
          *reinterpret_cast<u32x4*>(a.dgu + row * (2 * F) + F + c0) = pu;
          *reinterpret_cast<u32x4*>(a.hw + row * F + c0) = ph;
        }
        // the row's CG lanes are consecutive: add their sums in a fixed order
#pragma unroll
        for (int o = 1; o < CG; o <<= 1) sum += __shfl_xor(sum, o, 64);
        if (cg == 0 && ok) a.rowdot[(size_t)nt * a.rowdot_stride + row] = sum;
      } else {
        if (ok) {
          f32x4* o = reinterpret_cast<f32x4*>(a.out_f32 + row * D + c0);
          o[0] = d0;
          o[1] = d1;
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------- wgrad

template <int BM_, int BN_, int WM_, int WN_, int STAGES_>
struct WCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_;
  static constexpr int NW = WM * WN, NT = NW * 64;
  static constexpr int FM = BM / WM / 32, FN = BN / WN / 32;
  static constexpr int A_ELEMS = BK * BM, B_ELEMS = BK * BN;
  static constexpr int IPA = A_ELEMS / 8 / NT, IPB = B_ELEMS / 8 / NT, IPS = IPA + IPB;
  static constexpr int CPA = BM / 8, RPA = 64 / CPA, CPB = BN / 8, RPB = 64 / CPB;
  static_assert(FM >= 1 && FN >= 1 && IPA * NT * 8 == A_ELEMS && IPB * NT * 8 == B_ELEMS, "tiling");
  static_assert(CPA >= 8 && CPB >= 8 && BK % (RPA * NW) == 0 && BK % (RPB * NW) == 0, "stage loading");
  static_assert(STAGES >= 2 && IPS * (STAGES - 2) <= 63, "pipeline");
};

template <class C, bool BF16_OUT>
__global__ __launch_bounds__(C::NT) void wgrad_kernel(BwdWgradArgs a) {
  __shared__ __align__(16) bf16_t smem[C::STAGES][C::A_ELEMS + C::B_ELEMS];

  const int mtiles = a.m_total / C::BM, ntiles = a.n_total / C::BN;
  const int nunits = E * mtiles * ntiles;
  const int nper = (nunits + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  const int logical = (blockIdx.x & 7) * nper + slot;
  if (slot >= nper || logical >= nunits) return;
  const int e = logical / (mtiles * ntiles);
  const int rem = logical - e * mtiles * ntiles;
  const int mt = rem / ntiles, nt = rem - mt * ntiles;
  const int r0 = a.offsets[e];
  const int rows = a.offsets[e + 1] - r0;
  const int KT = (rows + BK - 1) / BK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / C::WN, wn = wv % C::WN;

  // both operands K-outer: load j of A fills k-rows (wv*IPA + j)*RPA + lane/CPA, slot lane%CPA (B
  // alike), so a wave's loads of one stage cover KW consecutive k-rows of either operand
  constexpr int KW = C::IPA * C::RPA;
  static_assert(KW == C::IPB * C::RPB, "a wave's k-rows of a stage");
  int ka[C::IPA], oa[C::IPA], kb[C::IPB], ob[C::IPB];
#pragma unroll
  for (int j = 0; j < C::IPA; ++j) {
    ka[j] = (wv * C::IPA + j) * C::RPA + lane / C::CPA;
    oa[j] = mt * C::BM + (((lane % C::CPA) ^ ((ka[j] & 3) << 1)) << 3);
  }
#pragma unroll
  for (int j = 0; j < C::IPB; ++j) {
    kb[j] = (wv * C::IPB + j) * C::RPB + lane / C::CPB;
    ob[j] = nt * C::BN + (((lane % C::CPB) ^ ((kb[j] & 3) << 1)) << 3);
  }
  // a gathered operand reads row rows_x[r0 + k] for the expert's row k; the KW ids a wave needs
  // for a stage come from one scalar load of the table (read through the constant address space,
  // so the load is counted by lgkmcnt and leaves the vmcnt accounting of the LDS-DMA ring alone),
  // fetched a stage before they are used.  The table is padded past its last row, so the ids of a
  // stage's rows beyond the expert's count can be read (and are not used).
  const bool gather = a.a_rows != nullptr || a.b_rows != nullptr;
  const auto gtab = as_const(a.a_rows ? a.a_rows : a.b_rows);
  auto load_ids = [&](int kt, int (&ids)[KW]) {
    const int base = __builtin_amdgcn_readfirstlane(r0 + kt * BK + wv * KW);
#pragma unroll
    for (int i = 0; i < KW; ++i) ids[i] = gtab[base + i];
  };
  // the id of the k-row that load j of a lane reads (RP rows per load, lane / CP the row)
  auto pick = [&](const int (&ids)[KW], int j, auto rp_tag, int cp) __attribute__((always_inline)) {
    constexpr int RP = decltype(rp_tag)::value;
    int v = ids[j * RP];
#pragma unroll
    for (int q = 1; q < RP; ++q) v = lane / cp == q ? ids[j * RP + q] : v;
    return v;
  };
  auto issue = [&](int kt, int sl, int j0, int j1, const int (&ids)[KW]) {
#pragma unroll
    for (int j = 0; j < C::IPS; ++j) {
      if (j < j0 || j >= j1) continue;
      if (j < C::IPA) {
        const int k = kt * BK + ka[j];   // rows past the expert's count read zeros
        const int srow = a.a_rows ? pick(ids, j, std::integral_constant<int, C::RPA>{}, C::CPA) : r0 + k;
        const bf16_t* src = k < rows ? a.a + (size_t)srow * a.lda + oa[j] : a.zero + (oa[j] - mt * C::BM);
        __builtin_amdgcn_global_load_lds(GPTR(src), LPTR(&smem[sl][(wv * C::IPA + j) * C::RPA * C::BM]), 16, 0, 0);
      } else {
        const int jb = j - C::IPA;
        const int k = kt * BK + kb[jb];
        const int srow = a.b_rows ? pick(ids, jb, std::integral_constant<int, C::RPB>{}, C::CPB) : r0 + k;
        const bf16_t* src = k < rows ? a.b + (size_t)srow * a.ldb + ob[jb] : a.zero + (ob[jb] - nt * C::BN);
        __builtin_amdgcn_global_load_lds(GPTR(src),
                                         LPTR(&smem[sl][C::A_ELEMS + (wv * C::IPB + jb) * C::RPB * C::BN]), 16, 0, 0);
      }
    }
  };

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // idn: ids of the next stage to issue; idf: of the one after it.  The first two stages' ids are
  // waited for here, once, so that inside the loop only the one-stage-ahead load is in flight
  static_assert(C::STAGES == 2, "the id prefetch assumes a two-stage ring");
  int idn[KW] = {}, idf[KW] = {};
  if (KT > 0) {
    if (gather) {
      load_ids(0, idf);
      if (KT > 1) load_ids(1, idn);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt unconstrained
    }
    issue(0, 0, 0, C::IPS, idf);
  }
  constexpr int NKK = BK / 16;
  for (int kt = 0; kt < KT; ++kt) {
    if (gather && kt + C::STAGES < KT) load_ids(kt + C::STAGES, idf);
    wait_stage_b<C::STAGES - 2, C::IPS>(min(C::STAGES - 2, KT - 1 - kt));
    const bool more = kt + C::STAGES - 1 < KT;
    const int next_slot = (kt + C::STAGES - 1) % C::STAGES;
    const bf16_t* As = smem[kt % C::STAGES];
    const bf16_t* Bs = As + C::A_ELEMS;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (more) issue(kt + C::STAGES - 1, next_slot, kk * C::IPS / NKK, (kk + 1) * C::IPS / NKK, idn);
      bf16x8 af[C::FM], bfr[C::FN];
      static_assert(C::FM % 2 == 0 && C::FN % 2 == 0, "operands are read in pairs");
#pragma unroll
      for (int i = 0; i < C::FM; i += 2)
        frag_kout2<C::BM>(As, kk, wm * (C::BM / C::WM) + i * 32, wm * (C::BM / C::WM) + i * 32 + 32, lane, af[i],
                          af[i + 1]);
#pragma unroll
      for (int j = 0; j < C::FN; j += 2)
        frag_kout2<C::BN>(Bs, kk, wn * (C::BN / C::WN) + j * 32, wn * (C::BN / C::WN) + j * 32 + 32, lane, bfr[j],
                          bfr[j + 1]);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < KW; ++i) idn[i] = idf[i];
  }

  // output row m (of m_total) goes to out0 below m_split, out1 above; the gradients are not read
  // again here, so the stores are non-temporal.  fp32: each fragment value straight from its lane
  // (staging the tile through LDS for 16-byte stores measured no faster)
  const int m_base = mt * C::BM + wm * (C::BM / C::WM);
  const int n_base = nt * C::BN + wn * (C::BN / C::WN);
  if constexpr (!BF16_OUT) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m_base + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
          const int n = n_base + j * 32 + (lane & 31);
          float* o = m < a.m_split ? static_cast<float*>(a.out0) + (size_t)e * a.out_stride + (size_t)m * a.n_total
                                   : static_cast<float*>(a.out1) + (size_t)e * a.out_stride +
                                         (size_t)(m - a.m_split) * a.n_total;
          __builtin_nontemporal_store(acc[i][j][v], &o[n]);
        }
  } else {
    // bf16: the accumulators go through the drained LDS ring one slice (fragment row i of every
    // wave: WM*32 rows x BN columns, fp32) at a time, and each thread converts 8 consecutive columns
    // of a row into one 16-byte store, consecutive across the lanes (faster than packed pairs stored
    // from the fragments: 0.53 -> 0.49 ms per backward at 256 tokens, 1.77 -> 1.70 at 4096)
    constexpr int SR = C::WM * 32;
    constexpr int CG = C::BN / 8;
    constexpr int RPP = C::NT / CG;
    constexpr int PASSES = SR / RPP;
    static_assert(SR * C::BN * 4 <= C::STAGES * (C::A_ELEMS + C::B_ELEMS) * 2, "a slice fits the LDS ring");
    static_assert(C::NT % CG == 0 && SR % RPP == 0 && SR * C::FM == C::BM, "slice mapping");
    float* S = reinterpret_cast<float*>(&smem[0][0]);
    const int cg = tid % CG, rsub = tid / CG;
    const int n0 = nt * C::BN + cg * 8;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      __syncthreads();   // the ring (or the previous slice) is no longer read
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          S[(wm * 32 + (lane >> 5) * 4 + (v >> 2) * 8 + (v & 3)) * C::BN + wn * (C::BN / C::WN) + j * 32 +
            (lane & 31)] = acc[i][j][v];
      __syncthreads();
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        const int rl = ps * RPP + rsub;   // slice row: wave row block rl / 32, row rl % 32 of fragment row i
        const int m = mt * C::BM + (rl >> 5) * (C::BM / C::WM) + i * 32 + (rl & 31);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&S[rl * C::BN + cg * 8]);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&S[rl * C::BN + cg * 8 + 4]);
        uint16_t* o = static_cast<uint16_t*>(m < a.m_split ? a.out0 : a.out1) + (size_t)e * a.out_stride +
                      (size_t)(m < a.m_split ? m : m - a.m_split) * a.n_total + n0;
        const u32x4 pk = {cvt_bf16x2(d0[0], d0[1]), cvt_bf16x2(d0[2], d0[3]), cvt_bf16x2(d1[0], d1[1]),
                          cvt_bf16x2(d1[2], d1[3])};
        __builtin_nontemporal_store(pk, reinterpret_cast<u32x4*>(o));
      }
    }
  }
}

using DgDH = DCfg<128, 128, 2, 2, 3, EPI_DH>;
using DgDX = DCfg<128, 128, 2, 2, 3, EPI_F32>;
// small batches (an expert's rows fit one 64-row tile): 64x256 tiles on 8 waves, three stages, so
// less of each staged tile is padding rows and more weight bytes are in flight per CU (at 256
// tokens 104 + 65 us against 110 + 73 us for the two products)
using DgDHS = DCfg<64, 256, 2, 4, 3, EPI_DH>;
using DgDXS = DCfg<64, 256, 2, 4, 3, EPI_F32>;
constexpr int DGRAD_SMALL_TOKENS = 320;
// large batches: 256x256 tiles on 8 waves (4% off the backward at 4096 tokens; at 256 tokens, with
// one partly filled row tile per expert, the 128-row tiles are faster)
using DgDHL = DCfg<256, 256, 4, 2, 2, EPI_DH>;
using DgDXL = DCfg<256, 256, 4, 2, 2, EPI_F32>;
// the 128-row tiles keep the lead while experts hold up to about 100 rows (backward 0.729 against
// 0.757 ms at 512 tokens, 0.808 against 0.827 at 768; 0.918 against 0.904 at 1024)
constexpr int DGRAD_LARGE_TOKENS = 768;
// 256x256 tiles on 8 waves: each operand row is re-read half as often as with 128x128 tiles on 4
// waves, and the fewer, larger units also write their fp32 gradients faster (measured 13% off the
// whole backward at both 256 and 4096 tokens)
using WgCfg = WCfg<256, 256, 4, 2, 2>;

}  // namespace

int bwd_tile_rows(int T) {
  return T > DGRAD_LARGE_TOKENS ? DgDHL::BM : T > DGRAD_SMALL_TOKENS ? DgDH::BM : DgDHS::BM;
}

template <class C>
constexpr int dot_parts_of() { return C::ND / C::BN; }
static_assert(dot_parts_of<DgDH>() <= BWD_MAX_DOT_PARTS && dot_parts_of<DgDHS>() <= BWD_MAX_DOT_PARTS &&
              dot_parts_of<DgDHL>() <= BWD_MAX_DOT_PARTS, "row-sum parts");

int bwd_dot_parts(int T) {
  return T > DGRAD_LARGE_TOKENS ? dot_parts_of<DgDHL>() : T > DGRAD_SMALL_TOKENS ? dot_parts_of<DgDH>()
                                                                                : dot_parts_of<DgDHS>();
}

template <class C>
hipError_t launch_dgrad_cfg(const BwdDgradArgs& a, int T, hipStream_t stream) {
  const int grid = (max_row_tiles(T, C::BM) * (C::ND / C::BN) + 7) / 8 * 8;
  hipLaunchKernelGGL(dgrad_kernel<C>, dim3(grid), dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_dgrad(const BwdDgradArgs& a, int T, bool dh, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  static_assert(DgDH::BM == DgDX::BM && DgDHL::BM == DgDXL::BM && DgDHS::BM == DgDXS::BM,
                "both dgrad products share the tile list");
  static_assert(DgDHS::BM >= MIN_TILE_ROWS, "tile lists are sized for MIN_TILE_ROWS");
  if (T > DGRAD_LARGE_TOKENS) return dh ? launch_dgrad_cfg<DgDHL>(a, T, stream) : launch_dgrad_cfg<DgDXL>(a, T, stream);
  if (T > DGRAD_SMALL_TOKENS) return dh ? launch_dgrad_cfg<DgDH>(a, T, stream) : launch_dgrad_cfg<DgDX>(a, T, stream);
  return dh ? launch_dgrad_cfg<DgDHS>(a, T, stream) : launch_dgrad_cfg<DgDXS>(a, T, stream);
}

hipError_t launch_wgrad(const BwdWgradArgs& a, hipStream_t stream) {
  const int units = E * (a.m_total / WgCfg::BM) * (a.n_total / WgCfg::BN);
  const int grid = (units + 7) / 8 * 8;
  if (a.out_bf16)
    hipLaunchKernelGGL((wgrad_kernel<WgCfg, true>), dim3(grid), dim3(WgCfg::NT), 0, stream, a);
  else
    hipLaunchKernelGGL((wgrad_kernel<WgCfg, false>), dim3(grid), dim3(WgCfg::NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace olmoe
