// C ABI of the OLMoE MoE library: argument checks, workspace layout, and the
// launch sequence router -> scan -> permute -> gate/up -> down -> combine on
// the caller's stream.  Declarations and contracts: include/olmoe_moe.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/olmoe_moe.h"
#include "common.hpp"
#include "kernels.hpp"

namespace {

using namespace olmoe;

thread_local std::string g_err;

olmoe_status_t fail(olmoe_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

olmoe_status_t ok() {
  g_err.clear();
  return OLMOE_OK;
}

struct Layout {
  size_t clip, tiles_gu, tiles_dn, planes, partial, ids, probs, lrank, blk_counts, blk_psum, blk_lse2, blk_base,
      offsets, tp_gu, tp_dn, perm, inv, h, y, total;
};

Layout make_layout(int64_t T) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  const size_t rows = 8 * static_cast<size_t>(T);
  const size_t nblk = static_cast<size_t>((T + 15) / 16);
  // first, at offset 0 of every workspace (the backward and expert-choice layouts start with this
  // one): the count of fp16 intermediates stored clipped, zeroed by each call's dispatch kernel
  L.clip = take(4);
  L.offsets = take(65 * 4);
  L.tp_gu = take(65 * 4);
  L.tp_dn = take(65 * 4);
  // sized for the largest possible tile count (+8 spare entries); GEMM workgroups beyond the
  // real count return before reading the list
  const size_t max_tiles = static_cast<size_t>(max_row_tiles(static_cast<int>(T), MIN_TILE_ROWS)) + 8;
  L.tiles_gu = take(max_tiles * 8);
  L.tiles_dn = take(max_tiles * 8);
  L.planes = take(3 * 64 * 2048 * 2);
  L.partial = take(static_cast<size_t>(T) * router_slices(static_cast<int>(T)) * 64 * 8);
  L.ids = take(rows * 4);
  L.probs = take(rows * 4);
  L.lrank = take(rows);
  L.blk_counts = take(nblk * 64 * 4);
  L.blk_psum = take(nblk * 64 * 4);
  L.blk_lse2 = take(nblk * 4);
  L.blk_base = take(nblk * 64 * 4);
  L.perm = take((rows + 64) * 4);   // 64 spare entries: the weight-gradient kernel reads a stage's ids at once
  L.inv = take(rows * 4);
  L.h = take(rows * OLMOE_F * 2);
  L.y = take(rows * OLMOE_D * 2);
  L.total = off;
  return L;
}

// backward workspace: the forward's layout followed by the backward's own buffers
struct BwdLayout {
  Layout f;
  size_t p_all, lse, row_w, gu, dgu, hw, dxr, dlogits, dwr_part, zero, tp_bwd, tiles_bwd, rowdot, total;
};
BwdLayout make_bwd_layout(int64_t T) {
  BwdLayout B{};
  B.f = make_layout(T);
  size_t off = B.f.total;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  const size_t t = static_cast<size_t>(T), rows = 8 * t;
  B.p_all = take(t * OLMOE_E * 4);
  B.lse = take(t * 4);
  B.row_w = take(rows * 4);
  B.gu = take(rows * 2 * OLMOE_F * 4);
  B.dgu = take(rows * 2 * OLMOE_F * 2);
  B.hw = take(rows * OLMOE_F * 2);
  B.dxr = take(rows * OLMOE_D * 4);
  B.dlogits = take(t * OLMOE_E * 4);
  B.dwr_part = take(static_cast<size_t>(bwd_router_splits(static_cast<int>(T))) * OLMOE_E * OLMOE_D * 4);
  B.zero = take(4096);
  B.tp_bwd = take(65 * 4);
  B.tiles_bwd = take((static_cast<size_t>(max_row_tiles(static_cast<int>(T), MIN_TILE_ROWS)) + 8) * 8);
  B.rowdot = take(rows * BWD_MAX_DOT_PARTS * 4);
  B.total = off;
  return B;
}

// expert-choice workspace: the forward layout for 8C "tokens" (64C rows, every expert C of
// them; C = ceil(8T / 64) >= T / 8, so all row buffers and tile lists fit), then its own tables
struct EcLayout {
  Layout f;
  size_t pT, lse, inv_ec, row_w, total;
};
EcLayout make_ec_layout(int64_t T) {
  EcLayout L{};
  const int64_t C = ec_capacity(static_cast<int>(T));
  L.f = make_layout(8 * C);
  size_t off = L.f.total;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  const size_t t = static_cast<size_t>(T);
  L.pT = take(t * OLMOE_E * 4);
  L.lse = take(t * 4);
  L.inv_ec = take(t * OLMOE_E * 4);
  L.row_w = take(static_cast<size_t>(C) * OLMOE_E * 4);
  L.total = off;
  return L;
}

bool misaligned(const void* p, size_t a = 16) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// gfx950 check, cached per device
std::mutex g_dev_mu;
std::vector<int> g_dev_ok;  // -1 unknown, 0 no, 1 yes

olmoe_status_t check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return fail(OLMOE_ENODEVICE, "no HIP device: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_dev_ok.size() <= dev) g_dev_ok.resize(dev + 1, -1);
  if (g_dev_ok[dev] < 0) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return fail(OLMOE_ENODEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    g_dev_ok[dev] = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    if (!g_dev_ok[dev]) return fail(OLMOE_ENODEVICE, "device %d is %s, the library is built for gfx950", dev, p.gcnArchName);
  }
  if (!g_dev_ok[dev]) return fail(OLMOE_ENODEVICE, "current device is not gfx950");
  return OLMOE_OK;
}

// ---------------------------------------------------------------- side streams

// After the dH dgrad, the backward's two weight-gradient GEMMs depend on nothing the dX dgrad
// writes, and the weight gradients are mostly stores of fp32 results while the dgrad is mostly
// MFMA work: the two run on side streams of the calling thread (created once per device, default
// priority, not synchronising with the null stream), forked from the caller's stream after the
// dH dgrad and joined back into it at the end, so the caller's stream still orders all of a
// call's work.  Calls from one thread share its side streams, which serialises their weight
// gradients but keeps each call's order.  The streams live until the process ends.
struct SideStreams {
  hipStream_t s[2] = {nullptr, nullptr};
  hipEvent_t fork = nullptr;
  hipEvent_t join[2] = {nullptr, nullptr};
};
thread_local std::vector<SideStreams> g_side;   // per device, for this thread

hipError_t side_streams(SideStreams** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((int)g_side.size() <= dev) g_side.resize(dev + 1);
  SideStreams& ss = g_side[dev];
  if (!ss.fork) {
    SideStreams n;
    for (int i = 0; i < 2 && e == hipSuccess; ++i) {
      e = hipStreamCreateWithFlags(&n.s[i], hipStreamNonBlocking);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join[i], hipEventDisableTiming);
    }
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
    if (e != hipSuccess) {
      for (int i = 0; i < 2; ++i) {
        if (n.s[i]) (void)hipStreamDestroy(n.s[i]);
        if (n.join[i]) (void)hipEventDestroy(n.join[i]);
      }
      return e;
    }
    ss = n;
  }
  *out = &ss;
  return hipSuccess;
}

// the weight-gradient GEMMs wd and wgu on the side streams, after everything issued on s so far
hipError_t fork_wgrads(const BwdWgradArgs& wd, const BwdWgradArgs& wgu, hipStream_t s, SideStreams& ss) {
  hipError_t e = hipEventRecord(ss.fork, s);
  for (int i = 0; i < 2 && e == hipSuccess; ++i) {
    e = hipStreamWaitEvent(ss.s[i], ss.fork, 0);
    if (e == hipSuccess) e = launch_wgrad(i == 0 ? wd : wgu, ss.s[i]);
    if (e == hipSuccess) e = hipEventRecord(ss.join[i], ss.s[i]);
  }
  return e;
}

// s waits for the side streams' work
hipError_t join_wgrads(hipStream_t s, SideStreams& ss) {
  hipError_t e = hipSuccess;
  for (int i = 0; i < 2 && e == hipSuccess; ++i) e = hipStreamWaitEvent(s, ss.join[i], 0);
  return e;
}

// ---------------------------------------------------------------- stage timing

// router: logits and top-8 selection; dispatch: scan and permutation; then the
// three expert stages
constexpr int N_STAGES = 5;
const char* kStageNames[N_STAGES] = {"router", "dispatch", "gateup", "down", "combine"};

struct TimingState {
  int mask = 0;   // bit i: bracket stage i with events
  int every = 1;  // bracket every n-th call
  long long calls = 0;   // calls seen since the mask or the sampling step was set
  std::vector<std::vector<hipEvent_t>> pending;  // one set of N_STAGES+1 boundary events per call
};
thread_local TimingState g_timing;

// boundary b lies between stage b-1 and stage b; it is recorded when either side is timed
bool boundary_needed(int mask, int b) {
  return (b > 0 && (mask >> (b - 1) & 1)) || (b < N_STAGES && (mask >> b & 1));
}

struct StageRecorder {
  std::vector<hipEvent_t>* ev = nullptr;
  hipStream_t s;
  int next = 0;
  explicit StageRecorder(hipStream_t st) : s(st) {
    if (!g_timing.mask || g_timing.pending.size() >= 65536) return;
    if (g_timing.calls++ % g_timing.every != 0) return;
    g_timing.pending.emplace_back(N_STAGES + 1, nullptr);
    ev = &g_timing.pending.back();
    for (int b = 0; b <= N_STAGES; ++b)
      if (boundary_needed(g_timing.mask, b)) (void)hipEventCreate(&(*ev)[b]);
    record();
  }
  void record() {
    if ((*ev)[next]) (void)hipEventRecord((*ev)[next], s);
    ++next;
  }
  void mark() {
    if (ev && next <= N_STAGES) record();
  }
  void finish() {
    while (ev && next <= N_STAGES) record();
  }
};

olmoe_status_t forward_impl(const void* x, const float* W_router, const void* W_gate, const void* W_up,
                            const void* W_down, int64_t T, void* out, float* hres, void* x_next, float eps,
                            int32_t* route_ids, float* route_probs, int32_t* expert_counts, float* aux_loss,
                            float* z_loss, uint32_t route_flags, uint64_t keep_mask, void* workspace,
                            size_t workspace_bytes, void* stream);

// ---------------------------------------------------------------- library-owned scratch

// The workspace of olmoe_moe_forward_noalloc: one array per GPU, held until the process ends.  In
// host code the name below stands for the array but is not its device address; that address
// comes from hipGetSymbolAddress with the GPU current, once per GPU, and only it is passed on.
__device__ __align__(256) unsigned char scratch[OLMOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // device address of `scratch` per device (null: not looked up)

olmoe_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return fail(OLMOE_ENODEVICE, "no HIP device: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(OLMOE_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return OLMOE_OK;
}

}  // namespace

extern "C" {

int olmoe_abi_version(void) { return OLMOE_ABI_VERSION; }

const char* olmoe_last_error(void) { return g_err.c_str(); }

size_t olmoe_moe_workspace_bytes(int64_t T) {
  if (T < 0 || T > OLMOE_MAX_TOKENS) return 0;
  return make_layout(T).total;
}

olmoe_status_t olmoe_moe_workspace_layout(int64_t T, size_t* perm_off, size_t* inv_off,
                                          size_t* offsets_off) {
  if (T < 0 || T > OLMOE_MAX_TOKENS) return fail(OLMOE_EINVAL, "T=%lld out of range", (long long)T);
  const Layout L = make_layout(T);
  if (perm_off) *perm_off = L.perm;
  if (inv_off) *inv_off = L.inv;
  if (offsets_off) *offsets_off = L.offsets;
  return ok();
}

olmoe_status_t olmoe_moe_forward(const void* x, const float* W_router, const void* W_gate,
                                 const void* W_up, const void* W_down, int64_t T, void* out,
                                 int32_t* route_ids, float* route_probs, int32_t* expert_counts,
                                 float* aux_loss, float* z_loss, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return olmoe_moe_forward_ex(x, W_router, W_gate, W_up, W_down, T, out, route_ids, route_probs,
                              expert_counts, aux_loss, z_loss, 0u, OLMOE_KEEP_ALL, workspace,
                              workspace_bytes, stream);
}

olmoe_status_t olmoe_moe_forward_ex(const void* x, const float* W_router, const void* W_gate,
                                    const void* W_up, const void* W_down, int64_t T, void* out,
                                    int32_t* route_ids, float* route_probs, int32_t* expert_counts,
                                    float* aux_loss, float* z_loss, uint32_t route_flags,
                                    uint64_t keep_mask, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return forward_impl(x, W_router, W_gate, W_up, W_down, T, out, nullptr, nullptr, 0.f, route_ids,
                      route_probs, expert_counts, aux_loss, z_loss, route_flags, keep_mask, workspace,
                      workspace_bytes, stream);
}

olmoe_status_t olmoe_moe_forward_noalloc(const void* x, const float* W_router, const void* W_gate,
                                         const void* W_up, const void* W_down, int64_t T, void* out,
                                         int32_t* route_ids, float* route_probs, int32_t* expert_counts,
                                         float* aux_loss, float* z_loss, void* stream) {
  if (T < 0 || T > OLMOE_NOALLOC_MAX_TOKENS)
    return fail(OLMOE_EINVAL, "T=%lld: the library-owned scratch holds at most %d tokens", (long long)T,
                OLMOE_NOALLOC_MAX_TOKENS);
  const size_t need = make_layout(T).total;
  if (need > OLMOE_NOALLOC_SCRATCH_BYTES)   // a build inconsistency, not a caller error
    return fail(OLMOE_EWORKSPACE, "scratch of %zu bytes below the %zu needed for T=%lld",
                (size_t)OLMOE_NOALLOC_SCRATCH_BYTES, need, (long long)T);
  olmoe_status_t st = check_device();
  if (st != OLMOE_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != OLMOE_OK) return st;
  return forward_impl(x, W_router, W_gate, W_up, W_down, T, out, nullptr, nullptr, 0.f, route_ids, route_probs,
                      expert_counts, aux_loss, z_loss, 0u, OLMOE_KEEP_ALL, ws, OLMOE_NOALLOC_SCRATCH_BYTES, stream);
}

olmoe_status_t olmoe_moe_forward_residual(const void* x, const float* W_router, const void* W_gate,
                                          const void* W_up, const void* W_down, int64_t T, float* h,
                                          void* x_next, float eps, int32_t* route_ids, float* route_probs,
                                          int32_t* expert_counts, float* aux_loss, float* z_loss,
                                          uint32_t route_flags, uint64_t keep_mask, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  if (T > 0 && !h) return fail(OLMOE_EINVAL, "h is NULL");
  return forward_impl(x, W_router, W_gate, W_up, W_down, T, nullptr, h, x_next, eps, route_ids,
                      route_probs, expert_counts, aux_loss, z_loss, route_flags, keep_mask, workspace,
                      workspace_bytes, stream);
}

}  // extern "C"

namespace {

// the layer; out (bf16) for the plain forward, or h (+ x_next) for the residual epilogue
olmoe_status_t forward_impl(const void* x, const float* W_router, const void* W_gate, const void* W_up,
                            const void* W_down, int64_t T, void* out, float* hres, void* x_next, float eps,
                            int32_t* route_ids, float* route_probs, int32_t* expert_counts, float* aux_loss,
                            float* z_loss, uint32_t route_flags, uint64_t keep_mask, void* workspace,
                            size_t workspace_bytes, void* stream) {
  const bool residual = hres != nullptr;
  // ---- host-side checks; nothing is enqueued unless all pass
  if (route_flags & ~static_cast<uint32_t>(OLMOE_ROUTE_RENORMALIZE))
    return fail(OLMOE_EINVAL, "unknown route flags 0x%x", route_flags);
  if (__builtin_popcountll(keep_mask) < OLMOE_K)
    return fail(OLMOE_EINVAL, "keep_mask keeps %d experts, at least %d needed", __builtin_popcountll(keep_mask),
                OLMOE_K);
  if (T < 0 || T > OLMOE_MAX_TOKENS)
    return fail(OLMOE_EINVAL, "T=%lld out of range [0, %lld]", (long long)T, (long long)OLMOE_MAX_TOKENS);
  if (!W_router || !W_gate || !W_up || !W_down)
    return fail(OLMOE_EINVAL, "a weight pointer is NULL");
  if (T > 0 && (!x || (!residual && !out))) return fail(OLMOE_EINVAL, "x or out is NULL");
  const void* ptrs[] = {x, W_router, W_gate, W_up, W_down, out, route_ids, route_probs, expert_counts, hres, x_next};
  const char* names[] = {"x", "W_router", "W_gate", "W_up", "W_down", "out", "route_ids", "route_probs",
                         "expert_counts", "h", "x_next"};
  for (int i = 0; i < 11; ++i)
    if (ptrs[i] && misaligned(ptrs[i])) return fail(OLMOE_EINVAL, "%s is not 16-byte aligned", names[i]);
  if ((aux_loss && misaligned(aux_loss, 4)) || (z_loss && misaligned(z_loss, 4)))
    return fail(OLMOE_EINVAL, "aux_loss / z_loss not 4-byte aligned");
  if (residual && x_next && !(eps > 0.f)) return fail(OLMOE_EINVAL, "eps must be > 0");
  const size_t act = static_cast<size_t>(T) * OLMOE_D * 2;
  const size_t wexp = static_cast<size_t>(OLMOE_E) * OLMOE_F * OLMOE_D * 2;
  const size_t wr_bytes = (size_t)OLMOE_E * OLMOE_D * 4;
  // a written buffer may not overlap an input (x_next may be x itself: x is last read before
  // the epilogue runs, in stream order)
  auto hits_inputs = [&](const void* p, size_t n, bool allow_x) {
    return (!(allow_x && p == x) && overlaps(p, n, x, act)) || overlaps(p, n, W_router, wr_bytes) ||
           overlaps(p, n, W_gate, wexp) || overlaps(p, n, W_up, wexp) || overlaps(p, n, W_down, wexp);
  };
  if (hits_inputs(out, act, false)) return fail(OLMOE_EINVAL, "out overlaps an input");
  if (hits_inputs(hres, act * 2, false)) return fail(OLMOE_EINVAL, "h overlaps an input");
  if (hits_inputs(x_next, act, true)) return fail(OLMOE_EINVAL, "x_next overlaps an input other than x");
  if (overlaps(x_next, act, hres, act * 2)) return fail(OLMOE_EINVAL, "x_next overlaps h");
  const Layout L = make_layout(T);
  if (!workspace) return fail(OLMOE_EWORKSPACE, "workspace is NULL");
  if (misaligned(workspace, 256)) return fail(OLMOE_EINVAL, "workspace is not 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(OLMOE_EWORKSPACE, "workspace has %zu bytes, %zu needed for T=%lld", workspace_bytes, L.total,
                (long long)T);
  if (overlaps(out, act, workspace, L.total) || overlaps(hres, act * 2, workspace, L.total) ||
      overlaps(x_next, act, workspace, L.total))
    return fail(OLMOE_EINVAL, "an output overlaps the workspace");
  // the optional routing outputs: the kernels read ids and probs back while out / h are written,
  // so none of them may share bytes with an input, the workspace, a main output or each other
  {
    const size_t pairs = static_cast<size_t>(T) * OLMOE_K * 4;
    const void* ro[] = {route_ids, route_probs, expert_counts, aux_loss, z_loss};
    const size_t ro_n[] = {pairs, pairs, OLMOE_E * 4, 4, 4};
    const char* ro_name[] = {"route_ids", "route_probs", "expert_counts", "aux_loss", "z_loss"};
    for (int i = 0; i < 5; ++i) {
      if (!ro[i]) continue;
      if (hits_inputs(ro[i], ro_n[i], false)) return fail(OLMOE_EINVAL, "%s overlaps an input", ro_name[i]);
      if (overlaps(ro[i], ro_n[i], workspace, L.total))
        return fail(OLMOE_EINVAL, "%s overlaps the workspace", ro_name[i]);
      if (overlaps(ro[i], ro_n[i], out, act) || overlaps(ro[i], ro_n[i], hres, act * 2) ||
          overlaps(ro[i], ro_n[i], x_next, act))
        return fail(OLMOE_EINVAL, "%s overlaps out, h or x_next", ro_name[i]);
      for (int q = i + 1; q < 5; ++q)
        if (overlaps(ro[i], ro_n[i], ro[q], ro_n[q]))
          return fail(OLMOE_EINVAL, "%s overlaps %s", ro_name[i], ro_name[q]);
    }
  }
  olmoe_status_t st = check_device();
  if (st != OLMOE_OK) return st;

  // ---- launches
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int Ti = static_cast<int>(T);
  int32_t* ids = route_ids ? route_ids : reinterpret_cast<int32_t*>(ws + L.ids);
  float* probs = route_probs ? route_probs : reinterpret_cast<float*>(ws + L.probs);
  const GemmPlan plan = plan_gemm(Ti);
  StageRecorder rec(s);
  hipError_t he = hipSuccess;

  RouterArgs ra{static_cast<const uint16_t*>(x), W_router, Ti, reinterpret_cast<float2*>(ws + L.partial),
                reinterpret_cast<uint16_t*>(ws + L.planes)};
  SelectArgs se{reinterpret_cast<const float2*>(ws + L.partial), Ti, ids, probs,
                reinterpret_cast<uint8_t*>(ws + L.lrank), reinterpret_cast<int32_t*>(ws + L.blk_counts),
                reinterpret_cast<float*>(ws + L.blk_psum), reinterpret_cast<float*>(ws + L.blk_lse2),
                keep_mask, (route_flags & OLMOE_ROUTE_RENORMALIZE) ? 1 : 0};
  ScanArgs sa{Ti,
              reinterpret_cast<const int32_t*>(ws + L.blk_counts),
              reinterpret_cast<const float*>(ws + L.blk_psum),
              reinterpret_cast<const float*>(ws + L.blk_lse2),
              reinterpret_cast<int32_t*>(ws + L.blk_base),
              reinterpret_cast<int32_t*>(ws + L.offsets),
              reinterpret_cast<int32_t*>(ws + L.tp_gu), reinterpret_cast<int2*>(ws + L.tiles_gu), plan.bm_gu,
              reinterpret_cast<int32_t*>(ws + L.tp_dn), reinterpret_cast<int2*>(ws + L.tiles_dn), plan.bm_dn,
              expert_counts, aux_loss, z_loss, reinterpret_cast<int32_t*>(ws + L.clip)};
  PermuteArgs pa{Ti, ids, reinterpret_cast<const uint8_t*>(ws + L.lrank),
                 reinterpret_cast<const int32_t*>(ws + L.blk_base), reinterpret_cast<int32_t*>(ws + L.perm),
                 reinterpret_cast<int32_t*>(ws + L.inv)};
  he = launch_router_partial(ra, s);
  if (he == hipSuccess) he = launch_router_select(se, s);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "router launch: %s", hipGetErrorString(he));
  rec.mark();
  if (Ti <= SMALL_TOKENS) {
    he = launch_scan_permute(sa, pa, s);   // T == 0 included: zero counts and losses
  } else {
    he = launch_scan(sa, s);
    if (he == hipSuccess) he = launch_permute(pa, s);
  }
  if (he != hipSuccess) return fail(OLMOE_EHIP, "dispatch launch: %s", hipGetErrorString(he));
  rec.mark();
  if (Ti == 0) {
    rec.finish();
    return ok();
  }
  GemmArgs ga{Ti,
              static_cast<const uint16_t*>(x),
              static_cast<const uint16_t*>(W_gate),
              static_cast<const uint16_t*>(W_up),
              static_cast<const uint16_t*>(W_down),
              reinterpret_cast<const int32_t*>(ws + L.perm),
              reinterpret_cast<const int32_t*>(ws + L.offsets),
              reinterpret_cast<const int32_t*>(ws + L.tp_gu),
              reinterpret_cast<const int32_t*>(ws + L.tp_dn),
              reinterpret_cast<const int2*>(ws + L.tiles_gu),
              reinterpret_cast<const int2*>(ws + L.tiles_dn),
              reinterpret_cast<uint16_t*>(ws + L.h),
              reinterpret_cast<uint16_t*>(ws + L.y),
              nullptr,
              reinterpret_cast<int32_t*>(ws + L.clip)};
  he = launch_gateup(ga, plan, s);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "gate/up launch: %s", hipGetErrorString(he));
  rec.mark();
  he = launch_down(ga, plan, s);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "down launch: %s", hipGetErrorString(he));
  rec.mark();
  CombineArgs ca{Ti,    reinterpret_cast<const uint16_t*>(ws + L.y), reinterpret_cast<const int32_t*>(ws + L.inv),
                 probs, static_cast<uint16_t*>(out), hres, static_cast<uint16_t*>(x_next), eps};
  he = launch_combine(ca, s);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "combine launch: %s", hipGetErrorString(he));
  rec.mark();
  return ok();
}

// argument checks shared by the backward entry points (T already range-checked)
olmoe_status_t backward_checks(const void* x, const float* W_router, const void* W_gate, const void* W_up,
                               const void* W_down, int64_t T, const void* dout, float g_aux, float g_z, float* dx,
                               float* dW_router, void* dW_gate, void* dW_up, void* dW_down, void* workspace,
                               size_t workspace_bytes, size_t needed, size_t wgrad_elem = 4) {
  if (!W_router || !W_gate || !W_up || !W_down) return fail(OLMOE_EINVAL, "a weight pointer is NULL");
  if (!dW_router || !dW_gate || !dW_up || !dW_down) return fail(OLMOE_EINVAL, "a weight-gradient pointer is NULL");
  if (T > 0 && (!x || !dout || !dx)) return fail(OLMOE_EINVAL, "x, dout or dx is NULL");
  const void* ptrs[] = {x, W_router, W_gate, W_up, W_down, dout, dx, dW_router, dW_gate, dW_up, dW_down};
  const char* names[] = {"x", "W_router", "W_gate", "W_up", "W_down", "dout", "dx", "dW_router", "dW_gate",
                         "dW_up", "dW_down"};
  for (int i = 0; i < 11; ++i)
    if (ptrs[i] && misaligned(ptrs[i])) return fail(OLMOE_EINVAL, "%s is not 16-byte aligned", names[i]);
  if (!std::isfinite(g_aux) || !std::isfinite(g_z)) return fail(OLMOE_EINVAL, "g_aux / g_z not finite");
  const size_t act = static_cast<size_t>(T) * OLMOE_D * 2;
  const size_t wexp = static_cast<size_t>(OLMOE_E) * OLMOE_F * OLMOE_D * 2;
  const size_t wr_bytes = (size_t)OLMOE_E * OLMOE_D * 4;
  const void* ins[] = {x, dout, W_router, W_gate, W_up, W_down};
  const size_t in_n[] = {act, act, wr_bytes, wexp, wexp, wexp};
  void* outs[] = {dx, dW_router, dW_gate, dW_up, dW_down};
  const size_t wg = wexp / 2 * wgrad_elem;
  const size_t out_n[] = {act * 2, wr_bytes, wg, wg, wg};
  if (!workspace) return fail(OLMOE_EWORKSPACE, "workspace is NULL");
  if (misaligned(workspace, 256)) return fail(OLMOE_EINVAL, "workspace is not 256-byte aligned");
  if (workspace_bytes < needed)
    return fail(OLMOE_EWORKSPACE, "workspace has %zu bytes, %zu needed for T=%lld", workspace_bytes, needed,
                (long long)T);
  for (int o = 0; o < 5; ++o) {
    for (int i = 0; i < 6; ++i)
      if (overlaps(outs[o], out_n[o], ins[i], in_n[i])) return fail(OLMOE_EINVAL, "an output overlaps an input");
    for (int q = o + 1; q < 5; ++q)
      if (overlaps(outs[o], out_n[o], outs[q], out_n[q])) return fail(OLMOE_EINVAL, "two outputs overlap");
    if (overlaps(outs[o], out_n[o], workspace, needed)) return fail(OLMOE_EINVAL, "an output overlaps the workspace");
  }
  return check_device();
}

// the backward's forward part (token choice, default router): routing, the gate/up GEMM keeping
// the fp32 pre-activations G | U, and (with_y: for the layer's output) the down GEMM, all into the
// backward layout B.  The gradients need no expert outputs: the routing weights' gradient comes
// from the dH~ dgrad.
olmoe_status_t bwd_forward_state(const void* x, const float* W_router, const void* W_gate, const void* W_up,
                                 const void* W_down, int Ti, char* ws, const BwdLayout& B, int32_t* expert_counts,
                                 float* aux_loss, float* z_loss, bool with_y, hipStream_t s) {
  const Layout& L = B.f;
  const GemmPlan plan = plan_gemm(Ti);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + L.ids);
  float* probs = reinterpret_cast<float*>(ws + L.probs);
  RouterArgs ra{static_cast<const uint16_t*>(x), W_router, Ti, reinterpret_cast<float2*>(ws + L.partial),
                reinterpret_cast<uint16_t*>(ws + L.planes)};
  SelectArgs se{reinterpret_cast<const float2*>(ws + L.partial), Ti, ids, probs,
                reinterpret_cast<uint8_t*>(ws + L.lrank), reinterpret_cast<int32_t*>(ws + L.blk_counts),
                reinterpret_cast<float*>(ws + L.blk_psum), reinterpret_cast<float*>(ws + L.blk_lse2),
                OLMOE_KEEP_ALL, 0, reinterpret_cast<float*>(ws + B.p_all), reinterpret_cast<float*>(ws + B.lse)};
  ScanArgs sa{Ti,
              reinterpret_cast<const int32_t*>(ws + L.blk_counts),
              reinterpret_cast<const float*>(ws + L.blk_psum),
              reinterpret_cast<const float*>(ws + L.blk_lse2),
              reinterpret_cast<int32_t*>(ws + L.blk_base),
              reinterpret_cast<int32_t*>(ws + L.offsets),
              reinterpret_cast<int32_t*>(ws + L.tp_gu), reinterpret_cast<int2*>(ws + L.tiles_gu), plan.bm_gu,
              reinterpret_cast<int32_t*>(ws + L.tp_dn), reinterpret_cast<int2*>(ws + L.tiles_dn), plan.bm_dn,
              expert_counts, aux_loss, z_loss, reinterpret_cast<int32_t*>(ws + L.clip)};
  PermuteArgs pa{Ti, ids, reinterpret_cast<const uint8_t*>(ws + L.lrank),
                 reinterpret_cast<const int32_t*>(ws + L.blk_base), reinterpret_cast<int32_t*>(ws + L.perm),
                 reinterpret_cast<int32_t*>(ws + L.inv), probs, reinterpret_cast<float*>(ws + B.row_w)};
  hipError_t he = launch_router_partial(ra, s);
  if (he == hipSuccess) he = launch_router_select(se, s);
  if (he == hipSuccess) {
    if (Ti <= SMALL_TOKENS) {
      he = launch_scan_permute(sa, pa, s);
    } else {
      he = launch_scan(sa, s);
      if (he == hipSuccess) he = launch_permute(pa, s);
    }
  }
  if (he != hipSuccess) return fail(OLMOE_EHIP, "routing launch: %s", hipGetErrorString(he));
  const int32_t* perm = reinterpret_cast<const int32_t*>(ws + L.perm);
  const int32_t* offsets = reinterpret_cast<const int32_t*>(ws + L.offsets);
  if (Ti > 0) {
    GemmArgs ga{Ti,
                static_cast<const uint16_t*>(x),
                static_cast<const uint16_t*>(W_gate),
                static_cast<const uint16_t*>(W_up),
                static_cast<const uint16_t*>(W_down),
                perm, offsets,
                reinterpret_cast<const int32_t*>(ws + L.tp_gu),
                reinterpret_cast<const int32_t*>(ws + L.tp_dn),
                reinterpret_cast<const int2*>(ws + L.tiles_gu),
                reinterpret_cast<const int2*>(ws + L.tiles_dn),
                reinterpret_cast<uint16_t*>(ws + L.h),
                reinterpret_cast<uint16_t*>(ws + L.y),
                reinterpret_cast<float*>(ws + B.gu),
                reinterpret_cast<int32_t*>(ws + L.clip)};
    he = launch_gateup(ga, plan, s);
    if (he == hipSuccess && with_y) he = launch_down(ga, plan, s);
    if (he != hipSuccess) return fail(OLMOE_EHIP, "forward GEMM launch: %s", hipGetErrorString(he));
  }
  return OLMOE_OK;
}

// the gradients from the state bwd_forward_state left in B
olmoe_status_t bwd_gradients(const void* x, const float* W_router, const void* W_gate, const void* W_up,
                             const void* W_down, int Ti, const void* dout, float g_aux, float g_z, float* dx,
                             float* dW_router, void* dW_gate, void* dW_up, void* dW_down, char* ws,
                             const BwdLayout& B, hipStream_t s, bool grad_bf16 = false) {
  const Layout& L = B.f;
  int32_t* ids = reinterpret_cast<int32_t*>(ws + L.ids);
  const int32_t* perm = reinterpret_cast<const int32_t*>(ws + L.perm);
  const int32_t* offsets = reinterpret_cast<const int32_t*>(ws + L.offsets);
  hipError_t he = hipSuccess;
  BwdSmallArgs ba{Ti, static_cast<const uint16_t*>(x), W_router, ids,
                  reinterpret_cast<const float*>(ws + B.p_all), reinterpret_cast<const float*>(ws + B.lse),
                  offsets, perm, reinterpret_cast<const int32_t*>(ws + L.inv),
                  reinterpret_cast<const float*>(ws + B.rowdot), g_aux, g_z,
                  reinterpret_cast<float*>(ws + B.dlogits), reinterpret_cast<const float*>(ws + B.dxr), dx,
                  reinterpret_cast<float*>(ws + B.dwr_part), dW_router, reinterpret_cast<uint16_t*>(ws + B.zero),
                  reinterpret_cast<int32_t*>(ws + B.tp_bwd), reinterpret_cast<int2*>(ws + B.tiles_bwd)};
  ba.dot_parts = bwd_dot_parts(Ti);
  he = launch_bwd_prepare(ba, s);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "backward preparation launch: %s", hipGetErrorString(he));
  const uint16_t* dgu = reinterpret_cast<const uint16_t*>(ws + B.dgu);
  // dout and x rows are read through perm (expert order -> token) by the kernels that use them
  BwdWgradArgs wd{static_cast<const uint16_t*>(dout), OLMOE_D, reinterpret_cast<const uint16_t*>(ws + B.hw),
                  OLMOE_F, offsets, reinterpret_cast<const uint16_t*>(ws + B.zero), OLMOE_D, OLMOE_F, dW_down, dW_down,
                  OLMOE_D, (long)OLMOE_D * OLMOE_F, perm, nullptr, grad_bf16};
  BwdWgradArgs wgu{dgu, 2 * OLMOE_F, static_cast<const uint16_t*>(x), OLMOE_D, offsets,
                   reinterpret_cast<const uint16_t*>(ws + B.zero), 2 * OLMOE_F, OLMOE_D, dW_gate, dW_up, OLMOE_F,
                   (long)OLMOE_F * OLMOE_D, nullptr, perm, grad_bf16};
  SideStreams* ss = nullptr;
  he = side_streams(&ss);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "side streams: %s", hipGetErrorString(he));
  if (Ti > 0) {
    BwdDgradArgs dh{static_cast<const uint16_t*>(dout), perm, static_cast<const uint16_t*>(W_down),
                    nullptr, OLMOE_F, (long)OLMOE_D * OLMOE_F, 2 * OLMOE_F,
                    reinterpret_cast<const int32_t*>(ws + B.tp_bwd) + OLMOE_E,
                    reinterpret_cast<const int2*>(ws + B.tiles_bwd),
                    reinterpret_cast<const float*>(ws + B.row_w), reinterpret_cast<const float*>(ws + B.gu),
                    reinterpret_cast<uint16_t*>(ws + B.dgu), reinterpret_cast<uint16_t*>(ws + B.hw), nullptr,
                    reinterpret_cast<float*>(ws + B.rowdot), K * Ti};
    BwdDgradArgs dxa{dgu, nullptr, static_cast<const uint16_t*>(W_gate), static_cast<const uint16_t*>(W_up),
                     OLMOE_D, (long)OLMOE_F * OLMOE_D, OLMOE_F,
                     reinterpret_cast<const int32_t*>(ws + B.tp_bwd) + OLMOE_E,
                     reinterpret_cast<const int2*>(ws + B.tiles_bwd), nullptr, nullptr, nullptr, nullptr,
                     reinterpret_cast<float*>(ws + B.dxr)};
    he = launch_dgrad(dh, Ti, true, s);
    if (he == hipSuccess) he = fork_wgrads(wd, wgu, s, *ss);   // they need dH's outputs only
    if (he == hipSuccess) he = launch_bwd_router(ba, s);        // dlogits from dH's row sums
    if (he == hipSuccess) he = launch_dgrad(dxa, Ti, false, s);
    if (he != hipSuccess) return fail(OLMOE_EHIP, "gradient launch: %s", hipGetErrorString(he));
  } else {
    he = fork_wgrads(wd, wgu, s, *ss);
    if (he != hipSuccess) return fail(OLMOE_EHIP, "weight-gradient launch: %s", hipGetErrorString(he));
  }
  he = launch_bwd_finish(ba, s);
  if (he == hipSuccess) he = join_wgrads(s, *ss);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "router-gradient launch: %s", hipGetErrorString(he));
  return ok();
}

// expert-choice backward workspace: the expert-choice forward layout, then the backward's buffers
// for its 64C rows
struct EcBwdLayout {
  EcLayout c;
  size_t p_all, gu, dgu, hw, dxr, dlogits, dwr_part, zero, tp_bwd, tiles_bwd, rowdot, total;
};
EcBwdLayout make_ec_bwd_layout(int64_t T) {
  EcBwdLayout B{};
  B.c = make_ec_layout(T);
  size_t off = B.c.total;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  const int C = ec_capacity(static_cast<int>(T));
  const size_t t = static_cast<size_t>(T), rows = static_cast<size_t>(OLMOE_E) * C;
  B.p_all = take(t * OLMOE_E * 4);
  B.gu = take(rows * 2 * OLMOE_F * 4);
  B.dgu = take(rows * 2 * OLMOE_F * 2);
  B.hw = take(rows * OLMOE_F * 2);
  B.dxr = take(rows * OLMOE_D * 4);
  B.dlogits = take(t * OLMOE_E * 4);
  B.dwr_part = take(static_cast<size_t>(bwd_router_splits(static_cast<int>(T))) * OLMOE_E * OLMOE_D * 4);
  B.zero = take(4096);
  B.tp_bwd = take(65 * 4);
  B.tiles_bwd = take((static_cast<size_t>(max_row_tiles(8 * C, MIN_TILE_ROWS)) + 8) * 8);
  B.rowdot = take(rows * BWD_MAX_DOT_PARTS * 4);
  B.total = off;
  return B;
}

// the expert-choice backward's forward part: routing, the gate/up GEMM keeping G | U, and (with_y)
// the down GEMM, into the layout B; the selection and loss outputs are optional
olmoe_status_t ec_bwd_forward_state(const void* x, const float* W_router, const void* W_gate, const void* W_up,
                                    const void* W_down, int Ti, char* ws, const EcBwdLayout& B,
                                    int32_t* choice_tokens, float* choice_probs, float* aux_loss, float* z_loss,
                                    bool with_y, hipStream_t s) {
  const EcLayout& L = B.c;
  const int C = ec_capacity(Ti);
  const int Teff = 8 * C;
  const GemmPlan plan = plan_gemm(Teff);
  EcArgs ea{};
  ea.T = Ti;
  ea.C = C;
  ea.partial = reinterpret_cast<const float2*>(ws + L.f.partial);
  ea.pT = reinterpret_cast<float*>(ws + L.pT);
  ea.lse = reinterpret_cast<float*>(ws + L.lse);
  ea.inv_ec = reinterpret_cast<int32_t*>(ws + L.inv_ec);
  ea.perm = reinterpret_cast<int32_t*>(ws + L.f.perm);
  ea.row_w = reinterpret_cast<float*>(ws + L.row_w);
  ea.blk_psum = reinterpret_cast<float*>(ws + L.f.blk_psum);
  ea.blk_lse2 = reinterpret_cast<float*>(ws + L.f.blk_lse2);
  ea.offsets = reinterpret_cast<int32_t*>(ws + L.f.offsets);
  ea.tile_prefix_gu = reinterpret_cast<int32_t*>(ws + L.f.tp_gu);
  ea.tiles_gu = reinterpret_cast<int2*>(ws + L.f.tiles_gu);
  ea.bm_gu = plan.bm_gu;
  ea.tile_prefix_dn = reinterpret_cast<int32_t*>(ws + L.f.tp_dn);
  ea.tiles_dn = reinterpret_cast<int2*>(ws + L.f.tiles_dn);
  ea.bm_dn = plan.bm_dn;
  ea.p_all = reinterpret_cast<float*>(ws + B.p_all);
  ea.choice_tokens = choice_tokens;
  ea.choice_probs = choice_probs;
  ea.aux_loss = aux_loss;
  ea.z_loss = z_loss;
  ea.clip = reinterpret_cast<int32_t*>(ws + L.f.clip);
  hipError_t he = hipSuccess;
  if (Ti > 0) {
    RouterArgs ra{static_cast<const uint16_t*>(x), W_router, Ti, reinterpret_cast<float2*>(ws + L.f.partial),
                  reinterpret_cast<uint16_t*>(ws + L.f.planes)};
    he = launch_router_partial(ra, s);
    if (he == hipSuccess) he = launch_ec_softmax(ea, s);
  }
  if (he == hipSuccess) he = launch_ec_choose(ea, s);   // T == 0: zero offsets for the weight gradients
  if (he != hipSuccess) return fail(OLMOE_EHIP, "routing launch: %s", hipGetErrorString(he));
  const int32_t* perm = reinterpret_cast<const int32_t*>(ws + L.f.perm);
  const int32_t* offsets = reinterpret_cast<const int32_t*>(ws + L.f.offsets);
  if (Ti > 0) {
    GemmArgs ga{Teff,
                static_cast<const uint16_t*>(x),
                static_cast<const uint16_t*>(W_gate),
                static_cast<const uint16_t*>(W_up),
                static_cast<const uint16_t*>(W_down),
                perm, offsets,
                reinterpret_cast<const int32_t*>(ws + L.f.tp_gu),
                reinterpret_cast<const int32_t*>(ws + L.f.tp_dn),
                reinterpret_cast<const int2*>(ws + L.f.tiles_gu),
                reinterpret_cast<const int2*>(ws + L.f.tiles_dn),
                reinterpret_cast<uint16_t*>(ws + L.f.h),
                reinterpret_cast<uint16_t*>(ws + L.f.y),
                reinterpret_cast<float*>(ws + B.gu),
                reinterpret_cast<int32_t*>(ws + L.f.clip)};
    he = launch_gateup(ga, plan, s);
    if (he == hipSuccess && with_y) he = launch_down(ga, plan, s);
    if (he != hipSuccess) return fail(OLMOE_EHIP, "forward GEMM launch: %s", hipGetErrorString(he));
  }
  return OLMOE_OK;
}

// the expert-choice gradients from the state ec_bwd_forward_state left in B
olmoe_status_t ec_bwd_gradients(const void* x, const float* W_router, const void* W_gate, const void* W_up,
                                const void* W_down, int Ti, const void* dout, float g_aux, float g_z, float* dx,
                                float* dW_router, void* dW_gate, void* dW_up, void* dW_down, char* ws,
                                const EcBwdLayout& B, hipStream_t s, bool grad_bf16 = false) {
  const EcLayout& L = B.c;
  const int C = ec_capacity(Ti);
  const int Teff = 8 * C;
  const int32_t* perm = reinterpret_cast<const int32_t*>(ws + L.f.perm);
  const int32_t* offsets = reinterpret_cast<const int32_t*>(ws + L.f.offsets);
  hipError_t he = hipSuccess;
  BwdSmallArgs ba{Ti, static_cast<const uint16_t*>(x), W_router, nullptr,
                  reinterpret_cast<const float*>(ws + B.p_all), reinterpret_cast<const float*>(ws + L.lse),
                  offsets, perm, nullptr,
                  reinterpret_cast<const float*>(ws + B.rowdot), g_aux, g_z,
                  reinterpret_cast<float*>(ws + B.dlogits), reinterpret_cast<const float*>(ws + B.dxr), dx,
                  reinterpret_cast<float*>(ws + B.dwr_part), dW_router, reinterpret_cast<uint16_t*>(ws + B.zero),
                  reinterpret_cast<int32_t*>(ws + B.tp_bwd), reinterpret_cast<int2*>(ws + B.tiles_bwd),
                  reinterpret_cast<const int32_t*>(ws + L.inv_ec), OLMOE_E * C};
  ba.dot_parts = bwd_dot_parts(Teff);
  he = launch_bwd_prepare(ba, s);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "backward preparation launch: %s", hipGetErrorString(he));
  const uint16_t* dgu = reinterpret_cast<const uint16_t*>(ws + B.dgu);
  // dout and x rows are read through perm (expert order -> token) by the kernels that use them
  BwdWgradArgs wd{static_cast<const uint16_t*>(dout), OLMOE_D, reinterpret_cast<const uint16_t*>(ws + B.hw),
                  OLMOE_F, offsets, reinterpret_cast<const uint16_t*>(ws + B.zero), OLMOE_D, OLMOE_F, dW_down, dW_down,
                  OLMOE_D, (long)OLMOE_D * OLMOE_F, perm, nullptr, grad_bf16};
  BwdWgradArgs wgu{dgu, 2 * OLMOE_F, static_cast<const uint16_t*>(x), OLMOE_D, offsets,
                   reinterpret_cast<const uint16_t*>(ws + B.zero), 2 * OLMOE_F, OLMOE_D, dW_gate, dW_up, OLMOE_F,
                   (long)OLMOE_F * OLMOE_D, nullptr, perm, grad_bf16};
  SideStreams* ss = nullptr;
  he = side_streams(&ss);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "side streams: %s", hipGetErrorString(he));
  if (Ti > 0) {
    BwdDgradArgs dh{static_cast<const uint16_t*>(dout), perm, static_cast<const uint16_t*>(W_down),
                    nullptr, OLMOE_F, (long)OLMOE_D * OLMOE_F, 2 * OLMOE_F,
                    reinterpret_cast<const int32_t*>(ws + B.tp_bwd) + OLMOE_E,
                    reinterpret_cast<const int2*>(ws + B.tiles_bwd),
                    reinterpret_cast<const float*>(ws + L.row_w), reinterpret_cast<const float*>(ws + B.gu),
                    reinterpret_cast<uint16_t*>(ws + B.dgu), reinterpret_cast<uint16_t*>(ws + B.hw), nullptr,
                    reinterpret_cast<float*>(ws + B.rowdot), OLMOE_E * C};
    BwdDgradArgs dxa{dgu, nullptr, static_cast<const uint16_t*>(W_gate), static_cast<const uint16_t*>(W_up),
                     OLMOE_D, (long)OLMOE_F * OLMOE_D, OLMOE_F,
                     reinterpret_cast<const int32_t*>(ws + B.tp_bwd) + OLMOE_E,
                     reinterpret_cast<const int2*>(ws + B.tiles_bwd), nullptr, nullptr, nullptr, nullptr,
                     reinterpret_cast<float*>(ws + B.dxr)};
    he = launch_dgrad(dh, Teff, true, s);
    if (he == hipSuccess) he = fork_wgrads(wd, wgu, s, *ss);   // they need dH's outputs only
    if (he == hipSuccess) he = launch_bwd_router(ba, s);        // dlogits from dH's row sums
    if (he == hipSuccess) he = launch_dgrad(dxa, Teff, false, s);
    if (he != hipSuccess) return fail(OLMOE_EHIP, "gradient launch: %s", hipGetErrorString(he));
  } else {
    he = fork_wgrads(wd, wgu, s, *ss);
    if (he != hipSuccess) return fail(OLMOE_EHIP, "weight-gradient launch: %s", hipGetErrorString(he));
  }
  he = launch_bwd_finish(ba, s);
  if (he == hipSuccess) he = join_wgrads(s, *ss);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "router-gradient launch: %s", hipGetErrorString(he));
  return ok();
}


}  // namespace

extern "C" {

size_t olmoe_moe_backward_workspace_bytes(int64_t T) {
  if (T < 0 || T > OLMOE_MAX_TOKENS) return 0;
  return make_bwd_layout(T).total;
}

olmoe_status_t olmoe_moe_backward(const void* x, const float* W_router, const void* W_gate, const void* W_up,
                                  const void* W_down, int64_t T, const void* dout, float g_aux, float g_z,
                                  float* dx, float* dW_router, float* dW_gate, float* dW_up, float* dW_down,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return olmoe_moe_backward_ex(x, W_router, W_gate, W_up, W_down, T, dout, g_aux, g_z, dx, dW_router, dW_gate, dW_up,
                               dW_down, workspace, workspace_bytes, 0u, stream);
}

size_t olmoe_moe_saved_bytes(int64_t T) { return olmoe_moe_backward_workspace_bytes(T); }

olmoe_status_t olmoe_moe_forward_train(const void* x, const float* W_router, const void* W_gate, const void* W_up,
                                       const void* W_down, int64_t T, void* out, int32_t* route_ids,
                                       float* route_probs, int32_t* expert_counts, float* aux_loss, float* z_loss,
                                       void* saved, size_t saved_bytes, void* stream) {
  // ---- host-side checks; nothing is enqueued unless all pass
  if (T < 0 || T > OLMOE_MAX_TOKENS)
    return fail(OLMOE_EINVAL, "T=%lld out of range [0, %lld]", (long long)T, (long long)OLMOE_MAX_TOKENS);
  if (!W_router || !W_gate || !W_up || !W_down) return fail(OLMOE_EINVAL, "a weight pointer is NULL");
  if (T > 0 && (!x || !out)) return fail(OLMOE_EINVAL, "x or out is NULL");
  const void* ptrs[] = {x, W_router, W_gate, W_up, W_down, out, route_ids, route_probs, expert_counts};
  const char* names[] = {"x", "W_router", "W_gate", "W_up", "W_down", "out", "route_ids", "route_probs",
                         "expert_counts"};
  for (int i = 0; i < 9; ++i)
    if (ptrs[i] && misaligned(ptrs[i])) return fail(OLMOE_EINVAL, "%s is not 16-byte aligned", names[i]);
  if ((aux_loss && misaligned(aux_loss, 4)) || (z_loss && misaligned(z_loss, 4)))
    return fail(OLMOE_EINVAL, "aux_loss / z_loss not 4-byte aligned");
  const BwdLayout B = make_bwd_layout(T);
  if (!saved) return fail(OLMOE_EWORKSPACE, "saved is NULL");
  if (misaligned(saved, 256)) return fail(OLMOE_EINVAL, "saved is not 256-byte aligned");
  if (saved_bytes < B.total)
    return fail(OLMOE_EWORKSPACE, "saved has %zu bytes, %zu needed for T=%lld", saved_bytes, B.total, (long long)T);
  const size_t act = static_cast<size_t>(T) * OLMOE_D * 2;
  const size_t wexp = static_cast<size_t>(OLMOE_E) * OLMOE_F * OLMOE_D * 2;
  const size_t wr_bytes = (size_t)OLMOE_E * OLMOE_D * 4;
  const size_t rows = static_cast<size_t>(T) * OLMOE_K * 4;
  const void* ins[] = {x, W_router, W_gate, W_up, W_down};
  const size_t in_n[] = {act, wr_bytes, wexp, wexp, wexp};
  void* outs[] = {out, route_ids, route_probs, expert_counts, aux_loss, z_loss};
  const size_t out_n[] = {act, rows, rows, OLMOE_E * 4, 4, 4};
  for (int o = 0; o < 6; ++o) {
    for (int i = 0; i < 5; ++i)
      if (overlaps(outs[o], out_n[o], ins[i], in_n[i])) return fail(OLMOE_EINVAL, "an output overlaps an input");
    for (int q = o + 1; q < 6; ++q)
      if (overlaps(outs[o], out_n[o], outs[q], out_n[q])) return fail(OLMOE_EINVAL, "two outputs overlap");
    if (overlaps(outs[o], out_n[o], saved, B.total)) return fail(OLMOE_EINVAL, "an output overlaps saved");
  }
  olmoe_status_t st = check_device();
  if (st != OLMOE_OK) return st;
  // ---- launches: the backward's forward part (routing, G | U kept, Y), then the weighted sum
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(saved);
  const Layout& L = B.f;
  st = bwd_forward_state(x, W_router, W_gate, W_up, W_down, static_cast<int>(T), ws, B, expert_counts, aux_loss,
                         z_loss, true, s);
  if (st != OLMOE_OK) return st;
  if (T == 0) return ok();
  hipError_t he = hipSuccess;
  if (route_ids) he = hipMemcpyAsync(route_ids, ws + L.ids, rows, hipMemcpyDeviceToDevice, s);
  if (he == hipSuccess && route_probs) he = hipMemcpyAsync(route_probs, ws + L.probs, rows, hipMemcpyDeviceToDevice, s);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "routing copy: %s", hipGetErrorString(he));
  CombineArgs ca{static_cast<int>(T), reinterpret_cast<const uint16_t*>(ws + L.y),
                 reinterpret_cast<const int32_t*>(ws + L.inv), reinterpret_cast<const float*>(ws + L.probs),
                 static_cast<uint16_t*>(out), nullptr, nullptr, 0.f};
  he = launch_combine(ca, s);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "combine launch: %s", hipGetErrorString(he));
  return ok();
}

olmoe_status_t olmoe_moe_backward_saved(const void* x, const float* W_router, const void* W_gate, const void* W_up,
                                        const void* W_down, int64_t T, const void* dout, float g_aux, float g_z,
                                        float* dx, float* dW_router, float* dW_gate, float* dW_up, float* dW_down,
                                        void* saved, size_t saved_bytes, void* stream) {
  return olmoe_moe_backward_ex(x, W_router, W_gate, W_up, W_down, T, dout, g_aux, g_z, dx, dW_router, dW_gate, dW_up,
                               dW_down, saved, saved_bytes, OLMOE_BWD_SAVED, stream);
}

size_t olmoe_moe_ec_workspace_bytes(int64_t T) {
  if (T < 0 || T > OLMOE_EC_MAX_TOKENS) return 0;
  return make_ec_layout(T).total;
}

olmoe_status_t olmoe_moe_forward_expert_choice(const void* x, const float* W_router, const void* W_gate,
                                               const void* W_up, const void* W_down, int64_t T, void* out,
                                               int32_t* choice_tokens, float* choice_probs,
                                               int32_t* token_counts, float* aux_loss, float* z_loss,
                                               void* workspace, size_t workspace_bytes, void* stream) {
  // ---- host-side checks; nothing is enqueued unless all pass
  if (T < 0 || T > OLMOE_EC_MAX_TOKENS)
    return fail(OLMOE_EINVAL, "T=%lld out of range [0, %lld]", (long long)T, (long long)OLMOE_EC_MAX_TOKENS);
  if (!W_router || !W_gate || !W_up || !W_down) return fail(OLMOE_EINVAL, "a weight pointer is NULL");
  if (T > 0 && (!x || !out)) return fail(OLMOE_EINVAL, "x or out is NULL");
  const void* ptrs[] = {x, W_router, W_gate, W_up, W_down, out, choice_tokens, choice_probs, token_counts};
  const char* names[] = {"x", "W_router", "W_gate", "W_up", "W_down", "out", "choice_tokens", "choice_probs",
                         "token_counts"};
  for (int i = 0; i < 9; ++i)
    if (ptrs[i] && misaligned(ptrs[i])) return fail(OLMOE_EINVAL, "%s is not 16-byte aligned", names[i]);
  if ((aux_loss && misaligned(aux_loss, 4)) || (z_loss && misaligned(z_loss, 4)))
    return fail(OLMOE_EINVAL, "aux_loss / z_loss not 4-byte aligned");
  const int Ti = static_cast<int>(T);
  const int C = ec_capacity(Ti);
  const size_t act = static_cast<size_t>(T) * OLMOE_D * 2;
  const size_t wexp = static_cast<size_t>(OLMOE_E) * OLMOE_F * OLMOE_D * 2;
  const size_t wr_bytes = (size_t)OLMOE_E * OLMOE_D * 4;
  const size_t choice_n = static_cast<size_t>(C) * OLMOE_E * 4;
  const void* ins[] = {x, W_router, W_gate, W_up, W_down};
  const size_t in_n[] = {act, wr_bytes, wexp, wexp, wexp};
  void* outs[] = {out, choice_tokens, choice_probs, token_counts, aux_loss, z_loss};
  const size_t out_n[] = {act, choice_n, choice_n, static_cast<size_t>(T) * 4, 4, 4};
  const EcLayout L = make_ec_layout(T);
  if (!workspace) return fail(OLMOE_EWORKSPACE, "workspace is NULL");
  if (misaligned(workspace, 256)) return fail(OLMOE_EINVAL, "workspace is not 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(OLMOE_EWORKSPACE, "workspace has %zu bytes, %zu needed for T=%lld", workspace_bytes, L.total,
                (long long)T);
  for (int o = 0; o < 6; ++o) {
    for (int i = 0; i < 5; ++i)
      if (overlaps(outs[o], out_n[o], ins[i], in_n[i])) return fail(OLMOE_EINVAL, "an output overlaps an input");
    for (int q = o + 1; q < 6; ++q)
      if (overlaps(outs[o], out_n[o], outs[q], out_n[q])) return fail(OLMOE_EINVAL, "two outputs overlap");
    if (overlaps(outs[o], out_n[o], workspace, L.total)) return fail(OLMOE_EINVAL, "an output overlaps the workspace");
  }
  olmoe_status_t st = check_device();
  if (st != OLMOE_OK) return st;

  // ---- launches: router -> softmax (stage "router"), choose + losses ("dispatch"), the grouped
  // GEMMs on 64 blocks of C rows, combine
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int Teff = 8 * C;   // the GEMMs see 8*Teff = 64C rows, C per expert
  const GemmPlan plan = plan_gemm(Teff);
  StageRecorder rec(s);
  EcArgs ea{};
  ea.T = Ti;
  ea.C = C;
  ea.partial = reinterpret_cast<const float2*>(ws + L.f.partial);
  ea.pT = reinterpret_cast<float*>(ws + L.pT);
  ea.lse = reinterpret_cast<float*>(ws + L.lse);
  ea.inv_ec = reinterpret_cast<int32_t*>(ws + L.inv_ec);
  ea.perm = reinterpret_cast<int32_t*>(ws + L.f.perm);
  ea.row_w = reinterpret_cast<float*>(ws + L.row_w);
  ea.blk_psum = reinterpret_cast<float*>(ws + L.f.blk_psum);   // ceil(8C/16) >= ceil(T/16) blocks
  ea.blk_lse2 = reinterpret_cast<float*>(ws + L.f.blk_lse2);
  ea.offsets = reinterpret_cast<int32_t*>(ws + L.f.offsets);
  ea.tile_prefix_gu = reinterpret_cast<int32_t*>(ws + L.f.tp_gu);
  ea.tiles_gu = reinterpret_cast<int2*>(ws + L.f.tiles_gu);
  ea.bm_gu = plan.bm_gu;
  ea.tile_prefix_dn = reinterpret_cast<int32_t*>(ws + L.f.tp_dn);
  ea.tiles_dn = reinterpret_cast<int2*>(ws + L.f.tiles_dn);
  ea.bm_dn = plan.bm_dn;
  ea.choice_tokens = choice_tokens;
  ea.choice_probs = choice_probs;
  ea.y = reinterpret_cast<const uint16_t*>(ws + L.f.y);
  ea.out = static_cast<uint16_t*>(out);
  ea.token_counts = token_counts;
  ea.aux_loss = aux_loss;
  ea.z_loss = z_loss;
  ea.clip = reinterpret_cast<int32_t*>(ws + L.f.clip);
  hipError_t he = hipSuccess;
  if (Ti > 0) {
    RouterArgs ra{static_cast<const uint16_t*>(x), W_router, Ti, reinterpret_cast<float2*>(ws + L.f.partial),
                  reinterpret_cast<uint16_t*>(ws + L.f.planes)};
    he = launch_router_partial(ra, s);
    if (he == hipSuccess) he = launch_ec_softmax(ea, s);
    if (he != hipSuccess) return fail(OLMOE_EHIP, "router launch: %s", hipGetErrorString(he));
  }
  rec.mark();
  he = launch_ec_choose(ea, s);   // T == 0: zero offsets, and the losses (0)
  if (he != hipSuccess) return fail(OLMOE_EHIP, "expert-choice selection launch: %s", hipGetErrorString(he));
  rec.mark();
  if (Ti == 0) {
    rec.finish();
    return ok();
  }
  GemmArgs ga{Teff,
              static_cast<const uint16_t*>(x),
              static_cast<const uint16_t*>(W_gate),
              static_cast<const uint16_t*>(W_up),
              static_cast<const uint16_t*>(W_down),
              reinterpret_cast<const int32_t*>(ws + L.f.perm),
              reinterpret_cast<const int32_t*>(ws + L.f.offsets),
              reinterpret_cast<const int32_t*>(ws + L.f.tp_gu),
              reinterpret_cast<const int32_t*>(ws + L.f.tp_dn),
              reinterpret_cast<const int2*>(ws + L.f.tiles_gu),
              reinterpret_cast<const int2*>(ws + L.f.tiles_dn),
              reinterpret_cast<uint16_t*>(ws + L.f.h),
              reinterpret_cast<uint16_t*>(ws + L.f.y),
              nullptr,
              reinterpret_cast<int32_t*>(ws + L.f.clip)};
  he = launch_gateup(ga, plan, s);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "gate/up launch: %s", hipGetErrorString(he));
  rec.mark();
  he = launch_down(ga, plan, s);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "down launch: %s", hipGetErrorString(he));
  rec.mark();
  he = launch_ec_combine(ea, s);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "combine launch: %s", hipGetErrorString(he));
  rec.mark();
  return ok();
}

size_t olmoe_moe_ec_backward_workspace_bytes(int64_t T) {
  if (T < 0 || T > OLMOE_EC_MAX_TOKENS) return 0;
  return make_ec_bwd_layout(T).total;
}

olmoe_status_t olmoe_moe_backward_expert_choice(const void* x, const float* W_router, const void* W_gate,
                                                const void* W_up, const void* W_down, int64_t T, const void* dout,
                                                float g_aux, float g_z, float* dx, float* dW_router, float* dW_gate,
                                                float* dW_up, float* dW_down, void* workspace, size_t workspace_bytes,
                                                void* stream) {
  return olmoe_moe_backward_ex(x, W_router, W_gate, W_up, W_down, T, dout, g_aux, g_z, dx, dW_router, dW_gate, dW_up,
                               dW_down, workspace, workspace_bytes, OLMOE_BWD_EXPERT_CHOICE, stream);
}

size_t olmoe_moe_ec_saved_bytes(int64_t T) { return olmoe_moe_ec_backward_workspace_bytes(T); }

olmoe_status_t olmoe_moe_forward_expert_choice_train(const void* x, const float* W_router, const void* W_gate,
                                                     const void* W_up, const void* W_down, int64_t T, void* out,
                                                     int32_t* choice_tokens, float* choice_probs,
                                                     int32_t* token_counts, float* aux_loss, float* z_loss,
                                                     void* saved, size_t saved_bytes, void* stream) {
  // ---- host-side checks; nothing is enqueued unless all pass
  if (T < 0 || T > OLMOE_EC_MAX_TOKENS)
    return fail(OLMOE_EINVAL, "T=%lld out of range [0, %lld]", (long long)T, (long long)OLMOE_EC_MAX_TOKENS);
  if (!W_router || !W_gate || !W_up || !W_down) return fail(OLMOE_EINVAL, "a weight pointer is NULL");
  if (T > 0 && (!x || !out)) return fail(OLMOE_EINVAL, "x or out is NULL");
  const void* ptrs[] = {x, W_router, W_gate, W_up, W_down, out, choice_tokens, choice_probs, token_counts};
  const char* names[] = {"x", "W_router", "W_gate", "W_up", "W_down", "out", "choice_tokens", "choice_probs",
                         "token_counts"};
  for (int i = 0; i < 9; ++i)
    if (ptrs[i] && misaligned(ptrs[i])) return fail(OLMOE_EINVAL, "%s is not 16-byte aligned", names[i]);
  if ((aux_loss && misaligned(aux_loss, 4)) || (z_loss && misaligned(z_loss, 4)))
    return fail(OLMOE_EINVAL, "aux_loss / z_loss not 4-byte aligned");
  const EcBwdLayout B = make_ec_bwd_layout(T);
  if (!saved) return fail(OLMOE_EWORKSPACE, "saved is NULL");
  if (misaligned(saved, 256)) return fail(OLMOE_EINVAL, "saved is not 256-byte aligned");
  if (saved_bytes < B.total)
    return fail(OLMOE_EWORKSPACE, "saved has %zu bytes, %zu needed for T=%lld", saved_bytes, B.total, (long long)T);
  const int Ti = static_cast<int>(T);
  const int C = ec_capacity(Ti);
  const size_t act = static_cast<size_t>(T) * OLMOE_D * 2;
  const size_t wexp = static_cast<size_t>(OLMOE_E) * OLMOE_F * OLMOE_D * 2;
  const size_t wr_bytes = (size_t)OLMOE_E * OLMOE_D * 4;
  const size_t choice_n = static_cast<size_t>(C) * OLMOE_E * 4;
  const void* ins[] = {x, W_router, W_gate, W_up, W_down};
  const size_t in_n[] = {act, wr_bytes, wexp, wexp, wexp};
  void* outs[] = {out, choice_tokens, choice_probs, token_counts, aux_loss, z_loss};
  const size_t out_n[] = {act, choice_n, choice_n, static_cast<size_t>(T) * 4, 4, 4};
  for (int o = 0; o < 6; ++o) {
    for (int i = 0; i < 5; ++i)
      if (overlaps(outs[o], out_n[o], ins[i], in_n[i])) return fail(OLMOE_EINVAL, "an output overlaps an input");
    for (int q = o + 1; q < 6; ++q)
      if (overlaps(outs[o], out_n[o], outs[q], out_n[q])) return fail(OLMOE_EINVAL, "two outputs overlap");
    if (overlaps(outs[o], out_n[o], saved, B.total)) return fail(OLMOE_EINVAL, "an output overlaps saved");
  }
  olmoe_status_t st = check_device();
  if (st != OLMOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(saved);
  st = ec_bwd_forward_state(x, W_router, W_gate, W_up, W_down, Ti, ws, B, choice_tokens, choice_probs, aux_loss,
                            z_loss, true, s);
  if (st != OLMOE_OK || Ti == 0) return st == OLMOE_OK ? ok() : st;
  const EcLayout& L = B.c;
  EcArgs ea{};
  ea.T = Ti;
  ea.C = C;
  ea.inv_ec = reinterpret_cast<int32_t*>(ws + L.inv_ec);
  ea.row_w = reinterpret_cast<float*>(ws + L.row_w);
  ea.y = reinterpret_cast<const uint16_t*>(ws + L.f.y);
  ea.out = static_cast<uint16_t*>(out);
  ea.token_counts = token_counts;
  const hipError_t he = launch_ec_combine(ea, s);
  if (he != hipSuccess) return fail(OLMOE_EHIP, "combine launch: %s", hipGetErrorString(he));
  return ok();
}

olmoe_status_t olmoe_moe_backward_expert_choice_saved(const void* x, const float* W_router, const void* W_gate,
                                                      const void* W_up, const void* W_down, int64_t T,
                                                      const void* dout, float g_aux, float g_z, float* dx,
                                                      float* dW_router, float* dW_gate, float* dW_up, float* dW_down,
                                                      void* saved, size_t saved_bytes, void* stream) {
  return olmoe_moe_backward_ex(x, W_router, W_gate, W_up, W_down, T, dout, g_aux, g_z, dx, dW_router, dW_gate, dW_up,
                               dW_down, saved, saved_bytes, OLMOE_BWD_EXPERT_CHOICE | OLMOE_BWD_SAVED, stream);
}

olmoe_status_t olmoe_moe_backward_ex(const void* x, const float* W_router, const void* W_gate, const void* W_up,
                                     const void* W_down, int64_t T, const void* dout, float g_aux, float g_z,
                                     float* dx, float* dW_router, void* dW_gate, void* dW_up, void* dW_down,
                                     void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
  // ---- host-side checks; nothing is enqueued unless all pass
  if (flags & ~(OLMOE_BWD_SAVED | OLMOE_BWD_EXPERT_CHOICE | OLMOE_BWD_GRAD_BF16))
    return fail(OLMOE_EINVAL, "unknown backward flags 0x%x", flags);
  const bool ec = flags & OLMOE_BWD_EXPERT_CHOICE;
  const bool from_saved = flags & OLMOE_BWD_SAVED;
  const bool grad_bf16 = flags & OLMOE_BWD_GRAD_BF16;
  const int64_t t_max = ec ? OLMOE_EC_MAX_TOKENS : OLMOE_MAX_TOKENS;
  if (T < 0 || T > t_max) return fail(OLMOE_EINVAL, "T=%lld out of range [0, %lld]", (long long)T, (long long)t_max);
  const size_t wgrad_elem = grad_bf16 ? 2 : 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int Ti = static_cast<int>(T);
  olmoe_status_t st = OLMOE_OK;
  // ---- launches: recompute the forward (keeping p, lse, G, U, Y) unless the state was saved, then
  // the gradients
  if (ec) {
    const EcBwdLayout B = make_ec_bwd_layout(T);
    st = backward_checks(x, W_router, W_gate, W_up, W_down, T, dout, g_aux, g_z, dx, dW_router, dW_gate, dW_up,
                         dW_down, workspace, workspace_bytes, B.total, wgrad_elem);
    if (st == OLMOE_OK && !from_saved)
      st = ec_bwd_forward_state(x, W_router, W_gate, W_up, W_down, Ti, ws, B, nullptr, nullptr, nullptr, nullptr,
                                false, s);
    if (st != OLMOE_OK) return st;
    return ec_bwd_gradients(x, W_router, W_gate, W_up, W_down, Ti, dout, g_aux, g_z, dx, dW_router, dW_gate, dW_up,
                            dW_down, ws, B, s, grad_bf16);
  }
  const BwdLayout B = make_bwd_layout(T);
  st = backward_checks(x, W_router, W_gate, W_up, W_down, T, dout, g_aux, g_z, dx, dW_router, dW_gate, dW_up, dW_down,
                       workspace, workspace_bytes, B.total, wgrad_elem);
  if (st == OLMOE_OK && !from_saved)
    st = bwd_forward_state(x, W_router, W_gate, W_up, W_down, Ti, ws, B, nullptr, nullptr, nullptr, false, s);
  if (st != OLMOE_OK) return st;
  return bwd_gradients(x, W_router, W_gate, W_up, W_down, Ti, dout, g_aux, g_z, dx, dW_router, dW_gate, dW_up,
                       dW_down, ws, B, s, grad_bf16);
}

olmoe_status_t olmoe_rmsnorm_bf16(const float* h, float eps, int64_t T, void* x_out, void* stream) {
  if (T < 0 || T > OLMOE_MAX_TOKENS) return fail(OLMOE_EINVAL, "T=%lld out of range", (long long)T);
  if (!(eps > 0.f)) return fail(OLMOE_EINVAL, "eps must be > 0");
  if (T > 0 && (!h || !x_out)) return fail(OLMOE_EINVAL, "h or x_out is NULL");
  if (misaligned(h) || misaligned(x_out)) return fail(OLMOE_EINVAL, "h / x_out not 16-byte aligned");
  if (overlaps(h, (size_t)T * OLMOE_D * 4, x_out, (size_t)T * OLMOE_D * 2))
    return fail(OLMOE_EINVAL, "x_out overlaps h");
  if (T == 0) return ok();
  olmoe_status_t st = check_device();
  if (st != OLMOE_OK) return st;
  hipError_t he = launch_rmsnorm(h, eps, static_cast<int>(T), static_cast<uint16_t*>(x_out),
                                 static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return fail(OLMOE_EHIP, "rmsnorm launch: %s", hipGetErrorString(he));
  return ok();
}

olmoe_status_t olmoe_residual_add(float* h, const void* y, int64_t T, void* stream) {
  if (T < 0 || T > OLMOE_MAX_TOKENS) return fail(OLMOE_EINVAL, "T=%lld out of range", (long long)T);
  if (T > 0 && (!h || !y)) return fail(OLMOE_EINVAL, "h or y is NULL");
  if (misaligned(h) || misaligned(y)) return fail(OLMOE_EINVAL, "h / y not 16-byte aligned");
  if (overlaps(h, (size_t)T * OLMOE_D * 4, y, (size_t)T * OLMOE_D * 2))
    return fail(OLMOE_EINVAL, "y overlaps h");
  if (T == 0) return ok();
  olmoe_status_t st = check_device();
  if (st != OLMOE_OK) return st;
  hipError_t he = launch_residual_add(h, static_cast<const uint16_t*>(y), static_cast<int>(T),
                                      static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return fail(OLMOE_EHIP, "residual_add launch: %s", hipGetErrorString(he));
  return ok();
}

olmoe_status_t olmoe_timing_enable(int stage_mask) {
  if (stage_mask < 0 || stage_mask >= (1 << N_STAGES))
    return fail(OLMOE_EINVAL, "stage mask 0x%x has bits beyond the %d stages", stage_mask, N_STAGES);
  for (auto& set : g_timing.pending)
    for (auto& e : set)
      if (e) (void)hipEventDestroy(e);
  g_timing.pending.clear();
  g_timing.mask = stage_mask;
  g_timing.every = 1;
  g_timing.calls = 0;
  return ok();
}

olmoe_status_t olmoe_timing_every(int n) {
  if (n < 1) return fail(OLMOE_EINVAL, "timing sample step %d is below 1", n);
  g_timing.every = n;
  g_timing.calls = 0;
  return ok();
}

int olmoe_timing_read(double* stage_ms, int max_stages, int* calls) {
  if (!stage_ms && max_stages > 0) {
    fail(OLMOE_EINVAL, "stage_ms is NULL");
    return -1;
  }
  for (int i = 0; i < max_stages && i < N_STAGES; ++i) stage_ms[i] = 0.0;
  int n = 0;
  for (auto& set : g_timing.pending) {
    int last = N_STAGES;
    while (last > 0 && !set[last]) --last;
    if (set[last] && hipEventSynchronize(set[last]) != hipSuccess) {
      fail(OLMOE_EHIP, "hipEventSynchronize failed");
      return -1;
    }
    for (int i = 0; i < N_STAGES; ++i) {
      if (!set[i] || !set[i + 1] || !(g_timing.mask >> i & 1)) continue;
      float ms = 0.f;
      (void)hipEventElapsedTime(&ms, set[i], set[i + 1]);
      if (i < max_stages) stage_ms[i] += ms;
    }
    ++n;
  }
  if (calls) *calls = n;
  return N_STAGES;
}

const char* olmoe_timing_stage_name(int stage) {
  return (stage >= 0 && stage < N_STAGES) ? kStageNames[stage] : "";
}

}  // extern "C"
