// api.cpp -- the extern "C" boundary of libmoe.so (declared in include/moe.h).
//
// Host-side only: argument checks (before anything is enqueued), workspace
// carve-up and kernel launches on the caller's stream.  No allocation, no
// synchronisation, no state beyond a per-device cache of the CU count.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <mutex>

#include "../../include/moe.h"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
std::atomic<int> g_cus[64];
}  // namespace

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = g_cus[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

Workspace carve_workspace(void* base, int64_t T, int d, int E, int k, int H, int Hs, int S) {
  (void)d;
  Workspace w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return base ? static_cast<char*>(base) + o : nullptr;
  };
  const int tb = perm_block_tokens(T);
  const int64_t nblk = (T + tb - 1) / tb;
  const int nsplit = seq_partials_capacity(T, S);
  const int64_t nseq = S > 0 ? T / S : 0;
  w.scores = reinterpret_cast<float*>(take(sizeof(float) * T * E));
  w.tok_sum = reinterpret_cast<double*>(take(sizeof(double) * (S > 0 ? T : 0)));
  w.seq_p = reinterpret_cast<double*>(take(sizeof(double) * nseq * nsplit * E));
  w.seq_cnt = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * nseq * nsplit * E));
  w.blk_cnt = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * nblk * E));
  w.blk_base = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * nblk * E));
  w.h_routed = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * T * k * H));
  w.h_shared = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * T * Hs));
  w.unit_counters = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * kUnitCounters));
  w.total = off;
  return w;
}

}  // namespace moe

using moe::Workspace;

namespace {

moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARGUMENT;
  if (s->tokens < 0 || s->d_model <= 0 || s->n_experts <= 0 || s->top_k <= 0 || s->hidden <= 0 ||
      s->shared_hidden < 0 || s->seq_len < 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (s->top_k > s->n_experts) return MOE_ERR_INVALID_ARGUMENT;
  if (s->seq_len > 0 && s->tokens % s->seq_len != 0) return MOE_ERR_INVALID_ARGUMENT;
  if (s->n_experts > 1024 || s->top_k > 32) return MOE_ERR_UNSUPPORTED;
  if (s->d_model % 64 || s->hidden % 64 || s->shared_hidden % 64) return MOE_ERR_UNSUPPORTED;
  if (s->tokens * (static_cast<int64_t>(s->top_k) + 1) >= (int64_t{1} << 31))
    return MOE_ERR_UNSUPPORTED;
  // The grouped GEMMs address one expert's weights, and the token rows of x
  // they gather, with 32-bit byte offsets; the rows of x_perm and h are
  // addressed from each tile's first row, so their size is not limited.
  if (2 * s->tokens * s->d_model >= (int64_t{1} << 31) ||
      2 * static_cast<int64_t>(s->hidden) * s->d_model >= (int64_t{1} << 31) ||
      2 * static_cast<int64_t>(s->shared_hidden) * s->d_model >= (int64_t{1} << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The backward calls: their GEMMs also address whole [T*k, d or H] operands
// with 32-bit byte offsets.
moe_status check_bwd_shape(const moe_shape* s) {
  const moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  const int64_t widest = std::max<int64_t>({s->d_model, s->hidden, s->shared_hidden});
  if (2 * s->tokens * s->top_k * widest >= (int64_t{1} << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

Workspace carve(const moe_shape* s, void* base) {
  return moe::carve_workspace(base, s->tokens, s->d_model, s->n_experts, s->top_k, s->hidden,
                              s->shared_hidden, s->seq_len);
}

moe_status check_ws(const moe_shape* s, void* ws, size_t bytes) {
  const size_t need = carve(s, nullptr).total;
  if (!ws || bytes < need) return MOE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 256) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// ---- static scratch of moe_permute_noalloc
// The per-block count and first-row tables of the permutation, for callers
// that cannot allocate.  In host code `scratch` names a host-side stand-in,
// not device memory: kernels get the device address that hipGetSymbolAddress
// returns for the current device (each device holds its own copy).
constexpr size_t kScratchBytes = size_t{2} << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

// Device address of this device's scratch, looked up once per device.
moe_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Bytes of the permutation tables (the same carve-up as the workspace's).
size_t permute_table_bytes(int64_t T, int E) {
  const int tb = moe::perm_block_tokens(T);
  const int64_t nblk = (T + tb - 1) / tb;
  const size_t one = (sizeof(int32_t) * nblk * E + 255) / 256 * 256;
  return 2 * one;
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

}  // namespace

extern "C" {

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT: bad pointer or shape";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape outside what this build handles";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
    case MOE_ERR_SCRATCH_LIMIT:
      return "MOE_ERR_SCRATCH_LIMIT: shape needs more than the 2 MiB static scratch";
    default: return "unknown moe_status";
  }
}

moe_status moe_workspace_bytes(const moe_shape* shape, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  const moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  *bytes = carve(shape, nullptr).total;
  return MOE_OK;
}

moe_status moe_route(const moe_shape* shape, const uint16_t* x, const float* w_router,
                     const float* bias, int32_t* topk_idx, float* topk_gate, float* margin,
                     float* seq_balance, float alpha, void* workspace, size_t workspace_bytes,
                     void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->tokens == 0) return MOE_OK;
  if (!x || !w_router || !bias || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x)) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(shape, workspace, workspace_bytes)) != MOE_OK) return st;
  const Workspace w = carve(shape, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t T = shape->tokens;
  const int d = shape->d_model, E = shape->n_experts, k = shape->top_k, S = shape->seq_len;
  const bool stats = S > 0 && seq_balance != nullptr;
  bool fused = false;
  hipError_t e = moe::launch_route_fused(x, w_router, bias, topk_idx, topk_gate, margin, w.seq_p,
                                         w.seq_cnt, stats ? seq_balance : nullptr, alpha, T, d, E,
                                         k, S, s, &fused);
  if (e != hipSuccess || fused) return hip_status(e);
  e = moe::launch_router_scores(x, w_router, w.scores, T, d, E, s);
  if (e == hipSuccess)
    e = moe::launch_select(w.scores, bias, topk_idx, topk_gate, margin, stats ? w.tok_sum : nullptr,
                           T, E, k, s);
  if (e == hipSuccess && stats)
    e = moe::launch_seq_balance(w.scores, w.tok_sum, topk_idx, w.seq_p, w.seq_cnt, seq_balance,
                                alpha, T, E, k, S, s);
  return hip_status(e);
}

moe_status moe_permute(const moe_shape* shape, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* perm_src, int32_t* pos, const uint16_t* x,
                       uint16_t* x_perm, void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARGUMENT;
  // with no tokens the per-token arrays are empty and may be NULL
  if (shape->tokens > 0 && (!topk_idx || !perm_src || !pos)) return MOE_ERR_INVALID_ARGUMENT;
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (x_perm && (!aligned16(x) || !aligned16(x_perm))) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(shape, workspace, workspace_bytes)) != MOE_OK) return st;
  const Workspace w = carve(shape, workspace);
  // T == 0 still defines counts = 0 and offsets = 0: the kernels handle it.
  return hip_status(moe::launch_permute(topk_idx, counts, offsets, perm_src, pos, x, x_perm,
                                        w.blk_cnt, w.blk_base, shape->tokens, shape->d_model,
                                        shape->n_experts, shape->top_k,
                                        static_cast<hipStream_t>(stream)));
}

moe_status moe_permute_noalloc(const moe_shape* shape, const int32_t* topk_idx, int32_t* counts,
                               int32_t* offsets, int32_t* perm_src, int32_t* pos,
                               const uint16_t* x, uint16_t* x_perm, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARGUMENT;
  if (shape->tokens > 0 && (!topk_idx || !perm_src || !pos)) return MOE_ERR_INVALID_ARGUMENT;
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (x_perm && (!aligned16(x) || !aligned16(x_perm))) return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = permute_table_bytes(shape->tokens, shape->n_experts);
  if (need > kScratchBytes) return MOE_ERR_SCRATCH_LIMIT;
  void* base = nullptr;
  if ((st = scratch_of_current_device(&base)) != MOE_OK) return st;
  // the count kernel writes every count-table entry and the scan (when it
  // runs) every first-row entry before they are read: nothing is cleared
  int32_t* blk_cnt = static_cast<int32_t*>(base);
  int32_t* blk_base = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(base) + need / 2);
  return hip_status(moe::launch_permute(topk_idx, counts, offsets, perm_src, pos, x, x_perm,
                                        blk_cnt, blk_base, shape->tokens, shape->d_model,
                                        shape->n_experts, shape->top_k,
                                        static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_ffn(const moe_shape* shape, const uint16_t* x, const uint16_t* x_perm,
                           const int32_t* perm_src, const int32_t* offsets, const uint16_t* w1,
                           const uint16_t* w3, const uint16_t* w2, const uint16_t* ws1,
                           const uint16_t* ws3, const uint16_t* ws2, uint16_t* y_perm,
                           uint16_t* y_shared, void* workspace, size_t workspace_bytes,
                           void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->tokens == 0) return MOE_OK;
  const bool shared = shape->shared_hidden > 0;
  if (!x || !perm_src || !offsets || !w1 || !w3 || !w2 || !y_perm) return MOE_ERR_INVALID_ARGUMENT;
  if (shared != (ws1 && ws3 && ws2 && y_shared)) return MOE_ERR_INVALID_ARGUMENT;
  if (!shared && (ws1 || ws3 || ws2 || y_shared)) return MOE_ERR_INVALID_ARGUMENT;
  // the GEMMs load and store 16-byte chunks of every bf16 array
  const void* ptrs[] = {x,      x_perm ? x_perm : x, w1, w3, w2, ws1 ? ws1 : w1, ws3 ? ws3 : w1,
                        ws2 ? ws2 : w1, y_perm, y_shared ? y_shared : y_perm};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(shape, workspace, workspace_bytes)) != MOE_OK) return st;
  const Workspace w = carve(shape, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t T = shape->tokens;
  const int d = shape->d_model, E = shape->n_experts, H = shape->hidden, Hs = shape->shared_hidden;

  moe::GroupedGemmArgs g1{};
  g1.a_routed = x_perm ? x_perm : x;
  g1.a_row_map = x_perm ? nullptr : perm_src;
  g1.a_shared = shared ? x : nullptr;
  g1.a_routed_bytes = 2 * d * (x_perm ? T * shape->top_k : T);
  g1.a_shared_bytes = 2 * d * T;
  g1.w_routed = w1;
  g1.w3_routed = w3;
  g1.w_shared = shared ? ws1 : nullptr;
  g1.w3_shared = shared ? ws3 : nullptr;
  g1.c_routed = w.h_routed;
  g1.c_shared = shared ? w.h_shared : nullptr;
  g1.offsets = offsets;
  g1.T = T;
  g1.E = E;
  g1.top_k = shape->top_k;
  g1.K_r = d;
  g1.K_s = d;
  g1.N_r = H;
  g1.N_s = Hs;
  g1.unit_counter = w.unit_counters;
  hipError_t e = moe::launch_zero_counters(w.unit_counters, moe::kUnitCounters, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_gemm_swiglu(g1, s);
  if (e != hipSuccess) return MOE_ERR_HIP;

  moe::GroupedGemmArgs g2{};
  g2.a_routed = w.h_routed;
  g2.a_row_map = nullptr;
  g2.a_shared = shared ? w.h_shared : nullptr;
  g2.a_routed_bytes = 2 * static_cast<int64_t>(H) * T * shape->top_k;
  g2.a_shared_bytes = 2 * static_cast<int64_t>(Hs) * T;
  g2.w_routed = w2;
  g2.w_shared = shared ? ws2 : nullptr;
  g2.c_routed = y_perm;
  g2.c_shared = shared ? y_shared : nullptr;
  g2.offsets = offsets;
  g2.T = T;
  g2.E = E;
  g2.top_k = shape->top_k;
  g2.K_r = H;
  g2.K_s = Hs;
  g2.N_r = d;
  g2.N_s = d;
  g2.unit_counter = w.unit_counters + moe::kUnitCounters / 2;
  return hip_status(moe::launch_gemm_down(g2, s));
}

moe_status moe_combine(const moe_shape* shape, const uint16_t* y_perm, const uint16_t* y_shared,
                       const float* topk_gate, const int32_t* pos, const uint16_t* residual,
                       uint16_t* out, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->tokens == 0) return MOE_OK;
  if (!y_perm || !topk_gate || !pos || !out) return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {y_perm, y_shared ? y_shared : y_perm, residual ? residual : y_perm, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(moe::launch_combine(y_perm, y_shared, topk_gate, pos, residual, out,
                                        shape->tokens, shape->d_model, shape->top_k,
                                        static_cast<hipStream_t>(stream)));
}

moe_status moe_rmsnorm(const moe_shape* shape, const uint16_t* x, const float* gain, float eps,
                       uint16_t* out, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return MOE_ERR_INVALID_ARGUMENT;  // also rejects NaN
  if (shape->tokens == 0) return MOE_OK;
  if (!x || !gain || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(gain) || !aligned16(out)) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(moe::launch_rmsnorm(x, gain, eps, out, shape->tokens, shape->d_model,
                                        static_cast<hipStream_t>(stream)));
}

// ---- backward
namespace {
struct BwdWorkspace {
  uint16_t *dh, *h, *da, *dc;      // [T*k, H] bf16, expert-grouped rows
  uint16_t *dhs, *hs, *das, *dcs;  // [T, Hs] bf16, the shared expert
  float* scores;                   // [T, E]
  float* freq;                     // [T/S, E]
  float* dlogit;                   // [T, E]
  float* dwr_part;                 // [splits, d, E]
  float* wgrad_part;               // weight-gradient partial sums (split rows)
  int splits;
  size_t total;
};
// The weight-gradient launches of moe_grouped_ffn_backward: [0] dW2 = dy^T h,
// [1] dW1 and dW3 = [da dc]^T x.  Segment 0 is the shared expert if there is
// one, then the routed experts.
struct WgradPlans {
  int nseg;
  moe::WgradPlan p[2];
};
WgradPlans wgrad_plans(const moe_shape* s) {
  const int64_t T = s->tokens;
  const int E = s->n_experts, H = s->hidden, Hs = s->shared_hidden, d = s->d_model;
  const bool shared = Hs > 0;
  WgradPlans w{};
  w.nseg = shared ? 2 : 1;
  const int64_t rows[2] = {shared ? T : T * s->top_k, T * s->top_k};
  const int groups[2] = {shared ? 1 : E, E};
  const int m2[2] = {d, d}, n2[2] = {shared ? Hs : H, H};
  const int m13[2] = {2 * (shared ? Hs : H), 2 * H}, n13[2] = {d, d};
  w.p[0] = moe::plan_wgrad(w.nseg, rows, groups, m2, n2);
  w.p[1] = moe::plan_wgrad(w.nseg, rows, groups, m13, n13);
  return w;
}
BwdWorkspace carve_bwd(const moe_shape* s, void* base) {
  BwdWorkspace w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) / 256 * 256;
    return base ? static_cast<char*>(base) + o : nullptr;
  };
  const int64_t T = s->tokens, rk = T * s->top_k;
  const int H = s->hidden, Hs = s->shared_hidden, E = s->n_experts, d = s->d_model;
  w.dh = reinterpret_cast<uint16_t*>(take(2 * rk * H));
  w.h = reinterpret_cast<uint16_t*>(take(2 * rk * H));
  w.da = reinterpret_cast<uint16_t*>(take(2 * rk * H));
  w.dc = reinterpret_cast<uint16_t*>(take(2 * rk * H));
  w.dhs = reinterpret_cast<uint16_t*>(take(2 * T * Hs));
  w.hs = reinterpret_cast<uint16_t*>(take(2 * T * Hs));
  w.das = reinterpret_cast<uint16_t*>(take(2 * T * Hs));
  w.dcs = reinterpret_cast<uint16_t*>(take(2 * T * Hs));
  w.scores = reinterpret_cast<float*>(take(4 * T * E));
  w.freq = reinterpret_cast<float*>(take(4 * (s->seq_len > 0 ? T / s->seq_len : 0) * E));
  w.dlogit = reinterpret_cast<float*>(take(4 * T * E));
  w.splits = moe::route_bwd_splits(T);
  w.dwr_part = reinterpret_cast<float*>(take(4 * static_cast<int64_t>(w.splits) * d * E));
  const WgradPlans wp = wgrad_plans(s);
  w.wgrad_part = reinterpret_cast<float*>(
      take(4 * static_cast<size_t>(std::max(wp.p[0].part_floats, wp.p[1].part_floats))));
  w.total = off;
  return w;
}
moe_status check_bwd_ws(const moe_shape* s, void* ws, size_t bytes) {
  if (!ws || bytes < carve_bwd(s, nullptr).total) return MOE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 256) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}
}  // namespace

moe_status moe_backward_workspace_bytes(const moe_shape* shape, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  const moe_status st = check_bwd_shape(shape);
  if (st != MOE_OK) return st;
  *bytes = carve_bwd(shape, nullptr).total;
  return MOE_OK;
}

moe_status moe_combine_backward(const moe_shape* shape, const uint16_t* dout, const uint16_t* y_perm,
                                const float* topk_gate, const int32_t* pos, uint16_t* dy_perm,
                                float* dgate, void* stream) {
  moe_status st = check_bwd_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->tokens == 0) return MOE_OK;
  if (!dout || !y_perm || !topk_gate || !pos || !dy_perm || !dgate) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(dout) || !aligned16(y_perm) || !aligned16(dy_perm)) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(moe::launch_combine_bwd(dout, y_perm, topk_gate, pos, dy_perm, dgate,
                                            shape->tokens, shape->d_model, shape->top_k,
                                            static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_ffn_backward(const moe_shape* shape, const uint16_t* x,
                                    const uint16_t* x_perm, const int32_t* offsets,
                                    const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                                    const uint16_t* ws1, const uint16_t* ws3, const uint16_t* ws2,
                                    const uint16_t* dy_perm, const uint16_t* dout,
                                    uint16_t* dx_perm, uint16_t* dx_shared, float* dw1, float* dw3,
                                    float* dw2, float* dws1, float* dws3, float* dws2,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_bwd_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->tokens == 0) return MOE_OK;
  const bool shared = shape->shared_hidden > 0;
  if (!x || !x_perm || !offsets || !w1 || !w3 || !w2 || !dy_perm || !dx_perm || !dw1 || !dw3 || !dw2)
    return MOE_ERR_INVALID_ARGUMENT;
  if (shared != (ws1 && ws3 && ws2 && dout && dx_shared && dws1 && dws3 && dws2))
    return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x, x_perm, w1, w3, w2, dy_perm, dx_perm, dw1, dw3, dw2,
                        shared ? ws1 : w1, shared ? ws3 : w1, shared ? ws2 : w1,
                        shared ? dout : x, shared ? dx_shared : dx_perm,
                        shared ? dws1 : dw1, shared ? dws3 : dw1, shared ? dws2 : dw1};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_bwd_ws(shape, workspace, workspace_bytes)) != MOE_OK) return st;
  const BwdWorkspace w = carve_bwd(shape, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t T = shape->tokens;
  const int d = shape->d_model, E = shape->n_experts, H = shape->hidden, Hs = shape->shared_hidden;
  // segment 0: the shared expert (if any), then the routed experts
  const int ns = shared ? 2 : 1;
  moe::BwdSeg base[2]{};
  for (int i = 0; i < ns; ++i) {
    const bool sh = shared && i == 0;
    base[i].groups = sh ? 1 : E;
    base[i].offsets = sh ? nullptr : offsets;
    base[i].rows = sh ? static_cast<int>(T) : 0;
  }
  auto seg_h = [&](int i) { return shared && i == 0 ? Hs : H; };
  auto is_sh = [&](int i) { return shared && i == 0; };
  // all segments, or the shared expert's alone (nseg = 0: nothing to do)
  auto launch = [&](auto&& fill, int kind, bool shared_only = false) {
    moe::BwdGemmArgs g{};
    g.nseg = shared_only ? (shared ? 1 : 0) : ns;
    for (int i = 0; i < g.nseg; ++i) {
      g.seg[i] = base[i];
      fill(g.seg[i], i);
    }
    return g.nseg > 0 ? moe::launch_bwd_gemm(g, kind, s) : hipSuccess;
  };
  // Input gradients of the routed experts on the forward's streaming tile
  // with K-major weights where the shape takes it (weight-streaming shapes);
  // then the backward's own kernel for the rest.
  auto routed_dgrad = [&](const uint16_t* ar, const uint16_t* ar2, const uint16_t* wr,
                          const uint16_t* wr2, int K, int K2, int N, uint16_t* c, bool* done) {
    moe::GroupedGemmArgs g{};
    g.a_routed = ar;
    g.a2_routed = ar2;
    g.a_routed_bytes = 2 * static_cast<int64_t>(K) * T * shape->top_k;
    g.w_routed = wr;
    g.w3_routed = wr2;
    g.c_routed = c;
    g.offsets = offsets;
    g.T = T;
    g.E = E;
    g.top_k = shape->top_k;
    g.K_r = K;
    g.K2_r = K2;
    g.N_r = N;
    const hipError_t r = moe::launch_gemm_dgrad(g, s);
    *done = r == hipSuccess;
    return r == hipErrorNotSupported ? hipSuccess : r;
  };
  // dh = dy W2  (W2 [d, H] read as [K, N])
  bool dh_done = false;
  hipError_t e = routed_dgrad(dy_perm, nullptr, w2, nullptr, d, 0, H, w.dh, &dh_done);
  if (e == hipSuccess)
    e = launch(
        [&](moe::BwdSeg& q, int i) {
          const int Hh = seg_h(i);
          q.N = Hh; q.K = d;
          q.a = is_sh(i) ? dout : dy_perm; q.lda = d;
          q.b = is_sh(i) ? ws2 : w2; q.ldb = Hh; q.b_gstride = is_sh(i) ? 0 : static_cast<int64_t>(d) * H;
          q.c = is_sh(i) ? w.dhs : w.dh; q.ldc = Hh;
        },
        moe::kBwdDgradKM, dh_done);
  // a, c = x W1^T, x W3^T again -> h, da, dc: the forward's SwiGLU GEMM (same
  // tiles and sums, so h is the forward's) with the backward epilogue
  if (e == hipSuccess) {
    moe::GroupedGemmArgs g{};
    g.a_routed = x_perm;
    g.a_shared = shared ? x : nullptr;
    g.a_routed_bytes = 2 * static_cast<int64_t>(d) * T * shape->top_k;
    g.a_shared_bytes = 2 * static_cast<int64_t>(d) * T;
    g.w_routed = w1;
    g.w3_routed = w3;
    g.w_shared = shared ? ws1 : nullptr;
    g.w3_shared = shared ? ws3 : nullptr;
    g.c_routed = w.h;
    g.c_shared = shared ? w.hs : nullptr;
    g.offsets = offsets;
    g.T = T;
    g.E = E;
    g.top_k = shape->top_k;
    g.K_r = g.K_s = d;
    g.N_r = H;
    g.N_s = Hs;
    g.dh_routed = w.dh;
    g.dh_shared = shared ? w.dhs : nullptr;
    g.da_routed = w.da;
    g.da_shared = shared ? w.das : nullptr;
    g.dc_routed = w.dc;
    g.dc_shared = shared ? w.dcs : nullptr;
    e = moe::launch_gemm_swiglu_bwd(g, s);
  }
  // dx = da W1 + dc W3  (W1, W3 [H, d] read as [K, N])
  bool dx_done = false;
  if (e == hipSuccess) e = routed_dgrad(w.da, w.dc, w1, w3, H, H, d, dx_perm, &dx_done);
  if (e == hipSuccess)
    e = launch(
        [&](moe::BwdSeg& q, int i) {
          const int Hh = seg_h(i);
          q.N = d; q.K = Hh; q.K2 = Hh;
          q.a = is_sh(i) ? w.das : w.da; q.a2 = is_sh(i) ? w.dcs : w.dc; q.lda = Hh;
          q.b = is_sh(i) ? ws1 : w1; q.b2 = is_sh(i) ? ws3 : w3; q.ldb = d;
          q.b_gstride = is_sh(i) ? 0 : static_cast<int64_t>(H) * d;
          q.c = is_sh(i) ? dx_shared : dx_perm; q.ldc = d;
        },
        moe::kBwdDgradKM, dx_done);
  // dW2 = dy^T h, then [dW1; dW3] = [da dc]^T x  (K = the group's rows)
  const WgradPlans wp = wgrad_plans(shape);
  if (e == hipSuccess)
    e = launch(
        [&](moe::BwdSeg& q, int i) {
          const int Hh = seg_h(i);
          q.M = d; q.N = Hh; q.M1 = d; q.split = wp.p[0].split;
          q.a = is_sh(i) ? dout : dy_perm; q.lda = d;
          q.b = is_sh(i) ? w.hs : w.h; q.ldb = Hh;
          q.c = is_sh(i) ? dws2 : dw2; q.ldc = Hh; q.c_gstride = static_cast<int64_t>(d) * Hh;
          q.part = w.wgrad_part + (i == 1 ? wp.p[0].slots[0] * d * seg_h(0) : 0);
        },
        moe::kBwdWgrad);
  if (e == hipSuccess)
    e = launch(
        [&](moe::BwdSeg& q, int i) {
          const int Hh = seg_h(i);
          q.M = 2 * Hh; q.N = d; q.M1 = Hh; q.split = wp.p[1].split;
          q.a = is_sh(i) ? w.das : w.da; q.a2 = is_sh(i) ? w.dcs : w.dc; q.lda = Hh;
          q.b = is_sh(i) ? x : x_perm; q.ldb = d;
          q.c = is_sh(i) ? dws1 : dw1; q.c2 = is_sh(i) ? dws3 : dw3; q.ldc = d;
          q.c_gstride = static_cast<int64_t>(Hh) * d;
          q.part = w.wgrad_part + (i == 1 ? wp.p[1].slots[0] * 2 * seg_h(0) * d : 0);
        },
        moe::kBwdWgrad);
  return hip_status(e);
}

moe_status moe_route_backward(const moe_shape* shape, const uint16_t* x, const float* w_router,
                              const int32_t* topk_idx, const float* topk_gate, const float* dgate,
                              float alpha, const uint16_t* dx_perm, const uint16_t* dx_shared,
                              const int32_t* pos, const uint16_t* d_residual, uint16_t* dx,
                              float* dw_router, void* workspace, size_t workspace_bytes,
                              void* stream) {
  moe_status st = check_bwd_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->tokens == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_gate || !dgate || !dx_perm || !pos || !dx || !dw_router)
    return MOE_ERR_INVALID_ARGUMENT;
  if ((shape->shared_hidden > 0) != (dx_shared != nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (!(alpha >= 0.0f) || alpha > 3.0e38f) return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x, dx_perm, dx, dx_shared ? dx_shared : dx, d_residual ? d_residual : dx};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_bwd_ws(shape, workspace, workspace_bytes)) != MOE_OK) return st;
  const BwdWorkspace w = carve_bwd(shape, workspace);
  return hip_status(moe::launch_route_bwd(
      x, w_router, topk_idx, topk_gate, dgate, alpha, dx_perm, dx_shared, pos, d_residual, dx,
      dw_router, w.scores, w.freq, w.dlogit, w.dwr_part, w.splits, shape->tokens, shape->d_model,
      shape->n_experts, shape->top_k, shape->seq_len, static_cast<hipStream_t>(stream)));
}

moe_status moe_update_bias(const moe_shape* shape, const int32_t* counts, float* bias,
                           float gamma, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!counts || !bias) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(moe::launch_update_bias(counts, bias, gamma, shape->tokens, shape->n_experts,
                                            shape->top_k, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
