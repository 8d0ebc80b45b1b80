// api.cpp -- the extern "C" boundary of libmoe.so (declared in include/moe.h).
//
// Host-side only: argument checks (before anything is enqueued), workspace
// carve-up and kernel launches on the caller's stream.  No allocation, no
// synchronisation, no state beyond a per-device cache of the CU count.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>

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
  // grouped-GEMM operands are addressed with 32-bit byte offsets
  const int64_t widest = std::max<int64_t>({s->d_model, s->hidden, s->shared_hidden});
  if (2 * s->tokens * s->top_k * widest >= (int64_t{1} << 31) ||
      2 * static_cast<int64_t>(s->hidden) * s->d_model >= (int64_t{1} << 31) ||
      2 * static_cast<int64_t>(s->shared_hidden) * s->d_model >= (int64_t{1} << 31))
    return MOE_ERR_UNSUPPORTED;
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
  const void* ptrs[] = {x, x_perm ? x_perm : x, w1, w3, w2, ws1 ? ws1 : w1, ws3 ? ws3 : w1,
                        ws2 ? ws2 : w1};
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
  hipError_t e = moe::launch_gemm_swiglu(g1, s);
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

moe_status moe_update_bias(const moe_shape* shape, const int32_t* counts, float* bias,
                           float gamma, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!counts || !bias) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(moe::launch_update_bias(counts, bias, gamma, shape->tokens, shape->n_experts,
                                            shape->top_k, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
