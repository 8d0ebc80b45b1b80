// mla_api.cpp -- the C ABI of include/mla.h: argument checks, workspace
// layout and the launch sequence of the MLA attention kernels (mla.hip).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/mla.h"
#include "kernels.hpp"

namespace {

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }
moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe_status check_shape(const mla_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARGUMENT;
  if (s->batch < 0 || s->seq_len < 0 || s->max_len <= 0 || s->d_model <= 0 || s->n_heads <= 0 ||
      s->d_latent <= 0 || s->d_nope <= 0 || s->d_rope <= 0 || s->d_v <= 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!(s->rope_base > 1.0f) || !std::isfinite(s->rope_base)) return MOE_ERR_INVALID_ARGUMENT;
  if (s->seq_len > s->max_len) return MOE_ERR_INVALID_ARGUMENT;
  if (s->d_model % 64 || s->d_latent % 64 || (s->n_heads * s->d_v) % 64) return MOE_ERR_UNSUPPORTED;
  if (s->d_latent != 64 && s->d_latent != 128 && s->d_latent != 256) return MOE_ERR_UNSUPPORTED;
  if (s->n_heads > 16 || s->max_len > 65536) return MOE_ERR_UNSUPPORTED;
  if (s->d_nope % 8 || s->d_rope % 8 || s->d_nope + s->d_rope > 128 || s->d_rope > 64)
    return MOE_ERR_UNSUPPORTED;
  if (s->d_v != 8 && s->d_v != 16 && s->d_v != 32 && s->d_v != 64) return MOE_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(s->batch) * s->max_len >= (int64_t{1} << 31) || s->batch > 65535)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

struct MlaWorkspace {
  uint16_t* q;    // [tokens, H (d_nope + d_rope)]
  uint16_t* kvx;  // prefill: [tokens, H d_nope | H d_v]
  uint16_t* o;    // [tokens, H d_v]
  float* part;    // decode: [batch, H, max_len / 64, d_latent + 2] chunk partials
  uint16_t* qlat; // decode: [batch, H, d_latent] the queries in latent space
  size_t total;
};
MlaWorkspace carve(const mla_shape* s, int decode, void* base) {
  MlaWorkspace w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) / 256 * 256;
    return base ? reinterpret_cast<uint16_t*>(static_cast<char*>(base) + o) : nullptr;
  };
  const int64_t T = decode ? s->batch : static_cast<int64_t>(s->batch) * s->seq_len;
  const int64_t H = s->n_heads;
  w.q = take(2 * T * H * (s->d_nope + s->d_rope));
  w.kvx = take(decode ? 0 : 2 * T * H * (s->d_nope + s->d_v));
  w.o = take(2 * T * H * s->d_v);
  w.part = reinterpret_cast<float*>(
      take(decode ? 4 * T * H * ((s->max_len + 63) / 64) * static_cast<int64_t>(s->d_latent + 2) : 0));
  w.qlat = take(decode ? 2 * T * H * s->d_latent : 0);
  w.total = off;
  return w;
}

moe_status check_common(const mla_shape* s, const void* const* ptrs, int n, void* ws, size_t bytes,
                        int decode) {
  for (int i = 0; i < n; ++i)
    if (!ptrs[i] || !aligned16(ptrs[i])) return MOE_ERR_INVALID_ARGUMENT;
  if (!ws || bytes < carve(s, decode, nullptr).total || reinterpret_cast<uintptr_t>(ws) % 256)
    return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe::MlaGemmArgs projection(const mla_shape* s, int64_t tokens, const uint16_t* x,
                            const uint16_t* w_q, const uint16_t* w_dkv, const uint16_t* w_kr,
                            uint16_t* q, uint16_t* ckv, uint16_t* ckr, int seq,
                            const int32_t* pos) {
  moe::MlaGemmArgs g{};
  const int qw = s->d_nope + s->d_rope;
  g.M = static_cast<int>(tokens);
  g.n1 = s->n_heads * qw;
  g.n2 = g.n1 + s->d_latent;
  g.N = g.n2 + s->d_rope;
  g.K = s->d_model;
  g.a = x;
  g.lda = s->d_model;
  g.a_grp = g.M > 0 ? g.M : 1;
  g.a_grp_stride = 0;
  g.b0 = w_q;
  g.b1 = w_dkv;
  g.b2 = w_kr;
  g.q = q;
  g.ckv = ckv;
  g.ckr = ckr;
  g.qw = qw;
  g.dn = s->d_nope;
  g.dr = s->d_rope;
  g.dc = s->d_latent;
  g.max_len = s->max_len;
  g.seq = seq;
  g.pos = pos;
  g.log2_base = std::log2(s->rope_base);
  return g;
}

moe::MlaGemmArgs out_projection(const mla_shape* s, int64_t tokens, const uint16_t* o,
                                const uint16_t* w_o, const uint16_t* residual, uint16_t* out) {
  moe::MlaGemmArgs g{};
  g.M = static_cast<int>(tokens);
  g.N = s->d_model;
  g.K = s->n_heads * s->d_v;
  g.a = o;
  g.lda = g.K;
  g.a_grp = g.M > 0 ? g.M : 1;
  g.b0 = g.b1 = g.b2 = w_o;
  g.n1 = g.n2 = g.N;
  g.c = out;
  g.ldc = s->d_model;
  g.res = residual;
  return g;
}

moe::MlaAttnArgs attn(const mla_shape* s, const MlaWorkspace& w, const uint16_t* ckv,
                      const uint16_t* ckr) {
  moe::MlaAttnArgs a{};
  a.q = w.q;
  a.kvx = w.kvx;
  a.ckv = ckv;
  a.ckr = ckr;
  a.o = w.o;
  a.seq = s->seq_len;
  a.max_len = s->max_len;
  a.nh = s->n_heads;
  a.dc = s->d_latent;
  a.dn = s->d_nope;
  a.dr = s->d_rope;
  a.dv = s->d_v;
  a.scale = 1.0f / std::sqrt(static_cast<float>(s->d_nope + s->d_rope));
  return a;
}

}  // namespace

extern "C" {

moe_status mla_workspace_bytes(const mla_shape* shape, int decode, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  const moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  *bytes = carve(shape, decode ? 1 : 0, nullptr).total;
  return MOE_OK;
}

moe_status mla_prefill(const mla_shape* shape, const uint16_t* x, const uint16_t* w_q,
                       const uint16_t* w_dkv, const uint16_t* w_kr, const uint16_t* w_uk,
                       const uint16_t* w_uv, const uint16_t* w_o, const uint16_t* residual,
                       uint16_t* cache_kv, uint16_t* cache_kr, uint16_t* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const int64_t T = static_cast<int64_t>(shape->batch) * shape->seq_len;
  if (T == 0) return MOE_OK;
  if (T >= (int64_t{1} << 31) / 256) return MOE_ERR_UNSUPPORTED;
  const void* ptrs[] = {x, w_q, w_dkv, w_kr, w_uk, w_uv, w_o, cache_kv, cache_kr, out,
                        residual ? residual : out};
  if ((st = check_common(shape, ptrs, 11, workspace, workspace_bytes, 0)) != MOE_OK) return st;
  const MlaWorkspace w = carve(shape, 0, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // x -> q, latent, rotary key (the caches written at positions 0..S-1)
  moe::MlaGemmArgs g = projection(shape, T, x, w_q, w_dkv, w_kr, w.q, cache_kv, cache_kr,
                                  shape->seq_len, nullptr);
  hipError_t e = moe::launch_mla_gemm(g, moe::kMlaEpiProj, s);
  // every head's keys and values from the cached latents
  if (e == hipSuccess) {
    moe::MlaGemmArgs x2{};
    x2.M = static_cast<int>(T);
    x2.n1 = shape->n_heads * shape->d_nope;
    x2.N = x2.n1 + shape->n_heads * shape->d_v;
    x2.n2 = x2.N;
    x2.K = shape->d_latent;
    x2.a = cache_kv;
    x2.lda = shape->d_latent;
    x2.a_grp = shape->seq_len;
    x2.a_grp_stride = shape->max_len;
    x2.b0 = w_uk;
    x2.b1 = x2.b2 = w_uv;
    x2.c = w.kvx;
    x2.ldc = x2.N;
    e = moe::launch_mla_gemm(x2, moe::kMlaEpiPlain, s);
  }
  if (e == hipSuccess) e = moe::launch_mla_attn_prefill(attn(shape, w, cache_kv, cache_kr), shape->batch, s);
  if (e == hipSuccess)
    e = moe::launch_mla_gemm(out_projection(shape, T, w.o, w_o, residual, out), moe::kMlaEpiRes, s);
  return hip_status(e);
}

moe_status mla_decode(const mla_shape* shape, const uint16_t* x, const int32_t* pos,
                      const uint16_t* w_q, const uint16_t* w_dkv, const uint16_t* w_kr,
                      const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* w_o,
                      const uint16_t* residual, uint16_t* cache_kv, uint16_t* cache_kr,
                      uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const int64_t B = shape->batch;
  if (B == 0) return MOE_OK;
  if (!pos) return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x, w_q, w_dkv, w_kr, w_uk, w_uv, w_o, cache_kv, cache_kr, out,
                        residual ? residual : out};
  if ((st = check_common(shape, ptrs, 11, workspace, workspace_bytes, 1)) != MOE_OK) return st;
  const MlaWorkspace w = carve(shape, 1, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  moe::MlaGemmArgs g = projection(shape, B, x, w_q, w_dkv, w_kr, w.q, cache_kv, cache_kr, 0, pos);
  hipError_t e = moe::launch_mla_gemm(g, moe::kMlaEpiProj, s);
  if (e == hipSuccess) {
    moe::MlaAttnArgs a = attn(shape, w, cache_kv, cache_kr);
    a.w_uk = w_uk;
    a.w_uv = w_uv;
    a.pos = pos;
    a.part = w.part;
    a.qlat = w.qlat;
    e = moe::launch_mla_attn_decode(a, shape->batch, s);
  }
  if (e == hipSuccess)
    e = moe::launch_mla_gemm(out_projection(shape, B, w.o, w_o, residual, out), moe::kMlaEpiRes, s);
  return hip_status(e);
}

}  // extern "C"
