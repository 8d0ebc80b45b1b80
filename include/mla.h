/*
 * mla.h -- C ABI of the MLA attention in libmoe.so (gfx950): the other half
 * of the DeepSeek-V3 block, with the compressed key/value cache.
 *
 * Multi-head latent attention as the pages describe it ([ZH] "190行JAX复刻
 * DeepSeek V3" (openai-hub.com news), section 190行代码到底装进了什么; [VI]
 * "DeepSeek V3 viết lại bằng 190 dòng JAX thuần" (lehuy.net), section Những
 * gì có trong 190 dòng code): per token and layer the cache holds a latent of
 * d_latent numbers (128) and one rotary key of d_rope numbers (16) shared by
 * all heads, 144 numbers instead of the 480 that plain attention with 6 heads
 * of 48-number keys and 32-number values keeps.  With x a token row at
 * position p of its sequence:
 *   q_h      = W_q[h] x            (d_nope content + d_rope rotary numbers;
 *                                   the rotary part turned by rope(., p))
 *   c        = W_dkv x             (cached latent)
 *   k_r      = rope(W_kr x, p)     (cached rotary key)
 *   k_nope_h = W_uk[h] c,   v_h = W_uv[h] c
 *   o_h(i)   = sum_{s<=i} softmax_s((q_nope_h.k_nope_h(s) + q_rope_h.k_r(s))
 *                                   / sqrt(d_nope + d_rope)) v_h(s)
 *   out      = residual + W_o [o_1 .. o_H]
 * rope(u, p) turns each pair (u[2m], u[2m+1]) by p * rope_base^(-2m/d_rope).
 *
 * Weights are bf16 and stored [N, K] (K contiguous): w_q [H (d_nope+d_rope),
 * d], w_dkv [d_latent, d], w_kr [d_rope, d], w_uk [H d_nope, d_latent],
 * w_uv [H d_v, d_latent], w_o [d, H d_v].  Caches are bf16 [batch, max_len,
 * d_latent] and [batch, max_len, d_rope].  Stored intermediates (q, c, k_r,
 * the prefill's decompressed keys and values, the heads' outputs) are bf16;
 * sums and the softmax are fp32.
 *
 * Conventions are those of moe.h: device pointers owned by the caller, bf16
 * arrays as uint16_t on 16-byte boundaries, a 256-byte aligned workspace,
 * arguments checked on the host before anything is enqueued, nothing
 * allocated, calls only enqueue work on `stream`.
 *
 * Supported: d_model and n_heads*d_v multiples of 64; d_latent in {64, 128,
 * 256}; d_nope, d_rope multiples of 8 with d_nope + d_rope <= 128; d_v in
 * {8, 16, 32, 64}; 1 <= n_heads <= 16; seq_len <= max_len <= 65536;
 * batch * max_len < 2^31, batch <= 65535.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mla_shape {
  int32_t batch;     /* sequences */
  int32_t seq_len;   /* mla_prefill: tokens per sequence (positions 0..seq_len-1) */
  int32_t max_len;   /* positions each sequence's cache holds */
  int32_t d_model;
  int32_t n_heads;
  int32_t d_latent;  /* cached latent per token (128 in the mini model) */
  int32_t d_nope;    /* content part of a head's key and query (32) */
  int32_t d_rope;    /* rotary part, one key shared by the heads (16) */
  int32_t d_v;       /* value per head (32) */
  float rope_base;   /* 10000 */
} mla_shape;

/* Bytes of device workspace for mla_prefill (decode = 0) or mla_decode
 * (decode = 1) of this shape (256-aligned). */
moe_status mla_workspace_bytes(const mla_shape* shape, int decode, size_t* bytes);

/* Prefill: batch sequences of seq_len tokens, x [batch*seq_len, d] bf16
 * (sequence-major), positions 0..seq_len-1.  Writes both caches at positions
 * 0..seq_len-1 (other positions untouched) and out [batch*seq_len, d] bf16 =
 * residual + attention; residual [batch*seq_len, d] bf16 or NULL.  The keys
 * and values of every head are decompressed from the latents (the pages'
 * form) into the workspace. */
moe_status mla_prefill(const mla_shape* shape, const uint16_t* x, const uint16_t* w_q,
                       const uint16_t* w_dkv, const uint16_t* w_kr, const uint16_t* w_uk,
                       const uint16_t* w_uv, const uint16_t* w_o, const uint16_t* residual,
                       uint16_t* cache_kv, uint16_t* cache_kr, uint16_t* out, void* workspace,
                       size_t workspace_bytes, void* stream);

/* One decoding step: sequence b's new token x[b] (x [batch, d] bf16) sits at
 * position pos[b] (pos [batch] int32, device): its latent and rotary key are
 * written at pos[b] and it attends to positions 0..pos[b] of its cache,
 * which must hold the earlier tokens.  out [batch, d] bf16 = residual (NULL
 * allowed) + attention.  A sequence whose pos[b] lies outside [0, max_len)
 * gets a zero out row (plus its residual) and leaves its cache untouched.
 * The attention reads only the cache: W_uk is applied to the query (q_nope^T
 * W_uk[h] against each latent) and W_uv to the attended latent, which equals
 * the explicit decompression up to rounding order; the cached positions are
 * scored in chunks of 64 whose partial sums the workspace holds. */
moe_status mla_decode(const mla_shape* shape, const uint16_t* x, const int32_t* pos,
                      const uint16_t* w_q, const uint16_t* w_dkv, const uint16_t* w_kr,
                      const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* w_o,
                      const uint16_t* residual, uint16_t* cache_kv, uint16_t* cache_kr,
                      uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
