/*
 * moe.h -- C ABI of libmoe.so: the DeepSeekMoE layer forward on gfx950.
 *
 * Four calls make one layer forward, in this order, on one HIP stream:
 *   moe_route -> moe_permute -> moe_grouped_ffn -> moe_combine
 * and, once per training step and layer, moe_update_bias.  In a pre-norm
 * residual block moe_rmsnorm comes first and the block's input is
 * moe_combine's residual.
 *
 * Pages cited (title, then section):
 *   [ZH] "190行JAX复刻DeepSeek V3" (openai-hub.com news)
 *   [VI] "DeepSeek V3 viết lại bằng 190 dòng JAX thuần" (lehuy.net)
 *
 * Conventions shared by every call
 *   - Every array pointer is a DEVICE pointer owned by the caller.  The
 *     library allocates nothing, keeps no state between calls and never
 *     synchronises: each call only enqueues kernels on `stream` (a
 *     hipStream_t passed as void*; NULL means the default stream) and returns.
 *   - bf16 arrays are passed as uint16_t bit patterns.  Layouts are
 *     row-major and contiguous.  Every bf16 array must start on a 16-byte
 *     boundary (the kernels move 16-byte chunks); a misaligned one returns
 *     MOE_ERR_INVALID_ARGUMENT.  The workspace must start on a 256-byte
 *     boundary (else MOE_ERR_WORKSPACE).
 *   - Arguments are checked on the host before anything is enqueued.  A bad
 *     argument returns MOE_ERR_INVALID_ARGUMENT (or MOE_ERR_UNSUPPORTED for a
 *     legal shape this build does not handle, MOE_ERR_WORKSPACE for a too
 *     small workspace) and nothing is launched.  A failed launch returns
 *     MOE_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *     synchronisation, as with any stream API.
 *   - tokens == 0 is valid: nothing is computed, except that moe_permute
 *     still writes zero counts and offsets.
 *   - Outputs must not overlap inputs (except `bias` in moe_update_bias).
 *   - Calls are stateless and thread-safe; calls that share a workspace must
 *     be ordered (same stream, or synchronised).  The one exception is
 *     moe_permute_noalloc, whose static per-GPU scratch is shared by all its
 *     calls on that GPU (see there).
 *
 * Supported shapes: 1 <= E <= 1024, 1 <= k <= min(E, 32), d, H and Hs
 * multiples of 64, T*(k+1) < 2^31.  When seq_len > 0 it must divide T.
 * The grouped GEMMs address x, and one expert's weights, with 32-bit byte
 * offsets: 2*T*d, 2*H*d and 2*Hs*d must stay below 2^31 (else
 * MOE_ERR_UNSUPPORTED).  x_perm, h and the outputs have no such limit.  The
 * backward calls also need 2*T*k*max(d, H, Hs) < 2^31.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4,
  MOE_ERR_SCRATCH_LIMIT = 5 /* moe_permute_noalloc: shape beyond its static scratch */
} moe_status;

/* Layer shape.
 *   tokens        T, rows of x
 *   d_model       d
 *   n_experts     E routed experts (16 in the mini model, 256 in the official
 *                 shape: [ZH] 190行代码到底装进了什么 and the table in 先说结论)
 *   top_k         k experts chosen per token (4 mini, 8 official)
 *   hidden        H, hidden size of a routed expert
 *   shared_hidden Hs, hidden size of the always-on shared expert; 0 = none
 *   seq_len       S, tokens per sequence for the balance statistic; 0 = off */
typedef struct moe_shape {
  int64_t tokens;
  int32_t d_model;
  int32_t n_experts;
  int32_t top_k;
  int32_t hidden;
  int32_t shared_hidden;
  int32_t seq_len;
} moe_shape;

/* Static description of a status code; never NULL. */
const char* moe_status_str(int status);

/* Bytes of device workspace the calls need for `shape` (one buffer serves all
 * five calls of a layer).  The caller allocates it (256-byte alignment or
 * better) and passes it with its size.  Writes *bytes; MOE_ERR_INVALID_ARGUMENT
 * / MOE_ERR_UNSUPPORTED for a bad shape.  Host only: launches nothing. */
moe_status moe_workspace_bytes(const moe_shape* shape, size_t* bytes);

/* Routing (steps: router GEMM, affinity, biased top-k, gates, balance
 * statistic).  For every token t:
 *   logit[e] = fp32 fused multiply-add chain over d in ascending order of
 *              f32(x[t,i]) * w_router[i,e]
 *   s[e]     = sigmoid(logit[e]) evaluated in fp64, rounded once to fp32
 *   key[e]   = s[e] + bias[e]                       (fp32)
 *   topk_idx[t,j]  = expert with the j-th largest key; equal keys go to the
 *                    lower index; NaN keys rank below all others
 *   topk_gate[t,j] = s[idx_j] / sum_j' s[idx_j'] (fp32 sum in slot order;
 *                    1/k if that sum is 0)
 *   margin[t]      = key_(k) - key_(k+1) (fp32), +inf when k == E
 * The bias moves the choice of experts and never the gate values
 * ([ZH] 最有价值的实验:无辅助损失均衡真的有效; [VI] Những gì có trong 190 dòng
 * code).  When shape->seq_len > 0 and seq_balance != NULL, for each sequence b
 * of S tokens: seq_balance[b] = alpha * sum_i f_i P_i with
 * f_i = E/(kS) * #{t in b choosing i}, P_i = mean over t in b of
 * s[t,i]/sum_j s[t,j] -- the small sequence-wise balance loss, alpha = 1e-4 in
 * [ZH] 最有价值的实验 (formula: stated reading).
 *   x          [T, d]  bf16            (in)
 *   w_router   [d, E]  fp32            (in)
 *   bias       [E]     fp32            (in)
 *   topk_idx   [T, k]  int32           (out)
 *   topk_gate  [T, k]  fp32            (out)
 *   margin     [T]     fp32 or NULL    (out)
 *   seq_balance[T/S]   fp32 or NULL    (out)
 *   workspace  >= moe_workspace_bytes(shape) bytes                        */
moe_status moe_route(const moe_shape* shape, const uint16_t* x, const float* w_router,
                     const float* bias, int32_t* topk_idx, float* topk_gate, float* margin,
                     float* seq_balance, float alpha, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Grouping by expert (steps: histogram, scan, permutation).
 *   counts[e]    = number of (t, j) with topk_idx[t,j] == e (the per-expert
 *                  load behind the bias rule, [ZH] 最有价值的实验)
 *   offsets[e]   = sum_{e' < e} counts[e'], offsets[E] = T*k
 *   perm_src[r]  = token of row r; rows offsets[e] .. offsets[e+1]-1 hold the
 *                  tokens that chose e in ascending token order
 *   pos[t,j]     = row of (t, topk_idx[t,j])
 *   x_perm[r,:]  = x[perm_src[r], :] when x and x_perm are both non-NULL
 *                  (optional materialised gather; moe_grouped_ffn can gather
 *                  on the fly instead)
 * Only the chosen experts will run -- the sparse dispatch the pages' dense
 * reference does without ([VI] Những gì đã được đơn giản hóa).
 *   topk_idx [T, k] int32 (in; every entry must lie in [0, E) and a token's k
 *            entries must be distinct -- moe_route guarantees both; other
 *            input gives unspecified rows but no out-of-bounds access)
 *   counts [E], offsets [E+1], perm_src [T*k], pos [T, k] int32 (out)
 *   x [T, d] bf16 or NULL (in); x_perm [T*k, d] bf16 or NULL (out)      */
moe_status moe_permute(const moe_shape* shape, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* perm_src, int32_t* pos, const uint16_t* x,
                       uint16_t* x_perm, void* workspace, size_t workspace_bytes, void* stream);

/* moe_permute without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments (minus the workspace), results, checks
 * and error codes as moe_permute.  Its per-block count and first-row tables
 * live in a static 2 MiB device array of the library, one per GPU, held
 * until the process ends; the call allocates nothing.  Limit: the two tables
 * take 2 * 4 * ceil(T/256) * E bytes (each rounded up to 256), at most 2 MiB,
 * i.e. about T * E <= 67 million (T <= 262144 at E = 256); a larger shape
 * returns MOE_ERR_SCRATCH_LIMIT and nothing is enqueued.  The array of the
 * current device (hipGetDevice) is used, so `stream` must belong to that
 * device.  Every call on one GPU shares that array: calls that may overlap
 * on one GPU (different streams, or threads without ordering) race and must
 * be serialised by the caller. */
moe_status moe_permute_noalloc(const moe_shape* shape, const int32_t* topk_idx, int32_t* counts,
                               int32_t* offsets, int32_t* perm_src, int32_t* pos,
                               const uint16_t* x, uint16_t* x_perm, void* stream);

/* Expert feed-forward networks over the expert groups, plus the shared
 * expert on every token (steps: grouped GEMM 1 with SwiGLU, grouped GEMM 2).
 * For row r in group e (offsets[e] <= r < offsets[e+1]) with token
 * t = perm_src[r]:
 *   h        = bf16( silu(W1[e] x_t) * (W3[e] x_t) )    fp32 accumulation
 *   y_perm[r]= bf16( W2[e] h )                          fp32 accumulation
 * and y_shared[t] likewise with ws1, ws3, ws2.  The experts are feed-forward
 * networks and one shared expert always runs ([ZH] 190行代码到底装进了什么);
 * the gated-SiLU form is a stated reading.  Experts with no rows cost nothing.
 *   x        [T, d] bf16 (in), used when x_perm is NULL (rows gathered through
 *            perm_src); x_perm [T*k, d] bf16 or NULL (in)
 *   perm_src [T*k], offsets [E+1] int32 (in, from moe_permute)
 *   w1, w3   [E, H, d] bf16; w2 [E, d, H] bf16 (in)
 *   ws1, ws3 [Hs, d] bf16; ws2 [d, Hs] bf16 (in; NULL iff Hs == 0)
 *   y_perm   [T*k, d] bf16 (out); y_shared [T, d] bf16 (out; NULL iff Hs == 0)
 *   workspace >= moe_workspace_bytes(shape) bytes (holds h, and the work
 *            counters of the GEMM launches, which the call zeroes itself)  */
moe_status moe_grouped_ffn(const moe_shape* shape, const uint16_t* x, const uint16_t* x_perm,
                           const int32_t* perm_src, const int32_t* offsets, const uint16_t* w1,
                           const uint16_t* w3, const uint16_t* w2, const uint16_t* ws1,
                           const uint16_t* ws3, const uint16_t* ws2, uint16_t* y_perm,
                           uint16_t* y_shared, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Gate-weighted combine with the shared expert (step: combine):
 *   out[t] = bf16( residual[t] + y_shared[t] + sum_j topk_gate[t,j] * y_perm[pos[t,j]] )
 * accumulated in fp32.  The shared expert's output is added to the routed
 * mixture ([ZH] 190行代码到底装进了什么).  residual (the Transformer block's
 * residual stream) and y_shared may be NULL.
 *   y_perm [T*k, d], y_shared [T, d] or NULL, residual [T, d] or NULL: bf16 (in)
 *   topk_gate [T, k] fp32, pos [T, k] int32 (in); out [T, d] bf16 (out)   */
moe_status moe_combine(const moe_shape* shape, const uint16_t* y_perm, const uint16_t* y_shared,
                       const float* topk_gate, const int32_t* pos, const uint16_t* residual,
                       uint16_t* out, void* stream);

/* RMSNorm of the token rows, the input of the MoE in a pre-norm residual
 * block x_next = x + MoE(RMSNorm(x)): for every row t,
 *   out[t,i] = bf16( x[t,i] / sqrt(mean_j x[t,j]^2 + eps) * gain[i] )
 * with the mean of squares accumulated in fp32.  The pages list RMSNorm among
 * the model's functions ([ZH] "纯JAX"也需要打一个小星号) and place the MoE in a
 * residual Transformer block ([ZH] 先说结论); the pre-norm placement is a
 * stated reading.  The block's residual add is moe_combine's `residual`.
 * Only shape->tokens and shape->d_model are used (the shape is checked as
 * for the other calls).
 *   x [T, d] bf16 (in); gain [d] fp32 (in, 16-byte aligned); out [T, d] bf16
 *   (out, must not overlap x); eps >= 0 and finite (else
 *   MOE_ERR_INVALID_ARGUMENT; 1e-6 in the workloads)                   */
moe_status moe_rmsnorm(const moe_shape* shape, const uint16_t* x, const float* gain, float eps,
                       uint16_t* out, void* stream);

/* Auxiliary-loss-free balancing (step: bias update), once per step and layer:
 *   bias[i] = bias[i] + gamma * sgn(T*k - E*counts[i])      (fp32; sgn(0) = 0)
 * i.e. an overloaded expert's bias goes down and an idle one's goes up, at
 * speed gamma (1e-3 in [ZH] 最有价值的实验).  The sign is taken on integers.
 *   counts [E] int32 (in, from moe_permute); bias [E] fp32 (in/out)      */
moe_status moe_update_bias(const moe_shape* shape, const int32_t* counts, float* bias,
                           float gamma, void* stream);

/* ---- Backward (training) --------------------------------------------------
 * The pages' workload is training (12000 AdamW steps, [ZH] 如何在Mac上复现) on
 * a loss that adds the small sequence-wise balance loss ([ZH] 多Token预测也被保
 * 留了); the per-expert bias stays out of the loss and gets no gradient ([ZH]
 * 最有价值的实验).  With the forward's choice of experts held fixed, three calls
 * give the gradient of  sum_t <dout[t], out[t]> + sum_b L_b  with respect to
 * the layer's input and every weight, in this order on one stream:
 *   moe_combine_backward -> moe_grouped_ffn_backward -> moe_route_backward
 * They read the forward's results (choices, gates, offsets, perm_src, pos,
 * x_perm -- moe_permute must have materialised it -- and y_perm) and a
 * workspace of moe_backward_workspace_bytes().  Input gradients are bf16,
 * weight gradients fp32 (the master weights are fp32, [VI] Những gì có trong
 * 190 dòng code).  Conventions as above (device pointers, 16-byte aligned
 * bf16 arrays, checks before launch, no allocation). */

/* Bytes of device workspace for the three backward calls (256-aligned). */
moe_status moe_backward_workspace_bytes(const moe_shape* shape, size_t* bytes);

/* Through the combine out = r + y_shared + sum_j g_j y_perm[pos[t,j]]:
 *   dy_perm[pos[t,j]] = bf16( topk_gate[t,j] * dout[t] )   (expert-grouped rows)
 *   dgate[t,j]        = <dout[t], y_perm[pos[t,j]]>          (fp32)
 * The shared expert's and the residual's gradient is dout itself.
 *   dout [T, d], y_perm [T*k, d] bf16 (in); topk_gate [T, k] fp32, pos [T, k]
 *   int32 (in); dy_perm [T*k, d] bf16, dgate [T, k] fp32 (out)          */
moe_status moe_combine_backward(const moe_shape* shape, const uint16_t* dout, const uint16_t* y_perm,
                                const float* topk_gate, const int32_t* pos, uint16_t* dy_perm,
                                float* dgate, void* stream);

/* Through the experts, per expert group (rows offsets[e] .. offsets[e+1]-1,
 * x_perm the gathered inputs, dy_perm from moe_combine_backward) and for the
 * shared expert on every token (inputs x, upstream gradient dout):
 *   a, c = x W1^T, x W3^T (recomputed), h = bf16(silu(a) c)
 *   dh = bf16(dy W2), da = bf16(dh c silu'(a)), dc = bf16(dh silu(a))
 *   dx_perm (dx_shared) = bf16(da W1 + dc W3)
 *   dW2 = dy^T h,  dW1 = da^T x,  dW3 = dc^T x   (fp32; zero for an expert
 *   with no rows: unchosen experts get no gradient)
 *   x [T, d], x_perm [T*k, d], dy_perm [T*k, d], dout [T, d] bf16 (in);
 *   offsets [E+1] int32 (in); w1, w3 [E, H, d], w2 [E, d, H], ws1, ws3 [Hs, d],
 *   ws2 [d, Hs] bf16 (in); dx_perm [T*k, d], dx_shared [T, d] bf16 (out);
 *   dw1, dw3 [E, H, d], dw2 [E, d, H], dws1, dws3 [Hs, d], dws2 [d, Hs] fp32
 *   (out).  The shared arguments are NULL iff Hs == 0.                   */
moe_status moe_grouped_ffn_backward(const moe_shape* shape, const uint16_t* x,
                                    const uint16_t* x_perm, const int32_t* offsets,
                                    const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                                    const uint16_t* ws1, const uint16_t* ws3, const uint16_t* ws2,
                                    const uint16_t* dy_perm, const uint16_t* dout,
                                    uint16_t* dx_perm, uint16_t* dx_shared, float* dw1, float* dw3,
                                    float* dw2, float* dws1, float* dws3, float* dws2,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Through the routing: the scores s = sigmoid(x W_r) are recomputed (the
 * forward's fp32 chain); the gates g_j = s_j / sum s over the chosen experts
 * give ds_j = (dgate_j - sum_j' dgate_j' g_j') / sum; with shape->seq_len > 0
 * and alpha > 0 the balance statistic alpha sum_i f_i P_i of each sequence
 * adds ds_m += alpha/S (f_m - sum_i f_i s_i/Z) / Z (Z = sum_e s_e, f as in
 * moe_route); dlogit = ds s (1 - s).  Then
 *   dx[t]     = bf16( d_residual[t] + dx_shared[t] + sum_j dx_perm[pos[t,j]]
 *                     + sum_e dlogit[t,e] W_r[:,e] )
 *   dw_router = x^T dlogit  (fp32, [d, E]);  the bias gets no gradient.
 *   x [T, d] bf16, w_router [d, E] fp32, topk_idx / pos [T, k] int32,
 *   topk_gate / dgate [T, k] fp32, dx_perm [T*k, d] bf16 (in); dx_shared
 *   [T, d] bf16 (in; NULL iff Hs == 0); d_residual [T, d] bf16 or NULL (in);
 *   alpha >= 0; dx [T, d] bf16, dw_router [d, E] fp32 (out)              */
moe_status moe_route_backward(const moe_shape* shape, const uint16_t* x, const float* w_router,
                              const int32_t* topk_idx, const float* topk_gate, const float* dgate,
                              float alpha, const uint16_t* dx_perm, const uint16_t* dx_shared,
                              const int32_t* pos, const uint16_t* d_residual, uint16_t* dx,
                              float* dw_router, void* workspace, size_t workspace_bytes,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
