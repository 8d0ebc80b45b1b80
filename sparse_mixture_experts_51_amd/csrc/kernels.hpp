// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to libmoe.so).
// Each launcher enqueues on `stream` and returns the launch status; shapes are
// validated by the C ABI layer before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Workspace carve-up shared by the five calls of one layer.
struct Workspace {
  float* scores;          // [T, E] fp32 sigmoid scores
  double* tok_sum;        // [T] fp64 sum of a token's scores (balance statistic)
  double* seq_p;          // [nseq, nsplit, E] fp64 partial sums of normalised scores
  int32_t* seq_cnt;       // [nseq, nsplit, E] int32 partial choice counts
  int32_t* blk_cnt;       // [nblk, E] per-token-block expert counts
  int32_t* blk_base;      // [nblk, E] first row of each (block, expert)
  uint16_t* h_routed;     // [T*k, H] bf16 hidden activations, expert-grouped rows
  uint16_t* h_shared;     // [T, Hs] bf16 hidden activations of the shared expert
  int32_t* unit_counters; // [kUnitCounters] work counters of the grouped-GEMM launches
  size_t total;
};

constexpr int kPermTokens = 256;  // tokens per block of the permutation kernels
int perm_block_tokens(int64_t T);

int seq_splits(int64_t T, int S);
// Balance-statistic partials per sequence that the workspace holds.
int seq_partials_capacity(int64_t T, int S);
Workspace carve_workspace(void* base, int64_t T, int d, int E, int k, int H, int Hs, int S);

// Number of compute units of the current device (cached per device).
int device_cus();

hipError_t launch_router_scores(const uint16_t* x, const float* w_router, float* scores,
                                int64_t T, int d, int E, hipStream_t s);
// Router, selection and balance statistic in one pass when one block can hold
// all experts (E <= 64); *done is false when the shape takes the general path.
hipError_t launch_route_fused(const uint16_t* x, const float* w_router, const float* bias,
                              int32_t* idx, float* gate, float* margin, double* seq_p,
                              int32_t* seq_cnt, float* seq_out, float alpha, int64_t T, int d,
                              int E, int k, int S, hipStream_t s, bool* done);
hipError_t launch_select(const float* scores, const float* bias, int32_t* idx, float* gate,
                         float* margin, double* tok_sum, int64_t T, int E, int k, hipStream_t s);
hipError_t launch_seq_balance(const float* scores, const double* tok_sum, const int32_t* idx,
                              double* seq_p, int32_t* seq_cnt, float* out, float alpha,
                              int64_t T, int E, int k, int S, hipStream_t s);

hipError_t launch_permute(const int32_t* idx, int32_t* counts, int32_t* offsets,
                          int32_t* perm_src, int32_t* pos, const uint16_t* x, uint16_t* x_perm,
                          int32_t* blk_cnt, int32_t* blk_base, int64_t T, int d, int E, int k,
                          hipStream_t s);

// Grouped GEMM over E expert groups (rows offsets[e]..offsets[e+1]) plus an
// optional shared group of T rows.
struct GroupedGemmArgs {
  // A operand (row-major, K contiguous)
  const uint16_t* a_routed;
  const int32_t* a_row_map;  // NULL: A row = group row; else A row = a_row_map[group row]
  const uint16_t* a_shared;  // shared group's A rows (row t), NULL if no shared group
  int64_t a_routed_bytes, a_shared_bytes;  // extents of the A buffers (bounds of the loads)
  // B operand: weights [N_rows, K] per group, K contiguous
  const uint16_t* w_routed;   // [E, N, K]   (gate projection W1 for the SwiGLU stage)
  const uint16_t* w3_routed;  // [E, N, K]   up projection W3 (SwiGLU stage only)
  const uint16_t* w_shared;   // [Ns, Ks]
  const uint16_t* w3_shared;
  uint16_t* c_routed;   // [T*k, N]
  uint16_t* c_shared;   // [T, Ns]
  const int32_t* offsets;
  int64_t T;
  int E;
  int top_k;     // choices per token (tile configuration heuristic)
  int K_r, K_s;  // reduction lengths
  int N_r, N_s;  // output columns
  // SwiGLU stage of the backward (launch_gemm_swiglu_bwd): dh in, c = h, and
  // the derivatives da, dc out, all [rows, N] like c
  const uint16_t* dh_routed;
  const uint16_t* dh_shared;
  uint16_t* da_routed;
  uint16_t* da_shared;
  uint16_t* dc_routed;
  uint16_t* dc_shared;
  // Input gradients (launch_gemm_dgrad): the weights are stored [K, N] (K
  // major) -- w_routed [E][K_r][N_r], then K2_r more rows of K from w3_routed
  // [E][K2_r][N_r] against the A rows of a2_routed (row stride K_r too)
  const uint16_t* a2_routed;
  int K2_r;
  // Per-XCD unit counters (16 ints, zero at launch: the first 8 for this
  // launch, the next 8 for the shared expert's own launch beside streaming
  // tiles).  With them the loader-wave all-DMA tile hands out units in order
  // as blocks become free; NULL keeps the static round-robin order.
  int32_t* unit_counter;
};
constexpr int kUnitCounters = 32;  // two launches of 16
hipError_t launch_zero_counters(int32_t* p, int n, hipStream_t s);
hipError_t launch_gemm_swiglu(const GroupedGemmArgs& a, hipStream_t s);
// The SwiGLU stage again in the backward: the same tiles, MFMA order and h
// as the forward launch on the same shape, with h, da and dc written.
hipError_t launch_gemm_swiglu_bwd(const GroupedGemmArgs& a, hipStream_t s);
// C = A W (+ A2 W3) with K-major weights, routed groups only, on the
// streaming tile; hipErrorNotSupported for shapes it does not take (the
// caller then uses the backward's own kernel).
hipError_t launch_gemm_dgrad(const GroupedGemmArgs& a, hipStream_t s);
hipError_t launch_gemm_down(const GroupedGemmArgs& a, hipStream_t s);

hipError_t launch_combine(const uint16_t* y_perm, const uint16_t* y_shared, const float* gate,
                          const int32_t* pos, const uint16_t* residual, uint16_t* out,
                          int64_t T, int d, int k, hipStream_t s);
// Grouped GEMMs of the backward (bwd_gemm.hip): C_g = A_g B_g^T summed over K,
// per group g of consecutive rows.  A launch covers up to two segments of
// groups with their own operands and sizes (the shared expert: one group of
// `rows` rows; the routed experts: `groups` groups delimited by `offsets`).
struct BwdSeg {
  int groups;              // groups of the segment
  const int32_t* offsets;  // [groups + 1] first row of each group, or NULL (one group of `rows`)
  int rows;
  int M, N;                // output size that is not a group's rows (wgrad: M x N per group;
                           // input gradients: N columns)
  int K, K2;               // input gradients: K from a / b, then K2 more from a2 / b2
  int M1;                  // wgrad: output rows below M1 from a (into c), the rest from a2 (into c2)
  int split;               // wgrad: rows per split of a group's rows (0: none)
  const uint16_t* a;
  const uint16_t* a2;
  int64_t lda;
  const uint16_t* b;
  const uint16_t* b2;
  int64_t ldb, b_gstride;
  void* c;                 // bf16 rows [rows, N] (input gradients) or fp32 [groups][M1][N] (wgrad)
  void* c2;                // wgrad: fp32 [groups][M - M1][N]
  int64_t ldc, c_gstride;
  float* part;             // wgrad with split: partial sums [slots][M][N]
};
struct BwdGemmArgs {
  BwdSeg seg[2];
  int nseg;                // 1 or 2; the groups of seg[0] come first in the unit order
};
constexpr int kBwdDgradKM = 0;    // A K-contiguous, B stored [K, N], bf16 out
constexpr int kBwdWgrad = 2;      // both operands K-major rows, fp32 out
hipError_t launch_bwd_gemm(const BwdGemmArgs& a, int kind, hipStream_t s);
// Weight-gradient splits: rows per split (0: none) and the partial-sum slots
// a segment may need, for one launch over segments of total_rows[i] rows in
// groups[i] groups with tiles of M[i] x N[i] outputs.
struct WgradPlan {
  int split;
  int64_t slots[2];
  int64_t part_floats;  // slots[0] * M[0] * N[0] + slots[1] * M[1] * N[1]
};
WgradPlan plan_wgrad(int nseg, const int64_t* total_rows, const int* groups, const int* M,
                     const int* N);

hipError_t launch_combine_bwd(const uint16_t* dout, const uint16_t* y_perm, const float* gate,
                              const int32_t* pos, uint16_t* dy_perm, float* dgate, int64_t T,
                              int d, int k, hipStream_t s);
hipError_t launch_route_bwd(const uint16_t* x, const float* w_router, const int32_t* idx,
                            const float* gate, const float* dgate, float alpha,
                            const uint16_t* dx_perm, const uint16_t* dx_shared,
                            const int32_t* pos, const uint16_t* d_residual, uint16_t* dx,
                            float* dw_router, float* scores, float* freq, float* dlogit,
                            float* dwr_part, int dwr_splits, int64_t T, int d, int E, int k,
                            int S, hipStream_t s);
int route_bwd_splits(int64_t T);

// MLA attention (mla.hip)
struct MlaGemmArgs {
  int M, N, K;
  const uint16_t* a;           // A rows [.., K]: output row t reads row (t / a_grp) a_grp_stride + t % a_grp
  int64_t lda;
  int a_grp, a_grp_stride;
  const uint16_t* b0;          // B rows [N, K]: rows < n1 from b0, < n2 from b1, the rest from b2
  const uint16_t* b1;
  const uint16_t* b2;
  int n1, n2;
  uint16_t* c;                 // plain / residual epilogues: C [M, ldc]
  int64_t ldc;
  const uint16_t* res;         // residual [M, ldc] or NULL
  // projection epilogue: columns < n1 -> q [M, n1] (head blocks of qw, the
  // last dr of each turned), < n2 -> latent cache, the rest -> rotary cache
  uint16_t* q;
  uint16_t* ckv;
  uint16_t* ckr;
  int qw, dn, dr, dc, max_len;
  int seq;                     // > 0: token t is position t % seq of sequence t / seq
  const int32_t* pos;          // seq == 0: token t is sequence t at position pos[t]
  float log2_base;
};
constexpr int kMlaEpiProj = 0, kMlaEpiPlain = 1, kMlaEpiRes = 2;
hipError_t launch_mla_gemm(const MlaGemmArgs& a, int epi, hipStream_t s);
struct MlaAttnArgs {
  const uint16_t* q;    // [tokens, nh (dn + dr)]
  const uint16_t* kvx;  // prefill: decompressed [tokens, nh dn | nh dv]
  const uint16_t* ckv;  // caches [batch, max_len, dc] and [.., dr]
  const uint16_t* ckr;
  const uint16_t* w_uk;  // decode: [nh dn, dc], [nh dv, dc]
  const uint16_t* w_uv;
  const int32_t* pos;   // decode positions
  uint16_t* o;          // [tokens, nh dv]
  float* part;          // decode: per (sequence, head, 64 positions) max, sum, weighted latent
  uint16_t* qlat;       // decode: [batch, nh, dc] the heads' queries in latent space (bf16)
  int seq, max_len, nh, dc, dn, dr, dv;
  float scale;
};
hipError_t launch_mla_attn_prefill(const MlaAttnArgs& a, int batch, hipStream_t s);
hipError_t launch_mla_attn_decode(const MlaAttnArgs& a, int batch, hipStream_t s);

hipError_t launch_rmsnorm(const uint16_t* x, const float* gain, float eps, uint16_t* out,
                          int64_t T, int d, hipStream_t s);
hipError_t launch_update_bias(const int32_t* counts, float* bias, float gamma, int64_t T, int E,
                              int k, hipStream_t s);

}  // namespace moe
