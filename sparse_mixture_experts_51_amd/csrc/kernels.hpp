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
};
hipError_t launch_gemm_swiglu(const GroupedGemmArgs& a, hipStream_t s);
hipError_t launch_gemm_down(const GroupedGemmArgs& a, hipStream_t s);

hipError_t launch_combine(const uint16_t* y_perm, const uint16_t* y_shared, const float* gate,
                          const int32_t* pos, const uint16_t* residual, uint16_t* out,
                          int64_t T, int d, int k, hipStream_t s);
hipError_t launch_update_bias(const int32_t* counts, float* bias, float gamma, int64_t T, int E,
                              int k, hipStream_t s);

}  // namespace moe
