// bwd.hip -- the layer backward outside the expert GEMMs: the combine and the
// routing (gates, sequence balance statistic, sigmoid, router GEMM).
//
// Training adds the small sequence-wise balance loss to the language-model
// loss ("190行JAX复刻DeepSeek V3" (openai-hub.com), section 多Token预测也被保留了)
// and keeps the per-expert bias out of it (section 最有价值的实验: the bias only
// moves the choice of experts).  With the choice held fixed:
//   out = r + ys + sum_j g_j y_j                (combine)
//     dy_j = g_j dout,  dg_j = <dout, y_j>,  dys = dout,  dr = dout
//   g_j = s_j / sum_j' s_j'                     (gates over the chosen experts)
//     ds_j = (dg_j - sum_j' dg_j' g_j') / sum
//   L_b = alpha sum_i f_i P_i, P_i = mean_t s_i / Z_t   (balance statistic)
//     ds_m += alpha / S (f_m - sum_i f_i s_i / Z_t) / Z_t
//   s = sigmoid(logit):  dlogit = ds s (1 - s)
//   logit = x W_r:  dx += dlogit W_r^T,  dW_r = x^T dlogit
// The bias gets no gradient.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr int kBwdThreads = 256;
constexpr int kBwdRows = kBwdThreads / kWave;  // one wave per token

__device__ __forceinline__ float wsum64(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
}  // namespace

// ---- combine backward: one wave per token, lanes over 16-byte chunks of d.
// dy_perm[pos[t,j]] = bf16(g[t,j] dout[t]),  dgate[t,j] = <dout[t], y_perm[pos[t,j]]>
__global__ __launch_bounds__(kBwdThreads) void combine_bwd_kernel(
    const uint16_t* __restrict__ dout, const uint16_t* __restrict__ y_perm,
    const float* __restrict__ gate, const int32_t* __restrict__ pos, uint16_t* __restrict__ dy_perm,
    float* __restrict__ dgate, int64_t T, int d, int k) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kBwdRows + (threadIdx.x >> 6);
  if (t >= T) return;  // whole waves
  const int chunks = d / 8;
  const int64_t nrows = T * k;
  const uint4* dr = reinterpret_cast<const uint4*>(dout + t * d);
  for (int j = 0; j < k; ++j) {
    const int32_t r = pos[t * k + j];
    const float g = gate[t * k + j];
    float part = 0.0f;
    if (r >= 0 && r < nrows) {
      const uint4* yr = reinterpret_cast<const uint4*>(y_perm + static_cast<int64_t>(r) * d);
      uint4* dyr = reinterpret_cast<uint4*>(dy_perm + static_cast<int64_t>(r) * d);
      for (int c = lane; c < chunks; c += kWave) {
        float dv[8], yv[8];
        bf16x8_to_f32(dr[c], dv);
        bf16x8_to_f32(yr[c], yv);
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf(dv[e], yv[e], part);
        uint4 o;
        o.x = pack_bf16x2(g * dv[0], g * dv[1]);
        o.y = pack_bf16x2(g * dv[2], g * dv[3]);
        o.z = pack_bf16x2(g * dv[4], g * dv[5]);
        o.w = pack_bf16x2(g * dv[6], g * dv[7]);
        dyr[c] = o;
      }
    }
    part = wsum64(part);
    if (lane == 0) dgate[t * k + j] = part;
  }
}

hipError_t launch_combine_bwd(const uint16_t* dout, const uint16_t* y_perm, const float* gate,
                              const int32_t* pos, uint16_t* dy_perm, float* dgate, int64_t T,
                              int d, int k, hipStream_t s) {
  const int64_t blocks = (T + kBwdRows - 1) / kBwdRows;
  hipLaunchKernelGGL(combine_bwd_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBwdThreads), 0,
                     s, dout, y_perm, gate, pos, dy_perm, dgate, T, d, k);
  return hipGetLastError();
}

// ---- per-sequence choice frequencies f[b, e] = E/(kS) #{t in b : e chosen}
__global__ __launch_bounds__(kBwdThreads) void seq_freq_kernel(const int32_t* __restrict__ idx,
                                                               float* __restrict__ freq, int S,
                                                               int E, int k) {
  extern __shared__ int cnt[];
  const int64_t b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kBwdThreads) cnt[e] = 0;
  __syncthreads();
  for (int64_t i = threadIdx.x; i < static_cast<int64_t>(S) * k; i += kBwdThreads) {
    const int e = idx[b * S * k + i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  const float scale = static_cast<float>(E) / (static_cast<float>(k) * static_cast<float>(S));
  for (int e = threadIdx.x; e < E; e += kBwdThreads) freq[b * E + e] = scale * static_cast<float>(cnt[e]);
}

// ---- dlogit: one wave per token, lanes over experts (e = lane + 64 q)
template <int EPL>  // experts per lane held in registers
__global__ __launch_bounds__(kBwdThreads) void dlogit_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ idx, const float* __restrict__ gate,
    const float* __restrict__ dgate, const float* __restrict__ freq, float alpha,
    float* __restrict__ dlogit, int64_t T, int E, int k, int S) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kBwdRows + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* st = scores + t * E;
  float s[EPL], ds[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    const int e = lane + kWave * q;
    s[q] = e < E ? st[e] : 0.0f;
    ds[q] = 0.0f;
  }
  // gates: the fp32 sum of the chosen scores in slot order (as the forward)
  float sum = 0.0f, gs = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int e = idx[t * k + j];
    sum += (e >= 0 && e < E) ? st[e] : 0.0f;
    gs = fmaf(dgate[t * k + j], gate[t * k + j], gs);
  }
  if (sum != 0.0f) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e < 0 || e >= E) continue;
      const float v = (dgate[t * k + j] - gs) / sum;
#pragma unroll
      for (int q = 0; q < EPL; ++q)
        if (lane + kWave * q == e) ds[q] += v;
    }
  }
  if (freq != nullptr && S > 0) {
    const float* f = freq + (t / S) * E;
    float z = 0.0f, fz = 0.0f;
    float fl[EPL];
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      const int e = lane + kWave * q;
      fl[q] = e < E ? f[e] : 0.0f;
      z += s[q];
      fz = fmaf(fl[q], s[q], fz);
    }
    z = wsum64(z);
    fz = wsum64(fz);
    if (z != 0.0f) {
      const float qv = fz / z;
      const float c = alpha / static_cast<float>(S) / z;
#pragma unroll
      for (int q = 0; q < EPL; ++q) ds[q] = fmaf(c, fl[q] - qv, ds[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    const int e = lane + kWave * q;
    if (e < E) dlogit[t * E + e] = ds[q] * s[q] * (1.0f - s[q]);
  }
}

// ---- dx = bf16( d_residual + dx_shared + sum_j dx_perm[pos] + dlogit W_r^T ).
// A block computes a 64-token x 64-column tile.  The router term is an fp32
// GEMM over the experts on the matrix cores (v_mfma_f32_32x32x2_f32, each wave
// a 32 x 32 quarter): tiles of 32 experts of dlogit and of W_r are staged in
// LDS (a row per token or column, padded to 33 floats, so the 32 rows that a
// fragment read touches fall on distinct banks); the next tile's loads are in
// flight while the current one is multiplied.  The accumulators go through
// LDS once more (over the staging space), and each thread then adds 4 tokens
// x 4 columns of the expert rows to its sums.
constexpr int kDxT = 64, kDxC = 64, kDxE = 32, kDxPad = kDxE + 1, kDxOut = kDxC + 4;
constexpr int kDxLoads = kDxE * kDxT / kBwdThreads;  // per thread and operand
static_assert(kDxT == kDxC && kDxLoads * kBwdThreads == kDxE * kDxT, "staging map");
__global__ __launch_bounds__(kBwdThreads) void dx_assemble_kernel(
    const float* __restrict__ dlogit, const float* __restrict__ w_router,
    const uint16_t* __restrict__ dx_perm, const uint16_t* __restrict__ dx_shared,
    const int32_t* __restrict__ pos, const uint16_t* __restrict__ d_residual,
    uint16_t* __restrict__ dx, int64_t T, int d, int E, int k) {
  // staging: dlogit [token][expert], then W_r [column][expert]; afterwards the
  // router term [token][column]
  __shared__ __attribute__((aligned(16))) float smem[kDxT * kDxOut];
  static_assert(2 * kDxT * kDxPad <= kDxT * kDxOut, "staging fits the output tile");
  float (*const sl)[kDxPad] = reinterpret_cast<float (*)[kDxPad]>(smem);
  float (*const sw)[kDxPad] = reinterpret_cast<float (*)[kDxPad]>(smem + kDxT * kDxPad);
  float (*const so)[kDxOut] = reinterpret_cast<float (*)[kDxOut]>(smem);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wt = 32 * (wave >> 1), wc = 32 * (wave & 1);  // the wave's quarter
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kDxT;
  const int c0 = blockIdx.x * kDxC;
  // thread i stages expert i % 32 of rows i / 32 + 8 q
  const int se = threadIdx.x % kDxE, sr = threadIdx.x / kDxE;
  float rl[kDxLoads], rw[kDxLoads];
  auto load = [&](int e0) {
    const bool ein = e0 + se < E;
#pragma unroll
    for (int q = 0; q < kDxLoads; ++q) {
      const int r = sr + (kBwdThreads / kDxE) * q;
      const int64_t t = t0 + r;
      rl[q] = (ein && t < T) ? dlogit[t * E + e0 + se] : 0.0f;
      rw[q] = (ein && c0 + r < d) ? w_router[static_cast<int64_t>(c0 + r) * E + e0 + se] : 0.0f;
    }
  };
  f32x16 acc = {};
  load(0);
  for (int e0 = 0; e0 < E; e0 += kDxE) {
#pragma unroll
    for (int q = 0; q < kDxLoads; ++q) {
      const int r = sr + (kBwdThreads / kDxE) * q;
      sl[r][se] = rl[q];
      sw[r][se] = rw[q];
    }
    __syncthreads();
    if (e0 + kDxE < E) load(e0 + kDxE);
    // lane: row (token / column) lane % 32, expert 2 s + lane / 32
#pragma unroll
    for (int s = 0; s < kDxE / 2; ++s) {
      const int ee = 2 * s + lane / 32;
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sl[wt + lane % 32][ee], sw[wc + lane % 32][ee], acc, 0, 0, 0);
    }
    __syncthreads();
  }
  // lane holds tokens 8 (v / 4) + 4 (lane / 32) + v % 4 of column lane % 32
#pragma unroll
  for (int v = 0; v < 16; ++v) so[wt + 8 * (v / 4) + 4 * (lane / 32) + v % 4][wc + lane % 32] = acc[v];
  __syncthreads();
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;  // 16 x 16 threads
  const int64_t nrows = T * k;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int tt = ty + 16 * a;
    const int64_t t = t0 + tt;
    const int c = c0 + tx * 4;
    if (t >= T || c >= d) continue;
    const f32x4 r = *reinterpret_cast<const f32x4*>(&so[tt][tx * 4]);
    float v[4] = {r[0], r[1], r[2], r[3]};
    auto add4 = [&](const uint16_t* src) {
      const uint2 w = *reinterpret_cast<const uint2*>(src);
      v[0] += bf16_to_f32(static_cast<uint16_t>(w.x));
      v[1] += bf16_to_f32(static_cast<uint16_t>(w.x >> 16));
      v[2] += bf16_to_f32(static_cast<uint16_t>(w.y));
      v[3] += bf16_to_f32(static_cast<uint16_t>(w.y >> 16));
    };
    if (dx_shared) add4(dx_shared + t * d + c);
    for (int j = 0; j < k; ++j) {
      const int32_t r = pos[t * k + j];
      if (r >= 0 && r < nrows) add4(dx_perm + static_cast<int64_t>(r) * d + c);
    }
    if (d_residual) add4(d_residual + t * d + c);
    *reinterpret_cast<uint2*>(dx + t * d + c) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
}

// ---- dW_r = x^T dlogit: partial sums over token splits, then a reduction of
// the splits in order (deterministic).  A block: 64 columns of x x 64 experts
// over one split of the tokens, on the matrix cores (v_mfma_f32_32x32x2_f32,
// each wave a 32 x 32 quarter; x is bf16, exact in fp32).  Tokens are staged
// 32 at a time in LDS as fp32, a row per token, the next 32 tokens' loads in
// flight while the current ones are multiplied; a fragment read takes 32
// consecutive entries of one row (lanes 0-31) and of the next (lanes 32-63),
// and rows of 96 floats put the two halves on different banks.
constexpr int kWrC = 64, kWrE = 64, kWrT = 32, kWrRow = 96, kWrSplitTokens = 512;
constexpr int kWrX = kWrT * kWrC / (8 * kBwdThreads);   // 8-column pieces of x per thread
constexpr int kWrL = kWrT * kWrE / kBwdThreads;         // dlogit values per thread
static_assert(kWrX == 1 && kWrL * kBwdThreads == kWrT * kWrE, "staging map");
__global__ __launch_bounds__(kBwdThreads) void dwr_partial_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ dlogit, float* __restrict__ part,
    int64_t T, int d, int E) {
  __shared__ float sx[kWrT][kWrRow];  // x tile [token][column]
  __shared__ float sl[kWrT][kWrRow];  // dlogit tile [token][expert]
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wcol = 32 * (wave >> 1), wexp = 32 * (wave & 1);  // the wave's quarter
  const int c0 = blockIdx.x * kWrC, e0 = blockIdx.y * kWrE;
  const int64_t tb = static_cast<int64_t>(blockIdx.z) * kWrSplitTokens;
  const int64_t te = tb + kWrSplitTokens < T ? tb + kWrSplitTokens : T;
  // thread i stages columns 8 (i % 8) .. + 7 of token i / 8, and expert i % 64
  // of tokens i / 64 + 4 q
  const int xt = threadIdx.x / 8, xc = 8 * (threadIdx.x % 8);
  const int le = threadIdx.x % kWrE, lt = threadIdx.x / kWrE;
  const bool xvec = d % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  uint16_t rx[8];
  float rl[kWrL];
  auto load = [&](int64_t t0) {
    const int64_t t = t0 + xt;
    const int c = c0 + xc;
    if (xvec && t < te && c + 8 <= d) {
      const uint4 w = *reinterpret_cast<const uint4*>(x + t * d + c);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        rx[2 * j] = static_cast<uint16_t>(ww[j]);
        rx[2 * j + 1] = static_cast<uint16_t>(ww[j] >> 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) rx[j] = (t < te && c + j < d) ? x[t * d + c + j] : uint16_t{0};
    }
#pragma unroll
    for (int q = 0; q < kWrL; ++q) {
      const int64_t tq = t0 + lt + (kBwdThreads / kWrE) * q;
      rl[q] = (tq < te && e0 + le < E) ? dlogit[tq * E + e0 + le] : 0.0f;
    }
  };
  f32x16 acc = {};
  if (tb < te) load(tb);
  for (int64_t t0 = tb; t0 < te; t0 += kWrT) {
#pragma unroll
    for (int j = 0; j < 8; ++j) sx[xt][xc + j] = bf16_to_f32(rx[j]);
#pragma unroll
    for (int q = 0; q < kWrL; ++q) sl[lt + (kBwdThreads / kWrE) * q][le] = rl[q];
    __syncthreads();
    if (t0 + kWrT < te) load(t0 + kWrT);
    // lane: column / expert lane % 32 of token 2 s + lane / 32
#pragma unroll
    for (int s = 0; s < kWrT / 2; ++s) {
      const int tt = 2 * s + lane / 32;
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sx[tt][wcol + lane % 32], sl[tt][wexp + lane % 32], acc, 0, 0, 0);
    }
    __syncthreads();
  }
  // lane holds columns 8 (v / 4) + 4 (lane / 32) + v % 4 of expert lane % 32
  const int e = e0 + wexp + lane % 32;
  if (e >= E) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int c = c0 + wcol + 8 * (v / 4) + 4 * (lane / 32) + v % 4;
    if (c < d) part[(static_cast<int64_t>(blockIdx.z) * d + c) * E + e] = acc[v];
  }
}

__global__ __launch_bounds__(kBwdThreads) void dwr_reduce_kernel(const float* __restrict__ part,
                                                                 float* __restrict__ dwr,
                                                                 int64_t n, int splits) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (i >= n) return;
  float acc = 0.0f;
  for (int sp = 0; sp < splits; ++sp) acc += part[static_cast<int64_t>(sp) * n + i];
  dwr[i] = acc;
}

int route_bwd_splits(int64_t T) {
  return static_cast<int>((T + kWrSplitTokens - 1) / kWrSplitTokens);
}

hipError_t launch_route_bwd(const uint16_t* x, const float* w_router, const int32_t* idx,
                            const float* gate, const float* dgate, float alpha,
                            const uint16_t* dx_perm, const uint16_t* dx_shared,
                            const int32_t* pos, const uint16_t* d_residual, uint16_t* dx,
                            float* dw_router, float* scores, float* freq, float* dlogit,
                            float* dwr_part, int dwr_splits, int64_t T, int d, int E, int k,
                            int S, hipStream_t s) {
  // scores again, with the forward's own router kernel (the same fp32 chain)
  hipError_t e = launch_router_scores(x, w_router, scores, T, d, E, s);
  if (e != hipSuccess) return e;
  const bool balance = S > 0 && alpha != 0.0f;
  if (balance) {
    hipLaunchKernelGGL(seq_freq_kernel, dim3(static_cast<unsigned>(T / S)), dim3(kBwdThreads),
                       sizeof(int) * E, s, idx, freq, S, E, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const dim3 rows_grid(static_cast<unsigned>((T + kBwdRows - 1) / kBwdRows));
  const float* fr = balance ? freq : nullptr;
  const int epl = (E + kWave - 1) / kWave;
  if (epl <= 1) hipLaunchKernelGGL(dlogit_kernel<1>, rows_grid, dim3(kBwdThreads), 0, s, scores, idx, gate, dgate, fr, alpha, dlogit, T, E, k, S);
  else if (epl <= 4) hipLaunchKernelGGL(dlogit_kernel<4>, rows_grid, dim3(kBwdThreads), 0, s, scores, idx, gate, dgate, fr, alpha, dlogit, T, E, k, S);
  else hipLaunchKernelGGL(dlogit_kernel<16>, rows_grid, dim3(kBwdThreads), 0, s, scores, idx, gate, dgate, fr, alpha, dlogit, T, E, k, S);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(dx_assemble_kernel, dim3((d + kDxC - 1) / kDxC, static_cast<unsigned>((T + kDxT - 1) / kDxT)),
                     dim3(kBwdThreads), 0, s, dlogit, w_router, dx_perm, dx_shared, pos, d_residual,
                     dx, T, d, E, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(dwr_partial_kernel, dim3((d + kWrC - 1) / kWrC, (E + kWrE - 1) / kWrE, dwr_splits),
                     dim3(kBwdThreads), 0, s, x, dlogit, dwr_part, T, d, E);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t n = static_cast<int64_t>(d) * E;
  hipLaunchKernelGGL(dwr_reduce_kernel, dim3(static_cast<unsigned>((n + kBwdThreads - 1) / kBwdThreads)),
                     dim3(kBwdThreads), 0, s, dwr_part, dw_router, n, dwr_splits);
  return hipGetLastError();
}

}  // namespace moe
