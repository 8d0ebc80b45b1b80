// combine.hip -- gate-weighted combine with the shared expert, and the bias update.
//
// "190行JAX复刻DeepSeek V3" (openai-hub.com): section 190行代码到底装进了什么
// (the always-on shared expert is added to the routed experts' mixture) and
// section 最有价值的实验:无辅助损失均衡真的有效 (after every step the bias of an
// overloaded expert is lowered and that of an idle expert raised, speed 1e-3).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// One thread per (token, 16-byte column chunk), flattened so that a wave
// reads 1 KB runs of each row whatever d is, and tokens x chunks threads keep
// the chip busy even for a handful of tokens.
// out[t] = bf16(residual[t] + y_shared[t] + sum_j g[t,j] * y_perm[pos[t,j]]),
// fp32 accumulation, slots in order.  Rows outside [0, T*k) are skipped.
template <typename Index>
__global__ __launch_bounds__(256) void combine_kernel(
    const uint16_t* __restrict__ y_perm, const uint16_t* __restrict__ y_shared,
    const float* __restrict__ gate, const int32_t* __restrict__ pos,
    const uint16_t* __restrict__ residual, uint16_t* __restrict__ out, Index T, int d, int k) {
  const Index chunks = static_cast<Index>(d / 8);
  const Index i = static_cast<Index>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= T * chunks) return;
  const Index t = i / chunks;
  const Index c = i - t * chunks;
  const int64_t nrows = static_cast<int64_t>(T) * k;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  float v[8];
  const int64_t row_t = static_cast<int64_t>(t) * d + static_cast<int64_t>(c) * 8;
  if (residual) {
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(residual + row_t), v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += v[e];
  }
  if (y_shared) {
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(y_shared + row_t), v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += v[e];
  }
  // Slots in groups of 8: all positions and gates of a group, then all its
  // rows, are loaded before the first FMA, so the loads overlap instead of
  // each row waiting for its position; the FMAs still run in slot order.
  const int64_t slot0 = static_cast<int64_t>(t) * k;
  for (int j0 = 0; j0 < k; j0 += 8) {
    int row[8];
    float g[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const bool in = j0 + jj < k;
      row[jj] = in ? pos[slot0 + j0 + jj] : -1;
      g[jj] = in ? gate[slot0 + j0 + jj] : 0.0f;
    }
    u32x4 y[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const bool ok = row[jj] >= 0 && row[jj] < nrows;
      // y_perm rows are read once: the streaming hint keeps them out of the way
      y[jj] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                       y_perm + static_cast<int64_t>(row[jj]) * d + static_cast<int64_t>(c) * 8))
                 : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (row[jj] < 0 || row[jj] >= nrows) continue;
      bf16x8_to_f32(make_uint4(y[jj][0], y[jj][1], y[jj][2], y[jj][3]), v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(g[jj], v[e], acc[e]);
    }
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(out + row_t) = o;
}

hipError_t launch_combine(const uint16_t* y_perm, const uint16_t* y_shared, const float* gate,
                          const int32_t* pos, const uint16_t* residual, uint16_t* out,
                          int64_t T, int d, int k, hipStream_t s) {
  const int64_t n = T * (d / 8);
  const int64_t nblk = (n + 255) / 256;
  if (n + 256 < (int64_t{1} << 31)) {
    hipLaunchKernelGGL(combine_kernel<int32_t>, dim3(static_cast<unsigned>(nblk)), dim3(256), 0,
                       s, y_perm, y_shared, gate, pos, residual, out, static_cast<int32_t>(T), d, k);
  } else {
    hipLaunchKernelGGL(combine_kernel<int64_t>, dim3(static_cast<unsigned>(nblk)), dim3(256), 0,
                       s, y_perm, y_shared, gate, pos, residual, out, T, d, k);
  }
  return hipGetLastError();
}

// b_i <- b_i + gamma * sgn(T*k - E*counts_i), the sign taken on integers.
__global__ __launch_bounds__(256) void update_bias_kernel(const int32_t* __restrict__ counts,
                                                          float* __restrict__ bias, float gamma,
                                                          int64_t T, int E, int k) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= E) return;
  const long long diff = static_cast<long long>(T) * k - static_cast<long long>(E) * counts[i];
  const float sg = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);
  bias[i] = bias[i] + gamma * sg;
}

hipError_t launch_update_bias(const int32_t* counts, float* bias, float gamma, int64_t T, int E,
                              int k, hipStream_t s) {
  hipLaunchKernelGGL(update_bias_kernel, dim3((E + 255) / 256), dim3(256), 0, s, counts, bias,
                     gamma, T, E, k);
  return hipGetLastError();
}

}  // namespace moe
