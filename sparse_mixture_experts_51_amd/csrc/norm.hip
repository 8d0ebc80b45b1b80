// norm.hip -- RMSNorm of the token rows before the MoE of a pre-norm block.
//
// The model's layers are plain functions over arrays, RMSNorm among them
// ("190行JAX复刻DeepSeek V3" (openai-hub.com), section "纯JAX"也需要打一个小星号),
// and the MoE sits in a residual Transformer block (same page, section 先说结论):
// x_next = x + MoE(RMSNorm(x)), with
//   out[t,i] = bf16( x[t,i] * rsqrt(mean_j x[t,j]^2 + eps) * g[i] ).
//
// One wave per row, four rows per block.  The kernel moves 2d bytes in and 2d
// out per row and does 3d FLOPs: HBM-bound.  A lane holds chunks c = lane +
// 64 j (16 bytes, 8 values each) of its row in registers, so the row is read
// once; the sum of squares is fp32, combined across the wave with butterfly
// shuffles.  Rows wider than 64 * 8 * kMaxChunks values take a second read of
// the row (from L2) for the scaling pass.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {
constexpr int kNormThreads = 256;
constexpr int kNormRows = kNormThreads / kWave;  // rows per block
constexpr int kMaxChunks = 16;                   // 16-byte chunks per lane held in registers

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ uint4 scale_chunk(const uint4& xv, const float* g, float r) {
  float f[8];
  bf16x8_to_f32(xv, f);
  const float4 g0 = *reinterpret_cast<const float4*>(g);
  const float4 g1 = *reinterpret_cast<const float4*>(g + 4);
  const float gs[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  uint4 o;
  o.x = pack_bf16x2(f[0] * r * gs[0], f[1] * r * gs[1]);
  o.y = pack_bf16x2(f[2] * r * gs[2], f[3] * r * gs[3]);
  o.z = pack_bf16x2(f[4] * r * gs[4], f[5] * r * gs[5]);
  o.w = pack_bf16x2(f[6] * r * gs[6], f[7] * r * gs[7]);
  return o;
}
}  // namespace

// CPL: 16-byte chunks per lane held in registers (0: re-read the row).
template <int CPL>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                               const float* __restrict__ g,
                                                               float eps,
                                                               uint16_t* __restrict__ out,
                                                               int64_t T, int d) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kNormRows + (threadIdx.x >> 6);
  if (t >= T) return;  // whole waves leave together: the shuffles below see full waves
  const int chunks = d / 8;
  const uint4* xr = reinterpret_cast<const uint4*>(x + t * d);
  uint4* orow = reinterpret_cast<uint4*>(out + t * d);
  float ss = 0.0f;
  float f[8];
  if constexpr (CPL > 0) {
    uint4 v[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + kWave * j;
      v[j] = make_uint4(0, 0, 0, 0);
      if (c < chunks) {
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + c));
        v[j] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      bf16x8_to_f32(v[j], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
    }
    const float r = 1.0f / sqrtf(wave_sum(ss) / static_cast<float>(d) + eps);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + kWave * j;
      if (c < chunks) orow[c] = scale_chunk(v[j], g + 8 * c, r);
    }
  } else {
    for (int c = lane; c < chunks; c += kWave) {
      bf16x8_to_f32(xr[c], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
    }
    const float r = 1.0f / sqrtf(wave_sum(ss) / static_cast<float>(d) + eps);
    for (int c = lane; c < chunks; c += kWave) orow[c] = scale_chunk(xr[c], g + 8 * c, r);
  }
}

hipError_t launch_rmsnorm(const uint16_t* x, const float* gain, float eps, uint16_t* out,
                          int64_t T, int d, hipStream_t s) {
  const int64_t blocks = (T + kNormRows - 1) / kNormRows;
  const int per_lane = (d / 8 + kWave - 1) / kWave;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kNormThreads);
  if (per_lane <= 1) hipLaunchKernelGGL(rmsnorm_kernel<1>, grid, block, 0, s, x, gain, eps, out, T, d);
  else if (per_lane <= 2) hipLaunchKernelGGL(rmsnorm_kernel<2>, grid, block, 0, s, x, gain, eps, out, T, d);
  else if (per_lane <= 4) hipLaunchKernelGGL(rmsnorm_kernel<4>, grid, block, 0, s, x, gain, eps, out, T, d);
  else if (per_lane <= 8) hipLaunchKernelGGL(rmsnorm_kernel<8>, grid, block, 0, s, x, gain, eps, out, T, d);
  else if (per_lane <= kMaxChunks)
    hipLaunchKernelGGL(rmsnorm_kernel<kMaxChunks>, grid, block, 0, s, x, gain, eps, out, T, d);
  else hipLaunchKernelGGL(rmsnorm_kernel<0>, grid, block, 0, s, x, gain, eps, out, T, d);
  return hipGetLastError();
}

}  // namespace moe
