// bwd_gemm.hip -- grouped GEMMs of the layer backward on bf16 MFMA (gfx950).
//
// Training runs the layer backward ("190行JAX复刻DeepSeek V3" (openai-hub.com),
// section 如何在Mac上复现: 12000 AdamW steps).  With rows grouped by expert
// (moe_permute's order) and the upstream gradient already scaled by the gates
// (moe_combine_backward), every product of an expert's backward is a GEMM over
// contiguous rows, one per expert group:
//   dh   = dy W2                      rows x H,  K = d        (dgrad)
//   a, c = x W1^T, x W3^T  -> da, dc, h (SwiGLU derivative in the epilogue)
//   dx   = da W1 + dc W3               rows x d,  K = 2H       (dgrad)
//   dW2  = dy^T h                      d x H,     K = rows     (wgrad)
//   dW1  = da^T x,  dW3 = dc^T x       H x d,     K = rows     (wgrad)
// so the weights are read as stored (W1, W3 [H, d]; W2 [d, H]) and the
// operands come in two layouts: K contiguous (a row of K values) or K major
// (a row per index of K).  The group's rows are the ragged M of a dgrad and
// the ragged K of a wgrad; a group with no rows gets a zero weight gradient.
//
// Tile 128 x 128 x 32, four waves of 64 x 64 (2 x 2 tiles of 32x32x16 MFMAs,
// fp32 accumulators), two blocks per CU, persistent over units (group,
// n-tile, m-tile) with the XCD-aware block order of the forward.  Tiles are
// loaded to registers one K-step ahead (16-byte loads along the contiguous
// direction) and stored to LDS in two stages.  A K-contiguous tile sits as
// 64-byte rows (XOR-swizzled chunks) and gives a fragment per 16-byte read; a
// K-major tile sits row per K index (rows padded by 16 bytes) and a fragment
// is gathered from eight 2-byte reads.  The epilogue stores straight from the
// accumulators: bf16 (input gradients, dh) or fp32 (weight gradients), or for
// the recompute, h = silu(a) c, da = dh c silu'(a) and dc = dh silu(a).
#include "common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace moe {

namespace {
constexpr int kBTh = 256;                   // threads
constexpr int kBBM = 128, kBBN = 128, kBBK = 32;
constexpr int kBTM = 2, kBTN = 2;           // 32x32 tiles per wave
constexpr int kKCh = kBBK / 8;              // 16-byte chunks per K-contiguous tile row (4)
constexpr int kKMRow = kBBM + 8;            // K-major tile row in elements, padded (272 bytes)
constexpr int kKMCh = kBBM / 8;             // 16-byte chunks per K-major tile row (16)
constexpr int kBGroups = 1025;
static_assert(kBBM == kBBN, "one staging layout serves both operands");

__device__ __forceinline__ int bswz(int row, int chunk) {
  return row * kKCh + (chunk ^ ((row >> 2) & (kKCh - 1)));
}
}  // namespace

enum BwdEpi { kEpiBf16 = 0, kEpiF32 = 1, kEpiSwigluBwd = 2 };

template <bool A_KC, bool B_KC, int EPI>
__global__ __launch_bounds__(kBTh, 2) void bwd_gemm_kernel(BwdGemmArgs a) {
  // staging: K-contiguous tiles as u32x4 [128 * 4], K-major tiles as
  // uint16 [32][136]; one buffer per operand and stage, sized for the larger
  constexpr int kStageU4 = (kBBK * kKMRow * 2 + 15) / 16 > kBBM * kKCh ? (kBBK * kKMRow * 2 + 15) / 16
                                                                       : kBBM * kKCh;
  __shared__ u32x4 lds_a[2][kStageU4];
  __shared__ u32x4 lds_b[2][kStageU4];
  __shared__ int unit_start[kBGroups + 1];
  __shared__ int offs[kBGroups + 1];
  __shared__ int wsum[kBTh / 64];
  constexpr bool kPair = EPI == kEpiSwigluBwd;  // B rows [0,64) from b, [64,128) from b2
  constexpr int kCols = kPair ? kBBN / 2 : kBBN;  // output columns per unit

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int G = a.groups;
  auto group_rows = [&](int g) -> int {
    return a.offsets ? a.offsets[g + 1] - a.offsets[g] : a.rows;
  };
  // ---- unit table
  {
    constexpr int kPer = (kBGroups + kBTh - 1) / kBTh;
    const int per = (G + kBTh - 1) / kBTh;
    int local[kPer];
    int sum = 0;
    for (int i = 0; i < per; ++i) {
      const int g = tid * per + i;
      int u = 0;
      if (g < G) offs[g] = a.offsets ? a.offsets[g] : 0;
      if (g < G) {
        const int mt = a.ragged_k ? (a.M + kBBM - 1) / kBBM : (group_rows(g) + kBBM - 1) / kBBM;
        u = mt * ((a.N + kCols - 1) / kCols);
      }
      local[i] = u;
      sum += u;
    }
    int total;
    int run = block_scan<kBTh>(sum, &total, wsum);
    for (int i = 0; i < per; ++i) {
      const int g = tid * per + i;
      if (g < G) unit_start[g] = run;
      run += local[i];
    }
    if (tid == 0) {
      unit_start[G] = total;
      offs[G] = a.offsets ? a.offsets[G] : a.rows;
    }
    __syncthreads();
  }
  const int total_units = uni(unit_start[G]);
  const int NB = gridDim.x;
  const int lb = (blockIdx.x % kXcds) * (NB / kXcds) + blockIdx.x / kXcds;

  // fragments of the MFMAs: weight-side (B) first, so a lane holds output row
  // (lane & 31) and columns 8g + 4(lane >> 5) + 0..3 of each 32x32 tile
  const int fr = lane & 31, fhalf = lane >> 5;
  auto read_frag = [&](const u32x4* buf, bool kc, int row, int ks) -> bf16x8 {
    const int ch = 2 * ks + fhalf;
    if (kc) return __builtin_bit_cast(bf16x8, buf[bswz(row, ch)]);
    const uint16_t* e = reinterpret_cast<const uint16_t*>(buf) + (8 * ch) * kKMRow + row;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(e[(2 * i) * kKMRow]) | (static_cast<uint32_t>(e[(2 * i + 1) * kKMRow]) << 16);
    return __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
  };

  for (int u = lb; u < total_units; u += NB) {
    // ---- decode the unit (uniform)
    int below = 0;
    for (int base = 0; base < G; base += 64) {
      const int g = base + lane;
      below += __popcll(__ballot(g < G && unit_start[g] <= u));
    }
    const int g = uni(below - 1);
    const int R = uni(offs[g + 1] - offs[g]);
    const int off = uni(offs[g]);
    const int mrows = a.ragged_k ? a.M : R;
    const int mt = (mrows + kBBM - 1) / kBBM;
    const int local = u - uni(unit_start[g]);
    const int m0 = (local % mt) * kBBM;
    const int n0 = (local / mt) * kCols;
    const int Ktot = a.ragged_k ? R : a.K + a.K2;
    const int nk = (Ktot + kBBK - 1) / kBBK;
    const uint16_t* bg = a.b + static_cast<int64_t>(g) * a.b_gstride;
    const uint16_t* bg2 = a.b2 ? a.b2 + static_cast<int64_t>(g) * a.b_gstride : nullptr;

    // ---- loads of K-step kt into registers: two 16-byte chunks per operand
    // and thread; out-of-range elements are zero
    auto load_tile = [&](bool is_a, bool kc, int kt, u32x4 (&v)[2]) {
      const int k0 = kt * kBBK;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int q = tid + kBTh * p;
        v[p] = u32x4{0u, 0u, 0u, 0u};
        if (kc) {
          const int row = q / kKCh, ch = q % kKCh;  // row of the M (or N) tile, chunk of K
          const int kk = k0 + ch * 8;
          if (is_a) {
            // A K-contiguous: dgrad rows (ragged M) of a [rows, K] (+ a2 for K2)
            const int r = m0 + row;
            if (r < mrows && kk < Ktot) {
              const bool second = kk >= a.K;
              const uint16_t* src = second ? a.a2 : a.a;
              v[p] = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(off + r) * a.lda +
                                                       (second ? kk - a.K : kk));
            }
          } else {
            // B K-contiguous: weight rows [N, K]; the pair layout takes rows
            // [0, 64) from b and [64, 128) from b2 at the same columns
            const int nrow = kPair ? n0 + (row % kCols) : n0 + row;
            const uint16_t* src = kPair && row >= kCols ? bg2 : bg;
            if (nrow < a.N && kk < Ktot) v[p] = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(nrow) * a.ldb + kk);
          }
        } else {
          const int krow = q / kKMCh, ch = q % kKMCh;  // index of K, chunk of M (or N)
          const int kk = k0 + krow;
          const int col = (is_a ? m0 : n0) + ch * 8;
          const int ncols = is_a ? a.M : a.N;
          if (kk < Ktot && col < ncols) {
            if (a.ragged_k) {
              // wgrad: both operands are expert-grouped rows (index of K = row)
              const uint16_t* src = is_a ? a.a : a.b;
              const int64_t ld = is_a ? a.lda : a.ldb;
              v[p] = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(off + kk) * ld + col);
            } else {
              // dgrad B K-major: a weight stored [K, N] (+ b2 for K2)
              const bool second = kk >= a.K;
              const uint16_t* src = second ? bg2 : bg;
              v[p] = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(second ? kk - a.K : kk) * a.ldb + col);
            }
          }
        }
      }
    };
    auto store_tile = [&](u32x4* buf, bool kc, const u32x4 (&v)[2]) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int q = tid + kBTh * p;
        if (kc) {
          buf[bswz(q / kKCh, q % kKCh)] = v[p];
        } else {
          uint16_t* e = reinterpret_cast<uint16_t*>(buf) + (q / kKMCh) * kKMRow + (q % kKMCh) * 8;
          *reinterpret_cast<u32x4*>(e) = v[p];
        }
      }
    };

    f32x16 acc[kBTM][kBTN];
#pragma unroll
    for (int i = 0; i < kBTM; ++i)
#pragma unroll
      for (int j = 0; j < kBTN; ++j) acc[i][j] = f32x16{};
    // this wave's 32-row tiles (rows 32 (wm + 2 i)) and weight rows
    auto tile_row = [&](int i) { return 32 * (wm + 2 * i); };
    auto brow = [&](int j) { return kPair ? (j == 0 ? wn * 32 : kCols + wn * 32) : wn * 64 + 32 * j; };

    u32x4 va[2], vb[2];
    if (nk > 0) {
      load_tile(true, A_KC, 0, va);
      load_tile(false, B_KC, 0, vb);
      store_tile(lds_a[0], A_KC, va);
      store_tile(lds_b[0], B_KC, vb);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int st = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        load_tile(true, A_KC, kt + 1, va);
        load_tile(false, B_KC, kt + 1, vb);
      }
#pragma unroll
      for (int ks = 0; ks < kBBK / 16; ++ks) {
        bf16x8 af[kBTM], bfr[kBTN];
#pragma unroll
        for (int i = 0; i < kBTM; ++i) af[i] = read_frag(lds_a[st], A_KC, tile_row(i) + fr, ks);
#pragma unroll
        for (int j = 0; j < kBTN; ++j) bfr[j] = read_frag(lds_b[st], B_KC, brow(j) + fr, ks);
#pragma unroll
        for (int i = 0; i < kBTM; ++i)
#pragma unroll
          for (int j = 0; j < kBTN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
      }
      if (more) {
        store_tile(lds_a[st ^ 1], A_KC, va);
        store_tile(lds_b[st ^ 1], B_KC, vb);
      }
      __syncthreads();
    }

    // ---- epilogue
    const int lcol = fhalf * 4;
#pragma unroll
    for (int i = 0; i < kBTM; ++i) {
      const int r = m0 + tile_row(i) + fr;  // row of the output (within the group for dgrad)
      if (r >= mrows) continue;
      if constexpr (EPI == kEpiSwigluBwd) {
        const int64_t row = static_cast<int64_t>(off + r);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn * 32 + 8 * q + lcol;
          if (col >= a.N) continue;
          const uint2 dhv = *reinterpret_cast<const uint2*>(a.dh + row * a.ld_h + col);
          const float dhf[4] = {bf16_to_f32(static_cast<uint16_t>(dhv.x)), bf16_to_f32(static_cast<uint16_t>(dhv.x >> 16)),
                                bf16_to_f32(static_cast<uint16_t>(dhv.y)), bf16_to_f32(static_cast<uint16_t>(dhv.y >> 16))};
          float hv[4], dav[4], dcv[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float ga = acc[i][0][4 * q + t], up = acc[i][1][4 * q + t];
            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-ga));
            hv[t] = ga * sg * up;  // the forward's h, bit for bit
            dav[t] = dhf[t] * up * sg * (1.0f + ga * (1.0f - sg));
            dcv[t] = dhf[t] * ga * sg;
          }
          auto pack4 = [](const float (&f)[4]) {
            return make_uint2(bf16x2_bits(f[0], f[1]), bf16x2_bits(f[2], f[3]));
          };
          *reinterpret_cast<uint2*>(a.h + row * a.ld_h + col) = pack4(hv);
          *reinterpret_cast<uint2*>(a.da + row * a.ld_h + col) = pack4(dav);
          *reinterpret_cast<uint2*>(a.dc + row * a.ld_h + col) = pack4(dcv);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kBTN; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = n0 + wn * 64 + 32 * j + 8 * q + lcol;
            if (col >= a.N) continue;
            const float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                acc[i][j][4 * q + 3]};
            if constexpr (EPI == kEpiF32) {
              float* c = static_cast<float*>(a.c) + static_cast<int64_t>(g) * a.c_gstride +
                         static_cast<int64_t>(r) * a.ldc + col;
              *reinterpret_cast<float4*>(c) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
              uint16_t* c = static_cast<uint16_t*>(a.c) + static_cast<int64_t>(off + r) * a.ldc + col;
              *reinterpret_cast<uint2*>(c) = make_uint2(bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3]));
            }
          }
        }
      }
    }
  }
}

hipError_t launch_bwd_gemm(const BwdGemmArgs& a, int kind, hipStream_t s) {
  int grid = 2 * device_cus();
  grid = (grid / kXcds) * kXcds;
  if (grid <= 0) grid = kXcds;
  const dim3 gd(grid), bd(kBTh);
  switch (kind) {
    case kBwdDgradKM:  // A rows x K, B stored [K, N]
      hipLaunchKernelGGL((bwd_gemm_kernel<true, false, kEpiBf16>), gd, bd, 0, s, a);
      break;
    case kBwdRecompute:  // A rows x K, B = [W1; W3] rows x K
      hipLaunchKernelGGL((bwd_gemm_kernel<true, true, kEpiSwigluBwd>), gd, bd, 0, s, a);
      break;
    case kBwdWgrad:  // both operands expert-grouped rows, K = rows
      hipLaunchKernelGGL((bwd_gemm_kernel<false, false, kEpiF32>), gd, bd, 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
