// grouped_gemm.hip -- grouped expert GEMMs on bf16 MFMA (gfx950).
//
// The experts are feed-forward networks and only the chosen ones run; one
// shared expert runs on every token ("190行JAX复刻DeepSeek V3" (openai-hub.com),
// section 190行代码到底装进了什么; the pages' reference instead runs every
// expert on every token, same section and "DeepSeek V3 viết lại bằng 190 dòng
// JAX thuần" (lehuy.net), section Những gì đã được đơn giản hóa).
//
// Stage 1 (SwiGLU): h = bf16(silu(A W1^T) * (A W3^T)) per expert group, with A
// rows gathered from x through perm_src.  Stage 2 (down): y = bf16(h W2^T).
//
// Work decomposition.  A unit is (group, n-tile, m-tile) with a 128-row
// m-tile and a 128-row weight tile (stage 1: 64 rows of W1 and the same 64
// rows of W3, interleaved in 32-row groups so that a wave holds the gate and
// up accumulators of the same h columns; stage 2: 128 rows of W2).  Units of
// one group are ordered n-tile major, m-tile minor, so the m-tiles that share
// a weight tile run back to back.  The grid is persistent (2 blocks per CU);
// block b is remapped so that each XCD (blocks b = x mod 8) walks a contiguous
// range of units: the A rows and weight tiles of one expert stay in that
// XCD's L2.  The unit table is rebuilt by every block from offsets[] (no host
// round trip).
//
// Tile pipeline: 4 waves as 2 x 2, each wave 64 rows x 64 weight rows = 2 x 2
// MFMA 32x32x16 tiles (64 fp32 accumulators).  K advances 64 at a time
// through a double-buffered LDS tile (XOR-swizzled 16-byte chunks), with the
// next K-slice prefetched into registers while the MFMAs run.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kBM = 128;       // rows per m-tile
constexpr int kBW = 128;       // weight rows per tile
constexpr int kBK = 64;        // K per LDS stage
constexpr int kThreads = 256;
constexpr int kChunksPerRow = kBK / 8;  // 16-byte chunks per tile row (8)
constexpr int kMaxGroups = 1025;

__device__ __forceinline__ int swz(int row, int chunk) { return row * kChunksPerRow + (chunk ^ (row & 7)); }

// Exclusive scan of one value per thread over 256 threads.
__device__ __forceinline__ int block_scan_256(int v, int* total, int* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  const int base = (w > 0 ? wsum[0] : 0) + (w > 1 ? wsum[1] : 0) + (w > 2 ? wsum[2] : 0);
  *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return base + inc - v;
}

template <bool kSwiGLU>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_kernel(GroupedGemmArgs a) {
  __shared__ uint4 lds_a[2][kBM * kChunksPerRow];
  __shared__ uint4 lds_b[2][kBW * kChunksPerRow];
  __shared__ int unit_start[kMaxGroups + 1];
  __shared__ int wsum[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int E = a.E;
  const bool has_shared = a.w_shared != nullptr;
  const int ngroups = E + (has_shared ? 1 : 0);
  const int cols_per_tile = kSwiGLU ? kBW / 2 : kBW;  // output columns per unit

  // ---- unit table: units of group g start at unit_start[g]
  {
    const int per = (ngroups + kThreads - 1) / kThreads;  // <= 5
    int local[5];
    int sum = 0;
    for (int i = 0; i < per; ++i) {
      const int g = tid * per + i;
      int u = 0;
      if (g < ngroups) {
        const int64_t rows = g < E ? static_cast<int64_t>(a.offsets[g + 1] - a.offsets[g]) : a.T;
        const int n = g < E ? a.N_r : a.N_s;
        const int nt = (n + cols_per_tile - 1) / cols_per_tile;
        u = static_cast<int>((rows + kBM - 1) / kBM) * nt;
      }
      local[i] = u;
      sum += u;
    }
    int total;
    int run = block_scan_256(sum, &total, wsum);
    for (int i = 0; i < per; ++i) {
      const int g = tid * per + i;
      if (g < ngroups) unit_start[g] = run;
      run += local[i];
    }
    if (tid == 0) unit_start[ngroups] = total;
    __syncthreads();
  }
  const int total_units = unit_start[ngroups];

  const int G = gridDim.x;
  const int lb = (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds;

  const int ld_row = tid / kChunksPerRow;  // 0..31
  const int ld_chunk = tid % kChunksPerRow;

  for (int u = lb; u < total_units; u += G) {
    // ---- decode unit -> (group, n-tile, m-tile)
    int lo = 0, hi = ngroups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (unit_start[mid] <= u) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const bool routed = g < E;
    const int64_t grow0 = routed ? a.offsets[g] : 0;
    const int64_t rows = routed ? static_cast<int64_t>(a.offsets[g + 1] - a.offsets[g]) : a.T;
    const int mt = static_cast<int>((rows + kBM - 1) / kBM);
    const int local = u - unit_start[g];
    const int n_tile = local / mt, m_tile = local % mt;
    const int64_t m0 = static_cast<int64_t>(m_tile) * kBM;
    const int valid_rows = static_cast<int>((rows - m0) < kBM ? (rows - m0) : kBM);
    const int K = routed ? a.K_r : a.K_s;
    const int N = routed ? a.N_r : a.N_s;
    const int n0 = n_tile * cols_per_tile;

    // ---- per-thread source rows (4 A rows, 4 weight rows)
    const uint16_t* a_src[4];
    const uint16_t* b_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = ld_row + 32 * i;
      a_src[i] = nullptr;
      if (r < valid_rows) {
        if (routed) {
          const int64_t gr = grow0 + m0 + r;
          int64_t arow = gr;
          if (a.a_row_map) {
            arow = a.a_row_map[gr];
            if (arow < 0 || arow >= a.T) arow = 0;  // malformed permutation: stay in bounds
          }
          a_src[i] = a.a_routed + arow * K;
        } else {
          a_src[i] = a.a_shared + (m0 + r) * K;
        }
      }
      const uint16_t* wbase;
      int wrow;
      if (kSwiGLU) {
        // tile rows 0-31: W1[n0..], 32-63: W3[n0..], 64-95: W1[n0+32..], 96-127: W3[n0+32..]
        const bool up = (i & 1) != 0;
        wrow = n0 + (i >> 1) * 32 + ld_row;
        wbase = routed ? (up ? a.w3_routed : a.w_routed) + static_cast<int64_t>(g) * N * K
                       : (up ? a.w3_shared : a.w_shared);
      } else {
        wrow = n0 + 32 * i + ld_row;
        wbase = routed ? a.w_routed + static_cast<int64_t>(g) * N * K : a.w_shared;
      }
      b_src[i] = wrow < N ? wbase + static_cast<int64_t>(wrow) * K : nullptr;
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    uint4 ra[4], rb[4];
    auto fetch = [&](int k0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = a_src[i] ? *reinterpret_cast<const uint4*>(a_src[i] + k0 + ld_chunk * 8)
                         : make_uint4(0, 0, 0, 0);
        rb[i] = b_src[i] ? *reinterpret_cast<const uint4*>(b_src[i] + k0 + ld_chunk * 8)
                         : make_uint4(0, 0, 0, 0);
      }
    };
    auto stash = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = ld_row + 32 * i;
        lds_a[buf][swz(r, ld_chunk)] = ra[i];
        lds_b[buf][swz(r, ld_chunk)] = rb[i];
      }
    };

    const bool do_m0 = wm * 64 < valid_rows;
    const bool do_m1 = wm * 64 + 32 < valid_rows;
    const int nk = K / kBK;

    __syncthreads();  // previous unit's LDS reads are done
    fetch(0);
    stash(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) fetch((kt + 1) * kBK);
      if (do_m0) {
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
          const int ch = 2 * ks + (lane >> 5);
          const int fr = lane & 31;
          bf16x8 af[2], bfr[2];
#pragma unroll
          for (int i = 0; i < 2; ++i)
            af[i] = __builtin_bit_cast(bf16x8, lds_a[buf][swz(wm * 64 + 32 * i + fr, ch)]);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            bfr[j] = __builtin_bit_cast(bf16x8, lds_b[buf][swz(wn * 64 + 32 * j + fr, ch)]);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0], bfr[j], acc[0][j], 0, 0, 0);
            if (do_m1)
              acc[1][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[1], bfr[j], acc[1][j], 0, 0, 0);
          }
        }
      }
      if (kt + 1 < nk) {
        stash(buf ^ 1);
      }
      __syncthreads();
    }

    // ---- epilogue.  32x32 accumulator layout: lane holds column (lane & 31),
    // rows (v/4)*8 + (lane/32)*4 + v%4 for v = 0..15.
    const int col_l = lane & 31;
    const int row_l = (lane >> 5) * 4;
    uint16_t* cbase = routed ? a.c_routed : a.c_shared;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + 32 * i + (v >> 2) * 8 + row_l + (v & 3);
        if (r >= valid_rows) continue;
        const int64_t orow = grow0 + m0 + r;
        if (kSwiGLU) {
          const float ga = acc[i][0][v], up = acc[i][1][v];
          const float hval = ga / (1.0f + __expf(-ga)) * up;
          const int c = n0 + wn * 32 + col_l;
          cbase[orow * N + c] = f32_to_bf16(hval);
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int c = n0 + wn * 64 + 32 * j + col_l;
            if (c < N) cbase[orow * N + c] = f32_to_bf16(acc[i][j][v]);
          }
        }
      }
    }
  }
}

static int persistent_grid() {
  int g = 2 * device_cus();
  g = (g / kXcds) * kXcds;
  return g > 0 ? g : kXcds;
}

hipError_t launch_gemm_swiglu(const GroupedGemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((grouped_gemm_kernel<true>), dim3(persistent_grid()), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const GroupedGemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((grouped_gemm_kernel<false>), dim3(persistent_grid()), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
