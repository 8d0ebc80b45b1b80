// permute.hip -- per-expert loads, group offsets and the expert-grouped row order.
//
// Only the chosen experts run: rows are grouped by expert so that each expert
// sees one contiguous block of rows (the sparse dispatch that the pages' dense
// reference lacks -- "DeepSeek V3 viết lại bằng 190 dòng JAX thuần" (lehuy.net),
// section Những gì đã được đơn giản hóa).  The loads are what the bias rule
// reads ("190行JAX复刻DeepSeek V3" (openai-hub.com), section
// 最有价值的实验:无辅助损失均衡真的有效).
//
// Three kernels over blocks of TB = 256 tokens:
//   count:   LDS-privatised histogram of the block's k*tokens choices
//   scan:    one block; per expert a running sum over token blocks gives each
//            block's first row, and a block-wide scan over experts gives offsets
//   scatter: the block's choices as an LDS bitmap [E][TB bits]; the
//            rank of (t, e) among earlier tokens of the block choosing e is a
//            popcount, so rows inside a group are in ascending token order
//            without sorting.
// and, when x_perm is asked for, a gather of x rows into it over the whole
// chip (the scatter's few blocks would copy them on a few CUs).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Exclusive scan of one int per thread over a 1024-thread block; returns the
// block total through *total.
__device__ int block_exclusive_scan_1024(int v, int* total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < 16; ++i) {
      const int c = wsum[i];
      wsum[i] = run;
      run += c;
    }
    *total = run;
  }
  __syncthreads();
  return wsum[w] + inc - v;
}

template <int TB>
__global__ __launch_bounds__(TB) void perm_count_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ blk_cnt, int64_t T, int E, int k) {
  extern __shared__ int32_t cnt[];  // [E]
  for (int e = threadIdx.x; e < E; e += TB) cnt[e] = 0;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * TB + threadIdx.x;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += TB)
    blk_cnt[static_cast<int64_t>(blockIdx.x) * E + e] = cnt[e];
}

__global__ __launch_bounds__(1024) void perm_scan_kernel(
    const int32_t* __restrict__ blk_cnt, int32_t* __restrict__ blk_base,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int nblk, int E) {
  __shared__ int total;
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int b = 0; b < nblk; ++b) {
      const int64_t o = static_cast<int64_t>(b) * E + e;
      const int c = blk_cnt[o];
      blk_base[o] = run;
      run += c;
    }
    counts[e] = run;
  }
  const int off = block_exclusive_scan_1024(e < E ? run : 0, &total);
  if (e < E) {
    offsets[e] = off;
    for (int b = 0; b < nblk; ++b) blk_base[static_cast<int64_t>(b) * E + e] += off;
  }
  if (e == 0) offsets[E] = total;
}

// Exclusive scan of one int per thread over a TB-thread block.
template <int TB>
__device__ int block_exclusive_scan(int v, int* total) {
  __shared__ int wsum[TB / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < TB / 64; ++i) {
    base += i < w ? wsum[i] : 0;
    tot += wsum[i];
  }
  *total = tot;
  __syncthreads();
  return base + inc - v;
}

// fused_scan: the block derives its own first rows (and block 0 the counts and
// offsets) from the per-block count table, which is small enough for LDS;
// otherwise blk_base comes from perm_scan_kernel.
template <int TB>
__global__ __launch_bounds__(TB) void perm_scatter_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ blk_cnt,
    const int32_t* __restrict__ blk_base, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src, int32_t* __restrict__ pos,
    int64_t T, int E, int k, int nblk, int fused_scan) {
  constexpr int W = TB / 32;         // 32-bit words per expert row of the bitmap
  extern __shared__ uint32_t bits[];  // [E][W], base [E], total [E] (fused)
  int32_t* base = reinterpret_cast<int32_t*>(bits + E * W);
  int32_t* etot = base + E;
  for (int i = threadIdx.x; i < E * W; i += TB) bits[i] = 0;
  if (fused_scan) {
    // Per expert e: rows in blocks before this one, and in all blocks.  L
    // lanes share an expert (block b2 to lane b2 mod L); lane partial sums
    // are combined with shuffles inside groups of L consecutive lanes, which
    // must lie in one wave (at most 64 lanes, also when E < TB / 64).
    int L = E >= TB ? 1 : TB / E;  // power of two when E divides TB
    if (L > kWave) L = kWave;
    const int Lp = (L & (L - 1)) == 0 ? L : 1;
    const int l = threadIdx.x % Lp;
    for (int e = threadIdx.x / Lp; e < E; e += TB / Lp) {
      int before = 0, total = 0;
      for (int b2 = l; b2 < nblk; b2 += Lp) {
        const int c = blk_cnt[static_cast<int64_t>(b2) * E + e];
        before += b2 < static_cast<int>(blockIdx.x) ? c : 0;
        total += c;
      }
      for (int off = Lp >> 1; off > 0; off >>= 1) {
        before += __shfl_xor(before, off, Lp);
        total += __shfl_xor(total, off, Lp);
      }
      if (l == 0) {
        base[e] = before;
        etot[e] = total;
      }
    }
    __syncthreads();
    // exclusive scan of the totals over experts: offsets
    const int per = (E + TB - 1) / TB;
    const int c0 = threadIdx.x * per;
    int tot_local = 0;
    for (int e = c0; e < c0 + per && e < E; ++e) tot_local += etot[e];
    int all;
    int run = block_exclusive_scan<TB>(tot_local, &all);
    for (int e = c0; e < c0 + per && e < E; ++e) {
      const int total = etot[e];
      base[e] += run;
      if (blockIdx.x == 0) {
        counts[e] = total;
        offsets[e] = run;
      }
      run += total;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) offsets[E] = all;
  }
  __syncthreads();
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TB;
  const int64_t t = t0 + threadIdx.x;
  const int word = threadIdx.x / 32, bit = threadIdx.x % 32;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e >= 0 && e < E) atomicOr(&bits[e * W + word], 1u << bit);
    }
  }
  __syncthreads();
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      int row = -1;
      if (e >= 0 && e < E) {
        int rank = __popc(bits[e * W + word] & ((1u << bit) - 1u));
        for (int w = 0; w < word; ++w) rank += __popc(bits[e * W + w]);
        row = (fused_scan ? base[e] : blk_base[static_cast<int64_t>(blockIdx.x) * E + e]) + rank;
        perm_src[row] = static_cast<int32_t>(t);
      }
      pos[t * k + j] = row;
    }
  }
}

// x_perm[r] = x[perm_src[r]] for the rows r < offsets[E] that the scatter
// filled: 16 bytes per thread and trip, consecutive threads along a row,
// grid-strided.  A source index outside [0, T) (malformed choices) leaves its
// row untouched.
__global__ __launch_bounds__(256) void perm_gather_kernel(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ perm_src,
                                                          const int32_t* __restrict__ offsets,
                                                          uint16_t* __restrict__ x_perm, int64_t T,
                                                          int d, int E, int64_t nrows) {
  const int chunks = d / 8;
  const int64_t filled = offsets[E];
  const int64_t rows = filled < nrows ? filled : nrows;
  const int64_t work = rows * chunks;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < work; i += stride) {
    const int64_t r = i / chunks;
    const int c = static_cast<int>(i - r * chunks);
    const int64_t t = perm_src[r];
    if (t < 0 || t >= T) continue;
    reinterpret_cast<uint4*>(x_perm + r * d)[c] = reinterpret_cast<const uint4*>(x + t * d)[c];
  }
}

template <int TB>
static hipError_t launch_permute_tb(const int32_t* idx, int32_t* counts, int32_t* offsets,
                                    int32_t* perm_src, int32_t* pos, const uint16_t* x,
                                    uint16_t* x_perm, int32_t* blk_cnt, int32_t* blk_base,
                                    int64_t T, int d, int E, int k, hipStream_t s) {
  const int nblk = static_cast<int>((T + TB - 1) / TB);
  hipError_t err;
  if (nblk == 0) {
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, s, blk_cnt, blk_base, counts,
                       offsets, nblk, E);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((perm_count_kernel<TB>), dim3(nblk), dim3(TB), sizeof(int32_t) * E, s, idx,
                     blk_cnt, T, E, k);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  // Small count tables are summed by every scatter block itself (one launch
  // fewer); large ones go through the single-block scan.
  const size_t lds_base = sizeof(uint32_t) * E * (TB / 32);
  const size_t lds_fused = lds_base + 2 * sizeof(int32_t) * E;
  const int fused = static_cast<int64_t>(nblk) * E <= 16384 && lds_fused <= 64 * 1024;
  if (!fused) {
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, s, blk_cnt, blk_base, counts,
                       offsets, nblk, E);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL((perm_scatter_kernel<TB>), dim3(nblk), dim3(TB), fused ? lds_fused : lds_base,
                     s, idx, blk_cnt, blk_base, counts, offsets, perm_src, pos, T, E, k, nblk, fused);
  err = hipGetLastError();
  if (err != hipSuccess || x_perm == nullptr) return err;
  const int64_t nrows = T * k;
  const int64_t blocks = (nrows * (d / 8) + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(perm_gather_kernel, dim3(grid > 0 ? grid : 1), dim3(256), 0, s, x, perm_src, offsets,
                     x_perm, T, d, E, nrows);
  return hipGetLastError();
}

int perm_block_tokens(int64_t) { return kPermTokens; }

hipError_t launch_permute(const int32_t* idx, int32_t* counts, int32_t* offsets,
                          int32_t* perm_src, int32_t* pos, const uint16_t* x, uint16_t* x_perm,
                          int32_t* blk_cnt, int32_t* blk_base, int64_t T, int d, int E, int k,
                          hipStream_t s) {
  return launch_permute_tb<kPermTokens>(idx, counts, offsets, perm_src, pos, x, x_perm, blk_cnt,
                                        blk_base, T, d, E, k, s);
}

}  // namespace moe
