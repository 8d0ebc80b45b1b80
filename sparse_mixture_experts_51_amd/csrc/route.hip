// route.hip -- router GEMM, sigmoid affinity, biased top-k, gates, balance statistic.
//
// Pages: "190行JAX复刻DeepSeek V3" (openai-hub.com), sections
// 190行代码到底装进了什么 (16 routed experts, 4 chosen per token, one shared
// expert) and 最有价值的实验:无辅助损失均衡真的有效 (the per-expert bias changes
// which experts win but not their gate scores; sequence-wise balance loss
// with weight 1e-4).
//
// Kernel 1 (router_scores): logits by an fp32 FMA chain over d in ascending
// order, one chain per (token, expert) register, so every logit is the same
// bit pattern on any hardware that does IEEE fused multiply-add.  This is a
// SIMT fp32 GEMM (MFMA would reorder the sums); x and W_r are staged through
// LDS with a register prefetch of the next d-chunk.  Scores = sigmoid in fp64,
// rounded once to fp32.
// Kernel 2 (select): one group of G lanes per token (G = next power of two
// of E, at most 64).  k+1 rounds of a 64-bit group max over
// (orderable key << 32 | ~expert) pick the largest key with the lowest index
// on ties; the (k+1)-th gives the margin.
// Kernels 3-4 (seq balance): per-slice partial sums, then one block per
// sequence reduces them in a fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kRouteThreads = 256;
constexpr int kKC = 32;  // d-chunk staged per LDS pass

template <int EPT, int TPT>
__global__ __launch_bounds__(kRouteThreads) void router_scores_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ w_router,
    float* __restrict__ scores, int64_t T, int d, int E, int BE) {
  const int TPR = BE / EPT;                 // threads per token row
  const int rows = kRouteThreads / TPR;     // token rows per block
  const int BT = rows * TPT;                // tokens per block
  const int tid = threadIdx.x;
  const int tx = tid % TPR, ty = tid / TPR;
  const int n_eblk = (E + BE - 1) / BE;
  const int eb = blockIdx.x % n_eblk;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x / n_eblk) * BT;
  const int e0 = eb * BE;

  extern __shared__ float lds[];
  float* xs = lds;               // [kKC][BT]
  float* ws = lds + kKC * BT;    // [kKC][BE]

  // Register staging of one d-chunk: x as 16-byte pieces (8 bf16), W as floats.
  const int x_pieces = BT * (kKC / 8);
  const int x_per_thr = (x_pieces + kRouteThreads - 1) / kRouteThreads;   // <= 4
  const int w_elems = kKC * BE;
  const int w_per_thr = (w_elems + kRouteThreads - 1) / kRouteThreads;    // <= 8
  uint4 xr[4];
  float wr[8];

  auto fetch = [&](int k0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (p >= x_per_thr) break;
      const int piece = tid + p * kRouteThreads;
      xr[p] = make_uint4(0, 0, 0, 0);
      if (piece < x_pieces) {
        const int tok = piece / (kKC / 8), c = piece % (kKC / 8);
        const int64_t t = t0 + tok;
        if (t < T) xr[p] = *reinterpret_cast<const uint4*>(x + t * d + k0 + c * 8);
      }
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      if (p >= w_per_thr) break;
      const int el = tid + p * kRouteThreads;
      wr[p] = 0.0f;
      if (el < w_elems) {
        const int kk = el / BE, c = el % BE;
        if (e0 + c < E) wr[p] = w_router[static_cast<int64_t>(k0 + kk) * E + e0 + c];
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (p >= x_per_thr) break;
      const int piece = tid + p * kRouteThreads;
      if (piece < x_pieces) {
        const int tok = piece / (kKC / 8), c = piece % (kKC / 8);
        float v[8];
        bf16x8_to_f32(xr[p], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) xs[(c * 8 + i) * BT + tok] = v[i];
      }
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      if (p >= w_per_thr) break;
      const int el = tid + p * kRouteThreads;
      if (el < w_elems) ws[el] = wr[p];  // [kk][c] layout == el
    }
  };

  float acc[TPT][EPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int j = 0; j < EPT; ++j) acc[i][j] = 0.0f;

  fetch(0);
  for (int k0 = 0; k0 < d; k0 += kKC) {
    __syncthreads();          // previous chunk fully consumed
    stash();
    __syncthreads();
    if (k0 + kKC < d) fetch(k0 + kKC);  // in flight during the FMAs below
#pragma unroll 8
    for (int kk = 0; kk < kKC; ++kk) {
      float xv[TPT], wv[EPT];
#pragma unroll
      for (int i = 0; i < TPT; ++i) xv[i] = xs[kk * BT + ty * TPT + i];
#pragma unroll
      for (int j = 0; j < EPT; ++j) wv[j] = ws[kk * BE + tx * EPT + j];
#pragma unroll
      for (int i = 0; i < TPT; ++i)
#pragma unroll
        for (int j = 0; j < EPT; ++j) acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
    }
  }

#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int64_t t = t0 + ty * TPT + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = e0 + tx * EPT + j;
      if (e < E) scores[t * E + e] = static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(acc[i][j]))));
    }
  }
}

static int next_pow2(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

template <int EPT, int TPT>
static hipError_t launch_scores_cfg(const uint16_t* x, const float* w, float* sc, int64_t T, int d,
                                    int E, int BE, hipStream_t s) {
  const int TPR = BE / EPT;
  const int BT = (kRouteThreads / TPR) * TPT;
  const int64_t nblk = ((T + BT - 1) / BT) * ((E + BE - 1) / BE);
  const size_t lds = sizeof(float) * kKC * (BT + BE);
  hipLaunchKernelGGL((router_scores_kernel<EPT, TPT>), dim3(static_cast<unsigned>(nblk)),
                     dim3(kRouteThreads), lds, s, x, w, sc, T, d, E, BE);
  return hipGetLastError();
}

hipError_t launch_router_scores(const uint16_t* x, const float* w_router, float* scores,
                                int64_t T, int d, int E, hipStream_t s) {
  // Pick the largest per-thread tile that still gives one block per CU; with
  // few tokens, trade tile size for blocks (each (token, expert) chain is
  // sequential over d, so parallelism is bounded by T*E lanes).
  const int Emax = next_pow2(E) < 64 ? next_pow2(E) : 64;
  struct Cfg { int BE, EPT, TPT; };
  auto ept_of = [](int BE) { return BE >= 64 ? 4 : (BE >= 32 ? 2 : 1); };
  const int want = device_cus();
  Cfg pick{0, 0, 0};
  int64_t best_blocks = -1;
  Cfg last{0, 0, 0};
  const int be_list[4] = {64, 32, 16, 8};
  const int tpt_list[3] = {4, 2, 1};
  for (int ti = 0; ti < 3 && !pick.BE; ++ti) {
    for (int bi = 0; bi < 4; ++bi) {
      int BE = be_list[bi] < Emax ? be_list[bi] : Emax;
      if (bi > 0 && BE == (be_list[bi - 1] < Emax ? be_list[bi - 1] : Emax)) continue;
      const int EPT = ept_of(BE) > BE ? BE : ept_of(BE);
      const int TPR = BE / EPT;
      const int TPT = tpt_list[ti];
      const int BT = (kRouteThreads / TPR) * TPT;
      if (BT > 256) continue;
      const int64_t blocks = ((T + BT - 1) / BT) * ((E + BE - 1) / BE);
      if (blocks >= want) { pick = {BE, EPT, TPT}; break; }
      if (blocks > best_blocks) { best_blocks = blocks; last = {BE, EPT, TPT}; }
    }
  }
  if (!pick.BE) pick = last;
  if (!pick.BE) pick = {Emax, 1, 1};
#define MOE_SCORES_CASE(e, t)                                                      \
  if (pick.EPT == e && pick.TPT == t)                                              \
    return launch_scores_cfg<e, t>(x, w_router, scores, T, d, E, pick.BE, s);
  MOE_SCORES_CASE(4, 4) MOE_SCORES_CASE(4, 2) MOE_SCORES_CASE(4, 1)
  MOE_SCORES_CASE(2, 4) MOE_SCORES_CASE(2, 2) MOE_SCORES_CASE(2, 1)
  MOE_SCORES_CASE(1, 4) MOE_SCORES_CASE(1, 2) MOE_SCORES_CASE(1, 1)
#undef MOE_SCORES_CASE
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Top-k selection and gates

__device__ __forceinline__ uint64_t pack_key(float key, int e) {
  const uint32_t lo = 0xFFFFFFFFu - static_cast<uint32_t>(e);  // lower index wins ties
  if (key != key) return static_cast<uint64_t>(lo);             // NaN: below every number
  if (key == 0.0f) key = 0.0f;                                   // -0 == +0
  return (static_cast<uint64_t>(orderable(key)) << 32) | lo;
}

template <int EPL>
__global__ __launch_bounds__(256) void select_kernel(
    const float* __restrict__ scores, const float* __restrict__ bias, int32_t* __restrict__ idx,
    float* __restrict__ gate, float* __restrict__ margin, double* __restrict__ tok_sum,
    int64_t T, int E, int k, int G) {
  const int lane = threadIdx.x % G;
  const int grp = threadIdx.x / G;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (256 / G) + grp;
  if (t >= T) return;  // whole group leaves together
  const float* srow = scores + t * E;

  uint64_t pk[EPL];
  double ssum = 0.0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + i * G;
    pk[i] = 0;  // padding and taken entries
    if (e < E) {
      const float sv = srow[e];
      ssum += static_cast<double>(sv);
      pk[i] = pack_key(sv + bias[e], e);
    }
  }

  int my_e = 0;
  float kth = 0.0f, next = 0.0f;
  const int rounds = (k < E) ? k + 1 : k;
  for (int r = 0; r < rounds; ++r) {
    uint64_t v = pk[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) v = pk[i] > v ? pk[i] : v;
    for (int off = G >> 1; off > 0; off >>= 1) {
      const uint64_t o = __shfl_xor(v, off, G);
      v = o > v ? o : v;
    }
    const int e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(v));
    const uint32_t hi = static_cast<uint32_t>(v >> 32);
    const float key = hi ? from_orderable(hi) : __uint_as_float(0x7FC00000u);
    if (r < k) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + i * G == e) pk[i] = 0;
      if (lane == r) my_e = e;
      if (r == k - 1) kth = key;
    } else {
      next = key;
    }
  }

  // Gates from the unbiased scores of the winners, summed in slot order.
  const float s_mine = (lane < k) ? srow[my_e] : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += __shfl(s_mine, j, G);
  if (lane < k) {
    idx[t * k + lane] = my_e;
    gate[t * k + lane] = (sum == 0.0f) ? 1.0f / static_cast<float>(k) : s_mine / sum;
  }
  if (lane == 0 && margin) margin[t] = (k < E) ? kth - next : __builtin_inff();
  if (tok_sum) {
    for (int off = G >> 1; off > 0; off >>= 1) ssum += __shfl_xor(ssum, off, G);
    if (lane == 0) tok_sum[t] = ssum;
  }
}

hipError_t launch_select(const float* scores, const float* bias, int32_t* idx, float* gate,
                         float* margin, double* tok_sum, int64_t T, int E, int k, hipStream_t s) {
  const int G = next_pow2(E) < 64 ? next_pow2(E) : 64;
  const int epl = (E + G - 1) / G;
  const int64_t nblk = (T + (256 / G) - 1) / (256 / G);
  const dim3 grid(static_cast<unsigned>(nblk)), block(256);
#define MOE_SEL_CASE(n)                                                                      \
  if (epl <= n) {                                                                            \
    hipLaunchKernelGGL((select_kernel<n>), grid, block, 0, s, scores, bias, idx, gate, margin, \
                       tok_sum, T, E, k, G);                                                  \
    return hipGetLastError();                                                                \
  }
  MOE_SEL_CASE(1) MOE_SEL_CASE(2) MOE_SEL_CASE(4) MOE_SEL_CASE(8) MOE_SEL_CASE(16)
#undef MOE_SEL_CASE
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Sequence-wise balance statistic

int seq_splits(int64_t T, int S) {
  if (S <= 0) return 0;
  const int64_t nseq = T / S;
  int64_t sp = (256 + nseq - 1) / nseq;
  const int64_t max_sp = S / 64 > 0 ? S / 64 : 1;
  if (sp > max_sp) sp = max_sp;
  if (sp < 1) sp = 1;
  return static_cast<int>(sp);
}

// grid (nseq * nsplit): each block walks a slice of one sequence; thread e
// accumulates sum_t s[t,e]/tok_sum[t] in fp64 in token order, and the block
// counts choices with LDS atomics.
__global__ __launch_bounds__(256) void seq_partial_kernel(
    const float* __restrict__ scores, const double* __restrict__ tok_sum,
    const int32_t* __restrict__ idx, double* __restrict__ seq_p, int32_t* __restrict__ seq_cnt,
    int E, int k, int S, int nsplit) {
  extern __shared__ int32_t cnt[];  // [E]
  const int q = blockIdx.x / nsplit, sp = blockIdx.x % nsplit;
  const int64_t a = static_cast<int64_t>(q) * S + static_cast<int64_t>(S) * sp / nsplit;
  const int64_t b = static_cast<int64_t>(q) * S + static_cast<int64_t>(S) * (sp + 1) / nsplit;
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  for (int64_t i = a * k + threadIdx.x; i < b * k; i += 256) atomicAdd(&cnt[idx[i]], 1);
  for (int e = threadIdx.x; e < E; e += 256) {
    double p = 0.0;
    for (int64_t t = a; t < b; ++t) {
      const double tot = tok_sum[t];
      p += (tot == 0.0) ? 1.0 / E : static_cast<double>(scores[t * E + e]) / tot;
    }
    seq_p[static_cast<int64_t>(blockIdx.x) * E + e] = p;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) seq_cnt[static_cast<int64_t>(blockIdx.x) * E + e] = cnt[e];
}

__global__ __launch_bounds__(256) void seq_final_kernel(
    const double* __restrict__ seq_p, const int32_t* __restrict__ seq_cnt, float* __restrict__ out,
    float alpha, int E, int k, int S, int nsplit) {
  __shared__ double part[256];
  const int q = blockIdx.x;
  double acc = 0.0;
  for (int e = threadIdx.x; e < E; e += 256) {
    double p = 0.0;
    int64_t c = 0;
    for (int sp = 0; sp < nsplit; ++sp) {
      const int64_t o = (static_cast<int64_t>(q) * nsplit + sp) * E + e;
      p += seq_p[o];
      c += seq_cnt[o];
    }
    const double f = static_cast<double>(E) / (static_cast<double>(k) * S) * static_cast<double>(c);
    acc += f * (p / S);
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[q] = static_cast<float>(static_cast<double>(alpha) * part[0]);
}

hipError_t launch_seq_balance(const float* scores, const double* tok_sum, const int32_t* idx,
                              double* seq_p, int32_t* seq_cnt, float* out, float alpha,
                              int64_t T, int E, int k, int S, hipStream_t s) {
  const int nsplit = seq_splits(T, S);
  const int64_t nseq = T / S;
  hipLaunchKernelGGL(seq_partial_kernel, dim3(static_cast<unsigned>(nseq * nsplit)), dim3(256),
                     sizeof(int32_t) * E, s, scores, tok_sum, idx, seq_p, seq_cnt, E, k, S, nsplit);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(seq_final_kernel, dim3(static_cast<unsigned>(nseq)), dim3(256), 0, s, seq_p,
                     seq_cnt, out, alpha, E, k, S, nsplit);
  return hipGetLastError();
}

}  // namespace moe
