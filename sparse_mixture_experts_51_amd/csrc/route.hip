// route.hip -- router GEMM, sigmoid affinity, biased top-k, gates, balance statistic.
//
// Pages: "190行JAX复刻DeepSeek V3" (openai-hub.com), sections
// 190行代码到底装进了什么 (16 routed experts, 4 chosen per token, one shared
// expert) and 最有价值的实验:无辅助损失均衡真的有效 (the per-expert bias changes
// which experts win but not their gate scores; sequence-wise balance loss
// with weight 1e-4).
//
// Kernel 1 (router scores): logits by an fp32 FMA chain over d in ascending
// order, so every logit is the same bit pattern on any hardware that does
// IEEE fused multiply-add.  Two forms compute that same chain:
//   - router_scores_kernel / router_fused_kernel: a SIMT fp32 GEMM, one chain
//     per (token, expert) register, x and W_r staged through LDS with a
//     register prefetch of the next d-chunk;
//   - router_scores_mfma_kernel (many tokens, E a multiple of 64): the fp32
//     matrix cores with K = 1 (v_mfma_f32_16x16x1_4b_f32).  One instruction
//     adds one product to each output and rounds once, so a chain of them
//     over d ascending is the fmaf chain; a wider K would reorder the sums.
// Scores = sigmoid in fp64, rounded once to fp32.
// Kernel 2 (select): one group of G lanes per token (G = 16, 32 or 64 as E
// fits).  k+1 rounds of a 64-bit group max over (orderable key << 32 |
// ~expert), reduced with DPP lane moves, pick the largest key with the
// lowest index on ties; the (k+1)-th gives the margin.
// Kernels 3-4 (seq balance): per-slice partial sums, then one block per
// sequence reduces them in a fixed order.
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace moe {

constexpr int kRouteThreads = 256;
constexpr int kRouteLds = 64 * 1024;       // LDS budget of one router block (two per CU)
constexpr int kRouteLdsOne = 160 * 1024;   // ... when there are no more blocks than CUs

// LDS-only barrier: waits for this wave's LDS traffic, not for global loads,
// so the next chunk's loads stay in flight across it.
__device__ __forceinline__ void route_lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// Block tile: BT tokens x BE experts; thread tile: TPT tokens x EPT experts
// (TPR = BE/EPT threads per token row).  d is walked in chunks of KC.  A
// chunk's x rows (converted to fp32 when staged, [BT][KC]: the FMAs then
// need no conversion, which the BE / EPT threads of a token row would each
// repeat) and W_r columns (fp32, [TPR][KC][EPT]: a thread's EPT experts
// adjacent) sit in LDS with rows padded by 16 bytes, so the lanes of a wave
// read distinct banks; one 16-byte LDS read gives a thread 4 values.  With more than one chunk, the next chunk is
// prefetched into registers while this one is multiplied.  Every (token,
// expert) logit is one fp32 fmaf chain over d in ascending order.
template <int EPT, int TPT>
__device__ __forceinline__ void router_logits_tile(const uint16_t* __restrict__ x,
                                                   const float* __restrict__ w_router, int64_t T,
                                                   int d, int E, int BE, int KC,
                                                   unsigned char* lds_raw,
                                                   float (&acc)[TPT][EPT]) {
  const int TPR = BE / EPT;
  const int rows = kRouteThreads / TPR;
  const int BT = rows * TPT;
  const int tid = threadIdx.x;
  const int tx = tid % TPR, ty = tid / TPR;
  const int n_eblk = (E + BE - 1) / BE;
  const int e0 = (blockIdx.x % n_eblk) * BE;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x / n_eblk) * BT;
  const int nchunks = d / KC;

  const int xrow = KC * 4 + 16, wrow = KC * EPT * 4 + 16;  // padded row strides (bytes)
  const int bufbytes = BT * xrow + TPR * wrow;
  auto xs = [&](int b) { return lds_raw + b * bufbytes; };
  auto ws = [&](int b) { return lds_raw + b * bufbytes + BT * xrow; };

  // A chunk is BT*KC/8 16-byte pieces of x (a row has CX = KC/8) and KC*BE/4
  // pieces of W (a d-row has CW = BE/4).  Thread tid takes pieces tid,
  // tid + 256, ...; their (row, column) advance incrementally (no divisions).
  const int CX = KC / 8, CW = BE / 4;
  const int nx = (BT * CX - tid + kRouteThreads - 1) / kRouteThreads;  // x pieces of this thread
  const int nw = (KC * CW - tid + kRouteThreads - 1) / kRouteThreads;  // W pieces of this thread
  const int x_r0 = tid / CX, x_c0 = tid % CX;
  const int w_r0 = tid / CW, w_c0 = tid % CW;
  const int x_dr = kRouteThreads / CX, x_dc = kRouteThreads % CX;
  const int w_dr = kRouteThreads / CW, w_dc = kRouteThreads % CW;
  constexpr int kMaxX = 8, kMaxW = 8;  // LDS budget bounds both
  uint4 rx[kMaxX], rw[kMaxW];
  auto fetch = [&](int k0) {
    int r = x_r0, c = x_c0;
#pragma unroll
    for (int p = 0; p < kMaxX; ++p) {
      if (p >= nx) break;
      const int64_t t = t0 + r;
      rx[p] = t < T ? *reinterpret_cast<const uint4*>(x + t * d + k0 + c * 8) : make_uint4(0, 0, 0, 0);
      r += x_dr;
      c += x_dc;
      if (c >= CX) { c -= CX; ++r; }
    }
    r = w_r0;
    c = w_c0;
#pragma unroll
    for (int p = 0; p < kMaxW; ++p) {
      if (p >= nw) break;
      const int e = e0 + c * 4;
      const float* src = w_router + static_cast<int64_t>(k0 + r) * E + e;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e + 3 < E && ((E & 3) == 0)) {
        v = *reinterpret_cast<const float4*>(src);
      } else {
        if (e + 0 < E) v.x = src[0];
        if (e + 1 < E) v.y = src[1];
        if (e + 2 < E) v.z = src[2];
        if (e + 3 < E) v.w = src[3];
      }
      rw[p] = make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                         __float_as_uint(v.w));
      r += w_dr;
      c += w_dc;
      if (c >= CW) { c -= CW; ++r; }
    }
  };
  auto stash = [&](int b) {
    unsigned char* xb = xs(b);
    unsigned char* wb = ws(b);
    int r = x_r0, c = x_c0;
#pragma unroll
    for (int p = 0; p < kMaxX; ++p) {
      if (p >= nx) break;
      float f[8];
      bf16x8_to_f32(rx[p], f);
      *reinterpret_cast<float4*>(xb + r * xrow + c * 32) = make_float4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<float4*>(xb + r * xrow + c * 32 + 16) = make_float4(f[4], f[5], f[6], f[7]);
      r += x_dr;
      c += x_dc;
      if (c >= CX) { c -= CX; ++r; }
    }
    r = w_r0;
    c = w_c0;
#pragma unroll
    for (int p = 0; p < kMaxW; ++p) {
      if (p >= nw) break;
      // experts c*4 .. c*4+3 at d-row r -> [expert / EPT][r][expert % EPT]
      const uint32_t v[4] = {rw[p].x, rw[p].y, rw[p].z, rw[p].w};
      if constexpr (EPT == 4) {
        *reinterpret_cast<uint4*>(wb + c * wrow + r * 16) = rw[p];
      } else if constexpr (EPT == 2) {
        *reinterpret_cast<uint2*>(wb + (2 * c) * wrow + r * 8) = make_uint2(v[0], v[1]);
        *reinterpret_cast<uint2*>(wb + (2 * c + 1) * wrow + r * 8) = make_uint2(v[2], v[3]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(wb + (c * 4 + i) * wrow + r * 4) = v[i];
      }
      r += w_dr;
      c += w_dc;
      if (c >= CW) { c -= CW; ++r; }
    }
  };

#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int j = 0; j < EPT; ++j) acc[i][j] = 0.0f;

  // Small thread tiles unroll by four chunks of 8 (KC is a multiple of 32) so
  // that the scheduler can read the next chunks' operands from LDS while the
  // FMAs of the current one run; they run few waves per SIMD, and nothing
  // else would hide the LDS latency.  Large tiles have the ILP already and
  // would spend the registers.
  constexpr int kUnroll = TPT * EPT <= 2 ? 4 : 1;
  auto compute = [&](int b) {
    const unsigned char* xb = xs(b) + ty * TPT * xrow;
    const unsigned char* wb = ws(b) + tx * wrow;
#pragma unroll kUnroll
    for (int kk = 0; kk < KC; kk += 8) {
      float xv[TPT][8], wv[8 * EPT];
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        const float4 q0 = *reinterpret_cast<const float4*>(xb + i * xrow + kk * 4);
        const float4 q1 = *reinterpret_cast<const float4*>(xb + i * xrow + kk * 4 + 16);
        xv[i][0] = q0.x; xv[i][1] = q0.y; xv[i][2] = q0.z; xv[i][3] = q0.w;
        xv[i][4] = q1.x; xv[i][5] = q1.y; xv[i][6] = q1.z; xv[i][7] = q1.w;
      }
#pragma unroll
      for (int h = 0; h < 2 * EPT; ++h) {
        const float4 q = *reinterpret_cast<const float4*>(wb + kk * EPT * 4 + h * 16);
        wv[4 * h] = q.x; wv[4 * h + 1] = q.y; wv[4 * h + 2] = q.z; wv[4 * h + 3] = q.w;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < TPT; ++i)
#pragma unroll
          for (int j = 0; j < EPT; ++j) acc[i][j] = fmaf(xv[i][u], wv[u * EPT + j], acc[i][j]);
    }
  };

  fetch(0);
  stash(0);
  route_lds_barrier();
  for (int c = 0; c < nchunks; ++c) {
    if (c + 1 < nchunks) fetch((c + 1) * KC);  // in flight during the FMAs below
    compute(c & 1);
    if (c + 1 < nchunks) {
      stash((c + 1) & 1);
      route_lds_barrier();
    }
  }
}

// Affinity score: the logistic function evaluated in fp64, rounded once.
__device__ __forceinline__ float sigmoid_score(float logit) {
  return static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(logit))));
}

template <int EPT, int TPT>
__global__ __launch_bounds__(kRouteThreads) void router_scores_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ w_router,
    float* __restrict__ scores, int64_t T, int d, int E, int BE, int KC) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  float acc[TPT][EPT];
  router_logits_tile<EPT, TPT>(x, w_router, T, d, E, BE, KC, lds_raw, acc);
  const int TPR = BE / EPT;
  const int tx = threadIdx.x % TPR, ty = threadIdx.x / TPR;
  const int n_eblk = (E + BE - 1) / BE;
  const int e0 = (blockIdx.x % n_eblk) * BE;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x / n_eblk) * ((kRouteThreads / TPR) * TPT);
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int64_t t = t0 + ty * TPT + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = e0 + tx * EPT + j;
      if (e < E) scores[t * E + e] = sigmoid_score(acc[i][j]);
    }
  }
}

static int next_pow2(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// Lanes per token in the selection: 16, 32 or 64 (see group_max).
static int select_group(int E) { return E <= 16 ? 16 : (E <= 32 ? 32 : 64); }

struct RouterCfg {
  int BE, EPT, TPT, KC;
  int64_t blocks;
  size_t lds;
};

static RouterCfg router_cfg(int64_t T, int d, int E, int want_blocks, bool whole_e = false) {
  // Largest per-thread tile that still gives want_blocks blocks (with few
  // tokens, trade tile size for blocks: each (token, expert) chain is serial
  // over d, so parallelism is bounded by T*E lanes).  A chunk of d is the
  // whole of d when x and W_r tiles fit the LDS budget; else the longest
  // power-of-two double-buffered chunk that fits.
  // W_r is staged in 16-byte pieces of 4 experts, so a tile spans at least 4
  // (with E < 4 the missing experts are zero-filled and never stored)
  const int Emax = next_pow2(E) < 4 ? 4 : (next_pow2(E) < 64 ? next_pow2(E) : 64);
  auto ept_of = [](int BE) { return BE >= 64 ? 4 : (BE >= 32 ? 2 : 1); };
  RouterCfg best{0, 0, 0, 0, -1, 0};
  const int be_list[4] = {64, 32, 16, 8};
  const int tpt_list[3] = {4, 2, 1};
  for (int ti = 0; ti < 3; ++ti) {
    for (int bi = 0; bi < 4; ++bi) {
      const int BE = be_list[bi] < Emax ? be_list[bi] : Emax;
      if (whole_e && BE != Emax) continue;  // one block holds all experts of its tokens
      const int EPT = ept_of(BE) > BE ? BE : ept_of(BE);
      const int TPR = BE / EPT;
      const int TPT = tpt_list[ti];
      const int BT = (kRouteThreads / TPR) * TPT;
      if (BT > 256) continue;
      const int64_t blocks = ((T + BT - 1) / BT) * ((E + BE - 1) / BE);
      // few blocks (few tokens): one per CU, and all of its LDS for longer
      // chunks of d -- fewer chunk barriers and load round trips
      const size_t budget = blocks <= device_cus() ? kRouteLdsOne : kRouteLds;
      auto bytes = [&](int KC) {
        return static_cast<size_t>(BT * (KC * 4 + 16) + TPR * (KC * EPT * 4 + 16));
      };
      auto fits = [&](int KC) {  // at most 8 pieces of x and 8 of W per thread
        return static_cast<int64_t>(BT) * (KC / 8) <= 8 * kRouteThreads &&
               static_cast<int64_t>(KC) * (BE / 4) <= 8 * kRouteThreads;
      };
      int KC;
      size_t lds;
      if (bytes(d) <= budget && fits(d)) {
        KC = d;
        lds = bytes(d);
      } else {
        // the largest power-of-two chunk that divides d and fits twice: long
        // chunks give the register prefetch of the next one time to land
        KC = 32;
        for (int kc = 64; kc < d; kc *= 2)
          if (d % kc == 0 && 2 * bytes(kc) <= budget && fits(kc)) KC = kc;
        lds = 2 * bytes(KC);
      }
      const RouterCfg c{BE, EPT, TPT, KC, blocks, lds};
      if (blocks >= want_blocks) return c;
      if (blocks > best.blocks) best = c;
    }
  }
  return best;
}

template <int EPT, int TPT>
static hipError_t launch_scores_cfg(const uint16_t* x, const float* w, float* sc, int64_t T, int d,
                                    int E, const RouterCfg& c, hipStream_t s) {
  if (c.lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&router_scores_kernel<EPT, TPT>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(c.lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((router_scores_kernel<EPT, TPT>), dim3(static_cast<unsigned>(c.blocks)),
                     dim3(kRouteThreads), c.lds, s, x, w, sc, T, d, E, c.BE, c.KC);
  return hipGetLastError();
}

// Router scores on the fp32 matrix cores, for many tokens.  The fp32 MFMA
// with K = 1 (v_mfma_f32_16x16x1_4b_f32) adds one product per output per
// instruction with a single rounding, so a chain of them over d ascending is
// the same fmaf chain as in router_logits_tile, bit for bit, at twice the
// rate of the non-packed vector FMA.  The instruction holds four 16x16
// blocks: block b takes its 16 rows from A lanes 16b..16b+15 and its 16
// columns from B lanes 16b..16b+15, and element i of lane l is row
// 4 (l / 16) + i % 4, column l % 16 of block i / 4.  A wave puts the same 16
// tokens in every block's rows and 64 experts (16 per block) in the columns:
// 16 tokens x 64 experts per wave, one instruction per index of d.  A block of
// four waves (64 tokens) stages x as fp32 and W_r transposed to
// [expert][index of d] in LDS, in chunks of 128 of d.
constexpr int kMfTok = 64;     // tokens per block (16 per wave)
constexpr int kMfExp = 64;     // experts per block
constexpr int kMfKC = 128;     // d per staged chunk
constexpr int kMfRow = kMfKC + 4;  // LDS row in floats (16-byte pad)

__global__ __launch_bounds__(256) void router_scores_mfma_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ w_router, float* __restrict__ scores,
    int64_t T, int d, int E) {
  __shared__ float xs[2][kMfTok * kMfRow];
  __shared__ float wt[2][kMfExp * kMfRow];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kMfTok;
  const int e0 = blockIdx.y * kMfExp;
  // staging: x piece p (8 values) = row p / 16, cols 8 (p % 16); W piece q
  // (4 experts of one index of d) = index q / 16, experts 4 (q % 16)
  constexpr int kXP = kMfTok * kMfKC / 8 / 256;  // x pieces per thread (4)
  constexpr int kWP = kMfKC * kMfExp / 4 / 256;  // W pieces per thread (8)
  // Buffer loads: each thread's byte offsets are fixed and a chunk moves only
  // the scalar offset, so a fetch is twelve load instructions with no address
  // arithmetic or branches between them (64-bit address sums and a branch per
  // row check made the compiler wait for the first loads of a chunk before
  // issuing the rest).  The x descriptor covers this block's rows that exist:
  // a row past T reads as zeros and its scores are never stored.
  const int64_t xrows = T - t0 < kMfTok ? T - t0 : kMfTok;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + t0 * d), static_cast<short>(0), static_cast<int>(xrows * d * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(w_router + e0), static_cast<short>(0),
      static_cast<int>((static_cast<int64_t>(d) * E - e0) * 4), 0x00020000);
  int xoff[kXP], woff[kWP];
#pragma unroll
  for (int i = 0; i < kXP; ++i) {
    const int p = tid + 256 * i;
    xoff[i] = (p / 16) * d * 2 + (p % 16) * 16;
  }
#pragma unroll
  for (int i = 0; i < kWP; ++i) {
    const int q = tid + 256 * i;
    woff[i] = ((q / 16) * E + (q % 16) * 4) * 4;
  }
  u32x4 px[kXP], pw[kWP];
  auto fetch = [&](int c) {
    const int xs_off = c * kMfKC * 2, ws_off = c * kMfKC * E * 4;
#pragma unroll
    for (int i = 0; i < kXP; ++i)  // read once: non-temporal
      px[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[i], xs_off, 2);
#pragma unroll
    for (int i = 0; i < kWP; ++i) pw[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, woff[i], ws_off, 0);
  };
  auto stash_x = [&](int b, int i) __attribute__((always_inline)) {
    const int p = tid + 256 * i;
    float f[8];
    bf16x8_to_f32(make_uint4(px[i][0], px[i][1], px[i][2], px[i][3]), f);
    float* dst = &xs[b][(p / 16) * kMfRow + (p % 16) * 8];
    *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
  };
  auto stash_w = [&](int b, int i) __attribute__((always_inline)) {
    const int q = tid + 256 * i;
    const int kk = q / 16, e = (q % 16) * 4;
    wt[b][(e + 0) * kMfRow + kk] = __uint_as_float(pw[i][0]);
    wt[b][(e + 1) * kMfRow + kk] = __uint_as_float(pw[i][1]);
    wt[b][(e + 2) * kMfRow + kk] = __uint_as_float(pw[i][2]);
    wt[b][(e + 3) * kMfRow + kk] = __uint_as_float(pw[i][3]);
  };
  auto stash = [&](int b) {
#pragma unroll
    for (int i = 0; i < kXP; ++i) stash_x(b, i);
#pragma unroll
    for (int i = 0; i < kWP; ++i) stash_w(b, i);
  };
  f32x16 acc = {};
  const int nch = d / kMfKC;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    if (c + 1 < nch) fetch(c + 1);  // in flight during the MFMAs below
    const float* xr = &xs[c & 1][(16 * wave + (lane & 15)) * kMfRow];  // A: token lane % 16
    const float* wr = &wt[c & 1][lane * kMfRow];                      // B: expert lane
    const bool more = c + 1 < nch;
    const int nb = (c + 1) & 1;  // the buffers step c - 1 read
    // operands of 16 indices of d per group, read one group ahead so that
    // the LDS latency hides behind the previous group's MFMA chain
    float4 xa[2][4], wa[2][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xa[0][q] = *reinterpret_cast<const float4*>(xr + 4 * q);
      wa[0][q] = *reinterpret_cast<const float4*>(wr + 4 * q);
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int cb = g & 1;
      if (g + 1 < 8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xa[cb ^ 1][q] = *reinterpret_cast<const float4*>(xr + 16 * (g + 1) + 4 * q);
          wa[cb ^ 1][q] = *reinterpret_cast<const float4*>(wr + 16 * (g + 1) + 4 * q);
        }
      }
      // keeps those reads ahead of this group's MFMAs: left to itself the
      // scheduler sinks them to a few MFMAs before their use, and the chain
      // then waits on LDS reads queued behind the other waves'
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a4 = xa[cb][q], b4 = wa[cb][q];
        acc = __builtin_amdgcn_mfma_f32_16x16x1f32(a4.x, b4.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x1f32(a4.y, b4.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x1f32(a4.z, b4.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x1f32(a4.w, b4.w, acc, 0, 0, 0);
      }
      // the next chunk goes to LDS in the issue slots that the dependent
      // MFMA chain leaves, in the second half (its loads have landed by then)
      if (more) {
        if (g == 4) { stash_x(nb, 0); stash_x(nb, 1); }
        if (g == 5) { stash_x(nb, 2); stash_x(nb, 3); }
        if (g == 6) { stash_w(nb, 0); stash_w(nb, 1); stash_w(nb, 2); stash_w(nb, 3); }
        if (g == 7) { stash_w(nb, 4); stash_w(nb, 5); stash_w(nb, 6); stash_w(nb, 7); }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t t = t0 + 16 * wave + 4 * (lane / 16) + (i % 4);
    const int e = e0 + 16 * (i / 4) + (lane % 16);
    if (t < T) scores[t * E + e] = sigmoid_score(acc[i]);
  }
}

hipError_t launch_router_scores(const uint16_t* x, const float* w_router, float* scores,
                                int64_t T, int d, int E, hipStream_t s) {
  // (the kernel's buffer offsets are 32-bit: a block's rows of x and all of
  // W_r stay below 2 GiB)
  if (T >= 1024 && E % kMfExp == 0 && d % kMfKC == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(w_router) & 15) == 0 && static_cast<int64_t>(d) * E * 4 < 0x7FFFFFFF &&
      static_cast<int64_t>(kMfTok) * d * 2 < 0x7FFFFFFF) {
    const dim3 grid(static_cast<unsigned>((T + kMfTok - 1) / kMfTok), static_cast<unsigned>(E / kMfExp));
    hipLaunchKernelGGL(router_scores_mfma_kernel, grid, dim3(256), 0, s, x, w_router, scores, T, d, E);
    return hipGetLastError();
  }
  // two blocks per CU: with one, each SIMD holds a single wave and the LDS
  // latency of the operand reads is exposed
  const RouterCfg pick = router_cfg(T, d, E, 2 * device_cus());
#define MOE_SCORES_CASE(e, t)                                               \
  if (pick.EPT == e && pick.TPT == t)                                       \
    return launch_scores_cfg<e, t>(x, w_router, scores, T, d, E, pick, s);
  MOE_SCORES_CASE(4, 4) MOE_SCORES_CASE(4, 2) MOE_SCORES_CASE(4, 1)
  MOE_SCORES_CASE(2, 4) MOE_SCORES_CASE(2, 2) MOE_SCORES_CASE(2, 1)
  MOE_SCORES_CASE(1, 4) MOE_SCORES_CASE(1, 2) MOE_SCORES_CASE(1, 1)
#undef MOE_SCORES_CASE
  return hipErrorInvalidValue;
}

template <int EPL, int G>
__device__ __forceinline__ double select_token(const float* srow, const float* __restrict__ bias,
                                               int lane, int lane64, int E, int k,
                                               int32_t* __restrict__ idx_row,
                                               float* __restrict__ gate_row, float* margin_out,
                                               double* tok_sum_out);

// Fused routing for E <= 64, where one block holds all experts of its BT
// tokens: logits and scores (as router_scores_kernel), then selection,
// gates and margin from the scores kept in LDS (as select_kernel), and --
// with the balance statistic -- the block's partial sums for its sequence:
// P_e = sum over its tokens, in token order, of s[t,e] / sum_j s[t,j] (fp64)
// and the choice counts, at partial index blockIdx.x (a block lies inside one
// sequence, so seq_final_kernel adds S / BT partials per sequence).
template <int EPT, int TPT>
__global__ __launch_bounds__(kRouteThreads) void router_fused_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ w_router,
    const float* __restrict__ bias, int32_t* __restrict__ idx, float* __restrict__ gate,
    float* __restrict__ margin, double* __restrict__ seq_p, int32_t* __restrict__ seq_cnt,
    int64_t T, int d, int E, int k, int BE, int KC, int G) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  float acc[TPT][EPT];
  router_logits_tile<EPT, TPT>(x, w_router, T, d, E, BE, KC, lds_raw, acc);
  const int TPR = BE / EPT;
  const int tx = threadIdx.x % TPR, ty = threadIdx.x / TPR;
  const int BT = (kRouteThreads / TPR) * TPT;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * BT;
  float* sc = reinterpret_cast<float*>(lds_raw);                     // [BT][E]
  double* tsum = reinterpret_cast<double*>(lds_raw + ((BT * E * 4 + 15) & ~15));  // [BT]
  __syncthreads();  // every wave is done reading the staged x and W_r
#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tx * EPT + j;
      if (e < E) sc[(ty * TPT + i) * E + e] = sigmoid_score(acc[i][j]);
    }
  __syncthreads();
  auto select_all = [&](auto g_c) __attribute__((always_inline)) {
    constexpr int GG = decltype(g_c)::value;
    const int lane = threadIdx.x % GG, grp = threadIdx.x / GG, ngrp = kRouteThreads / GG;
    for (int tl = grp; tl < BT; tl += ngrp) {
      const int64_t t = t0 + tl;
      if (t >= T) continue;  // whole group skips together
      const double ts = select_token<1, GG>(sc + tl * E, bias, lane, threadIdx.x & 63, E, k,
                                            idx + t * k, gate + t * k,
                                            margin ? margin + t : nullptr, nullptr);
      if (lane == 0) tsum[tl] = ts;
    }
  };
  if (G == 16) select_all(std::integral_constant<int, 16>{});
  else if (G == 32) select_all(std::integral_constant<int, 32>{});
  else select_all(std::integral_constant<int, 64>{});
  if (!seq_p) return;
  // Partials: thread (e, lane l of L = 256 / E) sums s/sum(s) over the tokens
  // l, l + L, ... in order; the L lane sums are then added in lane order.
  // Counts: one LDS atomic per (token, slot) of this block.
  double* part = tsum + BT;                                  // [256]
  int* cnt = reinterpret_cast<int*>(part + kRouteThreads);   // [E]
  for (int e = threadIdx.x; e < E; e += kRouteThreads) cnt[e] = 0;
  __syncthreads();  // tsum, cnt and this block's idx rows are complete
  const int nt = (T - t0) < BT ? static_cast<int>(T - t0) : BT;
  for (int i = threadIdx.x; i < nt * k; i += kRouteThreads) {
    const int e = idx[t0 * k + i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  const int L = kRouteThreads / E;
  {
    const int e = threadIdx.x % E, l = threadIdx.x / E;
    double pe = 0.0;
    if (l < L)
      for (int tl = l; tl < nt; tl += L) {
        const double tot = tsum[tl];
        pe += (tot == 0.0) ? 1.0 / E : static_cast<double>(sc[tl * E + e]) / tot;
      }
    part[threadIdx.x] = pe;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteThreads) {
    double pe = 0.0;
    for (int l = 0; l < L; ++l) pe += part[l * E + e];
    seq_p[static_cast<int64_t>(blockIdx.x) * E + e] = pe;
    seq_cnt[static_cast<int64_t>(blockIdx.x) * E + e] = cnt[e];
  }
}

// ---------------------------------------------------------------------------
// Top-k selection and gates

__device__ __forceinline__ uint64_t pack_key(float key, int e) {
  const uint32_t lo = 0xFFFFFFFFu - static_cast<uint32_t>(e);  // lower index wins ties
  if (key != key) return static_cast<uint64_t>(lo);             // NaN: below every number
  if (key == 0.0f) key = 0.0f;                                   // -0 == +0
  return (static_cast<uint64_t>(orderable(key)) << 32) | lo;
}

// Group reductions of the selection run on DPP lane moves, which stay in the
// vector ALU (a shuffle through ds_bpermute is an LDS round trip).  A group
// is one 16-lane DPP row (G = 16), two rows (G = 32) or the wave (G = 64).
// Row step: quad_perm [1,0,3,2] and [2,3,0,1] (lane xor 1, 2), then row_ror
// by 12 and 8 (lane i reads lane i + 4, then i + 8, mod 16); after the four
// steps every lane of a row holds the row's reduction.  Rows are then joined
// with row_bcast:15 (lane 15 of a row into the next row) and row_bcast:31
// (lane 31 into rows 2 and 3), which leave the group's result in its last
// lane (31 or 63); readlane makes it wave-uniform.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, ROWS, 0xF, false));
}

// A candidate: 64-bit key (hi:lo as pack_key) and the unbiased score of its
// expert, which rides along so that the winners' scores need no lookup.
struct Cand {
  uint32_t hi, lo;
  float s;
};
__device__ __forceinline__ void cand_max(Cand& a, const Cand& b) {
  const bool take = b.hi > a.hi || (b.hi == a.hi && b.lo > a.lo);
  a.hi = take ? b.hi : a.hi;
  a.lo = take ? b.lo : a.lo;
  a.s = take ? b.s : a.s;
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ Cand dpp_cand(const Cand& v) {
  return Cand{dpp_u32<CTRL, ROWS>(v.hi), dpp_u32<CTRL, ROWS>(v.lo),
              __uint_as_float(dpp_u32<CTRL, ROWS>(__float_as_uint(v.s)))};
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = dpp_u32<CTRL, ROWS>(static_cast<uint32_t>(u));
  const uint32_t hi = dpp_u32<CTRL, ROWS>(static_cast<uint32_t>(u >> 32));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRor12 = 0x12C, kDppRor8 = 0x128;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

// Group maximum, the same in every lane of the group.
template <int G>
__device__ __forceinline__ Cand group_max(Cand v, int lane64) {
  cand_max(v, dpp_cand<kDppXor1>(v));
  cand_max(v, dpp_cand<kDppXor2>(v));
  cand_max(v, dpp_cand<kDppRor12>(v));
  cand_max(v, dpp_cand<kDppRor8>(v));
  if constexpr (G == 16) {
    return v;
  } else {
    cand_max(v, dpp_cand<kDppBcast15, 0xA>(v));  // rows 1, 3 take rows 0, 2
    if constexpr (G == 64) cand_max(v, dpp_cand<kDppBcast31, 0xC>(v));
    auto pick = [&](int src) __attribute__((always_inline)) {
      return Cand{static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v.hi), src)),
                  static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v.lo), src)),
                  __uint_as_float(static_cast<uint32_t>(
                      __builtin_amdgcn_readlane(static_cast<int>(__float_as_uint(v.s)), src)))};
    };
    if constexpr (G == 64) return pick(63);
    const Cand g0 = pick(31), g1 = pick(63);
    return lane64 < 32 ? g0 : g1;
  }
}

// Group sum (fp64) with the same lane moves; the tree differs from a
// sequential sum, so the value is compared within a tolerance, never
// bit-for-bit.
template <int G>
__device__ __forceinline__ double group_sum(double v, int lane64) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppRor12>(v);
  v += dpp_f64<kDppRor8>(v);
  if constexpr (G == 16) {
    return v;
  } else {
    // rows 1 and 3 add rows 0 and 2; with G = 64 row 3 then adds row 1
    const double b15 = dpp_f64<kDppBcast15, 0xA>(v);
    v = (lane64 & 16) ? v + b15 : v;
    if constexpr (G == 64) {
      const double b31 = dpp_f64<kDppBcast31, 0xC>(v);
      v = (lane64 >= 48) ? v + b31 : v;
    }
    auto pick = [&](int src) __attribute__((always_inline)) {
      const uint64_t u = __double_as_longlong(v);
      const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), src));
      const uint32_t hi =
          static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u >> 32), src));
      return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
    };
    if constexpr (G == 64) return pick(63);
    const double g0 = pick(31), g1 = pick(63);
    return lane64 < 32 ? g0 : g1;
  }
}

// Top-k of one token by a group of G lanes (lane = index in the group, lane64
// = index in the wave); lane i holds experts i, i + G, ... (EPL of them).
// k + 1 rounds of a group maximum over (orderable key << 32 | ~expert) pick
// the largest key with the lowest index on ties; the (k+1)-th gives the
// margin.  The gate sum adds the winners' unbiased scores in slot order.
template <int EPL, int G>
__device__ __forceinline__ double select_token(const float* srow, const float* __restrict__ bias,
                                               int lane, int lane64, int E, int k,
                                               int32_t* __restrict__ idx_row,
                                               float* __restrict__ gate_row, float* margin_out,
                                               double* tok_sum_out) {
  Cand pk[EPL];
  double ssum = 0.0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + i * G;
    pk[i] = Cand{0, 0, 0.0f};  // padding and taken entries
    if (e < E) {
      const float sv = srow[e];
      ssum += static_cast<double>(sv);
      const uint64_t key = pack_key(sv + bias[e], e);
      pk[i] = Cand{static_cast<uint32_t>(key >> 32), static_cast<uint32_t>(key), sv};
    }
  }

  int my_e = 0;
  float s_mine = 0.0f, sum = 0.0f, kth = 0.0f, next = 0.0f;
  const int rounds = (k < E) ? k + 1 : k;
  for (int r = 0; r < rounds; ++r) {
    Cand v = pk[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) cand_max(v, pk[i]);
    v = group_max<G>(v, lane64);
    const int e = static_cast<int>(0xFFFFFFFFu - v.lo);
    const float key = v.hi ? from_orderable(v.hi) : __uint_as_float(0x7FC00000u);
    if (r < k) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + i * G == e) pk[i] = Cand{0, 0, 0.0f};
      if (lane == r) {
        my_e = e;
        s_mine = v.s;
      }
      sum += v.s;
      if (r == k - 1) kth = key;
    } else {
      next = key;
    }
  }

  // Gates from the unbiased scores of the winners, normalised over them.
  if (lane < k) {
    idx_row[lane] = my_e;
    gate_row[lane] = (sum == 0.0f) ? 1.0f / static_cast<float>(k) : s_mine / sum;
  }
  if (lane == 0 && margin_out) *margin_out = (k < E) ? kth - next : __builtin_inff();
  ssum = group_sum<G>(ssum, lane64);
  if (lane == 0 && tok_sum_out) *tok_sum_out = ssum;
  return ssum;
}

template <int EPL, int G>
__global__ __launch_bounds__(256) void select_kernel(
    const float* __restrict__ scores, const float* __restrict__ bias, int32_t* __restrict__ idx,
    float* __restrict__ gate, float* __restrict__ margin, double* __restrict__ tok_sum,
    int64_t T, int E, int k) {
  const int lane64 = threadIdx.x & 63;
  const int lane = threadIdx.x % G;
  const int grp = threadIdx.x / G;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (256 / G) + grp;
  if (t >= T) return;  // whole group leaves together
  select_token<EPL, G>(scores + t * E, bias, lane, lane64, E, k, idx + t * k, gate + t * k,
                       margin ? margin + t : nullptr, tok_sum ? tok_sum + t : nullptr);
}

hipError_t launch_select(const float* scores, const float* bias, int32_t* idx, float* gate,
                         float* margin, double* tok_sum, int64_t T, int E, int k, hipStream_t s) {
  const int G = select_group(E);
  const int epl = (E + G - 1) / G;
  const int64_t nblk = (T + (256 / G) - 1) / (256 / G);
  const dim3 grid(static_cast<unsigned>(nblk)), block(256);
#define MOE_SEL_CASE(n, g)                                                                     \
  if (epl <= n && G == g) {                                                                    \
    hipLaunchKernelGGL((select_kernel<n, g>), grid, block, 0, s, scores, bias, idx, gate, margin, \
                       tok_sum, T, E, k);                                                       \
    return hipGetLastError();                                                                  \
  }
  MOE_SEL_CASE(1, 16) MOE_SEL_CASE(1, 32) MOE_SEL_CASE(1, 64) MOE_SEL_CASE(2, 64)
  MOE_SEL_CASE(4, 64) MOE_SEL_CASE(8, 64) MOE_SEL_CASE(16, 64)
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

constexpr int kSeqThreads = 1024;

// grid (nseq * nsplit): each block walks a slice of one sequence.  Thread
// (token lane tl, expert e) sums s[t,e]/tok_sum[t] in fp64 over the slice's
// tokens t = a + tl, a + tl + L, ...; the L lanes of an expert are then added
// in lane order (deterministic).  Choices are counted with LDS atomics.
// 1024 threads give several lanes per expert even for 256 experts, and the
// unrolled token loop keeps several loads in flight per lane.
__global__ __launch_bounds__(kSeqThreads) void seq_partial_kernel(
    const float* __restrict__ scores, const double* __restrict__ tok_sum,
    const int32_t* __restrict__ idx, double* __restrict__ seq_p, int32_t* __restrict__ seq_cnt,
    int E, int k, int S, int nsplit) {
  extern __shared__ int32_t cnt[];               // [E]
  __shared__ double part[kSeqThreads];
  const int q = blockIdx.x / nsplit, sp = blockIdx.x % nsplit;
  const int64_t a = static_cast<int64_t>(q) * S + static_cast<int64_t>(S) * sp / nsplit;
  const int64_t b = static_cast<int64_t>(q) * S + static_cast<int64_t>(S) * (sp + 1) / nsplit;
  for (int e = threadIdx.x; e < E; e += kSeqThreads) cnt[e] = 0;
  __syncthreads();
  for (int64_t i = a * k + threadIdx.x; i < b * k; i += kSeqThreads) {
    const int e = idx[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  const double inv_e = 1.0 / E;
  for (int e0 = 0; e0 < E; e0 += kSeqThreads) {
    const int ne = (E - e0) < kSeqThreads ? (E - e0) : kSeqThreads;
    const int L = kSeqThreads / ne;  // token lanes per expert
    const int e = e0 + threadIdx.x % ne, tl = threadIdx.x / ne;
    double p = 0.0;
    if (tl < L) {
#pragma unroll 4
      for (int64_t t = a + tl; t < b; t += L) {
        const double tot = tok_sum[t];
        p += (tot == 0.0) ? inv_e : static_cast<double>(scores[t * E + e]) / tot;
      }
    }
    part[threadIdx.x] = p;
    __syncthreads();
    if (threadIdx.x < ne) {
      double s2 = 0.0;
      for (int l = 0; l < L; ++l) s2 += part[l * ne + threadIdx.x];
      seq_p[static_cast<int64_t>(blockIdx.x) * E + e0 + threadIdx.x] = s2;
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < E; e += kSeqThreads) seq_cnt[static_cast<int64_t>(blockIdx.x) * E + e] = cnt[e];
}

// One block per sequence.  Experts are taken NT / ne lanes at a time
// (ne = experts of the pass): lane l of expert e adds the partials l, l + L,
// ... in order (unrolled, so several loads are in flight), the L lane sums
// are added in lane order, and the experts' terms f_e * P_e / S are then
// summed by a tree over the block.  NT = 256 serves the fused path's few
// experts and splits; long sequences of many experts take 1024.
template <int NT>
__global__ __launch_bounds__(NT) void seq_final_kernel(
    const double* __restrict__ seq_p, const int32_t* __restrict__ seq_cnt, float* __restrict__ out,
    float alpha, int E, int k, int S, int nsplit) {
  __shared__ double part[NT];
  __shared__ int64_t pcnt[NT];
  const int q = blockIdx.x;
  double acc = 0.0;
  for (int e0 = 0; e0 < E; e0 += NT) {
    const int ne = (E - e0) < NT ? (E - e0) : NT;
    const int L = NT / ne;
    const int e = e0 + threadIdx.x % ne, l = threadIdx.x / ne;
    double p = 0.0;
    int64_t c = 0;
    if (l < L) {
#pragma unroll 4
      for (int sp = l; sp < nsplit; sp += L) {
        const int64_t o = (static_cast<int64_t>(q) * nsplit + sp) * E + e;
        p += seq_p[o];
        c += seq_cnt[o];
      }
    }
    __syncthreads();  // the previous pass is done with part / pcnt
    part[threadIdx.x] = p;
    pcnt[threadIdx.x] = c;
    __syncthreads();
    if (threadIdx.x < ne) {
      double pe = 0.0;
      int64_t ce = 0;
      for (int j = 0; j < L; ++j) {
        pe += part[j * ne + threadIdx.x];
        ce += pcnt[j * ne + threadIdx.x];
      }
      const double f = static_cast<double>(E) / (static_cast<double>(k) * S) * static_cast<double>(ce);
      acc += f * (pe / S);
    }
  }
  __syncthreads();
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = NT / 2; w > 0; w >>= 1) {
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
  hipLaunchKernelGGL(seq_partial_kernel, dim3(static_cast<unsigned>(nseq * nsplit)),
                     dim3(kSeqThreads), sizeof(int32_t) * E, s, scores, tok_sum, idx, seq_p, seq_cnt,
                     E, k, S, nsplit);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(seq_final_kernel<kSeqThreads>, dim3(static_cast<unsigned>(nseq)),
                     dim3(kSeqThreads), 0, s, seq_p, seq_cnt, out, alpha, E, k, S, nsplit);
  return hipGetLastError();
}

int seq_partials_capacity(int64_t T, int S) {
  if (S <= 0) return 0;
  const int a = seq_splits(T, S);
  const int b = S / 16 > 0 ? S / 16 : 1;  // the fused path's blocks hold >= 16 tokens
  return a > b ? a : b;
}

hipError_t launch_route_fused(const uint16_t* x, const float* w_router, const float* bias,
                              int32_t* idx, float* gate, float* margin, double* seq_p,
                              int32_t* seq_cnt, float* seq_out, float alpha, int64_t T, int d,
                              int E, int k, int S, hipStream_t s, bool* done) {
  *done = false;
  if (E > 64) return hipSuccess;
  // two blocks per CU: a second wave per SIMD hides the first one's LDS latency
  const RouterCfg c = router_cfg(T, d, E, 2 * device_cus(), true);
  if (c.blocks <= 0 || c.BE < E) return hipSuccess;
  const int TPR = c.BE / c.EPT;
  const int BT = (kRouteThreads / TPR) * c.TPT;
  const bool stats = seq_out != nullptr && S > 0;
  if (stats && (S % BT != 0 || S / BT > seq_partials_capacity(T, S))) return hipSuccess;
  const int G = select_group(E);
  // scores [BT][E] f32, tok sums [BT] f64, lane partials [256] f64, counts [E] i32
  const size_t tail = static_cast<size_t>(((BT * E * 4 + 15) & ~15) + BT * 8 + kRouteThreads * 8 +
                                          E * 4);
  const size_t lds = c.lds > tail ? c.lds : tail;
#define MOE_FUSED_CASE(ep, tp)                                                                  \
  if (c.EPT == ep && c.TPT == tp) {                                                             \
    if (lds > 64 * 1024) {                                                                      \
      const hipError_t ae = hipFuncSetAttribute(                                                \
          reinterpret_cast<const void*>(&router_fused_kernel<ep, tp>),                          \
          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));                   \
      if (ae != hipSuccess) return ae;                                                          \
    }                                                                                           \
    hipLaunchKernelGGL((router_fused_kernel<ep, tp>), dim3(static_cast<unsigned>(c.blocks)),     \
                       dim3(kRouteThreads), lds, s, x, w_router, bias, idx, gate, margin,        \
                       stats ? seq_p : nullptr, seq_cnt, T, d, E, k, c.BE, c.KC, G);             \
  } else
  MOE_FUSED_CASE(4, 4) MOE_FUSED_CASE(4, 2) MOE_FUSED_CASE(4, 1)
  MOE_FUSED_CASE(2, 4) MOE_FUSED_CASE(2, 2) MOE_FUSED_CASE(2, 1)
  MOE_FUSED_CASE(1, 4) MOE_FUSED_CASE(1, 2) MOE_FUSED_CASE(1, 1)
  { return hipErrorInvalidValue; }
#undef MOE_FUSED_CASE
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (stats) {
    hipLaunchKernelGGL(seq_final_kernel<256>, dim3(static_cast<unsigned>(T / S)), dim3(256), 0, s, seq_p,
                       seq_cnt, seq_out, alpha, E, k, S, S / BT);
    err = hipGetLastError();
  }
  *done = err == hipSuccess;
  return err;
}

}  // namespace moe
