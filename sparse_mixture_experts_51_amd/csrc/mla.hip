// mla.hip -- MLA attention on gfx950: projections, cache writes, prefill and
// decode attention.
//
// Multi-head latent attention as "190行JAX复刻DeepSeek V3" (openai-hub.com),
// section 190行代码到底装进了什么, and "DeepSeek V3 viết lại bằng 190 dòng JAX
// thuần" (lehuy.net), section Những gì có trong 190 dòng code, describe it: a
// token caches a latent c (d_latent numbers) and one rotary key k_r (d_rope)
// shared by the heads; a head's key is [W_uk[h] c, k_r] and its value
// W_uv[h] c; the query's rotary part and k_r are turned by the position.
//
// Kernels:
//   mla_gemm_kernel<EPI>   C = A B^T on bf16 MFMA, 64 x 64 x 64 tiles (four
//       waves of 32 x 32), K-contiguous operands staged through LDS one step
//       ahead.  Three epilogues: the input projection (q with its rotary
//       part turned, the latent and the turned rotary key written into the
//       caches at the token's position), plain bf16 (the prefill's
//       decompressed keys and values) and bf16 with a residual (the output
//       projection).
//   mla_attn_prefill_mfma_kernel  one block per (128 queries, head,
//       sequence), keys and values in chunks of 64 through LDS, scores and
//       P V on 32x32x16 bf16 MFMAs with online softmax in fp32 (head sizes
//       with d_nope + d_rope a multiple of 16 and d_v 32 or 64);
//   mla_attn_prefill_kernel  the other head sizes: one block per (query tile
//       of 64, head, sequence); one wave per 16 query rows, a lane per key
//       for the scores, lanes split (value dim, key group) for P V.
//   mla_decode_partial_kernel / mla_decode_combine_kernel   reads only the
//       cache: one wave per (sequence, head, 64 cached positions) scores
//       them against the head's query taken into latent space (q_nope^T
//       W_uk[h]) and sums the weighted latents; the combine merges a head's
//       chunks (softmax rescaled to the largest maximum) and applies W_uv[h].  This is the
//       explicit decompression of the pages regrouped (associativity), so it
//       equals it up to rounding order while reading 144 numbers per cached
//       token instead of decompressing every key and value.
#include "common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace moe {

namespace {
constexpr int kTh = 256;
constexpr int kGM = 64, kGN = 64, kGK = 64;  // GEMM tile
constexpr int kGCh = kGK / 8;                 // 16-byte chunks per staged row

__device__ __forceinline__ int gsidx(int r, int c) {
  return r * kGCh + ((c ^ (r >> 1) ^ (r >> 3)) & (kGCh - 1));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// the pair (v0, v1) turned by position p, pair index m of d_rope numbers
__device__ __forceinline__ void rope_pair(float& v0, float& v1, int m, int d_rope, float p,
                                          float log2_base) {
  const float inv = exp2f(-2.0f * static_cast<float>(m) / static_cast<float>(d_rope) * log2_base);
  float s, c;
  sincosf(p * inv, &s, &c);
  const float a = v0, b = v1;
  v0 = a * c - b * s;
  v1 = a * s + b * c;
}
}  // namespace

template <int EPI>
__global__ __launch_bounds__(kTh) void mla_gemm_kernel(MlaGemmArgs a) {
  __shared__ u32x4 sa[2][kGM * kGCh];
  __shared__ u32x4 sb[2][kGN * kGCh];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.x * kGM, n0 = blockIdx.y * kGN;
  const int fr = lane & 31, fhalf = lane >> 5;

  // two 16-byte chunks per thread and operand: chunk q = tid + 256 p is row
  // q / 8, chunk q % 8 of the tile
  const uint16_t* ap[2];
  const uint16_t* bp[2];
  bool aok[2], bok[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = (tid + kTh * p) >> 3;
    const int t = m0 + row;
    aok[p] = t < a.M;
    const int arow = aok[p] ? (t / a.a_grp) * a.a_grp_stride + t % a.a_grp : 0;
    ap[p] = a.a + static_cast<int64_t>(arow) * a.lda;
    const int n = n0 + row;
    bok[p] = n < a.N;
    const int nn = bok[p] ? n : 0;
    bp[p] = nn < a.n1 ? a.b0 + static_cast<int64_t>(nn) * a.K
                      : (nn < a.n2 ? a.b1 + static_cast<int64_t>(nn - a.n1) * a.K
                                   : a.b2 + static_cast<int64_t>(nn - a.n2) * a.K);
  }
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
  u32x4 va[2], vb[2];
  auto load = [&](int kt) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int ch = (tid + kTh * p) & 7;
      const int k = kt * kGK + 8 * ch;
      va[p] = aok[p] ? *reinterpret_cast<const u32x4*>(ap[p] + k) : zero4;
      vb[p] = bok[p] ? *reinterpret_cast<const u32x4*>(bp[p] + k) : zero4;
    }
  };
  auto store = [&](int st) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int q = tid + kTh * p;
      sa[st][gsidx(q >> 3, q & 7)] = va[p];
      sb[st][gsidx(q >> 3, q & 7)] = vb[p];
    }
  };
  f32x16 acc = f32x16{};
  const int nk = a.K / kGK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      const bf16x8 af = __builtin_bit_cast(bf16x8, sa[st][gsidx(32 * wm + fr, 2 * ks + fhalf)]);
      const bf16x8 bf = __builtin_bit_cast(bf16x8, sb[st][gsidx(32 * wn + fr, 2 * ks + fhalf)]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf, af, acc, 0, 0, 0);
    }
    if (kt + 1 < nk) store(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue: this lane holds row m, columns n .. n+3 per q
  const int m = m0 + 32 * wm + fr;
  if (m >= a.M) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int n = n0 + 32 * wn + 8 * q + 4 * fhalf;
    if (n >= a.N) continue;
    float v[4] = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    if constexpr (EPI == kMlaEpiProj) {
      // the token's sequence and position
      int b, p;
      if (a.seq > 0) {
        b = m / a.seq;
        p = m % a.seq;
      } else {
        b = m;
        p = a.pos[m];
      }
      const bool in_cache = p >= 0 && p < a.max_len;
      if (n < a.n1) {  // query of head n / qw
        const int j = n % a.qw;
        if (j >= a.dn) {
          const int mr = (j - a.dn) >> 1;
          rope_pair(v[0], v[1], mr, a.dr, static_cast<float>(p), a.log2_base);
          rope_pair(v[2], v[3], mr + 1, a.dr, static_cast<float>(p), a.log2_base);
        }
        *reinterpret_cast<uint2*>(a.q + static_cast<int64_t>(m) * a.n1 + n) =
            make_uint2(bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3]));
      } else if (!in_cache) {
        continue;
      } else if (n < a.n2) {  // latent
        *reinterpret_cast<uint2*>(a.ckv + (static_cast<int64_t>(b) * a.max_len + p) * a.dc + (n - a.n1)) =
            make_uint2(bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3]));
      } else {  // rotary key
        const int j = n - a.n2;
        rope_pair(v[0], v[1], j >> 1, a.dr, static_cast<float>(p), a.log2_base);
        rope_pair(v[2], v[3], (j >> 1) + 1, a.dr, static_cast<float>(p), a.log2_base);
        *reinterpret_cast<uint2*>(a.ckr + (static_cast<int64_t>(b) * a.max_len + p) * a.dr + j) =
            make_uint2(bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3]));
      }
    } else {
      if constexpr (EPI == kMlaEpiRes) {
        if (a.res) {
          const uint2 r = *reinterpret_cast<const uint2*>(a.res + static_cast<int64_t>(m) * a.ldc + n);
          v[0] += bf16_to_f32(static_cast<uint16_t>(r.x));
          v[1] += bf16_to_f32(static_cast<uint16_t>(r.x >> 16));
          v[2] += bf16_to_f32(static_cast<uint16_t>(r.y));
          v[3] += bf16_to_f32(static_cast<uint16_t>(r.y >> 16));
        }
      }
      *reinterpret_cast<uint2*>(a.c + static_cast<int64_t>(m) * a.ldc + n) =
          make_uint2(bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3]));
    }
  }
}

namespace {
constexpr int kQT = 64;           // query rows per prefill block
constexpr int kRowsPerWave = kQT / 4;
constexpr int kMaxQwCh = 16;      // d_nope + d_rope <= 128
constexpr int kKRow = 8 * kMaxQwCh + 8;  // staged key row (bf16), padded
constexpr int kVRow = 64 + 8;            // staged value row (bf16), padded

__device__ __forceinline__ float dot8(const u32x4& x, const u32x4& y) {
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    s = fmaf(__uint_as_float(x[w] << 16), __uint_as_float(y[w] << 16), s);
    s = fmaf(__uint_as_float(x[w] & 0xFFFF0000u), __uint_as_float(y[w] & 0xFFFF0000u), s);
  }
  return s;
}
}  // namespace

__global__ __launch_bounds__(kTh) void mla_attn_prefill_kernel(MlaAttnArgs a) {
  __shared__ uint16_t qs[kQT * kKRow];
  __shared__ uint16_t ks[64 * kKRow];
  __shared__ uint16_t vs[64 * kVRow];
  __shared__ float ps[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
  const int i0 = blockIdx.x * kQT, h = blockIdx.y, b = blockIdx.z;
  const int S = a.seq, qw = a.dn + a.dr, qwc = qw / 8, dv = a.dv;
  const int G = 64 / dv, j = lane % dv, grp = lane / dv;
  const int64_t qld = static_cast<int64_t>(a.nh) * qw;
  const int64_t kvld = static_cast<int64_t>(a.nh) * (a.dn + dv);
  const int64_t tok0 = static_cast<int64_t>(b) * S;

  // queries of the tile
  for (int idx = tid; idx < kQT * qwc; idx += kTh) {
    const int r = idx / qwc, c = idx % qwc;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (i0 + r < S) v = *reinterpret_cast<const u32x4*>(a.q + (tok0 + i0 + r) * qld + h * qw + 8 * c);
    *reinterpret_cast<u32x4*>(qs + r * kKRow + 8 * c) = v;
  }
  float mrow[kRowsPerWave], lrow[kRowsPerWave], acc[kRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    mrow[r] = -INFINITY;
    lrow[r] = 0.0f;
    acc[r] = 0.0f;
  }
  const int last = min(i0 + kQT, S) - 1;  // last query of the tile
  for (int c0 = 0; c0 <= last; c0 += 64) {
    __syncthreads();  // the previous chunk is no longer read
    // keys [k_nope_h, k_r] and values v_h of positions c0 .. c0+63
    const int kch = a.dn / 8, rch = a.dr / 8, vch = dv / 8;
    for (int idx = tid; idx < 64 * (qwc + vch); idx += kTh) {
      const int r = idx / (qwc + vch), c = idx % (qwc + vch);
      const int s = c0 + r;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (s < S) {
        if (c < kch)
          v = *reinterpret_cast<const u32x4*>(a.kvx + (tok0 + s) * kvld + h * a.dn + 8 * c);
        else if (c < kch + rch)
          v = *reinterpret_cast<const u32x4*>(a.ckr + (static_cast<int64_t>(b) * a.max_len + s) * a.dr +
                                              8 * (c - kch));
        else
          v = *reinterpret_cast<const u32x4*>(a.kvx + (tok0 + s) * kvld + a.nh * a.dn + h * dv +
                                              8 * (c - qwc));
      }
      if (c < qwc) *reinterpret_cast<u32x4*>(ks + r * kKRow + 8 * c) = v;
      else *reinterpret_cast<u32x4*>(vs + r * kVRow + 8 * (c - qwc)) = v;
    }
    __syncthreads();
    // this lane's key row
    u32x4 kr[kMaxQwCh];
#pragma unroll
    for (int c = 0; c < kMaxQwCh; ++c)
      if (c < qwc) kr[c] = *reinterpret_cast<const u32x4*>(ks + lane * kKRow + 8 * c);
    const int s = c0 + lane;
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const int rr = wave * kRowsPerWave + r;
      const int i = i0 + rr;
      if (i > last || i < c0) continue;  // uniform per wave
      float sc = 0.0f;
#pragma unroll
      for (int c = 0; c < kMaxQwCh; ++c)
        if (c < qwc) sc += dot8(*reinterpret_cast<const u32x4*>(qs + rr * kKRow + 8 * c), kr[c]);
      const bool ok = s <= i;
      sc = ok ? sc * a.scale : -INFINITY;
      const float mnew = fmaxf(mrow[r], wave_max(sc));
      const float corr = __expf(mrow[r] - mnew);
      const float p = ok ? __expf(sc - mnew) : 0.0f;
      lrow[r] = lrow[r] * corr + wave_sum(p);
      mrow[r] = mnew;
      ps[wave][lane] = p;  // read back by the other lanes of this wave only
      __builtin_amdgcn_wave_barrier();
      float t = 0.0f;
      for (int k2 = grp; k2 < 64; k2 += G) t = fmaf(ps[wave][k2], bf16_to_f32(vs[k2 * kVRow + j]), t);
      __builtin_amdgcn_wave_barrier();
      acc[r] = acc[r] * corr + t;
    }
  }
  // combine the key groups and write o
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int rr = wave * kRowsPerWave + r;
    const int i = i0 + rr;
    float t = acc[r];
    for (int o = dv; o < 64; o <<= 1) t += __shfl_xor(t, o, 64);
    if (i <= last && grp == 0)
      a.o[(tok0 + i) * static_cast<int64_t>(a.nh) * dv + h * dv + j] = f32_to_bf16(t / lrow[r]);
  }
}

namespace {
constexpr int kFQ = 128;  // queries per block of the matrix-core prefill (32 per wave)
constexpr int kFK = 64;   // keys per staged chunk
constexpr int kFKRow = 128 + 8;  // staged key row (bf16), padded: 16 rows hit distinct banks
constexpr int kFVRow = kFK + 8;  // staged V^T row (bf16)
}  // namespace

// Prefill attention on the matrix cores (d_nope + d_rope a multiple of 16,
// d_v = 32 DVT): per wave 32 queries; per 32-key slice, S = K Q^T on
// 32x32x16 MFMAs (a lane then holds 16 scores of one query), online softmax
// in fp32 across the lane pair that shares the query, and O += V^T P^T where
// the scores' registers are the P operand as they stand: V^T is read with
// the keys in the order the score tile holds them (keys 4g..4g+3 and
// 8+4g..8+4g+3 of each 16 for lane half g).
template <int DVT>
__global__ __launch_bounds__(kTh) void mla_attn_prefill_mfma_kernel(MlaAttnArgs a) {
  __shared__ uint16_t ks[kFK * kFKRow];
  __shared__ uint16_t vt[32 * DVT * kFVRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
  const int qb0 = blockIdx.x * kFQ, h = blockIdx.y, b = blockIdx.z;
  const int S = a.seq, dn = a.dn, qw = a.dn + a.dr, kst = qw / 16, dv = 32 * DVT;
  const int fr = lane & 31, fhalf = lane >> 5;
  const int q0 = qb0 + 32 * wave;  // this wave's first query
  const int64_t qld = static_cast<int64_t>(a.nh) * qw;
  const int64_t kvld = static_cast<int64_t>(a.nh) * (dn + dv);
  const int64_t tok0 = static_cast<int64_t>(b) * S;
  const int my_q = q0 + fr;

  bf16x8 qf[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (t < kst && my_q < S)
      v = *reinterpret_cast<const u32x4*>(a.q + (tok0 + my_q) * qld + h * qw + 16 * t + 8 * fhalf);
    qf[t] = __builtin_bit_cast(bf16x8, v);
  }
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 oacc[DVT];
#pragma unroll
  for (int t = 0; t < DVT; ++t) oacc[t] = f32x16{};

  const int last = min(qb0 + kFQ, S) - 1;
  const int kch = dn / 8, qwc = qw / 8, vch = dv / 8;
  for (int c0 = 0; c0 <= last; c0 += kFK) {
    __syncthreads();
    for (int idx = tid; idx < kFK * qwc; idx += kTh) {
      const int r = idx / qwc, c = idx % qwc, key = c0 + r;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (key < S)
        v = c < kch ? *reinterpret_cast<const u32x4*>(a.kvx + (tok0 + key) * kvld + h * dn + 8 * c)
                    : *reinterpret_cast<const u32x4*>(a.ckr + (static_cast<int64_t>(b) * a.max_len + key) * a.dr +
                                                      8 * (c - kch));
      *reinterpret_cast<u32x4*>(ks + r * kFKRow + 8 * c) = v;
    }
    for (int idx = tid; idx < kFK * vch; idx += kTh) {
      const int r = idx / vch, c = idx % vch, key = c0 + r;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (key < S) v = *reinterpret_cast<const u32x4*>(a.kvx + (tok0 + key) * kvld + a.nh * dn + h * dv + 8 * c);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vt[(8 * c + 2 * w) * kFVRow + r] = static_cast<uint16_t>(v[w]);
        vt[(8 * c + 2 * w + 1) * kFVRow + r] = static_cast<uint16_t>(v[w] >> 16);
      }
    }
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < kFK / 32; ++sub) {
      const int c = c0 + 32 * sub;
      if (c > q0 || q0 >= S) continue;  // uniform: keys past the wave's queries, or no queries
      f32x16 sc = f32x16{};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t >= kst) break;
        const bf16x8 kf = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(ks + (32 * sub + fr) * kFKRow + 16 * t + 8 * fhalf));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], sc, 0, 0, 0);
      }
      // this lane: query my_q, keys c + 8q + 4 fhalf + e
      float mx = -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = c + 8 * q + 4 * fhalf + e;
          const float v = key <= my_q ? sc[4 * q + e] * a.scale : -INFINITY;
          sc[4 * q + e] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float corr = __expf(m_run - m_new);
      float ps = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __expf(sc[i] - m_new);
        sc[i] = p;
        ps += p;
      }
      ps += __shfl_xor(ps, 32, 64);
      l_run = l_run * corr + ps;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < DVT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[t][i] *= corr;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const u32x4 pw = u32x4{bf16x2_bits(sc[8 * k2], sc[8 * k2 + 1]), bf16x2_bits(sc[8 * k2 + 2], sc[8 * k2 + 3]),
                               bf16x2_bits(sc[8 * k2 + 4], sc[8 * k2 + 5]), bf16x2_bits(sc[8 * k2 + 6], sc[8 * k2 + 7])};
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
        const int kb = 32 * sub + 16 * k2 + 4 * fhalf;
#pragma unroll
        for (int t = 0; t < DVT; ++t) {
          const uint16_t* row = vt + (32 * t + fr) * kFVRow;
          const uint2 lo = *reinterpret_cast<const uint2*>(row + kb);
          const uint2 hi = *reinterpret_cast<const uint2*>(row + kb + 8);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[t], 0, 0, 0);
        }
      }
    }
  }
  if (my_q < S) {
    const float inv = 1.0f / l_run;
    uint16_t* orow = a.o + (tok0 + my_q) * static_cast<int64_t>(a.nh) * dv + h * dv;
#pragma unroll
    for (int t = 0; t < DVT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x16& v = oacc[t];
        *reinterpret_cast<uint2*>(orow + 32 * t + 8 * q + 4 * fhalf) =
            make_uint2(bf16x2_bits(v[4 * q] * inv, v[4 * q + 1] * inv),
                       bf16x2_bits(v[4 * q + 2] * inv, v[4 * q + 3] * inv));
      }
  }
}

namespace {
constexpr int kMaxLat = 256;  // d_latent
}  // namespace

// Decode, split over the cache: one wave per (sequence, head, chunk of 64
// cached positions) scores its chunk against the head's query taken into
// latent space (W_uk[h]^T q_nope; a lane per cached row, the rows staged in
// dynamic LDS for the weighted sum), and writes the chunk's max score, sum of weights and weighted latent sum;
// mla_decode_combine_kernel merges a head's chunks and applies W_uv[h].
// Block b runs on XCD b % 8; the heads and chunks of a sequence share its XCD
// (and the cached rows in that L2).
__global__ __launch_bounds__(64) void mla_decode_partial_kernel(MlaAttnArgs a, int batch, int nchunk) {
  extern __shared__ uint16_t rows[];  // [64][d_latent + d_rope + 8]
  __shared__ float qlat[kMaxLat];
  __shared__ float qr[128];  // the head's query (content, then rotary part)
  __shared__ float ps[64];
  const int lane = threadIdx.x;
  const int nh = a.nh, dc = a.dc, dn = a.dn, dr = a.dr, qw = dn + dr;
  const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  const int per_seq = nh * nchunk;
  const int b = xcd + kXcds * (j / per_seq), rem = j % per_seq;
  const int ci = rem / nh, h = rem % nh;
  if (b >= batch) return;
  float* part = a.part + ((static_cast<int64_t>(b) * nh + h) * nchunk + ci) * (dc + 2);
  const int p = a.pos[b], c0 = 64 * ci;
  if (p < 0 || p >= a.max_len || c0 > p) {
    if (lane == 0) {
      part[0] = -INFINITY;
      part[1] = 0.0f;
    }
    return;
  }
  const int rs = dc + dr + 8, dcc = dc / 8, rc = dcc + dr / 8;
  // the chunk's cached rows into LDS, coalesced: a load instruction covers
  // 64 / dcc whole latent rows (dcc, a power of two, 16-byte chunks per row)
  const int s = c0 + lane;
  const bool ok = s <= p;
  const int64_t cbase = static_cast<int64_t>(b) * a.max_len;
  const int lg = __builtin_ctz(dcc);
  for (int idx = lane; idx < 64 * dcc; idx += 64) {
    const int r = idx >> lg, c = idx & (dcc - 1);
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (c0 + r <= p) v = *reinterpret_cast<const u32x4*>(a.ckv + (cbase + c0 + r) * dc + 8 * c);
    *reinterpret_cast<u32x4*>(rows + r * rs + 8 * c) = v;
  }
  for (int idx = lane; idx < 64 * (rc - dcc); idx += 64) {
    const int r = idx / (rc - dcc), c = idx % (rc - dcc);
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (c0 + r <= p) v = *reinterpret_cast<const u32x4*>(a.ckr + (cbase + c0 + r) * dr + 8 * c);
    *reinterpret_cast<u32x4*>(rows + r * rs + dc + 8 * c) = v;
  }
  // the head's query, then W_uk[h]^T q_nope: lane (row group g, 8-column
  // chunk c8) sums rows g, g + groups, ... with 16-byte loads; the groups are
  // added across lanes
  const uint16_t* qb = a.q + (static_cast<int64_t>(b) * nh + h) * qw;
  for (int jj = lane; jj < qw; jj += 64) qr[jj] = bf16_to_f32(qb[jj]);
  __syncthreads();
  {
    const int nc8 = dc / 8, groups = 64 / nc8, g = lane / nc8, c8 = lane % nc8;
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    const uint16_t* wk = a.w_uk + static_cast<int64_t>(h) * dn * dc + 8 * c8;
#pragma unroll 4
    for (int jj = g; jj < dn; jj += groups) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(wk + static_cast<int64_t>(jj) * dc);
      const float qj = qr[jj];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(qj, __uint_as_float(w[e] << 16), acc[2 * e]);
        acc[2 * e + 1] = fmaf(qj, __uint_as_float(w[e] & 0xFFFF0000u), acc[2 * e + 1]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      for (int o = nc8; o < 64; o <<= 1) acc[e] += __shfl_xor(acc[e], o, 64);
    if (g == 0)
#pragma unroll
      for (int e = 0; e < 8; ++e) qlat[8 * c8 + e] = acc[e];
  }
  __syncthreads();
  float sc = 0.0f;
#pragma unroll 2
  for (int c = 0; c < rc; ++c) {
    const u32x4 kv = *reinterpret_cast<const u32x4*>(rows + lane * rs + 8 * c);
    const float* q8 = c < dcc ? qlat + 8 * c : qr + dn + 8 * (c - dcc);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sc = fmaf(q8[2 * w], __uint_as_float(kv[w] << 16), sc);
      sc = fmaf(q8[2 * w + 1], __uint_as_float(kv[w] & 0xFFFF0000u), sc);
    }
  }
  sc = ok ? sc * a.scale : -INFINITY;
  const float m = wave_max(sc);
  const float pr = ok ? __expf(sc - m) : 0.0f;
  const float l = wave_sum(pr);
  ps[lane] = pr;
  __syncthreads();
  // weighted latent sum: lane (8-column chunk c8, key group kg) reads 16 bytes
  // of every kg-th row; the key groups are added across lanes
  {
    const int nc8 = dc / 8, kgroups = 64 / nc8, kg = lane / nc8, c8 = lane % nc8;
    float t[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
    for (int k2 = kg; k2 < 64; k2 += kgroups) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(rows + k2 * rs + 8 * c8);
      const float pk = ps[k2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        t[2 * e] = fmaf(pk, __uint_as_float(v[e] << 16), t[2 * e]);
        t[2 * e + 1] = fmaf(pk, __uint_as_float(v[e] & 0xFFFF0000u), t[2 * e + 1]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      for (int o = nc8; o < 64; o <<= 1) t[e] += __shfl_xor(t[e], o, 64);
    if (kg == 0)
#pragma unroll
      for (int e = 0; e < 8; ++e) part[2 + 8 * c8 + e] = t[e];
  }
  if (lane == 0) {
    part[0] = m;
    part[1] = l;
  }
}

// The heads' queries in latent space, once per decode step: one wave per
// (sequence, head) writes bf16(W_uk[h]^T q_nope) to qlat [batch, nh, dc]
// (lane: row group g, 8-column chunk c8 with 16-byte loads; groups added
// across lanes).
__global__ __launch_bounds__(64) void mla_decode_qlat_kernel(MlaAttnArgs a, int batch) {
  __shared__ float qn[128];
  const int lane = threadIdx.x;
  const int nh = a.nh, dc = a.dc, dn = a.dn, qw = dn + a.dr;
  const int b = blockIdx.x / nh, h = blockIdx.x % nh;
  if (b >= batch) return;
  const uint16_t* qb = a.q + (static_cast<int64_t>(b) * nh + h) * qw;
  for (int jj = lane; jj < dn; jj += 64) qn[jj] = bf16_to_f32(qb[jj]);
  __syncthreads();
  const int nc8 = dc / 8, groups = 64 / nc8, g = lane / nc8, c8 = lane % nc8;
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  const uint16_t* wk = a.w_uk + static_cast<int64_t>(h) * dn * dc + 8 * c8;
#pragma unroll 4
  for (int jj = g; jj < dn; jj += groups) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(wk + static_cast<int64_t>(jj) * dc);
    const float qj = qn[jj];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = fmaf(qj, __uint_as_float(w[e] << 16), acc[2 * e]);
      acc[2 * e + 1] = fmaf(qj, __uint_as_float(w[e] & 0xFFFF0000u), acc[2 * e + 1]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
    for (int o = nc8; o < 64; o <<= 1) acc[e] += __shfl_xor(acc[e], o, 64);
  if (g == 0)
    *reinterpret_cast<u32x4*>(a.qlat + (static_cast<int64_t>(b) * nh + h) * dc + 8 * c8) =
        u32x4{bf16x2_bits(acc[0], acc[1]), bf16x2_bits(acc[2], acc[3]), bf16x2_bits(acc[4], acc[5]),
              bf16x2_bits(acc[6], acc[7])};
}

// Decode on the matrix cores: one wave per (sequence, run of cps chunks of
// 64 cached positions) takes all heads at once (the 32 rows of the MFMA
// tile, heads past nh zero).  Per chunk: scores S = K Q^T over the latent and
// rotary key (K rows read straight from the cache; positions past the token
// zeroed, so stale cache contents never reach P V), and O^T += V^T P^T with
// V^T the chunk's latents staged transposed in LDS and P taken from the
// score registers as they stand (keys 4g..4g+3 and 8+4g..8+4g+3 of each 16
// for lane half g); the softmax statistics run across the block's chunks,
// the accumulated sums rescaled when the maximum grows.  Writes the run's
// per-head max, sum of weights and weighted latent sum into partial slot
// `split` (a slot per chunk in mla_decode_partial_kernel).
template <int DC, int DR>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void mla_decode_mfma_kernel(MlaAttnArgs a, int batch, int nchunk, int cps) {
  constexpr int KST = (DC + DR + 15) / 16;  // k-steps of the scores
  constexpr int LST = DC / 16;              // of them, on the latent
  static_assert(DR == 16 && DC % 16 == 0, "one rotary step of 16 after the latent steps");
  constexpr int NCT = DC / 32;              // latent tiles of P V
  constexpr int VROW = 64 + 8;              // staged V^T row (bf16)
  __shared__ uint16_t vt[DC * VROW];
  const int lane = threadIdx.x, fr = lane & 31, fhalf = lane >> 5;
  const int nh = a.nh, qw = a.dn + DR;
  const int nsplit = (nchunk + cps - 1) / cps;
  const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  const int b = xcd + kXcds * (j / nsplit), split = j % nsplit;
  if (b >= batch) return;
  const int p = a.pos[b], cfirst = split * cps;
  if (p < 0 || p >= a.max_len || 64 * cfirst > p) return;  // the combine reads only runs with positions
  // the heads' fragments: head fr, k = 16 t + 8 fhalf .. +7 (latent, then rotary part)
  bf16x8 qf[KST];
  const bool hv = fr < nh;
  const int64_t hrow = static_cast<int64_t>(b) * nh + (hv ? fr : 0);
#pragma unroll
  for (int t = 0; t < KST; ++t) {
    const int k = 16 * t + 8 * fhalf;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (hv) {
      if (k < DC) v = *reinterpret_cast<const u32x4*>(a.qlat + hrow * DC + k);
      else if (k < DC + DR) v = *reinterpret_cast<const u32x4*>(a.q + hrow * qw + a.dn + (k - DC));
    }
    qf[t] = __builtin_bit_cast(bf16x8, v);
  }
  const int64_t cbase = static_cast<int64_t>(b) * a.max_len;
  // Cache rows by buffer loads, a chunk's all issued before the first is
  // used: the descriptors cover the rows 0..p of this sequence, so a key row
  // past p reads zeros (its score is masked below), and whether a piece is
  // latent or rotary is fixed per step.  (With a bounds branch per load the
  // compiler waited for each load before the next.)
  const __amdgpu_buffer_rsrc_t rkv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.ckv + cbase * DC), static_cast<short>(0), (p + 1) * DC * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rkr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.ckr + cbase * DR), static_cast<short>(0), (p + 1) * DR * 2, 0x00020000);
  float mrun = -INFINITY, lrun = 0.0f;  // head fr's running max and sum of weights
  f32x16 oacc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) oacc[ct] = f32x16{};
  const int cend = cfirst + cps < nchunk ? cfirst + cps : nchunk;
  for (int ci = cfirst; ci < cend && 64 * ci <= p; ++ci) {
    const int c0 = 64 * ci;
    if (ci > cfirst) __syncthreads();  // the previous chunk's P V has read V^T
    u32x4 rows[2][KST];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int s = c0 + 32 * half + fr;  // this lane's key row
#pragma unroll
      for (int t = 0; t < KST; ++t) {
        const int k = 16 * t + 8 * fhalf;
        if (t < LST)
          rows[half][t] = __builtin_amdgcn_raw_buffer_load_b128(rkv, (s * DC + k) * 2, 0, 0);
        else
          rows[half][t] = __builtin_amdgcn_raw_buffer_load_b128(rkr, (s * DR + (k - DC)) * 2, 0, 0);
      }
    }
    f32x16 sc[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      sc[half] = f32x16{};
#pragma unroll
      for (int t = 0; t < KST; ++t) {
        const int k = 16 * t + 8 * fhalf;
        const u32x4 v = rows[half][t];
        if (t < LST) {
          // V^T: latent column k + i, key 32 half + fr
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            vt[(k + 2 * w) * VROW + 32 * half + fr] = static_cast<uint16_t>(v[w]);
            vt[(k + 2 * w + 1) * VROW + 32 * half + fr] = static_cast<uint16_t>(v[w] >> 16);
          }
        }
        sc[half] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v), qf[t], sc[half], 0, 0, 0);
      }
    }
    // softmax statistics of head fr (lanes fr and fr + 32 share it): the
    // chunk's maximum joins the running one, and what was summed under the
    // old maximum is rescaled to the new
    float mx = -INFINITY;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = c0 + 32 * half + 8 * (i >> 2) + 4 * fhalf + (i & 3);
        const float v = key <= p ? sc[half][i] * a.scale : -INFINITY;
        sc[half][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(mrun, mx);  // finite: the chunk holds key c0 <= p
    const float alpha = __expf(mrun - mnew);  // 0 for the first chunk
    float ls = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __expf(sc[half][i] - mnew);
        sc[half][i] = e;
        ls += e;
      }
    ls += __shfl_xor(ls, 32, 64);
    lrun = lrun * alpha + ls;
    mrun = mnew;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[ct][i] *= alpha;
    __syncthreads();  // V^T staged
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f32x16& pv = sc[ks >> 1];
      const int q0 = 2 * (ks & 1);
      const bf16x8 pf = __builtin_bit_cast(
          bf16x8, u32x4{bf16x2_bits(pv[4 * q0], pv[4 * q0 + 1]), bf16x2_bits(pv[4 * q0 + 2], pv[4 * q0 + 3]),
                        bf16x2_bits(pv[4 * q0 + 4], pv[4 * q0 + 5]), bf16x2_bits(pv[4 * q0 + 6], pv[4 * q0 + 7])});
      const int kb = 16 * ks + 4 * fhalf;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const uint16_t* row = vt + (32 * ct + fr) * VROW;
        const uint2 lo = *reinterpret_cast<const uint2*>(row + kb);
        const uint2 hi = *reinterpret_cast<const uint2*>(row + kb + 8);
        oacc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y}), pf, oacc[ct], 0, 0, 0);
      }
    }
  }
  // this lane: head fr, latent columns 32 ct + 8 q + 4 fhalf + e
  if (hv) {
    float* part = a.part + ((static_cast<int64_t>(b) * nh + fr) * nchunk + split) * (DC + 2);
    if (fhalf == 0) {
      part[0] = mrun;
      part[1] = lrun;
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x16& o = oacc[ct];
        float* dst = part + 2 + 32 * ct + 8 * q + 4 * fhalf;
        dst[0] = o[4 * q];
        dst[1] = o[4 * q + 1];
        dst[2] = o[4 * q + 2];
        dst[3] = o[4 * q + 3];
      }
  }
}

// Merges a head's partial slots (each covers cps chunks of 64 positions;
// rescaled to the largest maximum) and applies W_uv[h] to the attended
// latent: one wave per (sequence, head).  Loads are issued in batches (slot
// statistics, then the slots' latent sums, then eight W_uv row pieces at a
// time) so that each phase costs one memory trip.
__global__ __launch_bounds__(64) void mla_decode_combine_kernel(MlaAttnArgs a, int batch, int nchunk, int cps) {
  __shared__ float olat[kMaxLat];
  __shared__ float wts[64];
  const int lane = threadIdx.x;
  const int nh = a.nh, dc = a.dc, dv = a.dv;
  const int b = blockIdx.x / nh, h = blockIdx.x % nh;
  if (b >= batch) return;
  const int64_t orow = (static_cast<int64_t>(b) * nh + h) * dv;
  const int p = a.pos[b];
  if (p < 0 || p >= a.max_len) {
    for (int jj = lane; jj < dv; jj += 64) a.o[orow + jj] = 0;
    return;
  }
  const int nc = p / 64 / cps + 1;  // slots with cached positions
  const float* part = a.part + (static_cast<int64_t>(b) * nh + h) * nchunk * (dc + 2);
  // chunk statistics: chunk i in lane i (and i + 64, ...)
  float M = -INFINITY;
  for (int i = lane; i < nc; i += 64) M = fmaxf(M, part[static_cast<int64_t>(i) * (dc + 2)]);
  M = wave_max(M);
  float L = 0.0f;
  for (int i0 = 0; i0 < nc; i0 += 64) {
    const int i = i0 + lane;
    float w = 0.0f;
    if (i < nc) {
      w = __expf(part[static_cast<int64_t>(i) * (dc + 2)] - M);
      L += w * part[static_cast<int64_t>(i) * (dc + 2) + 1];
    }
    __syncthreads();
    wts[lane] = w;
    __syncthreads();
    for (int c = lane; c < dc; c += 64) {
      float t = i0 > 0 ? olat[c] : 0.0f;
#pragma unroll 4
      for (int k = 0; k < min(64, nc - i0); ++k)
        t = fmaf(wts[k], part[static_cast<int64_t>(i0 + k) * (dc + 2) + 2 + c], t);
      olat[c] = t;
    }
  }
  L = wave_sum(L);
  __syncthreads();
  // W_uv[h] olat / L: lane (8-column chunk c8, row group g), rows g, g +
  // groups, ...; eight rows' 16-byte pieces loaded before they are used
  const int nc8 = dc / 8, groups = 64 / nc8, g = lane / nc8, c8 = lane % nc8;
  const uint16_t* wv = a.w_uv + static_cast<int64_t>(h) * dv * dc + 8 * c8;
  float ol[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ol[e] = olat[8 * c8 + e] / L;
  for (int j0 = 0; j0 < dv; j0 += 8 * groups) {
    u32x4 w[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int jj = j0 + groups * r + g;
      w[r] = jj < dv ? *reinterpret_cast<const u32x4*>(wv + static_cast<int64_t>(jj) * dc) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int jj = j0 + groups * r + g;
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = fmaf(__uint_as_float(w[r][e] << 16), ol[2 * e], s);
        s = fmaf(__uint_as_float(w[r][e] & 0xFFFF0000u), ol[2 * e + 1], s);
      }
      for (int o = 1; o < nc8; o <<= 1) s += __shfl_xor(s, o, 64);
      if (c8 == 0 && jj < dv) a.o[orow + jj] = f32_to_bf16(s);
    }
  }
}

hipError_t launch_mla_gemm(const MlaGemmArgs& a, int epi, hipStream_t s) {
  const dim3 grid((a.M + kGM - 1) / kGM, (a.N + kGN - 1) / kGN), block(kTh);
  switch (epi) {
    case kMlaEpiProj:
      hipLaunchKernelGGL(mla_gemm_kernel<kMlaEpiProj>, grid, block, 0, s, a);
      break;
    case kMlaEpiPlain:
      hipLaunchKernelGGL(mla_gemm_kernel<kMlaEpiPlain>, grid, block, 0, s, a);
      break;
    case kMlaEpiRes:
      hipLaunchKernelGGL(mla_gemm_kernel<kMlaEpiRes>, grid, block, 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mla_attn_prefill(const MlaAttnArgs& a, int batch, hipStream_t s) {
  if ((a.dn + a.dr) % 16 == 0 && (a.dv == 32 || a.dv == 64)) {
    const dim3 grid((a.seq + kFQ - 1) / kFQ, a.nh, batch);
    if (a.dv == 32) hipLaunchKernelGGL(mla_attn_prefill_mfma_kernel<1>, grid, dim3(kTh), 0, s, a);
    else hipLaunchKernelGGL(mla_attn_prefill_mfma_kernel<2>, grid, dim3(kTh), 0, s, a);
  } else {
    const dim3 grid((a.seq + kQT - 1) / kQT, a.nh, batch);
    hipLaunchKernelGGL(mla_attn_prefill_kernel, grid, dim3(kTh), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_mla_attn_decode(const MlaAttnArgs& a, int batch, hipStream_t s) {
  const int nchunk = (a.max_len + 63) / 64;
  const bool mfma = a.dr == 16 && (a.dc == 128 || a.dc == 64);
  int cps = 1;  // chunks per partial slot
  if (mfma) {
    hipLaunchKernelGGL(mla_decode_qlat_kernel, dim3(batch * a.nh), dim3(64), 0, s, a, batch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // chunks per block: runs of up to 8 chunks while the grid keeps about 8
    // blocks per CU (long contexts then write and merge 8x fewer partials)
    const int64_t seqs = kXcds * ((static_cast<int64_t>(batch) + kXcds - 1) / kXcds);
    const int64_t want = 8 * static_cast<int64_t>(device_cus());
    while (cps < 8 && seqs * ((nchunk + 2 * cps - 1) / (2 * cps)) >= want) cps *= 2;
    const int64_t blocks = seqs * ((nchunk + cps - 1) / cps);
    if (a.dc == 128)
      hipLaunchKernelGGL((mla_decode_mfma_kernel<128, 16>), dim3(static_cast<unsigned>(blocks)), dim3(64), 0, s, a,
                         batch, nchunk, cps);
    else
      hipLaunchKernelGGL((mla_decode_mfma_kernel<64, 16>), dim3(static_cast<unsigned>(blocks)), dim3(64), 0, s, a,
                         batch, nchunk, cps);
  } else {
    const int per_seq = a.nh * nchunk;
    const int blocks = kXcds * ((batch + kXcds - 1) / kXcds) * per_seq;
    const size_t lds = sizeof(uint16_t) * 64 * static_cast<size_t>(a.dc + a.dr + 8);
    hipLaunchKernelGGL(mla_decode_partial_kernel, dim3(blocks), dim3(64), lds, s, a, batch, nchunk);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_decode_combine_kernel, dim3(batch * a.nh), dim3(64), 0, s, a, batch, nchunk, cps);
  return hipGetLastError();
}

}  // namespace moe
