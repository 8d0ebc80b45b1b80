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
// Work decomposition.  A unit is (group, n-tile, m-tile): BM rows of the group
// against a BW-row weight tile (stage 1: BW/2 rows of W1 and the same rows of
// W3; stage 2: BW rows of W2).  Units of one group are ordered n-tile major,
// m-tile minor.  The grid is persistent; block b is remapped so that each XCD
// (blocks b = x mod 8) walks a contiguous range of units and the A rows of
// one expert stay in that XCD's L2.  Every block rebuilds the unit table from
// offsets[] (no host round trip).
//
// Two tile configurations:
//   kStream  BM = 256, BW = 128, 8 waves, 1 block/CU.  For weight-streaming
//            shapes (few rows per expert, weights far beyond the caches): one
//            unit covers all rows of an expert, so each weight byte is read
//            from HBM once (two 128-row m-tiles streaming the same weights
//            drift apart and both miss L2).
//   kCompute BM = BW = 128, 4 waves, 2 blocks/CU.  For shapes whose weights
//            stay in L2/MALL and whose groups have thousands of rows: more,
//            smaller units keep every CU busy.
//
// Pipeline.  A block's units run as an outer loop; each unit's K-loop (64 of
// K per step, an odd step count padded by one MFMA-free step) is
// straight-line code.  The fetcher runs two steps ahead of the MFMAs and
// crosses into the next unit during the last two steps, choosing the source
// with scalar selects.  Loads are buffer loads (uniform descriptor + 32-bit
// offset) into registers, stored to one of two XOR-swizzled LDS buffers.
// Barriers are raw s_barrier after an LDS-only wait: __syncthreads() would
// also drain the in-flight global loads.
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace moe {

constexpr int kBK = 64;                      // K per step
constexpr int kChunksPerRow = kBK / 8;       // 16-byte chunks per tile row
constexpr int kMaxGroups = 1025;

template <int BM_, int BW_, int WM_, int WN_, int BPC_, bool XU_>
struct TileCfg {
  static constexpr int BM = BM_;     // rows per unit
  static constexpr int BW = BW_;     // weight rows per unit
  static constexpr int WM = WM_;     // waves along M
  static constexpr int WN = WN_;     // waves along the weight tile
  static constexpr int BPC = BPC_;   // blocks per CU
  static constexpr bool XU = XU_;    // prefetch across unit boundaries
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int kRowsPerPass = kThreads / kChunksPerRow;
  static constexpr int kLoadsA = BM / kRowsPerPass;
  static constexpr int kLoadsB = BW / kRowsPerPass;
  static constexpr int TM = BM / WM / 32;  // 32-row MFMA tiles per wave
  static constexpr int TN = BW / WN / 32;  // 32-column MFMA tiles per wave
  static_assert(BM % kRowsPerPass == 0 && BW % (2 * kRowsPerPass) == 0, "load passes");
  static_assert(TN % 2 == 0, "SwiGLU pairs gate and up tiles inside a wave");
};
using kStream = TileCfg<256, 128, 4, 2, 1, true>;
using kCompute = TileCfg<128, 128, 2, 2, 2, true>;

// XOR swizzle of the 16-byte chunks of a row, so that the 32 rows an MFMA
// fragment read touches at one chunk hit distinct LDS banks.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kChunksPerRow + (chunk ^ (row & (kChunksPerRow - 1)));
}

// Compile-time loop: calls f(integral_constant<int, I>) for I = 0..N-1, so
// register arrays indexed by I are split into registers from the first
// optimisation pass on (a #pragma unroll comes too late for that).
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}
#define MOE_FOR(I, N, ...) \
  static_for<0, N>([&](auto I##_c) { constexpr int I = decltype(I##_c)::value; __VA_ARGS__ });

// LDS-only barrier: waits for this wave's LDS traffic, not for global loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Exclusive scan of one value per thread over a block of kThreads threads.
template <int kThreads>
__device__ __forceinline__ int block_scan(int v, int* total, int* wsum) {
  constexpr int kWaves = kThreads / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < kWaves; ++i) {
    base += i < w ? wsum[i] : 0;
    tot += wsum[i];
  }
  *total = tot;
  __syncthreads();
  return base + inc - v;
}

// Wave-uniform description of one unit (held in scalar registers).
struct Unit {
  int g;           // group (E = shared)
  int valid_rows;  // rows of this m-tile that exist
  int n0;          // first output column
  int K, N, nk;
  int orow0;       // output row of the tile's first row
  int routed;      // 1: routed expert group, 0: shared expert
};

template <class C, bool kSwiGLU>
__device__ __forceinline__ Unit decode_unit(const GroupedGemmArgs& a, const int* unit_start,
                                            const int* offs, int ngroups, int u) {
  int lo = 0, hi = ngroups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (uni(unit_start[mid]) <= u) lo = mid; else hi = mid - 1;
  }
  Unit r;
  r.g = uni(lo);
  r.routed = r.g < a.E;
  const int grow0 = r.routed ? uni(offs[r.g]) : 0;
  const int rows = r.routed ? uni(offs[r.g + 1]) - grow0 : static_cast<int>(a.T);
  const int mt = (rows + C::BM - 1) / C::BM;
  const int local = u - uni(unit_start[r.g]);
  const int n_tile = local / mt, m_tile = local % mt;
  const int m0 = m_tile * C::BM;
  r.valid_rows = uni((rows - m0) < C::BM ? (rows - m0) : C::BM);
  r.K = r.routed ? a.K_r : a.K_s;
  r.N = r.routed ? a.N_r : a.N_s;
  r.nk = r.K / kBK;
  r.n0 = n_tile * (kSwiGLU ? C::BW / 2 : C::BW);
  r.orow0 = uni(grow0 + m0);
  return r;
}

template <class C, bool kSwiGLU>
__global__ __launch_bounds__(C::kThreads, C::BPC) void grouped_gemm_kernel(GroupedGemmArgs a) {
  constexpr int kThreads = C::kThreads, RPP = C::kRowsPerPass;
  constexpr int LA = C::kLoadsA, LB = C::kLoadsB, TM = C::TM, TN = C::TN;
  __shared__ u32x4 lds_a[2][C::BM * kChunksPerRow];
  __shared__ u32x4 lds_b[2][C::BW * kChunksPerRow];
  __shared__ int unit_start[kMaxGroups + 1];
  __shared__ int offs[kMaxGroups + 1];  // copy of offsets[0..E]
  __shared__ int wsum[kThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int E = a.E;
  const bool has_shared = a.w_shared != nullptr;
  const int ngroups = E + (has_shared ? 1 : 0);
  constexpr int cols_per_tile = kSwiGLU ? C::BW / 2 : C::BW;

  // ---- unit table: units of group g start at unit_start[g]
  {
    constexpr int kPer = (kMaxGroups + kThreads - 1) / kThreads;
    const int per = (ngroups + kThreads - 1) / kThreads;
    int local[kPer];
    int sum = 0;
    for (int i = 0; i < per; ++i) {
      const int g = tid * per + i;
      int u = 0;
      if (g <= E) offs[g] = a.offsets[g];
      if (g < ngroups) {
        const int64_t rows = g < E ? static_cast<int64_t>(a.offsets[g + 1] - a.offsets[g]) : a.T;
        const int n = g < E ? a.N_r : a.N_s;
        const int nt = (n + cols_per_tile - 1) / cols_per_tile;
        u = static_cast<int>((rows + C::BM - 1) / C::BM) * nt;
      }
      local[i] = u;
      sum += u;
    }
    int total;
    int run = block_scan<kThreads>(sum, &total, wsum);
    for (int i = 0; i < per; ++i) {
      const int g = tid * per + i;
      if (g < ngroups) unit_start[g] = run;
      run += local[i];
    }
    if (tid == 0) {
      unit_start[ngroups] = total;
      offs[E] = a.offsets[E];
    }
    __syncthreads();
  }
  const int total_units = uni(unit_start[ngroups]);
  const int G = gridDim.x;
  const int lb = (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds;
  if (lb >= total_units) return;
  auto decode = [&](int u) __attribute__((always_inline)) {
    return decode_unit<C, kSwiGLU>(a, unit_start, offs, ngroups, u);
  };

  const int ld_row = tid / kChunksPerRow;  // 0..RPP-1
  const int ld_chunk = tid % kChunksPerRow;

  // ---- source of a unit: buffer descriptors (wave-uniform, scalar
  // registers) plus 32-bit byte offsets.  An A row (a gathered token) needs a
  // per-thread offset per load pass; a weight row is a uniform row base (the
  // scalar offset of the load) plus one per-thread term.  Rows are clamped to
  // rows that exist (a tile's first row always does) so every load is
  // unconditional; rows and columns past the tile's edge give results the
  // epilogue never stores.  The descriptors' ranges make any stray offset read
  // zeros.  perm_src entries are loaded one unit ahead and consumed only when
  // that unit becomes current, so their latency hides behind a whole unit.
  struct Src {
    __amdgpu_buffer_rsrc_t ra, rb0, rb1;  // A rows; W1 (or W2) rows; W3 rows
    int a_off[LA];                        // per thread, bytes
    int b_row[LB];                        // uniform, bytes: weight row base of each pass
    int b_thr;                            // per thread, bytes
    int nk;                               // K-steps with data
  };
  int pend_row[LA];  // prepared unit: group row / token per thread row
  int pend_map[LA];  // prepared unit: perm_src[pend_row] when gathering
  Unit pend;
  auto prepare = [&](int u) __attribute__((always_inline)) {
    pend = decode(u);
    const bool gather = pend.routed && a.a_row_map;
    MOE_FOR(i, LA, {
      int r = ld_row + RPP * i;
      if (r >= pend.valid_rows) r = 0;
      pend_row[i] = pend.orow0 + r;
      // branch-free, so the loaded value is not touched until the unit switch
      const int32_t* src = gather ? a.a_row_map + pend_row[i] : a.offsets;
      pend_map[i] = *src;
    })
  };
  constexpr int kRsrcFlags = 0x00020000;  // raw (untyped) buffer
  auto rsrc = [](const void* base, int64_t bytes) __attribute__((always_inline)) {
    const int n = bytes < 0x7FFFFFFF ? static_cast<int>(bytes) : 0x7FFFFFFF;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n,
                                             kRsrcFlags);
  };
  auto source_of_pending = [&]() __attribute__((always_inline)) {
    Src sr;
    const bool routed = pend.routed;
    const int K = pend.K, N = pend.N, g = pend.g, n0 = pend.n0;
    const bool gather = routed && a.a_row_map;
    sr.ra = routed ? rsrc(a.a_routed, a.a_routed_bytes) : rsrc(a.a_shared, a.a_shared_bytes);
    const int64_t wbytes = static_cast<int64_t>(N) * K * 2;
    const uint16_t* w0 = routed ? a.w_routed + static_cast<int64_t>(g) * N * K : a.w_shared;
    const uint16_t* w1 =
        kSwiGLU ? (routed ? a.w3_routed + static_cast<int64_t>(g) * N * K : a.w3_shared) : w0;
    sr.rb0 = rsrc(w0, wbytes);
    sr.rb1 = rsrc(w1, wbytes);
    MOE_FOR(i, LA, {
      int row = gather ? pend_map[i] : pend_row[i];
      if (gather && (row < 0 || row >= a.T)) row = 0;  // malformed permutation: stay in bounds
      sr.a_off[i] = (row * K + ld_chunk * 8) * 2;
    })
    // weight tile: SwiGLU stage rows [0, BW/2) = W1[n0..], [BW/2, BW) = W3[n0..]
    // (each load pass lies in one half, so one descriptor per pass); down
    // stage rows [0, BW) = W2[n0..]
    MOE_FOR(i, LB, {
      constexpr int t0 = RPP * i;
      int wrow = kSwiGLU ? n0 + t0 % (C::BW / 2) : n0 + t0;
      if (wrow >= N) wrow = 0;
      sr.b_row[i] = uni(wrow * K * 2);
    })
    sr.b_thr = (ld_row * K + ld_chunk * 8) * 2;
    sr.nk = pend.nk;
    return sr;
  };

  struct Slice {
    u32x4 a[LA], b[LB];
  };
  // Loads K-step f of the current source (f < steps0) or step f - steps0 of
  // the next one, chosen by a uniform test (scalar selects, no branches, so
  // the K-loop stays straight-line).  A step at or past nk (the padding step
  // of an odd count) reloads the last slice and is never multiplied.
  auto load2 = [&](Slice& sl, const Src& c0, const Src& c1, int steps0, int f)
      __attribute__((always_inline)) {
    const bool nxt = f >= steps0;
    const int j = nxt ? f - steps0 : f;
    const int nk = nxt ? c1.nk : c0.nk;
    const int kb = (j < nk ? j : nk - 1) * (kBK * 2);
    const __amdgpu_buffer_rsrc_t ra = nxt ? c1.ra : c0.ra;
    const __amdgpu_buffer_rsrc_t rb0 = nxt ? c1.rb0 : c0.rb0;
    const __amdgpu_buffer_rsrc_t rb1 = nxt ? c1.rb1 : c0.rb1;
    const int bt = (nxt ? c1.b_thr : c0.b_thr) + kb;
    MOE_FOR(i, LA, {
      const int ao = (nxt ? c1.a_off[i] : c0.a_off[i]) + kb;
      sl.a[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, ao, 0, 0));
    })
    MOE_FOR(i, LB, {
      constexpr bool up = kSwiGLU && RPP * i >= C::BW / 2;
      const int br = nxt ? c1.b_row[i] : c0.b_row[i];
      sl.b[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(up ? rb1 : rb0, bt, br, 0));
    })
  };
  auto stash = [&](const Slice& sl, int buf) __attribute__((always_inline)) {
    MOE_FOR(i, LA, { lds_a[buf][swz(ld_row + RPP * i, ld_chunk)] = sl.a[i]; })
    MOE_FOR(i, LB, { lds_b[buf][swz(ld_row + RPP * i, ld_chunk)] = sl.b[i]; })
  };

  // Accumulators: acc[tm][tn], rows wm*BM/WM + 32*tm, weight-tile rows
  // SwiGLU: tn < TN/2 gate rows wn*HC + 32*tn, tn >= TN/2 the up rows of the
  // same h columns (BW/2 further); down: rows wn*BW/WN + 32*tn.
  constexpr int HC = C::BW / 2 / C::WN;  // h columns per wave (SwiGLU)
  f32x16 acc[TM][TN];
  auto zero_acc = [&]() __attribute__((always_inline)) {
    MOE_FOR(i, TM, { MOE_FOR(j, TN, { acc[i][j] = f32x16{}; }) })
  };
  auto brow = [&](int tn) __attribute__((always_inline)) {
    if (kSwiGLU)
      return tn < TN / 2 ? wn * HC + 32 * tn : C::BW / 2 + wn * HC + 32 * (tn - TN / 2);
    return wn * (C::BW / C::WN) + 32 * tn;
  };

  auto mma = [&](int buf, int mrows) __attribute__((always_inline)) {
    // mrows: 32-row tiles of this wave that hold valid rows (0..TM)
    if (mrows <= 0) return;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int ch = 2 * ks + (lane >> 5);
      const int fr = lane & 31;
      bf16x8 af[TM], bfr[TN];
      MOE_FOR(i, TM, {
        af[i] = __builtin_bit_cast(bf16x8, lds_a[buf][swz(wm * (C::BM / C::WM) + 32 * i + fr, ch)]);
      })
      MOE_FOR(j, TN, { bfr[j] = __builtin_bit_cast(bf16x8, lds_b[buf][swz(brow(j) + fr, ch)]); })
      MOE_FOR(i, TM, {
        if (i < mrows) {
          MOE_FOR(j, TN, {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
          })
        }
      })
      // Keep each sub-step's fragment reads next to its MFMAs: hoisting them
      // all costs registers and spills the in-flight slices.
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto epilogue = [&](const Unit& cu) __attribute__((always_inline)) {
    // 32x32 accumulator layout: lane holds column (lane & 31), rows
    // (v/4)*8 + (lane/32)*4 + v%4 for v = 0..15.
    const int col_l = lane & 31;
    const int row_l = (lane >> 5) * 4;
    uint16_t* cbase = cu.routed ? a.c_routed : a.c_shared;
    MOE_FOR(i, TM, {
      MOE_FOR(v, 16, {
        const int r = wm * (C::BM / C::WM) + 32 * i + (v >> 2) * 8 + row_l + (v & 3);
        if (r < cu.valid_rows) {
          uint16_t* orow = cbase + (static_cast<int64_t>(cu.orow0) + r) * cu.N;
          if (kSwiGLU) {
            MOE_FOR(j, TN / 2, {
              const float ga = acc[i][j][v], up = acc[i][j + TN / 2][v];
              const float hval = ga / (1.0f + __expf(-ga)) * up;
              orow[cu.n0 + wn * HC + 32 * j + col_l] = f32_to_bf16(hval);
            })
          } else {
            MOE_FOR(j, TN, {
              const int c = cu.n0 + wn * (C::BW / C::WN) + 32 * j + col_l;
              if (c < cu.N) orow[c] = f32_to_bf16(acc[i][j][v]);
            })
          }
        }
      })
    })
  };

  // ---- software pipeline.  Each unit runs an even number of K-steps; the
  // fetcher stays two steps ahead, running into the next unit during the last
  // two steps of the current one.  The unit after the last one is the last
  // one again: its loads are valid and never used.
  auto next_of = [&](int u) __attribute__((always_inline)) {
    return u + G < total_units ? u + G : u;
  };
  Slice r0, r1;
  if constexpr (C::XU) {
    prepare(lb);
    Src cur = source_of_pending();
    Unit cu = pend;
    prepare(next_of(lb));
    load2(r0, cur, cur, 1 << 30, 0);
    load2(r1, cur, cur, 1 << 30, 1);
    stash(r0, 0);
    lds_barrier();
    for (int u = lb; u < total_units; u += G) {
      const Src nxt = source_of_pending();
      const Unit nu = pend;
      prepare(next_of(next_of(u)));
      const int steps = cur.nk + (cur.nk & 1);
      // 32-row tiles of this wave with valid rows
      int mrows = (cu.valid_rows - wm * (C::BM / C::WM) + 31) / 32;
      mrows = mrows < 0 ? 0 : (mrows > TM ? TM : mrows);
      zero_acc();
      for (int kt = 0; kt < steps; kt += 2) {
        load2(r0, cur, nxt, steps, kt + 2);
        mma(0, mrows);
        stash(r1, 1);
        lds_barrier();
        load2(r1, cur, nxt, steps, kt + 3);
        mma(1, kt + 1 < cur.nk ? mrows : 0);
        stash(r0, 0);
        lds_barrier();
      }
      epilogue(cu);
      cur = nxt;
      cu = nu;
    }
  } else {
    // Units are long (many K-steps): the pipeline restarts at each unit and
    // only the perm_src lookups run one unit ahead.
    prepare(lb);
    for (int u = lb; u < total_units; u += G) {
      const Src cur = source_of_pending();
      const Unit cu = pend;
      prepare(next_of(u));
      const int steps = cur.nk + (cur.nk & 1);
      int mrows = (cu.valid_rows - wm * (C::BM / C::WM) + 31) / 32;
      mrows = mrows < 0 ? 0 : (mrows > TM ? TM : mrows);
      load2(r0, cur, cur, 1 << 30, 0);
      load2(r1, cur, cur, 1 << 30, 1);
      lds_barrier();  // the previous unit's last LDS reads are done
      stash(r0, 0);
      lds_barrier();
      zero_acc();
      for (int kt = 0; kt < steps; kt += 2) {
        load2(r0, cur, cur, 1 << 30, kt + 2 < steps ? kt + 2 : steps - 1);
        mma(0, mrows);
        stash(r1, 1);
        lds_barrier();
        load2(r1, cur, cur, 1 << 30, kt + 3 < steps ? kt + 3 : steps - 1);
        mma(1, kt + 1 < cur.nk ? mrows : 0);
        stash(r0, 0);
        lds_barrier();
      }
      epilogue(cu);
    }
  }
}

template <class C>
static int persistent_grid() {
  int g = C::BPC * device_cus();
  g = (g / kXcds) * kXcds;
  return g > 0 ? g : kXcds;
}

// The 256-row tile pays off when experts hold between one and two 128-row
// m-tiles of rows and their weights are far beyond the on-chip caches (each
// weight byte is then read once instead of once per m-tile).  With fewer
// rows (decode) a 128-row m-tile already covers an expert and two blocks per
// CU keep more weight bytes in flight.
static bool streaming_shape(const GroupedGemmArgs& a) {
  const int64_t rows_per_expert = a.T * a.top_k / (a.E > 0 ? a.E : 1);
  const int64_t weight_bytes = static_cast<int64_t>(a.E) * a.N_r * a.K_r * 2 * 3;
  return rows_per_expert > 64 && rows_per_expert <= 256 && weight_bytes > (int64_t{1} << 30);
}

template <bool kSwiGLU>
static hipError_t launch_gemm(const GroupedGemmArgs& a, hipStream_t s) {
  if (streaming_shape(a)) {
    hipLaunchKernelGGL((grouped_gemm_kernel<kStream, kSwiGLU>), dim3(persistent_grid<kStream>()),
                       dim3(kStream::kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((grouped_gemm_kernel<kCompute, kSwiGLU>), dim3(persistent_grid<kCompute>()),
                       dim3(kCompute::kThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_swiglu(const GroupedGemmArgs& a, hipStream_t s) { return launch_gemm<true>(a, s); }
hipError_t launch_gemm_down(const GroupedGemmArgs& a, hipStream_t s) { return launch_gemm<false>(a, s); }

}  // namespace moe
