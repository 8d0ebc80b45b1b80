// bwd_gemm.hip -- grouped GEMMs of the layer backward on bf16 MFMA (gfx950).
//
// Training runs the layer backward ("190行JAX复刻DeepSeek V3" (openai-hub.com),
// section 如何在Mac上复现: 12000 AdamW steps).  With rows grouped by expert
// (moe_permute's order) and the upstream gradient already scaled by the gates
// (moe_combine_backward), every product of an expert's backward is a GEMM over
// contiguous rows, one per expert group:
//   dh   = dy W2                      rows x H,  K = d        (input gradient)
//   a, c = x W1^T, x W3^T  -> da, dc, h (the forward's SwiGLU GEMM again,
//                                         grouped_gemm.hip, with the SwiGLU
//                                         derivative in its epilogue)
//   dx   = da W1 + dc W3               rows x d,  K = 2H       (input gradient)
//   dW2  = dy^T h                      d x H,     K = rows     (weight gradient)
//   dW1  = da^T x,  dW3 = dc^T x       2H x d,    K = rows     (one launch)
// so the weights are read as stored (W1, W3 [H, d]; W2 [d, H]) and the
// operands come in two layouts: K contiguous (a row of K values) or K major
// (a row per index of K).  The group's rows are the ragged M of an input
// gradient and the ragged K of a weight gradient; a group with no rows gets
// a zero weight gradient.  One launch covers the shared expert (one group of
// all T rows, its own operands) and the routed experts.
//
// Input gradients (bwd_gemm_kernel): tile 128 x 128 x 64,
// four waves of 64 x 64 (2 x 2 MFMA tiles of 32x32x16, fp32 accumulators),
// two blocks per CU, persistent over units (group, m-tile, n-tile); each XCD
// runs an eighth of the units in order, so the units of one group share its
// L2.  Each operand's K-step is loaded to registers two steps ahead (kDepth):
// four 16-byte loads per thread, along the contiguous direction.  Both layouts
// are staged in LDS the same way, a row of the tile (an M or N index) holding
// its 64 K values as eight 16-byte chunks, so every MFMA fragment is one
// 16-byte LDS read.  The K-major operand (the weight of dh and dx) gets there
// through a transpose in registers: a thread loads 4 rows of K x 8 columns
// and writes 8 columns x 4 values of K (8 bytes each).  The chunk order within
// a row is XOR-swizzled with bits 1-3 of the row (chunk ^ (row >> 1) ^
// (row >> 3)): fragment reads and K-contiguous stores hit 64 distinct banks
// per 16 lanes, the transposed stores two ways at most.
//
// Weight gradients (wgrad_kernel, described above it) have both operands K
// major.  With too few tiles to fill the chip (small d and H) they split a
// group's rows into pieces of `split` rows; each piece writes fp32 partial
// sums and wgrad_reduce_kernel adds them in piece order, so the result does
// not depend on timing.
#include "common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

#include <algorithm>
#include <type_traits>

namespace moe {

namespace {
constexpr int kTh = 256;                    // threads
constexpr int kTM = 128, kTN = 128, kTK = 64;
constexpr int kRowCh = kTK / 8;             // 16-byte chunks per staged row (8)
constexpr int kStageU4 = kTM * kRowCh;      // one operand stage, in u32x4 (16 KB)
constexpr int kMaxG = 1024 + 1;             // routed groups + the shared expert
constexpr int kSplitTarget = 1024;          // weight-gradient units wanted per launch
constexpr int kMinSplit = 512;              // rows per split at least (8 K-steps)
#ifndef MOE_BWD_DEPTH
#define MOE_BWD_DEPTH 2
#endif
constexpr int kDepth = MOE_BWD_DEPTH;       // K-steps loaded ahead, in registers

static_assert(kTM == kTN, "one staging layout serves both operands");

// u32x4 index of chunk c (8 values of K) of staged row r
__device__ __forceinline__ int sidx(int r, int c) {
  return r * kRowCh + ((c ^ (r >> 1) ^ (r >> 3)) & (kRowCh - 1));
}

__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// the segment's field f, for a wave-uniform segment index
#define SEGF(sg, f) ((sg) ? a.seg[1].f : a.seg[0].f)

// rows of group h of segment sg
__device__ __forceinline__ int seg_group_rows(const BwdGemmArgs& a, int sg, int h) {
  const int32_t* o = SEGF(sg, offsets);
  return o ? o[h + 1] - o[h] : SEGF(sg, rows);
}
}  // namespace

template <int KIND>
__global__ __launch_bounds__(kTh, 2) void bwd_gemm_kernel(BwdGemmArgs a) {
  // stages: A in lds[0], lds[1]; B in lds[2], lds[3]
  __shared__ u32x4 lds[4][kStageU4];
  u32x4 (*const lds_a)[kStageU4] = lds;
  u32x4 (*const lds_b)[kStageU4] = lds + 2;
  __shared__ int ustart[kMaxG + 1];  // first unit of each group
  __shared__ int goff[kMaxG + 1];    // first row of each group in its segment's arrays
  __shared__ int wsum[kTh / 64];
  static_assert(KIND == kBwdDgradKM, "input gradients");
  constexpr int kCols = kTN;                     // output columns per unit

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int G0 = a.seg[0].groups;
  const int G = G0 + (a.nseg > 1 ? a.seg[1].groups : 0);

  // ---- unit table: per group, units = m-tiles x n-tiles
  {
    constexpr int kPer = (kMaxG + kTh - 1) / kTh;
    int lu[kPer];
    int su = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int gg = tid * kPer + i;
      int u = 0;
      if (gg < G) {
        const int sg = gg >= G0 ? 1 : 0;
        const int h = gg - (sg ? G0 : 0);
        const int32_t* o = SEGF(sg, offsets);
        goff[gg] = o ? o[h] : 0;
        u = cdiv(seg_group_rows(a, sg, h), kTM) * cdiv(SEGF(sg, N), kCols);
      }
      lu[i] = u;
      su += u;
    }
    int tot_u;
    int run_u = block_scan<kTh>(su, &tot_u, wsum);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int gg = tid * kPer + i;
      if (gg < G) ustart[gg] = run_u;
      run_u += lu[i];
    }
    if (tid == 0) ustart[G] = tot_u;
    __syncthreads();
  }
  const int total_units = uni(ustart[G]);
  // XCD x (blocks b with b % 8 == x) takes the x-th eighth of the units in
  // order, so the units of a group (which share their rows and weights) run
  // on one XCD and its L2
  const int xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds;
  const int u_lo = static_cast<int>(static_cast<int64_t>(total_units) * xcd / kXcds);
  const int u_hi = static_cast<int>(static_cast<int64_t>(total_units) * (xcd + 1) / kXcds);

  // fragments: weight-side (B) operand first, so a lane holds output row
  // (lane & 31) and columns 8q + 4(lane >> 5) + 0..3 of each 32x32 tile
  const int fr = lane & 31, fhalf = lane >> 5;
  // K-contiguous loads: chunk q = tid + 256 p is row q / 8, chunk q % 8;
  // K-major loads: rows 4 kb .. 4 kb + 3 of K at columns 8 cb .. 8 cb + 7
  const int cb = tid & 15, kb = tid >> 4;

  // ---- a unit: its uniform description
  struct Unit {
    int gg, sg, g, off, R, N, K, m0, n0, kend, nk;
  };
  auto decode = [&](int u) {
    Unit t;
    int below = 0;
    for (int base = 0; base < G; base += 64) {
      const int gi = base + lane;
      below += __popcll(__ballot(gi < G && ustart[gi] <= u));
    }
    t.gg = uni(below - 1);
    t.sg = t.gg >= G0 ? 1 : 0;
    t.g = t.gg - (t.sg ? G0 : 0);
    t.off = uni(goff[t.gg]);
    t.R = uni(seg_group_rows(a, t.sg, t.g));
    const int local = u - uni(ustart[t.gg]);
    t.N = SEGF(t.sg, N);
    t.K = SEGF(t.sg, K);
    const int mt = cdiv(t.R, kTM);
    t.m0 = (local % mt) * kTM;
    t.n0 = (local / mt) * kCols;
    t.kend = t.K + SEGF(t.sg, K2);
    t.nk = cdiv(t.kend, kTK);
    return t;
  };

  // ---- per-thread load addressing of the unit being loaded.  Loads are not
  // predicated: an out-of-range chunk reads a valid address of the unit and
  // is zeroed when it is stored to LDS, so the compiler can wait for one
  // K-step's loads while later ones are in flight.
  const uint16_t *A = nullptr, *A2 = nullptr, *B = nullptr, *B2 = nullptr;
  int64_t lda = 0, ldb = 0, bgs = 0;
  int a_row[4];                    // K-contiguous A: element offset of the row
  bool a_ok[4];                    // ... inside the group
  int km_b_col = 0;                // K-major B: first column
  bool km_b_ok = false;
  auto setup = [&](const Unit& t) {
    A = SEGF(t.sg, a);
    A2 = SEGF(t.sg, a2);
    lda = SEGF(t.sg, lda);
    B = SEGF(t.sg, b);
    B2 = SEGF(t.sg, b2);
    ldb = SEGF(t.sg, ldb);
    bgs = static_cast<int64_t>(t.g) * SEGF(t.sg, b_gstride);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int row = (tid + kTh * p) >> 3;
      a_ok[p] = t.m0 + row < t.R;
      a_row[p] = (t.off + (a_ok[p] ? t.m0 + row : t.m0)) * static_cast<int>(lda);
    }
    km_b_ok = t.n0 + 8 * cb < t.N;
    km_b_col = km_b_ok ? t.n0 + 8 * cb : t.n0;
  };

  // ---- loads of K-step kt (16-byte chunks)
  auto load_a = [&](const Unit& t, int kt, u32x4 (&v)[4]) {
    const int k0 = kt * kTK;
    const bool second = k0 >= t.K;
    const uint16_t* base = (second ? A2 : A) + (second ? k0 - t.K : k0);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int ch = (tid + kTh * p) & 7;
      v[p] = *reinterpret_cast<const u32x4*>(base + a_row[p] + 8 * ch);
    }
  };
  auto load_b = [&](const Unit& t, int kt, u32x4 (&v)[4]) {
    // a weight stored [K, N] (+ b2 for the K2 rows after K)
    const int k0 = kt * kTK;
    const bool second = k0 >= t.K;
    const uint16_t* base = (second ? B2 : B) + bgs +
                           static_cast<int64_t>((second ? k0 - t.K : k0) + 4 * kb) * ldb + km_b_col;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const u32x4*>(base + i * ldb);
  };
  // ---- stores of a loaded K-step into a stage (out-of-range chunks as zero)
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
  auto store_kc = [&](u32x4* buf, const u32x4 (&v)[4], const bool (&ok)[4]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int q = tid + kTh * p;
      buf[sidx(q >> 3, q & 7)] = ok[p] ? v[p] : zero4;
    }
  };
  auto store_km = [&](u32x4* buf, const u32x4 (&v)[4], bool col_ok, const Unit& t, int kt) {
    // column j of the 8 loaded: values of K 4 kb .. 4 kb + 3 -> 8 bytes of
    // chunk kb / 2 of staged row 8 cb + j
    const int krow = kt * kTK + 4 * kb;
    u32x4 z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = col_ok && krow + i < t.kend ? v[i] : zero4;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int w = j >> 1;
      uint32_t lo, hi;
      if (j & 1) {
        lo = (z[0][w] >> 16) | (z[1][w] & 0xFFFF0000u);
        hi = (z[2][w] >> 16) | (z[3][w] & 0xFFFF0000u);
      } else {
        lo = (z[0][w] & 0xFFFFu) | (z[1][w] << 16);
        hi = (z[2][w] & 0xFFFFu) | (z[3][w] << 16);
      }
      uint2* dst = reinterpret_cast<uint2*>(buf + sidx(8 * cb + j, kb >> 1)) + (kb & 1);
      *dst = make_uint2(lo, hi);
    }
  };
  auto store_a = [&](u32x4* buf, const u32x4 (&v)[4], const Unit&, int) { store_kc(buf, v, a_ok); };
  auto store_b = [&](u32x4* buf, const u32x4 (&v)[4], const Unit& t, int kt) {
    store_km(buf, v, km_b_ok, t, kt);
  };

  f32x16 acc[2][2];
  auto arow = [&](int i) { return 64 * wm + 32 * i + fr; };
  auto brow = [&](int j) { return 64 * wn + 32 * j + fr; };
  auto compute = [&](const u32x4* sa, const u32x4* sb) {
#pragma unroll
    for (int ks = 0; ks < kTK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
      const int ch = 2 * ks + fhalf;
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = __builtin_bit_cast(bf16x8, sa[sidx(arow(i), ch)]);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = __builtin_bit_cast(bf16x8, sb[sidx(brow(j), ch)]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  };

  // kDepth K-steps in registers: slot s holds the K-step that goes to stage s
  // next; stage kt & 1 holds K-step kt while it is multiplied.  A unit's
  // first kDepth K-steps are loaded before the previous unit's epilogue.
  u32x4 ra[kDepth][4], rb[kDepth][4];
  auto load_first = [&](const Unit& t) {
    if (t.nk > 0) {
      load_a(t, 0, ra[0]);
      load_b(t, 0, rb[0]);
    }
    if constexpr (kDepth == 2) {
      if (t.nk > 1) {
        load_a(t, 1, ra[1]);
        load_b(t, 1, rb[1]);
      }
    }
  };
  const int lcol = fhalf * 4;
  auto epilogue = [&](const Unit& t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = t.m0 + 64 * wm + 32 * i + fr;  // output row within the group
      if (r >= t.R) continue;
      uint16_t* crow = static_cast<uint16_t*>(SEGF(t.sg, c)) + static_cast<int64_t>(t.off + r) * SEGF(t.sg, ldc);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = t.n0 + 64 * wn + 32 * j + 8 * q + lcol;
          if (col >= t.N) continue;
          const f32x16& v = acc[i][j];
          *reinterpret_cast<uint2*>(crow + col) =
              make_uint2(bf16x2_bits(v[4 * q], v[4 * q + 1]), bf16x2_bits(v[4 * q + 2], v[4 * q + 3]));
        }
    }
  };

  int u = u_lo + static_cast<int>(blockIdx.x) / kXcds;
  bool have = u < u_hi;
  Unit cur{};
  if (have) {
    cur = decode(u);
    setup(cur);
    load_first(cur);
  }
  while (have) {
    if (cur.nk > 0) {
      store_a(lds_a[0], ra[0], cur, 0);
      store_b(lds_b[0], rb[0], cur, 0);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    auto step = [&](auto st_c, int kt) {
      constexpr int st = decltype(st_c)::value;       // == kt & 1
      constexpr int next = kDepth == 2 ? st ^ 1 : 0;  // slot of K-step kt + 1
      if constexpr (kDepth == 2) {
        if (kt + 2 < cur.nk) {
          load_a(cur, kt + 2, ra[st]);
          load_b(cur, kt + 2, rb[st]);
        }
      } else {
        if (kt + 1 < cur.nk) {
          load_a(cur, kt + 1, ra[0]);
          load_b(cur, kt + 1, rb[0]);
        }
      }
      compute(lds_a[st], lds_b[st]);
      if (kt + 1 < cur.nk) {
        store_a(lds_a[st ^ 1], ra[next], cur, kt + 1);
        store_b(lds_b[st ^ 1], rb[next], cur, kt + 1);
      }
      __syncthreads();
    };
    for (int kt = 0; kt < cur.nk; kt += 2) {
      step(std::integral_constant<int, 0>{}, kt);
      if (kt + 1 < cur.nk) step(std::integral_constant<int, 1>{}, kt + 1);
    }
    // the next unit's first loads go out before this unit's stores
    const int un = u + per_xcd;
    const bool have_next = un < u_hi;
    Unit nxt{};
    if (have_next) {
      nxt = decode(un);
      setup(nxt);
      load_first(nxt);
    }
    epilogue(cur);
    cur = nxt;
    u = un;
    have = have_next;
  }
}

// ---- weight gradients ------------------------------------------------------
//
// dW[g] = A_g^T B_g, K = the group's rows: both operands K-major.  A step's
// tiles (64 rows of K x 128 columns per operand) go from memory into LDS by
// DMA as they are stored, one K row per 256 bytes, the four 64-byte pieces of
// row k rotated by k mod 4.  gfx950's ds_read_b64_tr_b16 reads such a tile
// transposed: within each 16 lanes, lane s names 4 values of row s / 4 and
// receives 4 consecutive rows of one column, so two reads give a lane the 8
// consecutive K values of its MFMA fragment and nothing is shuffled between
// threads.  Per 32 lanes a read covers 4 rows x 64 bytes, which the rotation
// puts on all 64 banks.
//
// Four waves (2 x 2 of 64 x 64), two blocks per CU, two step stages.  vmcnt
// counts a wave's loads and stores in one order, so the DMA waited for must
// not come after output stores that the write stream keeps in flight: every
// unit issues the same operations in the same order -- the DMA of its step 0
// (during the previous unit's last step), the DMA of its step 1 and the
// previous unit's 16 output stores per thread (in the epilogue), then one
// DMA per further step, with a DMA of every lane out of range for a step
// that does not exist and an empty descriptor for an output block outside
// the gradient -- and the waits count exactly: step 0 waits with 24 younger
// operations in flight, step 1 with the 16 stores, later steps with none
// (their DMA went out after the stores, which have had a unit's time).
// (One block per CU with loader waves that issue only DMA, four stages
// ahead, measured 8% slower: two independent blocks hide more.)  LDS is
// touched only through asm, which the compiler does not tie to the DMA it
// cannot track.
namespace {
constexpr int kWgT = 128;                                 // output tile, M and N
constexpr int kWgK = 64;                                  // rows of K per step
constexpr int kWgThreads = 256;
constexpr int kWgOp = kWgK * kWgT * 2;                    // bytes of one operand's step tile
constexpr int kWgDma = kWgOp / (kWgThreads * 16);         // DMA per thread, operand and step
constexpr int kWgStep = 2 * kWgDma;                       // a thread's DMA of a step
constexpr int kWgStores = kWgT * kWgT * 4 / (kWgThreads * 16);  // output stores per thread and unit
constexpr int kWgStage = 2 * kWgOp;                       // A tile, then B tile
constexpr int kWgHalf = 32 * 64 * 4;                      // a wave's 32 x 64 fp32 half block
constexpr unsigned kWgOut = 0x80000000u;                  // past every descriptor's range
constexpr int kWgRsrcFlags = 0x00020000;                  // raw (untyped) buffer
constexpr int kWgNT = 2;                                  // cache policy: non-temporal
static_assert(kWgStep + kWgStores < 64 && kWgStores == 16, "vmcnt range; two halves of 8 stores");

typedef short v4i16 __attribute__((ext_vector_type(4)));

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));  // lgkmcnt, expcnt free
}

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
}

__device__ __forceinline__ bf16x8 cat8(v4i16 lo, v4i16 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One MFMA sub-step's fragments: two of each operand, each the two 4-value
// halves of its 8 K values (the second 4 rows of K further), complete on return.
template <int kOff>
__device__ __forceinline__ void tr_frags(unsigned a0, unsigned a1, unsigned b0, unsigned b1,
                                         bf16x8 (&af)[2], bf16x8 (&bf)[2]) {
  v4i16 r[8];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
      "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
      "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
      "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
        "=&v"(r[7])
      : "v"(a0), "v"(a1), "v"(b0), "v"(b1), "i"(kOff), "i"(kOff + 4 * 256)
      : "memory");
  af[0] = cat8(r[0], r[1]);
  af[1] = cat8(r[2], r[3]);
  bf[0] = cat8(r[4], r[5]);
  bf[1] = cat8(r[6], r[7]);
}

// Eight 16-byte LDS writes (no wait: the same wave's reads come after them).
__device__ __forceinline__ void lds_write8_b128(const unsigned (&ad)[8], const u32x4 (&v)[8]) {
  asm volatile(
      "ds_write_b128 %0, %8\n\t"
      "ds_write_b128 %1, %9\n\t"
      "ds_write_b128 %2, %10\n\t"
      "ds_write_b128 %3, %11\n\t"
      "ds_write_b128 %4, %12\n\t"
      "ds_write_b128 %5, %13\n\t"
      "ds_write_b128 %6, %14\n\t"
      "ds_write_b128 %7, %15"
      :
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]),
        "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7])
      : "memory");
}
}  // namespace

__global__ __launch_bounds__(kWgThreads, 2) void wgrad_kernel(BwdGemmArgs a) {
  __shared__ u32x4 lds[2][kWgStage / 16];  // [stage][A tile | B tile]
  __shared__ int ustart[kMaxG + 1];        // first unit of each group
  __shared__ int goff[kMaxG + 1];          // first row of each group in its segment's arrays
  __shared__ int grows[kMaxG + 1];         // rows of each group (read here, not from memory
                                           // the stores may share: that would be a vector load)
  __shared__ int wsum[kWgThreads / 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int G0 = a.seg[0].groups;
  const int G = G0 + (a.nseg > 1 ? a.seg[1].groups : 0);
  auto mtiles = [&](int sg) {
    const int M = SEGF(sg, M), M1 = SEGF(sg, M1);
    return cdiv(M1, kWgT) + cdiv(M - M1, kWgT);
  };

  // ---- unit table: per group, (m-tiles of both halves) x n-tiles x splits
  {
    constexpr int kPer = (kMaxG + kWgThreads - 1) / kWgThreads;
    int lu[kPer];
    int su = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int gg = tid * kPer + i;
      int u = 0;
      if (gg < G) {
        const int sg = gg >= G0 ? 1 : 0;
        const int h = gg - (sg ? G0 : 0);
        const int32_t* o = SEGF(sg, offsets);
        goff[gg] = o ? o[h] : 0;
        const int R = seg_group_rows(a, sg, h);
        grows[gg] = R;
        const int split = SEGF(sg, split);
        const int ns = split > 0 ? std::max(1, cdiv(R, split)) : 1;
        u = mtiles(sg) * cdiv(SEGF(sg, N), kWgT) * ns;
      }
      lu[i] = u;
      su += u;
    }
    int tot_u;
    int run_u = block_scan<kWgThreads>(su, &tot_u, wsum);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int gg = tid * kPer + i;
      if (gg < G) ustart[gg] = run_u;
      run_u += lu[i];
    }
    if (tid == 0) ustart[G] = tot_u;
    __syncthreads();
  }
  const int total_units = uni(ustart[G]);
  // partial-sum slots of the segment's groups before group h (split mode):
  // groups of more than `split` rows take one slot per piece
  auto slots_before = [&](int sg, int h) {
    const int split = SEGF(sg, split), gbase = sg ? G0 : 0;
    int n = 0;
    for (int base = 0; base < h; base += 64) {
      const int hi = base + lane;
      int v = 0;
      if (hi < h) {
        const int ns = std::max(1, cdiv(grows[gbase + hi], split));
        v = ns > 1 ? ns : 0;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
      n += v;
    }
    return uni(n);
  };
  const int xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds;
  const int u_lo = static_cast<int>(static_cast<int64_t>(total_units) * xcd / kXcds);
  const int u_hi = static_cast<int>(static_cast<int64_t>(total_units) * (xcd + 1) / kXcds);

  struct WUnit {
    int gg, sg, g, half, m0, n0, kbeg, kend, nk, split_idx, nsplit;
    __amdgpu_buffer_rsrc_t ra, rb;  // the unit's rows kbeg..kend-1 of A and of B
    int va, vb;                     // this thread's DMA offset in step 0 (kWgOut: column outside)
    int lda2, ldb2;                 // row pitch in bytes
  };
  // DMA p of a wave covers rows 16 p + 4 wave .. + 3 of an operand's step
  // tile; lane l writes LDS bytes 16 l of them: row 16 p + 4 wave + l / 16,
  // stored piece ((l & 15) >> 2), which holds logical piece ((l & 15) >> 2) ^
  // (l >> 4) -- the rotation by the row mod 4 -- and chunk l & 3 of it.
  const int dma_row = 4 * wave + (lane >> 4);
  const int dma_col = 8 * (((((lane & 15) >> 2) ^ (lane >> 4)) << 2) | (lane & 3));
  auto decode = [&](int u) {
    WUnit t;
    int below = 0;
    for (int base = 0; base < G; base += 64) {
      const int gi = base + lane;
      below += __popcll(__ballot(gi < G && ustart[gi] <= u));
    }
    t.gg = uni(below - 1);
    t.sg = t.gg >= G0 ? 1 : 0;
    t.g = t.gg - (t.sg ? G0 : 0);
    const int off = uni(goff[t.gg]);
    const int R = uni(grows[t.gg]);
    const int local = u - uni(ustart[t.gg]);
    const int M = SEGF(t.sg, M), N = SEGF(t.sg, N), M1 = SEGF(t.sg, M1);
    const int split = SEGF(t.sg, split);
    t.nsplit = split > 0 ? std::max(1, cdiv(R, split)) : 1;
    const int mt1 = cdiv(M1, kWgT), mt = mtiles(t.sg);
    const int tiles = mt * cdiv(N, kWgT);
    t.split_idx = local / tiles;
    const int r = local - t.split_idx * tiles;
    // the 32 units that an XCD's CUs run at once cover 4 m-tiles x 8 n-tiles
    // where the tiles divide so, rather than 32 m-tiles of one n-tile: the
    // tile that all of them would read is the hot spot (12% slower)
    const int nt = tiles / mt;
    int mi, ni;
    if (mt % 4 == 0 && nt % 8 == 0) {
      const int bi = r / 32, w = r % 32;
      mi = (bi % (mt / 4)) * 4 + w % 4;
      ni = (bi / (mt / 4)) * 8 + w / 4;
    } else {
      mi = r % mt;
      ni = r / mt;
    }
    t.n0 = ni * kWgT;
    t.half = mi >= mt1 ? 1 : 0;
    t.m0 = (t.half ? mi - mt1 : mi) * kWgT;
    t.kbeg = t.nsplit > 1 ? t.split_idx * split : 0;
    t.kend = t.nsplit > 1 ? std::min(R, t.kbeg + split) : R;
    t.nk = std::max(1, cdiv(t.kend - t.kbeg, kWgK));
    const int64_t lda = SEGF(t.sg, lda), ldb = SEGF(t.sg, ldb);
    const int rows = t.kend - t.kbeg;
    const uint16_t* A = t.half ? SEGF(t.sg, a2) : SEGF(t.sg, a);
    const uint16_t* B = SEGF(t.sg, b);
    t.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A + (off + t.kbeg) * lda), static_cast<short>(0),
                                             static_cast<int>(rows * lda * 2), kWgRsrcFlags);
    t.rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(B + (off + t.kbeg) * ldb), static_cast<short>(0),
                                             static_cast<int>(rows * ldb * 2), kWgRsrcFlags);
    const int acols = t.half ? M - M1 : M1;
    t.va = t.m0 + dma_col < acols ? static_cast<int>((dma_row * lda + t.m0 + dma_col) * 2) : static_cast<int>(kWgOut);
    t.vb = t.n0 + dma_col < N ? static_cast<int>((dma_row * ldb + t.n0 + dma_col) * 2) : static_cast<int>(kWgOut);
    t.lda2 = static_cast<int>(lda * 2);
    t.ldb2 = static_cast<int>(ldb * 2);
    return t;
  };

  // ---- DMA of step kt of unit t into stage st (rows past the unit's K range
  // are past its descriptors and arrive as zeros)
  // (none: a step that does not exist, every lane out of range -- the same
  // eight operations into the same stage, so the counts stay exact)
  auto issue = [&](const WUnit& t, int kt, int st, bool none) {
    const bool oa_out = none || t.va == static_cast<int>(kWgOut);
    const bool ob_out = none || t.vb == static_cast<int>(kWgOut);
#pragma unroll
    for (int p = 0; p < kWgDma; ++p) {
      const int ra = (kt * kWgK + 16 * p) * t.lda2, rb = (kt * kWgK + 16 * p) * t.ldb2;
      dma_b128(t.ra, &lds[st][(4 * p + wave) * 64], oa_out ? static_cast<int>(kWgOut) : t.va + ra, 0);
      dma_b128(t.rb, &lds[st][kWgOp / 16 + (4 * p + wave) * 64], ob_out ? static_cast<int>(kWgOut) : t.vb + rb, 0);
    }
  };

  // ---- fragments: lane l reads 4 values of row (l & 15) / 4 (+ 8 for lanes
  // 32..63), columns 16 ((l >> 4) & 1) + 4 (l & 3) of the 32-column tile; the
  // tile's logical piece is rotated by that row mod 4
  const int tr_row = 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_in = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int tr_rot = (lane & 15) >> 2;
  const unsigned lds0 = lds_addr(&lds[0][0]);
  unsigned fa[2], fb[2];  // stage 0; stage 1 is kWgStage further
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    fa[i] = lds0 + tr_row * 256 + (((2 * wm + i) ^ tr_rot) << 6) + tr_in * 2;
    fb[i] = lds0 + kWgOp + tr_row * 256 + (((2 * wn + i) ^ tr_rot) << 6) + tr_in * 2;
  }
  f32x16 acc[2][2];
  auto compute = [&](int st) {
    const unsigned so = st * kWgStage;
    MOE_FOR(ks, kWgK / 16, {
      bf16x8 af[2], bfr[2];
      tr_frags<ks * 16 * 256>(fa[0] + so, fa[1] + so, fb[0] + so, fb[1] + so, af, bfr);
      MOE_FOR(i, 2, {
        MOE_FOR(j, 2, { acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0); })
      })
    })
  };

  // ---- epilogue: the wave's 64 x 64 block through its 8 KB of the stage the
  // last step read, 32 rows at a time (rows of 16 chunks of four values,
  // chunk c of row r at c ^ (r & 15)), into registers; then 16 row stores,
  // to an empty descriptor for a block outside the output
  const int fr = lane & 31, fhalf = lane >> 5;
  const int lrow = lane >> 4, lcol = 4 * (lane & 15);
  u32x4 outv[2][8];
  auto stage_out = [&](int st) {
    const unsigned sbase = lds0 + st * kWgStage + wave * kWgHalf;
    MOE_FOR(h, 2, {
      unsigned wa[8];
      u32x4 wv[8];
      MOE_FOR(j, 2, {
        MOE_FOR(q, 4, {
          const int ch = 8 * j + 2 * q + fhalf;
          wa[4 * j + q] = sbase + (fr * 16 + (ch ^ (fr & 15))) * 16;
          const f32x16& v = acc[h][j];
          wv[4 * j + q] = u32x4{__float_as_uint(v[4 * q]), __float_as_uint(v[4 * q + 1]),
                                __float_as_uint(v[4 * q + 2]), __float_as_uint(v[4 * q + 3])};
        })
      })
      lds_write8_b128(wa, wv);
      const u32x4* src[8];
      MOE_FOR(it, 8, {
        const int rr = 4 * it + lrow, ch = lane & 15;
        src[it] = reinterpret_cast<const u32x4*>(&lds[st][0]) + wave * (kWgHalf / 16) + rr * 16 + (ch ^ (rr & 15));
      })
      lds_read_n<8>(src, outv[h]);
    })
  };
  auto store_out = [&](const WUnit& t) {
    const int M = SEGF(t.sg, M), N = SEGF(t.sg, N), M1 = SEGF(t.sg, M1);
    const int rw = t.m0 + 64 * wm, cw = t.n0 + 64 * wn;  // rw: row within the half
    const bool inside = rw < (t.half ? M - M1 : M1) && cw < N;
    float* base;
    int64_t ld;
    if (t.nsplit > 1) {
      const int slot = slots_before(t.sg, t.g) + t.split_idx;
      base = SEGF(t.sg, part) + (static_cast<int64_t>(slot) * M + (t.half ? M1 : 0) + rw) * N + cw;
      ld = N;
    } else {
      base = static_cast<float*>(t.half ? SEGF(t.sg, c2) : SEGF(t.sg, c)) +
             static_cast<int64_t>(t.g) * SEGF(t.sg, c_gstride) + static_cast<int64_t>(rw) * SEGF(t.sg, ldc) + cw;
      ld = SEGF(t.sg, ldc);
    }
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        inside ? base : SEGF(t.sg, part), static_cast<short>(0), inside ? static_cast<int>(64 * ld * 4) : 0,
        kWgRsrcFlags);
    if (t.nsplit > 1) {
      // partial sums: read back by wgrad_reduce_kernel, kept in L2
      MOE_FOR(h, 2, {
        MOE_FOR(it, 8, {
          const int off = static_cast<int>(((32 * h + 4 * it + lrow) * ld + lcol) * 4);
          __builtin_amdgcn_raw_buffer_store_b128(outv[h][it], rs, off, 0, 0);
        })
      })
    } else {
      // final gradients: streamed past L2, which keeps the operands
      MOE_FOR(h, 2, {
        MOE_FOR(it, 8, {
          const int off = static_cast<int>(((32 * h + 4 * it + lrow) * ld + lcol) * 4);
          __builtin_amdgcn_raw_buffer_store_b128(outv[h][it], rs, off, 0, kWgNT);
        })
      })
    }
  };

  int u = u_lo + static_cast<int>(blockIdx.x) / kXcds;
  if (u >= u_hi) return;  // nothing issued yet
  WUnit cur = decode(u);
  issue(cur, 0, 0, false);
  issue(cur, 1, 1, cur.nk < 2);
  bool first = true;  // no stores issued yet
  int gs = 0;         // stage of the unit's step 0
  for (;;) {
    const int un = u + per_xcd;
    const bool have_next = un < u_hi;
    WUnit nxt = cur;
    if (have_next) nxt = decode(un);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    for (int kt = 0; kt < cur.nk; ++kt) {
      const int st = (gs + kt) & 1;
      if (kt == 0) {
        // a unit of one step overwrites the stage of the empty step 1 below:
        // that DMA too must have landed
        if (cur.nk == 1) {
          if (first) vm_wait<0>();
          else vm_wait<kWgStores>();
        } else {
          if (first) vm_wait<kWgStep>();
          else vm_wait<kWgStep + kWgStores>();
        }
      } else if (kt == 1) {
        if (first) vm_wait<0>();
        else vm_wait<kWgStores>();
      } else {
        vm_wait<0>();
      }
      lds_barrier();  // every wave's DMA of this step has landed; the other stage is free
      if (kt > 0 || cur.nk == 1) {
        if (kt + 1 < cur.nk) issue(cur, kt + 1, st ^ 1, false);
        else issue(nxt, 0, st ^ 1, !have_next);
      }
      compute(st);
    }
    const int st_last = (gs + cur.nk - 1) & 1;
    lds_barrier();  // every wave is done with the last step's stage
    stage_out(st_last);
    lds_barrier();  // ... and with its staged outputs
    issue(nxt, 1, st_last, !have_next || nxt.nk < 2);
    store_out(cur);
    if (!have_next) break;
    gs = (gs + cur.nk) & 1;
    cur = nxt;
    u = un;
    first = false;
  }
  vm_wait<0>();  // no DMA left in flight into LDS
}

// Sum of a split group's partial sums, in split order, into the weight
// gradient.  blockIdx.y = group over both segments, x strides over M x N.
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(BwdGemmArgs a) {
  __shared__ int before_s;
  const int G0 = a.seg[0].groups;
  const int gg = blockIdx.y;
  const int sg = gg >= G0 ? 1 : 0;
  const int g = gg - (sg ? G0 : 0);
  const int split = SEGF(sg, split);
  const int R = seg_group_rows(a, sg, g);
  const int ns = split > 0 ? std::max(1, cdiv(R, split)) : 1;
  if (ns <= 1) return;  // written by the GEMM itself
  if (threadIdx.x < 64) {
    int before = 0;  // slots of the segment's groups before g
    for (int h = threadIdx.x; h < g; h += 64) {
      const int n = std::max(1, cdiv(seg_group_rows(a, sg, h), split));
      before += n > 1 ? n : 0;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) before += __shfl_xor(before, o, 64);
    if (threadIdx.x == 0) before_s = before;
  }
  __syncthreads();
  const int M = SEGF(sg, M), N = SEGF(sg, N), M1 = SEGF(sg, M1);
  const int64_t MN = static_cast<int64_t>(M) * N;
  const float* part = SEGF(sg, part) + static_cast<int64_t>(before_s) * MN;
  float* c = static_cast<float*>(SEGF(sg, c));
  float* c2 = static_cast<float*>(SEGF(sg, c2));
  const int64_t ldc = SEGF(sg, ldc), cgs = SEGF(sg, c_gstride);
  for (int64_t e = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4; e < MN;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x * 4) {
    float4 s = *reinterpret_cast<const float4*>(part + e);
    for (int p = 1; p < ns; ++p) {
      const float4 t = *reinterpret_cast<const float4*>(part + p * MN + e);
      s.x += t.x;
      s.y += t.y;
      s.z += t.z;
      s.w += t.w;
    }
    const int m = static_cast<int>(e / N), n = static_cast<int>(e % N);
    float* dst = (m < M1 ? c + static_cast<int64_t>(m) * ldc : c2 + static_cast<int64_t>(m - M1) * ldc) +
                 static_cast<int64_t>(g) * cgs + n;
    *reinterpret_cast<float4*>(dst) = s;
  }
}

WgradPlan plan_wgrad(int nseg, const int64_t* total_rows, const int* groups, const int* M,
                     const int* N) {
  WgradPlan p{};
  int64_t units = 0, work = 0;
  for (int i = 0; i < nseg; ++i) {
    const int64_t tiles = static_cast<int64_t>(cdiv(M[i], kTM)) * cdiv(N[i], kTN);
    units += groups[i] * tiles;
    work += total_rows[i] * tiles;
  }
  if (units >= kSplitTarget) return p;
  int64_t split = (work + kSplitTarget - 1) / kSplitTarget;
  split = std::max<int64_t>(kMinSplit, (split + kTK - 1) / kTK * kTK);
  p.split = static_cast<int>(std::min<int64_t>(split, int64_t{1} << 30));
  for (int i = 0; i < nseg; ++i) {
    // only groups of more than `split` rows take slots, ceil(R / split) <= 2 R / split of them
    const int64_t rows = total_rows[i];
    const int64_t s = std::min(rows / p.split + groups[i], 2 * rows / p.split);
    p.slots[i] = rows > p.split ? s : 0;
    p.part_floats += p.slots[i] * M[i] * N[i];
  }
  return p;
}

hipError_t launch_bwd_gemm(const BwdGemmArgs& a, int kind, hipStream_t s) {
  int grid = 2 * device_cus();
  grid = (grid / kXcds) * kXcds;
  if (grid <= 0) grid = kXcds;
  const dim3 gd(grid), bd(kTh);
  switch (kind) {
    case kBwdDgradKM:
      hipLaunchKernelGGL(bwd_gemm_kernel<kBwdDgradKM>, gd, bd, 0, s, a);
      break;
    case kBwdWgrad: {
      hipLaunchKernelGGL(wgrad_kernel, gd, dim3(kWgThreads), 0, s, a);
      bool split = false;
      int groups = 0;
      int64_t mn = 0;
      for (int i = 0; i < a.nseg; ++i) {
        split = split || a.seg[i].split > 0;
        groups += a.seg[i].groups;
        mn = std::max<int64_t>(mn, static_cast<int64_t>(a.seg[i].M) * a.seg[i].N);
      }
      if (split) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t bx = std::min<int64_t>((mn / 4 + 255) / 256, 64);
        hipLaunchKernelGGL(wgrad_reduce_kernel, dim3(static_cast<unsigned>(bx), groups), dim3(256), 0, s, a);
      }
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
