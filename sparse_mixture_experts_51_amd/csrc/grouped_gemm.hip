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
// m-tile minor.  The grid is persistent; XCD x (blocks b = x mod 8) works
// through the x-th eighth of the units in order, so the A rows and weights of
// one expert stay in that XCD's L2.  Every block rebuilds the unit table from
// offsets[] (no host round trip).
//
// Four tile configurations:
//   kStream  BM = 192, BW = 256, 8 MFMA waves plus 4 loader waves, 1
//            block/CU.  For weight-streaming shapes (about 64 to 256 rows per
//            expert, weights far beyond the caches): one unit covers all rows
//            of a typical expert, so each weight byte is read from HBM once
//            (two m-tiles streaming the same weights drift apart and both
//            miss L2).  Weight tiles go from memory straight to LDS (three
//            stages) with the non-temporal hint, as nothing else in the launch
//            reads them.  The loader waves issue every tile load: under a full
//            memory queue a load instruction waits to issue, and a wave that
//            also runs MFMAs would hold them back meanwhile.
//   kCompute BM = BW = 128, 4 waves, 2 blocks/CU.  For few rows per expert
//            (decode) and small models: more, smaller units keep every CU
//            busy and two blocks per CU keep more weight bytes in flight.
//            Weight loads carry the non-temporal hint (decode reads 6.6 TB/s
//            with it, 6.0 TB/s without).
//   kBig     BM = 256, BW = 128, 8 waves, 1 block/CU, A and weight tiles both
//            by LDS DMA in three stages.  For hundreds of rows per expert.
//   kBigL    kBig plus 4 loader waves that issue the DMA, so the MFMA waves
//            read fragments with plain LDS loads the compiler schedules.  For
//            long K: the shared expert when the routed experts stream (it then
//            runs as a launch of its own; 10% faster than kBig there) and
//            groups of hundreds of rows at d = 7168 (4% faster); no gain on
//            the mini model's six K-steps per unit.
//
// Pipeline.  A block's units run as an outer loop; each unit's K-loop (64 of
// K per step; with register-staged A an odd step count is padded by one
// MFMA-free step) is straight-line code apart from uniform branches.  The
// fetcher runs two steps ahead of the MFMAs and crosses into the next unit
// during the last steps of the current one, choosing the source with scalar
// selects.  Loads are buffer loads (uniform descriptor + 32-bit offset); in
// the tiles without loader waves the loads of one step are spread over the
// four MFMA sub-steps of the step two earlier, so that a full memory queue
// stalls one wave briefly instead of holding all its MFMAs back.  Tiles sit in XOR-swizzled LDS buffers.
// Barriers are raw s_barrier after an LDS-only wait: __syncthreads() would
// also drain the in-flight global loads.  The epilogue stages the output
// tile in the LDS buffers no load in flight writes and leaves it as 16-byte
// non-temporal row stores.
#include "common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace moe {

constexpr int kBK = 64;                      // K per step
constexpr int kChunksPerRow = kBK / 8;       // 16-byte chunks per tile row
constexpr int kMaxGroups = 1025;
// Cache-policy operand of the buffer-load builtins on gfx950: bit 1 is the
// non-temporal hint (the `nt` modifier of buffer_load).
constexpr int kCachePolicyNT = 2;

template <int BM_, int BW_, int WM_, int WN_, int BPC_, bool DMAB_, bool DMAA_ = false,
          int NSA_ = 2, int PW_ = 0>
struct TileCfg {
  static constexpr int BM = BM_;     // rows per unit
  static constexpr int BW = BW_;     // weight rows per unit
  static constexpr int WM = WM_;     // waves along M
  static constexpr int WN = WN_;     // waves along the weight tile
  static constexpr int BPC = BPC_;   // blocks per CU
  static constexpr bool DMAB = DMAB_;  // weight tiles go from memory straight to LDS
  static constexpr bool DMAA = DMAA_;  // A tiles too (then two stages, one step ahead)
  static constexpr int NSA = DMAA ? NSA_ : 2;          // LDS buffers (stages) of the A tile
  static constexpr int NSB = DMAA ? NSA : (DMAB ? 3 : 2);  // ... and of the weight tile
  static constexpr int PW = PW_;     // loader waves (0: the MFMA waves load their own tiles)
  static constexpr int kThreads = 64 * WM * WN;        // MFMA threads
  static constexpr int kAllThreads = kThreads + 64 * PW;
  static constexpr int kLoaders = PW > 0 ? 64 * PW : kThreads;  // threads that issue tile loads
  static constexpr int kRowsPerPass = kLoaders / kChunksPerRow;
  static constexpr int kLoadsA = BM / kRowsPerPass;
  static constexpr int kLoadsB = BW / kRowsPerPass;
  static constexpr int TM = BM / WM / 32;  // 32-row MFMA tiles per wave
  static constexpr int TN = BW / WN / 32;  // 32-column MFMA tiles per wave
  static_assert(BM % kRowsPerPass == 0 && BW % (2 * kRowsPerPass) == 0, "load passes");
  static_assert(TN % 2 == 0, "SwiGLU pairs gate and up tiles inside a wave");
  static_assert(!DMAA || (DMAB && TM % 2 == 0), "A by DMA implies weights by DMA");
  static_assert(PW == 0 || DMAB, "loader waves: weights by DMA");
};
using kStream = TileCfg<192, 256, 2, 4, 1, true, false, 2, 4>;
using kCompute = TileCfg<128, 128, 2, 2, 2, false>;
using kBig = TileCfg<256, 128, 4, 2, 1, true, true, 3>;
using kBigL = TileCfg<256, 128, 4, 2, 1, true, true, 3, 4>;  // kBig with loader waves

// XOR swizzle of the 16-byte chunks of a 128-byte row.  gfx950's LDS has 64
// four-byte banks (256 bytes per clock), so a 16-byte-per-lane access is
// served 16 lanes at a time.  An MFMA fragment read has those 16 lanes on 16
// consecutive rows at one logical chunk: rows 2j and 2j+1 fall in different
// 128-byte halves of a bank line, and XOR with (row / 2) mod 8 spreads the 8
// row pairs over the 8 chunks.  The stores (8 lanes per row, 2 rows per 16
// lanes) stay conflict-free too.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kChunksPerRow + (chunk ^ ((row >> 1) & (kChunksPerRow - 1)));
}

// Two MFMA fragments of a K-major tile (rows of K, 512 bytes apart), read
// transposed by ds_read_b64_tr_b16: within each 16 lanes, lane s names 4
// values of row s / 4 and receives 4 consecutive rows of one column, so a
// fragment's 8 values of K are two reads, the second 4 rows further.
// Complete on return (the wait is in the asm).
typedef short v4i16 __attribute__((ext_vector_type(4)));
template <int kOff>
__device__ __forceinline__ void tr_read2(unsigned a0, unsigned a1, bf16x8& f0, bf16x8& f1) {
  v4i16 r[4];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
      "ds_read_b64_tr_b16 %2, %5 offset:%6\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a0), "v"(a1), "i"(kOff), "i"(kOff + 4 * 512)
      : "memory");
  f0 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r[0], r[1], 0, 1, 2, 3, 4, 5, 6, 7));
  f1 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r[2], r[3], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Wave-uniform description of one unit (held in scalar registers).
struct Unit {
  int g;           // group (E = shared)
  int valid_rows;  // rows of this m-tile that exist
  int n0;          // first output column
  int K, N, nk;
  int nk1;         // K-major weights: K-steps of the first part (A, W; then A2, W3)
  int orow0;       // output row of the tile's first row
  int routed;      // 1: routed expert group, 0: shared expert
};

template <class C, bool kSwiGLU, bool kWKM = false>
__device__ __forceinline__ Unit decode_unit(const GroupedGemmArgs& a, const int* unit_start,
                                            const int* offs, int ngroups, int u) {
  // The group is the last one whose first unit is <= u (unit_start does not
  // decrease): the lanes of the wave test 64 groups at a time and count the
  // hits, so the LDS reads are independent instead of a binary search chain.
  const int lane = threadIdx.x & 63;
  int below = 0;
  for (int base = 0; base < ngroups; base += 64) {
    const int g = base + lane;
    const bool hit = g < ngroups && unit_start[g] <= u;
    below += __popcll(__ballot(hit));
  }
  Unit r;
  r.g = uni(below - 1);
  r.routed = r.g < a.E;
  const int grow0 = r.routed ? uni(offs[r.g]) : 0;
  const int rows = r.routed ? uni(offs[r.g + 1]) - grow0 : static_cast<int>(a.T);
  const int mt = (rows + C::BM - 1) / C::BM;
  const int local = u - uni(unit_start[r.g]);
  // Units run n-tile major, m-tile minor, so the units an XCD runs together
  // share a weight tile across m-tiles and an A tile across n-tiles.  A group
  // of very many m-tiles (the shared expert over tens of thousands of tokens,
  // whose x no longer fits the MALL) is walked in panels of kPanel m-tiles:
  // otherwise the XCD's concurrent units would be m-tiles of one n-tile, and
  // every A tile would come from HBM again for each of the group's n-tiles
  // (V3 layer at 32768 tokens: FFN 29.6 -> 28.9 ms; with panels from 8
  // m-tiles on, no gain at 4096 tokens and the mini model a little slower).
  constexpr int kPanel = 4;
  int n_tile, m_tile;
  if (mt >= 64) {
    constexpr int cols = kSwiGLU ? C::BW / 2 : C::BW;
    const int nt = ((r.routed ? a.N_r : a.N_s) + cols - 1) / cols;
    const int full = mt / kPanel;  // whole panels; the last one holds mt % kPanel m-tiles
    const int panel = local / (kPanel * nt);
    const int h = panel < full ? kPanel : mt - full * kPanel;
    const int within = local - panel * kPanel * nt;
    n_tile = within / h;
    m_tile = panel * kPanel + within % h;
  } else {
    n_tile = local / mt;
    m_tile = local % mt;
  }
  const int m0 = m_tile * C::BM;
  r.valid_rows = uni((rows - m0) < C::BM ? (rows - m0) : C::BM);
  r.K = r.routed ? a.K_r : a.K_s;
  r.N = r.routed ? a.N_r : a.N_s;
  r.nk = r.K / kBK;
  if constexpr (kWKM) {
    r.nk1 = r.nk;
    r.nk += a.K2_r / kBK;  // routed groups only
  }
  r.n0 = n_tile * (kSwiGLU ? C::BW / 2 : C::BW);
  r.orow0 = uni(grow0 + m0);
  return r;
}

template <class C, bool kSwiGLU, bool kBwd = false, bool kWKM = false>
__global__ __launch_bounds__(C::kAllThreads, C::BPC) void grouped_gemm_kernel(GroupedGemmArgs a) {
  static_assert(!kBwd || kSwiGLU, "the backward epilogue is the SwiGLU stage's");
  // K-major weights: the streaming tile's plain-output form only
  static_assert(!kWKM || (!kSwiGLU && C::PW > 0 && C::DMAB && !C::DMAA), "K-major weights");
  constexpr int kThreads = C::kThreads, RPP = C::kRowsPerPass;
  constexpr int LA = C::kLoadsA, LB = C::kLoadsB, TM = C::TM, TN = C::TN;
  __shared__ u32x4 lds_a[C::NSA][C::BM * kChunksPerRow];  // buffers or DMA stages
  __shared__ u32x4 lds_b[C::NSB][C::BW * kChunksPerRow];
  __shared__ int unit_start[kMaxGroups + 1];
  __shared__ int offs[kMaxGroups + 1];  // copy of offsets[0..E]
  __shared__ int wsum[C::kAllThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uni(tid >> 6);  // wave-uniform, so tile choices stay scalar
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int E = a.E;
  const bool has_shared = a.w_shared != nullptr;
  const int ngroups = E + (has_shared ? 1 : 0);
  constexpr int cols_per_tile = kSwiGLU ? C::BW / 2 : C::BW;

  // ---- unit table: units of group g start at unit_start[g]
  {
    constexpr int kPer = (kMaxGroups + C::kAllThreads - 1) / C::kAllThreads;
    const int per = (ngroups + C::kAllThreads - 1) / C::kAllThreads;
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
    int run = block_scan<C::kAllThreads>(sum, &total, wsum);
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
  // XCD x (blocks b with b % 8 == x) takes the x-th eighth of the units in
  // order: a group's units share its rows and weights in that XCD's L2
  const int G = gridDim.x / kXcds;
  const int ux = blockIdx.x % kXcds;
  const int uend = static_cast<int>(static_cast<int64_t>(total_units) * (ux + 1) / kXcds);
  const int ustart = static_cast<int>(static_cast<int64_t>(total_units) * ux / kXcds);
  const int lb = ustart + blockIdx.x / kXcds;
  if (lb >= uend) return;
  // Unit order.  Static: a block runs lb, lb + G, lb + 2G, ...  Dynamic (the
  // loader-wave all-DMA tile given counters, in launches of at least 64
  // units per block): the first two units are the static ones, every later
  // one is claimed from the XCD's counter, so the units an XCD runs at any
  // time stay a window of consecutive units.  In the static order, blocks
  // that share a weight or A tile drift apart over a long launch: in the V3
  // layer at 32768 tokens (160 SwiGLU units per block) the blocks that share
  // a weight tile started a median 540 us apart, four units, and 40 us apart
  // with the claims (FFN 29.2 -> 27.7 ms).  With about 20 units per block
  // (1024 rows per expert over 4096 tokens) the static order keeps them
  // 25 us apart and its fixed m-tile per block does better than the claims
  // (FFN 3.25 vs 3.43 ms).  Thread 0 claims the unit of iteration i + 3 at
  // the start of iteration i and publishes it in useq after that iteration's
  // K-loop; the epilogue's barriers make it visible before any wave reads it.
  constexpr int kEnd = 0x7FFFFFFF;
  constexpr bool kDynTile = C::PW > 0 && C::DMAA;
  const bool dyn = kDynTile && a.unit_counter != nullptr &&
                   total_units >= 64 * static_cast<int64_t>(gridDim.x);
  __shared__ int useq[4];
  // (useq is accessed in asm: the compiler would otherwise wait for every LDS
  // DMA in flight before a plain access)
  auto publish = [&](int i, int claim) __attribute__((always_inline)) {
    const int64_t u = static_cast<int64_t>(ustart) + 2 * static_cast<int64_t>(G) + claim;
    lds_write_b32(&useq[i & 3], u < uend ? static_cast<int>(u) : kEnd);
  };
  auto unit_at = [&](int i) __attribute__((always_inline)) {  // the block's i-th unit or kEnd
    if (i == 0) return lb;
    if (!dyn || i == 1) {
      const int64_t u = lb + static_cast<int64_t>(i) * G;
      return u < uend ? static_cast<int>(u) : kEnd;
    }
    return uni(lds_read_b32(&useq[i & 3]));
  };
  if (dyn && tid == 0) publish(2, atomicAdd(a.unit_counter + ux, 1));
  auto decode = [&](int u) __attribute__((always_inline)) {
    return decode_unit<C, kSwiGLU, kWKM>(a, unit_start, offs, ngroups, u);
  };

  // loader thread geometry (the loader waves follow the MFMA waves)
  const bool loader = C::PW == 0 || wave >= C::WM * C::WN;
  const int ltid = C::PW > 0 ? tid - kThreads : tid;
  const int lwave = C::PW > 0 ? wave - C::WM * C::WN : wave;
  const int ld_row = ltid / kChunksPerRow;  // 0..RPP-1
  const int ld_chunk = ltid % kChunksPerRow;

  // ---- source of a unit: buffer descriptors (wave-uniform, scalar
  // registers) plus 32-bit byte offsets.  An A row (a gathered token) needs a
  // per-thread offset per load pass; a weight row is a uniform row base (the
  // scalar offset of the load) plus one per-thread term.  Every load is
  // unconditional: an A row past the tile's valid rows gets an offset beyond
  // the descriptor's range, which returns zeros without a memory access, and
  // columns past the edge give results the epilogue never stores.  perm_src
  // entries are loaded a unit ahead (pend_map) and copied to map_ready during
  // the first K-step of the current unit, where the compiler's wait for them
  // counts exactly the loads issued since; at the unit switch, where its count
  // would have to cover every K-loop trip, it would drain the prefetched
  // tiles of the next unit.
  struct Src {
    __amdgpu_buffer_rsrc_t ra, rb0, rb1;  // A rows; W1 (or W2) rows; W3 rows
    __amdgpu_buffer_rsrc_t ra2;           // K-major weights: A rows of the second part
    int nk1;                              // ... and the K-steps of the first part
    int wkm_step;                         // ... and the bytes of one step's 64 rows of K
    int a_off[LA];                        // per thread, bytes (kOutOfRange: no row)
    int b_row[LB];                        // uniform, bytes: weight row base of each pass
    int b_thr;                            // per thread, bytes
    int rot;                              // K-step the unit starts at (down stage of the streaming tile)
    int nk;                               // K-steps with data
    int rows;                             // valid A rows of the unit
  };
  // Above any descriptor range (ranges are clamped to 2^31 - 1 bytes); offsets
  // are advanced in unsigned arithmetic, so they stay out of range.
  constexpr unsigned kOutOfRange = 0x80000000u;
  // Down stage of the streaming tile: each unit starts its K loop at its own
  // step (and wraps round), so that units running together read different
  // column offsets of their 4 KB weight rows (prefill down stage 1553 ->
  // 1520 us; rotating the SwiGLU stage's 14 KB rows gained nothing).  The
  // sums run in another order, so y differs from the unrotated kernel's in
  // rounding.
  constexpr bool kRotK = !kSwiGLU && C::PW > 0 && !C::DMAA;
  int pend_row[LA];  // prepared unit: group row / token per thread row
  int pend_map[LA];   // prepared unit: perm_src[pend_row] when gathering (in flight)
  int map_ready[LA];  // the same values once landed (see settle)
  Unit pend;
  auto prepare_into = [&](int u, Unit& pu, int (&prow)[LA], int (&pmap)[LA])
      __attribute__((always_inline)) {
    pu = decode(u);
    const bool gather = pu.routed && a.a_row_map;
    MOE_FOR(i, LA, {
      int r = ld_row + RPP * i;
      if (r >= pu.valid_rows) r = 0;  // a row that exists; its offset is replaced below
      prow[i] = pu.orow0 + r;
      // branch-free, so the loaded value is not touched until the unit switch
      const int32_t* src = gather ? a.a_row_map + prow[i] : a.offsets;
      pmap[i] = *src;
    })
  };
  auto prepare = [&](int u) __attribute__((always_inline)) {
    prepare_into(u, pend, pend_row, pend_map);
  };
  // The empty asm makes each value a new one defined here, so the compiler
  // waits for the load at this point and cannot fold the copy away.
  auto settle_into = [&](const int (&pmap)[LA], int (&ready)[LA]) __attribute__((always_inline)) {
    MOE_FOR(i, LA, {
      int v = pmap[i];
      asm volatile("" : "+v"(v));
      ready[i] = v;
    })
  };
  auto settle = [&]() __attribute__((always_inline)) { settle_into(pend_map, map_ready); };
  constexpr int kRsrcFlags = 0x00020000;  // raw (untyped) buffer
  auto rsrc = [](const void* base, int64_t bytes) __attribute__((always_inline)) {
    const int n = bytes < 0x7FFFFFFF ? static_cast<int>(bytes) : 0x7FFFFFFF;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n,
                                             kRsrcFlags);
  };
  auto source_of = [&](const Unit& pu, const int (&prow)[LA], const int (&ready)[LA])
      __attribute__((always_inline)) {
    Src sr;
    const bool routed = pu.routed;
    const int K = pu.K, N = pu.N, g = pu.g, n0 = pu.n0;
    const bool gather = routed && a.a_row_map;
    // Rows that are not gathered are the unit's own consecutive rows of A:
    // their descriptor starts at the unit's first row, so the 32-bit offsets
    // stay within one tile however large the buffer is.  Gathered rows are
    // token rows of x, addressed from x itself.
    const int64_t a_row0 = gather ? 0 : pu.orow0;
    const uint16_t* a_base = (routed ? a.a_routed : a.a_shared) + a_row0 * K;
    const int64_t a_bytes = gather ? a.a_routed_bytes : static_cast<int64_t>(pu.valid_rows) * K * 2;
    sr.ra = rsrc(a_base, a_bytes);
    const int64_t wbytes = static_cast<int64_t>(N) * K * 2;
    const uint16_t* w0 = routed ? a.w_routed + static_cast<int64_t>(g) * N * K : a.w_shared;
    const uint16_t* w1 =
        kSwiGLU ? (routed ? a.w3_routed + static_cast<int64_t>(g) * N * K : a.w3_shared) : w0;
    sr.rb0 = rsrc(w0, wbytes);
    sr.rb1 = rsrc(w1, wbytes);
    if constexpr (kWKM) {
      // [K, N] per group; the second part [K2, N] from w3_routed and a2_routed
      const int K2 = a.K2_r;
      sr.rb1 = rsrc(K2 > 0 ? a.w3_routed + static_cast<int64_t>(g) * N * K2 : w0,
                    static_cast<int64_t>(N) * (K2 > 0 ? K2 : K) * 2);
      // the second part's rows: the same rows of a2_routed (row stride K too)
      sr.ra2 = K2 > 0 ? rsrc(a.a2_routed + a_row0 * K, a_bytes) : sr.ra;
      sr.nk1 = pu.nk1;
      sr.wkm_step = kBK * N * 2;
    }
    // A by DMA: lane l writes physical chunk l % 8 of its row, so it loads the
    // logical chunk the swizzle puts there (as for the weights below).
    const int a_chunk = C::DMAA ? (ld_chunk ^ ((ld_row >> 1) & (kChunksPerRow - 1))) : ld_chunk;
    MOE_FOR(i, LA, {
      int row = gather ? ready[i] : prow[i] - pu.orow0;
      if (gather && (row < 0 || row >= a.T)) row = 0;  // malformed permutation: stay in bounds
      sr.a_off[i] = ld_row + RPP * i < pu.valid_rows ? (row * K + a_chunk * 8) * 2
                                                     : static_cast<int>(kOutOfRange);
    })
    sr.rows = pu.valid_rows;
    // weight tile: SwiGLU stage rows [0, BW/2) = W1[n0..], [BW/2, BW) = W3[n0..]
    // (each load pass lies in one half, so one descriptor per pass); down
    // stage rows [0, BW) = W2[n0..]
    if constexpr (kWKM) {
      // The stage holds the step's 64 rows of K x BW columns, 512 bytes per
      // row of K, the row's 64-byte pieces p stored at p ^ (row & 3) (within
      // each half row), which the transposing fragment reads need to meet
      // every bank once.  Pass i of loader wave w is LDS block 4 i + w (1 KB):
      // rows of K 2 (4 i + w) and + 1, lane l at row + (l >> 5), stored
      // 16-byte chunk l & 31.  Pass offsets (uniform) go in the scalar offset.
      const int kq = (2 * lwave + (lane >> 5)) & 3;  // that row & 3
      const int sp = (lane & 31) >> 2;
      const int col = 8 * (((sp ^ kq) << 2) | (lane & 3));
      MOE_FOR(i, LB, { sr.b_row[i] = uni(2 * (4 * i + lwave) * N * 2); })
      sr.b_thr = ((lane >> 5) * N + n0 + col) * 2;
    } else {
      MOE_FOR(i, LB, {
        constexpr int t0 = RPP * i;
        int wrow = kSwiGLU ? n0 + t0 % (C::BW / 2) : n0 + t0;
        if (wrow >= N) wrow = 0;
        sr.b_row[i] = uni(wrow * K * 2);
      })
      // Register path: thread (ld_row, ld_chunk) loads that logical chunk and
      // stores it swizzled.  DMA path: lane l of a wave writes physical slot
      // l % 8 of row ld_row (8 rows per wave and pass), so it loads the logical
      // chunk that the swizzle puts there (pass offsets are multiples of 64 rows
      // and leave the swizzle unchanged).
      const int b_chunk = C::DMAB ? (ld_chunk ^ ((ld_row >> 1) & (kChunksPerRow - 1))) : ld_chunk;
      sr.b_thr = (ld_row * K + b_chunk * 8) * 2;
    }
    sr.nk = pu.nk;
    sr.rot = kRotK ? (pu.n0 / C::BW + 3 * pu.g) % pu.nk : 0;
    return sr;
  };
  auto source_of_pending = [&]() __attribute__((always_inline)) {
    return source_of(pend, pend_row, map_ready);
  };

  // A K-step in flight: A rows in registers (and the weight rows too unless
  // they go straight to LDS).
  struct Slice {
    u32x4 a[C::DMAA ? 1 : LA], b[C::DMAB ? 1 : LB];
    int rows;  // valid A rows of the unit the slice belongs to (uniform)
  };
  // Loads K-step f of the current source (f < steps0) or step f - steps0 of
  // the next one, chosen by a uniform test (scalar selects, no branches, so
  // the K-loop stays straight-line).  A step at or past nk (the padding step
  // of an odd count) reloads the last slice and is never multiplied.  With
  // part P in 0..3 only loads i (A passes first, then weight passes) with
  // i % 4 == P are issued, so that a step's loads can be spread over the four
  // MFMA sub-steps; P < 0 issues them all.
  auto load2 = [&](Slice& sl, const Src& c0, const Src& c1, int steps0, int f, int bstage,
                   auto part_c) __attribute__((always_inline)) {
    constexpr int P = decltype(part_c)::value;
    const bool nxt = f >= steps0;
    const int j = nxt ? f - steps0 : f;
    const int nk = nxt ? c1.nk : c0.nk;
    int kj = (j < nk ? j : nk - 1) + (nxt ? c1.rot : c0.rot);
    if (kj >= nk) kj -= nk;
    int kb = kj * (kBK * 2);
    __amdgpu_buffer_rsrc_t ra = nxt ? c1.ra : c0.ra;
    __amdgpu_buffer_rsrc_t rb0 = nxt ? c1.rb0 : c0.rb0;
    const __amdgpu_buffer_rsrc_t rb1 = nxt ? c1.rb1 : c0.rb1;
    int bt = (nxt ? c1.b_thr : c0.b_thr) + kb;
    int bk = 0;  // K-major weights: the step's rows of K, in the scalar offset
    if constexpr (kWKM) {
      const int nk1 = nxt ? c1.nk1 : c0.nk1;
      const bool second = kj >= nk1;
      const int kp = second ? kj - nk1 : kj;  // step within its part
      kb = kp * (kBK * 2);
      ra = second ? (nxt ? c1.ra2 : c0.ra2) : ra;
      rb0 = second ? rb1 : rb0;
      bt = nxt ? c1.b_thr : c0.b_thr;
      bk = kp * (nxt ? c1.wkm_step : c0.wkm_step);
    }
    sl.rows = nxt ? c1.rows : c0.rows;
    if constexpr (!C::DMAA) {
      MOE_FOR(i, LA, {
        if constexpr (P < 0 || i % 4 == P) {
          const unsigned ao = static_cast<unsigned>(nxt ? c1.a_off[i] : c0.a_off[i]) + kb;
          sl.a[i] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, static_cast<int>(ao), 0, 0));
        }
      })
    }
    MOE_FOR(i, LB, {
      if constexpr (P >= 0 && (LA + i) % 4 != P) return;
      constexpr bool up = kSwiGLU && RPP * i >= C::BW / 2;
      const int br = nxt ? c1.b_row[i] : c0.b_row[i];
      if constexpr (C::DMAB) {
        // 64 lanes x 16 bytes land at consecutive LDS slots: rows
        // RPP*i + 8*wave .. +8 of the stage.  Non-temporal: this path
        // streams weights that no other unit of the launch reads (prefill
        // FFN 4.71 -> 4.57 ms, bit-identical); the all-DMA tiles, whose
        // weights later m-tiles read again from L2, keep the default.
        dma_b128<kCachePolicyNT>(up ? rb1 : rb0, &lds_b[bstage][(RPP * i + 8 * lwave) * kChunksPerRow], bt,
                                 br + bk);
      } else {
        // non-temporal: each weight byte is read once per unit and never
        // again in the launch (decode FFN 3.19 -> 2.88 ms, bit-identical)
        sl.b[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(up ? rb1 : rb0, bt, br, kCachePolicyNT));
      }
    })
  };
  auto stash = [&](const Slice& sl, int buf, int bstage) __attribute__((always_inline)) {
    // A passes wholly past the valid rows are not stored.  A pass spans whole
    // 32-row MFMA tiles, so every tile the MFMAs read was stored from this
    // unit (rows past the valid ones as zeros) and the others are skipped.
    if constexpr (!C::DMAA) {
      MOE_FOR(i, LA, {
        if (RPP * i < sl.rows) lds_a[buf][swz(ld_row + RPP * i, ld_chunk)] = sl.a[i];
      })
    }
    if constexpr (!C::DMAB) {
      MOE_FOR(i, LB, { lds_b[bstage][swz(ld_row + RPP * i, ld_chunk)] = sl.b[i]; })
    }
  };

  // Accumulators: acc[tm][tn] pairs token rows tile_row(tm) .. +31 with
  // weight-tile rows (output columns) -- SwiGLU: tn < TN/2 gate rows
  // wn*HC + 32*tn, tn >= TN/2 the up rows of the same h columns (BW/2
  // further); down: rows wn*BW/WN + 32*tn.
  constexpr int HC = C::BW / 2 / C::WN;  // h columns per wave (SwiGLU)
  f32x16 acc[TM][TN];
  auto zero_acc = [&]() __attribute__((always_inline)) {
    MOE_FOR(i, TM, { MOE_FOR(j, TN, { acc[i][j] = f32x16{}; }) })
  };
  // 32-row MFMA tiles are dealt to the WM wave rows in turn (tile i of wave
  // row wm starts at row 32 * (wm + WM * i)), so a unit with fewer valid rows
  // than BM still spreads its MFMAs over every wave instead of leaving the
  // waves of the last rows idle at the barrier.
  auto tile_row = [&](int i) __attribute__((always_inline)) { return 32 * (wm + C::WM * i); };
  // tiles of this wave that hold valid rows (0..TM)
  auto valid_tiles = [&](int valid_rows) __attribute__((always_inline)) {
    const int m = ((valid_rows + 31) / 32 - wm + C::WM - 1) / C::WM;
    return m < 0 ? 0 : (m > TM ? TM : m);
  };
  auto brow = [&](int tn) __attribute__((always_inline)) {
    if (kSwiGLU)
      return tn < TN / 2 ? wn * HC + 32 * tn : C::BW / 2 + wn * HC + 32 * (tn - TN / 2);
    return wn * (C::BW / C::WN) + 32 * tn;
  };

  // after(integral_constant<int, ks>) runs after the MFMAs of sub-step ks
  // (also when the wave has no valid tiles).
  auto mma = [&](int buf, int bstage, int mrows, auto&& after) __attribute__((always_inline)) {
    // mrows: 32-row tiles of this wave that hold valid rows (0..TM)
    MOE_FOR(ks, kBK / 16, {
     if (mrows > 0) {
      const int ch = 2 * ks + (lane >> 5);
      const int fr = lane & 31;
      bf16x8 af[TM], bfr[TN];
      MOE_FOR(i, TM, {
        if (i < mrows)
          af[i] = __builtin_bit_cast(bf16x8, lds_a[buf][swz(tile_row(i) + fr, ch)]);
      })
      if constexpr (kWKM) {
        // K-major weight stage (see source_of): fragment j of sub-step ks is
        // rows 16 ks .. + 15 of its 32 columns, logical piece brow(j) / 32
        const unsigned sb = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_ptr_t)&lds_b[bstage][0]));
        const unsigned base = sb + (8 * (lane >> 5) + ((lane & 15) >> 2)) * 512 +
                              (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
        const int rot = (lane & 15) >> 2;
        tr_read2<ks * 16 * 512>(base + ((((brow(0) >> 5) ^ rot)) << 6), base + ((((brow(1) >> 5) ^ rot)) << 6),
                                bfr[0], bfr[1]);
      } else if constexpr (C::DMAB) {
        // The compiler would put a full vmcnt(0) before any LDS read of a
        // buffer that DMA writes, which drains the prefetched loads; vm_wait
        // already orders these reads after the DMA, so they are issued in asm.
        static_assert(TN == 2, "two weight fragments per sub-step");
        u32x4 b0, b1;
        lds_read2_b128(&lds_b[bstage][swz(brow(0) + fr, ch)], &lds_b[bstage][swz(brow(1) + fr, ch)],
                       b0, b1);
        bfr[0] = __builtin_bit_cast(bf16x8, b0);
        bfr[1] = __builtin_bit_cast(bf16x8, b1);
      } else {
        MOE_FOR(j, TN, { bfr[j] = __builtin_bit_cast(bf16x8, lds_b[bstage][swz(brow(j) + fr, ch)]); })
      }
      MOE_FOR(i, TM, {
        if (i < mrows) {
          MOE_FOR(j, TN, {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
          })
        }
      })
     }
      after(ks_c);
      // Keep each sub-step's fragment reads next to its MFMAs: hoisting them
      // all costs registers and spills the in-flight slices.
      __builtin_amdgcn_sched_barrier(0);
    })
  };

  // All-DMA tiles: K-step f of source c (the last step again past nk) goes
  // into LDS stage `stage` -- A passes wholly past the valid rows are skipped
  // (their tiles are never multiplied) -- with the K offset in the scalar
  // offset of each load.
  // Part P (0..3, or all with P = -1) as in load2; P = kOnlyA / kOnlyB issues
  // all A / all weight passes.
  constexpr int kOnlyA = -2, kOnlyB = -3;
  auto issue = [&](const Src& c, int f, int stage, auto part_c) __attribute__((always_inline)) {
    constexpr int P = decltype(part_c)::value;
    const int kb = (f < c.nk ? f : c.nk - 1) * (kBK * 2);
    MOE_FOR(i, LA, {
      if constexpr (P == kOnlyB || (P >= 0 && i % 4 != P)) return;
      // with more than two stages the wait counts every load, so passes past
      // the valid rows are issued too (out-of-range offsets, no memory access)
      if (C::NSA > 2 || RPP * i < c.rows)
        dma_b128(c.ra, &lds_a[stage][(RPP * i + 8 * lwave) * kChunksPerRow], c.a_off[i], kb);
    })
    MOE_FOR(i, LB, {
      if constexpr (P == kOnlyA || (P >= 0 && (LA + i) % 4 != P)) return;
      constexpr bool up = kSwiGLU && RPP * i >= C::BW / 2;
      dma_b128(up ? c.rb1 : c.rb0, &lds_b[stage][(RPP * i + 8 * lwave) * kChunksPerRow], c.b_thr,
               c.b_row[i] + kb);
    })
  };
  // MFMAs on an all-DMA stage; every fragment read is in asm (see mma).
  // after(integral_constant<int, ks>) runs after the MFMAs of sub-step ks.
  auto mma_dma = [&](int stage, int mrows, auto&& after) __attribute__((always_inline)) {
    MOE_FOR(ks, kBK / 16, {
     if (mrows > 0) {
      const int ch = 2 * ks + (lane >> 5);
      const int fr = lane & 31;
      bf16x8 af[TM], bfr[TN];
      const int r0 = tile_row(0) + fr;
      constexpr int kTs = 32 * C::WM;  // row stride between a wave's tiles
      if (TM == 2 && TN == 2 && mrows == 2) {
        const u32x4* const ptr[4] = {
            &lds_a[stage][swz(r0, ch)], &lds_a[stage][swz(r0 + kTs, ch)],
            &lds_b[stage][swz(brow(0) + fr, ch)], &lds_b[stage][swz(brow(1) + fr, ch)]};
        u32x4 v[4];
        lds_read4_b128(ptr, v);
        af[0] = __builtin_bit_cast(bf16x8, v[0]);
        af[TM > 1 ? 1 : 0] = __builtin_bit_cast(bf16x8, v[1]);
        bfr[0] = __builtin_bit_cast(bf16x8, v[2]);
        bfr[1] = __builtin_bit_cast(bf16x8, v[3]);
      } else if (TM == 4 && TN == 2 && mrows == 4) {
        // the common case: all fragments under one wait
        const u32x4* const ptr[6] = {
            &lds_a[stage][swz(r0, ch)], &lds_a[stage][swz(r0 + kTs, ch)],
            &lds_a[stage][swz(r0 + 2 * kTs, ch)], &lds_a[stage][swz(r0 + 3 * kTs, ch)],
            &lds_b[stage][swz(brow(0) + fr, ch)], &lds_b[stage][swz(brow(1) + fr, ch)]};
        u32x4 v[6];
        lds_read6_b128(ptr, v);
        MOE_FOR(i, TM, { af[i] = __builtin_bit_cast(bf16x8, v[i < 4 ? i : 0]); })
        bfr[0] = __builtin_bit_cast(bf16x8, v[4]);
        bfr[1] = __builtin_bit_cast(bf16x8, v[5]);
      } else {
        u32x4 v0, v1;
        MOE_FOR(i2, TM / 2, {
          if (2 * i2 < mrows) {
            lds_read2_b128(&lds_a[stage][swz(r0 + 2 * kTs * i2, ch)],
                           &lds_a[stage][swz(r0 + 2 * kTs * i2 + kTs, ch)], v0, v1);
            af[2 * i2] = __builtin_bit_cast(bf16x8, v0);
            af[2 * i2 + 1] = __builtin_bit_cast(bf16x8, v1);
          }
        })
        lds_read2_b128(&lds_b[stage][swz(brow(0) + fr, ch)], &lds_b[stage][swz(brow(1) + fr, ch)],
                       v0, v1);
        bfr[0] = __builtin_bit_cast(bf16x8, v0);
        bfr[1] = __builtin_bit_cast(bf16x8, v1);
      }
      MOE_FOR(i, TM, {
        if (i < mrows) {
          MOE_FOR(j, TN, {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
          })
        }
      })
     }
      after(ks_c);
      __builtin_amdgcn_sched_barrier(0);
    })
  };

  // MFMA waves of loader-wave tiles issue no DMA, so their fragment reads are
  // plain LDS loads the compiler schedules freely (no drain before them).
  auto mma_plain = [&](int abuf, int bstage, int mrows) __attribute__((always_inline)) {
    MOE_FOR(ks, kBK / 16, {
      if (mrows > 0) {
        const int ch = 2 * ks + (lane >> 5);
        const int fr = lane & 31;
        bf16x8 af[TM], bfr[TN];
        MOE_FOR(i, TM, {
          if (i < mrows) af[i] = __builtin_bit_cast(bf16x8, lds_a[abuf][swz(tile_row(i) + fr, ch)]);
        })
        MOE_FOR(j, TN, { bfr[j] = __builtin_bit_cast(bf16x8, lds_b[bstage][swz(brow(j) + fr, ch)]); })
        MOE_FOR(i, TM, {
          if (i < mrows) {
            MOE_FOR(j, TN, {
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
            })
          }
        })
      }
    })
  };

  // SiLU(gate) * up in fp32 (v_rcp_f32 for the quotient).
  auto swiglu = [](float ga, float up) __attribute__((always_inline)) {
    return ga * __builtin_amdgcn_rcpf(1.0f + __expf(-ga)) * up;
  };
  // The MFMAs take the weight fragment as the first operand, so acc holds the
  // transposed tile: lane l has token row (l & 31) of its 32x32 tile and, for
  // g = 0..3, the four adjacent output columns 8g + 4(l >> 5) + 0..3 as
  // values 4g .. 4g+3.
  const int lrow = lane & 31;
  const int lcol = (lane >> 5) * 4;
  // fa, fb: the A buffer and the weight stage that no load in flight writes
  // (both free since the barrier after the unit's last K-step); mrows: the
  // wave's tiles with valid rows.
  //
  // The output tile goes through those buffers (rows [0, kRowsA) of a pass in
  // lds_a[fa], the rest in lds_b[fb]) and leaves as 16-byte row stores, in
  // passes of kPassRows rows when it is larger than the buffers.  A lane
  // writes its four adjacent columns as one 8-byte word; one write
  // instruction covers 32 rows at one 16-byte chunk, so chunk q of (pass-
  // relative) row r sits at chunk q ^ sw(r), which spreads those rows over
  // all 64 banks (and keeps a row's chunks on distinct banks for the reads).
  constexpr int kCols = kSwiGLU ? C::BW / 2 : C::BW;
  constexpr int RB = kCols * 2;                                       // bytes per output row
  constexpr int C16 = RB / 16;                                        // 16-byte chunks per row
  constexpr int kRowsA = (C::BM * kChunksPerRow * 16 / RB) / 32 * 32;  // whole tiles in lds_a[fa]
  constexpr int kRowsB = C::BW * kChunksPerRow * 16 / RB;             // rows in lds_b[fb]
  constexpr int kPassRows = (kRowsA + kRowsB) / 32 * 32;
  constexpr int kPasses = (C::BM + kPassRows - 1) / kPassRows;
  static_assert(kPassRows > 0 && C16 >= 8 && (C16 & (C16 - 1)) == 0, "output staging layout");
  auto epilogue = [&](const Unit& cu, int mrows, int fa, int fb) __attribute__((always_inline)) {
    uint16_t* cbase = cu.routed ? a.c_routed : a.c_shared;
    if constexpr (kBwd) {
      // Backward: each lane's quads straight from the accumulators -- dh
      // read, h (the forward's, bit for bit), da = dh up s (1 + a (1 - s))
      // and dc = dh a s (s = sigmoid(a)) written as 8-byte words -- with the
      // staging form's two barriers per pass, which the loader waves count.
      const uint16_t* dhp = cu.routed ? a.dh_routed : a.dh_shared;
      uint16_t* dap = cu.routed ? a.da_routed : a.da_shared;
      uint16_t* dcp = cu.routed ? a.dc_routed : a.dc_shared;
      MOE_FOR(p, kPasses, {
        const int r_lo = p * kPassRows;
        MOE_FOR(i, TM, {
          const int r_tile = tile_row(i) - r_lo;
          if (i < mrows && r_tile >= 0 && r_tile < kPassRows) {
            const int rr = tile_row(i) + lrow;  // row of the unit
            const bool row_ok = rr < cu.valid_rows;
            const int64_t base = (static_cast<int64_t>(cu.orow0) + (row_ok ? rr : 0)) * cu.N;
            MOE_FOR(j, TN / 2, {
              const int col0 = cu.n0 + wn * HC + 32 * j + lcol;
              uint2 dv[4];
              MOE_FOR(g, 4, {
                const int col = col0 + 8 * g;
                dv[g] = *reinterpret_cast<const uint2*>(dhp + base + (col < cu.N ? col : cu.N - 4));
              })
              MOE_FOR(g, 4, {
                const int col = col0 + 8 * g;
                if (row_ok && col < cu.N) {
                  const uint32_t dw[2] = {dv[g].x, dv[g].y};
                  float hv[4], dav[4], dcv[4];
                  MOE_FOR(t, 4, {
                    const float ga = acc[i][j][4 * g + t], up = acc[i][j + TN / 2][4 * g + t];
                    const float dhf = __uint_as_float((t & 1 ? dw[t >> 1] >> 16 : dw[t >> 1] & 0xFFFFu) << 16);
                    const float sgm = __builtin_amdgcn_rcpf(1.0f + __expf(-ga));
                    hv[t] = ga * sgm * up;
                    dav[t] = dhf * up * sgm * (1.0f + ga * (1.0f - sgm));
                    dcv[t] = dhf * ga * sgm;
                  })
                  auto pack = [](const float (&f)[4]) __attribute__((always_inline)) {
                    return make_uint2(bf16x2_bits(f[0], f[1]), bf16x2_bits(f[2], f[3]));
                  };
                  *reinterpret_cast<uint2*>(cbase + base + col) = pack(hv);
                  *reinterpret_cast<uint2*>(dap + base + col) = pack(dav);
                  *reinterpret_cast<uint2*>(dcp + base + col) = pack(dcv);
                }
              })
            })
          }
        })
        lds_barrier();
        lds_barrier();
      })
      return;
    }
    auto sw = [](int r) __attribute__((always_inline)) { return C16 >= 16 ? (r & 15) : ((r >> 1) & 7); };
    auto row_ptr = [&](int r) __attribute__((always_inline)) {
      return r < kRowsA ? reinterpret_cast<unsigned char*>(&lds_a[fa][0]) + r * RB
                        : reinterpret_cast<unsigned char*>(&lds_b[fb][0]) + (r - kRowsA) * RB;
    };
    const int ncols = cu.N - cu.n0 < kCols ? cu.N - cu.n0 : kCols;
    MOE_FOR(p, kPasses, {
      const int r_lo = p * kPassRows;
      MOE_FOR(i, TM, {
        const int r_tile = tile_row(i) - r_lo;
        if (i < mrows && r_tile >= 0 && r_tile < kPassRows) {
          // a 32-row tile lies in one region: kRowsA and kPassRows are multiples of 32
          const int r = r_tile + lrow;
          unsigned char* row = row_ptr(r);
          const int s = sw(r);
          MOE_FOR(j, (kSwiGLU ? TN / 2 : TN), {
            const int col0 = kSwiGLU ? wn * HC + 32 * j : wn * (C::BW / C::WN) + 32 * j;
            MOE_FOR(g, 4, {
              float v[4];
              MOE_FOR(t, 4, {
                v[t] = kSwiGLU ? swiglu(acc[i][j][4 * g + t], acc[i][kSwiGLU ? j + TN / 2 : j][4 * g + t])
                               : acc[i][j][4 * g + t];
              })
              const uint64_t w = static_cast<uint64_t>(bf16x2_bits(v[0], v[1])) |
                                 (static_cast<uint64_t>(bf16x2_bits(v[2], v[3])) << 32);
              const int q = (col0 >> 3) + g;  // 16-byte chunk of these columns
              lds_write_b64(row + ((q ^ s) << 4) + lcol * 2, w);
            })
          })
        }
      })
      lds_barrier();
      constexpr int kPr = (C::BM - p * kPassRows) < kPassRows ? (C::BM - p * kPassRows) : kPassRows;
      constexpr int kChunks = kPr * C16;
      auto store_chunk = [&](int r, int q, const u32x4& val) __attribute__((always_inline)) {
        if (r_lo + r < cu.valid_rows && q * 8 < ncols) {
          // non-temporal: the rows are not read again by this kernel, and the
          // streaming hint leaves the caches to the operands
          __builtin_nontemporal_store(
              val, reinterpret_cast<u32x4*>(cbase + (static_cast<int64_t>(cu.orow0) + r_lo + r) * cu.N +
                                            cu.n0 + q * 8));
        }
      };
      if constexpr (C::PW > 0 && TM * TN > 4) {
        // the loader waves leave no registers for batches
        for (int idx = tid; idx < kChunks; idx += kThreads) {
          const int r = idx / C16, q = idx % C16;
          if (r_lo + r < cu.valid_rows && q * 8 < ncols)
            store_chunk(r, q, lds_read_b128(row_ptr(r) + ((q ^ sw(r)) << 4)));
        }
      } else {
        // all of a thread's chunks are read under one wait, then stored
        static_assert(kChunks % kThreads == 0, "whole chunks per thread");
        constexpr int kIter = kChunks / kThreads;
        const u32x4* src[kIter];
        u32x4 val[kIter];
        MOE_FOR(it, kIter, {
          const int idx = tid + it * kThreads;
          const int r = idx / C16, q = idx % C16;
          src[it] = reinterpret_cast<const u32x4*>(row_ptr(r) + ((q ^ sw(r)) << 4));
        })
        lds_read_n<kIter>(src, val);
        MOE_FOR(it, kIter, {
          const int idx = tid + it * kThreads;
          store_chunk(idx / C16, idx % C16, val[it]);
        })
      }
      lds_barrier();  // the buffers are reused by the next pass or the next unit
    })
  };

  // ---- software pipeline.  Each unit runs an even number of K-steps; the
  // fetcher stays two steps ahead, running into the next unit during the last
  // two steps of the current one.  The unit after the last one is the last
  // one again: its loads are valid and never used.
  //
  // Weight tiles through registers: two LDS buffers, step k in buffer k % 2.
  // Weight tiles by LDS DMA: three LDS stages, step k in stage k % 3; the
  // stage written at step k (for step k + 2) was last read at step k - 1,
  // before the barrier that ends it.  At the end of step k the loads of
  // step k + 1 must have landed: the compiler waits for its A registers
  // before the store to LDS, and vm_wait waits for the DMA, which the
  // compiler does not track -- after it, this thread issued only the LA + LB
  // loads of step k + 2 (any extra younger memory operation makes the wait
  // stricter, not weaker).
  auto next_of = [&](int u) __attribute__((always_inline)) {
    return u + G < uend ? u + G : u;
  };
  auto vm_wait = [&]() __attribute__((always_inline)) {
    if constexpr (C::DMAB) {
      constexpr int n = LA + LB;
      static_assert(n < 64, "vmcnt range");
      // vmcnt(n) (low bits 3:0, high bits 15:14); lgkmcnt, expcnt unconstrained
      __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
    }
  };
  auto stage_after = [](int st, int d) __attribute__((always_inline)) {
    st += d;
    return st >= C::NSB ? st - C::NSB : st;
  };
  int cs = 0;  // weight stage of the current step
  if constexpr (C::PW > 0) {
    if (!loader && C::DMAA) {
      // MFMA waves of an all-DMA tile: the loader waves fill stage k % NS
      // (A and weights) for step k and hit the same barriers (one per K-step,
      // two per epilogue pass).
      constexpr int NS = C::NSA, D = NS - 1;
      auto st = [](int x) __attribute__((always_inline)) { return x >= NS ? x - NS : x; };
      Unit cu = decode(lb);
      lds_barrier();  // step 0 has landed (and useq holds iteration 2's unit)
      for (int i = 0, u = lb; u < uend; ++i) {
        const int un = unit_at(i + 1);
        const Unit nu = decode(un < uend ? un : u);
        int claim = 0;
        if (dyn && tid == 0) claim = atomicAdd(a.unit_counter + ux, 1);
        const int mrows = valid_tiles(cu.valid_rows);
        zero_acc();
        for (int kt = 0; kt < cu.nk; ++kt) {
          mma_plain(cs, cs, mrows);
          lds_barrier();
          cs = st(cs + 1);
        }
        if (dyn && tid == 0) publish(i + 3, claim);
        epilogue(cu, mrows, st(cs + D), st(cs + D));  // the stage the last step read
        cu = nu;
        u = un;
      }
      return;
    }
    if (!loader) {
      // MFMA waves: the loader waves fill A buffer k % 2 and weight stage
      // k % 3 for step k and hit the same barriers (one per K-step, two per
      // epilogue pass), so these waves issue no global load in the K-loop.
      Unit cu = decode(lb);
      lds_barrier();  // step 0 has landed
      for (int u = lb; u < uend; u += G) {
        const Unit nu = decode(next_of(u));
        const int steps = cu.nk + (cu.nk & 1);
        const int mrows = valid_tiles(cu.valid_rows);
        zero_acc();
        for (int kt = 0; kt < steps; kt += 2) {
          const int c1 = stage_after(cs, 1);
          mma(0, cs, mrows, [](auto) {});
          lds_barrier();
          mma(1, c1, kt + 1 < cu.nk ? mrows : 0, [](auto) {});
          cs = stage_after(c1, 1);
          lds_barrier();
        }
        epilogue(cu, mrows, 1, stage_after(cs, C::NSB - 1));
        cu = nu;
      }
      return;
    }
  }
  // The first two units' perm_src entries are loaded together, so the start
  // pays one round trip for them.
  Unit cu;
  int row0[LA], map0[LA], ready0[LA];
  prepare_into(lb, cu, row0, map0);
  prepare(unit_at(1) < uend ? unit_at(1) : lb);
  if constexpr (C::DMAA) {
    // All-DMA tiles in NS stages, D = NS - 1 steps ahead: the DMA of step
    // k + D (running into the next unit's first steps) is issued at step k
    // into the stage that step k - 1 read, before the barrier that ended it.
    // At the end of step k this thread waits until only the loads of steps
    // k + 2 .. k + D (LA + LB each) may still be in flight, so step k + 1 has
    // landed; the barrier then makes every wave's part visible.  Every group
    // has at least D K-steps (the launcher checks), so the first D steps of a
    // unit never reach past the next unit.
    constexpr int NS = C::NSA, D = NS - 1;
    constexpr int kAhead = (D - 1) * (LA + LB);
    static_assert(kAhead < 64, "vmcnt range");
    auto st = [](int x) __attribute__((always_inline)) { return x >= NS ? x - NS : x; };
    // The weight passes of the first D steps need no perm_src entry: they go
    // out first, and the A passes once the entries have landed.  Order: B of
    // steps 0..D-1, then A of steps 0..D-1, so step 0 has landed when only
    // the A passes of steps 1..D-1 may still be in flight.
    {
      const Src cur_b = source_of(cu, row0, row0);  // weight fields only (A ones unused)
      MOE_FOR(f, D, { issue(cur_b, f, f, std::integral_constant<int, kOnlyB>{}); })
    }
    settle_into(map0, ready0);
    Src cur = source_of(cu, row0, ready0);
    MOE_FOR(f, D, { issue(cur, f, f, std::integral_constant<int, kOnlyA>{}); })
    constexpr int kFirst = (D - 1) * LA;
    static_assert(kFirst < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | ((kFirst & 15) | ((kFirst >> 4) << 14)));
    lds_barrier();
    settle();  // free here: those loads are older than the A passes
    for (int i = 0, u = lb; u < uend; ++i) {
      const Src nxt = source_of_pending();
      const Unit nu = pend;
      const int u1 = unit_at(i + 1), u2 = unit_at(i + 2);
      prepare(u2 < uend ? u2 : (u1 < uend ? u1 : u));
      const int mrows = valid_tiles(cu.valid_rows);
      zero_acc();
      for (int kt = 0; kt < cur.nk; ++kt) {
        // step kt + D goes out between the MFMA sub-steps of step kt (all at
        // once from a loader wave)
        const int f = kt + D;
        const int sd = st(cs + D);
        if constexpr (C::PW > 0) {
          constexpr std::integral_constant<int, -1> kAllParts{};
          if (f < cur.nk) issue(cur, f, sd, kAllParts);
          else issue(nxt, f - cur.nk, sd, kAllParts);
        } else {
          mma_dma(cs, mrows, [&](auto ks_c) __attribute__((always_inline)) {
            if (f < cur.nk) issue(cur, f, sd, ks_c);
            else issue(nxt, f - cur.nk, sd, ks_c);
          });
        }
        if (kt == 0) settle();
        __builtin_amdgcn_s_waitcnt(0x0F70 | ((kAhead & 15) | ((kAhead >> 4) << 14)));
        lds_barrier();
        cs = st(cs + 1);
      }
      if constexpr (C::PW > 0) {
        for (int p = 0; p < kPasses; ++p) {  // the MFMA waves' epilogue barriers
          lds_barrier();
          lds_barrier();
        }
      } else {
        epilogue(cu, mrows, st(cs + D), st(cs + D));  // the stage the last step read
      }
      cur = nxt;
      cu = nu;
      u = u1;
    }
    return;
  }
  settle_into(map0, ready0);
  Src cur = source_of(cu, row0, ready0);
  Slice r0, r1;
  constexpr std::integral_constant<int, -1> kAll{};
  load2(r0, cur, cur, 1 << 30, 0, 0, kAll);
  load2(r1, cur, cur, 1 << 30, 1, 1 % C::NSB, kAll);
  stash(r0, 0, 0);
  vm_wait();
  lds_barrier();
  settle();  // those loads are older than the first two steps' loads
  for (int u = lb; u < uend; u += G) {
    const Src nxt = source_of_pending();
    const Unit nu = pend;
    prepare(next_of(next_of(u)));
    const int steps = cur.nk + (cur.nk & 1);
    // 32-row tiles of this wave with valid rows
    const int mrows = valid_tiles(cu.valid_rows);
    if constexpr (C::PW == 0) zero_acc();
    for (int kt = 0; kt < steps; kt += 2) {
      const int c1 = stage_after(cs, 1);
      // the loads of step kt + 2 go out between the MFMA sub-steps of step kt
      // (all at once from a loader wave)
      const int s2 = stage_after(cs, 2);
      if constexpr (C::PW > 0) {
        load2(r0, cur, nxt, steps, kt + 2, s2, kAll);
      } else {
        mma(0, cs, mrows, [&](auto ks_c) __attribute__((always_inline)) {
          load2(r0, cur, nxt, steps, kt + 2, s2, ks_c);
        });
      }
      if (kt == 0) settle();
      stash(r1, 1, c1);
      vm_wait();
      lds_barrier();
      const int s3 = stage_after(c1, 2);
      if constexpr (C::PW > 0) {
        load2(r1, cur, nxt, steps, kt + 3, s3, kAll);
      } else {
        mma(1, c1, kt + 1 < cur.nk ? mrows : 0, [&](auto ks_c) __attribute__((always_inline)) {
          load2(r1, cur, nxt, steps, kt + 3, s3, ks_c);
        });
      }
      cs = stage_after(c1, 1);
      stash(r0, 0, cs);
      vm_wait();
      lds_barrier();
    }
    // buffer 0 holds the next unit's first A slice, stage cs its first weight
    // slice and, with three stages, stage cs + 1 its second
    if constexpr (C::PW > 0) {
      for (int p = 0; p < kPasses; ++p) {  // the MFMA waves' epilogue barriers
        lds_barrier();
        lds_barrier();
      }
    } else {
      epilogue(cu, mrows, 1, stage_after(cs, C::NSB - 1));
    }
    cur = nxt;
    cu = nu;
  }
  if constexpr (C::PW > 0) __builtin_amdgcn_s_waitcnt(0x0F70);  // no DMA left in flight
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

// Groups of many rows (hundreds per expert and more): the 256x128 all-DMA
// tile moves a third fewer bytes per MFMA than 128x128, holds no tile data
// in registers and runs one step ahead.
constexpr int kLongK = 1024;  // reduction length from which the loader-wave form is used
static bool big_groups(const GroupedGemmArgs& a) {
  constexpr int kMinK = kBK * (kBig::NSA - 1);  // each unit at least D K-steps long
  if (a.K_r < kMinK || (a.w_shared && a.K_s < kMinK)) return false;
  return a.T * a.top_k / (a.E > 0 ? a.E : 1) >= 512;
}

template <class C, bool kSwiGLU, bool kBwd, bool kWKM = false>
static void launch_cfg(const GroupedGemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((grouped_gemm_kernel<C, kSwiGLU, kBwd, kWKM>), dim3(persistent_grid<C>()),
                     dim3(C::kAllThreads), 0, s, a);
}

template <bool kSwiGLU, bool kBwd = false>
static hipError_t launch_gemm(const GroupedGemmArgs& a, hipStream_t s) {
  if (streaming_shape(a)) {
    if (!a.w_shared) {
      launch_cfg<kStream, kSwiGLU, kBwd>(a, s);
      return hipGetLastError();
    }
    // The streaming tile would cover the shared expert's T rows in T / BM
    // units that each stream its whole weight tile again, at the CU time of a
    // routed unit; the shared expert runs as its own launch instead, with the
    // tile its row count calls for (and the routed units alone divide evenly
    // over the grid more often).
    GroupedGemmArgs routed = a;
    routed.w_shared = routed.w3_shared = nullptr;
    routed.a_shared = nullptr;
    routed.c_shared = nullptr;
    launch_cfg<kStream, kSwiGLU, kBwd>(routed, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    GroupedGemmArgs shared = a;  // one group: the shared expert's T rows
    shared.unit_counter = a.unit_counter ? a.unit_counter + 8 : nullptr;
    shared.E = 0;
    shared.w_routed = shared.w3_routed = nullptr;
    shared.a_routed = nullptr;
    shared.a_row_map = nullptr;
    shared.c_routed = nullptr;
    constexpr int kMinK = kBK * (kBigL::NSA - 1);
    if (a.T >= 512 && a.K_s >= kMinK) launch_cfg<kBigL, kSwiGLU, kBwd>(shared, s);
    else launch_cfg<kCompute, kSwiGLU, kBwd>(shared, s);
    return hipGetLastError();
  }
  // With long K the loader-wave form pays off (about 1024 rows per expert at
  // d = 7168, H = 2048: FFN 3.54 -> 3.39 ms, bit-identical); the mini model's
  // four to six K-steps per unit gain nothing from it.
  if (big_groups(a)) {
    if (a.K_r >= kLongK && (!a.w_shared || a.K_s >= kLongK)) launch_cfg<kBigL, kSwiGLU, kBwd>(a, s);
    else launch_cfg<kBig, kSwiGLU, kBwd>(a, s);
  } else {
    launch_cfg<kCompute, kSwiGLU, kBwd>(a, s);
  }
  return hipGetLastError();
}

__global__ void zero_counters_kernel(int32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}
hipError_t launch_zero_counters(int32_t* p, int n, hipStream_t s) {
  hipLaunchKernelGGL(zero_counters_kernel, dim3(1), dim3(64), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_gemm_swiglu(const GroupedGemmArgs& a, hipStream_t s) { return launch_gemm<true>(a, s); }
hipError_t launch_gemm_down(const GroupedGemmArgs& a, hipStream_t s) { return launch_gemm<false>(a, s); }
hipError_t launch_gemm_swiglu_bwd(const GroupedGemmArgs& a, hipStream_t s) {
  return launch_gemm<true, true>(a, s);
}
// The streaming tile with K-major weights: routed groups only, whole weight
// tiles (N a multiple of the tile's columns) and whole K-steps in each part.
hipError_t launch_gemm_dgrad(const GroupedGemmArgs& a, hipStream_t s) {
  if (!streaming_shape(a) || a.w_shared || a.N_r % kStream::BW || a.K_r % kBK || a.K2_r % kBK ||
      (a.K2_r > 0 && (!a.w3_routed || !a.a2_routed)))
    return hipErrorNotSupported;
  launch_cfg<kStream, false, false, true>(a, s);
  return hipGetLastError();
}

}  // namespace moe
