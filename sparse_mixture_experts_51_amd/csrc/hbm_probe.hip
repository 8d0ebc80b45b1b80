// hbm_probe.hip -- the achievable HBM read rate, for the measurements (a
// library of its own, libmoe_probe.so, next to libmoe.so; not part of the
// MoE interface).  Three ways of reading:
//
// - LDS DMA: one block per CU streams whole 1 MiB pieces of a buffer, 32 KiB
//   per step, straight into a three-stage LDS ring, two steps ahead, with the
//   non-temporal hint -- the access pattern of the grouped GEMM's streamed
//   weights without its MFMAs.
// - Non-temporal register loads: eight blocks of 256 threads per CU, each
//   thread with eight 16-byte loads in flight, grid-strided -- the pattern of
//   the register-path weight loads.
// - LDS DMA in the grouped GEMM's weight pattern (128 bytes of each of 256
//   weight rows per step, rows a given stride apart), fetched across unit
//   boundaries, and after every unit a burst of 16-byte non-temporal stores
//   to an output buffer -- a weight stream whose units each write their
//   output tile, as the GEMM's do (the SwiGLU stage writes h, the down stage
//   y), at a chosen ratio of written to read bytes.
//
// Each thread folds what it read into a per-thread value so that the loads
// have a consumer.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 512;
constexpr int kStep = 32 * 1024;      // bytes per step
constexpr int kPiece = 1024 * 1024;   // bytes per unit of work
constexpr int kStages = 3;
constexpr int kPolicyNT = 2;  // cache-policy operand: bit 1 is the non-temporal hint on gfx950
constexpr int kPasses = kStep / (kThreads * 16);  // 16-byte DMA per thread and pass
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const unsigned char* __restrict__ buf,
                                                            int pieces, uint32_t* __restrict__ sink) {
  __shared__ u32x4 ring[kStages][kStep / 16];
  const int tid = threadIdx.x, wave = tid >> 6;
  constexpr int kSteps = kPiece / kStep;
  uint32_t acc = 0;
  for (int p = blockIdx.x; p < pieces; p += gridDim.x) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(buf) + static_cast<int64_t>(p) * kPiece, static_cast<short>(0), kPiece,
        0x00020000);
    // step s into stage st: pass i covers bytes [i * 8 KiB, (i + 1) * 8 KiB)
    // of the step, lane l of wave w the 16 bytes at (w * 64 + l) * 16
    auto issue = [&](int s, int st) {
#pragma unroll
      for (int i = 0; i < kPasses; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)&ring[st][i * kThreads + wave * 64], 16,
                                                 tid * 16, s * kStep + i * kThreads * 16, 0, kPolicyNT);
    };
    issue(0, 0);
    issue(1, 1);
    for (int s = 0; s < kSteps; ++s) {
      const int f = s + 2;
      issue(f < kSteps ? f : kSteps - 1, f % kStages);  // past the end: the last step again
      // all but the newest step's kPasses loads have landed, so step s + 1 has
      __builtin_amdgcn_s_waitcnt(0x0F70 | kPasses);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      acc ^= ring[s % kStages][tid][0];
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) before the stage is reused
      __builtin_amdgcn_s_barrier();
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing in flight into the ring
    __builtin_amdgcn_s_barrier();
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;  // keeps the reads; practically never stored
}

// The read-and-write stream, in the grouped GEMM's weight pattern: a piece is
// 256 rows of row_bytes, and a 32 KiB step reads 128 bytes of every row (one
// 64-wide K-step of a 256-row weight tile), starting at column p mod (steps
// per piece) and wrapping round, as units that run together start their K
// loops at different steps.  A block's pieces (blockIdx.x, + gridDim.x, ...)
// form one sequence of steps, fetched two steps ahead across piece
// boundaries as the GEMM fetches across units; after the last step of piece p
// the block writes out_chunks 16-byte chunks at out + p * out_chunks while the
// next piece's first steps are in flight.
__global__ __launch_bounds__(kThreads) void hbm_read_write_kernel(const unsigned char* __restrict__ buf,
                                                                  int pieces, int row_bytes,
                                                                  u32x4* __restrict__ out, int out_chunks,
                                                                  uint32_t* __restrict__ sink) {
  __shared__ u32x4 ring[kStages][kStep / 16];
  const int tid = threadIdx.x, wave = tid >> 6;
  constexpr int kRows = 256, kRowsPerPass = kThreads / 8;  // 8 lanes of 16 bytes per 128-byte row piece
  const int steps = row_bytes / 128;
  const int mine = static_cast<int>(blockIdx.x) < pieces
                       ? (pieces - static_cast<int>(blockIdx.x) + static_cast<int>(gridDim.x) - 1) /
                             static_cast<int>(gridDim.x)
                       : 0;
  const int total = mine * steps;
  uint32_t acc = 0;
  auto issue = [&](int g, int st) {
    if (g >= total) g = total - 1;  // past the end: the last step again
    const int i = g / steps;
    const int64_t p = static_cast<int64_t>(blockIdx.x) + static_cast<int64_t>(i) * gridDim.x;
    int col = g - i * steps + static_cast<int>(p % steps);
    if (col >= steps) col -= steps;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(buf) + p * kRows * row_bytes, static_cast<short>(0), kRows * row_bytes,
        0x00020000);
#pragma unroll
    for (int j = 0; j < kPasses; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)&ring[st][j * kThreads + wave * 64], 16,
                                               (j * kRowsPerPass + tid / 8) * row_bytes + (tid % 8) * 16,
                                               col * 128, 0, kPolicyNT);
  };
  if (total > 0) {
    issue(0, 0);
    issue(1, 1);
    for (int g = 0; g < total; ++g) {
      issue(g + 2, (g + 2) % kStages);
      // all but the newest kPasses memory operations are done (stores count
      // too), so step g + 1 has landed
      __builtin_amdgcn_s_waitcnt(0x0F70 | kPasses);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      acc ^= ring[g % kStages][tid][0];
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) before the stage is reused
      __builtin_amdgcn_s_barrier();
      if (g % steps == steps - 1) {
        const int64_t p = static_cast<int64_t>(blockIdx.x) + static_cast<int64_t>(g / steps) * gridDim.x;
        u32x4* dst = out + p * out_chunks;
        for (int c = tid; c < out_chunks; c += kThreads)
          __builtin_nontemporal_store(u32x4{acc, static_cast<uint32_t>(p), static_cast<uint32_t>(c), 0u}, dst + c);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing in flight into the ring
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;  // keeps the reads; practically never stored
}

constexpr int kNtThreads = 256;
constexpr int kNtBlocksPerCu = 8;
constexpr int kNtInFlight = 8;  // 16-byte loads per thread per trip

__global__ __launch_bounds__(kNtThreads) void hbm_read_nt_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                                uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kNtThreads * kNtInFlight;
  uint32_t acc = 0;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kNtThreads * kNtInFlight + threadIdx.x; base < n16;
       base += stride) {
    u32x4 v[kNtInFlight];
#pragma unroll
    for (int u = 0; u < kNtInFlight; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * kNtThreads;
      v[u] = i < n16 ? __builtin_nontemporal_load(buf + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kNtInFlight; ++u) acc ^= v[u][0] ^ v[u][3];
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x / kNtBlocksPerCu] = acc;  // practically never stored
}

int compute_units(int* cus) {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess &&
                 hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && *cus > 0
             ? 0
             : 1;
}

}  // namespace

// Reads `bytes` (a multiple of 1 MiB, at most 2^31 MiB) at `buf` once.  `sink`
// holds one word per CU and is normally left untouched.  Returns 0, or 1 if
// the sizes are unusable or the launch fails.
extern "C" int moe_probe_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % kPiece != 0) return 1;
  int cus = 0;
  if (compute_units(&cus) != 0) return 1;
  const int64_t pieces = bytes / kPiece;
  if (pieces > 0x7FFFFFFF) return 1;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(cus), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const unsigned char*>(buf), static_cast<int>(pieces), sink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// The weight-pattern stream with writes: pieces of 256 rows of row_bytes,
// out_per_piece bytes written after each (piece p's at out + p * out_per_piece).
extern "C" int moe_probe_hbm_read_write(const void* buf, int64_t bytes, int64_t row_bytes, void* out,
                                        int64_t out_per_piece, uint32_t* sink, void* stream) {
  if (!buf || !out || !sink || row_bytes <= 0 || row_bytes % 128 != 0 || row_bytes > kPiece) return 1;
  const int64_t piece = 256 * row_bytes;
  if (bytes <= 0 || bytes % piece != 0 || out_per_piece <= 0 || out_per_piece > piece || out_per_piece % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(out) & 15) != 0)
    return 1;
  int cus = 0;
  if (compute_units(&cus) != 0) return 1;
  const int64_t pieces = bytes / piece;
  if (pieces > 0x7FFFFFFF) return 1;
  hipLaunchKernelGGL(hbm_read_write_kernel, dim3(cus), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const unsigned char*>(buf), static_cast<int>(pieces), static_cast<int>(row_bytes),
                     static_cast<u32x4*>(out), static_cast<int>(out_per_piece / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// The same contract with non-temporal register loads (kNtBlocksPerCu blocks
// per CU; `sink` again holds one word per CU).
extern "C" int moe_probe_hbm_read_nt(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % kPiece != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return 1;
  int cus = 0;
  if (compute_units(&cus) != 0) return 1;
  hipLaunchKernelGGL(hbm_read_nt_kernel, dim3(cus * kNtBlocksPerCu), dim3(kNtThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
