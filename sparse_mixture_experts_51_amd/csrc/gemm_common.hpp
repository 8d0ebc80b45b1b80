// gemm_common.hpp -- device helpers shared by the bf16 MFMA GEMM kernels of
// libmoe.so: compile-time loops, LDS traffic in asm (for buffers that LDS DMA
// also fills), LDS DMA, barriers and a block-wide scan.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "common.hpp"

namespace moe {

typedef __attribute__((address_space(3))) void* lds_ptr_t;  // LDS address (DMA destination)

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

// Two 16-byte LDS reads, complete on return: the wait sits in the same asm
// block, so the destination registers are never live while a read is in
// flight.
__device__ __forceinline__ void lds_read2_b128(const u32x4* p0, const u32x4* p1, u32x4& v0,
                                               u32x4& v1) {
  const unsigned a0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_ptr_t)p0));
  const unsigned a1 = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_ptr_t)p1));
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1)
      : "v"(a0), "v"(a1)
      : "memory");
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// dst + 16 * l (dst is wave-uniform).  kPolicy is the load's cache-policy
// operand (on gfx950 bit 1 is the non-temporal hint).
template <int kPolicy = 0>
__device__ __forceinline__ void dma_b128(__amdgpu_buffer_rsrc_t rsrc, void* dst, int voffset,
                                         int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)dst, 16, voffset, soffset, 0, kPolicy);
}

// Six 16-byte LDS reads under one wait (the fragments of one MFMA sub-step
// of a 4x2 tile), complete on return like lds_read2_b128.
__device__ __forceinline__ void lds_read6_b128(const u32x4* const (&p)[6], u32x4 (&v)[6]) {
  unsigned a[6];
#pragma unroll
  for (int i = 0; i < 6; ++i) a[i] = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_ptr_t)p[i]));
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %7\n\t"
      "ds_read_b128 %2, %8\n\t"
      "ds_read_b128 %3, %9\n\t"
      "ds_read_b128 %4, %10\n\t"
      "ds_read_b128 %5, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5])
      : "memory");
}

// Four 16-byte LDS reads under one wait (a 2x2 tile's sub-step fragments).
__device__ __forceinline__ void lds_read4_b128(const u32x4* const (&p)[4], u32x4 (&v)[4]) {
  unsigned a[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_ptr_t)p[i]));
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}

// The epilogue's LDS traffic is written in asm too: the compiler cannot tell
// its buffers from those that LDS DMA is filling and would otherwise drain
// every load in flight before the first access.  An 8-byte write at p
// (completed by the lgkmcnt(0) of the barrier that follows it) ...
__device__ __forceinline__ void lds_write_b64(void* p, uint64_t v) {
  const unsigned a = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
  asm volatile("ds_write_b64 %0, %1" : : "v"(a), "v"(v) : "memory");
}
// A 4-byte write and a 4-byte read (complete on return), for small LDS
// tables shared through the same barriers.
__device__ __forceinline__ void lds_write_b32(void* p, int v) {
  const unsigned a = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
  asm volatile("ds_write_b32 %0, %1" : : "v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ int lds_read_b32(const void* p) {
  const unsigned a = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
  int v;
  asm volatile(
      "ds_read_b32 %0, %1\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v)
      : "v"(a)
      : "memory");
  return v;
}
// ... and a 16-byte read, complete on return.
__device__ __forceinline__ u32x4 lds_read_b128(const void* p) {
  const unsigned a = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
  u32x4 v;
  asm volatile(
      "ds_read_b128 %0, %1\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v)
      : "v"(a)
      : "memory");
  return v;
}
// N 16-byte LDS reads, in groups of six, four, two and one under one wait each.
template <int N, int I = 0>
__device__ __forceinline__ void lds_read_n(const u32x4* const (&p)[N], u32x4 (&v)[N]) {
  if constexpr (N - I >= 6) {
    const u32x4* const q[6] = {p[I], p[I + 1], p[I + 2], p[I + 3], p[I + 4], p[I + 5]};
    u32x4 w[6];
    lds_read6_b128(q, w);
    for (int i = 0; i < 6; ++i) v[I + i] = w[i];
    lds_read_n<N, I + 6>(p, v);
  } else if constexpr (N - I >= 4) {
    const u32x4* const q[4] = {p[I], p[I + 1], p[I + 2], p[I + 3]};
    u32x4 w[4];
    lds_read4_b128(q, w);
    for (int i = 0; i < 4; ++i) v[I + i] = w[i];
    lds_read_n<N, I + 4>(p, v);
  } else if constexpr (N - I >= 2) {
    lds_read2_b128(p[I], p[I + 1], v[I], v[I + 1]);
    lds_read_n<N, I + 2>(p, v);
  } else if constexpr (N - I == 1) {
    v[I] = lds_read_b128(p[I]);
  }
}

// Two fp32 values to packed bf16 (round to nearest even) in one conversion.
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{lo, hi}, b2_t));
}

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

}  // namespace moe
