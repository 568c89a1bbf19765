// Building blocks of the LDS-staged kernels (tiled grouped GEMM, router
// GEMM): direct-to-LDS loads, explicit vm-counter waits and an LDS-only
// workgroup barrier.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace moe {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Slot of 16-byte chunk c of staged row r, for rows of 8 chunks (128 B) and
// of 16 chunks (256 B).  A direct-to-LDS instruction writes 1 KB
// contiguously (lane i at +16 i), so each lane fetches the global chunk that
// belongs in its slot; fragment reads (16 lanes on 16 consecutive rows, one
// chunk) then fall on distinct banks.  Measured conflict-free on gfx950.
__device__ __forceinline__ int slot8(int r, int c) { return c ^ (r & 7); }
__device__ __forceinline__ int slot16(int r, int c) { return c ^ (r & 15); }

// s_waitcnt vmcnt(v) for a runtime v in [0, VMAX] (the count is an immediate),
// other counters untouched (gfx9 encoding).
template <int VMAX>
__device__ __forceinline__ void wait_vmcnt_le(int v) {
  static_assert(VMAX >= 0 && VMAX < 64, "vmcnt range");
  if constexpr (VMAX > 0) {
    if (v >= VMAX) {
      __builtin_amdgcn_s_waitcnt((VMAX & 15) | ((VMAX >> 4) << 14) | (7 << 4) | (15 << 8));
      return;
    }
    wait_vmcnt_le<VMAX - 1>(v);
  } else {
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  }
}

// s_waitcnt vmcnt(V) for a compile-time V, other counters untouched.
template <int V>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(V >= 0 && V < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() would also
// wait for every outstanding vector-memory operation, including the
// direct-to-LDS loads of later chunks, and drain the pipeline; completion of
// the chunk about to be read is awaited explicitly with wait_vmcnt_le instead.
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ u32x4_t lds_read16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// One 1 KB direct-to-LDS block: lane i copies 16 bytes from src to dst + 16 i.
__device__ __forceinline__ void dma16(const void* src, uint8_t* dst_block) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst_block, 16, 0, 0);
}

// The same 1 KB block (lane i copies 16 bytes from base + off_i), issued from
// inline assembly.  The compiler's wait insertion then does not know of a
// pending LDS write: with the builtin in flight it waits for EVERY
// outstanding LDS read before the first use of any (the LDS counter then has
// two kinds of events), which defeats reads interleaved with MFMAs.  Callers
// order these loads against LDS reads themselves (wait_vmcnt_le + barrier).
// base must be wave-uniform; M0 (the LDS address) is written here and is not
// used by the compiler in kernels that issue no builtin direct-to-LDS loads.
__device__ __forceinline__ void dma16_untracked(const uint8_t* base, uint32_t off,
                                                uint8_t* dst_block) {
  const uint32_t la = (uint32_t)(size_t)(lds_ptr_t)dst_block;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(la), "v"(off), "s"(base) : "memory", "m0");
}

// 4 bytes per lane (lane i's dword from its own address to dst + 4 i), issued
// like dma16_untracked.
__device__ __forceinline__ void dma4_untracked(const void* src, uint8_t* dst) {
  const uint32_t la = (uint32_t)(size_t)(lds_ptr_t)dst;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(la), "v"(src) : "memory", "m0");
}

// Calls f(std::integral_constant<int, n>) for a runtime n in [0, N]: a tiled
// kernel's main loop is compiled once per count of valid row blocks, so its
// row-block checks are resolved at compile time instead of being one scalar
// branch per block and column.
template <int N, class F>
__device__ __forceinline__ void with_count(int n, F&& f) {
  if constexpr (N > 0) {
    if (n >= N) {
      f(std::integral_constant<int, N>{});
      return;
    }
    with_count<N - 1>(n, f);
  } else {
    f(std::integral_constant<int, 0>{});
  }
}

// The count a with_count callee was given, or a plain runtime count.
template <class T>
__device__ __forceinline__ constexpr int count_value(T n) {
  if constexpr (std::is_integral_v<T>) return n;
  else return T::value;
}

}  // namespace moe
