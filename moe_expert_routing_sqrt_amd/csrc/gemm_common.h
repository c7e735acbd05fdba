// Building blocks shared by the grouped GEMM kernels (bf16 and e4m3): LDS
// swizzle, direct-to-LDS DMA, explicit memory-counter waits and a fence-free
// barrier.  Device code only.
#pragma once

#include "common.h"

namespace moe {

// LDS operand rows are 128 bytes (8 chunks of 16 B).  gfx950's LDS serves 16
// lanes x 16 B per clock over 64 banks, so the 16 rows read together must land
// on distinct bank groups: even rows use banks 0-31, odd rows 32-63, and within
// each parity the chunk is XORed with (r >> 1) & 7.
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// Wait until at most n vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt
// left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Work-group barrier without the memory fence __syncthreads() carries: the
// fence would wait for every outstanding global load, including the LDS DMA of
// later pipeline stages.  Callers wait for exactly what they need first.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// 64 lanes x 16 bytes from global memory straight into 1 KB of LDS at
// lds + lane*16 (global_load_lds_dwordx4; M0 holds the wave-uniform LDS
// base, one wait state after writing it; lds must be wave-uniform, and
// readfirstlane keeps it in a scalar register whatever the compiler inferred).  Issued from asm so the compiler's
// memory-counter bookkeeping does not see an LDS writer: it would otherwise
// make every later LDS read wait for all DMA in flight.  There is no output
// register; completion is waited for explicitly (wait_vmcnt) before the
// barrier that publishes a stage.
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(gaddr) : "memory", "m0");
}

// The same load with a wave-uniform 64-bit base in scalar registers and a
// 32-bit per-lane byte offset (the saddr form): one address VGPR per load,
// and stepping through K is scalar arithmetic on the base.
__device__ __forceinline__ void dma16_s(const void* base, uint32_t voff, uint32_t lds) {
  // (readfirstlane yields an int: both halves go through uint32_t before
  // widening, so the low half is not sign-extended into the high one)
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b >> 32)));
  const uint64_t sb = (static_cast<uint64_t>(hi) << 32) | lo;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(sb) : "memory", "m0");
}

// 64 lanes x 4 bytes from global memory into 256 contiguous LDS bytes at
// lds + lane*4 (global_load_lds_dword), for per-row scale columns.
__device__ __forceinline__ void dma4(const void* gaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(gaddr) : "memory", "m0");
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace moe
