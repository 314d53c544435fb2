// Device helpers for streaming operand tiles from HBM into LDS with the gfx950
// LDS-DMA load (global_load_lds_dwordx4) and consuming them from a ring of LDS
// stages. Shared by the projection GEMM and the attention kernel.
#pragma once

#include "common.h"

namespace dflash {

// A pointer made provably wave-uniform (scalar registers), as the DMA base.
__device__ inline const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// One 16-byte-per-lane LDS-DMA load: each lane fetches sbase + voff and the
// wave's 64 chunks land at LDS bytes lds .. lds + 1023 (lane l at 16 l). It is
// issued as inline assembly so that the compiler's own wait counting never
// drains a ring on it (its waits can then only be more conservative, never
// short); completion is awaited explicitly with an s_waitcnt vmcnt. The
// s_nop gives the M0 write the wait state an LDS-DMA load needs after it.
// kStream sets the non-temporal cache policy: for data read exactly once (the
// KV cache in attention) it streams measurably faster from HBM than the
// default policy, which is kept for operands that other work-groups re-read
// through L2 (GEMM weights and activations).
template <bool kStream = false>
__device__ inline void lds_dma16(uint32_t voff, const void* sbase, uint32_t lds) {
  if constexpr (kStream)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}

// The 4-byte-per-lane form: the wave's 64 dwords land at LDS bytes
// lds .. lds + 255 (lane l at 4 l). Default cache policy.
__device__ inline void lds_dma4(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// s_waitcnt vmcnt(N) leaving expcnt and lgkmcnt alone (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14]).
#define DFLASH_VMWAIT(N) \
  __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (15 << 8) | ((((N) >> 4) & 3) << 14))

// Work-group barrier without the memory fence of __syncthreads (which would
// drain every outstanding load): the LDS reads it must order are awaited
// explicitly (lgkmcnt(0)), and the empty asm statements keep the compiler from
// moving LDS accesses across it.
__device__ inline void block_barrier() {
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ inline uint32_t lds_base(const void* shared_array) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)shared_array;
}

__device__ inline u32x4 lds_read16(uint32_t byte_addr) {
  return *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)byte_addr;
}

__device__ inline uint32_t lds_read_u8(uint32_t byte_addr) {
  return *(const __attribute__((address_space(3))) uint8_t*)(uintptr_t)byte_addr;
}

// Chunk swizzle for rows of CPR 16-byte chunks read 16 consecutive rows at a
// time (one MFMA operand): logical chunk c of row r is stored at c ^ rswz(r),
// which puts the 16 reads on distinct 16-byte bank groups when the hardware
// serves 8 or 16 lanes per ds_read_b128 pass. Depends on the row's low 4 bits.
// The projection GEMM uses it. gfx950 serves a ds_read_b128 in 32-lane passes
// of 8-byte halves over 128 banks (see the attention kernel's swizzles), and
// in that model these reads stall 4 cycles each; the GEMM with a swizzle that
// stalls none measured no faster (C3 q|k|v 41.7 against 41.1 us, 4096-row
// precompute 236 against 231 us on the same box), so it keeps this one.
template <int CPR> __device__ inline int rswz(int row) {
  if constexpr (CPR >= 16) return row & 15;
  else if constexpr (CPR == 8) return (row & 7) ^ ((row >> 3) & 1);
  else return ((row >> 1) ^ (row >> 2)) & 3;
}

}  // namespace dflash
