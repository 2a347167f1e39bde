// Device helpers shared by the MFMA GEMM kernels (gemm.hip, gemm_fewrow.hip): the LDS
// tile swizzle, explicit vector-memory waits, the 32x32x16 bf16 MFMA and the
// global-to-LDS DMA transfers.
#pragma once

#include "common.h"

namespace hymba {

// Tiles of rows x 64 k are fetched with global_load_lds_dwordx4 (each wave instruction
// fills 1 KB of LDS = 8 rows x 64 k), so no VGPR staging and no LDS store instructions.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Swizzle of the 8 16-byte k-chunks of row r: the 16 rows one fragment read touches
// land in distinct bank groups for both 8-lane and 16-lane LDS phases.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
  // vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// v_mfma_f32_32x32x16_bf16: lane l supplies row (l % 32) of A and column (l % 32) of B,
// 8 consecutive k each (block l / 32); it receives D[(e/4)*8 + (l/32)*4 + e%4][l % 32],
// e = 0..15.
__device__ __forceinline__ floatx16 mfma32x32x16(const bf16x8& a, const bf16x8& b,
                                                 const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// global_load_lds_dwordx4 of one 16-byte chunk per lane into the wave's 1 KB LDS block
// at `lptr`, issued from inline asm.  The compiler does not see this LDS write, so it
// adds no conservative vmcnt waits in front of LDS reads of the other stage (it cannot
// separate the two stages once a transfer is in flight across the loop back-edge).
// Every consumer waits explicitly (wait_vmcnt) and then passes a workgroup barrier.
// The instruction has no VGPR result; its address operands are read at issue.
__device__ __forceinline__ void dma16(const void* gptr, lds_void_t* lptr) {
  const uint32_t l = (uint32_t)(uintptr_t)lptr;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(l)), "v"(gptr) : "memory", "m0");
}

// The same transfer marked non-temporal: for a weight stream that is read once per call
// and is larger than the caches, so it does not evict data that later kernels re-read
// (the decode K/V ring).
__device__ __forceinline__ void dma16_nt(const void* gptr, lds_void_t* lptr) {
  const uint32_t l = (uint32_t)(uintptr_t)lptr;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :: "s"(__builtin_amdgcn_readfirstlane(l)), "v"(gptr) : "memory", "m0");
}

}  // namespace hymba
