// Shared device helpers for the gfx950 kernels of libhymba.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hymba {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float floatx4;
typedef __attribute__((ext_vector_type(16))) float floatx16;

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }  // RNE (v_cvt_pk_bf16_f32)

// 16-byte vector of raw bits, used for copies and vector loads.
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// MFMA D = A(16x32) * B(32x16) + C, bf16 inputs, fp32 accumulate.  Lane l supplies
// row (l % 16) of A and column (l % 16) of B, 8 consecutive k each (block l / 16);
// it receives D rows 4 * (l / 16) + r, r = 0..3, at column (l % 16).
__device__ __forceinline__ floatx4 mfma16x16x32(const bf16x8& a, const bf16x8& b,
                                                const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, then
// s_barrier.  __syncthreads(), and any release fence covering LDS, also drains every
// outstanding vector-memory operation including global_load_lds DMA (vmcnt(0)), which
// would empty a prefetch pipeline at every barrier.  Code reading DMA'd data waits for
// it explicitly (s_waitcnt vmcnt(N)) before calling this.  The memory clobber keeps
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLn2F = 0.6931471805599453f;

// softplus(z) = log(1 + e^z) on the hardware base-2 exp / log: e^z = 2^(z log2 e), and
// log1p(t) in the compensated form log(u) * t / (u - 1) with u = fl(1 + t), which cancels
// the rounding of 1 + t (Goldberg, "What every computer scientist should know about
// floating-point arithmetic", Theorem 4); u == 1 means log1p(t) = t to fp32 precision.
// Above 20, log(1 + e^z) - z = log1p(e^-z) < 2.1e-9 and z is returned.
__device__ __forceinline__ float softplus_f(float z) {
  const float t = __builtin_amdgcn_exp2f(z * kLog2eF);
  const float u = 1.f + t;
  const float d = u - 1.f;
  const float r = d == 0.f ? t : __builtin_amdgcn_logf(u) * kLn2F * (t * __builtin_amdgcn_rcpf(d));
  return z > 20.f ? z : r;
}
// SiLU(z) = z / (1 + e^-z) with the hardware reciprocal (1 ulp).
__device__ __forceinline__ float silu_f(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * kLog2eF));
}

}  // namespace hymba
