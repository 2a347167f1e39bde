// Probes of this chip's practical ceilings, for the measurement's rooflines: the rate of
// the hardware base-2 exponential (v_exp_f32), the dense bf16 MFMA rate under a pure MFMA
// loop, and the rate of a plain streaming read.  They are timed by the caller (HIP
// events around one launch); nothing here belongs to the layer.
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;

// Eight independent chains of x <- 2^-x per lane (x stays in [0.5, 1]), `iters` rounds:
// 8 * iters exponentials per lane, one v_exp_f32 (with a negate modifier) each.
__global__ __launch_bounds__(256) void exp_probe_kernel(float* out, int iters) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.5f + 0.01f * (float)((threadIdx.x + i) & 31);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Four independent accumulators per wave, `iters` rounds of v_mfma_f32_32x32x16_bf16 on
// each: 4 * iters * 32 * 32 * 16 * 2 flop per wave.
__global__ __launch_bounds__(256) void mfma_probe_kernel(float* out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (bf16)(0.001f * (float)((threadIdx.x + i) & 15));
    b[i] = (bf16)(0.002f * (float)((threadIdx.x + 3 * i) & 15));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// The same MFMA loop on GEMM-like operands: every lane cycles through 8 A and 8 B
// fragments loaded from `src` ([2][64][8][256] bf16x8: A then B, the caller's values), so
// consecutive instructions see different operands as in a GEMM's k loop (the matrix
// cores' rate depends on the operand bits).  `iters` rounds of 8 MFMAs on 4
// accumulators: 8 * iters * 32 * 32 * 16 * 2 flop per wave.
constexpr int kProbeFrags = 8;
constexpr size_t kProbeOperandBytes = (size_t)2 * 64 * kProbeFrags * 256 * 16;
__global__ __launch_bounds__(256) void mfma_data_probe_kernel(const bf16x8* __restrict__ src,
                                                              float* out, int iters) {
  const int t = threadIdx.x;
  const int64_t base = (int64_t)(blockIdx.x % 64) * kProbeFrags * 256;
  const bf16x8* fb = src + (int64_t)64 * kProbeFrags * 256;
  bf16x8 a[kProbeFrags], b[kProbeFrags];
#pragma unroll
  for (int i = 0; i < kProbeFrags; ++i) {
    a[i] = src[base + i * 256 + t];
    b[i] = fb[base + i * 256 + t];
  }
  f32x16 c[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kProbeFrags; ++i)
      c[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[i], c[i & 3], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[j][e];
  out[(int64_t)blockIdx.x * 256 + t] = s;
}

// Every 16-byte piece of `src` read once (grid-stride), one float per thread written.
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, int64_t n,
                                                         float* out) {
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const u32x4 v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = (float)(acc & 1023u);
}

}  // namespace

// kind 0: exp rate (out: blocks * 256 floats), 1: MFMA rate (out: blocks * 256 floats),
// 2: streaming read of src's `bytes` (out: 8192 * 256 floats), 3: MFMA rate on the
// operands at src (at least probe_operand_bytes(); out: blocks * 256 floats).
size_t probe_operand_bytes() { return kProbeOperandBytes; }

hipError_t launch_probe(int kind, int blocks, int iters, const void* src, size_t bytes, float* out,
                        hipStream_t s) {
  switch (kind) {
    case 3:
      if (bytes < kProbeOperandBytes) return hipErrorInvalidValue;
      mfma_data_probe_kernel<<<dim3(blocks), dim3(256), 0, s>>>((const bf16x8*)src, out, iters);
      break;
    case 0: exp_probe_kernel<<<dim3(blocks), dim3(256), 0, s>>>(out, iters); break;
    case 1: mfma_probe_kernel<<<dim3(blocks), dim3(256), 0, s>>>(out, iters); break;
    case 2: read_probe_kernel<<<dim3(8192), dim3(256), 0, s>>>((const u32x4*)src,
                                                               (int64_t)(bytes / 16), out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hymba
