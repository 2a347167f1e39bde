// SSM heads of the hybrid-head layer: Mamba selective scan with a diagonal A per
// channel, the D skip term and the SiLU output gate.
//
// Source: "Hymba: A Hybrid-head Architecture for Small Language Models" (outta.ai
// summary), Design formulation: the SSM mixing coefficient
// alpha_{i,j} = C_i (prod_{k=j+1..i} exp(A dt_k)) B_j dt_j and the gated head output
// Y_ssm = G * (alpha-mixed SSM input).  In recurrent form, per channel c and state n:
//   h_t[c,n] = exp(dt_t[c] A[c,n]) h_{t-1}[c,n] + dt_t[c] x_t[c] B_t[n]
//   y_t[c]   = sum_n C_t[n] h_t[c,n] + D[c] x_t[c];      out = y * SiLU(G)
// h = 0 before the first meta token.
//
// Prefill: a workgroup owns (sequence, block of channels); each lane keeps NS states
// of one channel in fp32 registers and walks the sequence in order.  Inputs for a
// chunk of TC tokens (x, G, dt of the block's channels and the shared B, C rows) are
// staged in LDS with coalesced loads; the per-token sum over states is a DPP
// butterfly across the channel's lanes.  A is pre-scaled by log2(e) so the decay is
// one v_exp_f32.  Every sequence replays the (batch-shared) meta prefix; only
// sequence 0 stores the meta rows.
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over groups of LPC consecutive lanes (LPC a power of two <= 64); every lane of
// the group receives the total.
template <int LPC>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPC >= 2) v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (LPC >= 4) v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (LPC >= 8) v += dpp<0x141>(v);  // row_half_mirror
  if constexpr (LPC >= 16) v += dpp<0x140>(v); // row_mirror
  if constexpr (LPC >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (LPC >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ void load8v(const bf16* p, float out[8]) {
  const bf16x8 v = *(const bf16x8*)p;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
}
__device__ __forceinline__ void load8v(const float* p, float out[8]) {
  const floatx4 a = *(const floatx4*)p, b = *(const floatx4*)(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[e] = a[e];
    out[4 + e] = b[e];
  }
}

// 8 consecutive elements held in their storage type until used, so that a load can
// stay in flight past later loads.
template <typename T>
struct Raw8;
template <>
struct Raw8<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *(const bf16x8*)p; }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)0.f;
  }
  __device__ __forceinline__ float operator[](int e) const { return (float)v[e]; }
};
template <>
struct Raw8<float> {
  floatx4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *(const floatx4*)p;
    b = *(const floatx4*)(p + 4);
  }
  __device__ __forceinline__ void zero() { a = b = floatx4{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ float operator[](int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

__device__ __forceinline__ int64_t seq_row(int t, int b, int n_meta, int L) {
  return t < n_meta ? (int64_t)t : (int64_t)n_meta + (int64_t)b * L + (t - n_meta);
}

}  // namespace

template <typename T, int NS, int LPC>
__global__ __launch_bounds__(256) void scan_prefill_kernel(ScanParams p) {
  constexpr int N = NS * LPC;
  constexpr int CB = 256 / LPC;  // channels per workgroup
  constexpr int TC = 32;         // tokens per staged chunk
  __shared__ float dt_s[TC][CB];
  __shared__ float b_s[TC][N];
  __shared__ float c_s[TC][N];
  __shared__ T x_s[TC][CB];
  __shared__ T g_s[TC][CB];
  __shared__ T y_s[TC][CB];

  const int tid = threadIdx.x;
  const int cl = tid / LPC, sg = tid % LPC;
  const int c0 = blockIdx.x * CB;
  const int b = blockIdx.y;
  const int c = c0 + cl;
  const bool cok = c < p.Di;

  float A2[NS], h[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    A2[k] = cok ? p.A[(int64_t)c * N + sg * NS + k] * kLog2e : 0.f;
    h[k] = (cok && p.h0 != nullptr) ? p.h0[(int64_t)c * N + sg * NS + k] : 0.f;
  }
  const float Dc = cok ? p.D[c] : 0.f;
  const T* z = (const T*)p.z;
  T* yout = (T*)p.y;
  const int total = p.n_meta + p.L;

  for (int t0 = 0; t0 < total; t0 += TC) {
    const int tn = min(TC, total - t0);
    for (int e = tid; e < tn * CB; e += 256) {
      const int tt = e / CB, cc = e % CB, ch = c0 + cc;
      const int64_t row = seq_row(t0 + tt, b, p.n_meta, p.L);
      if (ch < p.Di) {
        dt_s[tt][cc] = p.dt[row * p.Di + ch];
        x_s[tt][cc] = z[row * p.z_stride + p.xs_col + ch];
        g_s[tt][cc] = z[row * p.z_stride + p.g_col + ch];
      } else {
        dt_s[tt][cc] = 0.f;
        x_s[tt][cc] = from_f32<T>(0.f);
        g_s[tt][cc] = from_f32<T>(0.f);
      }
    }
    for (int e = tid; e < tn * 2 * N; e += 256) {
      const int tt = e / (2 * N), j = e % (2 * N);
      const int64_t row = seq_row(t0 + tt, b, p.n_meta, p.L);
      const float v = p.bc[row * 2 * N + j];
      if (j < N)
        b_s[tt][j] = v;
      else
        c_s[tt][j - N] = v;
    }
    __syncthreads();

    for (int tt = 0; tt < tn; ++tt) {
      const float dtv = dt_s[tt][cl];
      const float xv = to_f32(x_s[tt][cl]);
      const float dx = dtv * xv;
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const int n = sg * NS + k;
        const float a = __builtin_amdgcn_exp2f(dtv * A2[k]);
        h[k] = fmaf(a, h[k], dx * b_s[tt][n]);
        acc = fmaf(h[k], c_s[tt][n], acc);
      }
      acc = group_sum<LPC>(acc);
      if (sg == 0) {
        const float yv = fmaf(Dc, xv, acc);
        y_s[tt][cl] = from_f32<T>(yv * silu_f(to_f32(g_s[tt][cl])));
      }
    }
    __syncthreads();

    for (int e = tid; e < tn * CB; e += 256) {
      const int tt = e / CB, cc = e % CB, ch = c0 + cc;
      const int t = t0 + tt;
      if (ch < p.Di && (t >= p.n_meta || b == 0))
        yout[seq_row(t, b, p.n_meta, p.L) * p.y_stride + ch] = y_s[tt][cc];
    }
    // the next chunk's staging writes only after every lane passed this chunk's
    // compute (barrier above); y_s is rewritten only after the next barrier.
  }

  if (p.h_out != nullptr && cok) {
    float* dst = p.h_out + ((int64_t)b * p.Di + c) * N + sg * NS;
#pragma unroll
    for (int k = 0; k < NS; ++k) dst[k] = h[k];
  }
}

template <typename T, int NS, int LPC>
static hipError_t run_scan(const ScanParams& p, hipStream_t s) {
  constexpr int CB = 256 / LPC;
  dim3 grid((p.Di + CB - 1) / CB, p.B);
  scan_prefill_kernel<T, NS, LPC><<<grid, dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

template <typename T>
static hipError_t scan_dispatch(const ScanParams& p, hipStream_t s) {
  switch (p.N) {
    case 4: return run_scan<T, 4, 1>(p, s);
    case 8: return run_scan<T, 4, 2>(p, s);
    case 16: return run_scan<T, 4, 4>(p, s);
    case 32: return run_scan<T, 4, 8>(p, s);
    case 64: return run_scan<T, 8, 8>(p, s);
    case 128: return run_scan<T, 8, 16>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan_prefill(bool bf16_, const ScanParams& p, hipStream_t s) {
  if (p.B == 0 || p.Di == 0 || p.n_meta + p.L == 0) return hipSuccess;
  return bf16_ ? scan_dispatch<bf16>(p, s) : scan_dispatch<float>(p, s);
}

// --------------------------------------------------------------------- decode step
// Workgroup per (block of channels, group of SB sequences); thread per (channel, group
// of 4 states).  Every per-sequence operand that does not depend on dt (the state h as
// one float4 per thread, x, G, and the thread's 4 entries of B and C) is loaded first,
// so its latency overlaps the dt projection.  The lanes of a channel share
// dt = softplus(delta . W_dt[c] + b[c]) (delta rounded to the storage type, as the
// prefill path stores it): each lane streams its slice of W_dt[c] once and accumulates
// it against the SB sequences' deltas staged in LDS.  Then every sequence advances its
// states.  The thread of state group 0 of channel 0 advances pos[b]: every kernel that
// reads pos precedes this one.
template <typename T, int LPC, int SB>
__global__ __launch_bounds__(256) void ssm_step_kernel(SsmStepParams p) {
  constexpr int NS = 4;
  constexpr int N = NS * LPC;
  constexpr int CB = 256 / LPC;
  __shared__ float dl_s[SB][512];  // dt_rank <= 512, checked on the host
  const int tid = threadIdx.x, sg = tid % LPC;
  const int c_raw = blockIdx.x * CB + tid / LPC;
  const bool cok = c_raw < p.Di;
  const int c = cok ? c_raw : 0;
  const int b0 = blockIdx.y * SB;
  const int nb = min(SB, p.B - b0);
  const int xw = p.R + 2 * N;

  floatx4 hv[SB], bv[SB], cv[SB];
  float xv[SB], gv[SB];
#pragma unroll
  for (int bb = 0; bb < SB; ++bb) {
    const int b = b0 + min(bb, nb - 1);  // rows past the batch re-read the last one
    const T* z = (const T*)p.z + (int64_t)b * p.z_stride;
    const float* xr = p.xdbl + (int64_t)b * xw + p.R + sg * NS;
    hv[bb] = *(const floatx4*)(p.h + ((int64_t)b * p.Di + c) * N + sg * NS);
    bv[bb] = *(const floatx4*)xr;
    cv[bb] = *(const floatx4*)(xr + N);
    xv[bb] = to_f32(z[p.xs_col + c]);
    gv[bb] = to_f32(z[p.g_col + c]);
  }
  const floatx4 av = *(const floatx4*)(p.A + (int64_t)c * N + sg * NS);
  const float Dc = p.D[c], bias = p.dt_bias[c];

  // This thread's first 4 slices of W_dt[c] (the whole row for R <= 4 * LPC * 8), also
  // loaded before anything waits.
  constexpr int RSTEP = LPC * 8;
  const T* wrow = (const T*)p.w_dt + (int64_t)c * p.R;
  Raw8<T> wv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (sg * 8 + u * RSTEP < p.R)
      wv[u].load(wrow + sg * 8 + u * RSTEP);
    else
      wv[u].zero();
  }
  // Stage the SB deltas, 4 loads in flight per thread per round.
  for (int i0 = tid; i0 < SB * p.R; i0 += 4 * 256) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * 256, bb = i / p.R, r = i % p.R;
      v[u] = (i < SB * p.R && bb < nb) ? p.xdbl[(int64_t)(b0 + bb) * xw + r] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * 256;
      if (i < SB * p.R) dl_s[i / p.R][i % p.R] = to_f32(from_f32<T>(v[u]));
    }
  }
  __syncthreads();
  float part[SB];
#pragma unroll
  for (int bb = 0; bb < SB; ++bb) part[bb] = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r0 = sg * 8 + u * RSTEP;
    if (r0 >= p.R) break;
#pragma unroll
    for (int bb = 0; bb < SB; ++bb)
#pragma unroll
      for (int e = 0; e < 8; ++e) part[bb] = fmaf(dl_s[bb][r0 + e], wv[u][e], part[bb]);
  }
  for (int r0 = sg * 8 + 4 * RSTEP; r0 < p.R; r0 += RSTEP) {  // R > 4 * LPC * 8 only
    float w1[8];
    load8v(wrow + r0, w1);
#pragma unroll
    for (int bb = 0; bb < SB; ++bb)
#pragma unroll
      for (int e = 0; e < 8; ++e) part[bb] = fmaf(dl_s[bb][r0 + e], w1[e], part[bb]);
  }

#pragma unroll
  for (int bb = 0; bb < SB; ++bb) {
    if (bb >= nb) break;  // uniform across the workgroup
    const int b = b0 + bb;
    const float dtv = softplus_f(group_sum<LPC>(part[bb]) + bias);
    const float dx = dtv * xv[bb];
    float acc = 0.f;
    floatx4 hn;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const float a = __builtin_amdgcn_exp2f(dtv * av[k] * kLog2e);
      hn[k] = fmaf(a, hv[bb][k], dx * bv[bb][k]);
      acc = fmaf(hn[k], cv[bb][k], acc);
    }
    acc = group_sum<LPC>(acc);
    if (!cok) continue;
    *(floatx4*)(p.h + ((int64_t)b * p.Di + c) * N + sg * NS) = hn;
    if (sg == 0) {
      const float yv = fmaf(Dc, xv[bb], acc);
      ((T*)p.y)[(int64_t)b * p.y_stride + c] = from_f32<T>(yv * silu_f(gv[bb]));
      if (c == 0 && p.pos != nullptr) p.pos[b] += 1;
    }
  }
}

template <typename T, int LPC>
static hipError_t run_step(const SsmStepParams& p, hipStream_t s) {
  // Two sequences per workgroup: the most workgroups (and the fewest registers) for
  // the state stream; the W_dt slice is re-read from L2 by each sequence pair.
  constexpr int SB = 2;
  const int blocks = (p.Di * LPC + 255) / 256;
  ssm_step_kernel<T, LPC, SB><<<dim3(blocks, (p.B + SB - 1) / SB), dim3(256), 0, s>>>(p);
  return hipGetLastError();
}

template <typename T>
static hipError_t step_dispatch(const SsmStepParams& p, hipStream_t s) {
  switch (p.N) {
    case 4: return run_step<T, 1>(p, s);
    case 8: return run_step<T, 2>(p, s);
    case 16: return run_step<T, 4>(p, s);
    case 32: return run_step<T, 8>(p, s);
    case 64: return run_step<T, 16>(p, s);
    case 128: return run_step<T, 32>(p, s);
    case 256: return run_step<T, 64>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_ssm_step(bool bf16_, const SsmStepParams& p, hipStream_t s) {
  if (p.B == 0 || p.Di == 0) return hipSuccess;
  return bf16_ ? step_dispatch<bf16>(p, s) : step_dispatch<float>(p, s);
}

}  // namespace hymba
