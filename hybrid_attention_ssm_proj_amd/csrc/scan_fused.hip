// Prefill SSM heads with the dt projection fused in (bf16 path).
//
// Source: "Hymba: A Hybrid-head Architecture for Small Language Models" (outta.ai
// summary), Design formulation: the SSM head's mixing coefficient
// alpha_{i,j} = C_i (prod_{k=j+1..i} exp(A dt_k)) B_j dt_j and the gated output
// Y_ssm = G * (SSM output); dt = softplus(delta W_dt^T + b) with delta a low-rank
// linear map of the SSM input (Mamba).  Recurrent form per channel c and state n:
//   h_t[c,n] = exp(dt_t[c] A[c,n]) h_{t-1}[c,n] + dt_t[c] x_t[c] B_t[n]
//   y_t[c]   = sum_n C_t[n] h_t[c,n] + D[c] x_t[c];      out = y * SiLU(G)
//
// A workgroup owns (sequence, block of CB channels) and walks the sequence in chunks of
// TC tokens.  Per chunk:
//  * x, G, B, C and the delta rows are fetched with global_load_lds_dwordx4 into the
//    idle half of a double buffer while the previous chunk is scanned;
//  * dt^T [CB x TC] = W_dt[c0:c0+CB] delta^T runs on v_mfma_f32_16x16x32_bf16 (the W_dt
//    slice stays in LDS for the whole sequence), then softplus + bias;
//  * SiLU(G) is computed once per element;
//  * each lane advances NS states of one channel in fp32 registers, token by token;
//    the sum over states is a DPP butterfly across the channel's LPC lanes.
// delta rows keep their 16-byte chunks XOR-swizzled by (token & 15), so the 16 rows an
// MFMA operand read touches hit distinct LDS bank groups.  Every sequence replays the
// batch-shared meta prefix; only sequence 0 stores the meta rows.
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int LPC>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPC >= 2) v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (LPC >= 4) v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (LPC >= 8) v += dpp<0x141>(v);  // row_half_mirror
  if constexpr (LPC >= 16) v += dpp<0x140>(v); // row_mirror
  return v;
}

// Transpose-reduction over groups of LPC lanes: lane j of a group holds partials
// v[0..LPC) for LPC tokens; afterwards it holds the group's total for token j.  Each
// stage halves the list: the lane keeps the half matching its bit and adds what its
// partner (lane ^ 2^s) sends for that half.
template <int LPC>
__device__ __forceinline__ float transpose_reduce(float (&v)[LPC], int sg) {
  if constexpr (LPC == 1) {
    return v[0];
  } else if constexpr (LPC == 4) {
    // written out: two lane-bit selects per stage, masks computed once
    const bool b0 = sg & 1, b1 = sg & 2;
    const float q0 = (b0 ? v[1] : v[0]) + dpp<0xB1>(b0 ? v[0] : v[1]);
    const float q1 = (b0 ? v[3] : v[2]) + dpp<0xB1>(b0 ? v[2] : v[3]);
    return (b1 ? q1 : q0) + dpp<0x4E>(b1 ? q0 : q1);
  } else {
    int n = LPC;
#pragma unroll
    for (int st = 0; (1 << st) < LPC; ++st) {
      const bool bit = (sg >> st) & 1;
#pragma unroll
      for (int i = 0; i < LPC / 2; ++i) {
        if (2 * i + 1 < n) {
          const float keep = bit ? v[2 * i + 1] : v[2 * i];
          const float send = bit ? v[2 * i] : v[2 * i + 1];
          float recv;
          if ((1 << st) == 1)
            recv = dpp<0xB1>(send);
          else if ((1 << st) == 2)
            recv = dpp<0x4E>(send);
          else
            recv = __shfl_xor(send, 1 << st, 64);
          v[i] = keep + recv;
        }
      }
      n >>= 1;
    }
    return v[0];
  }
}

__device__ __forceinline__ int64_t seq_row(int t, int b, int n_meta, int L) {
  return t < n_meta ? (int64_t)t : (int64_t)n_meta + (int64_t)b * L + (t - n_meta);
}

}  // namespace

template <int NS, int LPC, int R>
struct FusedScanCfg {
  static constexpr int N = NS * LPC;
  static constexpr int CB = 256 / LPC;  // channels per workgroup
  static constexpr int TC = 32;         // tokens per chunk
  static constexpr int NC = R / 8;      // 16-byte chunks per delta row
  static constexpr int SWM = (NC < 16 ? NC : 16) - 1;  // swizzle mask
  static constexpr int XE = TC * CB;    // x / G / y elements per chunk
  static constexpr int X_SLOTS = XE / 8;
  static constexpr int BC_SLOTS = TC * N / 2;  // 2N floats per token
  static constexpr int D_SLOTS = TC * NC;
  static constexpr int WP = R + 8;      // W_dt slice row pitch (bf16)
  static constexpr int DTP = CB + 1;    // dt row pitch (fp32)
  static constexpr int PAIRS = (CB / 16) * (TC / 16);
  static_assert(X_SLOTS % 64 == 0 && BC_SLOTS % 64 == 0 && D_SLOTS % 64 == 0, "wave slots");
  static_assert(R % 32 == 0, "MFMA k-steps");
};

template <int NS, int LPC, int R>
__global__ __launch_bounds__(256) void scan_fused_kernel(ScanParams p, const bf16* __restrict__ delta,
                                                         const bf16* __restrict__ w_dt,
                                                         const float* __restrict__ dt_bias) {
  using C = FusedScanCfg<NS, LPC, R>;
  constexpr int N = C::N, CB = C::CB, TC = C::TC, NC = C::NC;
  __shared__ __attribute__((aligned(1024))) bf16 x_s0[C::XE];
  __shared__ __attribute__((aligned(1024))) bf16 x_s1[C::XE];
  __shared__ __attribute__((aligned(1024))) bf16 g_s0[C::XE];
  __shared__ __attribute__((aligned(1024))) bf16 g_s1[C::XE];
  __shared__ __attribute__((aligned(1024))) float bc_s0[TC * 2 * N];
  __shared__ __attribute__((aligned(1024))) float bc_s1[TC * 2 * N];
  __shared__ __attribute__((aligned(1024))) bf16 d_s0[TC * R];
  __shared__ __attribute__((aligned(1024))) bf16 d_s1[TC * R];
  __shared__ __attribute__((aligned(16))) bf16 w_s[CB * C::WP];
  __shared__ float dt_s[TC * C::DTP];
  __shared__ float bias_s[CB];
  __shared__ float gate_s[C::XE];
  __shared__ __attribute__((aligned(16))) bf16 y_s[C::XE];
  auto xs = [&](int i) { return i ? x_s1 : x_s0; };
  auto gs = [&](int i) { return i ? g_s1 : g_s0; };
  auto bcs = [&](int i) { return i ? bc_s1 : bc_s0; };
  auto ds = [&](int i) { return i ? d_s1 : d_s0; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cl = tid / LPC, sg = tid % LPC;
  const int c0 = blockIdx.x * CB;
  const int b = blockIdx.y;
  const int c = c0 + cl;  // Di % CB == 0 (checked on the host)
  const int total = p.n_meta + p.L;
  const bf16* z = (const bf16*)p.z;
  bf16* yout = (bf16*)p.y;

  // W_dt slice of the workgroup's channels, resident for the whole sequence.
  for (int q = tid; q < CB * NC; q += 256) {
    const int r = q / NC, j = q % NC;
    *(u32x4*)(w_s + r * C::WP + j * 8) = *(const u32x4*)(w_dt + (int64_t)(c0 + r) * R + j * 8);
  }
  float A2[NS], h[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    A2[k] = p.A[(int64_t)c * N + sg * NS + k] * kLog2e;
    h[k] = p.h0 != nullptr ? p.h0[(int64_t)c * N + sg * NS + k] : 0.f;
  }
  const float Dc = p.D[c];
  float beta8[8];
  static_assert(256 % (CB / 8) == 0, "store-phase channel group is fixed per thread");
#pragma unroll
  for (int e = 0; e < 8; ++e)
    beta8[e] = p.beta != nullptr ? p.beta[c0 + (tid % (CB / 8)) * 8 + e] : 1.f;
  for (int i = tid; i < CB; i += 256) bias_s[i] = dt_bias[c0 + i];

  // Stage chunk `t0` into buffer `buf`.  Slot q of an array is written by lane q % 64
  // of the wave instruction covering slots [64*(q/64), +64), at LDS address base +
  // 16*q; rows past the sequence load its last row (never used).
  auto stage = [&](int buf, int t0) {
    auto row_of = [&](int tt) { return seq_row(min(t0 + tt, total - 1), b, p.n_meta, p.L); };
#pragma unroll
    for (int j = 0; j < (C::X_SLOTS + 255) / 256; ++j) {
      const int q0 = j * 256 + wave * 64;
      if (q0 < C::X_SLOTS) {
        const int q = q0 + lane;
        const int tt = q / (CB / 8), j16 = q % (CB / 8);
        const int64_t rb = row_of(tt) * p.z_stride + c0 + j16 * 8;
        __builtin_amdgcn_global_load_lds((glb_void_t*)(z + rb + p.xs_col),
                                         (lds_void_t*)(xs(buf) + q0 * 8), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(z + rb + p.g_col),
                                         (lds_void_t*)(gs(buf) + q0 * 8), 16, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < (C::BC_SLOTS + 255) / 256; ++j) {
      const int q0 = j * 256 + wave * 64;
      if (q0 < C::BC_SLOTS) {
        const int q = q0 + lane;
        const int tt = q / (N / 2), j16 = q % (N / 2);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(p.bc + row_of(tt) * 2 * N + j16 * 4),
                                         (lds_void_t*)(bcs(buf) + q0 * 4), 16, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < (C::D_SLOTS + 255) / 256; ++j) {
      const int q0 = j * 256 + wave * 64;
      if (q0 < C::D_SLOTS) {
        const int q = q0 + lane;
        const int tt = q / NC, s = q % NC;
        const int cidx = s ^ (tt & C::SWM);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(delta + row_of(tt) * R + cidx * 8),
                                         (lds_void_t*)(ds(buf) + q0 * 8), 16, 0, 0);
      }
    }
  };

  const int nchunk = (total + TC - 1) / TC;
  stage(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  for (int k = 0; k < nchunk; ++k) {
    const int cur = k & 1;
    const int t0 = k * TC;
    const int tn = min(TC, total - t0);
    if (k + 1 < nchunk) stage(cur ^ 1, t0 + TC);

    // dt^T for the chunk: MFMA tiles of 16 channels x 16 tokens, k over the rank.
    for (int pi = wave; pi < C::PAIRS; pi += 4) {
      const int rbk = pi / (TC / 16), cbk = pi % (TC / 16);
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      const int tt = cbk * 16 + (lane & 15);
#pragma unroll
      for (int ks = 0; ks < R / 32; ++ks) {
        const int cidx = ks * 4 + (lane >> 4);
        const bf16x8 a = *(const bf16x8*)(w_s + (rbk * 16 + (lane & 15)) * C::WP + cidx * 8);
        const bf16x8 bb = *(const bf16x8*)(ds(cur) + (tt * NC + (cidx ^ (tt & C::SWM))) * 8);
        acc = mfma16x16x32(a, bb, acc);
      }
      // lane holds D[channel rbk*16 + 4*(lane/16) + i][token cbk*16 + lane%16]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = rbk * 16 + (lane >> 4) * 4 + i;
        dt_s[tt * C::DTP + ch] = tt < tn ? softplus_f(acc[i] + bias_s[ch]) : 0.f;
      }
    }
    for (int e = tid; e < C::XE; e += 256) gate_s[e] = silu_f((float)gs(cur)[e]);
    lds_barrier();  // the next chunk's loads stay in flight

    // Tokens in groups of LPC.  With few states per lane group (LPC * NS <= 16) the LDS
    // reads of group i + 1 are issued before the state updates of group i (two register
    // sets), so their latency hides behind the exponentials, and all TC tokens run:
    // tokens past the chunk have dt = 0, which leaves h unchanged (exp2(0) = 1 and a zero
    // input term), and their outputs are never stored.  Larger groups read just in time.
    // The transpose-reduction leaves lane sg with the full state sum of token g0 + sg, so
    // every lane finishes one token's output.
    const bf16* xc = xs(cur);
    const float* bcc = bcs(cur);
    constexpr bool kPipe = LPC * NS <= 16;
    float dtv[2][LPC], xv[2][LPC], bv[2][LPC][NS], cv[2][LPC][NS];
    auto fetch = [&](int slot, int g0) {
#pragma unroll
      for (int u = 0; u < LPC; ++u) {
        const int tt = g0 + u;
        dtv[slot][u] = dt_s[tt * C::DTP + cl];
        xv[slot][u] = (float)xc[tt * CB + cl];
        const float* brow = bcc + tt * 2 * N + sg * NS;
#pragma unroll
        for (int k4 = 0; k4 < NS; k4 += 4) {
          const floatx4 b4 = *(const floatx4*)(brow + k4);
          const floatx4 c4 = *(const floatx4*)(brow + N + k4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bv[slot][u][k4 + e] = b4[e];
            cv[slot][u][k4 + e] = c4[e];
          }
        }
      }
    };
    auto group = [&](int sl, int g0) {
      float part[LPC];
#pragma unroll
      for (int u = 0; u < LPC; ++u) {
        const float dx = dtv[sl][u] * xv[sl][u];
        float acc = 0.f;
#pragma unroll
        for (int kk = 0; kk < NS; ++kk) {
          const float a = __builtin_amdgcn_exp2f(dtv[sl][u] * A2[kk]);
          h[kk] = fmaf(a, h[kk], dx * bv[sl][u][kk]);
          acc = fmaf(h[kk], cv[sl][u][kk], acc);
        }
        part[u] = acc;
      }
      const float tot = transpose_reduce<LPC>(part, sg);
      const int tt = g0 + sg;
      const float xt = (float)xc[tt * CB + cl];
      y_s[tt * CB + cl] = (bf16)(fmaf(Dc, xt, tot) * gate_s[tt * CB + cl]);
    };
    if constexpr (kPipe) {
      fetch(0, 0);
#pragma unroll
      for (int gi = 0; gi < TC / LPC; ++gi) {
        if (gi + 1 < TC / LPC) fetch((gi & 1) ^ 1, (gi + 1) * LPC);
        group(gi & 1, gi * LPC);
      }
    } else {
      for (int g0 = 0; g0 < tn; g0 += LPC) {
        float dtw[LPC], xw[LPC], bw[LPC][NS], cw[LPC][NS];
#pragma unroll
        for (int u = 0; u < LPC; ++u) {
          const int tt = g0 + u;
          dtw[u] = dt_s[tt * C::DTP + cl];
          xw[u] = (float)xc[tt * CB + cl];
          const float* brow = bcc + tt * 2 * N + sg * NS;
#pragma unroll
          for (int k4 = 0; k4 < NS; k4 += 4) {
            const floatx4 b4 = *(const floatx4*)(brow + k4);
            const floatx4 c4 = *(const floatx4*)(brow + N + k4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              bw[u][k4 + e] = b4[e];
              cw[u][k4 + e] = c4[e];
            }
          }
        }
        float part[LPC];
#pragma unroll
        for (int u = 0; u < LPC; ++u) {
          const float dx = dtw[u] * xw[u];
          float acc = 0.f;
#pragma unroll
          for (int kk = 0; kk < NS; ++kk) {
            const float a = __builtin_amdgcn_exp2f(dtw[u] * A2[kk]);
            h[kk] = fmaf(a, h[kk], dx * bw[u][kk]);
            acc = fmaf(h[kk], cw[u][kk], acc);
          }
          part[u] = acc;
        }
        const float tot = transpose_reduce<LPC>(part, sg);
        const int tt = g0 + sg;
        const float xt = (float)xc[tt * CB + cl];
        y_s[tt * CB + cl] = (bf16)(fmaf(Dc, xt, tot) * gate_s[tt * CB + cl]);
      }
    }
    lds_barrier();

    // Store: thread q takes 8 channels of one token (8 consecutive lanes per token).  With
    // p.ssp the token row's sum of y^2 (of the rounded y, as a norm reading stored Y_ssm
    // sees it) over the workgroup's channels goes to ssp[ssp_col0 + blockIdx.x, row] and
    // beta * y is stored.
    for (int q = tid; q < C::X_SLOTS; q += 256) {
      const int tt = q / (CB / 8), j16 = q % (CB / 8);
      const int t = t0 + tt;
      const bool keep = tt < tn && (t >= p.n_meta || b == 0);
      const int64_t row = seq_row(min(t, total - 1), b, p.n_meta, p.L);
      bf16x8 o = *(const bf16x8*)(y_s + q * 8);
      if (p.ssp != nullptr) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)o[e];
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sq = fmaf(v[e], v[e], sq);
        sq = group_sum<CB / 8>(sq);
        if (keep && j16 == 0) p.ssp[(p.ssp_col0 + blockIdx.x) * p.ssp_ld + row] = sq;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (bf16)(v[e] * beta8[e]);
      }
      if (keep) *(bf16x8*)(yout + row * p.y_stride + c0 + j16 * 8) = o;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's DMA for the next chunk has landed
    lds_barrier();
  }

  if (p.h_out != nullptr) {
    float* dst = p.h_out + ((int64_t)b * p.Di + c) * N + sg * NS;
#pragma unroll
    for (int k = 0; k < NS; ++k) dst[k] = h[k];
  }
}

template <int NS, int LPC, int R>
static hipError_t run_fused(const ScanParams& p, const void* delta, const void* w_dt,
                            const float* bias, hipStream_t s) {
  constexpr int CB = 256 / LPC;
  if (p.Di % CB) return hipErrorInvalidValue;
  scan_fused_kernel<NS, LPC, R><<<dim3(p.Di / CB, p.B), dim3(256), 0, s>>>(
      p, (const bf16*)delta, (const bf16*)w_dt, bias);
  return hipGetLastError();
}

template <int R>
static hipError_t fused_by_state(const ScanParams& p, const void* delta, const void* w_dt,
                                 const float* bias, hipStream_t s) {
  switch (p.N) {
    case 16: return run_fused<4, 4, R>(p, delta, w_dt, bias, s);
    case 32: return run_fused<4, 8, R>(p, delta, w_dt, bias, s);
    case 64: return run_fused<8, 8, R>(p, delta, w_dt, bias, s);
    case 128: return run_fused<8, 16, R>(p, delta, w_dt, bias, s);
    default: return hipErrorInvalidValue;
  }
}

int scan_channel_blocks(int N, int Di) {
  // channels per workgroup: 256 / LPC with LPC = 4, 8, 8, 16 for N = 16, 32, 64, 128
  const int cb = N == 16 ? 64 : (N == 128 ? 16 : 32);
  return Di / cb;
}

bool scan_fused_supported(int N, int R, int Di) {
  if (R != 64 && R != 128) return false;
  int cb = 0;
  switch (N) {
    case 16: cb = 64; break;
    case 32: case 64: cb = 32; break;
    case 128: cb = 16; break;
    default: return false;
  }
  return Di % cb == 0;
}

hipError_t launch_scan_prefill_fused(const ScanParams& p, const void* delta, const void* w_dt,
                                     const float* dt_bias, int R, hipStream_t s) {
  if (p.B == 0 || p.Di == 0 || p.n_meta + p.L == 0) return hipSuccess;
  if (R == 128) return fused_by_state<128>(p, delta, w_dt, dt_bias, s);
  if (R == 64) return fused_by_state<64>(p, delta, w_dt, dt_bias, s);
  return hipErrorInvalidValue;
}

}  // namespace hymba
