// Mamba-2 SSM head: one scalar decay and one dt per head (prefill in the chunked matrix
// form on MFMA, and the decode step).
//
// Source: the Chinese Hymba summary (metaphor-xennon.pages.dev), section 实现细节: the
// layer's SSM head is a Mamba-2 head built with a number of heads.  Reading: head h owns
// P channels and a P x N state S; dt_t = softplus(u_t + b_h) and A_h are scalars of the
// head, B_t and C_t (N each) are shared by all heads:
//   S_t = exp(dt_t A_h) S_{t-1} + dt_t x_t B_t^T ;  y_t = S_t C_t + D x_t ;  out = y SiLU(G)
// Within a chunk of Q tokens, with cs_i = sum_{r <= i} dt_r A_h (chunk-local prefix):
//   y_i   = sum_{j <= i} exp(cs_i - cs_j) dt_j (C_i . B_j) x_j + exp(cs_i) S_prev C_i + D x_i
//   S_new = exp(cs_{Q-1}) S_prev + sum_j exp(cs_{Q-1} - cs_j) dt_j x_j B_j^T
// so a chunk is four small products on v_mfma (bf16 operands, fp32 accumulation):
//   G^T = B C^T (Q x Q, K = N), masked, decayed and scaled by dt into M (bf16);
//   Y   = exp(cs) (C S_prev^T) + M X (Q x P, K = N, then K = Q);
//   S  += X^T (w B) (P x N, K = Q), w_j = exp(cs_{Q-1} - cs_j) dt_j, with w B split
//         into a bf16 high part and a bf16 low part so the carried state keeps about
//         16 significant bits;
// and the state stays in fp32 accumulators from chunk to chunk.  A workgroup owns one
// (sequence, head) and walks its chunks in order; the operands of the next one or two
// chunks are in flight to registers while the current one is multiplied.  Every sequence replays
// the batch-shared meta prefix; only sequence 0 stores the meta rows.
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

constexpr int kP = 64;       // channels per head
constexpr int kQ = 64;       // tokens per chunk
constexpr int kXP = kQ + 8;  // row pitch (bf16) of M, (w B)^T and the output tile

// X^T and G^T rows (channel p, 64 tokens) keep their eight 16-byte token chunks
// XOR-permuted by f(p) = (p ^ (p >> 3)) & 7: the transposing writes (8 lanes, channels
// 8 apart, same token) and the operand reads (8 lanes, 8 consecutive channels, same
// chunk) then each touch 8 distinct chunks, i.e. all 32 banks once.
__device__ __forceinline__ int xt_at(int p, int j) {
  return p * kQ + ((((j >> 3) ^ p ^ (p >> 3)) & 7) << 3) + (j & 7);
}

__device__ __forceinline__ int64_t ssd_row(int t, int b, int n_meta, int L) {
  return t < n_meta ? (int64_t)t : (int64_t)n_meta + (int64_t)b * L + (t - n_meta);
}

// v_mfma_f32_32x32x16_bf16: lane l supplies row (l % 32) of the first operand and
// column (l % 32) of the second, 8 consecutive k each (block l / 32); it receives
// D[(e/4)*8 + (l/32)*4 + e%4][l % 32].
__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int N>
struct SsdCfg {
  static constexpr int CP = N + 8;        // row pitch (bf16) of C, B, S
  static constexpr int NB = N / 16;       // 16-column state blocks
  static constexpr int LPR = N / 2;       // lanes per token row of [B | C] (16 bytes each)
  static constexpr int RPP = 256 / LPR;   // token rows per pass of the workgroup
  static constexpr int PASSES = kQ / RPP; // float4 loads of [B | C] per thread
};

}  // namespace

template <int N, int PD>
__global__ __launch_bounds__(256) void scan_ssd_kernel(SsdParams p) {
  using Cfg = SsdCfg<N>;
  constexpr int CP = Cfg::CP, NB = Cfg::NB, LPR = Cfg::LPR, RPP = Cfg::RPP, PASSES = Cfg::PASSES;
  __shared__ __attribute__((aligned(16))) bf16 c_s[kQ * CP];    // C [i][n]
  __shared__ __attribute__((aligned(16))) bf16 b_s[kQ * CP];    // B [j][n]
  __shared__ __attribute__((aligned(16))) bf16 xt_s[kP * kQ];   // X^T [p][j] (xt_at)
  __shared__ __attribute__((aligned(16))) bf16 gt_s[kP * kQ];   // G^T [p][i] (xt_at)
  __shared__ __attribute__((aligned(16))) bf16 m_s[kQ * kXP];   // M [i][j]
  __shared__ __attribute__((aligned(16))) bf16 y_s[kQ * kXP];   // gated output [i][p]
  __shared__ __attribute__((aligned(16))) bf16 wh_s[N * kXP];   // (w B)^T [n][j], high
  __shared__ __attribute__((aligned(16))) bf16 wl_s[N * kXP];   // low part
  __shared__ __attribute__((aligned(16))) bf16 s_s[kP * CP];    // S_prev [p][n]
  __shared__ __attribute__((aligned(16))) float cs_s[kQ], dt_s[kQ], ecs_s[kQ];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hd = blockIdx.x, b = blockIdx.y;
  const int T = p.n_meta + p.L;
  const int c0 = hd * kP;
  const float A = p.A[hd], bias = p.dt_bias[hd];
  const bf16* z = (const bf16*)p.z;
  const int64_t seq_off = (int64_t)b * p.L;  // row(t) = t, or t + b L past the meta prefix

  // Loads are coalesced: 8 lanes take one token's 64 channels of x (and of G), LPR lanes
  // one token's [B | C] row; wave 0's lane j takes token t0 + j's u.  Tokens past the end
  // read the last token's row (no load waits at its issue) and are zeroed where used.
  auto row_of = [&](int t) { return (int64_t)t + (t >= p.n_meta ? seq_off : 0); };
  const int xq = tid & 7, xj = tid >> 3;           // x / G: channel group, token (+32 r)
  const int bq = tid % LPR, bj = tid / LPR;        // [B | C]: float4 index, token (+RPP r)
  struct Ops {
    float u;
    floatx4 bc[PASSES];
    bf16x8 x[2], g[2];
  };
  auto fetch = [&](Ops& o, int t0) {
    if (wave == 0) o.u = p.xbc[row_of(min(t0 + lane, T - 1)) * p.xbc_ld + hd];
#pragma unroll
    for (int r = 0; r < PASSES; ++r)
      o.bc[r] = *(const floatx4*)(p.xbc + row_of(min(t0 + bj + r * RPP, T - 1)) * p.xbc_ld +
                                  p.H + bq * 4);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const bf16* zr = z + row_of(min(t0 + xj + 32 * r, T - 1)) * p.z_stride + c0 + xq * 8;
      o.x[r] = *(const bf16x8*)(zr + p.xs_col);
      o.g[r] = *(const bf16x8*)(zr + p.g_col);
    }
  };

  // ---- state: wave w holds rows p in [w*16, +16) of S as NB 16 x 16 accumulator blocks
  // (v_mfma_f32_16x16x32_bf16 layout: lane l has column l % 16, rows 4 (l / 16) + r)
  floatx4 st[NB];
  const int sp0 = wave * 16 + 4 * (lane >> 4);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      st[nb][r] = p.h0 ? p.h0[(int64_t)(c0 + sp0 + r) * N + nb * 16 + (lane & 15)] : 0.f;
  auto write_s = [&]() {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_s[(sp0 + r) * CP + nb * 16 + (lane & 15)] = (bf16)st[nb][r];
  };

  // Y block of this wave: rows i in [yi*32, +32), channels p in [yp*32, +32)
  const int yi = wave >> 1, yp = wave & 1;
  const int pl = yp * 32 + (lane & 31);
  const float Dc = p.D[c0 + pl];

  const int nchunks = (T + kQ - 1) / kQ;
  // One chunk from the operand set o, which is then refilled with chunk k + PD.
  auto chunk = [&](int k, Ops& o) {
    const int t0 = k * kQ;
    const bool ok = t0 + lane < T;
    // ---- A: dt, the decay prefix, and the operands into LDS
    if (wave == 0) {
      const float dt = ok ? softplus_f(o.u + bias) : 0.f;
      float cs = dt * A;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float v = __shfl_up(cs, off, 64);
        if (lane >= off) cs += v;
      }
      cs_s[lane] = cs;
      dt_s[lane] = dt;
      ecs_s[lane] = __expf(cs);
    }
#pragma unroll
    for (int r = 0; r < PASSES; ++r) {  // B (first N/4 lanes of a row) or C
      const int j = bj + r * RPP;
      const bool okj = t0 + j < T;
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (bf16)(okj ? o.bc[r][e] : 0.f);
      if (bq < LPR / 2)
        *(bf16x4*)(b_s + j * CP + bq * 4) = v;
      else
        *(bf16x4*)(c_s + j * CP + (bq - LPR / 2) * 4) = v;
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int j = xj + 32 * r;
      const bool okj = t0 + j < T;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xt_s[xt_at(xq * 8 + e, j)] = okj ? o.x[r][e] : (bf16)0.f;
        gt_s[xt_at(xq * 8 + e, j)] = o.g[r][e];
      }
    }
    lds_barrier();

    // ---- B: (w B)^T in two bf16 parts, and M from G^T = B C^T
    if (bq < LPR / 2) {  // threads holding B: w_j = 0 for tokens past the end (dt = 0)
#pragma unroll
      for (int r = 0; r < PASSES; ++r) {
        const int j = bj + r * RPP;
        const float w = __expf(cs_s[kQ - 1] - cs_s[j]) * dt_s[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = w * o.bc[r][e];
          const bf16 hi = (bf16)v;
          wh_s[(bq * 4 + e) * kXP + j] = hi;
          wl_s[(bq * 4 + e) * kXP + j] = (bf16)(v - (float)hi);
        }
      }
    }
    if (wave < 3) {  // blocks (i, j) of M: (0, 0), (1, 0), (1, 1); (0, 1) lies above the diagonal
      const int bi = wave == 0 ? 0 : 1, bj = wave == 2 ? 1 : 0;
      floatx16 g;
#pragma unroll
      for (int e = 0; e < 16; ++e) g[e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < N / 16; ++ks) {
        const int ko = ks * 16 + (lane >> 5) * 8;
        const bf16x8 fb = *(const bf16x8*)(b_s + (bj * 32 + (lane & 31)) * CP + ko);
        const bf16x8 fc = *(const bf16x8*)(c_s + (bi * 32 + (lane & 31)) * CP + ko);
        g = mfma32(fb, fc, g);  // D[j][i]
      }
      const int i = bi * 32 + (lane & 31);
      const float csi = cs_s[i];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j0 = bj * 32 + q * 8 + (lane >> 5) * 4;
        const floatx4 csj = *(const floatx4*)(cs_s + j0), dtj = *(const floatx4*)(dt_s + j0);
        bf16x4 m;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          m[r] = (bf16)(j0 + r <= i ? g[4 * q + r] * __expf(csi - csj[r]) * dtj[r] : 0.f);
        *(bf16x4*)(m_s + i * kXP + j0) = m;
      }
    }
    if (k + PD < nchunks) fetch(o, t0 + PD * kQ);  // o is all in LDS now
    lds_barrier();

    // ---- C: Y = exp(cs) (C S_prev^T) + M X, gated into y_s; then the state
    {
      floatx16 y;
#pragma unroll
      for (int e = 0; e < 16; ++e) y[e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < N / 16; ++ks) {
        const int ko = ks * 16 + (lane >> 5) * 8;
        const bf16x8 fc = *(const bf16x8*)(c_s + (yi * 32 + (lane & 31)) * CP + ko);
        const bf16x8 fs = *(const bf16x8*)(s_s + (yp * 32 + (lane & 31)) * CP + ko);
        y = mfma32(fc, fs, y);  // D[i][p]
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const floatx4 e4 = *(const floatx4*)(ecs_s + yi * 32 + q * 8 + (lane >> 5) * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) y[4 * q + r] *= e4[r];
      }
      const int kend = yi == 0 ? 2 : 4;  // rows i < 32 see keys j < 32 only
      for (int ks = 0; ks < kend; ++ks) {
        const int ko = ks * 16 + (lane >> 5) * 8;
        const bf16x8 fm = *(const bf16x8*)(m_s + (yi * 32 + (lane & 31)) * kXP + ko);
        const bf16x8 fx = *(const bf16x8*)(xt_s + xt_at(yp * 32 + (lane & 31), ko));
        y = mfma32(fm, fx, y);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i4 = yi * 32 + q * 8 + (lane >> 5) * 4;
        const bf16x4 xv = *(const bf16x4*)(xt_s + xt_at(pl, i4));
        const bf16x4 gv = *(const bf16x4*)(gt_s + xt_at(pl, i4));
#pragma unroll
        for (int r = 0; r < 4; ++r)
          y_s[(i4 + r) * kXP + pl] =
              (bf16)((y[4 * q + r] + Dc * (float)xv[r]) * silu_f((float)gv[r]));
      }
    }
    {
      const float el = ecs_s[kQ - 1];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[nb][r] *= el;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int ko = ks * 32 + (lane >> 4) * 8;
        const bf16x8 fx = *(const bf16x8*)(xt_s + xt_at(wave * 16 + (lane & 15), ko));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int row = (nb * 16 + (lane & 15)) * kXP + ko;
          st[nb] = mfma16x16x32(fx, *(const bf16x8*)(wh_s + row), st[nb]);
          st[nb] = mfma16x16x32(fx, *(const bf16x8*)(wl_s + row), st[nb]);
        }
      }
    }
    lds_barrier();
    write_s();  // S_prev of the next chunk (read only after the next barrier)
    // the chunk's output rows: 8 lanes store one row's 64 channels (one 128-byte line),
    // so a wave instruction writes 8 whole lines; the meta rows are stored by sequence 0
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int idx = tid + 256 * r, j = idx >> 3, p8 = (idx & 7) * 8, t = t0 + j;
      if (t < T && (t >= p.n_meta || b == 0))
        *(bf16x8*)((bf16*)p.y + row_of(t) * p.y_stride + c0 + p8) =
            *(const bf16x8*)(y_s + j * kXP + p8);
    }
  };

  write_s();
  if constexpr (PD == 1) {
    Ops o0;
    fetch(o0, 0);
    for (int k = 0; k < nchunks; ++k) chunk(k, o0);
  } else {
    static_assert(PD == 2, "prefetch depth");
    Ops o0, o1;
    fetch(o0, 0);
    if (nchunks > 1) fetch(o1, kQ);
    for (int k = 0; k < nchunks; k += 2) {
      chunk(k, o0);
      if (k + 1 < nchunks) chunk(k + 1, o1);
    }
  }

  if (p.h_out != nullptr) {
    float* ho = p.h_out + ((int64_t)b * p.H * kP + c0) * N;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) ho[(int64_t)(sp0 + r) * N + nb * 16 + (lane & 15)] = st[nb][r];
  }
}

bool scan_ssd_supported(int N, int Di, int H) {
  return H > 0 && H % 4 == 0 && Di == H * kP && (N == 16 || N == 32 || N == 64 || N == 128);
}

hipError_t launch_scan_ssd(const SsdParams& p, hipStream_t s) {
  if (p.B == 0 || p.n_meta + p.L == 0) return hipSuccess;
  if (!scan_ssd_supported(p.N, p.H * kP, p.H) || p.xbc_ld % 4 || p.z_stride % 8 ||
      p.xs_col % 8 || p.g_col % 8 || p.y_stride % 8)
    return hipErrorInvalidValue;
  const dim3 grid(p.H, p.B);
  switch (p.N) {
    // two chunks of operands in flight where the registers allow it
    case 16: scan_ssd_kernel<16, 2><<<grid, dim3(256), 0, s>>>(p); break;
    case 32: scan_ssd_kernel<32, 1><<<grid, dim3(256), 0, s>>>(p); break;
    case 64: scan_ssd_kernel<64, 1><<<grid, dim3(256), 0, s>>>(p); break;
    case 128: scan_ssd_kernel<128, 1><<<grid, dim3(256), 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// --------------------------------------------------------------------- decode step
// Thread per (channel, 4 states); the LPC = N / 4 lanes of a channel are adjacent and
// sum their C . S parts with xor shuffles.  dt, exp(dt A) and B, C are per sequence and
// head, read from the x_proj row [u | B | C].  The thread of state group 0 of channel 0
// advances pos[b]: every kernel that reads pos precedes this one.
template <int LPC>
__global__ __launch_bounds__(256) void ssm2_step_kernel(SsmStepParams p) {
  constexpr int N = 4 * LPC, CB = 256 / LPC;
  const int tid = threadIdx.x, sg = tid % LPC;
  const int c = blockIdx.x * CB + tid / LPC, b = blockIdx.y;
  const int hd = c / kP;
  const float* xr = p.xdbl + (int64_t)b * (p.heads + 2 * N);
  const float dt = softplus_f(xr[hd] + p.dt_bias[hd]);
  const float a = __expf(dt * p.A[hd]);
  const floatx4 bv = *(const floatx4*)(xr + p.heads + sg * 4);
  const floatx4 cv = *(const floatx4*)(xr + p.heads + N + sg * 4);
  const bf16* z = (const bf16*)p.z + (int64_t)b * p.z_stride;
  const float xv = (float)z[p.xs_col + c], gv = (float)z[p.g_col + c];
  float* hp = p.h + ((int64_t)b * p.Di + c) * N + sg * 4;
  floatx4 hv = *(floatx4*)hp;
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    hv[k] = fmaf(a, hv[k], dt * xv * bv[k]);
    acc = fmaf(hv[k], cv[k], acc);
  }
  *(floatx4*)hp = hv;
#pragma unroll
  for (int off = LPC / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (sg == 0) {
    ((bf16*)p.y)[(int64_t)b * p.y_stride + c] = (bf16)(fmaf(p.D[c], xv, acc) * silu_f(gv));
    if (c == 0 && p.pos != nullptr) p.pos[b] += 1;
  }
}

hipError_t launch_ssm2_step(const SsmStepParams& p, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  if (!scan_ssd_supported(p.N, p.Di, p.heads)) return hipErrorInvalidValue;
  const int lpc = p.N / 4, cb = 256 / lpc;
  if (p.Di % cb) return hipErrorInvalidValue;
  const dim3 grid(p.Di / cb, p.B);
  switch (lpc) {
    case 4: ssm2_step_kernel<4><<<grid, dim3(256), 0, s>>>(p); break;
    case 8: ssm2_step_kernel<8><<<grid, dim3(256), 0, s>>>(p); break;
    case 16: ssm2_step_kernel<16><<<grid, dim3(256), 0, s>>>(p); break;
    case 32: ssm2_step_kernel<32><<<grid, dim3(256), 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hymba
