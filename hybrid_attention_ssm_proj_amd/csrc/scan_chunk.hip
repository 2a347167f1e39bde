// Prefill SSM heads (bf16 path): dt projection, selective scan and gate, chunk-carried
// over time.
//
// Source: "Hymba: A Hybrid-head Architecture for Small Language Models" (outta.ai
// summary), Design formulation: the SSM head's mixing coefficient
// alpha_{i,j} = C_i (prod_{k=j+1..i} exp(A dt_k)) B_j dt_j and the gated output
// Y_ssm = G * (SSM output); dt = softplus(delta W_dt^T + b) with delta a low-rank linear
// map of the SSM input (Mamba).  Recurrent form per channel c and state n:
//   h_t[c,n] = exp(dt_t[c] A[c,n]) h_{t-1}[c,n] + dt_t[c] x_t[c] B_t[n]
//   y_t[c]   = sum_n C_t[n] h_t[c,n] + D[c] x_t[c];      out = y * SiLU(G)
//
// Time chunks.  Because the recurrence is linear in h, the state after a span of tokens
// is P * h_in + h_loc, where P[c,n] = prod exp(A dt_k) = exp(A[c,n] * sum_k dt_k[c]) and
// h_loc is the span's end state when it starts from zero.  A sequence of T tokens is cut
// into chunks of `chunk` tokens and scanned in three launches:
//   1. summary: every chunk but the last, from zero -> h_loc and sum(dt) per channel;
//   2. carry: per (sequence, channel, state), an inclusive scan over the chunks inside a
//      wavefront (lanes = chunks, shuffles in log2 steps) with the composition
//      (P1, h1) then (P2, h2) = (P1 P2, P2 h1 + h2), seeded with the initial state;
//   3. main: every chunk from its carried state, producing outputs and the final h.
// With one chunk only launch 3 runs.  Chunks multiply the workgroups available to a
// short batch (B * Di / 64 without them) at the price of a second pass over all but the
// last chunk (about 3/4 of the main pass's instructions: no C, no outputs).
//
// Workgroup layout.  A workgroup owns 64 channels (one per lane) of one (sequence,
// chunk); wave w owns states [w*NS, (w+1)*NS) of those channels.  B_t and C_t are then
// the same for every lane of a wave and are read through the scalar data cache into
// scalar registers: no vector memory or LDS bandwidth is spent broadcasting them.  Per
// step of 16 or 32 tokens (32 when the grid is small enough for its LDS):
//  * x, G and the delta rows move global -> LDS by DMA (double-buffered, issued from
//    inline asm so the compiler adds no waits for them);
//  * dt for 16 tokens x 64 channels is one 16x16x32 MFMA tile per 16 channels over the
//    rank (the W_dt rows stay in registers; one tile row per 16 tokens of the step), then
//    bias + softplus; (dt, dt x) go to LDS;
//  * each wave runs its NS states over the 16 tokens in registers (4 VALU + 1 exp per
//    state and token) and writes its part of sum_n C h to LDS;
//  * the parts of the W waves are added, D x and the gate applied, and the row stored.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace hymba {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
// Output stores go through global-address-space pointers: through a generic pointer the
// compiler cannot rule out an LDS target and waits for every store in flight (vmcnt(0))
// before the next LDS read.
typedef __attribute__((address_space(1))) bf16x4 glb_bf16x4;
typedef __attribute__((address_space(1))) float glb_float;
typedef __attribute__((ext_vector_type(2))) float floatx2;
typedef __attribute__((address_space(4))) const floatx4 const_floatx4;
typedef __attribute__((address_space(4))) const floatx2 const_floatx2;

// NS floats at a wave-uniform address, loaded through the scalar data cache.  The buffer
// is written by an earlier launch and only read here.
// NS consecutive floats that every lane reads at the same LDS address (a broadcast).
template <int NS>
__device__ __forceinline__ void lds_uniform_load(float (&d)[NS], const float* p) {
  if constexpr (NS % 4 == 0) {
#pragma unroll
    for (int j = 0; j < NS; j += 4) {
      const floatx4 v = *(const floatx4*)(p + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) d[j + e] = v[e];
    }
  } else {
#pragma unroll
    for (int j = 0; j < NS; ++j) d[j] = p[j];
  }
}

template <int NS>
__device__ __forceinline__ void uniform_load(float (&d)[NS], const float* p) {
  if constexpr (NS % 4 == 0) {
#pragma unroll
    for (int j = 0; j < NS; j += 4) {
      const floatx4 v = *(const const_floatx4*)(p + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) d[j + e] = v[e];
    }
  } else {
    static_assert(NS == 2, "2 or a multiple of 4 states");
    const floatx2 v = *(const const_floatx2*)p;
    d[0] = v[0];
    d[1] = v[1];
  }
}
// NS consecutive floats per lane (16- or 8-byte accesses).
template <int NS>
__device__ __forceinline__ void lane_load(float (&d)[NS], const float* p) {
  if constexpr (NS % 4 == 0) {
#pragma unroll
    for (int j = 0; j < NS; j += 4) {
      const floatx4 v = *(const floatx4*)(p + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) d[j + e] = v[e];
    }
  } else {
    const floatx2 v = *(const floatx2*)p;
    d[0] = v[0];
    d[1] = v[1];
  }
}
template <int NS>
__device__ __forceinline__ void lane_store(float* p, const float (&d)[NS]) {
  if constexpr (NS % 4 == 0) {
#pragma unroll
    for (int j = 0; j < NS; j += 4) {
      const floatx4 v = {d[j], d[j + 1], d[j + 2], d[j + 3]};
      *(floatx4*)(p + j) = v;
    }
  } else {
    const floatx2 v = {d[0], d[1]};
    *(floatx2*)p = v;
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// Sum over each row of 16 lanes.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

// global_load_lds_dwordx4 of one 16-byte piece per lane into the wave's 1 KB LDS block at
// `lptr`, issued from inline asm.  The compiler does not see this LDS write, so it puts no
// conservative vmcnt wait in front of LDS reads of the other buffer (with the builtin it
// waits for every transfer in flight before any LDS read, which empties the double
// buffer).  The kernel waits for its own transfers (vmcnt) and then passes a barrier.  The
// instruction has no register result; its address operands are read at issue.
__device__ __forceinline__ void dma16(const void* gptr, lds_void_t* lptr) {
  const uint32_t l = (uint32_t)(uintptr_t)lptr;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(l)), "v"(gptr) : "memory", "m0");
}

// s_waitcnt vmcnt(n) for a wave-uniform n (at most 15; larger n waits for everything).
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  switch (n) {
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

template <int NS, int W, int R, int TC_>
struct ChunkCfg {
  static constexpr int N = NS * W;
  static constexpr int CB = 64;              // channels per workgroup, one per lane
  static constexpr int TC = TC_;             // tokens per step
  static constexpr int NT = 64 * W;          // threads
  static constexpr int NC = R / 8;           // 16-byte pieces per delta row
  static constexpr int SWM = (NC < 16 ? NC : 16) - 1;  // delta piece swizzle mask
  static constexpr int X_SLOTS = TC * CB / 8;          // 16-byte pieces of x (or G) per step
  static constexpr int D_SLOTS = TC * NC;              // ... of delta per step
  static constexpr int TPW = (4 + W - 1) / W;  // dt tiles (16 channels each) per wave
  static_assert((NS == 2 || NS % 4 == 0) && NS <= 16, "state group");
  static_assert(TC == 16 || TC == 32, "16-token MFMA tile rows per step");
  static_assert(R % 32 == 0, "MFMA k-steps");
};

}  // namespace

// kSum: summary pass (chunks 0 .. nchunks-2 from zero: end state and sum of dt).
// TC: tokens per step (32 halves the barriers and per-step costs per token where the LDS
// it takes still lets two workgroups share a CU; 16 otherwise).
template <int NS, int W, int R, bool kSum, int TC_>
__global__ __launch_bounds__(64 * W) void scan_chunk_kernel(ScanChunkParams p) {
  using C = ChunkCfg<NS, W, R, TC_>;
  constexpr int N = C::N, CB = C::CB, TC = C::TC, NC = C::NC, NT = C::NT;
  // Tokens per group of scalar loads.  With up to 8 states per wave two groups' B and C
  // rows are in flight at once (32 scalar registers; the summary pass reads B only);
  // with 16 the scalar registers hold one group, loaded just before it runs.
  constexpr bool kDB = NS <= 8;
  constexpr int GT = (kSum ? 16 : 8) / NS > 0 ? (kSum ? 16 : 8) / NS : 1;
  // kBCL (32-token steps, at most 16 states): the step's B|C rows are staged in LDS with
  // its other operands and read from there (broadcast reads); the delta rows take one
  // buffer, refilled for the next step once this step's dt phase has read them, which
  // keeps the LDS at the 80 KB that lets two workgroups share a CU.  Otherwise B and C
  // come through the scalar cache and the delta rows are double-buffered.
  constexpr bool kBCL = TC == 32 && N <= 16;
  constexpr int DBUF = kBCL ? 1 : 2;
  __shared__ __attribute__((aligned(1024))) bf16 x_s[2][TC * CB];
  __shared__ __attribute__((aligned(1024))) bf16 g_s[2][kSum ? 8 : TC * CB];
  __shared__ __attribute__((aligned(1024))) bf16 d_s[DBUF][TC * R];
  __shared__ __attribute__((aligned(1024))) float bc_s[kBCL ? 2 : 1][kBCL ? TC * 2 * N : 4];
  __shared__ __attribute__((aligned(16))) float2 dd_s[TC * CB];
  __shared__ __attribute__((aligned(16))) float part_s[kSum ? 4 : W * TC * CB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = blockIdx.x * CB;
  const int c = c0 + lane;
  const int nck = kSum ? p.nchunks - 1 : p.nchunks;
  const int b = blockIdx.y / nck, k = blockIdx.y % nck;
  const int tb = k * p.chunk, te = min(tb + p.chunk, p.T);
  const int n0 = wave * NS;
  // Everything the step loop addresses, from the sequence's token 0 (rows are consecutive).
  const int64_t rbase = (int64_t)p.row0 + (int64_t)b * p.T;
  const int64_t zst = p.z_stride;
  const bf16* zx = (const bf16*)p.z + rbase * zst + c0 + p.xs_col;
  const int64_t gofs = (int64_t)p.g_col - p.xs_col;
  const bf16* dl = (const bf16*)p.delta + rbase * R;
  const float* bcs = p.bc + rbase * (2 * N) + n0;
  bf16* ys = (bf16*)p.y + rbase * p.y_stride + c0;
  const int64_t yst = p.y_stride;
  float* ssps = p.ssp != nullptr ? p.ssp + (p.ssp_col0 + blockIdx.x) * p.ssp_ld + rbase : nullptr;
  const int64_t DN = (int64_t)p.Di * N;
  float* hdst = kSum ? p.hsum + ((int64_t)b * (p.nchunks - 1) + k) * DN
                     : (k == p.nchunks - 1 && p.h_out != nullptr ? p.h_out + (int64_t)b * DN
                                                                 : nullptr);
  float* sdst = kSum ? p.ssum + ((int64_t)b * (p.nchunks - 1) + k) * p.Di : nullptr;

  // The W_dt rows of this wave's dt tiles (the MFMA's B operand: lane l holds channel
  // rbk * 16 + l % 16, pieces ks * 4 + l / 16 of the rank) and their biases stay in
  // registers for the whole chunk.
  bf16x8 wfrag[C::TPW][R / 32];
  float bias[C::TPW];
#pragma unroll
  for (int t = 0; t < C::TPW; ++t) {
    const int rbk = wave + t * W;
    const int ch = c0 + (rbk < CB / 16 ? rbk : 0) * 16 + (lane & 15);
#pragma unroll
    for (int ks = 0; ks < R / 32; ++ks)
      wfrag[t][ks] = *(const bf16x8*)((const bf16*)p.w_dt + (int64_t)ch * R +
                                      (ks * 4 + (lane >> 4)) * 8);
    bias[t] = p.dt_bias[ch];
  }

  float A2[NS], h[NS];
  {
    const float* src = nullptr;
    if (!kSum) src = k == 0 ? p.h0 : p.hsum + ((int64_t)b * (p.nchunks - 1) + (k - 1)) * DN;
    lane_load<NS>(A2, p.A + (int64_t)c * N + n0);
#pragma unroll
    for (int e = 0; e < NS; ++e) {
      A2[e] *= kLog2eF;
      h[e] = 0.f;
    }
    if (src != nullptr) lane_load<NS>(h, src + (int64_t)c * N + n0);
  }
  float D4[4] = {0.f, 0.f, 0.f, 0.f}, beta4[4] = {1.f, 1.f, 1.f, 1.f};
  if (!kSum) {
    const int cj = c0 + (tid & 15) * 4;  // the epilogue's 4 channels (fixed per thread)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      D4[e] = p.D[cj + e];
      if (p.beta != nullptr) beta4[e] = p.beta[cj + e];
    }
  }
  float dtsum = 0.f;

  const float* bcrow = p.bc + rbase * (2 * N);  // the rows' B|C (every state)
  auto stage_delta = [&](int buf, int s0) {
#pragma unroll
    for (int i = 0; i * NT < C::D_SLOTS; ++i) {
      const int q0 = i * NT + wave * 64;
      if (q0 < C::D_SLOTS) {
        const int q = q0 + lane, tt = q / NC, s = q % NC;
        const int cidx = s ^ (tt & C::SWM);
        dma16(dl + min(s0 + tt, te - 1) * R + cidx * 8, (lds_void_t*)(d_s[buf] + q0 * 8));
      }
    }
  };
  // Stage the step starting at sequence token s0 into buffer `buf`.  Piece q of an array
  // is written by lane q % 64 of the wave instruction covering pieces [64*(q/64), +64), at
  // LDS address base + 16*q.  Tokens past the chunk load its last row (never used).
  auto stage = [&](int buf, int s0) {
#pragma unroll
    for (int i = 0; i * NT < C::X_SLOTS; ++i) {
      const int q0 = i * NT + wave * 64;
      if (q0 < C::X_SLOTS) {
        const int q = q0 + lane, tt = q >> 3, j16 = q & 7;
        const bf16* src = zx + min(s0 + tt, te - 1) * zst + j16 * 8;
        dma16(src, (lds_void_t*)(x_s[buf] + q0 * 8));
        if (!kSum) dma16(src + gofs, (lds_void_t*)(g_s[buf] + q0 * 8));
      }
    }
    if constexpr (kBCL) {  // the B|C rows of the step, 2N floats each
      constexpr int BC_SLOTS = TC * 2 * N / 4;
#pragma unroll
      for (int i = 0; i * NT < BC_SLOTS; ++i) {
        const int q0 = i * NT + wave * 64;
        if (q0 < BC_SLOTS) {
          const int q = q0 + lane, tt = q / (2 * N / 4), pc = q % (2 * N / 4);
          dma16(bcrow + min(s0 + tt, te - 1) * (2 * N) + pc * 4, (lds_void_t*)(bc_s[buf] + q0 * 4));
        }
      }
    } else {
      stage_delta(buf, s0);
    }
  };

  // store instructions this wave issues in a step's output phase (y, and the partial sum
  // of squares when kept): its share of the TC * 16 output items, NT per round
  const int epi_stores = kSum ? 0
                              : max(0, (TC * 16 - wave * 64 + NT - 1) / NT) *
                                    (ssps != nullptr ? 2 : 1);
  const int nst = (te - tb + TC - 1) / TC;  // 0 for an empty sequence: h passes through
  if (nst > 0) {
    stage(0, tb);
    if constexpr (kBCL) stage_delta(0, tb);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    const int s0 = tb + st * TC;
    const int tn = min(TC, te - s0);
    if (st + 1 < nst) stage(cur ^ 1, s0 + TC);

    // dt [16 tokens x 16 channels] per tile: delta rows (A operand) times W_dt rows
    // (B operand) over the rank; lane l ends with tokens 4*(l/16) + i of channel l % 16.
#pragma unroll
    for (int tw = 0; tw < C::TPW; ++tw) {
      const int rbk = wave + tw * W;
      if (rbk >= CB / 16) break;
      const int chl = rbk * 16 + (lane & 15);
#pragma unroll
      for (int th = 0; th < TC / 16; ++th) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        const int tt = th * 16 + (lane & 15);
#pragma unroll
        for (int ks = 0; ks < R / 32; ++ks) {
          const int cidx = ks * 4 + (lane >> 4);
          const bf16x8 a =
              *(const bf16x8*)(d_s[kBCL ? 0 : cur] + (tt * NC + (cidx ^ (tt & C::SWM))) * 8);
          acc = mfma16x16x32(a, wfrag[tw][ks], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = th * 16 + 4 * (lane >> 4) + i;
          const float dt = t < tn ? softplus_f(acc[i] + bias[tw]) : 0.f;
          const float xv = (float)x_s[cur][t * CB + chl];
          dd_s[t * CB + chl] = make_float2(dt, dt * xv);
        }
      }
    }
    lds_barrier();
    // single delta buffer: every wave has read this step's rows, refill it for the next
    // step (lands during the recurrence; the step's closing wait covers it)
    if constexpr (kBCL) {
      if (st + 1 < nst) stage_delta(0, s0 + TC);
    }

    // The recurrence over the step's tokens, GT at a time; the B (and C) rows of a group
    // arrive in scalar registers through the scalar cache.  Tokens past the chunk have
    // dt = 0, which leaves h unchanged (exp(0) = 1, zero input term).
    // kFull: a whole step, whose rows are consecutive from the step's first, so every
    // scalar load is the step's base address plus a constant; the last step of a chunk
    // may be partial and clamps its rows to the chunk's last.
    auto recurrence = [&](auto full) {
      constexpr bool kFull = decltype(full)::value;
      const float* bstep = bcs + (int64_t)s0 * (2 * N);
      const int tlast = te - 1 - s0;
      constexpr int NCQ = kSum ? 1 : NS;  // the summary pass reads no C
      float bq0[GT][NS], cq0[GT][NCQ], bq1[GT][NS], cq1[GT][NCQ];
      float2 dd0[GT], dd1[GT];
      // a group's operands: (dt, dt x) from LDS, the B (and C) rows from the scalar cache
      auto load = [&](float2 (&dd)[GT], float (&bq)[GT][NS], float (&cq)[GT][NCQ], int g0) {
#pragma unroll
        for (int u = 0; u < GT; ++u) {
          dd[u] = dd_s[(g0 + u) * CB + lane];
          if constexpr (kBCL) {  // staged rows (past the chunk: copies of its last row)
            lds_uniform_load<NS>(bq[u], bc_s[cur] + (g0 + u) * (2 * N) + n0);
            if constexpr (!kSum) lds_uniform_load<NS>(cq[u], bc_s[cur] + (g0 + u) * (2 * N) + N + n0);
          } else {
            const float* brow = bstep + (kFull ? g0 + u : min(g0 + u, tlast)) * (2 * N);
            uniform_load<NS>(bq[u], brow);
            if constexpr (!kSum) uniform_load<NS>(cq[u], brow + N);
          }
        }
      };
      auto run = [&](const float2 (&dd)[GT], const float (&bq)[GT][NS],
                     const float (&cq)[GT][NCQ], int g0) {
#pragma unroll
        for (int u = 0; u < GT; ++u) {
          const float2 d = dd[u];
          float acc = 0.f;
#pragma unroll
          for (int kk = 0; kk < NS; ++kk) {
            const float a = __builtin_amdgcn_exp2f(d.x * A2[kk]);
            h[kk] = fmaf(a, h[kk], d.y * bq[u][kk]);
            if constexpr (!kSum) acc = fmaf(h[kk], cq[u][kk], acc);
          }
          if (kSum) dtsum += d.x;
          else part_s[(wave * TC + g0 + u) * CB + lane] = acc;
        }
      };
      if constexpr (!kDB) {
#pragma unroll
        for (int g0 = 0; g0 < TC; g0 += GT) {
          load(dd0, bq0, cq0, g0);
          run(dd0, bq0, cq0, g0);
        }
        return;
      }
      // Two operand sets: the next group's loads are issued before the current group
      // runs, behind an explicit wait for everything requested so far (scalar loads
      // complete out of order, so only a full wait is exact).
      load(dd0, bq0, cq0, 0);
#pragma unroll
      for (int g0 = 0; g0 < TC; g0 += 2 * GT) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        if (g0 + GT < TC) load(dd1, bq1, cq1, g0 + GT);
        __builtin_amdgcn_sched_barrier(0);
        run(dd0, bq0, cq0, g0);
        if (g0 + GT < TC) {
          __builtin_amdgcn_s_waitcnt(0xC07F);
          __builtin_amdgcn_sched_barrier(0);
          if (g0 + 2 * GT < TC) load(dd0, bq0, cq0, g0 + 2 * GT);
          __builtin_amdgcn_sched_barrier(0);
          run(dd1, bq1, cq1, g0 + GT);
        }
      }
    };
    if (tn == TC) recurrence(std::true_type());
    else recurrence(std::false_type());

    if (!kSum) {
      lds_barrier();
      // Output: thread q takes 4 channels of one token (16 threads per token row): the
      // waves' parts of sum_n C h, plus D x, times SiLU(G).  With p.ssp the row's sum of
      // y^2 over the 64 channels (of the rounded y, as a norm reading the stored Y_ssm
      // sees it) goes to ssp[ssp_col0 + blockIdx.x, row] and beta * y is stored.
      for (int q = tid; q < TC * 16; q += NT) {
        const int tt = q >> 4, j4 = q & 15;
        floatx4 sum = *(const floatx4*)(part_s + tt * CB + j4 * 4);
#pragma unroll
        for (int w = 1; w < W; ++w) sum += *(const floatx4*)(part_s + (w * TC + tt) * CB + j4 * 4);
        const bf16x4 xv = *(const bf16x4*)(x_s[cur] + tt * CB + j4 * 4);
        const bf16x4 gv = *(const bf16x4*)(g_s[cur] + tt * CB + j4 * 4);
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = (bf16)(fmaf(D4[e], (float)xv[e], sum[e]) * silu_f((float)gv[e]));
        const bool keep = tt < tn;
        const int t = s0 + min(tt, tn - 1);
        if (ssps != nullptr) {
          float sq = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) sq = fmaf((float)o[e], (float)o[e], sq);
          sq = row16_sum(sq);
          if (keep && j4 == 0) *(glb_float*)(ssps + t) = sq;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)((float)o[e] * beta4[e]);
        }
        if (keep) *(glb_bf16x4*)(ys + t * yst + j4 * 4) = o;
      }
    }
    // This wave's DMA for the next step has landed.  Vector memory operations complete in
    // issue order, so in a whole step (every output row kept, every store instruction
    // issued) it is enough to leave this step's output stores in flight: epi_stores of
    // them, issued after the DMA.
    if (!kSum && tn == TC) wait_vmcnt_upto(epi_stores);
    else __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    lds_barrier();
  }

  if (hdst != nullptr) lane_store<NS>(hdst + (int64_t)c * N + n0, h);
  if (kSum && wave == 0) sdst[c] = dtsum;
  // the sequence's token count (the decode position), once per sequence: by the first
  // channel block's workgroup of the last chunk
  if (!kSum && p.pos_out != nullptr && blockIdx.x == 0 && k == p.nchunks - 1 && tid == 0)
    p.pos_out[b] = p.pos_val;
}

// Carries of the chunk summaries, in place: on entry hsum[b][k] is chunk k's end state
// from zero and ssum[b][k] its sum of dt; on exit hsum[b][k] is the state after chunks
// 0..k of sequence b started from h0 (zero when h0 is null), the initial state of chunk
// k + 1.  A workgroup takes 64 consecutive state elements of one sequence: it loads their
// Kc summaries row by row (coalesced) into LDS with the chunk decays P = exp(A sum dt),
// then each wave runs the inclusive scan over the chunks with lanes = chunks (J = 64 / KP
// elements per pass, shuffles by 1, 2, 4, ... within each group of KP lanes), and the
// carried states go back row by row.
template <int KP>
__global__ __launch_bounds__(256) void scan_carry_kernel(float* __restrict__ hsum,
                                                         const float* __restrict__ ssum,
                                                         const float* __restrict__ A,
                                                         const float* __restrict__ h0, int Di,
                                                         int N, int Kc) {
  constexpr int EW = 64, TP = EW + 1;  // elements per workgroup; LDS row pitch
  constexpr int J = 64 / KP;           // elements per wave pass
  static_assert(KP >= 4 && KP <= 64 && (16 % J) == 0, "chunk lanes");
  __shared__ float th[64 * TP], tp[64 * TP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t DN = (int64_t)Di * N;  // a multiple of 64: the workgroup's elements share b
  const int64_t base = (int64_t)blockIdx.x * EW;
  const int64_t b = base / DN, e0 = base % DN;
  for (int kc = wave; kc < Kc; kc += 4) {
    const int64_t e = e0 + lane;
    th[kc * TP + lane] = hsum[(b * Kc + kc) * DN + e];
    tp[kc * TP + lane] =
        __builtin_amdgcn_exp2f(A[e] * kLog2eF * ssum[(b * Kc + kc) * Di + e / N]);
  }
  __syncthreads();
  const int kc = lane % KP, j = lane / KP;
  for (int e = wave * 16 + j; e < wave * 16 + 16; e += J) {
    float hh = 0.f, P = 1.f;
    if (kc < Kc) {
      hh = th[kc * TP + e];
      P = tp[kc * TP + e];
    }
#pragma unroll
    for (int d = 1; d < KP; d <<= 1) {
      const float Pp = __shfl_up(P, d, 64);
      const float hp = __shfl_up(hh, d, 64);
      if (kc >= d) {
        hh = fmaf(P, hp, hh);
        P *= Pp;
      }
    }
    if (kc < Kc) {
      if (h0 != nullptr) hh = fmaf(P, h0[e0 + e], hh);
      th[kc * TP + e] = hh;
    }
  }
  __syncthreads();
  for (int kc = wave; kc < Kc; kc += 4) hsum[(b * Kc + kc) * DN + e0 + lane] = th[kc * TP + lane];
}

namespace {

// Tokens per step of a launch of `wgs` workgroups: 32 at 4 waves when the grid leaves at
// most two workgroups per CU, which is all the LDS of a 32-token step (about 80 KB) allows;
// otherwise 16 (40 KB: up to four per CU).  8-wave shapes take 16 (LDS), 1- and 2-wave
// shapes 16 (each wave would hold 4 or 2 dt tiles' MFMA operands).  Measured at
// d_inner 4096, N = 16: 0.500 -> 0.479 ms for 8 sequences of 2048 tokens in one chunk
// (512 workgroups); 1.09 -> 1.32 ms with 32-token steps at 4 x 8 chunks of 1024 (2048).
// Chunks that are not a multiple of 32 tokens (the meta rows' chunks of 16) keep
// 16-token steps: a 32-token step would run half empty at every chunk's end.
template <int W>
bool long_steps(int64_t wgs, int chunk) { return W == 4 && wgs <= 512 && chunk % 32 == 0; }

template <int NS, int W, int R, bool kSum>
void launch_steps(const ScanChunkParams& p, dim3 grid, hipStream_t s) {
  const dim3 blk(64 * W);
  if (long_steps<W>((int64_t)grid.x * grid.y, p.chunk))
    scan_chunk_kernel<NS, W, R, kSum, 32><<<grid, blk, 0, s>>>(p);
  else
    scan_chunk_kernel<NS, W, R, kSum, 16><<<grid, blk, 0, s>>>(p);
}

template <int NS, int W, int R>
hipError_t run_chunk(const ScanChunkParams& p, hipStream_t s) {
  const int cbk = p.Di / 64;
  if (p.nchunks > 1) {
    launch_steps<NS, W, R, true>(p, dim3(cbk, p.B * (p.nchunks - 1)), s);
    const int Kc = p.nchunks - 1;
    const int64_t elems = (int64_t)p.B * p.Di * p.N;
    auto carry = [&](auto kp) {
      constexpr int KP = decltype(kp)::value;
      scan_carry_kernel<KP><<<dim3((unsigned)(elems / 64)), dim3(256), 0, s>>>(
          p.hsum, p.ssum, p.A, p.h0, p.Di, p.N, Kc);
    };
    if (Kc <= 4) carry(std::integral_constant<int, 4>());
    else if (Kc <= 8) carry(std::integral_constant<int, 8>());
    else if (Kc <= 16) carry(std::integral_constant<int, 16>());
    else if (Kc <= 32) carry(std::integral_constant<int, 32>());
    else carry(std::integral_constant<int, 64>());
  }
  launch_steps<NS, W, R, false>(p, dim3(cbk, p.B * p.nchunks), s);
  return hipGetLastError();
}

template <int R>
hipError_t chunk_by_state(const ScanChunkParams& p, hipStream_t s) {
  switch (p.N) {
    case 4: return run_chunk<4, 1, R>(p, s);
    case 8: return run_chunk<4, 2, R>(p, s);
    case 16: return run_chunk<4, 4, R>(p, s);
    case 32: return run_chunk<8, 4, R>(p, s);
    case 64: return run_chunk<8, 8, R>(p, s);
    case 128: return run_chunk<16, 8, R>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool scan_chunk_supported(int N, int R, int Di) {
  return (R == 64 || R == 128) && Di % 64 == 0 && N >= 4 && N <= 128 && (N & (N - 1)) == 0;
}

int scan_channel_blocks(int /*N*/, int Di) { return Di / 64; }

int scan_chunk_count(int T, int chunk) { return T <= 0 ? 1 : (T + chunk - 1) / chunk; }

int scan_default_chunk(int B, int Di, int T) {
  // Measured on MI355X (the prefill shapes of the layer, d_inner 4096): with at least two
  // workgroups per CU from the batch alone, one chunk is fastest (the summary pass costs
  // more than the extra occupancy returns); below that, about 2048 (sequence, chunk)
  // workgroups, with chunks of at least 512 tokens.  A short sequence (the meta rows,
  // scanned once per call) is latency-bound: up to 8 chunks of at least 16 tokens.
  const int wgs = std::max(1, B * (Di / 64));
  if (wgs >= 512) return std::max(16, (T + 15) / 16 * 16);
  int k = (2048 + wgs - 1) / wgs;
  if (T < 1024) k = std::min(std::min(k, 8), (T + 15) / 16);
  else k = std::min(k, T / 512);
  k = std::max(1, std::min(k, 64));
  const int per = (T + k - 1) / k;
  return std::max(16, (per + 15) / 16 * 16);
}

hipError_t launch_scan_chunk(const ScanChunkParams& p, hipStream_t s) {
  if (p.B == 0 || p.Di == 0 || (p.T == 0 && p.h_out == nullptr)) return hipSuccess;
  if (p.chunk <= 0 || p.chunk % 16 || p.nchunks != scan_chunk_count(p.T, p.chunk) ||
      p.nchunks > 65 || !scan_chunk_supported(p.N, p.R, p.Di))
    return hipErrorInvalidValue;
  if (p.nchunks > 1 && (p.hsum == nullptr || p.ssum == nullptr)) return hipErrorInvalidValue;
  if (p.R == 128) return chunk_by_state<128>(p, s);
  return chunk_by_state<64>(p, s);
}

}  // namespace hymba
