// x_proj of the prefill rows: [delta | B | C] = Xs W_x^T, a product with few output
// columns (R + 2N: 160 at R = 128, N = 16) over a long K (d_inner).  Source: the SSM
// head of the design formulation in "Hymba: A Hybrid-head Architecture for Small
// Language Models" (outta.ai summary): dt, B and C are input-dependent linear maps of
// the SSM input (Mamba's selection mechanism).
//
// What bounds it: reading Xs (rows x d_inner bf16) once from HBM; W_x (N x K, 1.3 MB at
// the prefill shape) stays in the L2.  The tiled GEMM with 64-column tiles reads Xs once
// per column tile from a two-stage pipeline.  Here a workgroup owns a range of rows and
// every output column:
//  * the rows are split evenly over the grid, at most 96 per workgroup (three 32-row
//    MFMA blocks), so the prefill rows (B L + meta rows) take one workgroup per CU with
//    no straggler round;
//  * NP producer waves move the rows' Xs k-tiles (96 rows x 64 k, 12 KB) into a ring of
//    NSTG LDS stages by DMA, up to NSTG - 1 tiles ahead of the one being multiplied; with
//    PAIR two adjacent k-tiles are issued together, so each row's 256 contiguous bytes
//    are requested back to back;
//  * compute wave w owns columns [32w, 32w + 32): its W_x rows move into its own small
//    LDS ring by DMA, LB tiles ahead (L2 hits), and it runs the 32 x 32 x 16 MFMAs of
//    the row blocks against the Xs stage.
// Vector-memory loads complete in issue order within a wave, so the deep Xs queue and the
// short W_x queues live in different waves: each wave waits only for its own transfers.
// One workgroup barrier per k-tile hands an Xs stage from the producers (their DMA
// landed) to the compute waves, and the stage read in the previous k-tile back.
// Measured on the prefill shape (16512 x 160 x 4096, kernel traces): 51 us against 61 us
// for the tiled GEMM (its 128 x 64 tiles read Xs three times); 82 us with 64-row
// workgroups (258 of them at one per CU: two ran in a second round).
//
// MFMA k order: in k-step s of a k-tile, lanes 0-31 supply k = 8s .. 8s + 7 and lanes
// 32-63 supply k = 32 + 8s .. 32 + 8s + 7 (the same for both operands), so the 64 k of
// a tile are each used once.
#include "common.h"
#include "gemm_tile.h"
#include "kernels.h"

namespace hymba {

namespace {

constexpr int XP_CAP = 96;  // row capacity of a workgroup (three 32-row MFMA blocks)

// LDS: the Xs ring (NSTG stages of 96 rows x 64 k, 12 KB) and, per compute wave, a ring
// of LB + 1 stages of its 32 W_x rows x 64 k (4 KB), in dynamic shared memory.
template <int NSTG, int LB>
constexpr size_t xproj_lds_bytes(int ncw) {
  return (size_t)NSTG * XP_CAP * 128 + (size_t)ncw * (LB + 1) * 4096;
}

template <int MAXW, int NSTG, int LB, int NP, bool PAIR>
__global__ __launch_bounds__(MAXW * 64) void gemm_xproj_kernel(GemmOperands g, GemmOutput o) {
  extern __shared__ __attribute__((aligned(1024))) bf16 xp_lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ncw = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6) - NP);
  // Rows [r0, r1) of this workgroup: the M rows split evenly over the grid (at most 96
  // each), so a grid of one workgroup per CU has no straggler round.
  const int r0 = (int)(((int64_t)blockIdx.x * g.M) / gridDim.x);
  const int r1 = (int)(((int64_t)(blockIdx.x + 1) * g.M) / gridDim.x);
  const int KT = g.K / 64;
  auto ktile = [&](int j) { return min(j, KT - 1); };
  bf16* sA = xp_lds;

  if (wave >= ncw) {
    // Producers (NP waves).  Loop tile j goes to stage j % NSTG: instruction i fills the
    // 1 KB block of rows 8i .. 8i + 7, lane -> row 8i + lane / 8, slot lane % 8 holding
    // k-chunk (lane % 8) ^ swz(row); producer p issues instructions p, p + NP, ...  Tiles
    // past the last are issued as copies of the last (into a stage nobody reads again),
    // so the count of transfers in flight is the same at every wait.  Rows past r1 load
    // row r1 - 1 (never stored; L2 hits).
    const int pw = wave - ncw;
    const bf16* A = (const bf16*)g.a0;
    auto issue = [&](int j) {
      const int64_t kk = (int64_t)ktile(j) * 64;
      bf16* dst = sA + (j % NSTG) * (XP_CAP * 64);
#pragma unroll
      for (int i0 = 0; i0 < XP_CAP / 8; i0 += NP) {
        const int i = i0 + pw;
        const int r = i * 8 + (lane >> 3);
        const int64_t row = min(r0 + r, r1 - 1);
        dma16(A + (row * g.lda0 + kk + ((lane & 7) ^ swz(r)) * 8),
              (lds_void_t*)(dst + i * 512));
      }
    };
    if constexpr (PAIR) {
      // Tiles j and j + 1 issued together, their instructions interleaved per 8-row
      // block: each row's two 128-byte pieces are requested back to back (256 contiguous
      // bytes).  At an even j the stages of j - 2 and j - 1 are free; the pair is waited
      // for as a whole at its first tile.
      static_assert(NSTG % 2 == 0, "pairs of stages");
      auto issue2 = [&](int j) {
        const int64_t ka = (int64_t)ktile(j) * 64, kb = (int64_t)ktile(j + 1) * 64;
        bf16* da = sA + (j % NSTG) * (XP_CAP * 64);
        bf16* db = sA + ((j + 1) % NSTG) * (XP_CAP * 64);
#pragma unroll
        for (int i0 = 0; i0 < XP_CAP / 8; i0 += NP) {
          const int i = i0 + pw;
          const int r = i * 8 + (lane >> 3);
          const int64_t row = min(r0 + r, r1 - 1);
          const bf16* src = A + (row * g.lda0 + ((lane & 7) ^ swz(r)) * 8);
          dma16(src + ka, (lds_void_t*)(da + i * 512));
          dma16(src + kb, (lds_void_t*)(db + i * 512));
        }
      };
      for (int j = 0; j < NSTG - 2; j += 2) issue2(j);
      for (int j = 0; j < KT; ++j) {
        if ((j & 1) == 0) wait_vmcnt<(NSTG - 4) * (XP_CAP / 8 / NP)>();  // pair j, j + 1
        lds_barrier();
        if ((j & 1) == 0) issue2(j + NSTG - 2);
      }
    } else {
      for (int j = 0; j < NSTG - 1; ++j) issue(j);
      for (int j = 0; j < KT; ++j) {
        wait_vmcnt<(NSTG - 2) * (XP_CAP / 8 / NP)>();  // tile j has landed
        lds_barrier();                                  // ... for every wave; stage (j - 1) is free
        issue(j + NSTG - 1);
      }
    }
    wait_vmcnt<0>();  // no transfer may outlive the workgroup's LDS
    return;
  }

  // Compute wave: columns [32 * wave, 32 * wave + 32).  Its W_x rows (clamped to N - 1;
  // their outputs are never stored) move into its own LDS ring by DMA, LB tiles ahead:
  // 4 instructions of 8 rows x 128 bytes per tile, same slot permutation as Xs.  Only
  // this wave reads them, so its own vmcnt wait is all the hand-over needs.
  bf16* sB = xp_lds + NSTG * XP_CAP * 64 + wave * (LB + 1) * 2048;
  const bf16* Wb = (const bf16*)g.b;
  auto issue_b = [&](int j) {
    const int64_t kk = (int64_t)ktile(j) * 64;
    bf16* dst = sB + (j % (LB + 1)) * 2048;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * 8 + (lane >> 3);
      const int64_t row = min(wave * 32 + r, g.N - 1);
      dma16(Wb + (row * g.ldb + kk + ((lane & 7) ^ swz(r)) * 8), (lds_void_t*)(dst + i * 512));
    }
  };
  for (int j = 0; j < LB; ++j) issue_b(j);

  const int rl = lane & 31, kh = lane >> 5;
  int aoff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) aoff[s] = rl * 64 + (((kh * 4 + s) ^ swz(rl)) * 8);
  floatx16 acc[3];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    acc[0][e] = 0.f;
    acc[1][e] = 0.f;
    acc[2][e] = 0.f;
  }
  const bool third = r1 - r0 > 64;  // the third row block holds rows of this workgroup
  for (int j = 0; j < KT; ++j) {
    wait_vmcnt<(LB - 1) * 4>();  // this wave's W_x tile j has landed
    lds_barrier();               // Xs tile j is in its stage
    issue_b(j + LB);             // into the stage read in k-tile j - 1
    const bf16* st = sA + (j % NSTG) * (XP_CAP * 64);
    const bf16* sb = sB + (j % (LB + 1)) * 2048;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 b = *(const bf16x8*)(sb + aoff[s]);
      const bf16x8 a0 = *(const bf16x8*)(st + aoff[s]);
      const bf16x8 a1 = *(const bf16x8*)(st + 2048 + aoff[s]);
      acc[0] = mfma32x32x16(b, a0, acc[0]);
      acc[1] = mfma32x32x16(b, a1, acc[1]);
      if (third) {
        const bf16x8 a2 = *(const bf16x8*)(st + 4096 + aoff[s]);
        acc[2] = mfma32x32x16(b, a2, acc[2]);
      }
    }
  }
  wait_vmcnt<0>();  // the copies issued past the last tile
  // acc[rb] holds C^T of a 32 x 32 block: lane -> row r0 + 32 rb + l % 32, columns
  // 32 * wave + 8 (e / 4) + 4 (l / 32) + e % 4.  Columns below split_col go to c0 in
  // bf16, the others to c1 in fp32 (split_col is a multiple of 4: a group of 4 never
  // straddles it).
#pragma unroll
  for (int rb = 0; rb < 3; ++rb) {
    const int m = r0 + rb * 32 + rl;
    if (m >= r1) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = wave * 32 + q * 8 + kh * 4;
      if (n >= g.N) continue;
      const int valid = min(4, g.N - n);
      const float v[4] = {acc[rb][4 * q], acc[rb][4 * q + 1], acc[rb][4 * q + 2],
                          acc[rb][4 * q + 3]};
      if (n < o.split_col) {
        bf16* p = (bf16*)o.c0 + (int64_t)m * o.ldc0 + n;
        if (valid == 4 && ((uintptr_t)p & 7) == 0) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (bf16)v[e];
          *(bf16x4*)p = w;
        } else {
          for (int e = 0; e < valid; ++e) p[e] = (bf16)v[e];
        }
      } else {
        float* p = (float*)o.c1 + (int64_t)m * o.ldc1 + (n - o.split_col);
        if (valid == 4 && ((uintptr_t)p & 15) == 0) {
          *(floatx4*)p = floatx4{v[0], v[1], v[2], v[3]};
        } else {
          for (int e = 0; e < valid; ++e) p[e] = v[e];
        }
      }
    }
  }
}

}  // namespace

bool gemm_xproj_ok(const GemmOperands& op, const GemmOutput& out) {
  return out.kind == EpiKind::XProj && out.split_col % 4 == 0 && op.a_split >= op.M &&
         op.K % 64 == 0 && op.K > 0 && op.N > 32 && op.N <= 12 * 32 && op.lda0 % 8 == 0 &&
         op.ldb % 8 == 0 && ((uintptr_t)op.a0 & 15) == 0 && ((uintptr_t)op.b & 15) == 0;
}

// Workgroups for M rows: 64 rows each, unless that leaves a few workgroups over a
// multiple of 256 (one round per 256 CUs); then the multiple of 256 below, as long as it
// keeps every workgroup within its 96-row capacity (16512 rows: 256 workgroups of 64-65).
static unsigned xproj_grid(int M) {
  const int64_t g = ((int64_t)M + 63) / 64;
  const int64_t lo = g / 256 * 256;
  if (lo > 0 && lo < g && (int64_t)M <= lo * XP_CAP) return (unsigned)lo;
  return (unsigned)g;
}

template <int MAXW, int NSTG, int LB, int NP, bool PAIR>
static hipError_t run_xproj(const GemmOperands& op, const GemmOutput& out, int ncw,
                            hipStream_t s) {
  auto kern = gemm_xproj_kernel<MAXW, NSTG, LB, NP, PAIR>;
  const size_t lds = xproj_lds_bytes<NSTG, LB>(ncw);
  static bool attr_done = false;  // per instantiation; the largest size it can take
  if (!attr_done) {
    const hipError_t e =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)xproj_lds_bytes<NSTG, LB>(MAXW - NP));
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  kern<<<dim3(xproj_grid(op.M)), dim3((ncw + NP) * 64), lds, s>>>(op, out);
  return hipGetLastError();
}

hipError_t launch_gemm_xproj_bf16(const GemmOperands& op, const GemmOutput& out,
                                  hipStream_t s) {
  if (op.M <= 0) return hipSuccess;
  if (!gemm_xproj_ok(op, out)) return hipErrorInvalidValue;
  const int ncw = (op.N + 31) / 32;  // compute waves (the producers come on top)
  // LDS budget 160 KB: Xs stages x 12 KB + W_x stages x 4 KB per compute wave.
  // Template arguments: largest wave count, Xs stages, W_x lookahead, producers, pairs.
  if (ncw <= 5) return run_xproj<7, 8, 2, 2, true>(op, out, ncw, s);
  return run_xproj<14, 4, 1, 2, false>(op, out, ncw, s);
}

}  // namespace hymba
