// Projection GEMMs of the hybrid-head layer: in_proj (Z = X~ W_in^T), x_proj
// ([delta | B | C] = Xs W_x^T), dt_proj (dt = softplus(delta W_dt^T + b)) and
// out_proj (Y = F W_out^T).  Source: the in_proj / out_proj terms of the design
// formulation in "Hymba: A Hybrid-head Architecture for Small Language Models"
// (outta.ai summary); dt, B, C are linear maps of the SSM input (Mamba).
//
// bf16 path: LDS-staged MFMA tiles with fp32 accumulation: the 256x256 / 128x64 tiles
// (gemm_bf16_dl_kernel) issue v_mfma_f32_32x32x16_bf16, the 64x64 tile kernel
// (gemm_bf16_kernel) v_mfma_f32_16x16x32_bf16.  The few-row kernels of decode and of the
// meta rows are in gemm_fewrow.hip.  Operands are both
// K-contiguous ([rows, K] and [cols, K]); the MFMA is issued as (B-tile, A-tile) so each
// lane ends with runs of consecutive output columns of one row, which the epilogue
// writes with vector stores.
// fp32 path: a plain LDS-tiled VALU GEMM with the same epilogues.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "gemm_tile.h"
#include "kernels.h"

namespace hymba {

// --------------------------------------------------------------------- epilogues

template <typename T>
__device__ __forceinline__ void store4(T* p, const float v[4], int valid, bool vec_ok);

template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, const float v[4], int valid, bool vec_ok) {
  if (valid >= 4 && vec_ok) {
    bf16x4 o;
    o[0] = (bf16)v[0];
    o[1] = (bf16)v[1];
    o[2] = (bf16)v[2];
    o[3] = (bf16)v[3];
    *(bf16x4*)p = o;
  } else {
    for (int r = 0; r < valid && r < 4; ++r) p[r] = (bf16)v[r];
  }
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const float v[4], int valid, bool vec_ok) {
  if (valid >= 4 && vec_ok) {
    *(floatx4*)p = floatx4{v[0], v[1], v[2], v[3]};
  } else {
    for (int r = 0; r < valid && r < 4; ++r) p[r] = v[r];
  }
}

// Every epilogue receives the accumulator values of output (m, n..n+3).
template <typename T, EpiKind K>
struct Epilogue {
  GemmOutput o;
  __device__ __forceinline__ void operator()(int m, int n, const float v[4], int M, int N) const {
    if (m >= M || n >= N) return;
    const int valid = N - n;
    if constexpr (K == EpiKind::Store || K == EpiKind::Silu || K == EpiKind::AddStore) {
      T* base;
      int64_t ld;
      int mm;
      if (m < o.c_split) {
        base = (T*)o.c0;
        ld = o.ldc0;
        mm = m;
      } else {
        base = (T*)o.c1;
        ld = o.ldc1;
        mm = m - o.c_split;
      }
      if (base == nullptr) return;
      T* p = base + mm * ld + n;
      float w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        w[r] = v[r];
        if constexpr (K == EpiKind::Silu) w[r] = silu_f(v[r]);
        if constexpr (K == EpiKind::AddStore) w[r] = r < valid ? to_f32(p[r]) + v[r] : 0.f;
      }
      store4<T>(p, w, valid, ((uintptr_t)p & (4 * sizeof(T) - 1)) == 0);
    } else if constexpr (K == EpiKind::StoreF32) {
      float* p = (float*)o.c0 + m * o.ldc0 + n;
      store4<float>(p, v, valid, ((uintptr_t)p & 15) == 0);
    } else if constexpr (K == EpiKind::XProj) {
      if (n < o.split_col) {  // split_col is a multiple of 4: a group never straddles
        T* p = (T*)o.c0 + m * o.ldc0 + n;
        store4<T>(p, v, o.split_col - n, ((uintptr_t)p & (4 * sizeof(T) - 1)) == 0);
      } else {
        float* p = (float*)o.c1 + m * o.ldc1 + (n - o.split_col);
        store4<float>(p, v, valid, ((uintptr_t)p & 15) == 0);
      }
    } else {  // Softplus
      float w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = (n + r < N) ? softplus_f(v[r] + o.bias[n + r]) : 0.f;
      float* p = (float*)o.c0 + m * o.ldc0 + n;
      store4<float>(p, w, valid, ((uintptr_t)p & 15) == 0);
    }
  }
  // Unchecked path for a whole tile: rows [m0, m1) x columns [n0, n1) inside one
  // destination of the storage type, written with 16-byte stores (Store; XProj when the
  // tile lies in the delta columns).  The caller checks the bounds.
  __device__ __forceinline__ bool tile_fast(int m0, int m1, int n0, int n1) const {
    if constexpr (K == EpiKind::Store || K == EpiKind::Silu || K == EpiKind::AddStore) {
      const bool first = m1 <= o.c_split;
      if (!first && m0 < o.c_split) return false;
      const T* base = (const T*)(first ? o.c0 : o.c1);
      const int64_t ld = first ? o.ldc0 : o.ldc1;
      return base != nullptr && ld % 8 == 0 && ((uintptr_t)base & 15) == 0;
    } else if constexpr (K == EpiKind::XProj) {
      return n1 <= o.split_col && o.ldc0 % 8 == 0 && ((uintptr_t)o.c0 & 15) == 0;
    } else {
      return false;
    }
  }
  // Output (m, n..n+7) = lo[0..3], hi[0..3]; valid after tile_fast() returned true.
  __device__ __forceinline__ void store8(int m, int n, const float lo[4], const float hi[4]) const {
    if constexpr (K == EpiKind::Store || K == EpiKind::XProj || K == EpiKind::Silu ||
                  K == EpiKind::AddStore) {
      const bool first = K == EpiKind::XProj || m < o.c_split;
      T* p = (T*)(first ? o.c0 : o.c1) + (int64_t)(first ? m : m - o.c_split) *
                                             (first ? o.ldc0 : o.ldc1) + n;
      float v[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = lo[r];
        v[4 + r] = hi[r];
      }
      if constexpr (K == EpiKind::Silu) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = silu_f(v[e]);
      }
      if constexpr (K == EpiKind::AddStore) {
        const bf16x8 old = *(const bf16x8*)p;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += (float)old[e];
      }
      bf16x8 w;
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = (bf16)v[e];
      *(bf16x8*)p = w;
    }
  }
};

// --------------------------------------------------------------------- tile order

// Workgroups are handed to the 8 XCDs round-robin (id % 8).  Renumber so every XCD
// owns a contiguous range of the grouped tile order, keeping the A rows and B
// columns a range touches in that XCD's L2.
__device__ __forceinline__ void tile_coords(int pid, int nbm, int nbn, int group_m, int& bm,
                                            int& bn) {
  const int nblk = nbm * nbn;
  const int per = nblk / 8, rem = nblk % 8;
  const int xcd = pid % 8, idx = pid / 8;
  const int t = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  const int span = group_m * nbn;
  const int grp = t / span;
  const int first = grp * group_m;
  const int gsz = min(nbm - first, group_m);
  const int in = t - grp * span;
  bm = first + in % gsz;
  bn = in / gsz;
}

// --------------------------------------------------------------------- bf16 MFMA

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct MfmaCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int NT = WM * WN * kWave;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr int LDS = BK + 8;  // row pitch in bf16: 16-byte pad spreads rows over banks
  static constexpr int CPR = BK / 8;  // 16-byte chunks per row
  static constexpr int A_CH = BM * CPR / NT;
  static constexpr int B_CH = BN * CPR / NT;
  static constexpr size_t SMEM = (size_t)2 * (BM + BN) * LDS * sizeof(bf16);
  static_assert(BM * CPR % NT == 0 && BN * CPR % NT == 0, "loader must tile evenly");
  static_assert(TM % 16 == 0 && TN % 16 == 0 && BK % 32 == 0, "MFMA tiling");
};

template <typename Cfg, typename Epi>
__global__ __launch_bounds__(Cfg::NT) void gemm_bf16_kernel(GemmOperands g, Epi epi) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16* As = (bf16*)smem_raw;
  bf16* Bs = As + 2 * Cfg::BM * Cfg::LDS;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  const int nbm = (g.M + Cfg::BM - 1) / Cfg::BM, nbn = (g.N + Cfg::BN - 1) / Cfg::BN;
  int bm, bn;
  tile_coords(blockIdx.x, nbm, nbn, 8, bm, bn);
  const int m0 = bm * Cfg::BM, n0 = bn * Cfg::BN;

  // Per-thread loader state: fixed rows across the K loop.
  const bf16* a_src[Cfg::A_CH];
  int a_dst[Cfg::A_CH], a_kc[Cfg::A_CH];
#pragma unroll
  for (int j = 0; j < Cfg::A_CH; ++j) {
    const int q = tid + j * Cfg::NT, r = q / Cfg::CPR, kc = (q % Cfg::CPR) * 8;
    const int row = m0 + r;
    const bf16* base = nullptr;
    if (row < g.M)
      base = row < g.a_split ? (const bf16*)g.a0 + (int64_t)row * g.lda0
                             : (const bf16*)g.a1 + (int64_t)(row - g.a_split) * g.lda1;
    a_src[j] = base ? base + kc : nullptr;
    a_dst[j] = r * Cfg::LDS + kc;
    a_kc[j] = kc;
  }
  const bf16* b_src[Cfg::B_CH];
  int b_dst[Cfg::B_CH], b_kc[Cfg::B_CH];
#pragma unroll
  for (int j = 0; j < Cfg::B_CH; ++j) {
    const int q = tid + j * Cfg::NT, r = q / Cfg::CPR, kc = (q % Cfg::CPR) * 8;
    const int col = n0 + r;
    b_src[j] = col < g.N ? (const bf16*)g.b + (int64_t)col * g.ldb + kc : nullptr;
    b_dst[j] = r * Cfg::LDS + kc;
    b_kc[j] = kc;
  }

  u32x4 ra[Cfg::A_CH], rb[Cfg::B_CH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < Cfg::A_CH; ++j)
      ra[j] = (a_src[j] && k0 + a_kc[j] < g.K) ? *(const u32x4*)(a_src[j] + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < Cfg::B_CH; ++j)
      rb[j] = (b_src[j] && k0 + b_kc[j] < g.K) ? *(const u32x4*)(b_src[j] + k0) : u32x4{0, 0, 0, 0};
  };
  auto sstore = [&](int buf) {
    bf16* as = As + buf * Cfg::BM * Cfg::LDS;
    bf16* bs = Bs + buf * Cfg::BN * Cfg::LDS;
#pragma unroll
    for (int j = 0; j < Cfg::A_CH; ++j) *(u32x4*)(as + a_dst[j]) = ra[j];
#pragma unroll
    for (int j = 0; j < Cfg::B_CH; ++j) *(u32x4*)(bs + b_dst[j]) = rb[j];
  };

  floatx4 acc[Cfg::FM][Cfg::FN];
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int KT = (g.K + Cfg::BK - 1) / Cfg::BK;
  gload(0);
  sstore(0);
  __syncthreads();

  const int frag_row = lane & 15, frag_k = (lane >> 4) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * Cfg::BK);
    const bf16* as = As + buf * Cfg::BM * Cfg::LDS + (wm * Cfg::TM + frag_row) * Cfg::LDS + frag_k;
    const bf16* bs = Bs + buf * Cfg::BN * Cfg::LDS + (wn * Cfg::TN + frag_row) * Cfg::LDS + frag_k;
#pragma unroll
    for (int ks = 0; ks < Cfg::BK / 32; ++ks) {
      bf16x8 af[Cfg::FM], bfr[Cfg::FN];
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i) af[i] = *(const bf16x8*)(as + i * 16 * Cfg::LDS + ks * 32);
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) bfr[j] = *(const bf16x8*)(bs + j * 16 * Cfg::LDS + ks * 32);
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = mfma16x16x32(bfr[j], af[i], acc[i][j]);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  // acc[i][j] holds C^T for the (i, j) 16x16 block: lane -> row frag_row, columns
  // 4 * (lane / 16) + 0..3.
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int m = m0 + wm * Cfg::TM + i * 16 + frag_row;
      const int n = n0 + wn * Cfg::TN + j * 16 + (lane >> 4) * 4;
      const float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      epi(m, n, v, g.M, g.N);
    }
}

// ------------------------------------------------------------ bf16 MFMA, direct-to-LDS
// K % 64 == 0.  Tiles of BM x BN x 64 are fetched with global_load_lds_dwordx4 (each
// wave instruction fills 1 KB of LDS = 8 rows x 64 k), so no VGPR staging and no LDS
// store instructions.  Row r of a tile keeps its 8 16-byte k-chunks XOR-swizzled by
// f(r) = (r & 7) ^ ((r >> 3) & 1): the 16 rows an MFMA fragment read touches then hit
// distinct bank groups for both 16-lane and 8-lane LDS phases.

template <int BM_, int BN_, int WM_, int WN_>
struct DlCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64, WM = WM_, WN = WN_;
  static constexpr int NW = WM * WN, NT = NW * kWave;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;  // 32 x 32 MFMA blocks per wave
  static constexpr int A_INS = BM / 8 / NW;        // 8-row wave instructions per wave
  static constexpr int B_INS = BN / 8 / NW;
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "loader tiling");
};

// The k-loop: two LDS stages of BM x 64 and BN x 64; each wave reads the fragments of
// k-substep s + 1 (16 k) one substep ahead of the MFMAs; before the last substep's
// MFMAs every wave waits for tile t+1 to land, passes a barrier (after which nobody
// reads tile t's stage), refills that stage with tile t+2 and reads tile t+1's first
// fragments, so the barrier, the DMA issue and the LDS latency hide behind the last
// 16 MFMAs of the tile.  Each transfer has one full k-tile of MFMA work to land.
template <typename Cfg, typename Epi, bool RS = false>
__global__ __launch_bounds__(Cfg::NT) void gemm_bf16_dl_kernel(GemmOperands g, Epi epi,
                                                               RowScale rs) {
  __shared__ __attribute__((aligned(1024))) bf16 sA0[Cfg::BM * 64];
  __shared__ __attribute__((aligned(1024))) bf16 sB0[Cfg::BN * 64];
  __shared__ __attribute__((aligned(1024))) bf16 sA1[Cfg::BM * 64];
  __shared__ __attribute__((aligned(1024))) bf16 sB1[Cfg::BN * 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  const int nbm = (g.M + Cfg::BM - 1) / Cfg::BM, nbn = (g.N + Cfg::BN - 1) / Cfg::BN;
  int bm, bn;
  tile_coords(blockIdx.x, nbm, nbn, 8, bm, bn);
  const int m0 = bm * Cfg::BM, n0 = bn * Cfg::BN;

  // Loader: wave instruction j fills LDS chunks [(j*NW + wave)*64, +64): rows
  // (j*NW + wave)*8 + lane/8, slot lane%8 holding k-chunk (lane%8) ^ f(row).  A has a
  // single source here (a_split >= M); element offsets fit in 32 bits (checked on the
  // host).  Rows past M / N load a valid row and are never stored.
  const bf16* A = (const bf16*)g.a0;
  const bf16* Bm = (const bf16*)g.b;
  int a_off[Cfg::A_INS], b_off[Cfg::B_INS];
#pragma unroll
  for (int j = 0; j < Cfg::A_INS; ++j) {
    const int r = (j * Cfg::NW + wave) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    a_off[j] = min(m0 + r, g.M - 1) * (int)g.lda0 + c * 8;
  }
#pragma unroll
  for (int j = 0; j < Cfg::B_INS; ++j) {
    const int r = (j * Cfg::NW + wave) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    b_off[j] = min(n0 + r, g.N - 1) * (int)g.ldb + c * 8;
  }
  auto issue = [&](bf16* sa, bf16* sb, int k0) {
#pragma unroll
    for (int j = 0; j < Cfg::A_INS; ++j)
      dma16(A + k0 + a_off[j], (lds_void_t*)(sa + (j * Cfg::NW + wave) * 512));
#pragma unroll
    for (int j = 0; j < Cfg::B_INS; ++j)
      dma16(Bm + k0 + b_off[j], (lds_void_t*)(sb + (j * Cfg::NW + wave) * 512));
  };

  floatx16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Fragment reads: row (l % 32) of a 32-row block (32 rows = 2048 elements), k-chunk
  // 2*ks + l/32 swizzled by f(l % 16) (block bases are multiples of 16 rows).
  const int rl = lane & 31;
  int koff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    koff[ks] = rl * 64 + (((ks * 2 + (lane >> 5)) ^ swz(lane & 15)) * 8);
  const int a_row0 = wm * Cfg::TM * 64, b_row0 = wn * Cfg::TN * 64;
  bf16x8 af[2][Cfg::FM], bfr[2][Cfg::FN];
  auto load = [&](const bf16* sa, const bf16* sb, int buf, int ks) {
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
      af[buf][i] = *(const bf16x8*)(sa + a_row0 + i * 2048 + koff[ks]);
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j)
      bfr[buf][j] = *(const bf16x8*)(sb + b_row0 + j * 2048 + koff[ks]);
  };
  // MFMAs of one k-substep; the fragment reads of the next substep (issued just before)
  // are interleaved one after each of the first MFMAs instead of being bunched ahead
  // of waits the scheduler would otherwise place between single MFMAs.
  auto mm = [&](int buf) {
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j)
        acc[i][j] = mfma32x32x16(bfr[buf][j], af[buf][i], acc[i][j]);
#pragma unroll
    for (int q = 0; q < Cfg::FM + Cfg::FN; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, Cfg::FM * Cfg::FN - Cfg::FM - Cfg::FN, 0);
  };

  // Row scaling (RS): every accumulator of lane row i belongs to output row
  // m0 + wm*TM + i*32 + rl.  After the first segment's k-tiles the accumulators take the
  // factor ratio fa / fs, at the end fs.
  float ratio[Cfg::FM], fin[Cfg::FM];
  int ks_t = -1;
  if constexpr (RS) {
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
      const int m = min(m0 + wm * Cfg::TM + i * 32 + rl, g.M - 1);
      const float fa = rs.fac[2 * (int64_t)m], fs = rs.fac[2 * (int64_t)m + 1];
      ratio[i] = fa / fs;
      fin[i] = fs;
    }
    ks_t = rs.k_split / 64;
  }
  auto scale_rows = [&](const float (&f)[Cfg::FM]) {
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] *= f[i];
  };

  const int KT = g.K / 64;
  issue(sA0, sB0, 0);
  wait_vmcnt<0>();
  lds_barrier();
  if (KT > 1) issue(sA1, sB1, 64);
  load(sA0, sB0, 0, 0);
  // Two k-tiles per trip (stage 0, then stage 1); a single loop exit keeps the
  // accumulators in place, an odd last tile runs after the loop.
  int t = 0;
  for (; t + 1 < KT; t += 2) {
    load(sA0, sB0, 1, 1);
    mm(0);
    load(sA0, sB0, 0, 2);
    mm(1);
    load(sA0, sB0, 1, 3);
    mm(0);
    wait_vmcnt<0>();
    lds_barrier();
    if (t + 2 < KT) issue(sA0, sB0, (t + 2) * 64);
    load(sA1, sB1, 0, 0);
    mm(1);
    load(sA1, sB1, 1, 1);
    mm(0);
    load(sA1, sB1, 0, 2);
    mm(1);
    load(sA1, sB1, 1, 3);
    mm(0);
    if (t + 2 < KT) {
      wait_vmcnt<0>();
      lds_barrier();
      if (t + 3 < KT) issue(sA1, sB1, (t + 3) * 64);
      load(sA0, sB0, 0, 0);
    }
    mm(1);
    if constexpr (RS) {
      if (t + 2 == ks_t) scale_rows(ratio);  // first segment complete (ks_t is even)
    }
  }
  if (t < KT) {
    load(sA0, sB0, 1, 1);
    mm(0);
    load(sA0, sB0, 0, 2);
    mm(1);
    load(sA0, sB0, 1, 3);
    mm(0);
    mm(1);
  }

  if constexpr (RS) scale_rows(fin);
  // acc[i][j] holds C^T of the 32 x 32 block: lane -> row rl, columns
  // (e/4)*8 + (lane/32)*4 + 0..3.
  if (m0 + Cfg::BM <= g.M && n0 + Cfg::BN <= g.N &&
      epi.tile_fast(m0, m0 + Cfg::BM, n0, n0 + Cfg::BN)) {
    // Interior tile: v_permlane32_swap exchanges lanes 32..63 of its first operand with
    // lanes 0..31 of its second, so after swapping the column groups 2p (e = 8p..8p+3)
    // and 2p+1 (e = 8p+4..8p+7) lane l < 32 holds columns 16p + 0..7 of row l and lane
    // l + 32 holds columns 16p + 8..15: one 16-byte store each.
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          float lo[4], hi[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // (vector elements are copied to scalars first: a bit cast applied to the
            // subscript itself reads element 0)
            const float x0 = acc[i][j][8 * pp + r], x1 = acc[i][j][8 * pp + 4 + r];
            const auto sw = __builtin_amdgcn_permlane32_swap(
                __builtin_bit_cast(unsigned, x0), __builtin_bit_cast(unsigned, x1), false, false);
            lo[r] = __builtin_bit_cast(float, (unsigned)sw[0]);
            hi[r] = __builtin_bit_cast(float, (unsigned)sw[1]);
          }
          const int m = m0 + wm * Cfg::TM + i * 32 + rl;
          const int n = n0 + wn * Cfg::TN + j * 32 + pp * 16 + (lane >> 5) * 8;
          epi.store8(m, n, lo, hi);
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm * Cfg::TM + i * 32 + rl;
        const int n = n0 + wn * Cfg::TN + j * 32 + q * 8 + (lane >> 5) * 4;
        const float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                            acc[i][j][4 * q + 3]};
        epi(m, n, v, g.M, g.N);
      }
}

template <typename Cfg, typename Epi, bool RS = false>
static hipError_t run_bf16_dl(const GemmOperands& op, const Epi& epi, hipStream_t s,
                              const RowScale& rs = RowScale{}) {
  const int nbm = (op.M + Cfg::BM - 1) / Cfg::BM, nbn = (op.N + Cfg::BN - 1) / Cfg::BN;
  gemm_bf16_dl_kernel<Cfg, Epi, RS><<<dim3(nbm * nbn), dim3(Cfg::NT), 0, s>>>(op, epi, rs);
  return hipGetLastError();
}

template <typename Cfg, typename Epi>
static hipError_t run_bf16(const GemmOperands& op, const Epi& epi, hipStream_t s) {
  const int nbm = (op.M + Cfg::BM - 1) / Cfg::BM, nbn = (op.N + Cfg::BN - 1) / Cfg::BN;
  auto kern = gemm_bf16_kernel<Cfg, Epi>;
  static bool attr_done = false;  // per instantiation
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::SMEM);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  kern<<<dim3(nbm * nbn), dim3(Cfg::NT), Cfg::SMEM, s>>>(op, epi);
  return hipGetLastError();
}

// Large: in_proj / out_proj prefill.  Narrow: few output columns (x_proj) or mid
// sizes.  Skinny: decode (M = batch) where the weight stream dominates.
using CfgLarge = MfmaCfg<256, 128, 64, 2, 2>;
using CfgNarrow = MfmaCfg<128, 64, 64, 2, 2>;
using CfgSkinny = MfmaCfg<64, 64, 64, 2, 2>;

template <typename Epi>
static hipError_t dispatch_bf16(const GemmOperands& op, const Epi& epi, GemmShape shape,
                                hipStream_t s) {
  switch (shape) {
    case GemmShape::Large:
      if constexpr (std::is_same_v<Epi, Epilogue<bf16, EpiKind::Store>> ||
                    std::is_same_v<Epi, Epilogue<bf16, EpiKind::Silu>> ||
                    std::is_same_v<Epi, Epilogue<bf16, EpiKind::AddStore>>) {
        const bool one_src = op.a_split >= op.M;
        const bool fits32 = (int64_t)op.M * op.lda0 < (1ll << 31) && (int64_t)op.N * op.ldb < (1ll << 31);
        if (op.K % 64 == 0 && one_src && fits32) {
          // 256 x 256 tiles on 8 waves (2 x 4 of 128 x 64) once they fill the chip,
          // else 256 x 128 tiles
          const long t256 = (long)((op.M + 255) / 256) * ((op.N + 255) / 256);
          if (t256 >= 256) return run_bf16_dl<DlCfg<256, 256, 2, 4>>(op, epi, s);
          return run_bf16_dl<DlCfg<256, 128, 2, 4>>(op, epi, s);
        }
        return run_bf16<CfgLarge>(op, epi, s);
      } else {
        return run_bf16<CfgNarrow>(op, epi, s);
      }
    case GemmShape::Narrow: {
      // few output columns (x_proj: 160): 128 x 64 tiles moved by DMA, 4 waves of 64 x 32
      const bool one_src = op.a_split >= op.M;
      const bool fits32 = (int64_t)op.M * op.lda0 < (1ll << 31) && (int64_t)op.N * op.ldb < (1ll << 31);
      if (op.K % 64 == 0 && one_src && fits32) return run_bf16_dl<DlCfg<128, 64, 2, 2>>(op, epi, s);
      return run_bf16<CfgNarrow>(op, epi, s);
    }
    default:
      return run_bf16<CfgSkinny>(op, epi, s);
  }
}

bool gemm_bf16_rowscaled_ok(const GemmOperands& op, int k_split) {
  return op.K % 128 == 0 && k_split % 128 == 0 && k_split > 0 && k_split < op.K &&
         op.a_split >= op.M && (int64_t)op.M * op.lda0 < (1ll << 31) &&
         (int64_t)op.N * op.ldb < (1ll << 31);
}

hipError_t launch_gemm_bf16_rowscaled(const GemmOperands& op, const GemmOutput& out,
                                      const RowScale& rs, hipStream_t s) {
  if (op.M <= 0 || op.N <= 0) return hipSuccess;
  if (out.kind != EpiKind::Store || !gemm_bf16_rowscaled_ok(op, rs.k_split) || rs.fac == nullptr)
    return hipErrorInvalidValue;
  const Epilogue<bf16, EpiKind::Store> epi{out};
  const long t256 = (long)((op.M + 255) / 256) * ((op.N + 255) / 256);
  if (t256 >= 256) return run_bf16_dl<DlCfg<256, 256, 2, 4>, decltype(epi), true>(op, epi, s, rs);
  return run_bf16_dl<DlCfg<256, 128, 2, 4>, decltype(epi), true>(op, epi, s, rs);
}

hipError_t launch_gemm_bf16(const GemmOperands& op, const GemmOutput& out, GemmShape shape,
                            hipStream_t s) {
  if (op.M <= 0 || op.N <= 0) return hipSuccess;
  // The wide tile is kept for stores (plain, SiLU, add); the fp32 epilogues use the
  // narrower tiles (fewer live accumulators, no spills).
  if (shape == GemmShape::Large && out.kind != EpiKind::Store && out.kind != EpiKind::Silu &&
      out.kind != EpiKind::AddStore)
    shape = GemmShape::Narrow;
  switch (out.kind) {
    case EpiKind::Store:
      return dispatch_bf16(op, Epilogue<bf16, EpiKind::Store>{out}, shape, s);
    case EpiKind::Silu:
      return dispatch_bf16(op, Epilogue<bf16, EpiKind::Silu>{out}, shape, s);
    case EpiKind::AddStore:
      return dispatch_bf16(op, Epilogue<bf16, EpiKind::AddStore>{out}, shape, s);
    case EpiKind::StoreF32:
      return dispatch_bf16(op, Epilogue<bf16, EpiKind::StoreF32>{out}, shape, s);
    case EpiKind::XProj:
      return dispatch_bf16(op, Epilogue<bf16, EpiKind::XProj>{out}, shape, s);
    default:
      return dispatch_bf16(op, Epilogue<bf16, EpiKind::Softplus>{out}, shape, s);
  }
}

// --------------------------------------------------------------------- fp32 VALU

// 64 x 64 tile, BK = 16, 256 threads with 4 x 4 outputs each.
template <typename Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmOperands g, Epi epi) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int tid = threadIdx.x;
  const int nbm = (g.M + 63) / 64, nbn = (g.N + 63) / 64;
  int bm, bn;
  tile_coords(blockIdx.x, nbm, nbn, 8, bm, bn);
  const int m0 = bm * 64, n0 = bn * 64;
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += 16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = tid + j * 256, r = q / 16, kk = q % 16;
      const int row = m0 + r, col = n0 + r, k = k0 + kk;
      float av = 0.f, bv = 0.f;
      if (row < g.M && k < g.K) {
        const float* base = row < g.a_split ? (const float*)g.a0 + (int64_t)row * g.lda0
                                            : (const float*)g.a1 + (int64_t)(row - g.a_split) * g.lda1;
        av = base[k];
      }
      if (col < g.N && k < g.K) bv = ((const float*)g.b)[(int64_t)col * g.ldb + k];
      As[kk][r] = av;
      Bs[kk][r] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty * 4 + i];
        b[i] = Bs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) epi(m0 + ty * 4 + i, n0 + tx * 4, acc[i], g.M, g.N);
}

template <typename Epi>
static void run_f32(const GemmOperands& op, const Epi& epi, int nblk, hipStream_t s) {
  gemm_f32_kernel<Epi><<<dim3(nblk), dim3(256), 0, s>>>(op, epi);
}

hipError_t launch_gemm_f32(const GemmOperands& op, const GemmOutput& out, hipStream_t s) {
  if (op.M <= 0 || op.N <= 0) return hipSuccess;
  const int nblk = ((op.M + 63) / 64) * ((op.N + 63) / 64);
  switch (out.kind) {
    case EpiKind::Store:
      run_f32(op, Epilogue<float, EpiKind::Store>{out}, nblk, s);
      break;
    case EpiKind::StoreF32:
      run_f32(op, Epilogue<float, EpiKind::StoreF32>{out}, nblk, s);
      break;
    case EpiKind::XProj:
      run_f32(op, Epilogue<float, EpiKind::XProj>{out}, nblk, s);
      break;
    case EpiKind::Silu:
      run_f32(op, Epilogue<float, EpiKind::Silu>{out}, nblk, s);
      break;
    case EpiKind::AddStore:
      run_f32(op, Epilogue<float, EpiKind::AddStore>{out}, nblk, s);
      break;
    default:
      run_f32(op, Epilogue<float, EpiKind::Softplus>{out}, nblk, s);
      break;
  }
  return hipGetLastError();
}

}  // namespace hymba
