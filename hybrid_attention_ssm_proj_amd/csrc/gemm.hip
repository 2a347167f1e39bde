// Projection GEMMs of the hybrid-head layer: in_proj (Z = X~ W_in^T), x_proj
// ([delta | B | C] = Xs W_x^T), dt_proj (dt = softplus(delta W_dt^T + b)) and
// out_proj (Y = F W_out^T).  Source: the in_proj / out_proj terms of the design
// formulation in "Hymba: A Hybrid-head Architecture for Small Language Models"
// (outta.ai summary); dt, B, C are linear maps of the SSM input (Mamba).
//
// bf16 path: LDS-staged MFMA tiles with fp32 accumulation: the 256x256 / 128x64 tiles
// (gemm_bf16_dl_kernel) and the few-row kernel issue v_mfma_f32_32x32x16_bf16, the 64x64
// tile kernel (gemm_bf16_kernel) v_mfma_f32_16x16x32_bf16.  Operands are both
// K-contiguous ([rows, K] and [cols, K]); the MFMA is issued as (B-tile, A-tile) so each
// lane ends with runs of consecutive output columns of one row, which the epilogue
// writes with vector stores.
// fp32 path: a plain LDS-tiled VALU GEMM with the same epilogues.
#include <algorithm>
#include <type_traits>

#include "common.h"
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
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

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

// K % 64 == 0.  Two LDS stages of BM x 64 and BN x 64.  Per k-tile t: fragments of
// k-substeps 1..3 are read one substep ahead of the MFMAs; before the last substep's
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

// ------------------------------------------------------------ bf16 few-row GEMM (decode)
// Few rows (the decode batch): a workgroup owns a BM x 64 output tile and one K slice
// (blockIdx.y, a multiple of 256).  NS LDS stages of 64-k tiles, NS - 1 in flight ahead
// of the one being multiplied, keep the weight stream busy.  The MFMA takes the weight
// tile as its first operand, so a lane's accumulators hold runs of 4 consecutive
// columns of one row, which interior tiles turn into 16-byte stores.
// Epilogues (FewRowMode): fp32 atomics into one accumulator; fp32 partials, slice p of
// the K split at acc + p * slice_stride, plain stores (a later pass sums the slices:
// atomics from every slice onto the same addresses serialise in L2); or the decode
// in_proj store: Z in bf16 plus the producer's new K/V row at ring slot pos[b] % slots.
enum FewRowMode { kFewAtomic = 0, kFewPartial = 1, kFewStore = 2 };
struct FewRowOut {
  float* acc;        // atomic / partial mode: [M, ldacc] fp32 (per slice in partial mode)
  int64_t ldacc;
  int64_t slice_stride;
  bf16* z;           // store mode: [M, ldz]
  int64_t ldz;
  int k_col, v_col;  // store mode: K / V column ranges (k_col < 0: no ring write)
  bf16* ring_k;
  bf16* ring_v;
  int slots, kvw, head_dim, Hkv;
  const int32_t* pos;
  floatx4* zero;     // store mode: accumulators cleared by the grid (zero_n4 vectors)
  int64_t zero_n4;
  int vec;           // 16-byte stores allowed (aligned bases and strides)
};

template <int MODE, int BM, int NS>
__global__ __launch_bounds__(256) void gemm_bf16_fewrow_kernel(GemmOperands g, FewRowOut out,
                                                               int kslice) {
  constexpr int BN = 64, NW = 4, WN = 2;
  constexpr int TM = BM / 2, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int A_INS = BM / 8 / NW, B_INS = BN / 8 / NW, INS = A_INS + B_INS;
  // NS stages of one 64-k tile each: NS - 1 tiles stay in flight ahead of the one being
  // multiplied (the memory latency is covered by the bytes in flight per CU).
  static_assert(NS >= 2 && NS <= 8, "stages");
  constexpr int SA = BM * 64, SB = BN * 64;  // elements per stage
  __shared__ __attribute__((aligned(1024))) bf16 smem[NS * (SA + SB)];
  auto sa = [&](int st) { return smem + st * (SA + SB); };
  auto sb = [&](int st) { return smem + st * (SA + SB) + SA; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.z * BM;
  const int kb = blockIdx.y * kslice;
  // ring slot of row m0 + tid, loaded now and used after the K loop (one round trip per
  // workgroup instead of one per stored element)
  int my_slot = 0;
  if constexpr (MODE == kFewStore) {
    if (out.k_col >= 0 && tid < BM && m0 + tid < g.M) my_slot = max(out.pos[m0 + tid], 0) % out.slots;
    const int64_t nblk = (int64_t)gridDim.x * gridDim.z;
    for (int64_t i = (blockIdx.z * (int64_t)gridDim.x + blockIdx.x) * 256 + tid; i < out.zero_n4;
         i += nblk * 256)
      out.zero[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const bf16* A = (const bf16*)g.a0;
  const bf16* Bm = (const bf16*)g.b;
  int a_off[A_INS], b_off[B_INS];
#pragma unroll
  for (int j = 0; j < A_INS; ++j) {
    const int r = (j * NW + wave) * 8 + (lane >> 3);
    a_off[j] = min(m0 + r, g.M - 1) * (int)g.lda0 + ((lane & 7) ^ swz(r)) * 8;
  }
#pragma unroll
  for (int j = 0; j < B_INS; ++j) {
    const int r = (j * NW + wave) * 8 + (lane >> 3);
    b_off[j] = min(n0 + r, g.N - 1) * (int)g.ldb + ((lane & 7) ^ swz(r)) * 8;
  }
  auto issue = [&](int st, int k0) {
#pragma unroll
    for (int j = 0; j < A_INS; ++j)
      dma16(A + k0 + a_off[j], (lds_void_t*)(sa(st) + (j * NW + wave) * 512));
#pragma unroll
    for (int j = 0; j < B_INS; ++j)
      dma16_nt(Bm + k0 + b_off[j], (lds_void_t*)(sb(st) + (j * NW + wave) * 512));
  };
  // Two accumulator sets (even / odd k-steps) so consecutive MFMAs do not wait on each
  // other: with one 32 x 32 block per wave the tile's four k-steps would otherwise form
  // one dependent chain.
  floatx16 acc[FM][FN], acc2[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = acc2[i][j][e] = 0.f;
  const int rl = lane & 31;
  int koff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    koff[ks] = rl * 64 + (((ks * 2 + (lane >> 5)) ^ swz(lane & 15)) * 8);
  const int a_row0 = wm * TM * 64, b_row0 = wn * TN * 64;
  auto compute = [&](int st) {
    const bf16* a = sa(st);
    const bf16* b = sb(st);
    bf16x8 af[4][FM], bfr[4][FN];  // the whole tile's fragments, read before any MFMA
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int i = 0; i < FM; ++i) af[ks][i] = *(const bf16x8*)(a + a_row0 + i * 2048 + koff[ks]);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[ks][j] = *(const bf16x8*)(b + b_row0 + j * 2048 + koff[ks]);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ks += 2)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (MODE == kFewAtomic) {  // D = C: lanes along columns
            acc[i][j] = mfma32x32x16(af[ks][i], bfr[ks][j], acc[i][j]);
            acc2[i][j] = mfma32x32x16(af[ks + 1][i], bfr[ks + 1][j], acc2[i][j]);
          } else {  // D = C^T: lanes along rows
            acc[i][j] = mfma32x32x16(bfr[ks][j], af[ks][i], acc[i][j]);
            acc2[i][j] = mfma32x32x16(bfr[ks + 1][j], af[ks + 1][i], acc2[i][j]);
          }
        }
  };

  // Step t waits for tile t (the younger tiles, up to NS - 2 of them, stay in flight),
  // syncs, refills the stage tile t-1 used with tile t + NS - 1, then multiplies tile t.
  const int KT = min(kslice, g.K - kb) / 64;  // the last slice may be shorter
  for (int t = 0; t < NS - 1 && t < KT; ++t) issue(t, kb + t * 64);
  int st = 0;
  for (int t = 0; t < KT; ++t) {
    const int ahead = min(NS - 2, KT - 1 - t);  // tiles issued after tile t
    switch (ahead) {  // vmcnt counts this wave's INS transfers per tile, oldest first
      case 6: wait_vmcnt<6 * INS>(); break;
      case 5: wait_vmcnt<5 * INS>(); break;
      case 4: wait_vmcnt<4 * INS>(); break;
      case 3: wait_vmcnt<3 * INS>(); break;
      case 2: wait_vmcnt<2 * INS>(); break;
      case 1: wait_vmcnt<INS>(); break;
      default: wait_vmcnt<0>(); break;
    }
    lds_barrier();  // keeps the younger tiles in flight
    if (t + NS - 1 < KT) {
      const int sn = st == 0 ? NS - 1 : st - 1;  // the stage tile t - 1 used
      issue(sn, kb + (t + NS - 1) * 64);
    }
    compute(st);
    st = st + 1 == NS ? 0 : st + 1;
  }

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] += acc2[i][j][e];

  int* s_slot = (int*)smem;  // the stages are free after the last multiply
  if constexpr (MODE == kFewStore) {
    __syncthreads();
    if (tid < BM) s_slot[tid] = my_slot;
    __syncthreads();
  }

  // Store / partial modes: the MFMA runs with B as its first operand, so acc[i][j] holds
  // C^T of the 32 x 32 block: lane l has row l % 32, columns (e/4)*8 + (l/32)*4 + e%4.
  // Atomic mode keeps C (lane l has column l % 32, rows (e/4)*8 + (l/32)*4 + e%4): one
  // atomic instruction then covers two rows x 32 consecutive columns, two cache lines.
  auto ring_of = [&](int n, int& rel) -> bf16* {  // K / V ring holding column n, if any
    if (out.k_col < 0) return nullptr;
    if (n >= out.k_col && n < out.k_col + out.kvw) {
      rel = n - out.k_col;
      return out.ring_k;
    }
    if (n >= out.v_col && n < out.v_col + out.kvw) {
      rel = n - out.v_col;
      return out.ring_v;
    }
    return nullptr;
  };
  if (MODE != kFewAtomic && out.vec && m0 + BM <= g.M && n0 + BN <= g.N) {
    // Interior tile: v_permlane32_swap of the column groups 2p and 2p + 1 leaves lane
    // l < 32 with columns 16p + 0..7 of row l and lane l + 32 with columns 16p + 8..15,
    // so every lane stores 8 consecutive columns (16 bytes of bf16, two float4 partials).
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
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
          const int m = m0 + wm * TM + i * 32 + rl;
          const int n = n0 + wn * TN + j * 32 + pp * 16 + (lane >> 5) * 8;
          if constexpr (MODE == kFewPartial) {
            float* dst = out.acc + blockIdx.y * out.slice_stride + (int64_t)m * out.ldacc + n;
            *(floatx4*)dst = floatx4{lo[0], lo[1], lo[2], lo[3]};
            *(floatx4*)(dst + 4) = floatx4{hi[0], hi[1], hi[2], hi[3]};
          } else {
            bf16x8 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              v[r] = (bf16)lo[r];
              v[4 + r] = (bf16)hi[r];
            }
            *(bf16x8*)(out.z + (int64_t)m * out.ldz + n) = v;
            int rel = 0;
            bf16* ring = ring_of(n, rel);  // the 8 columns share one head (head_dim % 8 == 0)
            if (ring != nullptr) {
              const int gh = rel / out.head_dim, d = rel % out.head_dim;
              *(bf16x8*)(ring + (((int64_t)m * out.Hkv + gh) * out.slots + s_slot[m - m0]) *
                                    out.head_dim + d) = v;
            }
          }
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ec = (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        const int m = m0 + wm * TM + i * 32 + (MODE == kFewAtomic ? ec : rl);
        const int n = n0 + wn * TN + j * 32 + (MODE == kFewAtomic ? rl : ec);
        if (m >= g.M || n >= g.N) continue;
        if constexpr (MODE == kFewAtomic) {
          unsafeAtomicAdd(out.acc + (int64_t)m * out.ldacc + n, acc[i][j][e]);
        } else if constexpr (MODE == kFewPartial) {
          out.acc[blockIdx.y * out.slice_stride + (int64_t)m * out.ldacc + n] = acc[i][j][e];
        } else {
          const bf16 v = (bf16)acc[i][j][e];
          out.z[(int64_t)m * out.ldz + n] = v;
          int rel = 0;
          bf16* ring = ring_of(n, rel);
          if (ring != nullptr) {
            const int gh = rel / out.head_dim, d = rel % out.head_dim;
            ring[(((int64_t)m * out.Hkv + gh) * out.slots + s_slot[m - m0]) * out.head_dim + d] = v;
          }
        }
      }
    }
}

static bool fewrow_ok(const GemmOperands& op) {
  return op.K % 256 == 0 && op.a_split >= op.M && (int64_t)op.M * op.lda0 < (1ll << 31) &&
         (int64_t)op.N * op.ldb < (1ll << 31);
}

int splitk_slices(int K, int ksplit) {
  const int units = K / 256;
  if (units <= 0) return 1;
  ksplit = std::max(1, std::min(ksplit, units));
  const int kslice = (units + ksplit - 1) / ksplit;
  return (units + kslice - 1) / kslice;
}

hipError_t launch_gemm_bf16_splitk(const GemmOperands& op, float* acc, int64_t ldacc,
                                   int ksplit, hipStream_t s, int64_t slice_stride) {
  if (op.M <= 0 || op.N <= 0) return hipSuccess;
  if (!fewrow_ok(op)) return hipErrorInvalidValue;
  const int units = op.K / 256;
  ksplit = std::max(1, std::min(ksplit, units));
  const int kslice = ((units + ksplit - 1) / ksplit) * 256;
  const int ns = (op.K + kslice - 1) / kslice;
  if (slice_stride > 0 && slice_stride < (int64_t)op.M * ldacc) return hipErrorInvalidValue;
  FewRowOut out{};
  out.acc = acc;
  out.ldacc = ldacc;
  out.slice_stride = slice_stride;
  out.vec = ((uintptr_t)acc & 15) == 0 && ldacc % 4 == 0 && slice_stride % 4 == 0;
  dim3 grid((op.N + 63) / 64, ns, (op.M + 127) / 128);
  if (slice_stride > 0)
    gemm_bf16_fewrow_kernel<kFewPartial, 128, 4><<<grid, dim3(256), 0, s>>>(op, out, kslice);
  else if ((int64_t)grid.x * grid.y * grid.z < 128) {
    // a small grid (the narrow decode x_proj: 3 column tiles x 16 slices) takes 64-row
    // blocks, twice the workgroups (0.7 us faster at 128 rows)
    grid.z = (op.M + 63) / 64;
    gemm_bf16_fewrow_kernel<kFewAtomic, 64, 4><<<grid, dim3(256), 0, s>>>(op, out, kslice);
  } else {
    gemm_bf16_fewrow_kernel<kFewAtomic, 128, 4><<<grid, dim3(256), 0, s>>>(op, out, kslice);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ bf16 few-row streaming
// y[m, n] = sum_k x[m, k] w[n, k] for a few rows (M <= 4: a small decode batch), where the
// tiled few-row kernel would spend a 128-row MFMA tile on one row and leave the weight
// stream at a fraction of HBM bandwidth.  A workgroup stages the M rows of x in LDS.
// KS = 1: each wave owns CPW columns and streams their whole weight rows; KS = 4: the 4
// waves share the workgroup's CPW columns and take a quarter of K each (narrow outputs,
// where one wave per column would leave too few waves streaming), summed through LDS.
// A wave streams its rows with 16-byte non-temporal loads (lane l takes k = kb + 8l +
// 512i; the weights are read once per call), the next slice's loads issued before the
// current slice's dot products (v_dot2_f32_bf16, fp32 sums), then sums each column over
// its 64 lanes.  Optional epilogue: the producer's K / V columns also go to ring slot
// pos[m] % slots (decode in_proj).
template <int M, int CPW, int KS>
__global__ __launch_bounds__(256) void gemv_bf16_kernel(const bf16* __restrict__ x, int64_t ldx,
                                                        const bf16* __restrict__ w, int64_t ldw,
                                                        int N, int K, GemvOut out) {
  static_assert(KS == 1 || KS == 4, "waves per column group");
  extern __shared__ __attribute__((aligned(16))) bf16 xs[];  // [M][K]
  __shared__ float red[KS == 4 ? 4 : 1][CPW * M];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid * 8; i < M * K; i += 256 * 8) {
    const int m = i / K, k = i % K;
    *(u32x4*)(xs + i) = *(const u32x4*)(x + (int64_t)m * ldx + k);
  }
  __syncthreads();
  const int n0 = (KS == 1 ? blockIdx.x * 4 + wave : blockIdx.x) * CPW;
  if (n0 >= N) return;  // uniform over the workgroup when KS = 4
  // this wave's k range: [kb, ke), a multiple of 8 wide
  const int kq = KS == 1 ? K : ((K / 8 + KS - 1) / KS) * 8;
  const int kb = KS == 1 ? 0 : min(wave * kq, K), ke = min(kb + kq, K);
  const bf16* wr[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) wr[c] = w + (int64_t)min(n0 + c, N - 1) * ldw;
  float acc[CPW][M];
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[c][m] = 0.f;
  auto dot2 = [](uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  };
  int k = kb + lane * 8;
  u32x4 wn[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c)
    wn[c] = k < ke ? __builtin_nontemporal_load((const u32x4*)(wr[c] + k)) : u32x4{0, 0, 0, 0};
  for (; k < ke; k += 512) {
    u32x4 wc[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) wc[c] = wn[c];
    if (k + 512 < ke) {
#pragma unroll
      for (int c = 0; c < CPW; ++c) wn[c] = __builtin_nontemporal_load((const u32x4*)(wr[c] + k + 512));
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const u32x4 xv = *(const u32x4*)(xs + m * K + k);
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        float a = acc[c][m];
        a = dot2(wc[c][0], xv[0], a);
        a = dot2(wc[c][1], xv[1], a);
        a = dot2(wc[c][2], xv[2], a);
        a = dot2(wc[c][3], xv[3], a);
        acc[c][m] = a;
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v = acc[c][m];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
      acc[c][m] = v;
    }
  if constexpr (KS == 4) {  // the quarters of K: wave 0 adds the others' sums
    if (lane == 0) {
#pragma unroll
      for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int m = 0; m < M; ++m) red[wave][c * M + m] = acc[c][m];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int m = 0; m < M; ++m)
        acc[c][m] = red[0][c * M + m] + red[1][c * M + m] + red[2][c * M + m] + red[3][c * M + m];
  }
  // lane c * M + m stores column n0 + c of row m
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int n = n0 + c;
      if (lane != c * M + m || n >= N) continue;
      const float v = acc[c][m];
      if (out.f32) {
        ((float*)out.y)[(int64_t)m * out.ldy + n] = v;
        continue;
      }
      const bf16 b = (bf16)v;
      ((bf16*)out.y)[(int64_t)m * out.ldy + n] = b;
      if (out.k_col >= 0) {
        bf16* ring = nullptr;
        int rel = 0;
        if (n >= out.k_col && n < out.k_col + out.kvw) {
          ring = (bf16*)out.ring_k;
          rel = n - out.k_col;
        } else if (n >= out.v_col && n < out.v_col + out.kvw) {
          ring = (bf16*)out.ring_v;
          rel = n - out.v_col;
        }
        if (ring != nullptr) {
          const int slot = max(out.pos[m], 0) % out.slots;
          const int gh = rel / out.head_dim, d = rel % out.head_dim;
          ring[(((int64_t)m * out.Hkv + gh) * out.slots + slot) * out.head_dim + d] = b;
        }
      }
    }
}

bool gemv_bf16_ok(int M, int K, int64_t ldx, int64_t ldw) {
  return M >= 1 && M <= kGemvMaxRows && K > 0 && K % 8 == 0 && ldx % 8 == 0 && ldw % 8 == 0 &&
         (size_t)M * K * 2 <= 64 * 1024;
}

hipError_t launch_gemv_bf16(const void* x, int64_t ldx, const void* w, int64_t ldw, int M, int N,
                            int K, const GemvOut& out, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (!gemv_bf16_ok(M, K, ldx, ldw) || out.y == nullptr || ((uintptr_t)x & 15) ||
      ((uintptr_t)w & 15))
    return hipErrorInvalidValue;
  const size_t lds = (size_t)M * K * 2;
  // Wide outputs (in_proj): a wave per 4 columns, N / 16 workgroups.  Narrower ones split
  // K over the 4 waves of a workgroup: 4 columns per workgroup from N = 1024 (out_proj:
  // 512 workgroups), 1 column below (x_proj).
  const int mode = N >= 8192 ? 0 : (N >= 1024 ? 1 : 2);
  const dim3 grid(mode == 0 ? (N + 15) / 16 : mode == 1 ? (N + 3) / 4 : N), blk(256);
  auto go = [&](auto mc, auto cc, auto kc) {
    constexpr int MM = decltype(mc)::value, CC = decltype(cc)::value, KK = decltype(kc)::value;
    gemv_bf16_kernel<MM, CC, KK><<<grid, blk, lds, s>>>((const bf16*)x, ldx, (const bf16*)w, ldw,
                                                        N, K, out);
  };
  auto by_cpw = [&](auto mc) {
    if (mode == 0) go(mc, std::integral_constant<int, 4>(), std::integral_constant<int, 1>());
    else if (mode == 1) go(mc, std::integral_constant<int, 4>(), std::integral_constant<int, 4>());
    else go(mc, std::integral_constant<int, 1>(), std::integral_constant<int, 4>());
  };
  switch (M) {
    case 1: by_cpw(std::integral_constant<int, 1>()); break;
    case 2: by_cpw(std::integral_constant<int, 2>()); break;
    case 3: by_cpw(std::integral_constant<int, 3>()); break;
    default: by_cpw(std::integral_constant<int, 4>()); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_decode_in(const GemmOperands& op, void* z, int64_t ldz, int k_col,
                                      int v_col, void* ring_k, void* ring_v, int slots, int Hkv,
                                      int head_dim, const int32_t* pos, float* zero,
                                      int64_t zero_n, hipStream_t s) {
  if (op.M <= 0 || op.N <= 0) return hipSuccess;
  if (!fewrow_ok(op) || zero_n % 4 != 0 || ((uintptr_t)zero & 15)) return hipErrorInvalidValue;
  FewRowOut out{};
  out.zero = (floatx4*)zero;
  out.zero_n4 = zero_n / 4;
  out.z = (bf16*)z;
  out.ldz = ldz;
  out.k_col = k_col;
  out.v_col = v_col;
  out.ring_k = (bf16*)ring_k;
  out.ring_v = (bf16*)ring_v;
  out.slots = slots;
  out.kvw = Hkv * head_dim;
  out.head_dim = head_dim;
  out.Hkv = Hkv;
  out.pos = pos;
  out.vec = ((uintptr_t)z & 15) == 0 && ldz % 8 == 0 &&
            (k_col < 0 || (((uintptr_t)ring_k & 15) == 0 && ((uintptr_t)ring_v & 15) == 0 &&
                           head_dim % 8 == 0 && k_col % 8 == 0 && v_col % 8 == 0));
  // 128-row blocks: each weight slice is streamed by one workgroup (64-row blocks, twice
  // the workgroups, measured about 10% slower at 128 rows)
  dim3 grid((op.N + 63) / 64, 1, (op.M + 127) / 128);
  gemm_bf16_fewrow_kernel<kFewStore, 128, 4><<<grid, dim3(256), 0, s>>>(op, out, op.K);
  return hipGetLastError();
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
