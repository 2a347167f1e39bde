// Attention heads of the hybrid-head layer.
//
// Source: "Hymba: A Hybrid-head Architecture for Small Language Models" (outta.ai
// summary): Design formulation, attention-head equation (softmax(Q K^T) mixing the
// meta-prefixed tokens); "Meta Tokens" (meta keys are always attended);
// "Combine global and local attention" (sliding window); "Cross-layer KV sharing"
// (a layer may read its producer's K/V).  GQA grouping per the Chinese summary's
// KV-sharing section.  Mask: key j is visible to query i iff j <= i and
// (j < M or window == 0 or i - j < window); scale 1/sqrt(head_dim) unless given.
//
// Prefill (bf16): flash-style, one workgroup per (query block, kv head, head
// subgroup).  Its waves each own 16 * QT query rows of one q head (QT = 2: 32 rows,
// 8 waves, two per SIMD); all share the K/V tiles of their kv head staged in LDS.  The
// waves compute S^T = K Q^T with v_mfma_f32_16x16x32_bf16, so the softmax statistics
// of a query live in one lane column, and O^T = V^T P^T takes P^T straight from the S^T
// accumulators (the 32-key k-order of the second MFMA is permuted to match them; V is
// staged transposed and permuted the same way).  The key loop is software-pipelined:
// a wave forms S^T of the next tile while it runs the softmax of the current one.  Key
// tiles that hold no visible key for the block (outside the meta prefix and the
// window) are skipped; which tiles those are is a closed form of the block's range.
// Measured on MI355X: 4 waves of 48 or 64 query rows (one wave per SIMD, half the LDS
// reads per MFMA) and 4 K/V stages instead of 3 were not faster.
#include <float.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.f;  // lazy-rescaling headroom (log2 units)

// X~ position -> row of the query / Z arrays.
__device__ __forceinline__ int64_t q_row(const AttnParams& p, int pos, int b) {
  return pos < p.n_meta ? (int64_t)pos
                        : (int64_t)p.meta_rows + (int64_t)b * p.L + (pos - p.n_meta);
}

template <typename T>
__device__ __forceinline__ const T* key_ptr(const T* meta, const T* seq, const AttnParams& p,
                                            int b, int g, int j) {
  if (j < p.n_meta) return meta + g * p.meta_head_stride + (int64_t)j * p.meta_row_stride;
  const int slot = (j - p.n_meta) % p.seq_slots;
  return seq + (int64_t)b * p.seq_batch_stride + g * p.seq_head_stride +
         (int64_t)slot * p.seq_row_stride;
}


}  // namespace

// ------------------------------------------------- bf16 prefill, direct-to-LDS tiles
// V^T staging: the P V product needs, per lane, 8 consecutive keys of one head_dim
// column (the k operand of the MFMA), while V is stored key-major.  A small kernel
// writes V^T per (sequence, kv head): vt[b][g][d][slot] over the meta-prefixed key axis
// (tpad = keys rounded up to 64, zero past the end), keys permuted inside each 32-key
// block to the slot order of the S^T accumulators (slot_key).  Then both the K tile
// (64 keys x head_dim, key-major) and the V^T tile (head_dim x 64 slots) move straight
// from global memory into LDS with global_load_lds_dwordx4 (no register staging, no
// scattered LDS stores), NS stages deep.
namespace {
// Slot order of V^T inside a 64-key tile: the P^T operand a lane builds from its S^T
// accumulators holds, for k-block q = lane / 16 of 32-key half blk, the keys
// blk*32 + 4q + (0..3) and blk*32 + 16 + 4q + (0..3); V^T slots blk*32 + 8q + (0..7)
// hold the same keys in the same order.  slot_key maps a slot to its key.
__device__ __forceinline__ int slot_key(int s) {
  const int blk = s >> 5, q = (s & 31) >> 3, i = s & 7;
  return blk * 32 + (i < 4 ? q * 4 + i : 16 + q * 4 + (i - 4));
}
// Chunk permutation of a 128-byte LDS row r (8 16-byte chunks) for tiles whose fragment
// reads take row (lane % 16), chunk (lane / 16) + const: a bit permutation of r's low
// three bits, free of LDS bank conflicts for that read on gfx950 (measured; the
// (r & 7) ^ (r >> 3 & 1) form spends half its read cycles in conflicts there).
__device__ __forceinline__ int swz8(int r) { return (r & 1) | ((r << 1) & 4) | ((r >> 1) & 2); }
// Sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (same butterflies as below).
__device__ __forceinline__ float sum_over_key_lanes(float x) {
  const auto s16 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x), false, false);
  const float y = __builtin_bit_cast(float, (unsigned)s16[0]) +
                  __builtin_bit_cast(float, (unsigned)s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, y),
                                                    __builtin_bit_cast(unsigned, y), false, false);
  return __builtin_bit_cast(float, (unsigned)s32[0]) + __builtin_bit_cast(float, (unsigned)s32[1]);
}
// Maximum over lanes l, l ^ 16, l ^ 32, l ^ 48: v_permlane16_swap exchanges the odd
// 16-lane rows of its first operand with the even rows of its second, v_permlane32_swap
// the upper half of the first with the lower half of the second; with both operands a
// copy of x, the two results hold the butterfly partners.
__device__ __forceinline__ float max_over_key_lanes(float x) {
  const auto s16 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x), false, false);
  const float y = fmaxf(__builtin_bit_cast(float, (unsigned)s16[0]),
                        __builtin_bit_cast(float, (unsigned)s16[1]));
  const auto s32 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, y),
                                                    __builtin_bit_cast(unsigned, y), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)s32[0]),
               __builtin_bit_cast(float, (unsigned)s32[1]));
}
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void dma16(const void* gptr, lds_void_t* lptr) {
  // global_load_lds_dwordx4 from inline asm: no VGPR result; the consumer waits
  // explicitly (vmcnt) and then passes a workgroup barrier.
  const uint32_t l = (uint32_t)(uintptr_t)lptr;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(l)), "v"(gptr) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
}  // namespace

template <int DH>
__global__ __launch_bounds__(256) void vt_build_kernel(AttnParams p, bf16* vt, int tpad) {
  __shared__ bf16 vs[64][DH + 8];
  const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int total = p.n_meta + p.L;
  constexpr int CPR = DH / 8;
  for (int q = tid; q < 64 * CPR; q += 256) {
    const int k = q / CPR, c = q % CPR, j = t * 64 + k;
    u32x4 v = u32x4{0, 0, 0, 0};
    if (j < total) v = *(const u32x4*)(key_ptr((const bf16*)p.v_meta, (const bf16*)p.v_seq, p, b, g, j) + c * 8);
    *(u32x4*)(&vs[k][c * 8]) = v;
  }
  __syncthreads();
  bf16* dst = vt + ((int64_t)b * p.Hkv + g) * DH * tpad + t * 64;
  for (int q = tid; q < DH * 8; q += 256) {
    const int d = q / 8, c = q % 8;
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = vs[slot_key(c * 8 + i)][d];
    *(bf16x8*)(dst + (int64_t)d * tpad + c * 8) = o;
  }
}

template <int DH, int NW, int NS, int QT>
__global__ __launch_bounds__(NW * 64, 1) void attn_prefill_dl_kernel(
    AttnParams p, const bf16* __restrict__ vt, int tpad, int gq, int qb, int nblk_seq) {
  constexpr int KT = 64;
  constexpr int KB = KT * DH;            // elements of a K tile and of a V^T tile
  constexpr int INS = DH / 8 / NW;       // 1 KB DMA wave instructions per wave, per matrix
  static_assert(INS >= 1 && NS >= 3 && NS <= 4, "tile loader");
  __shared__ __attribute__((aligned(1024))) bf16 smem[NS * 2 * KB];
  auto kst = [&](int st) { return smem + st * 2 * KB; };
  auto vst = [&](int st) { return smem + st * 2 * KB + KB; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // One grid dimension, ordered longest blocks first across every head group and
  // sequence (the blocks of the last query range see the most keys), so the heaviest
  // workgroups start first and the short ones fill the tail; the meta blocks come last.
  // The sequence varies fastest: workgroups go to the 8 XCDs round-robin, so with 8
  // sequences each XCD's L2 serves the K/V of one sequence.
  const int ngrp = p.Hq / gq;
  const int nseq = p.B * nblk_seq * ngrp;
  int b, p0, plim, hgi;
  if ((int)blockIdx.x < nseq) {
    b = blockIdx.x % p.B;
    hgi = (blockIdx.x / p.B) % ngrp;
    const int qi = nblk_seq - 1 - blockIdx.x / (p.B * ngrp);
    p0 = p.n_meta + qi * qb;
    plim = p.n_meta + min(p.L, (qi + 1) * qb);
  } else {
    b = 0;
    hgi = (blockIdx.x - nseq) % ngrp;
    const int mi = (blockIdx.x - nseq) / ngrp;
    p0 = mi * qb;
    plim = min(p.n_meta, (mi + 1) * qb);
  }
  const int h0 = hgi * gq;
  const int h = h0 + (wave % gq);
  const int g = (h0 * p.Hkv) / p.Hq;
  constexpr int QW = 16 * QT;  // queries per wave
  const int wp0 = p0 + (wave / gq) * QW;

  const bf16* qbase = (const bf16*)p.q;
  // K rows of this (sequence, kv head): meta key j at kmeta + j*meta_row_stride, key
  // j >= n_meta at kseq + (j - n_meta)*seq_row_stride (prefill sources hold every
  // position: seq_slots >= L, so no ring wrap).
  const bf16* kmeta = (const bf16*)p.k_meta + g * p.meta_head_stride;
  const bf16* kseq = (const bf16*)p.k_seq + (int64_t)b * p.seq_batch_stride + g * p.seq_head_stride;
  const bf16* vtb = vt + ((int64_t)b * p.Hkv + g) * DH * tpad;

  bf16x8 qf[QT][DH / 32];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int pos = wp0 + qt * 16 + (lane & 15);
    const bool ok = pos < plim;
    const bf16* src = qbase + q_row(p, ok ? pos : p0, b) * p.q_row_stride + h * DH +
                      (lane >> 4) * 8;
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks) {
      u32x4 v = ok ? *(const u32x4*)(src + ks * 32) : u32x4{0, 0, 0, 0};
      qf[qt][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  floatx4 oacc[DH / 16][QT];
  float mrow[QT];
  floatx4 lacc[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int i = 0; i < DH / 16; ++i) oacc[i][qt] = floatx4{0.f, 0.f, 0.f, 0.f};
    mrow[qt] = -INFINITY;
    lacc[qt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (bf16)1.f;

  // Key tiles with a visible key for this block: the meta tiles [0, mt) and the tiles
  // from the window's start wt on, up to ntile (all wave-uniform).
  const int meta_end = min(p.n_meta, plim);
  const int wlo = p.window > 0 ? max(p.n_meta, p0 - p.window + 1) : p.n_meta;
  const int ntile = __builtin_amdgcn_readfirstlane((plim + KT - 1) / KT);
  const int mt = __builtin_amdgcn_readfirstlane((meta_end + KT - 1) / KT);
  const int wt = __builtin_amdgcn_readfirstlane(wlo / KT);
  auto next_tile = [&](int t) {
    const int u = t + 1 < mt ? t + 1 : max(t + 1, wt);
    return min(u, ntile);
  };

  // DMA of tile t into stage st.  K: 1 KB block (j*NW + wave) of the tile holds rows
  // of 256 B (DH 128: 4 rows) or 128 B (DH 64: 8 rows), each row's 16-byte chunks
  // XOR-permuted (chunk ^ (row & 15), resp. chunk ^ swz8(row)).  V^T rows are 128 B
  // (64 slots), chunk ^ swz8(row).  Keys past the visible end read the last one (masked).
  // A tile wholly inside the sequence's keys takes the per-lane offsets below plus one
  // wave-uniform base per matrix.
  int krow_of[INS], kof[INS], vof[INS];
#pragma unroll
  for (int j = 0; j < INS; ++j) {
    const int blk = j * NW + wave;
    int row, gch;
    if constexpr (DH == 128) {
      row = blk * 4 + (lane >> 4);
      gch = (lane & 15) ^ (row & 15);
    } else {
      row = blk * 8 + (lane >> 3);
      gch = (lane & 7) ^ swz8(row);
    }
    krow_of[j] = row;
    kof[j] = row * p.seq_row_stride + gch * 8;
    const int vr = blk * 8 + (lane >> 3);
    vof[j] = vr * tpad + ((lane & 7) ^ swz8(vr)) * 8;
  }
  auto issue = [&](int st, int t) {
    const int a = t * KT;
    if (a >= p.n_meta && a + KT <= plim) {
      const bf16* kb = kseq + (int64_t)(a - p.n_meta) * p.seq_row_stride;
#pragma unroll
      for (int j = 0; j < INS; ++j) {
        const int blk = j * NW + wave;
        dma16(kb + kof[j], (lds_void_t*)(kst(st) + blk * 512));
        dma16(vtb + a + vof[j], (lds_void_t*)(vst(st) + blk * 512));
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < INS; ++j) {
      const int blk = j * NW + wave;
      const int row = krow_of[j];
      const int gch = (kof[j] - row * p.seq_row_stride) / 8;
      const int key = min(a + row, plim - 1);
      const bf16* krow = key < p.n_meta ? kmeta + (int64_t)key * p.meta_row_stride
                                        : kseq + (int64_t)(key - p.n_meta) * p.seq_row_stride;
      dma16(krow + gch * 8, (lds_void_t*)(kst(st) + blk * 512));
      dma16(vtb + a + vof[j], (lds_void_t*)(vst(st) + blk * 512));
    }
  };

  const float c2 = p.scale * kLog2e;
  // Software pipeline over the key tiles: while a wave runs the softmax of tile t (VALU),
  // it forms S^T of the next tile (MFMA), so the two kinds of work overlap inside the
  // wave.  During step t the tiles t and tq[0] are resident in LDS; tq[1..] may be in
  // flight.
  int t = mt > 0 ? 0 : min(wt, ntile);
  int tq[NS - 1];  // tiles issued after the current one, in order (ntile: none)
  int st = 0;
  if (t < ntile) issue(0, t);
  {
    int prev = t;
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) {
      tq[i] = prev < ntile ? next_tile(prev) : ntile;
      if (tq[i] < ntile) issue(i + 1, tq[i]);
      prev = tq[i];
    }
  }
  // wait until at most n tiles' DMAs are still in flight (this wave's; a barrier follows)
  auto wait_tiles = [&](int n) {
    if (n >= 2) wait_vm<4 * INS>();
    else if (n == 1) wait_vm<2 * INS>();
    else wait_vm<0>();
  };
  {
    int n = 0;
#pragma unroll
    for (int i = 1; i < NS - 1; ++i) n += tq[i] < ntile;
    wait_tiles(n);
  }
  lds_barrier();

  constexpr int KS = DH / 32;  // k-steps of S^T = K Q^T
  auto load_k = [&](const bf16* kt_, int ks, bf16x8 (&kf)[4]) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int row = kt * 16 + (lane & 15), c = ks * 4 + (lane >> 4);
      const int sw = DH == 128 ? (c ^ (row & 15)) : (c ^ swz8(row));
      kf[kt] = *(const bf16x8*)(kt_ + row * DH + sw * 8);
    }
  };
  auto s_mfma = [&](const bf16x8 (&kf)[4], int ks, floatx4 (&s)[4][QT]) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[kt][qt] = mfma16x16x32(kf[kt], qf[qt][ks], s[kt][qt]);
  };
  auto zero_s = [&](floatx4 (&s)[4][QT]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[i][qt] = floatx4{0.f, 0.f, 0.f, 0.f};
  };
  // Mask S^T[key j][query i] of tile tt to -inf where j is not visible.  Lane holds keys
  // j = a + c + 4 (lane / 16) with c = 16 kt + r, so each condition is one compare of
  // the constant c with a per-lane threshold: j <= i <=> c <= lim; j < n_meta <=>
  // c < mlim; i - j < window <=> c > lim - window.
  auto mask = [&](floatx4 (&s)[4][QT], int tt) {
    const int a = tt * KT;
    const int i_lo = wp0, i_hi = min(wp0 + QW - 1, plim - 1);
    const bool full = a + KT - 1 <= i_lo &&
                      (p.window <= 0 || a + KT <= p.n_meta || i_hi - max(a, p.n_meta) < p.window);
    if (full) return;
    const int lq = (lane >> 4) * 4;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int lim = wp0 + qt * 16 + (lane & 15) - a - lq;
      if (p.window <= 0) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kt * 16 + r > lim) s[kt][qt][r] = -INFINITY;
      } else {
        const int mlim = p.n_meta - a - lq, wlim = lim - p.window;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int c = kt * 16 + r;
            if (c > lim || (c >= mlim && c <= wlim)) s[kt][qt][r] = -INFINITY;
          }
      }
    }
  };

  // One step: softmax of tile t held in `sc` and its P V product, overlapped with S^T of
  // the next tile into `sn` (kNext).  Returns true after the last tile.
  auto step = [&](auto next_c, floatx4 (&sc)[4][QT], floatx4 (&sn)[4][QT])
                  __attribute__((always_inline)) {
    constexpr bool kNext = decltype(next_c)::value;
    const bf16* ktn = kst(st + 1 == NS ? 0 : st + 1);
    const bf16* vt_ = vst(st);
    mask(sc, t);
    // Row maxima of the tile, then lazy rescaling: the running max m moves only when
    // some row's tile max exceeds it by more than kLazyLog2 in log2 units (wave-uniform
    // decision), so O and l are rescaled rarely and every exp2 argument stays <=
    // kLazyLog2 (P <= 2^kLazyLog2, exact in the fp32 sums and in bf16 for the MFMA).
    // O / l is unchanged by the choice of m.  The first half of the next tile's S^T
    // MFMAs runs beside the maxima.
    bf16x8 kf0[4], kf1[4];
    if constexpr (kNext) {
      zero_s(sn);
      load_k(ktn, 0, kf0);
      if constexpr (KS > 2) load_k(ktn, 1, kf1);
    }
    float tmax[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = sc[0][qt][0];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[kt][qt][r]);
      tmax[qt] = max_over_key_lanes(mx);
    }
    if constexpr (kNext) {
      s_mfma(kf0, 0, sn);
      if constexpr (KS > 2) s_mfma(kf1, 1, sn);
    }
    const float thr = kLazyLog2 / c2;
    bool grow = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) grow = grow || tmax[qt] > mrow[qt] + thr;
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float mnew = fmaxf(mrow[qt], tmax[qt]);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f((mrow[qt] - muse) * c2);  // 0 from -inf
        mrow[qt] = mnew;
        lacc[qt] *= alpha;
#pragma unroll
        for (int d = 0; d < DH / 16; ++d) oacc[d][qt] *= alpha;
      }
    }
    // P^T in bf16 (the B operand of both MFMAs below); the row sums l come from the same
    // rounded P through an MFMA with an all-ones A operand (every output row of it is
    // the column sum, so each lane ends with the full sum of its query).  The second
    // half of the next tile's S^T MFMAs runs beside the exponentials.
    if constexpr (kNext) {
      load_k(ktn, KS > 2 ? 2 : 1, kf0);
      if constexpr (KS > 2) load_k(ktn, 3, kf1);
    }
    bf16x8 pf[2][QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float mc2 = (mrow[qt] == -INFINITY ? 0.f : mrow[qt]) * c2;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        bf16x8 f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f[r] = (bf16)__builtin_amdgcn_exp2f(fmaf(sc[2 * k2][qt][r], c2, -mc2));
          f[4 + r] = (bf16)__builtin_amdgcn_exp2f(fmaf(sc[2 * k2 + 1][qt][r], c2, -mc2));
        }
        pf[k2][qt] = f;
        lacc[qt] = mfma16x16x32(ones, f, lacc[qt]);
      }
    }
    if constexpr (kNext) {
      s_mfma(kf0, KS > 2 ? 2 : 1, sn);
      if constexpr (KS > 2) s_mfma(kf1, 3, sn);
    }
    // O^T += V^T P^T (the V^T fragments are read only now: earlier they would be live
    // beside both S^T tiles)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < DH / 16; ++d) {
      bf16x8 vf[2];
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int row = d * 16 + (lane & 15), c = k2 * 4 + (lane >> 4);
        vf[k2] = *(const bf16x8*)(vt_ + row * 64 + ((c ^ swz8(row)) * 8));
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          oacc[d][qt] = mfma16x16x32(vf[k2], pf[k2][qt], oacc[d][qt]);
    }
    if constexpr (!kNext) return true;
    // hand-over: tiles tq[0] and tq[1] are resident, every wave is done with this stage,
    // which then takes the tile after the ones issued
    {
      int n = 0;
#pragma unroll
      for (int i = 2; i < NS - 1; ++i) n += tq[i] < ntile;
      wait_tiles(n);
    }
    lds_barrier();
    int tlast = t;
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) tlast = tq[i] < ntile ? tq[i] : tlast;
    const int tnew = tq[NS - 2] < ntile ? next_tile(tlast) : ntile;
    if (tnew < ntile) issue(st, tnew);
    t = tq[0];
#pragma unroll
    for (int i = 0; i + 1 < NS - 1; ++i) tq[i] = tq[i + 1];
    tq[NS - 2] = tnew;
    st = st + 1 == NS ? 0 : st + 1;
    return false;
  };

  floatx4 sa[4][QT], sb[4][QT];
  if (t < ntile) {  // S^T of the first tile
    zero_s(sa);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 kf[4];
      load_k(kst(st), ks, kf);
      s_mfma(kf, ks, sa);
    }
    while (tq[0] < ntile) {
      step(std::true_type{}, sa, sb);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) sa[i][qt] = sb[i][qt];
    }
    step(std::false_type{}, sa, sb);
  }

  // O^T layout: lane holds head_dim entries d*16 + 4*(lane/16) + r of query lane % 16.
  // With p.ssp, O is rounded to bf16 first (as stored O would be); the row's sum of its
  // squares over this head (the 4 lanes of a query) goes to ssp[h, row] and beta * O is
  // stored.
  bf16* obase = (bf16*)p.o;
  const float* bh = p.beta != nullptr ? p.beta + h * DH + (lane >> 4) * 4 : nullptr;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float l = lacc[qt][0];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int pos = wp0 + qt * 16 + (lane & 15);
    float o[DH / 16][4];
#pragma unroll
    for (int d = 0; d < DH / 16; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[d][r] = oacc[d][qt][r] * inv;
    const int64_t row = q_row(p, pos < plim ? pos : p0, b);
    if (p.ssp != nullptr) {
      float q = 0.f;
#pragma unroll
      for (int d = 0; d < DH / 16; ++d)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          o[d][r] = (float)(bf16)o[d][r];
          q = fmaf(o[d][r], o[d][r], q);
        }
      q = sum_over_key_lanes(q);
      if (pos < plim && lane < 16) p.ssp[h * p.ssp_ld + row] = q;
#pragma unroll
      for (int d = 0; d < DH / 16; ++d) {
        const floatx4 bv = *(const floatx4*)(bh + d * 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) o[d][r] *= bv[r];
      }
    }
    if (pos >= plim) continue;
    bf16* dst = obase + row * p.o_row_stride + h * DH + (lane >> 4) * 4;
#pragma unroll
    for (int d = 0; d < DH / 16; ++d) {
      bf16x4 ov;
      ov[0] = (bf16)o[d][0];
      ov[1] = (bf16)o[d][1];
      ov[2] = (bf16)o[d][2];
      ov[3] = (bf16)o[d][3];
      *(bf16x4*)(dst + d * 16) = ov;
    }
  }
}

template <int DH, int NW, int NS, int QT>
static hipError_t run_attn_dl(const AttnParams& p, void* vt, hipStream_t s) {
  const int total = p.n_meta + p.L;
  const int tpad = (total + 63) / 64 * 64;
  const int vb = (p.B > 0 ? p.B : 1);
  vt_build_kernel<DH><<<dim3(tpad / 64, p.Hkv, vb), dim3(256), 0, s>>>(p, (bf16*)vt, tpad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grp = p.Hq / p.Hkv;
  const int gq = grp % 4 == 0 ? 4 : (grp % 2 == 0 ? 2 : 1);
  const int qb = 16 * QT * (NW / gq);
  const int nblk_seq = (p.L + qb - 1) / qb;
  const int nblk_meta = p.meta_rows > 0 ? (p.n_meta + qb - 1) / qb : 0;
  const int nx = p.B * nblk_seq + nblk_meta;
  if (nx == 0) return hipSuccess;
  attn_prefill_dl_kernel<DH, NW, NS, QT><<<dim3(nx * (p.Hq / gq)), dim3(NW * 64), 0, s>>>(
      p, (const bf16*)vt, tpad, gq, qb, nblk_seq);
  return hipGetLastError();
}

size_t attention_vt_bytes(int n_meta, int L, int B, int Hkv, int head_dim) {
  const int64_t tpad = (int64_t)(n_meta + L + 63) / 64 * 64;
  return (size_t)(B > 0 ? B : 1) * Hkv * head_dim * tpad * 2;
}

hipError_t launch_attention_prefill_bf16_dl(const AttnParams& p, void* vt, hipStream_t s) {
  if (p.head_dim == 128) return run_attn_dl<128, 8, 3, 2>(p, vt, s);
  if (p.head_dim == 64) return run_attn_dl<64, 8, 3, 2>(p, vt, s);
  return hipErrorInvalidValue;
}

// --------------------------------------------------------------------- fp32 prefill
// One wave per (query row, q head); lanes cover head_dim (<= 128).  Plain online
// softmax over the visible keys.
template <typename T>
__global__ __launch_bounds__(64) void attn_prefill_simple_kernel(AttnParams p) {
  const int r = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  int b, i;
  if (r < p.meta_rows) {
    b = 0;
    i = r;
  } else {
    b = (r - p.meta_rows) / p.L;
    i = p.n_meta + (r - p.meta_rows) % p.L;
  }
  const int g = (h * p.Hkv) / p.Hq;
  const int dh = p.head_dim;
  const T* q = (const T*)p.q + (int64_t)r * p.q_row_stride + h * dh;
  const float q0 = lane < dh ? to_f32(q[lane]) : 0.f;
  const float q1 = lane + 64 < dh ? to_f32(q[lane + 64]) : 0.f;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  const int jlo = p.window > 0 ? max(p.n_meta, i - p.window + 1) : p.n_meta;
  for (int j = 0; j <= i; ++j) {
    if (j >= p.n_meta && j < jlo) {
      j = jlo - 1;
      continue;
    }
    const T* k = key_ptr((const T*)p.k_meta, (const T*)p.k_seq, p, b, g, j);
    const T* v = key_ptr((const T*)p.v_meta, (const T*)p.v_seq, p, b, g, j);
    float part = (lane < dh ? q0 * to_f32(k[lane]) : 0.f) +
                 (lane + 64 < dh ? q1 * to_f32(k[lane + 64]) : 0.f);
    const float s = wave_sum(part) * p.scale;
    const float mn = fmaxf(m, s);
    const float al = __expf(m - mn);
    const float e = __expf(s - mn);
    l = l * al + e;
    o0 = o0 * al + e * (lane < dh ? to_f32(v[lane]) : 0.f);
    o1 = o1 * al + e * (lane + 64 < dh ? to_f32(v[lane + 64]) : 0.f);
    m = mn;
  }
  T* o = (T*)p.o + (int64_t)r * p.o_row_stride + h * dh;
  if (lane < dh) o[lane] = from_f32<T>(o0 / l);
  if (lane + 64 < dh) o[lane + 64] = from_f32<T>(o1 / l);
}

hipError_t launch_attention_prefill_f32(const AttnParams& p, hipStream_t s) {
  const int rows = p.meta_rows + p.B * p.L;
  if (rows == 0) return hipSuccess;
  attn_prefill_simple_kernel<float><<<dim3(rows, p.Hq), dim3(64), 0, s>>>(p);
  return hipGetLastError();
}

// --------------------------------------------------------------------- decode
// Workgroup per (key split, kv head, sequence); 4 waves of 64 keys each.  A key's
// head_dim values are spread over LPK lanes that each own one 16-byte chunk, so a wave
// instruction reads KPI whole rows of K (or V) contiguously.  Scores: every lane dots
// its chunk with the same chunk of each q head (held in registers), then a DPP
// butterfly over the key's lanes finishes the sums.  Values: each lane accumulates
// its chunk of O for every head; lanes of different keys are summed at the end.
// Keys of sequence b in order: M meta entries, then X-positions pos - span + 1 .. pos
// at ring slot (position % slots), span = min(pos + 1, span_max).
namespace {

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// Sum over aligned groups of LPK lanes (LPK in {4, 8, 16}), result in every lane.
template <int LPK>
__device__ __forceinline__ float lane_group_sum(float v) {
  v += dppf<0xB1>(v);                           // quad_perm [1,0,3,2]
  v += dppf<0x4E>(v);                           // quad_perm [2,3,0,1]
  if constexpr (LPK >= 8) v += dppf<0x141>(v);  // row_half_mirror
  if constexpr (LPK >= 16) v += dppf<0x140>(v); // row_mirror
  return v;
}

template <typename T>
struct Chunk;
template <>
struct Chunk<bf16> {
  static constexpr int E = 8;
  static __device__ __forceinline__ void cvt(const u32x4& r, float* f) {
    const bf16x8 v = __builtin_bit_cast(bf16x8, r);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (float)v[e];
  }
};
template <>
struct Chunk<float> {
  static constexpr int E = 4;
  static __device__ __forceinline__ void cvt(const u32x4& r, float* f) {
    const floatx4 v = __builtin_bit_cast(floatx4, r);
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = v[e];
  }
};

}  // namespace

template <typename T, int DH, int GQ, int KPS>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnDecodeParams p) {
  constexpr int E = Chunk<T>::E;     // elements per 16-byte chunk
  constexpr int LPK = DH / E;        // lanes per key
  constexpr int KPI = 64 / LPK;      // keys per wave instruction
  constexpr int KPW = KPS / 4;       // keys per wave
  constexpr int NI = KPW / KPI;      // instructions per wave
  static_assert(LPK >= 4 && LPK <= 16, "lane grouping");
  static_assert(KPS % (4 * KPI) == 0 && KPS % 64 == 0, "keys per split");
  __shared__ float s_s[GQ][KPS];
  __shared__ float mstat[GQ], lstat[GQ];
  __shared__ float o_s[4][GQ][DH];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h0 = g * GQ;
  const int posb = max(p.pos[b], 0);  // a negative position is treated as 0
  const int span = min(posb + 1, p.span_max);
  const int nkeys = p.n_meta + span;
  const int k0 = split * KPS;
  const int nk = min(KPS, nkeys - k0);  // may be <= 0: empty split
  const int dc = lane % LPK, kin = lane / LPK;

  float q[GQ][E];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    float f[E];
    Chunk<T>::cvt(*(const u32x4*)((const T*)p.q + (int64_t)b * p.q_row_stride + (h0 + h) * DH + dc * E), f);
#pragma unroll
    for (int e = 0; e < E; ++e) q[h][e] = f[e] * p.scale;
  }

  auto row_of = [&](const T* meta, const T* ring, int idx) -> const T* {
    if (idx < p.n_meta) return meta + ((int64_t)g * p.n_meta + idx) * DH;
    const int xpos = posb - span + 1 + (idx - p.n_meta);
    return ring + (((int64_t)b * p.Hkv + g) * p.slots + (xpos % p.slots)) * DH;
  };

  // scores
  u32x4 raw[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int kk = wave * KPW + i * KPI + kin;
    raw[i] = kk < nk ? *(const u32x4*)(row_of((const T*)p.k_meta, (const T*)p.k, k0 + kk) + dc * E)
                     : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int kk = wave * KPW + i * KPI + kin;
    float kf[E];
    Chunk<T>::cvt(raw[i], kf);
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) part = fmaf(q[h][e], kf[e], part);
      part = lane_group_sum<LPK>(part);
      if (dc == 0) s_s[h][kk] = kk < nk ? part : -INFINITY;
    }
  }
  // V loads do not depend on the softmax: issue them before the reduction.
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int kk = wave * KPW + i * KPI + kin;
    raw[i] = kk < nk ? *(const u32x4*)(row_of((const T*)p.v_meta, (const T*)p.v, k0 + kk) + dc * E)
                     : u32x4{0, 0, 0, 0};
  }
  __syncthreads();

  for (int h = wave; h < GQ; h += 4) {
    float mx = -INFINITY;
    for (int k = lane; k < KPS; k += 64) mx = fmaxf(mx, s_s[h][k]);
    mx = wave_max(mx);
    const float muse = mx == -INFINITY ? 0.f : mx;
    float sum = 0.f;
    for (int k = lane; k < KPS; k += 64) {
      const float e = __expf(s_s[h][k] - muse);
      s_s[h][k] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      mstat[h] = mx;
      lstat[h] = sum;
    }
  }
  __syncthreads();

  float o[GQ][E];
#pragma unroll
  for (int h = 0; h < GQ; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) o[h][e] = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int kk = wave * KPW + i * KPI + kin;
    float vf[E];
    Chunk<T>::cvt(raw[i], vf);
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      const float pk = s_s[h][kk];
#pragma unroll
      for (int e = 0; e < E; ++e) o[h][e] = fmaf(pk, vf[e], o[h][e]);
    }
  }
  // sum the KPI key groups of the wave (lanes with the same chunk index)
#pragma unroll
  for (int h = 0; h < GQ; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float v = o[h][e];
#pragma unroll
      for (int off = LPK; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
      o[h][e] = v;
    }
  if (kin == 0) {
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
      for (int e = 0; e < E; ++e) o_s[wave][h][dc * E + e] = o[h][e];
  }
  __syncthreads();
  for (int i = tid; i < GQ * DH; i += 256) {
    const int h = i / DH, d = i % DH;
    const float sum = o_s[0][h][d] + o_s[1][h][d] + o_s[2][h][d] + o_s[3][h][d];
    float* dst = p.part + (((int64_t)b * p.Hq + h0 + h) * p.nsplit + split) * (DH + 4);
    dst[d] = nk > 0 ? sum : 0.f;
    if (d == 0) {
      dst[DH] = nk > 0 ? mstat[h] : -INFINITY;
      dst[DH + 1] = nk > 0 ? lstat[h] : 0.f;
    }
  }
}

// Stream mode (bf16): one workgroup per (sequence, kv head) walks the whole key list in
// chunks of CK keys per wave (waves take chunks round-robin), optionally double-buffered
// in registers so the next chunk's K and V are in flight while the current one is
// scored and accumulated.  Each wave keeps an online softmax (running max m, sum l and O,
// rescaled when m grows; the max is shared by the wave's lanes so lane groups can be
// summed at the end); the four waves are merged through LDS and O is stored, rounded to
// bf16, straight into its row.  Used when sequences x kv heads fill the chip.
// The arithmetic is packed: q.k is accumulated with v_dot2_f32_bf16 on the stored bf16
// pairs (no unpacking of K), and P V pairs the keys of two consecutive instructions
// (same lane, same head_dim chunk): (p_i, p_j) . (v_i[d], v_j[d]) per d, with P rounded
// to bf16 as the prefill kernel rounds it for its MFMA.
namespace {
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ bf16x2_t as_bf2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf2(a), as_bf2(b), c, false);
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const bf16x2_t v{(bf16)lo, (bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
}  // namespace

template <int DH, int GQ, int NW, int NI, bool DB>
__global__ __launch_bounds__(NW * 64) void attn_decode_stream_kernel(AttnDecodeParams p) {
  constexpr int LPK = DH / 8;      // lanes per key (one 16-byte chunk each)
  constexpr int KPI = 64 / LPK;    // keys per wave instruction
  constexpr int CK = NI * KPI;     // keys per chunk (NI wave instructions, K and V each)
  static_assert(NI % 2 == 0, "instructions are paired for P V");
  __shared__ float red_m[NW][GQ], red_l[NW][GQ];
  __shared__ float red_o[NW][GQ][DH];

  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h0 = g * GQ;
  const int posb = max(p.pos[b], 0);
  const int span = min(posb + 1, p.span_max);
  const int nkeys = p.n_meta + span;
  const int nchunks = (nkeys + CK - 1) / CK;
  const int dc = lane % LPK, kin = lane / LPK;
  const float sl2 = p.scale * 1.4426950408889634f;  // scores in log2 units

  u32x4 q[GQ];
#pragma unroll
  for (int h = 0; h < GQ; ++h)
    q[h] = *(const u32x4*)((const bf16*)p.q + (int64_t)b * p.q_row_stride + (h0 + h) * DH + dc * 8);
  // Key idx < n_meta is meta row idx; key idx >= n_meta is X-position
  // posb - span + 1 + (idx - n_meta) at ring slot (position % slots).  Within a chunk the
  // ring slot advances by KPI per instruction with one wrap (slots >= KPI, checked on the
  // host); keys past the end read ring slot 0 and are masked.
  const int64_t ring_off = ((int64_t)b * p.Hkv + g) * p.slots * DH + dc * 8;
  const int64_t meta_off = (int64_t)g * p.n_meta * DH + dc * 8;
  const bf16* km = (const bf16*)p.k_meta + meta_off;
  const bf16* vm = (const bf16*)p.v_meta + meta_off;
  const bf16* kg = (const bf16*)p.k + ring_off;
  const bf16* vg = (const bf16*)p.v + ring_off;
  const int xpos0 = posb - span + 1 - p.n_meta;  // X-position of key idx = xpos0 + idx
  auto fetch = [&](u32x4 (&kr)[NI], u32x4 (&vr)[NI], int j) {
    const int idx0 = j * CK + kin;
    int slot = (xpos0 + idx0) % p.slots;
    if (slot < 0) slot += p.slots;  // meta keys: slot unused
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int idx = idx0 + i * KPI;
      const bool meta = idx < p.n_meta;
      const int ro = idx < nkeys ? slot * DH : 0;
      kr[i] = *(const u32x4*)(meta ? km + idx * DH : kg + ro);
      vr[i] = *(const u32x4*)(meta ? vm + idx * DH : vg + ro);
      slot += KPI;
      if (slot >= p.slots) slot -= p.slots;
    }
  };

  float m[GQ], l[GQ], o[GQ][8];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }
  auto consume = [&](const u32x4 (&kr)[NI], const u32x4 (&vr)[NI], int j) {
    float sc[NI][GQ];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool valid = j * CK + i * KPI + kin < nkeys;
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        float d = dot2(q[h][0], kr[i][0], 0.f);
        d = dot2(q[h][1], kr[i][1], d);
        d = dot2(q[h][2], kr[i][2], d);
        d = dot2(q[h][3], kr[i][3], d);
        d = lane_group_sum<LPK>(d);
        sc[i][h] = valid ? d * sl2 : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      float cm = sc[0][h];
#pragma unroll
      for (int i = 1; i < NI; ++i) cm = fmaxf(cm, sc[i][h]);
#pragma unroll
      for (int off = LPK; off < 64; off <<= 1) cm = fmaxf(cm, __shfl_xor(cm, off, 64));
      const float mn = fmaxf(m[h], cm);  // finite: every chunk holds a valid key
      const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
      m[h] = mn;
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < NI; i += 2) {
      // (v_i[d], v_{i+1}[d]) pairs: low halves for even d, high halves for odd d
      uint32_t vp[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vp[2 * w] = __builtin_amdgcn_perm(vr[i + 1][w], vr[i][w], 0x05040100u);
        vp[2 * w + 1] = __builtin_amdgcn_perm(vr[i + 1][w], vr[i][w], 0x07060302u);
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const float pa = __builtin_amdgcn_exp2f(sc[i][h] - m[h]);
        const float pb = __builtin_amdgcn_exp2f(sc[i + 1][h] - m[h]);
        l[h] += pa + pb;
        const uint32_t pp = pack_bf2(pa, pb);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = dot2(pp, vp[e], o[h][e]);
      }
    }
  };

  if constexpr (DB) {  // two register buffers: the next chunk loads during this one
    u32x4 k0[NI], v0[NI], k1[NI], v1[NI];
    int j = wave;
    if (j < nchunks) fetch(k0, v0, j);
    for (; j < nchunks; j += 2 * NW) {
      if (j + NW < nchunks) fetch(k1, v1, j + NW);
      consume(k0, v0, j);
      if (j + NW >= nchunks) break;
      if (j + 2 * NW < nchunks) fetch(k0, v0, j + 2 * NW);
      consume(k1, v1, j + NW);
    }
  } else {  // one buffer; the other waves of the SIMD cover the latency
    u32x4 k0[NI], v0[NI];
    for (int j = wave; j < nchunks; j += NW) {
      fetch(k0, v0, j);
      consume(k0, v0, j);
    }
  }

  // lane groups of the wave (same chunk index dc) share m: sum l and O over them
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) l[h] += __shfl_xor(l[h], off, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = o[h][e];
#pragma unroll
      for (int off = LPK; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
      o[h][e] = v;
    }
  }
  if (kin == 0) {
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[wave][h][dc * 8 + e] = o[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      red_m[wave][h] = m[h];
      red_l[wave][h] = l[h];
    }
  }
  __syncthreads();
  for (int i = tid; i < GQ * DH; i += NW * 64) {
    const int h = i / DH, d = i % DH;
    float mx = red_m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) mx = fmaxf(mx, red_m[w][h]);
    float ls = 0.f, os = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = red_m[w][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(red_m[w][h] - mx);
      ls = fmaf(red_l[w][h], wt, ls);
      os = fmaf(red_o[w][h][d], wt, os);
    }
    ((bf16*)p.o)[(int64_t)b * p.o_stride + (h0 + h) * DH + d] = (bf16)(os / ls);
  }
}

template <int DH, int NW, int NI, bool DB>
static hipError_t run_decode_stream(const AttnDecodeParams& p, hipStream_t s) {
  dim3 grid(p.Hkv, p.B);
  switch (p.Hq / p.Hkv) {
    case 1: attn_decode_stream_kernel<DH, 1, NW, NI, DB><<<grid, dim3(NW * 64), 0, s>>>(p); break;
    case 2: attn_decode_stream_kernel<DH, 2, NW, NI, DB><<<grid, dim3(NW * 64), 0, s>>>(p); break;
    case 4: attn_decode_stream_kernel<DH, 4, NW, NI, DB><<<grid, dim3(NW * 64), 0, s>>>(p); break;
    case 8: attn_decode_stream_kernel<DH, 8, NW, NI, DB><<<grid, dim3(NW * 64), 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
// Four waves, 6-instruction chunks, one register buffer (measured fastest on the
// 128-sequence, 4-kv-head, 1152-key case; a second buffer costs more in occupancy than
// it gains in overlap).
template <int DH>
static hipError_t run_decode_stream(const AttnDecodeParams& p, hipStream_t s) {
  return run_decode_stream<DH, 4, 6, false>(p, s);
}

template <typename T, int DH, int KPS>
static hipError_t run_decode_kps(const AttnDecodeParams& p, hipStream_t s) {
  dim3 grid(p.nsplit, p.Hkv, p.B);
  switch (p.Hq / p.Hkv) {
    case 1: attn_decode_kernel<T, DH, 1, KPS><<<grid, dim3(256), 0, s>>>(p); break;
    case 2: attn_decode_kernel<T, DH, 2, KPS><<<grid, dim3(256), 0, s>>>(p); break;
    case 4: attn_decode_kernel<T, DH, 4, KPS><<<grid, dim3(256), 0, s>>>(p); break;
    case 8: attn_decode_kernel<T, DH, 8, KPS><<<grid, dim3(256), 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int DH>
static hipError_t run_decode(const AttnDecodeParams& p, hipStream_t s) {
  if (p.o != nullptr) {
    if constexpr (std::is_same_v<T, bf16>) return run_decode_stream<DH>(p, s);
    return hipErrorInvalidValue;  // stream mode is bf16 only
  }
  switch (p.keys_per_split) {
    case 64: return run_decode_kps<T, DH, 64>(p, s);
    case 128: return run_decode_kps<T, DH, 128>(p, s);
    case 192: return run_decode_kps<T, DH, 192>(p, s);
    case 256: return run_decode_kps<T, DH, 256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention_decode(bool bf16_, const AttnDecodeParams& p, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  if (bf16_) {
    if (p.head_dim == 128) return run_decode<bf16, 128>(p, s);
    if (p.head_dim == 64) return run_decode<bf16, 64>(p, s);
  } else {
    if (p.head_dim == 64) return run_decode<float, 64>(p, s);
    if (p.head_dim == 32) return run_decode<float, 32>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace hymba
