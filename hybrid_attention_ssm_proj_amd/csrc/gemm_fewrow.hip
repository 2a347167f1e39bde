// Few-row projection GEMMs: the decode projections (in_proj with the producer's ring
// write, x_proj, out_proj) over a decode batch, and the meta rows of prefill.  Source:
// the in_proj / out_proj terms of the design formulation in "Hymba: A Hybrid-head
// Architecture for Small Language Models" (outta.ai summary); the decode step's cache
// update from its Introduction (KV cache plus recurrent state).
//
// gemm_bf16_fewrow_kernel: 128- (or 64-) row MFMA tiles over one K slice, weights
// streamed through LDS by DMA, with store, split-K atomic and split-K partial epilogues.
// gemv_bf16_kernel: one to four rows, weights streamed straight into registers.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "gemm_tile.h"
#include "kernels.h"

namespace hymba {

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

}  // namespace hymba
