// Host-side launchers of the gfx950 kernels (internal to libhymba).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hymba {

// ----------------------------------------------------------------- GEMM
// C[M, N] = A[M, K] * B[N, K]^T.  A's rows come from two sources: rows < a_split
// from a0 (stride lda0), the rest from a1 (stride lda1).  Element type of A and B is
// `bf16` (MFMA) or fp32 (VALU), per the launcher.
struct GemmOperands {
  const void* a0;
  int64_t lda0;
  const void* a1;
  int64_t lda1;
  int a_split;
  const void* b;
  int64_t ldb;
  int M, N, K;
};

enum class EpiKind { Store, StoreF32, XProj, Softplus, Silu, AddStore };

// Output description for the epilogues.
//  Store:    rows < c_split -> c0 (stride ldc0, skipped if c0 == nullptr), others ->
//            c1 (stride ldc1); storage type = the input type.
//  StoreF32: fp32 rows into c0 (stride ldc0).
//  XProj:    columns < split_col -> c0 (storage type, stride ldc0), columns >= split_col
//            -> c1 fp32 (stride ldc1, column - split_col).
//  Softplus: fp32 c0[m, n] = softplus(acc + bias[n]).
//  Silu:     as Store, of SiLU(acc).
//  AddStore: as Store, of the destination's value plus acc (c += A B^T, in place).
struct GemmOutput {
  EpiKind kind;
  void* c0;
  int64_t ldc0;
  void* c1;
  int64_t ldc1;
  int c_split;
  int split_col;
  const float* bias;
};

enum class GemmShape { Large, Narrow, Skinny };

// Row scaling of a product whose K range splits in two segments (the attention and SSM
// halves of F): out[m, n] = fac[2m] * sum_{k < k_split} A B^T + fac[2m+1] * sum_{k >= k_split}.
struct RowScale {
  const float* fac;
  int k_split;
};

hipError_t launch_gemm_bf16(const GemmOperands& op, const GemmOutput& out, GemmShape shape,
                            hipStream_t s);
hipError_t launch_gemm_f32(const GemmOperands& op, const GemmOutput& out, hipStream_t s);
// x_proj (XProj epilogue, bf16): every output column of up to 96 rows per workgroup, Xs
// streamed once through a deep LDS ring.  gemm_xproj_ok tells whether the operands fit
// (single-source A, K % 64 == 0, 32 < N <= 384, 16-byte aligned rows).
bool gemm_xproj_ok(const GemmOperands& op, const GemmOutput& out);
hipError_t launch_gemm_xproj_bf16(const GemmOperands& op, const GemmOutput& out, hipStream_t s);
// Few-row (decode) GEMMs, K % 256 == 0, single-source A.
// K split into up to `ksplit` slices that run as separate workgroups (splitk_slices
// gives the count).  slice_stride == 0: acc[M, N] (fp32, row stride ldacc) += A B^T
// through atomics.  slice_stride > 0: slice p stores its partial product at
// acc + p * slice_stride (stride >= M * ldacc); nothing is accumulated.
int splitk_slices(int K, int ksplit);
hipError_t launch_gemm_bf16_splitk(const GemmOperands& op, float* acc, int64_t ldacc, int ksplit,
                                   hipStream_t s, int64_t slice_stride = 0);
// bf16 C = row-scaled A B^T (see RowScale) with the plain store epilogue; K and k_split
// multiples of 128, 0 < k_split < K.  Returns hipErrorInvalidValue when the operands do
// not suit the 256-wide tile kernel (check with gemm_bf16_rowscaled_ok first).
bool gemm_bf16_rowscaled_ok(const GemmOperands& op, int k_split);
hipError_t launch_gemm_bf16_rowscaled(const GemmOperands& op, const GemmOutput& out,
                                      const RowScale& rs, hipStream_t s);
// Z = bf16(A B^T) (row stride ldz); with k_col >= 0 the K / V columns of row b are also
// written to ring slot pos[b] % slots of ring_k / ring_v ([B, Hkv, slots, head_dim]).
// Also clears `zero_n` floats at `zero` (16-byte aligned, zero_n % 4 == 0): the split-K
// accumulators the later decode projections add into.
hipError_t launch_gemm_bf16_decode_in(const GemmOperands& op, void* z, int64_t ldz, int k_col,
                                      int v_col, void* ring_k, void* ring_v, int slots, int Hkv,
                                      int head_dim, const int32_t* pos, float* zero,
                                      int64_t zero_n, hipStream_t s);

// Few-row streaming products (gemv_bf16_kernel): y[m, n] = sum_k x[m, k] w[n, k] for
// M <= kGemvMaxRows rows of x (row stride ldx) and N rows of w (row stride ldw), fp32 sums;
// y bf16 or fp32 (row stride ldy).  With k_col >= 0 (bf16 y) the K / V columns of row m are
// also written to ring slot pos[m] % slots of ring_k / ring_v ([M, Hkv, slots, head_dim]).
constexpr int kGemvMaxRows = 4;
struct GemvOut {
  void* y;
  int64_t ldy;
  bool f32;
  int k_col = -1, v_col = -1, kvw = 0, head_dim = 0, Hkv = 0, slots = 0;
  void* ring_k = nullptr;  // bf16
  void* ring_v = nullptr;
  const int32_t* pos = nullptr;
};
bool gemv_bf16_ok(int M, int K, int64_t ldx, int64_t ldw);
hipError_t launch_gemv_bf16(const void* x, int64_t ldx, const void* w, int64_t ldw, int M, int N,
                            int K, const GemvOut& out, hipStream_t s);

// ----------------------------------------------------------------- attention
// Keys/values at X~ position j of sequence b: j < n_meta from the meta arrays
// (meta + g*meta_head_stride + j*meta_row_stride), otherwise from the sequence
// arrays (seq + b*seq_batch_stride + g*seq_head_stride + ((j - n_meta) % seq_slots) *
// seq_row_stride).  Queries and outputs: row r of q / o; the first meta_rows rows are
// the meta queries (meta_rows = n_meta, or 0 when the meta rows are cached and not
// recomputed), then sequence b = (r - meta_rows) / L at X-position
// n_meta + (r - meta_rows) % L.
struct AttnParams {
  const void* q;
  int64_t q_row_stride;
  const void* k_meta;
  const void* v_meta;
  int64_t meta_head_stride, meta_row_stride;
  const void* k_seq;
  const void* v_seq;
  int64_t seq_batch_stride, seq_head_stride, seq_row_stride;
  int seq_slots;
  void* o;
  int64_t o_row_stride;
  int n_meta, L, B, Hq, Hkv, head_dim, window;
  float scale;
  int meta_rows;
  // bf16 prefill only: with ssp != nullptr the kernel writes beta[h*head_dim + d] * O
  // and the row's sum of O^2 over head h to ssp[h * ssp_ld + row] (row as for q).
  float* ssp;
  int64_t ssp_ld;
  const float* beta;
};
hipError_t launch_attention_prefill_f32(const AttnParams& p, hipStream_t s);
// bf16 prefill with direct-to-LDS K / V^T tiles; `vt` is scratch of
// attention_vt_bytes(...) bytes (16-byte aligned) that receives V^T first.
size_t attention_vt_bytes(int n_meta, int L, int B, int Hkv, int head_dim);
hipError_t launch_attention_prefill_bf16_dl(const AttnParams& p, void* vt, hipStream_t s);

// Decode: one query per sequence at X-position pos[b]; keys = meta + the
// min(pos+1, span_max) most recent ring positions.  Partial results per split go to
// part (fp32): [B, Hq, nsplit, head_dim + 4] holding (o[head_dim], m, l, 2 pad) so every
// split record starts 16-byte aligned.
struct AttnDecodeParams {
  const void* q;  // row b at q + b*q_row_stride (+ h*head_dim)
  int64_t q_row_stride;
  const void* k_meta;
  const void* v_meta;  // [Hkv, M, dh]
  const void* k;
  const void* v;  // [B, Hkv, S, dh]
  int slots;
  const int32_t* pos;
  float* part;     // split mode: partials (see above)
  int nsplit, keys_per_split;
  void* o;         // stream mode (o != nullptr): O rows at o + b*o_stride, storage type
  int64_t o_stride;
  int n_meta, B, Hq, Hkv, head_dim, span_max;
  float scale;
};
hipError_t launch_attention_decode(bool bf16, const AttnDecodeParams& p, hipStream_t s);

// ----------------------------------------------------------------- scan
struct ScanParams {
  const void* z;       // in_proj output, rows as for attention queries
  int64_t z_stride;
  int xs_col, g_col;   // column offsets of Xs and G in z
  const float* dt;     // [rows, Di]
  const float* bc;     // [rows, 2N] (B then C)
  const float* A;      // [Di, N]
  const float* D;      // [Di]
  void* y;             // gated output, row stride y_stride (storage type)
  int64_t y_stride;
  float* h_out;        // [B, Di, N] or nullptr
  const float* h0;     // [Di, N] initial state of every sequence, or nullptr (zero)
  int n_meta, L, B, Di, N;
};
hipError_t launch_scan_prefill(bool bf16, const ScanParams& p, hipStream_t s);

// bf16 prefill SSM heads with the dt projection inside (dt = softplus(delta W_dt^T + b),
// delta [rows, R] bf16, W_dt [Di, R] bf16), chunk-carried over time.  Sequence b's token
// t is row row0 + b * T + t of z, delta, bc, y (and ssp).  The T tokens are cut into
// nchunks = scan_chunk_count(T, chunk) chunks of `chunk` tokens (a multiple of 16, at most
// 65 chunks); with more than one, hsum [B, nchunks - 1, Di, N] and ssum [B, nchunks - 1,
// Di] (fp32) receive the chunk summaries and carries.  h0 [Di, N] is every sequence's
// state before token 0 (zero when null); h_out [B, Di, N] the state after token T - 1.
// ssp / ssp_col0 / beta as for ScanParams (scan_channel_blocks() blocks of 64 channels).
struct ScanChunkParams {
  const void* z;
  int64_t z_stride;
  int xs_col, g_col;
  const void* delta;
  const float* bc;       // [rows, 2N] (B then C)
  const void* w_dt;
  const float* dt_bias;  // [Di]
  const float* A;        // [Di, N]
  const float* D;        // [Di]
  void* y;
  int64_t y_stride;
  const float* h0;
  float* h_out;
  int row0, T, B, Di, N, R;
  int chunk, nchunks;
  float* hsum;
  float* ssum;
  float* ssp;
  int64_t ssp_ld;
  int ssp_col0;
  const float* beta;
  int32_t* pos_out;  // when set: pos_out[b] = pos_val, written by the main pass
  int pos_val;
};
bool scan_chunk_supported(int N, int R, int Di);
int scan_channel_blocks(int N, int Di);
int scan_chunk_count(int T, int chunk);
// Chunk length for B sequences of T tokens: one chunk when the batch gives every CU two
// workgroups, otherwise about 2048 (sequence, chunk) workgroups of at least 512 tokens
// (sequences shorter than 1024 tokens: up to 8 chunks of at least 16).
int scan_default_chunk(int B, int Di, int T);
hipError_t launch_scan_chunk(const ScanChunkParams& p, hipStream_t s);

// Mamba-2 SSM head (heads of 64 channels, one dt and one A per head, B and C shared),
// bf16 prefill in the chunked matrix form.  xbc [rows, H + 2N] fp32 holds u | B | C per
// row (dt = softplus(u + dt_bias[h])); rows as for ScanParams (the meta prefix then the
// sequence's own rows); y is the gated output; h0 / h_out as for ScanParams.
struct SsdParams {
  const void* z;
  int64_t z_stride;
  int xs_col, g_col;
  const float* xbc;
  int64_t xbc_ld;
  const float* dt_bias;  // [H]
  const float* A;        // [H]
  const float* D;        // [Di]
  const float* h0;       // [Di, N] or nullptr
  void* y;
  int64_t y_stride;
  float* h_out;          // [B, Di, N] or nullptr
  int n_meta, L, B, H, N;
};
bool scan_ssd_supported(int N, int Di, int H);
hipError_t launch_scan_ssd(const SsdParams& p, hipStream_t s);

// Decode: one step per sequence, h updated in place, pos[b] += 1 when pos != nullptr.
// dt is computed in place from the x_proj output: dt = softplus(delta W_dt^T + b) with
// delta = xdbl[b, :R] (rounded to bf16 first when round_delta), B = xdbl[b, R:R+N],
// C = xdbl[b, R+N:R+2N].
struct SsmStepParams {
  const void* z;
  int64_t z_stride;
  int xs_col, g_col;
  const float* xdbl;    // [B, R + 2N] fp32
  const void* w_dt;     // [Di, R] storage type
  const float* dt_bias; // [Di]
  const float* A;
  const float* D;
  float* h;             // [B, Di, N]
  void* y;              // row b at y + b*y_stride
  int64_t y_stride;
  int32_t* pos;
  int B, Di, N, R;
  int heads;            // > 0: Mamba-2 head; xdbl rows are [u (heads) | B | C], no w_dt
};
hipError_t launch_ssm_step(bool bf16, const SsmStepParams& p, hipStream_t s);
hipError_t launch_ssm2_step(const SsmStepParams& p, hipStream_t s);  // bf16, heads > 0

// ----------------------------------------------------------------- fusion
// F[r, :] = 0.5 * [beta_a * rms(F[r, :wa]) ; beta_s * rms(F[r, wa:wa+ws])], in place.
// Group-normalisation variant of launch_fuse_norm: each branch in groups of g channels
// (power of two, 8..512, dividing wa and ws), (v - mean) / sqrt(var + eps) per group,
// then 0.5 * beta.
hipError_t launch_group_norm(bool bf16, void* f, int64_t f_stride, int rows, int wa, int ws,
                             const float* beta_a, const float* beta_s, float eps, int g,
                             hipStream_t s);
// Block wrapper.  out[r, :] = rms(in[r, :]) * g (storage type, d % 8 == 0).
hipError_t launch_rms_norm_rows(bool bf16, const void* in, int64_t in_ld, void* out,
                                int64_t out_ld, int rows, int d, const float* g, float eps,
                                hipStream_t s);
// u = x + y written over y (rounded to the storage type), then v = rms(u) * g.
hipError_t launch_residual_norm(bool bf16, const void* x, int64_t x_ld, void* y, int64_t y_ld,
                                void* v, int64_t v_ld, int rows, int d, const float* g,
                                float eps, hipStream_t s);
// Decode: merge the split-key attention partials into F's attention columns (no norm).
hipError_t launch_decode_combine(bool bf16, const float* part, int nsplit, void* f,
                                 int64_t f_stride, int B, int Hq, int head_dim, hipStream_t s);
hipError_t launch_fuse_norm(bool bf16, void* f, int64_t f_stride, int rows, int wa, int ws,
                            const float* beta_a, const float* beta_s, float eps,
                            hipStream_t s);
// Row factors of the deferred branch norms: for every row, fa = 0.5 / sqrt(sum of the
// na partials ssp[0:na, row] / wa + eps) and fs likewise over ssp[na:na+ns, row] / ws
// (partial i of row r at ssp[i * ssp_ld + r]); fac[2*row] = fa, fac[2*row+1] = fs.
// Rows < scale_rows of f (storage bf16, row stride f_stride) are scaled in place:
// columns < wa by fa, the rest by fs.
hipError_t launch_row_factors(const float* ssp, int64_t ssp_ld, int na, int ns, int rows,
                              int wa, int ws, float eps, float* fac, void* f, int64_t f_stride,
                              int scale_rows, hipStream_t s);
// Decode: merge the split-attention partials into O (rounded to the storage type),
// write it to F[b, :wa], then normalise F[b] as above.
hipError_t launch_decode_combine_norm(bool bf16, const float* part, int nsplit, void* f,
                                      int64_t f_stride, int B, int Hq, int head_dim, int ws,
                                      const float* beta_a, const float* beta_s, float eps,
                                      hipStream_t s);

// ----------------------------------------------------------------- cache / misc
// Prefill: copy K/V columns of z into the cache (meta rows -> k_meta/v_meta, the last
// min(L, slots) positions of every sequence -> ring slot p % slots).
hipError_t launch_kv_write_prefill(bool bf16, const void* z, int64_t z_stride, int k_col,
                                   int v_col, void* k_meta, void* v_meta, void* k, void* v,
                                   int slots, int n_meta, int L, int B, int Hkv,
                                   int head_dim, hipStream_t s);
// Copy the last n_last positions p of every sequence from src (slot p % src_slots) to
// dst (slot p % dst_slots), and the n_meta meta entries when copy_meta.
hipError_t launch_kv_ring_fill(bool bf16, const void* src_k, const void* src_v, int src_slots,
                               const void* src_k_meta, const void* src_v_meta, void* dst_k,
                               void* dst_v, int dst_slots, void* dst_k_meta, void* dst_v_meta,
                               bool copy_meta, int n_meta, int L, int n_last, int B, int Hkv,
                               int head_dim, hipStream_t s);
// Decode: write row b's K/V at slot pos[b] % slots.
hipError_t launch_kv_write_decode(bool bf16, const void* z, int64_t z_stride, int k_col,
                                  int v_col, void* k, void* v, int slots,
                                  const int32_t* pos, int B, int Hkv, int head_dim,
                                  hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t value, int n, hipStream_t s);
// Zero `n` floats (n % 4 == 0, 16-byte aligned).
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s);
// y[B, d] (storage type, contiguous) = sum over p < nslices of acc[p * slice_stride +
// (B, d)] fp32, plus y's old value when `accumulate`, then SiLU when `silu` (one rounding
// of the fp32 result); slice_stride % 4 == 0 when nslices > 1.
hipError_t launch_store_rows(bool bf16, const float* acc, void* y, int B, int d, hipStream_t s,
                             int nslices = 1, int64_t slice_stride = 0, bool accumulate = false,
                             bool silu = false);
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
// Ceiling probes (probe.hip): kind 0 exponential rate, 1 bf16 MFMA rate, 2 streaming read.
size_t probe_operand_bytes();
hipError_t launch_probe(int kind, int blocks, int iters, const void* src, size_t bytes, float* out,
                        hipStream_t s);

}  // namespace hymba
