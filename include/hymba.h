/*
 * hymba.h -- C ABI of libhymba: the forward pass of the Hymba fused hybrid-head
 * layer on one AMD Instinct MI355X (gfx950), for prefill and single-token decode.
 *
 * The layer (source: "Hymba: A Hybrid-head Architecture for Small Language Models",
 * reader's summary on blog.outta.ai, section "A Fused Hybrid Head Module / Design
 * formulation"):
 *   X~ = [meta; X]                 meta tokens prefixed to every sequence
 *   Z  = X~ W_in^T  split by columns into [Q | K | V | Xs | G]
 *   attention heads:  O = softmax(s Q K^T + mask) V    (GQA, causal, optional
 *                     sliding window; meta keys always visible)
 *   SSM heads (Mamba selective scan, diagonal A):
 *       [delta | B | C] = Xs W_x^T,  dt = softplus(delta W_dt^T + dt_bias)
 *       h_t = exp(dt_t * A) * h_{t-1} + (dt_t * x_t) B_t,   y_t = h_t C_t + D * x_t
 *       Y_ssm = y * SiLU(G)
 *   fusion:  F = 0.5 [beta_attn * rms(O) ; beta_ssm * rms(Y_ssm)]    (total fusion
 *            equation, with the averaging of the Chinese summary "Hymba ... hybrid
 *            attention-SSM heads", sections 核心架构 and 实现细节)
 *   Y = F W_out^T;  y = rows of X, y_meta = rows of the meta tokens.
 * Readings where the pages are silent: softmax scale 1/sqrt(head_dim), no positional
 * encoding, a window of W keys counts the query itself, q head h uses kv head
 * floor(h * Hkv / Hq), RMSNorm over each branch's full width, h = 0 before the first
 * meta token, only dt_proj has a bias.
 *
 * Conventions for every entry point
 *  - All pointers are DEVICE pointers unless stated otherwise; descriptor and
 *    weight-table structs themselves live in host memory and are read during the
 *    call only.
 *  - The caller owns every buffer.  The library allocates no device memory on these
 *    paths and keeps no per-call state.
 *  - Every call is asynchronous and ordered on `stream` (a hipStream_t; NULL is the
 *    default stream).  No host synchronisation happens inside.
 *  - Arguments are validated on the host before anything is launched: an error
 *    return means nothing was enqueued and no output was touched.  No exception or
 *    abort crosses the ABI.
 *  - Row-major layouts; weights use the [out, in] convention.
 *  - Device pointers must be 16-byte aligned (HYMBA_ERR_ALIGNMENT otherwise).
 *
 * Precision contract (dtype HYMBA_DTYPE_BF16): weights, meta, X, Z, delta, O, Y_ssm,
 * F, y, y_meta and the K/V cache are bf16 (round to nearest even where produced);
 * dt, B, C, A, D, beta, the SSM state h and all accumulation and softmax arithmetic
 * are fp32.  dtype HYMBA_DTYPE_F32: fp32 storage and arithmetic throughout.
 */
#ifndef HYMBA_H
#define HYMBA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HYMBA_ABI_VERSION 3

typedef enum {
  HYMBA_DTYPE_F32 = 0,
  HYMBA_DTYPE_BF16 = 1
} hymba_dtype;

typedef enum {
  HYMBA_OK = 0,
  HYMBA_ERR_INVALID_ARG = 1,   /* null pointer, negative or inconsistent size        */
  HYMBA_ERR_UNSUPPORTED = 2,   /* valid shape with no kernel (e.g. head_dim, d_state) */
  HYMBA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required          */
  HYMBA_ERR_ALIGNMENT = 4,     /* a device pointer is not 16-byte aligned             */
  HYMBA_ERR_HIP = 5            /* a HIP launch failed; see hymba_last_hip_error()     */
} hymba_status;

/* Layer shape.  Supported: head_dim 64 or 128 (bf16) / 32 or 64 (fp32); d_state a power
 * of two from 4 to 128; n_q_heads / n_kv_heads in {1, 2, 4, 8}; d_model, d_inner,
 * dt_rank and head_dim multiples of 8; dt_rank <= 512.
 *
 * SSM head type.  ssm_heads = 0: the Mamba head of the Hymba summary's design
 * formulation (per-channel A [Di, N], dt = softplus(delta W_dt^T + b) with delta of rank
 * dt_rank).  ssm_heads = H > 0: the Mamba-2 head of the Chinese summary's implementation
 * pseudocode ("实现细节"), read as one group: H heads of P = Di / H channels, one
 * dt = softplus(u + b[h]) and one A[h] per head, B and C shared, D per channel; x_proj
 * gives [u | B | C] (H + 2N rows of w_x), there is no w_dt and dt_rank is ignored.
 * Supported for bf16 with P = 64, H a multiple of 4 and d_state in {16, 32, 64, 128}.
 *
 * Branch normalisation.  norm_group = 0: each branch is RMS-normalised over its full
 * width (the Chinese summary's RMSNorm per branch).  norm_group = g > 0: group
 * normalisation, the variant the hybrid-architecture summary ("설계 통찰 / 아키텍처 변형")
 * recommends for intra-layer hybrids, in groups of g channels; beta and the 0.5
 * average apply as before.
 *
 * Time chunks of the Mamba-head scan (bf16, dt_rank 64 or 128, d_inner a multiple of
 * 64).  The recurrence is linear in h, so a span of tokens maps h_in to P * h_in + h_loc
 * with P = exp(A * sum dt); the prefill cuts each sequence into chunks of scan_chunk
 * tokens, summarises every chunk but the last from h = 0, carries the summaries across
 * chunks and rescans each chunk from its carried state (the same result up to rounding
 * order).  scan_chunk = 0 lets the library choose (one chunk when the batch fills the
 * GPU); otherwise a multiple of 16 giving at most 65 chunks per sequence. */
typedef struct {
  int32_t d_model;      /* d                                                      */
  int32_t n_q_heads;    /* Hq                                                     */
  int32_t n_kv_heads;   /* Hkv (divides Hq)                                       */
  int32_t head_dim;     /* dh                                                     */
  int32_t d_inner;      /* Di: SSM channels                                       */
  int32_t d_state;      /* N: SSM states per channel                              */
  int32_t dt_rank;      /* R: rank of the dt projection                           */
  int32_t n_meta;       /* M: meta tokens (>= 0)                                  */
  int32_t window;       /* 0 = full causal; > 0: a non-meta key is visible if it is
                           fewer than `window` positions back (the query counts)  */
  int32_t kv_share;     /* 0 = producer (own K/V columns in w_in);
                           1 = consumer (no K/V columns; reads the producer's)    */
  int32_t dtype;        /* hymba_dtype                                            */
  float rms_eps;        /* RMSNorm epsilon, e.g. 1e-6                             */
  float softmax_scale;  /* 0 => 1/sqrt(head_dim)                                  */
  int32_t ssm_heads;    /* 0 = Mamba head; H > 0 = Mamba-2 head with H heads      */
  int32_t norm_group;   /* 0 = RMSNorm over each branch; g > 0 = group norm in
                           groups of g channels (a power of two, 8..512, dividing
                           Hq*dh and Di): (v - mean) / sqrt(var + eps) per group   */
  int32_t scan_chunk;   /* tokens per time chunk of the scan (0 = chosen per call)  */
} hymba_layer_desc;

/* Weights (device).  n_in = Hq*dh + (kv_share ? 0 : 2*Hkv*dh) + 2*Di; column
 * blocks of w_in's output in that order: Q, K, V, Xs, G. */
typedef struct {
  const void *w_in;       /* [n_in, d]            dtype                          */
  const void *w_x;        /* [R + 2N, Di]         dtype  (rows: delta, B, C)
                             Mamba-2 heads: [H + 2N, Di] (rows: u, B, C)        */
  const void *w_dt;       /* [Di, R]              dtype  (Mamba-2 heads: NULL)   */
  const void *w_out;      /* [d, Hq*dh + Di]      dtype                          */
  const float *dt_bias;   /* [Di]                        (Mamba-2 heads: [H])    */
  const float *A;         /* [Di, N]                     (Mamba-2 heads: [H])    */
  const float *D;         /* [Di]                                                */
  const float *beta_attn; /* [Hq*dh]                                             */
  const float *beta_ssm;  /* [Di]                                                */
} hymba_layer_weights;

/* Attention cache (device, dtype).  X-position p of sequence b lives at slot
 * p % slots of k/v; the M meta entries are batch-shared.  is_ring = 1: a ring holding the
 * last `slots` positions (the sliding-window decode cache); is_ring = 0: every position
 * has its own slot, so the cache must cover every position a call writes or reads
 * (a prefill's kv_out needs slots >= L; a decode needs pos[b] < slots, which the caller
 * guarantees).  A consumer's kv_in always needs every position (slots >= L). */
typedef struct {
  void *k_meta;    /* [Hkv, M, dh]            */
  void *v_meta;    /* [Hkv, M, dh]            */
  void *k;         /* [B, Hkv, slots, dh]     */
  void *v;         /* [B, Hkv, slots, dh]     */
  int32_t slots;   /* capacity S (> 0)        */
  int32_t is_ring; /* 1: slot = p % slots     */
} hymba_kv;

/* SSM recurrent state (device). */
typedef struct {
  float *h;       /* [B, Di, N] fp32                                   */
  int32_t *pos;   /* [B] number of X tokens already consumed per sequence */
} hymba_ssm_state;

/* ---------------------------------------------------------------------------
 * hymba_layer_prefill: the layer over [meta; X_b] for every sequence b.
 *   meta      [M, d] dtype (batch-shared; its rows are computed once per call)
 *   x         [B, L, d] dtype
 *   kv_in     consumer only (kv_share = 1): the producer's cache holding all L
 *             positions (slots >= L) and its meta entries; must be NULL otherwise.
 *   kv_out    producer only, may be NULL: receives the meta K/V and the last
 *             min(L, slots) positions of every sequence.
 *   state_out may be NULL: receives h after the last token and pos[b] = L.
 *   y         [B, L, d] dtype;   y_meta [M, d] dtype or NULL.
 *   workspace device scratch of at least hymba_layer_workspace_bytes(desc, B, L, 0).
 * Source: Design formulation (meta prefix, in_proj split, both heads, fusion);
 * "Cross-layer KV sharing" (consumer reads the producer's K/V); "Combine global and
 * local attention" (window).
 * ------------------------------------------------------------------------- */
hymba_status hymba_layer_prefill(const hymba_layer_desc *desc, const hymba_layer_weights *w,
                                 const void *meta, const void *x, int32_t batch,
                                 int32_t seq_len, const hymba_kv *kv_in, hymba_kv *kv_out,
                                 hymba_ssm_state *state_out, void *y, void *y_meta,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * hymba_layer_decode: one new token per sequence at X-position pos[b].
 *   x    [B, d] dtype;  y [B, d] dtype.
 *   kv   producer: writes K/V of the new token at slot pos[b] % slots, then attends;
 *        consumer: reads the producer's cache (enqueue the producer's decode first).
 *        Attention covers the M meta entries and the min(pos[b]+1, W) most recent
 *        positions, W = window (window > 0; requires slots >= window) or
 *        W = slots (window = 0: equals full causal attention while pos[b] < slots).
 *   state h is advanced one step in place; pos[b] += 1.
 * Source: summary sections "Introduction" (attention keeps a KV cache, the SSM a
 * recurrent state) and "Meta Tokens" (meta entries are a fixed cache prefix).
 * ------------------------------------------------------------------------- */
hymba_status hymba_layer_decode(const hymba_layer_desc *desc, const hymba_layer_weights *w,
                                const void *x, int32_t batch, hymba_kv *kv,
                                hymba_ssm_state *state, void *y, void *workspace,
                                size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * hymba_kv_ring_fill: copies the last min(L, dst->slots) positions of every sequence
 * from src (slot p % src->slots) into dst (slot p % dst->slots), and src's M meta entries
 * into dst's when the two meta arrays differ.  For a KV-sharing pair whose prefill runs
 * on a full-length cache (the consumer reads every position) while decode keeps a
 * window-sized ring ("Cross-layer KV sharing"; "Combine global and local attention").
 * src must hold those positions: src->slots >= L, or src->is_ring with src->slots >=
 * min(L, dst->slots).  dtype, n_kv_heads, head_dim and n_meta describe both caches.
 * Ordered on `stream` after the prefill that wrote src.
 * ------------------------------------------------------------------------- */
hymba_status hymba_kv_ring_fill(const hymba_kv *src, hymba_kv *dst, int32_t batch,
                                int32_t seq_len, int32_t n_meta, int32_t n_kv_heads,
                                int32_t head_dim, int32_t dtype, void *stream);

/* ---------------------------------------------------------------------------
 * hymba_layer_decode_static: hymba_layer_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as hymba_layer_decode, without the workspace:
 * the library uses a fixed scratch array of HYMBA_STATIC_SCRATCH_BYTES in device memory
 * instead (one per device, resident from the library's first use on that device until
 * the process ends; its address is looked up once per device, with that device current).
 * The call allocates nothing and frees nothing.
 *   Returns HYMBA_ERR_WORKSPACE when the decode workspace for this batch and ring
 *   (hymba_layer_workspace_bytes(desc, batch, kv->slots, 1)) exceeds the array.
 *   Every call on a device shares that device's array and leaves its contents behind;
 *   nothing is assumed about them on entry (the split-K accumulators are cleared by the
 *   call's own first kernel).  Calls that overlap on one device (other streams, other host
 *   threads) race on the array: order them on one stream.
 * ------------------------------------------------------------------------- */
#define HYMBA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
hymba_status hymba_layer_decode_static(const hymba_layer_desc *desc,
                                       const hymba_layer_weights *w, const void *x,
                                       int32_t batch, hymba_kv *kv, hymba_ssm_state *state,
                                       void *y, void *stream);

/* ---------------------------------------------------------------------------
 * Meta-prefix cache: what a layer computes over its M meta tokens alone.  The meta
 * tokens are fixed at inference and act as a learned initialisation of the KV cache and
 * of the SSM state ("Meta Tokens"), so these values do not depend on X and can be built
 * once per weight set:
 *   k_meta, v_meta  [Hkv, M, dh] dtype: the meta keys and values (producer layers;
 *                   NULL for a consumer, whose meta keys are its producer's);
 *   h               [Di, N] fp32: the SSM state after the meta tokens;
 *   y_meta          [M, d] dtype: the layer's output rows of the meta tokens (NULL:
 *                   not produced).
 * Owned by the caller (device memory).
 * ------------------------------------------------------------------------- */
typedef struct {
  void *k_meta;
  void *v_meta;
  float *h;
  void *y_meta;
} hymba_meta_cache;

/* hymba_layer_meta_cache_build: fills *cache from meta [M, d] (dtype).  A consumer
 * (kv_share = 1) passes its producer's cache in kv_in (only k_meta / v_meta are read);
 * a producer passes kv_in = NULL.  workspace: hymba_layer_workspace_bytes(desc, 0, 0, 0).
 * Source: "Meta Tokens" (learned cache initialisation); Design formulation. */
hymba_status hymba_layer_meta_cache_build(const hymba_layer_desc *desc,
                                          const hymba_layer_weights *w, const void *meta,
                                          const hymba_kv *kv_in, hymba_meta_cache *cache,
                                          void *workspace, size_t workspace_bytes,
                                          void *stream);

/* hymba_layer_prefill_cached: hymba_layer_prefill over X with the meta rows taken from
 * a built cache instead of being recomputed: attention reads the meta K/V from the cache
 * (a consumer: from kv_in as usual), every sequence's scan starts from cache->h, and no
 * y_meta is produced.  kv_out (producer, may be NULL) receives only the sequence
 * positions; a later decode reads the meta K/V through kv->k_meta = cache->k_meta.
 * workspace: hymba_layer_workspace_bytes(desc, B, L, 2).  Results equal those of
 * hymba_layer_prefill on the same meta tokens. */
hymba_status hymba_layer_prefill_cached(const hymba_layer_desc *desc,
                                        const hymba_layer_weights *w,
                                        const hymba_meta_cache *cache, const void *x,
                                        int32_t batch, int32_t seq_len, const hymba_kv *kv_in,
                                        hymba_kv *kv_out, hymba_ssm_state *state_out, void *y,
                                        void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes for mode 0 (prefill of batch x seq_len), 1 (decode of batch; seq_len
 * carries the ring capacity) or 2 (prefill_cached of batch x seq_len).
 * Returns 0 if the descriptor or sizes are invalid. */
size_t hymba_layer_workspace_bytes(const hymba_layer_desc *desc, int32_t batch,
                                   int32_t seq_len, int32_t mode);

/* ---------------------------------------------------------------------------
 * Block wrapper: the layer inside a pre-norm residual block with an FFN.  The Chinese
 * summary's implementation details ("实现细节") print the layer's configuration with an
 * FFN intermediate size and nothing else of the block; reading, over every row of
 * [meta; X]:
 *     u   = x + Layer(rms(x) * norm1)
 *     out = u + W_down SiLU(W_up (rms(u) * norm2))
 * with rms the RMSNorm of the descriptor's rms_eps, W_up [I, d], W_down [d, I] in the
 * layer's dtype (I = intermediate, a multiple of 8) and norm1, norm2 [d] fp32.  The
 * layer's meta input is rms(meta) * norm1; its y_meta feeds the meta rows' residual.
 * Host structs, device pointers, 16-byte aligned. */
typedef struct {
  const float *norm1;   /* [d]    */
  const float *norm2;   /* [d]    */
  const void *w_up;     /* [I, d] */
  const void *w_down;   /* [d, I] */
  int32_t intermediate; /* I      */
} hymba_block_weights;

/* Workspace of the block calls: mode 0 = hymba_block_prefill for (batch, seq_len),
 * mode 1 = hymba_block_decode for batch sequences with a ring of seq_len slots.  0 on
 * an invalid descriptor or intermediate size. */
size_t hymba_block_workspace_bytes(const hymba_layer_desc *desc, int32_t intermediate,
                                   int32_t batch, int32_t seq_len, int32_t mode);

/* The block over [meta; X_b] for every sequence b: arguments as hymba_layer_prefill
 * (kv_in, kv_out, state_out are the layer's), plus bw.  y [B, L, d] receives the block
 * output; y_meta [M, d] (may be NULL: the meta rows' block outputs are then skipped)
 * the meta rows'. */
hymba_status hymba_block_prefill(const hymba_layer_desc *desc, const hymba_layer_weights *w,
                                 const hymba_block_weights *bw, const void *meta,
                                 const void *x, int32_t batch, int32_t seq_len,
                                 const hymba_kv *kv_in, hymba_kv *kv_out,
                                 hymba_ssm_state *state_out, void *y, void *y_meta,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* One block step per sequence: arguments as hymba_layer_decode, plus bw. */
hymba_status hymba_block_decode(const hymba_layer_desc *desc, const hymba_layer_weights *w,
                                const hymba_block_weights *bw, const void *x, int32_t batch,
                                hymba_kv *kv, hymba_ssm_state *state, void *y,
                                void *workspace, size_t workspace_bytes, void *stream);

const char *hymba_status_str(int32_t status);  /* any value; unknown ones say so */
int32_t hymba_abi_version(void);
/* Last hipError_t seen by a failing call on this thread (0 if none). */
int32_t hymba_last_hip_error(void);

/* ---------------------------------------------------------------------------
 * Stage timing.  hymba_timer_enable(mask) selects stages by bit (1 << stage; -1 = all,
 * 0 = off).  Every launch of a selected stage inside the two layer calls is then
 * bracketed by a pair of HIP events recorded on the call's stream.  hymba_timer_read
 * waits for the recorded events of `stage`, returns the summed milliseconds and the
 * number of launches, and forgets them.  Host-side state; not thread-safe.  At most
 * 4096 launches are remembered per stage between reads.
 * ------------------------------------------------------------------------- */
typedef enum {
  HYMBA_STAGE_IN_PROJ = 0,   /* in_proj GEMM over the X rows (decode: all rows)    */
  HYMBA_STAGE_ATTN = 1,      /* attention (prefill) / split attention (decode)   */
  HYMBA_STAGE_XPROJ = 2,     /* x_proj GEMM: delta, B, C                         */
  HYMBA_STAGE_DTPROJ = 3,    /* dt_proj GEMM + softplus (prefill)                */
  HYMBA_STAGE_SCAN = 4,      /* selective scan + gate (prefill) / SSM step       */
  HYMBA_STAGE_NORM = 5,      /* RMSNorm + beta + average                         */
  HYMBA_STAGE_OUT_PROJ = 6,  /* out_proj GEMM                                    */
  HYMBA_STAGE_KV_WRITE = 7,  /* cache writes                                     */
  HYMBA_STAGE_META = 8,      /* in_proj and out_proj GEMMs over the meta rows   */
  HYMBA_STAGE_MISC = 9,      /* accumulator clears, format conversions, pos fill */
  HYMBA_STAGE_BLOCK = 10,    /* block wrapper: pre-norms, residuals, FFN GEMMs    */
  HYMBA_NUM_STAGES = 11
} hymba_stage;

hymba_status hymba_timer_enable(int32_t stage_mask);
hymba_status hymba_timer_read(int32_t stage, double *total_ms, int32_t *launches);

/* ---------------------------------------------------------------------------
 * Single-kernel entry points used by the tests and the bandwidth calibration.
 * hymba_op_gemm: C[M, N] = A[M, K] B[N, K]^T with fp32 accumulation, on the same
 *   kernel the layer uses for `dtype` (bf16: MFMA).  lda/ldb/ldc in elements;
 *   c_dtype is the storage type of C (HYMBA_DTYPE_F32 or the input dtype).
 * hymba_op_copy: a plain 16-byte-per-lane device copy of `bytes` (multiple of 16).
 * ------------------------------------------------------------------------- */
hymba_status hymba_op_gemm(int32_t dtype, const void *a, int64_t lda, const void *b,
                           int64_t ldb, void *c, int64_t ldc, int32_t c_dtype, int32_t m,
                           int32_t n, int32_t k, void *stream);
hymba_status hymba_op_copy(const void *src, void *dst, size_t bytes, void *stream);
/* hymba_op_probe: one launch of a probe of the chip's practical ceilings, for the
 *   benchmark's rooflines (the caller times it).  kind 0: `blocks` x 256 lanes each run
 *   8 independent chains of `iters` base-2 exponentials (v_exp_f32); kind 1: `blocks` x 4
 *   waves each run 4 independent chains of `iters` v_mfma_f32_32x32x16_bf16; kind 2: a
 *   streaming read of `bytes` (multiple of 16) at `src`; kind 3: as kind 1 with 8 rounds
 *   of MFMAs per iteration whose operands change every instruction, read from `src`
 *   (bf16, at least 4 MiB = bytes: 64 x 8 x 256 A fragments of 8 values, then as many B
 *   fragments; the caller fills them, e.g. with the layer's activation and weight
 *   distributions).  out: fp32, blocks x 256 (kinds 0, 1, 3) or 8192 x 256 (kind 2)
 *   values, written so the work is kept. */
hymba_status hymba_op_probe(int32_t kind, int32_t blocks, int32_t iters, const void *src,
                            size_t bytes, float *out, void *stream);

/* ---------------------------------------------------------------------------
 * hymba_op_attn: the attention heads alone (step a4), on the kernels the layer uses.
 * Source: Design formulation, attention-head equation (softmax(Q K^T) mixing over the
 * meta-prefixed tokens); "Meta Tokens" (meta keys always visible); "Combine global and
 * local attention" (window); GQA grouping from the KV-sharing section.
 *   Rows: the n_meta batch-shared meta rows, then batch * seq_len sequence rows (row
 *   n_meta + b*seq_len + j is X-position j of sequence b).
 *   q [rows, row stride q_ld], head h at columns h*head_dim ..; k, v [rows, kv_ld],
 *   kv head g at columns g*head_dim ..; o [rows, o_ld] receives O (head h at
 *   h*head_dim), all `dtype`.  Key j is visible to query i iff j <= i and (j < n_meta
 *   or window == 0 or i - j < window); q head h reads kv head h*Hkv/Hq.
 *   scale: 0 => 1/sqrt(head_dim).  Strides in elements, multiples of 8; pointers
 *   16-byte aligned.  bf16: head_dim 64 or 128; fp32: 32 or 64.
 *   workspace: device scratch of hymba_op_attn_workspace_bytes(...) bytes (V^T staging
 *   for bf16; may be NULL when that is 0).  Errors as for the layer calls.
 * ------------------------------------------------------------------------- */
size_t hymba_op_attn_workspace_bytes(int32_t dtype, int32_t n_meta, int32_t seq_len,
                                     int32_t batch, int32_t n_kv_heads, int32_t head_dim);
hymba_status hymba_op_attn(int32_t dtype, const void *q, int64_t q_ld, const void *k,
                           const void *v, int64_t kv_ld, void *o, int64_t o_ld, int32_t n_meta,
                           int32_t seq_len, int32_t batch, int32_t n_q_heads,
                           int32_t n_kv_heads, int32_t head_dim, int32_t window, float scale,
                           void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * hymba_op_scan: the SSM heads alone (steps a3's dt projection and a5), on the kernels
 * the layer uses.  Source: Design formulation, SSM-head mixing coefficients and the
 * gated output Y_ssm = G * SSM(X); dt = softplus(delta W_dt^T + b) (Mamba).
 *   Rows as for hymba_op_attn.  z [rows, z_ld] dtype holds the SSM input x at columns
 *   xs_col .. xs_col + d_inner and G at g_col .. g_col + d_inner; delta [rows, dt_rank]
 *   dtype (dense); bc [rows, 2*d_state] fp32 (B then C); w_dt [d_inner, dt_rank] dtype;
 *   dt_bias [d_inner], A [d_inner, d_state], D [d_inner] fp32.
 *   Every sequence starts from h = 0 and runs over the meta rows, then its own rows:
 *     dt = softplus(delta W_dt^T + dt_bias); h = exp(dt A) h + dt x B; y = C.h + D x;
 *   y [rows, y_ld] (dtype) receives y * SiLU(G) (the meta rows once);
 *   h_out [batch, d_inner, d_state] fp32 (may be NULL) the final states.
 *   chunk_tokens: time chunk of the bf16 scan, as hymba_layer_desc.scan_chunk.
 *   workspace: hymba_op_scan_workspace_bytes(...) bytes (the post-meta state and chunk
 *   summaries of the bf16 scan, or fp32 dt for the other shapes; may be NULL when that
 *   is 0).  Errors as for the layer calls.
 * ------------------------------------------------------------------------- */
size_t hymba_op_scan_workspace_bytes(int32_t dtype, int32_t n_meta, int32_t seq_len,
                                     int32_t batch, int32_t d_inner, int32_t d_state,
                                     int32_t dt_rank, int32_t chunk_tokens);
hymba_status hymba_op_scan(int32_t dtype, const void *z, int64_t z_ld, int32_t xs_col,
                           int32_t g_col, const void *delta, const float *bc,
                           const void *w_dt, const float *dt_bias, const float *A,
                           const float *D, void *y, int64_t y_ld, float *h_out,
                           int32_t n_meta, int32_t seq_len, int32_t batch, int32_t d_inner,
                           int32_t d_state, int32_t dt_rank, int32_t chunk_tokens,
                           void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* HYMBA_H */
