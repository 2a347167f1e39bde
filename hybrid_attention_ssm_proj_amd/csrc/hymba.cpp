// C ABI of libhymba: argument validation, workspace layout and the launch sequence of
// the Hymba hybrid-head layer (prefill and decode).  The method's steps follow the
// design formulation of "Hymba: A Hybrid-head Architecture for Small Language Models"
// (outta.ai summary): meta-prefixed in_proj, attention heads and SSM heads on the same
// split, normalised + beta-scaled fusion, out_proj.
#include "../../include/hymba.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "kernels.h"

using namespace hymba;

namespace {

thread_local int32_t g_last_hip_error = 0;

hymba_status fail_hip(hipError_t e) {
  g_last_hip_error = (int32_t)e;
  return HYMBA_ERR_HIP;
}

// ----------------------------------------------------------------- stage timers
struct StageTimer {
  std::vector<hipEvent_t> start, stop;
  int used = 0;
};
uint32_t g_timer_mask = 0;
StageTimer g_timers[HYMBA_NUM_STAGES];
constexpr int kMaxTimedLaunches = 4096;

struct TimerScope {
  StageTimer* t = nullptr;
  hipStream_t s;
  int idx = -1;
  TimerScope(int stage, hipStream_t stream) : s(stream) {
    if (!(g_timer_mask & (1u << stage))) return;
    t = &g_timers[stage];
    if (t->used >= kMaxTimedLaunches) {
      t = nullptr;
      return;
    }
    if (t->used == (int)t->start.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess) {
        t = nullptr;
        return;
      }
      if (hipEventCreate(&b) != hipSuccess) {
        (void)hipEventDestroy(a);
        t = nullptr;
        return;
      }
      t->start.push_back(a);
      t->stop.push_back(b);
    }
    idx = t->used++;
    (void)hipEventRecord(t->start[idx], s);
  }
  ~TimerScope() {
    if (t != nullptr && idx >= 0) (void)hipEventRecord(t->stop[idx], s);
  }
};

#define HYMBA_LAUNCH(stage, expr)            \
  do {                                       \
    TimerScope ts_((stage), stream);         \
    hipError_t e_ = (expr);                  \
    if (e_ != hipSuccess) return fail_hip(e_); \
  } while (0)

// ----------------------------------------------------------------- shapes
struct Shape {
  int d, Hq, Hkv, dh, Di, N, R, M, W, share, es;
  int H2;  // Mamba-2 heads (0: Mamba head with per-channel A and a rank-R dt projection)
  int G;   // branch-norm groups of G channels (0: RMSNorm over each branch)
  int nx;  // x_proj output width: (H2 ? H2 : R) + 2N
  int chunk;  // time chunk of the Mamba-head scan in tokens (0: chosen per call)
  bool bf16;
  int64_t qw, kvw, n_in, fw, xs_col, g_col, k_col, v_col;
  float scale;
};

bool is_pow2_in(int v, int lo, int hi) {
  if (v < lo || v > hi) return false;
  return (v & (v - 1)) == 0;
}

hymba_status make_shape(const hymba_layer_desc* desc, Shape& s) {
  if (desc == nullptr) return HYMBA_ERR_INVALID_ARG;
  const hymba_layer_desc& d = *desc;
  if (d.d_model <= 0 || d.n_q_heads <= 0 || d.n_kv_heads <= 0 || d.head_dim <= 0 ||
      d.d_inner <= 0 || d.d_state <= 0 || d.n_meta < 0 || d.window < 0 || d.ssm_heads < 0)
    return HYMBA_ERR_INVALID_ARG;
  const bool head_ssm = d.ssm_heads > 0;
  if (!head_ssm && d.dt_rank <= 0) return HYMBA_ERR_INVALID_ARG;
  if (d.kv_share != 0 && d.kv_share != 1) return HYMBA_ERR_INVALID_ARG;
  if (d.dtype != HYMBA_DTYPE_F32 && d.dtype != HYMBA_DTYPE_BF16) return HYMBA_ERR_INVALID_ARG;
  if (!(d.rms_eps >= 0.f) || !std::isfinite(d.rms_eps)) return HYMBA_ERR_INVALID_ARG;
  if (!(d.softmax_scale >= 0.f) || !std::isfinite(d.softmax_scale)) return HYMBA_ERR_INVALID_ARG;
  if (d.n_q_heads % d.n_kv_heads != 0) return HYMBA_ERR_INVALID_ARG;
  const bool bf16 = d.dtype == HYMBA_DTYPE_BF16;
  // kernels: 16-byte row chunks, 4-column epilogue groups, <= 16 q heads per kv head
  if (d.d_model % 8 || d.d_inner % 8 || d.head_dim % 8 || (!head_ssm && d.dt_rank % 8))
    return HYMBA_ERR_UNSUPPORTED;
  // Mamba-2 heads: bf16, heads of 64 channels, a multiple of 4 heads, N in {16..128}
  if (head_ssm && (!bf16 || !scan_ssd_supported(d.d_state, d.d_inner, d.ssm_heads)))
    return HYMBA_ERR_UNSUPPORTED;
  const int grp = d.n_q_heads / d.n_kv_heads;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8) return HYMBA_ERR_UNSUPPORTED;
  if (bf16 ? (d.head_dim != 64 && d.head_dim != 128) : (d.head_dim != 32 && d.head_dim != 64))
    return HYMBA_ERR_UNSUPPORTED;
  if (!is_pow2_in(d.d_state, 4, 128)) return HYMBA_ERR_UNSUPPORTED;
  if (!head_ssm && d.dt_rank > 512) return HYMBA_ERR_UNSUPPORTED;
  if (d.norm_group < 0 || d.scan_chunk < 0) return HYMBA_ERR_INVALID_ARG;
  if (d.scan_chunk % 16) return HYMBA_ERR_UNSUPPORTED;
  if (d.norm_group > 0 &&
      (!is_pow2_in(d.norm_group, 8, 512) || (d.n_q_heads * d.head_dim) % d.norm_group ||
       d.d_inner % d.norm_group))
    return HYMBA_ERR_UNSUPPORTED;
  s.d = d.d_model;
  s.Hq = d.n_q_heads;
  s.Hkv = d.n_kv_heads;
  s.dh = d.head_dim;
  s.Di = d.d_inner;
  s.N = d.d_state;
  s.R = head_ssm ? 0 : d.dt_rank;
  s.H2 = head_ssm ? d.ssm_heads : 0;
  s.G = d.norm_group;
  s.chunk = d.scan_chunk;
  s.nx = (head_ssm ? d.ssm_heads : d.dt_rank) + 2 * d.d_state;
  s.M = d.n_meta;
  s.W = d.window;
  s.share = d.kv_share;
  s.bf16 = bf16;
  s.es = bf16 ? 2 : 4;
  s.qw = (int64_t)s.Hq * s.dh;
  s.kvw = (int64_t)s.Hkv * s.dh;
  s.k_col = s.qw;
  s.v_col = s.qw + s.kvw;
  s.xs_col = s.qw + (s.share ? 0 : 2 * s.kvw);
  s.g_col = s.xs_col + s.Di;
  s.n_in = s.g_col + s.Di;
  s.fw = s.qw + s.Di;
  s.scale = d.softmax_scale > 0.f ? d.softmax_scale : 1.0f / std::sqrt((float)s.dh);
  if (s.n_in > (1 << 30) || s.fw > (1 << 30)) return HYMBA_ERR_UNSUPPORTED;
  return HYMBA_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Carve {
  size_t z, delta, bc, dt, f, vt, macc, ssp, fac, hmeta, hsum, ssum, part, xdbl, yacc, total;
};


// Keys per decode-attention split: the largest of 256 / 192 / 128 that tiles the
// longest key list (meta + window) without a partly empty last split, else 256.
// Keys per split of the split-key decode attention: the widest split (256, 192 or 128
// keys dividing the key count, else 256) whose grid of batch x kv heads x splits still
// holds at least 128 workgroups; a smaller batch takes 64-key splits, the most
// workgroups (one sequence with 4 kv heads and 1152 keys: 72 instead of 24).
int decode_kps(const Shape& s, int span_max, int batch) {
  const int n = s.M + span_max;
  const int64_t units = (int64_t)std::max(batch, 1) * s.Hkv;
  for (int k : {256, 192, 128})
    if (n % k == 0 && units * ((n + k - 1) / k) >= 128) return k;
  if (units * ((n + 255) / 256) >= 128) return 256;
  return 64;
}
int decode_nsplit(const Shape& s, int span_max, int batch) {
  const int k = decode_kps(s, span_max, batch);
  return (s.M + span_max + k - 1) / k;
}

bool fused_dt(const Shape& s) {
  return s.H2 == 0 && s.bf16 && scan_chunk_supported(s.N, s.R, s.Di);
}

// Time chunk of the chunk-carried scan over B sequences of T tokens (chunk_override > 0:
// the caller's), the number of chunks, and the chunk summaries one launch needs (in
// units of a [Di, N] state plus a [Di] sum of dt).
int scan_chunk_for(int chunk_override, int B, int Di, int T) {
  return chunk_override > 0 ? chunk_override : scan_default_chunk(B, Di, T);
}
int scan_chunks(int chunk_override, int B, int Di, int T) {
  return scan_chunk_count(T, scan_chunk_for(chunk_override, B, Di, T));
}
int64_t scan_summaries(int chunk_override, int B, int Di, int T) {
  if (B <= 0 || T <= 0) return 0;
  return (int64_t)B * (scan_chunks(chunk_override, B, Di, T) - 1);
}
// At most 65 chunks (the carry scan runs over one wavefront) and a grid of at most 65535
// (sequence, chunk) rows.
bool scan_chunks_ok(int chunk_override, int B, int Di, int T) {
  if (B <= 0 || T <= 0) return true;
  const int k = scan_chunks(chunk_override, B, Di, T);
  return k <= 65 && (int64_t)B * k <= 65535;
}

// Prefill: rows = meta rows + batch * tokens.  dt is materialised only when the scan
// does not compute it in place.
// K slices for a split-K projection so that the grid holds ~1 workgroup per CU.
int splitk_factor(int M, int N, int K) {
  const int tiles = std::max(1, ((N + 63) / 64) * ((M + 127) / 128));
  const int want = (256 + tiles - 1) / tiles;
  return std::max(1, std::min(want, K / 256));
}

// Decode projections split along K (bf16, every K a multiple of 256): x_proj into fp32
// atomics, out_proj into per-slice fp32 partials summed by the row store.
bool decode_splitk(const Shape& s) {
  return s.bf16 && s.d % 256 == 0 && s.Di % 256 == 0 && s.fw % 256 == 0;
}

int out_proj_slices(const Shape& s, int rows) {
  if (rows <= 0 || s.d <= 0) return 1;
  return splitk_slices((int)s.fw, splitk_factor(rows, s.d, (int)s.fw));
}

Carve carve_prefill(const Shape& s, int64_t rows, int B, int L, bool cached = false) {
  Carve c{};
  size_t off = 0;
  c.z = off;
  off = align_up(off + (size_t)rows * s.n_in * s.es);
  c.delta = off;  // Mamba head: delta [rows, R]; Mamba-2 heads: none
  off = align_up(off + (size_t)rows * s.R * s.es);
  c.bc = off;     // [rows, 2N] fp32 (B | C); Mamba-2 heads: [rows, H2 + 2N] (u | B | C)
  off = align_up(off + (size_t)rows * (s.H2 + 2 * s.N) * 4);
  c.dt = off;
  if (s.H2 == 0 && !fused_dt(s)) off = align_up(off + (size_t)rows * s.Di * 4);
  c.f = off;
  off = align_up(off + (size_t)rows * s.fw * s.es);
  c.vt = off;  // bf16 attention: V^T staging
  if (s.bf16) off = align_up(off + attention_vt_bytes(s.M, L, B, s.Hkv, s.dh));
  c.macc = off;  // bf16: fp32 partials of the split-K out_proj over the meta rows
  if (s.bf16 && !cached) off = align_up(off + (size_t)out_proj_slices(s, s.M) * s.M * s.d * 4);
  c.ssp = off;   // bf16 + fused scan: per-row partial sums of squares of the branches
  if (s.bf16 && fused_dt(s))
    off = align_up(off + (size_t)rows * (s.Hq + scan_channel_blocks(s.N, s.Di)) * 4);
  c.fac = off;   // and the two row factors derived from them
  if (s.bf16 && fused_dt(s)) off = align_up(off + (size_t)rows * 2 * 4);
  // fused scan: the state after the meta rows (scanned once, then every sequence starts
  // from it) and the chunk summaries of the larger of its two launches
  c.hmeta = off;
  const int Mr = cached ? 0 : s.M;
  if (fused_dt(s) && Mr > 0 && B > 0) off = align_up(off + (size_t)s.Di * s.N * 4);
  const int64_t nsum = fused_dt(s) ? std::max(scan_summaries(s.chunk, 1, s.Di, Mr),
                                              scan_summaries(s.chunk, B, s.Di, L))
                                   : 0;
  c.hsum = off;
  off = align_up(off + (size_t)nsum * s.Di * s.N * 4);
  c.ssum = off;
  off = align_up(off + (size_t)nsum * s.Di * 4);
  c.total = off;
  return c;
}

// Decode: one row per sequence.  The fp32 accumulators of the split-K projections
// (xdbl, yacc) are contiguous and last, so one fill clears them.
Carve carve_decode(const Shape& s, int batch, int nsplit) {
  Carve c{};
  size_t off = 0;
  c.z = off;
  off = align_up(off + (size_t)batch * s.n_in * s.es);
  c.f = off;
  off = align_up(off + (size_t)batch * s.fw * s.es);
  c.part = off;
  off = align_up(off + (size_t)batch * s.Hq * nsplit * (s.dh + 4) * 4);
  c.xdbl = off;
  off = align_up(off + (size_t)batch * s.nx * 4);
  c.yacc = off;  // out_proj partials, one [batch, d] fp32 block per K slice
  off = align_up(off + (size_t)(decode_splitk(s) ? out_proj_slices(s, batch) : 1) * batch * s.d * 4);
  c.total = off;
  return c;
}

bool misaligned(const void* p) { return p != nullptr && ((uintptr_t)p & 15) != 0; }

template <typename... P>
bool any_misaligned(P... ptrs) {
  return (misaligned((const void*)ptrs) || ...);
}

hymba_status check_weights(const hymba_layer_weights* w, const Shape& s) {
  if (w == nullptr || !w->w_in || !w->w_x || (s.H2 == 0 && !w->w_dt) || !w->w_out ||
      !w->dt_bias || !w->A || !w->D || !w->beta_attn || !w->beta_ssm)
    return HYMBA_ERR_INVALID_ARG;
  if (any_misaligned(w->w_in, w->w_x, w->w_dt, w->w_out, w->dt_bias, w->A, w->D, w->beta_attn,
                     w->beta_ssm))
    return HYMBA_ERR_ALIGNMENT;
  return HYMBA_OK;
}

char* ws_ptr(void* ws, size_t off) { return (char*)ws + off; }

// ----------------------------------------------------------------- static scratch
// The workspace of hymba_layer_decode_static: a fixed array in device memory, one copy per
// device the library runs on, held until the process ends.  In host code `scratch` names a
// host-side stand-in; its device address on the current device comes from
// hipGetSymbolAddress, once per device, and only that address is passed to kernels.
constexpr size_t kStaticScratchBytes = HYMBA_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hymba_status static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return HYMBA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e);
    if (p == nullptr) return fail_hip(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HYMBA_OK;
}

}  // namespace

// ===================================================================== ABI

extern "C" {

int32_t hymba_abi_version(void) { return HYMBA_ABI_VERSION; }

int32_t hymba_last_hip_error(void) { return g_last_hip_error; }

const char* hymba_status_str(int32_t s) {
  // an int, not the enum: a C caller may pass any value, and a C++ enum without a fixed
  // underlying type cannot hold values outside its enumerators' range
  switch (s) {
    case HYMBA_OK: return "ok";
    case HYMBA_ERR_INVALID_ARG: return "invalid argument";
    case HYMBA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case HYMBA_ERR_WORKSPACE: return "workspace missing or too small";
    case HYMBA_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
    case HYMBA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

size_t hymba_layer_workspace_bytes(const hymba_layer_desc* desc, int32_t batch, int32_t seq_len,
                                   int32_t mode) {
  Shape s;
  if (make_shape(desc, s) != HYMBA_OK || batch < 0 || seq_len < 0) return 0;
  if (mode == 0) {
    const int64_t rows = (int64_t)s.M + (int64_t)batch * seq_len;
    return carve_prefill(s, rows, batch, seq_len).total;
  }
  if (mode == 2) {  // prefill from a meta-prefix cache: the meta rows are not recomputed
    return carve_prefill(s, (int64_t)batch * seq_len, batch, seq_len, true).total;
  }
  if (mode == 1) {
    // seq_len carries the ring capacity (slots) for decode.
    const int span_max = s.W > 0 ? std::min(s.W, seq_len) : seq_len;
    return carve_decode(s, batch, decode_nsplit(s, span_max, batch)).total;
  }
  return 0;
}

hymba_status hymba_timer_enable(int32_t stage_mask) {
  g_timer_mask = (uint32_t)stage_mask & ((1u << HYMBA_NUM_STAGES) - 1);
  return HYMBA_OK;
}

hymba_status hymba_timer_read(int32_t stage, double* total_ms, int32_t* launches) {
  if (stage < 0 || stage >= HYMBA_NUM_STAGES || total_ms == nullptr || launches == nullptr)
    return HYMBA_ERR_INVALID_ARG;
  StageTimer& t = g_timers[stage];
  double sum = 0.0;
  for (int i = 0; i < t.used; ++i) {
    hipError_t e = hipEventSynchronize(t.stop[i]);
    if (e != hipSuccess) return fail_hip(e);
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, t.start[i], t.stop[i]);
    if (e != hipSuccess) return fail_hip(e);
    sum += ms;
  }
  *total_ms = sum;
  *launches = t.used;
  t.used = 0;
  return HYMBA_OK;
}

}  // extern "C"

namespace {

// The prefill pass.  Three uses: the plain call (meta rows computed with the batch),
// the meta-cache build (batch 0: meta rows only; h_meta_out receives the state after
// them), and the cached call (cache != nullptr: the meta rows are not recomputed; their
// K/V and the post-meta state come from the cache).  Mr = meta rows held in Z and F.
hymba_status prefill_impl(const hymba_layer_desc* desc, const hymba_layer_weights* w,
                          const void* meta, const void* x, int32_t batch, int32_t seq_len,
                          const hymba_kv* kv_in, hymba_kv* kv_out, hymba_ssm_state* state_out,
                          void* y, void* y_meta, const hymba_meta_cache* cache,
                          float* h_meta_out, void* workspace, size_t workspace_bytes,
                          void* stream_) {
  Shape s;
  hymba_status st = make_shape(desc, s);
  if (st != HYMBA_OK) return st;
  if ((st = check_weights(w, s)) != HYMBA_OK) return st;
  if (batch < 0 || seq_len < 0) return HYMBA_ERR_INVALID_ARG;
  const bool cached = cache != nullptr;
  const int B = batch, L = seq_len, M = s.M, Mr = cached ? 0 : s.M;
  const int64_t BL = (int64_t)B * L;
  const int64_t rows = Mr + BL;
  if (rows >= (int64_t)1 << 31 || BL >= (int64_t)1 << 31) return HYMBA_ERR_UNSUPPORTED;
  if (Mr > 0 && meta == nullptr) return HYMBA_ERR_INVALID_ARG;
  if (h_meta_out != nullptr && BL != 0) return HYMBA_ERR_INVALID_ARG;
  if (cached) {
    if (M > 0 && cache->h == nullptr) return HYMBA_ERR_INVALID_ARG;
    if (!s.share && M > 0 && (cache->k_meta == nullptr || cache->v_meta == nullptr))
      return HYMBA_ERR_INVALID_ARG;
    if (any_misaligned(cache->k_meta, cache->v_meta, cache->h)) return HYMBA_ERR_ALIGNMENT;
  }
  if (BL > 0 && (x == nullptr || y == nullptr)) return HYMBA_ERR_INVALID_ARG;
  if (s.share) {
    if (kv_in == nullptr || kv_out != nullptr) return HYMBA_ERR_INVALID_ARG;
    if (kv_in->k == nullptr || kv_in->v == nullptr || kv_in->slots < L || kv_in->slots <= 0)
      return HYMBA_ERR_INVALID_ARG;
    if (M > 0 && (kv_in->k_meta == nullptr || kv_in->v_meta == nullptr))
      return HYMBA_ERR_INVALID_ARG;
    if (any_misaligned(kv_in->k, kv_in->v, kv_in->k_meta, kv_in->v_meta))
      return HYMBA_ERR_ALIGNMENT;
  } else {
    if (kv_in != nullptr) return HYMBA_ERR_INVALID_ARG;
    if (kv_out != nullptr) {
      if (kv_out->slots <= 0 || kv_out->k == nullptr || kv_out->v == nullptr)
        return HYMBA_ERR_INVALID_ARG;
      if (kv_out->is_ring != 0 && kv_out->is_ring != 1) return HYMBA_ERR_INVALID_ARG;
      if (!kv_out->is_ring && kv_out->slots < L) return HYMBA_ERR_INVALID_ARG;
      if (Mr > 0 && (kv_out->k_meta == nullptr || kv_out->v_meta == nullptr))
        return HYMBA_ERR_INVALID_ARG;
      if (any_misaligned(kv_out->k, kv_out->v, kv_out->k_meta, kv_out->v_meta))
        return HYMBA_ERR_ALIGNMENT;
    }
  }
  if (state_out != nullptr) {
    if (state_out->h == nullptr) return HYMBA_ERR_INVALID_ARG;
    if (any_misaligned(state_out->h, state_out->pos)) return HYMBA_ERR_ALIGNMENT;
  }
  if (any_misaligned(meta, x, y, y_meta, workspace)) return HYMBA_ERR_ALIGNMENT;
  if (fused_dt(s) && (!scan_chunks_ok(s.chunk, 1, s.Di, Mr) || !scan_chunks_ok(s.chunk, B, s.Di, L)))
    return HYMBA_ERR_UNSUPPORTED;
  const Carve cv = carve_prefill(s, rows, B, L, cached);
  if (rows > 0 && (workspace == nullptr || workspace_bytes < cv.total)) return HYMBA_ERR_WORKSPACE;
  hipStream_t stream = (hipStream_t)stream_;
  if (h_meta_out != nullptr && M == 0)  // no meta tokens: the post-meta state is zero
    HYMBA_LAUNCH(HYMBA_STAGE_MISC, launch_zero_f32(h_meta_out, (int64_t)s.Di * s.N, stream));
  if (rows == 0) return HYMBA_OK;

  char* z = ws_ptr(workspace, cv.z);
  char* delta = ws_ptr(workspace, cv.delta);
  float* bc = (float*)ws_ptr(workspace, cv.bc);
  float* dt = (float*)ws_ptr(workspace, cv.dt);
  char* f = ws_ptr(workspace, cv.f);
  const bool b16 = s.bf16;
  auto gemm = [&](const GemmOperands& op, const GemmOutput& out, GemmShape shape) {
    return b16 ? launch_gemm_bf16(op, out, shape, stream) : launch_gemm_f32(op, out, stream);
  };

  // The RMS norms of the two branches are applied inside out_proj (bf16, fused scan):
  // attention and the scan store beta * O and beta * Y_ssm plus partial sums of squares
  // (per head, per channel block); a small kernel turns them into two factors per row,
  // and out_proj scales the two K segments of F by them.  This drops the separate pass
  // that rewrote F.
  const bool few_meta = b16 && s.d % 256 == 0 && s.fw % 256 == 0;
  const GemmOperands op_out{f + (size_t)Mr * s.fw * s.es, s.fw, nullptr, 0, (int)BL, w->w_out,
                            s.fw, (int)BL, s.d, (int)s.fw};
  const bool defer_norm = b16 && fused_dt(s) && s.G == 0 && s.qw % 128 == 0 &&
                          (BL == 0 || gemm_bf16_rowscaled_ok(op_out, (int)s.qw)) &&
                          !any_misaligned(w->beta_attn, w->beta_ssm);
  const int n_sblk = defer_norm ? scan_channel_blocks(s.N, s.Di) : 0;
  const int64_t ssp_ld = rows;  // partial column i of row r at ssp[i * rows + r]
  float* ssp = defer_norm ? (float*)ws_ptr(workspace, cv.ssp) : nullptr;
  float* fac = defer_norm ? (float*)ws_ptr(workspace, cv.fac) : nullptr;

  // 1. in_proj over [meta; X]: the batch-shared meta rows once, then the X rows.
  // The meta rows are few: the few-row kernel (64-row blocks, every column tile its own
  // workgroup) fills the chip better than 256-row tiles.
  if (Mr > 0) {
    GemmOperands op{meta, s.d, nullptr, 0, M, w->w_in, s.d, M, (int)s.n_in, s.d};
    if (few_meta) {
      HYMBA_LAUNCH(HYMBA_STAGE_META,
                   launch_gemm_bf16_decode_in(op, z, s.n_in, -1, -1, nullptr, nullptr, 1, s.Hkv,
                                              s.dh, nullptr, nullptr, 0, stream));
    } else {
      GemmOutput out{EpiKind::Store, z, s.n_in, nullptr, 0, M, 0, nullptr};
      HYMBA_LAUNCH(HYMBA_STAGE_META, gemm(op, out, GemmShape::Large));
    }
  }
  if (BL > 0) {
    GemmOperands op{x, s.d, nullptr, 0, (int)BL, w->w_in, s.d, (int)BL, (int)s.n_in, s.d};
    GemmOutput out{EpiKind::Store, z + (size_t)Mr * s.n_in * s.es, s.n_in, nullptr, 0, (int)BL, 0,
                   nullptr};
    HYMBA_LAUNCH(HYMBA_STAGE_IN_PROJ, gemm(op, out, GemmShape::Large));
  }
  // 2. producer cache.
  if (!s.share && kv_out != nullptr) {
    HYMBA_LAUNCH(HYMBA_STAGE_KV_WRITE,
                 launch_kv_write_prefill(b16, z, s.n_in, (int)s.k_col, (int)s.v_col, kv_out->k_meta,
                                         kv_out->v_meta, kv_out->k, kv_out->v, kv_out->slots, Mr,
                                         L, B, s.Hkv, s.dh, stream));
  }
  // 3. attention heads -> F[:, :qw].
  {
    AttnParams ap{};
    ap.q = z;
    ap.q_row_stride = s.n_in;
    if (s.share) {
      ap.k_meta = kv_in->k_meta;
      ap.v_meta = kv_in->v_meta;
      ap.meta_head_stride = (int64_t)M * s.dh;
      ap.meta_row_stride = s.dh;
      ap.k_seq = kv_in->k;
      ap.v_seq = kv_in->v;
      ap.seq_batch_stride = (int64_t)s.Hkv * kv_in->slots * s.dh;
      ap.seq_head_stride = (int64_t)kv_in->slots * s.dh;
      ap.seq_row_stride = s.dh;
      ap.seq_slots = kv_in->slots;
    } else {
      if (cached) {  // meta K/V from the cache, [Hkv, M, dh]
        ap.k_meta = cache->k_meta;
        ap.v_meta = cache->v_meta;
        ap.meta_head_stride = (int64_t)M * s.dh;
        ap.meta_row_stride = s.dh;
      } else {
        ap.k_meta = z + s.k_col * s.es;
        ap.v_meta = z + s.v_col * s.es;
        ap.meta_head_stride = s.dh;
        ap.meta_row_stride = s.n_in;
      }
      ap.k_seq = z + ((size_t)Mr * s.n_in + s.k_col) * s.es;
      ap.v_seq = z + ((size_t)Mr * s.n_in + s.v_col) * s.es;
      ap.seq_batch_stride = (int64_t)L * s.n_in;
      ap.seq_head_stride = s.dh;
      ap.seq_row_stride = s.n_in;
      ap.seq_slots = L > 0 ? L : 1;
    }
    ap.o = f;
    ap.o_row_stride = s.fw;
    ap.n_meta = M;
    ap.meta_rows = Mr;
    ap.L = L;
    ap.B = B;
    ap.Hq = s.Hq;
    ap.Hkv = s.Hkv;
    ap.head_dim = s.dh;
    ap.window = s.W;
    ap.scale = s.scale;
    ap.ssp = ssp;
    ap.ssp_ld = ssp_ld;
    ap.beta = w->beta_attn;
    HYMBA_LAUNCH(HYMBA_STAGE_ATTN,
                 b16 ? launch_attention_prefill_bf16_dl(ap, ws_ptr(workspace, cv.vt), stream)
                     : launch_attention_prefill_f32(ap, stream));
  }
  // 4. x_proj: [delta | B | C] = Xs W_x^T (Mamba-2 heads: [u | B | C], all fp32).
  {
    GemmOperands op{z + s.xs_col * s.es, s.n_in, nullptr, 0, (int)rows, w->w_x, s.Di, (int)rows,
                    s.nx, s.Di};
    GemmOutput out = s.H2 ? GemmOutput{EpiKind::StoreF32, bc, s.nx, nullptr, 0, 0, 0, nullptr}
                          : GemmOutput{EpiKind::XProj, delta, s.R, bc, 2 * s.N, 0, s.R, nullptr};
    HYMBA_LAUNCH(HYMBA_STAGE_XPROJ, b16 && gemm_xproj_ok(op, out)
                                        ? launch_gemm_xproj_bf16(op, out, stream)
                                        : gemm(op, out, GemmShape::Narrow));
  }
  // 5. dt_proj + softplus (unless the scan computes it in place, or the heads take dt
  // straight from x_proj).
  const bool fuse = fused_dt(s);
  if (!fuse && s.H2 == 0) {
    GemmOperands op{delta, s.R, nullptr, 0, (int)rows, w->w_dt, s.R, (int)rows, s.Di, s.R};
    GemmOutput out{EpiKind::Softplus, dt, s.Di, nullptr, 0, 0, 0, w->dt_bias};
    HYMBA_LAUNCH(HYMBA_STAGE_DTPROJ, gemm(op, out, GemmShape::Narrow));
  }
  bool pos_written = false;  // the chunked scan writes state_out->pos itself
  // 6. selective scan + gate -> F[:, qw:].
  {
    ScanParams sp{};
    sp.z = z;
    sp.z_stride = s.n_in;
    sp.xs_col = (int)s.xs_col;
    sp.g_col = (int)s.g_col;
    sp.dt = dt;
    sp.bc = bc;
    sp.A = w->A;
    sp.D = w->D;
    sp.y = f + s.qw * s.es;
    sp.y_stride = s.fw;
    sp.h_out = state_out ? state_out->h : nullptr;
    sp.h0 = cached ? cache->h : nullptr;
    sp.n_meta = Mr;
    sp.L = L;
    sp.B = B;
    sp.Di = s.Di;
    sp.N = s.N;
    if (B == 0) {  // meta rows only: run them as one sequence of length 0
      sp.B = 1;
      sp.h_out = h_meta_out;
    }
    if (s.H2) {
      SsdParams qp{};
      qp.z = z;
      qp.z_stride = s.n_in;
      qp.xs_col = (int)s.xs_col;
      qp.g_col = (int)s.g_col;
      qp.xbc = bc;
      qp.xbc_ld = s.nx;
      qp.dt_bias = w->dt_bias;
      qp.A = w->A;
      qp.D = w->D;
      qp.h0 = sp.h0;
      qp.y = sp.y;
      qp.y_stride = sp.y_stride;
      qp.h_out = sp.h_out;
      qp.n_meta = Mr;
      qp.L = L;
      qp.B = sp.B;
      qp.H = s.H2;
      qp.N = s.N;
      HYMBA_LAUNCH(HYMBA_STAGE_SCAN, launch_scan_ssd(qp, stream));
    } else if (fuse) {
      // The meta rows once from h = 0 (their state is batch-shared), then every sequence
      // from that state (or from the cache's), each launch chunk-carried over time.
      ScanChunkParams cp{};
      cp.z = z;
      cp.z_stride = s.n_in;
      cp.xs_col = (int)s.xs_col;
      cp.g_col = (int)s.g_col;
      cp.delta = delta;
      cp.bc = bc;
      cp.w_dt = w->w_dt;
      cp.dt_bias = w->dt_bias;
      cp.A = w->A;
      cp.D = w->D;
      cp.y = sp.y;
      cp.y_stride = s.fw;
      cp.Di = s.Di;
      cp.N = s.N;
      cp.R = s.R;
      cp.hsum = (float*)ws_ptr(workspace, cv.hsum);
      cp.ssum = (float*)ws_ptr(workspace, cv.ssum);
      cp.ssp = ssp;
      cp.ssp_ld = ssp_ld;
      cp.ssp_col0 = s.Hq;
      cp.beta = defer_norm ? w->beta_ssm : nullptr;
      float* hmeta = (float*)ws_ptr(workspace, cv.hmeta);
      if (Mr > 0) {
        ScanChunkParams mp = cp;
        mp.row0 = 0;
        mp.T = Mr;
        mp.B = 1;
        mp.h0 = nullptr;
        mp.h_out = B > 0 ? hmeta : h_meta_out;
        mp.chunk = scan_chunk_for(s.chunk, 1, s.Di, Mr);
        mp.nchunks = scan_chunk_count(Mr, mp.chunk);
        HYMBA_LAUNCH(HYMBA_STAGE_META, launch_scan_chunk(mp, stream));
      }
      if (B > 0) {
        cp.row0 = Mr;
        cp.T = L;
        cp.B = B;
        cp.h0 = cached ? cache->h : (M > 0 ? hmeta : nullptr);
        cp.h_out = state_out ? state_out->h : nullptr;
        cp.chunk = scan_chunk_for(s.chunk, B, s.Di, L);
        cp.nchunks = scan_chunk_count(L, cp.chunk);
        if (state_out != nullptr && state_out->pos != nullptr) {  // pos[b] = L, by the scan
          cp.pos_out = state_out->pos;
          cp.pos_val = L;
          pos_written = true;
        }
        HYMBA_LAUNCH(HYMBA_STAGE_SCAN, launch_scan_chunk(cp, stream));
      }
    } else {
      HYMBA_LAUNCH(HYMBA_STAGE_SCAN, launch_scan_prefill(b16, sp, stream));
    }
  }
  // 7. RMSNorm + beta + average: in place, or as row factors for out_proj (the meta
  // rows, projected by the split-K kernel, are scaled in place by the same launch).
  if (defer_norm) {
    HYMBA_LAUNCH(HYMBA_STAGE_NORM,
                 launch_row_factors(ssp, ssp_ld, s.Hq, n_sblk, (int)rows, (int)s.qw, s.Di,
                                    desc->rms_eps, fac, f, s.fw,
                                    y_meta != nullptr ? Mr : 0, stream));
  } else if (s.G) {
    HYMBA_LAUNCH(HYMBA_STAGE_NORM, launch_group_norm(b16, f, s.fw, (int)rows, (int)s.qw, s.Di,
                                                     w->beta_attn, w->beta_ssm, desc->rms_eps,
                                                     s.G, stream));
  } else {
    HYMBA_LAUNCH(HYMBA_STAGE_NORM, launch_fuse_norm(b16, f, s.fw, (int)rows, (int)s.qw, s.Di,
                                                    w->beta_attn, w->beta_ssm, desc->rms_eps,
                                                    stream));
  }
  const RowScale rs_seq{fac != nullptr ? fac + 2 * (int64_t)Mr : nullptr, (int)s.qw};
  // 8. out_proj: sequence rows -> y, then the batch-shared meta rows -> y_meta.  Two
  // launches keep the large one on whole 256-row tiles (B*L rows), so it runs as an
  // exact number of rounds over the CUs.
  if (BL > 0) {
    GemmOutput out{EpiKind::Store, y, s.d, nullptr, 0, (int)BL, 0, nullptr};
    if (defer_norm) {
      HYMBA_LAUNCH(HYMBA_STAGE_OUT_PROJ, launch_gemm_bf16_rowscaled(op_out, out, rs_seq, stream));
    } else {
      HYMBA_LAUNCH(HYMBA_STAGE_OUT_PROJ, gemm(op_out, out, GemmShape::Large));
    }
  }
  if (Mr > 0 && y_meta != nullptr) {
    GemmOperands op{f, s.fw, nullptr, 0, M, w->w_out, s.fw, M, s.d, (int)s.fw};
    if (few_meta) {  // K is long: split it into fp32 partials, then sum and round to bf16
      float* macc = (float*)ws_ptr(workspace, cv.macc);
      const int64_t stride = (int64_t)M * s.d;
      HYMBA_LAUNCH(HYMBA_STAGE_META,
                   launch_gemm_bf16_splitk(op, macc, s.d, splitk_factor(M, s.d, (int)s.fw),
                                           stream, stride));
      HYMBA_LAUNCH(HYMBA_STAGE_META, launch_store_rows(true, macc, y_meta, M, s.d, stream,
                                                       out_proj_slices(s, M), stride));
    } else {
      GemmOutput out{EpiKind::Store, y_meta, s.d, nullptr, 0, M, 0, nullptr};
      HYMBA_LAUNCH(HYMBA_STAGE_META, gemm(op, out, GemmShape::Large));
    }
  }
  if (state_out != nullptr && state_out->pos != nullptr && B > 0 && !pos_written) {
    HYMBA_LAUNCH(HYMBA_STAGE_MISC, launch_fill_i32(state_out->pos, L, B, stream));
  }
  return HYMBA_OK;
}

}  // namespace

extern "C" {

hymba_status hymba_layer_prefill(const hymba_layer_desc* desc, const hymba_layer_weights* w,
                                 const void* meta, const void* x, int32_t batch,
                                 int32_t seq_len, const hymba_kv* kv_in, hymba_kv* kv_out,
                                 hymba_ssm_state* state_out, void* y, void* y_meta,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(desc, w, meta, x, batch, seq_len, kv_in, kv_out, state_out, y, y_meta,
                      nullptr, nullptr, workspace, workspace_bytes, stream);
}

hymba_status hymba_layer_meta_cache_build(const hymba_layer_desc* desc,
                                          const hymba_layer_weights* w, const void* meta,
                                          const hymba_kv* kv_in, hymba_meta_cache* cache,
                                          void* workspace, size_t workspace_bytes,
                                          void* stream) {
  if (desc == nullptr || cache == nullptr || cache->h == nullptr) return HYMBA_ERR_INVALID_ARG;
  if (desc->kv_share) {
    // the consumer's meta keys are the producer's: kv_in holds them
    if (kv_in == nullptr) return HYMBA_ERR_INVALID_ARG;
    hymba_kv src = *kv_in;
    if (src.k == nullptr || src.v == nullptr) {  // no sequence positions are read
      src.k = src.k_meta;
      src.v = src.v_meta;
    }
    if (src.slots <= 0) src.slots = 1;
    return prefill_impl(desc, w, meta, nullptr, 0, 0, &src, nullptr, nullptr, nullptr,
                        cache->y_meta, nullptr, cache->h, workspace, workspace_bytes, stream);
  }
  if (kv_in != nullptr) return HYMBA_ERR_INVALID_ARG;
  // producer: the meta K/V go to the cache (no sequence slots are written at batch 0)
  hymba_kv out{cache->k_meta, cache->v_meta, cache->k_meta, cache->v_meta, 1};
  return prefill_impl(desc, w, meta, nullptr, 0, 0, nullptr,
                      desc->n_meta > 0 ? &out : nullptr, nullptr, nullptr, cache->y_meta,
                      nullptr, cache->h, workspace, workspace_bytes, stream);
}

hymba_status hymba_layer_prefill_cached(const hymba_layer_desc* desc,
                                        const hymba_layer_weights* w,
                                        const hymba_meta_cache* cache, const void* x,
                                        int32_t batch, int32_t seq_len, const hymba_kv* kv_in,
                                        hymba_kv* kv_out, hymba_ssm_state* state_out, void* y,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  if (cache == nullptr) return HYMBA_ERR_INVALID_ARG;
  return prefill_impl(desc, w, nullptr, x, batch, seq_len, kv_in, kv_out, state_out, y, nullptr,
                      cache, nullptr, workspace, workspace_bytes, stream);
}

hymba_status hymba_kv_ring_fill(const hymba_kv* src, hymba_kv* dst, int32_t batch,
                                int32_t seq_len, int32_t n_meta, int32_t n_kv_heads,
                                int32_t head_dim, int32_t dtype, void* stream) {
  if (src == nullptr || dst == nullptr || batch < 0 || seq_len < 0 || n_meta < 0 ||
      n_kv_heads <= 0 || head_dim <= 0)
    return HYMBA_ERR_INVALID_ARG;
  if (dtype != HYMBA_DTYPE_F32 && dtype != HYMBA_DTYPE_BF16) return HYMBA_ERR_INVALID_ARG;
  if ((src->is_ring != 0 && src->is_ring != 1) || (dst->is_ring != 0 && dst->is_ring != 1))
    return HYMBA_ERR_INVALID_ARG;
  const bool b16 = dtype == HYMBA_DTYPE_BF16;
  if (head_dim % (b16 ? 8 : 4)) return HYMBA_ERR_UNSUPPORTED;
  if (src->slots <= 0 || dst->slots <= 0) return HYMBA_ERR_INVALID_ARG;
  const int n_last = std::min(seq_len, dst->slots);
  // src must hold positions [L - n_last, L); a non-ring dst must hold every position
  if (src->is_ring ? src->slots < n_last : src->slots < seq_len) return HYMBA_ERR_INVALID_ARG;
  if (!dst->is_ring && dst->slots < seq_len) return HYMBA_ERR_INVALID_ARG;
  const bool copy_meta = n_meta > 0 && (src->k_meta != dst->k_meta || src->v_meta != dst->v_meta);
  if (batch > 0 && n_last > 0 &&
      (src->k == nullptr || src->v == nullptr || dst->k == nullptr || dst->v == nullptr))
    return HYMBA_ERR_INVALID_ARG;
  if (copy_meta && (src->k_meta == nullptr || src->v_meta == nullptr || dst->k_meta == nullptr ||
                    dst->v_meta == nullptr))
    return HYMBA_ERR_INVALID_ARG;
  if (any_misaligned(src->k, src->v, src->k_meta, src->v_meta, dst->k, dst->v, dst->k_meta,
                     dst->v_meta))
    return HYMBA_ERR_ALIGNMENT;
  if ((int64_t)batch * n_last + n_meta >= ((int64_t)1 << 31)) return HYMBA_ERR_UNSUPPORTED;
  hipStream_t stream_ = (hipStream_t)stream;
  {
    hipStream_t stream = stream_;  // for the stage timer
    HYMBA_LAUNCH(HYMBA_STAGE_KV_WRITE,
                 launch_kv_ring_fill(b16, src->k, src->v, src->slots, src->k_meta, src->v_meta,
                                     dst->k, dst->v, dst->slots, dst->k_meta, dst->v_meta,
                                     copy_meta, n_meta, seq_len, n_last, batch, n_kv_heads,
                                     head_dim, stream));
  }
  return HYMBA_OK;
}

hymba_status hymba_layer_decode_static(const hymba_layer_desc* desc,
                                       const hymba_layer_weights* w, const void* x,
                                       int32_t batch, hymba_kv* kv, hymba_ssm_state* state,
                                       void* y, void* stream) {
  if (batch < 0 || kv == nullptr || kv->slots <= 0) return HYMBA_ERR_INVALID_ARG;
  const size_t need = hymba_layer_workspace_bytes(desc, batch, kv->slots, 1);
  if (need == 0 && batch > 0) {  // the descriptor itself is rejected: let the call say why
    return hymba_layer_decode(desc, w, x, batch, kv, state, y, nullptr, 0, stream);
  }
  if (need > kStaticScratchBytes) return HYMBA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (batch > 0) {
    hymba_status st = static_scratch(&ws);
    if (st != HYMBA_OK) return st;
  }
  return hymba_layer_decode(desc, w, x, batch, kv, state, y, ws, kStaticScratchBytes, stream);
}

hymba_status hymba_layer_decode(const hymba_layer_desc* desc, const hymba_layer_weights* w,
                                const void* x, int32_t batch, hymba_kv* kv,
                                hymba_ssm_state* state, void* y, void* workspace,
                                size_t workspace_bytes, void* stream_) {
  Shape s;
  hymba_status st = make_shape(desc, s);
  if (st != HYMBA_OK) return st;
  if ((st = check_weights(w, s)) != HYMBA_OK) return st;
  if (batch < 0) return HYMBA_ERR_INVALID_ARG;
  const int B = batch, M = s.M;
  if (kv == nullptr || state == nullptr) return HYMBA_ERR_INVALID_ARG;
  if (kv->slots <= 0 || kv->k == nullptr || kv->v == nullptr) return HYMBA_ERR_INVALID_ARG;
  if (M > 0 && (kv->k_meta == nullptr || kv->v_meta == nullptr)) return HYMBA_ERR_INVALID_ARG;
  if (s.W > 0 && kv->slots < s.W) return HYMBA_ERR_INVALID_ARG;
  if (state->h == nullptr || state->pos == nullptr) return HYMBA_ERR_INVALID_ARG;
  if (B > 0 && (x == nullptr || y == nullptr)) return HYMBA_ERR_INVALID_ARG;
  if (any_misaligned(x, y, kv->k, kv->v, kv->k_meta, kv->v_meta, state->h, state->pos, workspace))
    return HYMBA_ERR_ALIGNMENT;
  const int span_max = s.W > 0 ? s.W : kv->slots;
  const int nsplit = decode_nsplit(s, span_max, B);
  const Carve cv = carve_decode(s, B, nsplit);
  if (B > 0 && (workspace == nullptr || workspace_bytes < cv.total)) return HYMBA_ERR_WORKSPACE;
  hipStream_t stream = (hipStream_t)stream_;
  if (B == 0) return HYMBA_OK;

  char* z = ws_ptr(workspace, cv.z);
  char* f = ws_ptr(workspace, cv.f);
  float* part = (float*)ws_ptr(workspace, cv.part);
  float* xdbl = (float*)ws_ptr(workspace, cv.xdbl);
  float* yacc = (float*)ws_ptr(workspace, cv.yacc);
  const bool b16 = s.bf16;
  const int nx = s.nx;
  // Attention (bf16): one workgroup per (sequence, kv head) streaming all keys once the
  // pairs fill the chip (256 CUs), else key splits merged by the combine kernel.
  const bool stream_attn = b16 && (int64_t)B * s.Hkv >= 256 && kv->slots >= 64;

  // in_proj.  bf16 with every K a multiple of 256: the few-row GEMM writes Z and the
  // producer's new K/V row into its ring slot in the same pass, and x_proj / out_proj
  // run split-K into fp32 accumulators.  Otherwise the tiled GEMM writes Z directly and
  // a copy kernel fills the ring.
  const bool splitk = decode_splitk(s);
  // A small batch (at most kGemvMaxRows sequences, bf16) streams the weights through the
  // few-row kernel instead: its three projections store their results directly (no K
  // slices, no accumulator to clear), and in_proj writes the producer's ring slot too.
  const bool gemv = b16 && B <= kGemvMaxRows && (s.xs_col * s.es) % 16 == 0 &&
                    gemv_bf16_ok(B, s.d, s.d, s.d) && gemv_bf16_ok(B, s.Di, s.n_in, s.Di) &&
                    gemv_bf16_ok(B, (int)s.fw, s.fw, s.fw);
  auto gemm = [&](const GemmOperands& op, const GemmOutput& out) {
    return b16 ? launch_gemm_bf16(op, out, GemmShape::Skinny, stream)
               : launch_gemm_f32(op, out, stream);
  };
  if (gemv) {
    GemvOut out{z, s.n_in, false};
    if (!s.share) {
      out.k_col = (int)s.k_col;
      out.v_col = (int)s.v_col;
      out.kvw = s.Hkv * s.dh;
      out.head_dim = s.dh;
      out.Hkv = s.Hkv;
      out.slots = kv->slots;
      out.ring_k = kv->k;
      out.ring_v = kv->v;
      out.pos = state->pos;
    }
    HYMBA_LAUNCH(HYMBA_STAGE_IN_PROJ,
                 launch_gemv_bf16(x, s.d, w->w_in, s.d, B, (int)s.n_in, s.d, out, stream));
  } else if (splitk) {
    // the same launch clears the x_proj accumulator
    GemmOperands op{x, s.d, nullptr, 0, B, w->w_in, s.d, B, (int)s.n_in, s.d};
    HYMBA_LAUNCH(HYMBA_STAGE_IN_PROJ,
                 launch_gemm_bf16_decode_in(op, z, s.n_in, s.share ? -1 : (int)s.k_col,
                                            (int)s.v_col, kv->k, kv->v, kv->slots, s.Hkv, s.dh,
                                            state->pos, xdbl, (int64_t)(cv.yacc - cv.xdbl) / 4,
                                            stream));
  } else {
    GemmOperands op{x, s.d, nullptr, 0, B, w->w_in, s.d, B, (int)s.n_in, s.d};
    GemmOutput out{EpiKind::Store, z, s.n_in, nullptr, 0, B, 0, nullptr};
    HYMBA_LAUNCH(HYMBA_STAGE_IN_PROJ, gemm(op, out));
    if (!s.share) {
      HYMBA_LAUNCH(HYMBA_STAGE_KV_WRITE,
                   launch_kv_write_decode(b16, z, s.n_in, (int)s.k_col, (int)s.v_col, kv->k,
                                          kv->v, kv->slots, state->pos, B, s.Hkv, s.dh, stream));
    }
  }
  {
    AttnDecodeParams ap{};
    ap.q = z;
    ap.q_row_stride = s.n_in;
    ap.k_meta = kv->k_meta;
    ap.v_meta = kv->v_meta;
    ap.k = kv->k;
    ap.v = kv->v;
    ap.slots = kv->slots;
    ap.pos = state->pos;
    ap.part = part;
    ap.nsplit = nsplit;
    ap.keys_per_split = decode_kps(s, span_max, B);
    ap.n_meta = M;
    ap.B = B;
    ap.Hq = s.Hq;
    ap.Hkv = s.Hkv;
    ap.head_dim = s.dh;
    ap.span_max = span_max;
    ap.scale = s.scale;
    if (stream_attn) {  // O straight into F; no split partials
      ap.o = f;
      ap.o_stride = s.fw;
    }
    HYMBA_LAUNCH(HYMBA_STAGE_ATTN, launch_attention_decode(b16, ap, stream));
  }
  // x_proj -> xdbl [B, R + 2N] fp32 (delta, B, C).
  {
    GemmOperands op{z + s.xs_col * s.es, s.n_in, nullptr, 0, B, w->w_x, s.Di, B, nx, s.Di};
    if (gemv) {
      HYMBA_LAUNCH(HYMBA_STAGE_XPROJ,
                   launch_gemv_bf16(z + s.xs_col * s.es, s.n_in, w->w_x, s.Di, B, nx, s.Di,
                                    GemvOut{xdbl, nx, true}, stream));
    } else if (splitk) {
      HYMBA_LAUNCH(HYMBA_STAGE_XPROJ, launch_gemm_bf16_splitk(op, xdbl, nx,
                                                              splitk_factor(B, nx, s.Di), stream));
    } else {
      GemmOutput out{EpiKind::StoreF32, xdbl, nx, nullptr, 0, 0, 0, nullptr};
      HYMBA_LAUNCH(HYMBA_STAGE_XPROJ, gemm(op, out));
    }
  }
  // dt_proj + softplus + one scan step + gate (h in place, pos += 1).
  {
    SsmStepParams sp{};
    sp.z = z;
    sp.z_stride = s.n_in;
    sp.xs_col = (int)s.xs_col;
    sp.g_col = (int)s.g_col;
    sp.xdbl = xdbl;
    sp.w_dt = w->w_dt;
    sp.dt_bias = w->dt_bias;
    sp.A = w->A;
    sp.D = w->D;
    sp.h = state->h;
    sp.y = f + s.qw * s.es;
    sp.y_stride = s.fw;
    sp.pos = state->pos;
    sp.B = B;
    sp.Di = s.Di;
    sp.N = s.N;
    sp.R = s.R;
    sp.heads = s.H2;
    HYMBA_LAUNCH(HYMBA_STAGE_SCAN,
                 s.H2 ? launch_ssm2_step(sp, stream) : launch_ssm_step(b16, sp, stream));
  }
  if (s.G) {  // group norm: merge the key splits first (if any), then normalise F
    if (!stream_attn) {
      HYMBA_LAUNCH(HYMBA_STAGE_NORM,
                   launch_decode_combine(b16, part, nsplit, f, s.fw, B, s.Hq, s.dh, stream));
    }
    HYMBA_LAUNCH(HYMBA_STAGE_NORM, launch_group_norm(b16, f, s.fw, B, (int)s.qw, s.Di,
                                                     w->beta_attn, w->beta_ssm, desc->rms_eps,
                                                     s.G, stream));
  } else if (stream_attn || nsplit > 8) {
    // more than 8 key splits: merge them over (q head, sequence) workgroups into F first;
    // the per-row merge would read every split of a row on one CU
    if (!stream_attn) {
      HYMBA_LAUNCH(HYMBA_STAGE_NORM,
                   launch_decode_combine(b16, part, nsplit, f, s.fw, B, s.Hq, s.dh, stream));
    }
    HYMBA_LAUNCH(HYMBA_STAGE_NORM, launch_fuse_norm(b16, f, s.fw, B, (int)s.qw, s.Di,
                                                    w->beta_attn, w->beta_ssm, desc->rms_eps,
                                                    stream));
  } else {
    HYMBA_LAUNCH(HYMBA_STAGE_NORM,
                 launch_decode_combine_norm(b16, part, nsplit, f, s.fw, B, s.Hq, s.dh, s.Di,
                                            w->beta_attn, w->beta_ssm, desc->rms_eps, stream));
  }
  {
    GemmOperands op{f, s.fw, nullptr, 0, B, w->w_out, s.fw, B, s.d, (int)s.fw};
    if (gemv) {
      HYMBA_LAUNCH(HYMBA_STAGE_OUT_PROJ,
                   launch_gemv_bf16(f, s.fw, w->w_out, s.fw, B, s.d, (int)s.fw,
                                    GemvOut{y, s.d, false}, stream));
    } else if (splitk) {
      const int64_t stride = (int64_t)B * s.d;
      HYMBA_LAUNCH(HYMBA_STAGE_OUT_PROJ,
                   launch_gemm_bf16_splitk(op, yacc, s.d, splitk_factor(B, s.d, (int)s.fw),
                                           stream, stride));
      HYMBA_LAUNCH(HYMBA_STAGE_MISC, launch_store_rows(true, yacc, y, B, s.d, stream,
                                                       out_proj_slices(s, B), stride));
    } else {
      GemmOutput out{EpiKind::Store, y, s.d, nullptr, 0, B, 0, nullptr};
      HYMBA_LAUNCH(HYMBA_STAGE_OUT_PROJ, gemm(op, out));
    }
  }
  return HYMBA_OK;
}

hymba_status hymba_op_gemm(int32_t dtype, const void* a, int64_t lda, const void* b, int64_t ldb,
                           void* c, int64_t ldc, int32_t c_dtype, int32_t m, int32_t n, int32_t k,
                           void* stream) {
  if (dtype != HYMBA_DTYPE_F32 && dtype != HYMBA_DTYPE_BF16) return HYMBA_ERR_INVALID_ARG;
  if (c_dtype != HYMBA_DTYPE_F32 && c_dtype != dtype) return HYMBA_ERR_INVALID_ARG;
  if (m < 0 || n < 0 || k < 0 || lda < k || ldb < k || ldc < n) return HYMBA_ERR_INVALID_ARG;
  if ((int64_t)m * n > 0 && (a == nullptr || b == nullptr || c == nullptr))
    return HYMBA_ERR_INVALID_ARG;
  if (k % 8 || lda % 8 || ldb % 8 || ldc % 4) return HYMBA_ERR_UNSUPPORTED;
  if (any_misaligned(a, b, c)) return HYMBA_ERR_ALIGNMENT;
  if ((int64_t)m * n == 0) return HYMBA_OK;
  GemmOperands op{a, lda, nullptr, 0, m, b, ldb, m, n, k};
  GemmOutput out{c_dtype == dtype ? EpiKind::Store : EpiKind::StoreF32, c, ldc, nullptr, 0, m, 0,
                 nullptr};
  hipError_t e = dtype == HYMBA_DTYPE_BF16
                     ? launch_gemm_bf16(op, out, GemmShape::Large, (hipStream_t)stream)
                     : launch_gemm_f32(op, out, (hipStream_t)stream);
  return e == hipSuccess ? HYMBA_OK : fail_hip(e);
}

size_t hymba_op_attn_workspace_bytes(int32_t dtype, int32_t n_meta, int32_t seq_len,
                                     int32_t batch, int32_t n_kv_heads, int32_t head_dim) {
  if (n_meta < 0 || seq_len < 0 || batch < 0 || n_kv_heads <= 0 || head_dim <= 0) return 0;
  if (dtype != HYMBA_DTYPE_BF16) return 0;
  return attention_vt_bytes(n_meta, seq_len, batch, n_kv_heads, head_dim);
}

hymba_status hymba_op_attn(int32_t dtype, const void* q, int64_t q_ld, const void* k,
                           const void* v, int64_t kv_ld, void* o, int64_t o_ld, int32_t n_meta,
                           int32_t seq_len, int32_t batch, int32_t n_q_heads,
                           int32_t n_kv_heads, int32_t head_dim, int32_t window, float scale,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != HYMBA_DTYPE_F32 && dtype != HYMBA_DTYPE_BF16) return HYMBA_ERR_INVALID_ARG;
  if (n_meta < 0 || seq_len < 0 || batch < 0 || window < 0 || n_q_heads <= 0 ||
      n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0)
    return HYMBA_ERR_INVALID_ARG;
  const bool b16 = dtype == HYMBA_DTYPE_BF16;
  if (b16 ? (head_dim != 64 && head_dim != 128) : (head_dim != 32 && head_dim != 64))
    return HYMBA_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)n_meta + (int64_t)batch * seq_len;
  if (rows >= (int64_t)1 << 31) return HYMBA_ERR_UNSUPPORTED;
  if (q_ld < (int64_t)n_q_heads * head_dim || kv_ld < (int64_t)n_kv_heads * head_dim ||
      o_ld < (int64_t)n_q_heads * head_dim)
    return HYMBA_ERR_INVALID_ARG;
  if (q_ld % 8 || kv_ld % 8 || o_ld % 8) return HYMBA_ERR_UNSUPPORTED;
  if (rows == 0) return HYMBA_OK;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return HYMBA_ERR_INVALID_ARG;
  if (any_misaligned(q, k, v, o, workspace)) return HYMBA_ERR_ALIGNMENT;
  const size_t need = hymba_op_attn_workspace_bytes(dtype, n_meta, seq_len, batch, n_kv_heads,
                                                    head_dim);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return HYMBA_ERR_WORKSPACE;
  const size_t es = b16 ? 2 : 4;
  AttnParams ap{};
  ap.q = q;
  ap.q_row_stride = q_ld;
  ap.k_meta = k;
  ap.v_meta = v;
  ap.meta_head_stride = head_dim;
  ap.meta_row_stride = kv_ld;
  ap.k_seq = (const char*)k + (size_t)n_meta * kv_ld * es;
  ap.v_seq = (const char*)v + (size_t)n_meta * kv_ld * es;
  ap.seq_batch_stride = (int64_t)seq_len * kv_ld;
  ap.seq_head_stride = head_dim;
  ap.seq_row_stride = kv_ld;
  ap.seq_slots = seq_len > 0 ? seq_len : 1;
  ap.o = o;
  ap.o_row_stride = o_ld;
  ap.n_meta = n_meta;
  ap.meta_rows = n_meta;
  ap.L = seq_len;
  ap.B = batch;
  ap.Hq = n_q_heads;
  ap.Hkv = n_kv_heads;
  ap.head_dim = head_dim;
  ap.window = window;
  ap.scale = scale > 0.f ? scale : 1.f / std::sqrt((float)head_dim);
  hipStream_t st = (hipStream_t)stream;
  const hipError_t e = b16 ? launch_attention_prefill_bf16_dl(ap, workspace, st)
                           : launch_attention_prefill_f32(ap, st);
  return e == hipSuccess ? HYMBA_OK : fail_hip(e);
}

size_t hymba_op_scan_workspace_bytes(int32_t dtype, int32_t n_meta, int32_t seq_len,
                                     int32_t batch, int32_t d_inner, int32_t d_state,
                                     int32_t dt_rank, int32_t chunk_tokens) {
  if (n_meta < 0 || seq_len < 0 || batch < 0 || d_inner <= 0 || chunk_tokens < 0) return 0;
  const int64_t rows = (int64_t)n_meta + (int64_t)batch * seq_len;
  if (dtype == HYMBA_DTYPE_BF16 && scan_chunk_supported(d_state, dt_rank, d_inner)) {
    // the post-meta state, then the chunk summaries of the larger launch
    const int64_t nsum = std::max(scan_summaries(chunk_tokens, 1, d_inner, n_meta),
                                  scan_summaries(chunk_tokens, batch, d_inner, seq_len));
    size_t need = (n_meta > 0 && batch > 0) ? align_up((size_t)d_inner * d_state * 4) : 0;
    need += align_up((size_t)nsum * d_inner * d_state * 4) + align_up((size_t)nsum * d_inner * 4);
    return need;
  }
  return (size_t)rows * d_inner * 4;
}

hymba_status hymba_op_scan(int32_t dtype, const void* z, int64_t z_ld, int32_t xs_col,
                           int32_t g_col, const void* delta, const float* bc, const void* w_dt,
                           const float* dt_bias, const float* A, const float* D, void* y,
                           int64_t y_ld, float* h_out, int32_t n_meta, int32_t seq_len,
                           int32_t batch, int32_t d_inner, int32_t d_state, int32_t dt_rank,
                           int32_t chunk_tokens, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (dtype != HYMBA_DTYPE_F32 && dtype != HYMBA_DTYPE_BF16) return HYMBA_ERR_INVALID_ARG;
  if (n_meta < 0 || seq_len < 0 || batch < 0 || d_inner <= 0 || dt_rank <= 0 || xs_col < 0 ||
      g_col < 0 || xs_col + d_inner > z_ld || g_col + d_inner > z_ld || y_ld < d_inner ||
      chunk_tokens < 0)
    return HYMBA_ERR_INVALID_ARG;
  if (d_state < 4 || d_state > 128 || (d_state & (d_state - 1)) || d_inner % 8 || dt_rank % 8 ||
      dt_rank > 512 || z_ld % 8 || xs_col % 8 || g_col % 8 || y_ld % 8 || chunk_tokens % 16)
    return HYMBA_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)n_meta + (int64_t)batch * seq_len;
  if (rows >= (int64_t)1 << 31) return HYMBA_ERR_UNSUPPORTED;
  const bool chunked = dtype == HYMBA_DTYPE_BF16 && scan_chunk_supported(d_state, dt_rank, d_inner);
  if (chunked && (!scan_chunks_ok(chunk_tokens, 1, d_inner, n_meta) ||
                  !scan_chunks_ok(chunk_tokens, batch, d_inner, seq_len)))
    return HYMBA_ERR_UNSUPPORTED;
  if (rows == 0 || batch == 0) return HYMBA_OK;
  if (z == nullptr || delta == nullptr || bc == nullptr || w_dt == nullptr || dt_bias == nullptr ||
      A == nullptr || D == nullptr || y == nullptr)
    return HYMBA_ERR_INVALID_ARG;
  if (any_misaligned(z, delta, bc, w_dt, y, h_out, workspace)) return HYMBA_ERR_ALIGNMENT;
  const size_t need = hymba_op_scan_workspace_bytes(dtype, n_meta, seq_len, batch, d_inner,
                                                    d_state, dt_rank, chunk_tokens);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return HYMBA_ERR_WORKSPACE;
  const bool b16 = dtype == HYMBA_DTYPE_BF16;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (chunked) {
    // the meta rows once, then every sequence from the state after them
    const size_t hm = (n_meta > 0) ? align_up((size_t)d_inner * d_state * 4) : 0;
    const int64_t nsum = std::max(scan_summaries(chunk_tokens, 1, d_inner, n_meta),
                                  scan_summaries(chunk_tokens, batch, d_inner, seq_len));
    ScanChunkParams cp{};
    cp.z = z;
    cp.z_stride = z_ld;
    cp.xs_col = xs_col;
    cp.g_col = g_col;
    cp.delta = delta;
    cp.bc = bc;
    cp.w_dt = w_dt;
    cp.dt_bias = dt_bias;
    cp.A = A;
    cp.D = D;
    cp.y = y;
    cp.y_stride = y_ld;
    cp.Di = d_inner;
    cp.N = d_state;
    cp.R = dt_rank;
    cp.hsum = (float*)ws_ptr(workspace, hm);
    cp.ssum = (float*)ws_ptr(workspace, hm + align_up((size_t)nsum * d_inner * d_state * 4));
    float* hmeta = (float*)workspace;
    if (n_meta > 0) {
      ScanChunkParams mp = cp;
      mp.row0 = 0;
      mp.T = n_meta;
      mp.B = 1;
      mp.h_out = hmeta;
      mp.chunk = scan_chunk_for(chunk_tokens, 1, d_inner, n_meta);
      mp.nchunks = scan_chunk_count(n_meta, mp.chunk);
      e = launch_scan_chunk(mp, st);
    }
    if (e == hipSuccess) {
      cp.row0 = n_meta;
      cp.T = seq_len;
      cp.B = batch;
      cp.h0 = n_meta > 0 ? hmeta : nullptr;
      cp.h_out = h_out;
      cp.chunk = scan_chunk_for(chunk_tokens, batch, d_inner, seq_len);
      cp.nchunks = scan_chunk_count(seq_len, cp.chunk);
      e = launch_scan_chunk(cp, st);
    }
  } else {
    ScanParams sp{};
    sp.z = z;
    sp.z_stride = z_ld;
    sp.xs_col = xs_col;
    sp.g_col = g_col;
    sp.dt = (const float*)workspace;
    sp.bc = bc;
    sp.A = A;
    sp.D = D;
    sp.y = y;
    sp.y_stride = y_ld;
    sp.h_out = h_out;
    sp.n_meta = n_meta;
    sp.L = seq_len;
    sp.B = batch;
    sp.Di = d_inner;
    sp.N = d_state;
    GemmOperands op{delta, dt_rank, nullptr, 0, (int)rows, w_dt, dt_rank, (int)rows, d_inner,
                    dt_rank};
    GemmOutput out{EpiKind::Softplus, workspace, d_inner, nullptr, 0, 0, 0, dt_bias};
    e = b16 ? launch_gemm_bf16(op, out, GemmShape::Narrow, st) : launch_gemm_f32(op, out, st);
    if (e == hipSuccess) e = launch_scan_prefill(b16, sp, st);
  }
  return e == hipSuccess ? HYMBA_OK : fail_hip(e);
}

hymba_status hymba_op_probe(int32_t kind, int32_t blocks, int32_t iters, const void* src,
                            size_t bytes, float* out, void* stream) {
  if (kind < 0 || kind > 3 || out == nullptr) return HYMBA_ERR_INVALID_ARG;
  if (kind != 2 && (blocks <= 0 || iters <= 0)) return HYMBA_ERR_INVALID_ARG;
  if (kind >= 2 && (src == nullptr || bytes == 0)) return HYMBA_ERR_INVALID_ARG;
  if (kind == 2 && bytes % 16) return HYMBA_ERR_UNSUPPORTED;
  if (kind == 3 && bytes < probe_operand_bytes()) return HYMBA_ERR_INVALID_ARG;
  if (any_misaligned(src, out)) return HYMBA_ERR_ALIGNMENT;
  hipError_t e = launch_probe(kind, blocks, iters, src, bytes, out, (hipStream_t)stream);
  return e == hipSuccess ? HYMBA_OK : fail_hip(e);
}

hymba_status hymba_op_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes % 16) return HYMBA_ERR_UNSUPPORTED;
  if (bytes > 0 && (src == nullptr || dst == nullptr)) return HYMBA_ERR_INVALID_ARG;
  if (any_misaligned(src, dst)) return HYMBA_ERR_ALIGNMENT;
  hipError_t e = launch_copy(src, dst, bytes, (hipStream_t)stream);
  return e == hipSuccess ? HYMBA_OK : fail_hip(e);
}


}  // extern "C"

// ----------------------------------------------------------------- block wrapper

namespace {

// Workspace of a block call: the layer's, then xn (the pre-normed rows), v (the
// pre-normed residual rows) and h (the FFN's hidden rows), all in the storage type.
struct BlockCarve {
  size_t layer, xn, v, h, acc, total;
};

// FFN down-projections over few rows (the meta rows of a prefill, a decode batch) split
// K = intermediate into fp32 partial slices, summed onto the residual by the row store.
bool ffn_down_splitk(const Shape& s, int inter) {
  return s.bf16 && inter % 256 == 0 && s.d % 64 == 0;
}

int ffn_down_slices(const Shape& s, int rows, int inter) {
  if (rows <= 0 || !ffn_down_splitk(s, inter)) return 0;
  return splitk_slices(inter, splitk_factor(rows, s.d, inter));
}

// The up-projection over few rows (a decode batch) likewise: K = d split into fp32
// partials, summed, passed through SiLU and rounded by the row store.
int ffn_up_slices(const Shape& s, int rows, int inter) {
  if (rows <= 0 || !s.bf16 || s.d % 256 != 0 || inter % 64 != 0) return 0;
  return splitk_slices(s.d, splitk_factor(rows, inter, s.d));
}

// few_rows: the rows that take the few-row down-projection (meta rows / the batch).
BlockCarve carve_block(const Shape& s, size_t layer_bytes, int64_t rows, int inter,
                       int few_rows) {
  BlockCarve c{};
  c.layer = 0;
  size_t off = align_up(layer_bytes);
  c.xn = off;
  off = align_up(off + (size_t)rows * s.d * s.es);
  c.v = off;
  off = align_up(off + (size_t)rows * s.d * s.es);
  c.h = off;
  off = align_up(off + (size_t)rows * inter * s.es);
  c.acc = off;
  off = align_up(off + std::max((size_t)ffn_down_slices(s, few_rows, inter) * s.d,
                                (size_t)ffn_up_slices(s, few_rows, inter) * inter) *
                           few_rows * 4);
  c.total = off;
  return c;
}

hymba_status check_block(const Shape& s, const hymba_block_weights* bw) {
  if (bw == nullptr || !bw->norm1 || !bw->norm2 || !bw->w_up || !bw->w_down ||
      bw->intermediate <= 0)
    return HYMBA_ERR_INVALID_ARG;
  if (bw->intermediate % 8) return HYMBA_ERR_UNSUPPORTED;
  if (any_misaligned(bw->norm1, bw->norm2, bw->w_up, bw->w_down)) return HYMBA_ERR_ALIGNMENT;
  (void)s;
  return HYMBA_OK;
}

// The FFN's two GEMMs.  ffn_up: h = SiLU(v W_up^T) over `rows` rows of v (contiguous).
// ffn_down: out += h W_down^T over `rows` rows of h, written to c (leading dimension ldc).
hipError_t ffn_gemm(const Shape& s, const GemmOperands& op, const GemmOutput& out, bool skinny,
                    hipStream_t stream) {
  return s.bf16 ? launch_gemm_bf16(op, out, skinny ? GemmShape::Skinny : GemmShape::Large, stream)
                : launch_gemm_f32(op, out, stream);
}

hymba_status ffn_up(const Shape& s, const hymba_block_weights* bw, const void* v, void* h,
                    int rows, bool skinny, float* acc, hipStream_t stream) {
  const int I = bw->intermediate;
  GemmOperands op{v, s.d, nullptr, 0, rows, bw->w_up, s.d, rows, I, s.d};
  const int slices = skinny && acc != nullptr ? ffn_up_slices(s, rows, I) : 0;
  if (slices > 0) {
    const int64_t stride = (int64_t)rows * I;
    HYMBA_LAUNCH(HYMBA_STAGE_BLOCK, launch_gemm_bf16_splitk(op, acc, I,
                                                           splitk_factor(rows, I, s.d), stream,
                                                           stride));
    HYMBA_LAUNCH(HYMBA_STAGE_BLOCK,
                 launch_store_rows(true, acc, h, rows, I, stream, slices, stride, false, true));
    return HYMBA_OK;
  }
  GemmOutput out{EpiKind::Silu, h, I, nullptr, 0, rows, 0, nullptr};
  HYMBA_LAUNCH(HYMBA_STAGE_BLOCK, ffn_gemm(s, op, out, skinny, stream));
  return HYMBA_OK;
}

// few: the rows are few (the meta rows, a decode batch); c is then contiguous (ldc = d)
// and, where ffn_down_splitk holds, K is split into fp32 partials at acc.
hymba_status ffn_down(const Shape& s, const hymba_block_weights* bw, const void* h, int rows,
                      void* c, int64_t ldc, bool few, float* acc, hipStream_t stream) {
  const int I = bw->intermediate;
  GemmOperands op{h, I, nullptr, 0, rows, bw->w_down, I, rows, s.d, I};
  const int slices = few ? ffn_down_slices(s, rows, I) : 0;
  if (slices > 0) {
    const int64_t stride = (int64_t)rows * s.d;
    HYMBA_LAUNCH(HYMBA_STAGE_BLOCK, launch_gemm_bf16_splitk(op, acc, s.d,
                                                           splitk_factor(rows, s.d, I), stream,
                                                           stride));
    HYMBA_LAUNCH(HYMBA_STAGE_BLOCK,
                 launch_store_rows(true, acc, c, rows, s.d, stream, slices, stride, true));
    return HYMBA_OK;
  }
  GemmOutput out{EpiKind::AddStore, c, ldc, nullptr, 0, rows, 0, nullptr};
  HYMBA_LAUNCH(HYMBA_STAGE_BLOCK, ffn_gemm(s, op, out, few, stream));
  return HYMBA_OK;
}

}  // namespace

extern "C" {

size_t hymba_block_workspace_bytes(const hymba_layer_desc* desc, int32_t intermediate,
                                   int32_t batch, int32_t seq_len, int32_t mode) {
  Shape s;
  if (make_shape(desc, s) != HYMBA_OK || intermediate <= 0 || intermediate % 8) return 0;
  if (mode != 0 && mode != 1) return 0;
  const size_t lb = hymba_layer_workspace_bytes(desc, batch, seq_len, mode);
  if (lb == 0) return 0;
  const int64_t rows = mode == 0 ? (int64_t)s.M + (int64_t)batch * seq_len : batch;
  return carve_block(s, lb, rows, intermediate, mode == 0 ? s.M : batch).total;
}

hymba_status hymba_block_prefill(const hymba_layer_desc* desc, const hymba_layer_weights* w,
                                 const hymba_block_weights* bw, const void* meta,
                                 const void* x, int32_t batch, int32_t seq_len,
                                 const hymba_kv* kv_in, hymba_kv* kv_out,
                                 hymba_ssm_state* state_out, void* y, void* y_meta,
                                 void* workspace, size_t workspace_bytes, void* stream_) {
  Shape s;
  hymba_status st = make_shape(desc, s);
  if (st != HYMBA_OK) return st;
  if ((st = check_block(s, bw)) != HYMBA_OK) return st;
  if (batch < 0 || seq_len < 0) return HYMBA_ERR_INVALID_ARG;
  const int B = batch, L = seq_len, M = s.M;
  const int64_t BL = (int64_t)B * L, rows = M + BL;
  if ((BL > 0 && (x == nullptr || y == nullptr)) || (M > 0 && meta == nullptr))
    return HYMBA_ERR_INVALID_ARG;
  if (any_misaligned(meta, x, y, y_meta, workspace)) return HYMBA_ERR_ALIGNMENT;
  const size_t lb = hymba_layer_workspace_bytes(desc, B, L, 0);
  const BlockCarve cv = carve_block(s, lb, rows, bw->intermediate, M);
  if (rows > 0 && (workspace == nullptr || workspace_bytes < cv.total)) return HYMBA_ERR_WORKSPACE;
  if (rows == 0) return HYMBA_OK;
  hipStream_t stream = (hipStream_t)stream_;
  const bool b16 = s.bf16;
  char* xn = ws_ptr(workspace, cv.xn);
  char* v = ws_ptr(workspace, cv.v);
  char* hbuf = ws_ptr(workspace, cv.h);
  const size_t rb = (size_t)s.d * s.es;  // bytes per row
  const float eps = desc->rms_eps;
  // pre-norm of [meta; X] into xn (meta rows first)
  HYMBA_LAUNCH(HYMBA_STAGE_BLOCK, launch_rms_norm_rows(b16, meta, s.d, xn, s.d, M, s.d,
                                                      bw->norm1, eps, stream));
  HYMBA_LAUNCH(HYMBA_STAGE_BLOCK, launch_rms_norm_rows(b16, x, s.d, xn + M * rb, s.d, (int)BL,
                                                      s.d, bw->norm1, eps, stream));
  // the layer on the normed rows: its outputs land in y / y_meta
  st = hymba_layer_prefill(desc, w, xn, xn + M * rb, batch, seq_len, kv_in, kv_out, state_out,
                           y, y_meta, workspace, lb, stream_);
  if (st != HYMBA_OK) return st;
  // residuals (u over y / y_meta) and the FFN's pre-norm into v (meta rows first)
  const int Mf = y_meta != nullptr ? M : 0;  // meta rows carried through the block
  HYMBA_LAUNCH(HYMBA_STAGE_BLOCK, launch_residual_norm(b16, meta, s.d, y_meta, s.d, v, s.d, Mf,
                                                      s.d, bw->norm2, eps, stream));
  HYMBA_LAUNCH(HYMBA_STAGE_BLOCK,
               launch_residual_norm(b16, x, s.d, y, s.d, v + Mf * rb, s.d, (int)BL, s.d,
                                    bw->norm2, eps, stream));
  // The up-projection takes the meta and X rows in one launch.  The down-projection's
  // output has d columns only, so its tiles over the X rows fill whole waves when B*L is a
  // multiple of the tile height; the meta rows take the few-row tiles in a launch of their
  // own instead of adding a nearly empty wave.
  if ((st = ffn_up(s, bw, v, hbuf, (int)(Mf + BL), false, nullptr, stream)) != HYMBA_OK)
    return st;
  const size_t hb = (size_t)bw->intermediate * s.es;  // bytes per row of h
  if ((st = ffn_down(s, bw, hbuf + Mf * hb, (int)BL, y, s.d, false, nullptr, stream)) !=
      HYMBA_OK)
    return st;
  return ffn_down(s, bw, hbuf, Mf, y_meta, s.d, true, (float*)ws_ptr(workspace, cv.acc), stream);
}

hymba_status hymba_block_decode(const hymba_layer_desc* desc, const hymba_layer_weights* w,
                                const hymba_block_weights* bw, const void* x, int32_t batch,
                                hymba_kv* kv, hymba_ssm_state* state, void* y,
                                void* workspace, size_t workspace_bytes, void* stream_) {
  Shape s;
  hymba_status st = make_shape(desc, s);
  if (st != HYMBA_OK) return st;
  if ((st = check_block(s, bw)) != HYMBA_OK) return st;
  if (batch < 0 || kv == nullptr) return HYMBA_ERR_INVALID_ARG;
  const int B = batch;
  if (B > 0 && (x == nullptr || y == nullptr)) return HYMBA_ERR_INVALID_ARG;
  if (any_misaligned(x, y, workspace)) return HYMBA_ERR_ALIGNMENT;
  const size_t lb = hymba_layer_workspace_bytes(desc, B, kv->slots, 1);
  const BlockCarve cv = carve_block(s, lb, B, bw->intermediate, B);
  if (B > 0 && (workspace == nullptr || workspace_bytes < cv.total)) return HYMBA_ERR_WORKSPACE;
  if (B == 0) return HYMBA_OK;
  hipStream_t stream = (hipStream_t)stream_;
  const bool b16 = s.bf16;
  char* xn = ws_ptr(workspace, cv.xn);
  char* v = ws_ptr(workspace, cv.v);
  char* hbuf = ws_ptr(workspace, cv.h);
  const float eps = desc->rms_eps;
  HYMBA_LAUNCH(HYMBA_STAGE_BLOCK, launch_rms_norm_rows(b16, x, s.d, xn, s.d, B, s.d, bw->norm1,
                                                      eps, stream));
  st = hymba_layer_decode(desc, w, xn, batch, kv, state, y, workspace, lb, stream_);
  if (st != HYMBA_OK) return st;
  HYMBA_LAUNCH(HYMBA_STAGE_BLOCK, launch_residual_norm(b16, x, s.d, y, s.d, v, s.d, B, s.d,
                                                      bw->norm2, eps, stream));
  if ((st = ffn_up(s, bw, v, hbuf, B, true, (float*)ws_ptr(workspace, cv.acc), stream)) !=
      HYMBA_OK)
    return st;
  return ffn_down(s, bw, hbuf, B, y, s.d, true, (float*)ws_ptr(workspace, cv.acc), stream);
}

}  // extern "C"

