// Host-side exercise of libhymba's argument validation and workspace sizing, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code (the device code is
// compiled as usual and never launched).  Every call below returns before the first HIP
// call, so this runs on a machine without a GPU.  Exit status 0 and no sanitizer report
// mean the host logic read and wrote only what it owns, with no undefined behaviour.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/hymba.h"

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      g_fail = 1;                                                      \
    }                                                                  \
  } while (0)

static hymba_layer_desc base_desc() {
  hymba_layer_desc d;
  std::memset(&d, 0, sizeof d);
  d.d_model = 2048;
  d.n_q_heads = 16;
  d.n_kv_heads = 4;
  d.head_dim = 128;
  d.d_inner = 4096;
  d.d_state = 16;
  d.dt_rank = 128;
  d.n_meta = 128;
  d.window = 0;
  d.kv_share = 0;
  d.dtype = HYMBA_DTYPE_BF16;
  d.rms_eps = 1e-6f;
  return d;
}

int main() {
  // fake, 256-byte aligned device addresses: nothing is dereferenced
  char* const p = (char*)(uintptr_t)4096;
  hymba_layer_weights w;
  const void** wp = (const void**)&w;
  for (size_t i = 0; i < sizeof w / sizeof(void*); ++i) wp[i] = p + 256 * i;

  // workspace sizing over a sweep of shapes, dtypes, variants and time chunks
  const int states[] = {4, 8, 16, 24, 32, 64, 128, 256};
  const int ranks[] = {8, 16, 64, 128, 512, 520};
  const int chunks[] = {0, 16, 48, 1024, 40, -16};
  const int windows[] = {0, 1, 33, 1024};
  size_t total = 0;
  for (int dt = 0; dt < 2; ++dt)
    for (int si = 0; si < 8; ++si)
      for (int ri = 0; ri < 6; ++ri)
        for (int ci = 0; ci < 6; ++ci)
          for (int wi = 0; wi < 4; ++wi) {
            hymba_layer_desc d = base_desc();
            d.dtype = dt ? HYMBA_DTYPE_BF16 : HYMBA_DTYPE_F32;
            d.head_dim = dt ? 128 : 64;
            d.d_state = states[si];
            d.dt_rank = ranks[ri];
            d.scan_chunk = chunks[ci];
            d.window = windows[wi];
            d.ssm_heads = (si == 2 && ri == 0) ? 64 : 0;
            d.norm_group = (wi == 2) ? 128 : 0;
            const int Bs[] = {0, 1, 3, 8, 128};
            const int Ls[] = {0, 1, 17, 2048, 32768};
            for (int bi = 0; bi < 5; ++bi)
              for (int li = 0; li < 5; ++li)
                for (int mode = -1; mode < 4; ++mode) {
                  total += hymba_layer_workspace_bytes(&d, Bs[bi], Ls[li], mode);
                  total += hymba_block_workspace_bytes(&d, 5632, Bs[bi], Ls[li], mode);
                }
            total += hymba_layer_workspace_bytes(&d, -1, 10, 0);
            total += hymba_op_scan_workspace_bytes(d.dtype, d.n_meta, 777, 3, d.d_inner, d.d_state,
                                                   d.dt_rank, chunks[ci]);
            total += hymba_op_attn_workspace_bytes(d.dtype, d.n_meta, 777, 3, 4, d.head_dim);
          }
  EXPECT(total > 0);

  // prefill validation: every case stops before a launch
  hymba_layer_desc d = base_desc();
  EXPECT(hymba_layer_prefill(nullptr, &w, p, p, 1, 4, nullptr, nullptr, nullptr, p, nullptr, p,
                             1 << 20, nullptr) == HYMBA_ERR_INVALID_ARG);
  EXPECT(hymba_layer_prefill(&d, nullptr, p, p, 1, 4, nullptr, nullptr, nullptr, p, nullptr, p,
                             1 << 20, nullptr) == HYMBA_ERR_INVALID_ARG);
  EXPECT(hymba_layer_prefill(&d, &w, p, p, 1, 4, nullptr, nullptr, nullptr, p, nullptr, p, 100,
                             nullptr) == HYMBA_ERR_WORKSPACE);
  EXPECT(hymba_layer_prefill(&d, &w, p + 2, p, 1, 4, nullptr, nullptr, nullptr, p, nullptr, p,
                             1 << 20, nullptr) == HYMBA_ERR_ALIGNMENT);
  EXPECT(hymba_layer_prefill(&d, &w, p, p, 2, 1 << 30, nullptr, nullptr, nullptr, p, nullptr, p,
                             100, nullptr) == HYMBA_ERR_UNSUPPORTED);
  hymba_kv kv = {p, p, p, p, 16, 0};
  EXPECT(hymba_layer_prefill(&d, &w, p, p, 1, 64, nullptr, &kv, nullptr, p, nullptr, p, 100,
                             nullptr) == HYMBA_ERR_INVALID_ARG);
  kv.is_ring = 1;
  EXPECT(hymba_layer_prefill(&d, &w, p, p, 1, 64, nullptr, &kv, nullptr, p, nullptr, p, 100,
                             nullptr) == HYMBA_ERR_WORKSPACE);
  hymba_layer_desc bad = base_desc();
  bad.d_state = 24;
  EXPECT(hymba_layer_prefill(&bad, &w, p, p, 1, 4, nullptr, nullptr, nullptr, p, nullptr, p,
                             1 << 20, nullptr) == HYMBA_ERR_UNSUPPORTED);
  bad = base_desc();
  bad.scan_chunk = 16;  // 2048 tokens in 16-token chunks: more than 65 chunks
  EXPECT(hymba_layer_prefill(&bad, &w, p, p, 1, 2048, nullptr, nullptr, nullptr, p, nullptr, p,
                             1 << 20, nullptr) == HYMBA_ERR_UNSUPPORTED);

  // decode validation, the allocation-free variant's size limit, the ring fill
  hymba_layer_desc dd = base_desc();
  dd.window = 1024;
  hymba_kv ring = {p, p, p, p, 1024, 1};
  hymba_ssm_state st = {(float*)p, (int32_t*)p};
  EXPECT(hymba_layer_decode(&dd, &w, p, 2, nullptr, &st, p, p, 1 << 30, nullptr) ==
         HYMBA_ERR_INVALID_ARG);
  EXPECT(hymba_layer_decode(&dd, &w, p, 2, &ring, &st, p, p, 16, nullptr) == HYMBA_ERR_WORKSPACE);
  EXPECT(hymba_layer_decode_static(&dd, &w, p, 100000, &ring, &st, p, nullptr) ==
         HYMBA_ERR_WORKSPACE);
  EXPECT(hymba_layer_decode_static(&dd, &w, p, 2, nullptr, &st, p, nullptr) ==
         HYMBA_ERR_INVALID_ARG);
  hymba_kv full = {p, p, p, p, 64, 0};
  EXPECT(hymba_kv_ring_fill(&full, &ring, 2, 100, 8, 4, 128, HYMBA_DTYPE_BF16, nullptr) ==
         HYMBA_ERR_INVALID_ARG);
  EXPECT(hymba_kv_ring_fill(&full, &ring, 2, 64, 8, 4, 12, HYMBA_DTYPE_BF16, nullptr) ==
         HYMBA_ERR_UNSUPPORTED);

  // single-step entry points
  EXPECT(hymba_op_gemm(7, p, 64, p, 64, p, 64, 1, 4, 4, 64, nullptr) == HYMBA_ERR_INVALID_ARG);
  EXPECT(hymba_op_scan(HYMBA_DTYPE_BF16, p, 1024, 0, 512, p, (const float*)p, p,
                       (const float*)p, (const float*)p, (const float*)p, p, 512, nullptr, 8, 64,
                       2, 512, 16, 64, 24, nullptr, 0, nullptr) == HYMBA_ERR_UNSUPPORTED);
  EXPECT(hymba_op_attn(HYMBA_DTYPE_BF16, p, 1024, p, p, 256, p, 1024, 8, 64, 2, 6, 4, 128, 0,
                       0.f, p, 0, nullptr) == HYMBA_ERR_INVALID_ARG);

  // status strings and the ABI version
  for (int s = -1; s < 8; ++s) EXPECT(hymba_status_str(s) != nullptr);
  EXPECT(hymba_abi_version() == HYMBA_ABI_VERSION);
  double ms = 0.0;
  int32_t n = 0;
  EXPECT(hymba_timer_read(-1, &ms, &n) == HYMBA_ERR_INVALID_ARG);
  EXPECT(hymba_timer_read(0, nullptr, &n) == HYMBA_ERR_INVALID_ARG);

  if (g_fail) return 1;
  std::printf("host checks passed (%zu bytes of workspace sized)\n", total);
  return 0;
}
