// Fusion epilogue, cache writes and small utility kernels of the hybrid-head layer.
//
// Fusion source: "Hymba: A Hybrid-head Architecture for Small Language Models"
// (outta.ai summary), Design formulation, total fusion equation (each branch
// normalised, rescaled by a learnable vector, then combined before out_proj) and the
// Chinese summary's 核心架构 / 实现细节 (RMSNorm per branch, 0.5 average).  The
// branches have different widths, so F = 0.5 [beta_a rms(O) ; beta_s rms(Y_ssm)] is
// the concatenation that out_proj consumes.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

template <typename T>
struct Vec8;
template <>
struct Vec8<bf16> {
  static __device__ __forceinline__ void load(const bf16* p, float v[8]) {
    const bf16x8 x = *(const bf16x8*)p;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
  }
  static __device__ __forceinline__ void store(bf16* p, const float v[8]) {
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (bf16)v[e];
    *(bf16x8*)p = x;
  }
};
template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float v[8]) {
    const floatx4 a = *(const floatx4*)p, b = *(const floatx4*)(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  }
  static __device__ __forceinline__ void store(float* p, const float v[8]) {
    *(floatx4*)p = floatx4{v[0], v[1], v[2], v[3]};
    *(floatx4*)(p + 4) = floatx4{v[4], v[5], v[6], v[7]};
  }
};

// Block-wide sums of two values (up to 1024 threads).
__device__ __forceinline__ void block_sum2(float& a, float& b) {
  __shared__ float ra[16], rb[16];
  a = wave_sum(a);
  b = wave_sum(b);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, nw = blockDim.x >> 6;
  if (l == 0) {
    ra[w] = a;
    rb[w] = b;
  }
  __syncthreads();
  a = 0.f;
  b = 0.f;
  for (int i = 0; i < nw; ++i) {
    a += ra[i];
    b += rb[i];
  }
  __syncthreads();
}

// Normalise one row of F in place: [0, wa) by the attention rms, [wa, wa + ws) by the
// SSM rms.  wa and ws are multiples of 8.
template <typename T>
__device__ __forceinline__ void norm_row(T* f, int wa, int ws, const float* ba, const float* bs,
                                         float eps) {
  float sa = 0.f, ss = 0.f;
  const int step = blockDim.x * 8;
  for (int i = threadIdx.x * 8; i < wa + ws; i += step) {
    float v[8];
    Vec8<T>::load(f + i, v);
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) q = fmaf(v[e], v[e], q);
    if (i < wa)
      sa += q;
    else
      ss += q;
  }
  block_sum2(sa, ss);
  const float ia = 0.5f * rsqrtf(sa / (float)wa + eps);
  const float is = 0.5f * rsqrtf(ss / (float)ws + eps);
  for (int i = threadIdx.x * 8; i < wa + ws; i += step) {
    float v[8];
    Vec8<T>::load(f + i, v);
    const bool att = i < wa;
    const float* beta = att ? ba + i : bs + (i - wa);
    const float sc = att ? ia : is;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * sc * beta[e];
    Vec8<T>::store(f + i, v);
  }
}

}  // namespace

template <typename T>
__global__ __launch_bounds__(256) void fuse_norm_kernel(T* f, int64_t stride, int wa, int ws,
                                                        const float* ba, const float* bs, float eps) {
  norm_row<T>(f + (int64_t)blockIdx.x * stride, wa, ws, ba, bs, eps);
}

// The same for rows of at most 256 x 4 chunks of 8 (the decode rows: 6144 values): every
// chunk and its beta values are loaded at once and the row stays in registers between the
// sums and the scaled store (one memory round trip instead of a read, a re-read and the
// beta loads in turn).
constexpr int kNormChunks = 4;
template <typename T>
__global__ __launch_bounds__(256) void fuse_norm_regs_kernel(T* f, int64_t stride, int wa, int ws,
                                                             const float* ba, const float* bs,
                                                             float eps) {
  T* row = f + (int64_t)blockIdx.x * stride;
  const int nch = (wa + ws) / 8;
  float v[kNormChunks][8], bt[kNormChunks][8];
#pragma unroll
  for (int c = 0; c < kNormChunks; ++c) {
    const int ch = threadIdx.x + c * 256;
    if (ch < nch) {
      const int i = ch * 8;
      Vec8<T>::load(row + i, v[c]);
      const float* beta = i < wa ? ba + i : bs + (i - wa);
#pragma unroll
      for (int e = 0; e < 8; ++e) bt[c][e] = beta[e];
    }
  }
  float sa = 0.f, ss = 0.f;
#pragma unroll
  for (int c = 0; c < kNormChunks; ++c) {
    const int ch = threadIdx.x + c * 256;
    if (ch >= nch) break;
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) q = fmaf(v[c][e], v[c][e], q);
    if (ch * 8 < wa)
      sa += q;
    else
      ss += q;
  }
  block_sum2(sa, ss);
  const float ia = 0.5f * rsqrtf(sa / (float)wa + eps);
  const float is = 0.5f * rsqrtf(ss / (float)ws + eps);
#pragma unroll
  for (int c = 0; c < kNormChunks; ++c) {
    const int ch = threadIdx.x + c * 256;
    if (ch >= nch) break;
    const float sc = ch * 8 < wa ? ia : is;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[c][e] = v[c][e] * sc * bt[c][e];
    Vec8<T>::store(row + ch * 8, v[c]);
  }
}

hipError_t launch_fuse_norm(bool bf16_, void* f, int64_t f_stride, int rows, int wa, int ws,
                            const float* beta_a, const float* beta_s, float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (wa + ws <= 256 * kNormChunks * 8) {
    if (bf16_)
      fuse_norm_regs_kernel<bf16><<<dim3(rows), dim3(256), 0, s>>>((bf16*)f, f_stride, wa, ws,
                                                                   beta_a, beta_s, eps);
    else
      fuse_norm_regs_kernel<float><<<dim3(rows), dim3(256), 0, s>>>((float*)f, f_stride, wa, ws,
                                                                    beta_a, beta_s, eps);
    return hipGetLastError();
  }
  if (bf16_)
    fuse_norm_kernel<bf16><<<dim3(rows), dim3(256), 0, s>>>((bf16*)f, f_stride, wa, ws, beta_a,
                                                            beta_s, eps);
  else
    fuse_norm_kernel<float><<<dim3(rows), dim3(256), 0, s>>>((float*)f, f_stride, wa, ws, beta_a,
                                                             beta_s, eps);
  return hipGetLastError();
}

// Block wrapper norms: one workgroup per row, 8 elements per thread per pass.
template <typename T>
__global__ __launch_bounds__(256) void rms_norm_rows_kernel(const T* in, int64_t in_ld, T* out,
                                                            int64_t out_ld, int d, const float* g,
                                                            float eps) {
  const T* r = in + (int64_t)blockIdx.x * in_ld;
  T* o = out + (int64_t)blockIdx.x * out_ld;
  float sq = 0.f, dummy = 0.f;
  for (int i = threadIdx.x * 8; i < d; i += 256 * 8) {
    float v[8];
    Vec8<T>::load(r + i, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) sq = fmaf(v[e], v[e], sq);
  }
  block_sum2(sq, dummy);
  const float sc = rsqrtf(sq / (float)d + eps);
  for (int i = threadIdx.x * 8; i < d; i += 256 * 8) {
    float v[8];
    Vec8<T>::load(r + i, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * sc * g[i + e];
    Vec8<T>::store(o + i, v);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void residual_norm_kernel(const T* x, int64_t x_ld, T* y,
                                                            int64_t y_ld, T* v, int64_t v_ld,
                                                            int d, const float* g, float eps) {
  const T* xr = x + (int64_t)blockIdx.x * x_ld;
  T* yr = y + (int64_t)blockIdx.x * y_ld;
  T* vr = v + (int64_t)blockIdx.x * v_ld;
  float sq = 0.f, dummy = 0.f;
  for (int i = threadIdx.x * 8; i < d; i += 256 * 8) {
    float a[8], b[8];
    Vec8<T>::load(xr + i, a);
    Vec8<T>::load(yr + i, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      b[e] = to_f32(from_f32<T>(a[e] + b[e]));  // u as stored
      sq = fmaf(b[e], b[e], sq);
    }
    Vec8<T>::store(yr + i, b);
  }
  block_sum2(sq, dummy);  // (its barrier also orders the u stores before the reads below)
  const float sc = rsqrtf(sq / (float)d + eps);
  for (int i = threadIdx.x * 8; i < d; i += 256 * 8) {
    float u[8];
    Vec8<T>::load(yr + i, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = u[e] * sc * g[i + e];
    Vec8<T>::store(vr + i, u);
  }
}

hipError_t launch_rms_norm_rows(bool bf16_, const void* in, int64_t in_ld, void* out,
                                int64_t out_ld, int rows, int d, const float* g, float eps,
                                hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d % 8) return hipErrorInvalidValue;
  if (bf16_)
    rms_norm_rows_kernel<bf16><<<dim3(rows), dim3(256), 0, s>>>((const bf16*)in, in_ld,
                                                                (bf16*)out, out_ld, d, g, eps);
  else
    rms_norm_rows_kernel<float><<<dim3(rows), dim3(256), 0, s>>>((const float*)in, in_ld,
                                                                 (float*)out, out_ld, d, g, eps);
  return hipGetLastError();
}

hipError_t launch_residual_norm(bool bf16_, const void* x, int64_t x_ld, void* y, int64_t y_ld,
                                void* v, int64_t v_ld, int rows, int d, const float* g,
                                float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d % 8) return hipErrorInvalidValue;
  if (bf16_)
    residual_norm_kernel<bf16><<<dim3(rows), dim3(256), 0, s>>>(
        (const bf16*)x, x_ld, (bf16*)y, y_ld, (bf16*)v, v_ld, d, g, eps);
  else
    residual_norm_kernel<float><<<dim3(rows), dim3(256), 0, s>>>(
        (const float*)x, x_ld, (float*)y, y_ld, (float*)v, v_ld, d, g, eps);
  return hipGetLastError();
}

// Group normalisation of one row of F per workgroup.  A thread holds 8 channels; the
// g / 8 threads of a group are adjacent lanes of one wave (g <= 512), so the group's
// mean and then its variance about the mean are xor-shuffle sums over them.  The groups
// never straddle the branch boundary (g divides wa).
template <typename T>
__global__ __launch_bounds__(256) void group_norm_kernel(T* f, int64_t stride, int wa, int ws,
                                                         const float* ba, const float* bs,
                                                         float eps, int g) {
  T* row = f + (int64_t)blockIdx.x * stride;
  const int tpg = g / 8;  // threads per group
  const float inv_g = 1.f / (float)g;
  for (int i = threadIdx.x * 8; i < wa + ws; i += 256 * 8) {
    float v[8];
    Vec8<T>::load(row + i, v);
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sum += v[e];
    for (int off = 1; off < tpg; off <<= 1) sum += __shfl_xor(sum, off, 64);
    const float mean = sum * inv_g;
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] -= mean;
      sq = fmaf(v[e], v[e], sq);
    }
    for (int off = 1; off < tpg; off <<= 1) sq += __shfl_xor(sq, off, 64);
    const float sc = 0.5f * rsqrtf(sq * inv_g + eps);
    const bool att = i < wa;
    const float* beta = att ? ba + i : bs + (i - wa);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * sc * beta[e];
    Vec8<T>::store(row + i, v);
  }
}

hipError_t launch_group_norm(bool bf16_, void* f, int64_t f_stride, int rows, int wa, int ws,
                             const float* beta_a, const float* beta_s, float eps, int g,
                             hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (g < 8 || g > 512 || (g & (g - 1)) || wa % g || ws % g) return hipErrorInvalidValue;
  if (bf16_)
    group_norm_kernel<bf16><<<dim3(rows), dim3(256), 0, s>>>((bf16*)f, f_stride, wa, ws, beta_a,
                                                             beta_s, eps, g);
  else
    group_norm_kernel<float><<<dim3(rows), dim3(256), 0, s>>>((float*)f, f_stride, wa, ws,
                                                              beta_a, beta_s, eps, g);
  return hipGetLastError();
}

// Row factors of the deferred branch norms.  Blocks [0, nfac) take 256 rows each, one
// row per thread (consecutive threads read consecutive rows of each partial column);
// blocks from nfac on scale one of the first scale_rows rows of F in place, recomputing
// that row's two factors from its partials.
// Sum of n partials r[0], r[ld], ...: eight independent loads in flight at a time.
__device__ __forceinline__ float col_sum(const float* r, int64_t ld, int n) {
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int i = 0;
  for (; i + 8 <= n; i += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = r[(i + u) * ld];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += v[u];
  }
  for (; i < n; ++i) acc[0] += r[i * ld];
  return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}
__device__ __forceinline__ void row_sums(const float* r, int64_t ld, int na, int ns, float& sa,
                                         float& ss) {
  sa = col_sum(r, ld, na);
  ss = col_sum(r + na * ld, ld, ns);
}

__global__ __launch_bounds__(256) void row_factors_kernel(const float* ssp, int64_t ld, int na,
                                                          int ns, int rows, int wa, int ws,
                                                          float eps, float* fac, bf16* f,
                                                          int64_t f_stride, int nfac) {
  if ((int)blockIdx.x < nfac) {
    const int row = blockIdx.x * 256 + threadIdx.x;
    if (row >= rows) return;
    float sa, ss;
    row_sums(ssp + row, ld, na, ns, sa, ss);
    fac[2 * (int64_t)row] = 0.5f * rsqrtf(sa / (float)wa + eps);
    fac[2 * (int64_t)row + 1] = 0.5f * rsqrtf(ss / (float)ws + eps);
    return;
  }
  const int row = blockIdx.x - nfac;
  float sa, ss;
  row_sums(ssp + row, ld, na, ns, sa, ss);
  const float fa = 0.5f * rsqrtf(sa / (float)wa + eps);
  const float fs = 0.5f * rsqrtf(ss / (float)ws + eps);
  bf16* fr = f + row * f_stride;
  for (int i = threadIdx.x * 8; i < wa + ws; i += 256 * 8) {
    float v[8];
    Vec8<bf16>::load(fr + i, v);
    const float sc = i < wa ? fa : fs;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= sc;
    Vec8<bf16>::store(fr + i, v);
  }
}

hipError_t launch_row_factors(const float* ssp, int64_t ssp_ld, int na, int ns, int rows,
                              int wa, int ws, float eps, float* fac, void* f, int64_t f_stride,
                              int scale_rows, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (wa % 8 || ws % 8 || scale_rows > rows) return hipErrorInvalidValue;
  const int nfac = (rows + 255) / 256;
  row_factors_kernel<<<dim3(nfac + scale_rows), dim3(256), 0, s>>>(
      ssp, ssp_ld, na, ns, rows, wa, ws, eps, fac, (bf16*)f, f_stride, nfac);
  return hipGetLastError();
}

// Decode: merge the split partials (o, m, l) of every q head of sequence b into O,
// round O to the storage type (as the prefill path stores O), then normalise the row
// with the SSM half that the SSM step already wrote.  One block of 256 threads per
// sequence; each thread owns up to kCombineChunks 8-element chunks of the row and keeps
// them in registers between the two block sums and the scaled store.
constexpr int kCombineChunks = 4;

// Merge of any number of splits, G at a time: a group's loads are all issued before the
// first use (one memory round trip per group; the partials come from other CUs' L2
// through the last-level cache), and the running sums are rescaled when a group raises
// the running maximum (the same online rule as the attention kernels).
template <typename T, int G = 16>
__device__ __forceinline__ void combine_chunk(const float* ph, int nsplit, int rec, int d0,
                                              float v[8]) {
  float mx = -INFINITY, lsum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += G) {
    float m[G], l[G];
    floatx4 a[G], c[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (s0 + j < nsplit) {
        const float* r = ph + (s0 + j) * rec;
        const floatx4 ml = *(const floatx4*)(r + rec - 4);
        m[j] = ml[0];
        l[j] = ml[1];
        a[j] = *(const floatx4*)(r + d0);
        c[j] = *(const floatx4*)(r + d0 + 4);
      } else {
        m[j] = -INFINITY;
        l[j] = 0.f;
        a[j] = c[j] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
    float gm = mx;
#pragma unroll
    for (int j = 0; j < G; ++j) gm = fmaxf(gm, m[j]);
    if (gm == -INFINITY) continue;  // every split so far is empty
    const float sc = mx == -INFINITY ? 0.f : __expf(mx - gm);
    lsum *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= sc;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float w = m[j] == -INFINITY ? 0.f : __expf(m[j] - gm);  // empty split: 0
      lsum = fmaf(l[j], w, lsum);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = fmaf(a[j][e], w, v[e]);
        v[4 + e] = fmaf(c[j][e], w, v[4 + e]);
      }
    }
    mx = gm;
  }
  const float inv = 1.f / lsum;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = to_f32(from_f32<T>(v[e] * inv));
}

// Same merge for at most S splits: every load is issued before the first use, so the
// chunk costs one memory round trip.
template <typename T, int S>
__device__ __forceinline__ void combine_chunk_fixed(const float* ph, int nsplit, int rec, int d0,
                                                    float v[8]) {
  float m[S], l[S];
  floatx4 a[S], c[S];
#pragma unroll
  for (int sp = 0; sp < S; ++sp) {
    if (sp < nsplit) {
      const float* r = ph + sp * rec;
      const floatx4 ml = *(const floatx4*)(r + rec - 4);
      m[sp] = ml[0];
      l[sp] = ml[1];
      a[sp] = *(const floatx4*)(r + d0);
      c[sp] = *(const floatx4*)(r + d0 + 4);
    } else {
      m[sp] = -INFINITY;
      l[sp] = 0.f;
      a[sp] = c[sp] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < S; ++sp) mx = fmaxf(mx, m[sp]);
  float lsum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = 0.f;
#pragma unroll
  for (int sp = 0; sp < S; ++sp) {
    const float w = m[sp] == -INFINITY ? 0.f : __expf(m[sp] - mx);  // empty split: 0
    lsum = fmaf(l[sp], w, lsum);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = fmaf(a[sp][e], w, v[e]);
      v[4 + e] = fmaf(c[sp][e], w, v[4 + e]);
    }
  }
  const float inv = 1.f / lsum;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = to_f32(from_f32<T>(v[e] * inv));
}

template <typename T>
__global__ __launch_bounds__(256) void decode_combine_norm_kernel(const float* part, int nsplit,
                                                                 T* f, int64_t stride, int Hq,
                                                                 int dh, int ws, const float* ba,
                                                                 const float* bs, float eps) {
  const int b = blockIdx.x;
  T* row = f + (int64_t)b * stride;
  const int wa = Hq * dh, nch = (wa + ws) / 8, rec = dh + 4;
  float v[kCombineChunks][8];
  float sa = 0.f, ss = 0.f;
  // the SSM half's chunks are plain loads: issue them first, so they overlap the merges'
  // round trips
#pragma unroll
  for (int c = 0; c < kCombineChunks; ++c) {
    const int ch = threadIdx.x + c * 256;
    if (ch < nch && ch * 8 >= wa) Vec8<T>::load(row + ch * 8, v[c]);
  }
#pragma unroll
  for (int c = 0; c < kCombineChunks; ++c) {
    const int ch = threadIdx.x + c * 256;
    if (ch >= nch) break;
    const int i = ch * 8;
    if (i < wa) {
      const int h = i / dh;
      const float* ph = part + ((int64_t)b * Hq + h) * nsplit * rec;
      if (nsplit <= 8)
        combine_chunk_fixed<T, 8>(ph, nsplit, rec, i - h * dh, v[c]);
      else
        combine_chunk<T>(ph, nsplit, rec, i - h * dh, v[c]);
    }
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) q = fmaf(v[c][e], v[c][e], q);
    if (i < wa)
      sa += q;
    else
      ss += q;
  }
  block_sum2(sa, ss);
  const float ia = 0.5f * rsqrtf(sa / (float)wa + eps);
  const float is = 0.5f * rsqrtf(ss / (float)ws + eps);
#pragma unroll
  for (int c = 0; c < kCombineChunks; ++c) {
    const int ch = threadIdx.x + c * 256;
    if (ch >= nch) break;
    const int i = ch * 8;
    const bool att = i < wa;
    const float* beta = att ? ba + i : bs + (i - wa);
    const float sc = att ? ia : is;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[c][e] = v[c][e] * sc * beta[e];
    Vec8<T>::store(row + i, v[c]);
  }
}

// Rows wider than 256 x kCombineChunks x 8 elements: merge into F first (same thread
// layout as the norm pass reads it back), then normalise in place.
template <typename T>
__global__ __launch_bounds__(256) void decode_combine_wide_kernel(const float* part, int nsplit,
                                                                 T* f, int64_t stride, int Hq,
                                                                 int dh, int ws, const float* ba,
                                                                 const float* bs, float eps) {
  const int b = blockIdx.x;
  T* row = f + (int64_t)b * stride;
  const int wa = Hq * dh, rec = dh + 4;
  for (int i = threadIdx.x * 8; i < wa; i += 256 * 8) {
    const int h = i / dh;
    float v[8];
    combine_chunk<T>(part + ((int64_t)b * Hq + h) * nsplit * rec, nsplit, rec, i - h * dh, v);
    Vec8<T>::store(row + i, v);
  }
  __syncthreads();
  norm_row<T>(row, wa, ws, ba, bs, eps);
}

// Merge of the split partials into O, one workgroup per (q head, sequence): the head's
// dh / 8 chunks of 8 dims times SL = 256 / (dh / 8) split lanes.  Lane sl of a chunk
// merges splits sl, sl + SL, ... (online rule), the SL partial merges meet in LDS and the
// chunk's first lane merges them and stores O rounded to the storage type.  Spreads the
// read of the partials over B x Hq workgroups (one workgroup per sequence reads all of a
// row's partials on one CU).
template <typename T, int DH>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* part, int nsplit, T* f,
                                                          int64_t stride, int Hq) {
  constexpr int CPH = DH / 8, SL = 256 / CPH;
  __shared__ float s_m[SL][CPH], s_l[SL][CPH];
  __shared__ float s_v[SL][CPH][8];
  const int h = blockIdx.x, b = blockIdx.y;
  const int c = threadIdx.x % CPH, sl = threadIdx.x / CPH;
  const int rec = DH + 4;
  const float* ph = part + ((int64_t)b * Hq + h) * nsplit * rec;
  float mx = -INFINITY, lsum = 0.f, v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = 0.f;
#pragma unroll 4
  for (int sp = sl; sp < nsplit; sp += SL) {
    const float* r = ph + sp * rec;
    const floatx4 ml = *(const floatx4*)(r + rec - 4);
    const floatx4 x0 = *(const floatx4*)(r + c * 8), x1 = *(const floatx4*)(r + c * 8 + 4);
    const float m = ml[0];
    if (m == -INFINITY) continue;  // empty split
    const float nm = fmaxf(mx, m);
    const float so = mx == -INFINITY ? 0.f : __expf(mx - nm), w = __expf(m - nm);
    lsum = fmaf(ml[1], w, lsum * so);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = fmaf(x0[e], w, v[e] * so);
      v[4 + e] = fmaf(x1[e], w, v[4 + e] * so);
    }
    mx = nm;
  }
  s_m[sl][c] = mx;
  s_l[sl][c] = lsum;
#pragma unroll
  for (int e = 0; e < 8; ++e) s_v[sl][c][e] = v[e];
  __syncthreads();
  if (sl != 0) return;
  float gm = -INFINITY;
  for (int j = 0; j < SL; ++j) gm = fmaxf(gm, s_m[j][c]);
  float tl = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  for (int j = 0; j < SL; ++j) {
    const float m = s_m[j][c];
    if (m == -INFINITY) continue;
    const float w = __expf(m - gm);
    tl = fmaf(s_l[j][c], w, tl);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = fmaf(s_v[j][c][e], w, o[e]);
  }
  const float inv = 1.f / tl;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] *= inv;
  Vec8<T>::store(f + (int64_t)b * stride + h * DH + c * 8, o);
}

hipError_t launch_decode_combine(bool bf16_, const float* part, int nsplit, void* f,
                                 int64_t f_stride, int B, int Hq, int head_dim, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const dim3 grid(Hq, B), blk(256);
  if (bf16_) {
    if (head_dim == 128)
      decode_merge_kernel<bf16, 128><<<grid, blk, 0, s>>>(part, nsplit, (bf16*)f, f_stride, Hq);
    else if (head_dim == 64)
      decode_merge_kernel<bf16, 64><<<grid, blk, 0, s>>>(part, nsplit, (bf16*)f, f_stride, Hq);
    else
      return hipErrorInvalidValue;
  } else {
    if (head_dim == 64)
      decode_merge_kernel<float, 64><<<grid, blk, 0, s>>>(part, nsplit, (float*)f, f_stride, Hq);
    else if (head_dim == 32)
      decode_merge_kernel<float, 32><<<grid, blk, 0, s>>>(part, nsplit, (float*)f, f_stride, Hq);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_combine_norm(bool bf16_, const float* part, int nsplit, void* f,
                                      int64_t f_stride, int B, int Hq, int head_dim, int ws,
                                      const float* beta_a, const float* beta_s, float eps,
                                      hipStream_t s) {
  if (B == 0) return hipSuccess;
  const bool narrow = Hq * head_dim + ws <= 256 * kCombineChunks * 8;
  if (bf16_) {
    if (narrow)
      decode_combine_norm_kernel<bf16><<<dim3(B), dim3(256), 0, s>>>(
          part, nsplit, (bf16*)f, f_stride, Hq, head_dim, ws, beta_a, beta_s, eps);
    else
      decode_combine_wide_kernel<bf16><<<dim3(B), dim3(256), 0, s>>>(
          part, nsplit, (bf16*)f, f_stride, Hq, head_dim, ws, beta_a, beta_s, eps);
  } else {
    if (narrow)
      decode_combine_norm_kernel<float><<<dim3(B), dim3(256), 0, s>>>(
          part, nsplit, (float*)f, f_stride, Hq, head_dim, ws, beta_a, beta_s, eps);
    else
      decode_combine_wide_kernel<float><<<dim3(B), dim3(256), 0, s>>>(
          part, nsplit, (float*)f, f_stride, Hq, head_dim, ws, beta_a, beta_s, eps);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------- cache writes
// One thread per 16-byte chunk.  Chunk index space: [meta rows | B * n_last rows] x
// Hkv x (head_dim * sizeof(T) / 16) x {K, V}.
template <typename T>
__global__ __launch_bounds__(256) void kv_write_prefill_kernel(const T* z, int64_t zs, int k_col,
                                                               int v_col, T* k_meta, T* v_meta,
                                                               T* k, T* v, int slots, int n_meta,
                                                               int L, int B, int Hkv, int dh,
                                                               int n_last) {
  constexpr int EPC = 16 / sizeof(T);
  const int cpr = dh / EPC;
  const int64_t total = (int64_t)(n_meta + (int64_t)B * n_last) * Hkv * cpr * 2;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  int64_t r = gid;
  const int which = (int)(r % 2);
  r /= 2;
  const int dc = (int)(r % cpr);
  r /= cpr;
  const int g = (int)(r % Hkv);
  r /= Hkv;
  const int64_t rr = r;  // row in [meta | B * n_last]
  int64_t zrow;
  T* dst;
  if (rr < n_meta) {
    zrow = rr;
    dst = (which ? v_meta : k_meta) + ((int64_t)g * n_meta + rr) * dh;
  } else {
    const int64_t q = rr - n_meta;
    const int b = (int)(q / n_last);
    const int p = L - n_last + (int)(q % n_last);
    zrow = n_meta + (int64_t)b * L + p;
    dst = (which ? v : k) + (((int64_t)b * Hkv + g) * slots + (p % slots)) * dh;
  }
  const T* src = z + zrow * zs + (which ? v_col : k_col) + g * dh + dc * EPC;
  *(u32x4*)(dst + dc * EPC) = *(const u32x4*)src;
}

hipError_t launch_kv_write_prefill(bool bf16_, const void* z, int64_t z_stride, int k_col,
                                   int v_col, void* k_meta, void* v_meta, void* k, void* v,
                                   int slots, int n_meta, int L, int B, int Hkv, int head_dim,
                                   hipStream_t s) {
  const int n_last = L < slots ? L : slots;
  const int esz = bf16_ ? 2 : 4;
  const int64_t total = (int64_t)(n_meta + (int64_t)B * n_last) * Hkv * (head_dim * esz / 16) * 2;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (bf16_)
    kv_write_prefill_kernel<bf16><<<dim3(blocks), dim3(256), 0, s>>>(
        (const bf16*)z, z_stride, k_col, v_col, (bf16*)k_meta, (bf16*)v_meta, (bf16*)k, (bf16*)v,
        slots, n_meta, L, B, Hkv, head_dim, n_last);
  else
    kv_write_prefill_kernel<float><<<dim3(blocks), dim3(256), 0, s>>>(
        (const float*)z, z_stride, k_col, v_col, (float*)k_meta, (float*)v_meta, (float*)k,
        (float*)v, slots, n_meta, L, B, Hkv, head_dim, n_last);
  return hipGetLastError();
}

// One 16-byte piece per thread: rows [meta entries (when copying them) | B * n_last
// positions] x Hkv heads x head_dim pieces x {K, V}.
template <typename T>
__global__ __launch_bounds__(256) void kv_ring_fill_kernel(const T* sk, const T* sv, int sslots,
                                                           const T* skm, const T* svm, T* dk,
                                                           T* dv, int dslots, T* dkm, T* dvm,
                                                           int n_meta_copy, int n_meta, int L,
                                                           int n_last, int B, int Hkv, int dh) {
  constexpr int EPC = 16 / sizeof(T);
  const int cpr = dh / EPC;
  const int64_t total = (int64_t)(n_meta_copy + (int64_t)B * n_last) * Hkv * cpr * 2;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  int64_t r = gid;
  const int which = (int)(r % 2);
  r /= 2;
  const int dc = (int)(r % cpr);
  r /= cpr;
  const int g = (int)(r % Hkv);
  r /= Hkv;
  const T* src;
  T* dst;
  if (r < n_meta_copy) {
    const int64_t o = ((int64_t)g * n_meta + r) * dh;
    src = (which ? svm : skm) + o;
    dst = (which ? dvm : dkm) + o;
  } else {
    const int64_t q = r - n_meta_copy;
    const int b = (int)(q / n_last);
    const int p = L - n_last + (int)(q % n_last);
    src = (which ? sv : sk) + (((int64_t)b * Hkv + g) * sslots + (p % sslots)) * dh;
    dst = (which ? dv : dk) + (((int64_t)b * Hkv + g) * dslots + (p % dslots)) * dh;
  }
  *(u32x4*)(dst + dc * EPC) = *(const u32x4*)(src + dc * EPC);
}

hipError_t launch_kv_ring_fill(bool bf16_, const void* src_k, const void* src_v, int src_slots,
                               const void* src_k_meta, const void* src_v_meta, void* dst_k,
                               void* dst_v, int dst_slots, void* dst_k_meta, void* dst_v_meta,
                               bool copy_meta, int n_meta, int L, int n_last, int B, int Hkv,
                               int head_dim, hipStream_t s) {
  const int esz = bf16_ ? 2 : 4;
  const int nm = copy_meta ? n_meta : 0;
  const int64_t total = (int64_t)(nm + (int64_t)B * n_last) * Hkv * (head_dim * esz / 16) * 2;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (bf16_)
    kv_ring_fill_kernel<bf16><<<dim3(blocks), dim3(256), 0, s>>>(
        (const bf16*)src_k, (const bf16*)src_v, src_slots, (const bf16*)src_k_meta,
        (const bf16*)src_v_meta, (bf16*)dst_k, (bf16*)dst_v, dst_slots, (bf16*)dst_k_meta,
        (bf16*)dst_v_meta, nm, n_meta, L, n_last, B, Hkv, head_dim);
  else
    kv_ring_fill_kernel<float><<<dim3(blocks), dim3(256), 0, s>>>(
        (const float*)src_k, (const float*)src_v, src_slots, (const float*)src_k_meta,
        (const float*)src_v_meta, (float*)dst_k, (float*)dst_v, dst_slots, (float*)dst_k_meta,
        (float*)dst_v_meta, nm, n_meta, L, n_last, B, Hkv, head_dim);
  return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(256) void kv_write_decode_kernel(const T* z, int64_t zs, int k_col,
                                                              int v_col, T* k, T* v, int slots,
                                                              const int32_t* pos, int B, int Hkv,
                                                              int dh) {
  constexpr int EPC = 16 / sizeof(T);
  const int cpr = dh / EPC;
  const int64_t total = (int64_t)B * Hkv * cpr * 2;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  int64_t r = gid;
  const int which = (int)(r % 2);
  r /= 2;
  const int dc = (int)(r % cpr);
  r /= cpr;
  const int g = (int)(r % Hkv);
  const int b = (int)(r / Hkv);
  const int slot = max(pos[b], 0) % slots;
  const T* src = z + (int64_t)b * zs + (which ? v_col : k_col) + g * dh + dc * EPC;
  T* dst = (which ? v : k) + (((int64_t)b * Hkv + g) * slots + slot) * dh + dc * EPC;
  *(u32x4*)dst = *(const u32x4*)src;
}

hipError_t launch_kv_write_decode(bool bf16_, const void* z, int64_t z_stride, int k_col,
                                  int v_col, void* k, void* v, int slots, const int32_t* pos,
                                  int B, int Hkv, int head_dim, hipStream_t s) {
  const int esz = bf16_ ? 2 : 4;
  const int64_t total = (int64_t)B * Hkv * (head_dim * esz / 16) * 2;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (bf16_)
    kv_write_decode_kernel<bf16><<<dim3(blocks), dim3(256), 0, s>>>(
        (const bf16*)z, z_stride, k_col, v_col, (bf16*)k, (bf16*)v, slots, pos, B, Hkv, head_dim);
  else
    kv_write_decode_kernel<float><<<dim3(blocks), dim3(256), 0, s>>>(
        (const float*)z, z_stride, k_col, v_col, (float*)k, (float*)v, slots, pos, B, Hkv,
        head_dim);
  return hipGetLastError();
}

// ----------------------------------------------------------------- utilities
__global__ void fill_i32_kernel(int32_t* p, int32_t value, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = value;
}

hipError_t launch_fill_i32(int32_t* p, int32_t value, int n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  fill_i32_kernel<<<dim3((n + 255) / 256), dim3(256), 0, s>>>(p, value, n);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_f32_kernel(floatx4* p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    p[i] = floatx4{0.f, 0.f, 0.f, 0.f};
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 4096);
  zero_f32_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>((floatx4*)p, n4);
  return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(256) void store_rows_kernel(const float* acc, T* y, int64_t n,
                                                         int nslices, int64_t slice_stride,
                                                         bool accumulate, bool silu) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  floatx4 a = *(const floatx4*)(acc + i);
  for (int p = 1; p < nslices; ++p) {
    const floatx4 b = *(const floatx4*)(acc + p * slice_stride + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] += b[e];
  }
  if (accumulate) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] += to_f32(y[i + e]);
  }
  if (silu) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = silu_f(a[e]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) y[i + e] = from_f32<T>(a[e]);
}

hipError_t launch_store_rows(bool bf16_, const float* acc, void* y, int B, int d, hipStream_t s,
                             int nslices, int64_t slice_stride, bool accumulate, bool silu) {
  const int64_t n = (int64_t)B * d;
  if (n == 0) return hipSuccess;
  if (nslices < 1 || (nslices > 1 && (slice_stride < n || slice_stride % 4 != 0)))
    return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((n / 4 + 255) / 256);
  if (bf16_)
    store_rows_kernel<bf16><<<dim3(blocks), dim3(256), 0, s>>>(acc, (bf16*)y, n, nslices,
                                                               slice_stride, accumulate, silu);
  else
    store_rows_kernel<float><<<dim3(blocks), dim3(256), 0, s>>>(acc, (float*)y, n, nslices,
                                                                slice_stride, accumulate, silu);
  return hipGetLastError();
}

// Plain copy, 16 bytes per lane, grid-stride.  Used to calibrate HBM traffic counters.
__global__ __launch_bounds__(256) void copy16_kernel(const u32x4* src, u32x4* dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = src[i];
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  copy16_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>((const u32x4*)src, (u32x4*)dst, n);
  return hipGetLastError();
}

}  // namespace hymba
