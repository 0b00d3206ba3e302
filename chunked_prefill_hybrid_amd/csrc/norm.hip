// Token-wise row ops of the hybrid batch (they run on the flattened C+B rows, like every
// non-attention op of a hybrid iteration: junupark.xyz notes on Sarathi-Serve, "The effect of mixed
// batching", step 1).
//
//   norm_rows:  v = resid + sum of a GEMM's split partials (in a fixed order), optionally stored
//               (the residual stream h1), then RMSNorm v / sqrt(mean(v^2) + eps) * g or LayerNorm
//               (v - mean) / sqrt(var + eps) * g + b (biased variance).  Rows past the batch are
//               written as zeros so the next GEMM computes on zeros there.
//   ffn_act:    the FFN activation silu(gate) * up or gelu(up) from split partials of the up GEMM.
//   resid_sum:  out = resid + sum of a GEMM's split partials (the layer output y = h1 + FFN).
// One workgroup per row (norms), 4-element vectors, float32 sums.
#include "kernels.h"

namespace sarathi {
namespace {

constexpr int kThreads = 256;

template <typename T> __device__ __forceinline__ void load4(const T *p, float *v);
template <> __device__ __forceinline__ void load4<float>(const float *p, float *v) {
  const float4 f = *reinterpret_cast<const float4 *>(p);
  v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
}
template <> __device__ __forceinline__ void load4<bf16_t>(const bf16_t *p, float *v) {
  const uint2 u = *reinterpret_cast<const uint2 *>(p);
  v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
  v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
}
template <typename T> __device__ __forceinline__ void store4(T *p, const float *v);
template <> __device__ __forceinline__ void store4<float>(float *p, const float *v) {
  *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <> __device__ __forceinline__ void store4<bf16_t>(bf16_t *p, const float *v) {
  uint2 u;
  u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  *reinterpret_cast<uint2 *>(p) = u;
}

template <int NT> __device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += red[w];
  return t;
}

constexpr int kMaxSplits = 8;   // split partials a consumer sums (the planner never makes more)
// A norm row is handled by one workgroup of NT threads: 1024 (16 waves, so that the ~300 rows of a
// batch still keep several waves of memory requests per SIMD in flight) while the rows' workgroups
// all fit on the GPU at once, else 512.  A compute unit holds 32 waves, so 1024-thread workgroups for
// more than kNormWideRows rows would run in two rounds.
#ifndef SARATHI_NORM_WIDE_ROWS
#define SARATHI_NORM_WIDE_ROWS 512
#endif
constexpr int kNormWideRows = SARATHI_NORM_WIDE_ROWS;
template <int NT> struct NormGeom {
  static constexpr int kPieces = kMaxHidden / (4 * NT);   // 4-element pieces per thread
  static_assert(4 * NT * kPieces == kMaxHidden, "row width limit");
};

// v[0..3] += sum_s part[s][off..off+3] in split order; every split's load is issued before its add
// so a thread keeps several loads in flight.
__device__ __forceinline__ void add_splits(const float *part, int splits, size_t slice, size_t off,
                                           float *v) {
  float p[kMaxSplits][4];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < splits) load4<float>(part + s * slice + off, p[s]);
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < splits) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += p[s][e];
    }
}

// One row per workgroup: the row stays in registers (up to kRowPieces 4-element pieces per thread),
// so the norm needs one read of its inputs.
template <typename T> __device__ __forceinline__ float round_to(float v);
template <> __device__ __forceinline__ float round_to<float>(float v) { return v; }
template <> __device__ __forceinline__ float round_to<bf16_t>(float v) {
  return __uint_as_float((uint32_t)f32_to_bf16(v) << 16);
}

// sum_out: the sum v stored in float32; sum_lo: v rounded to the output type, stored row-major, and
// the norm then taken of the rounded values (a layer's output y and the next layer's norm 1 in one
// pass, with the same result as storing y and normalising it in a separate launch).
template <typename Tres, typename Tout, bool LN, int NT>
__global__ __launch_bounds__(NT) void norm_rows(const Tres *resid, const float *part,
                                                      int splits, float *sum_out, Tout *sum_lo,
                                                      const float *g, const float *b, Tout *out,
                                                      int H, int rows, float eps, int kmajor_rows,
                                                      int kmajor_shift) {
  constexpr int kRowPieces = NormGeom<NT>::kPieces;
  __shared__ float red[NT / 64];
  const int r = blockIdx.x;
  // Element c of this row: row-major, or k-tile-major (tiles of 2^kmajor_shift columns by
  // kmajor_rows rows each).
  auto at = [&](int c) -> Tout * {
    return kmajor_rows ? out + (((size_t)(c >> kmajor_shift) * kmajor_rows + r) << kmajor_shift) +
                             (c & ((1 << kmajor_shift) - 1))
                       : out + (size_t)r * H + c;
  };
  if (r >= rows) {
    const float z[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = threadIdx.x * 4; c < H; c += NT * 4) store4<Tout>(at(c), z);
    return;
  }
  const size_t slice = (size_t)rows * H, row_off = (size_t)r * H;
  const int nch = (H / 4 - threadIdx.x + NT - 1) / NT;   // chunks of this thread
  float v[kRowPieces][4];
#pragma unroll
  for (int i = 0; i < kRowPieces; ++i)
    if (i < nch) load4<Tres>(resid + row_off + (threadIdx.x + i * NT) * 4, v[i]);
  if (splits > 0) {
#pragma unroll
    for (int i = 0; i < kRowPieces; ++i)
      if (i < nch) add_splits(part, splits, slice, row_off + (threadIdx.x + i * NT) * 4, v[i]);
  }
  float s1 = 0.f;
#pragma unroll
  for (int i = 0; i < kRowPieces; ++i)
    if (i < nch) {
      if (sum_out) store4<float>(sum_out + row_off + (threadIdx.x + i * NT) * 4, v[i]);
      if (sum_lo) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[i][e] = round_to<Tout>(v[i][e]);
        store4<Tout>(sum_lo + row_off + (threadIdx.x + i * NT) * 4, v[i]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) s1 += LN ? v[i][e] : v[i][e] * v[i][e];
    }
  s1 = block_sum<NT>(s1, red);
  float mean = 0.f, ms;
  if (LN) {
    mean = s1 / (float)H;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < kRowPieces; ++i)
      if (i < nch) {
#pragma unroll
        for (int e = 0; e < 4; ++e) q += (v[i][e] - mean) * (v[i][e] - mean);
      }
    ms = block_sum<NT>(q, red) / (float)H;
  } else {
    ms = s1 / (float)H;
  }
  const float rstd = 1.0f / sqrtf(ms + eps);
#pragma unroll
  for (int i = 0; i < kRowPieces; ++i)
    if (i < nch) {
      const int c = (threadIdx.x + i * NT) * 4;
      float w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[e] = (v[i][e] - mean) * rstd * g[c + e];
        if (LN) w[e] += b[c + e];
      }
      store4<Tout>(at(c), w);
    }
}

// Elementwise over [rows, cols]: one 4-element chunk per thread.
template <typename Tout>
__global__ __launch_bounds__(kThreads) void resid_sum(const float *resid, const float *part,
                                                      int splits, Tout *out, int rows, int cols) {
  const size_t n4 = (size_t)rows * cols / 4;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= n4) return;
  const size_t off = idx * 4;
  float v[4];
  load4<float>(resid + off, v);
  add_splits(part, splits, (size_t)rows * cols, off, v);
  store4<Tout>(out + off, v);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }
__device__ __forceinline__ float gelu_f(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

template <typename Tout, bool GATED>
__global__ __launch_bounds__(kThreads) void ffn_act(const float *part, int splits, Tout *out,
                                                    int rows, int F, int col0, int ld, int kmajor,
                                                    int rows_alloc) {
  const size_t n4 = (size_t)rows * F / 4;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= n4) return;
  const int r = (int)(idx / (F / 4)), c = (int)(idx % (F / 4)) * 4;
  const int n_part = GATED ? 2 * F : F;
  const size_t slice = (size_t)rows * n_part, off = (size_t)r * n_part + c;
  float a[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
  add_splits(part, splits, slice, off, a);
  if (GATED) add_splits(part, splits, slice, off + F, u);
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = GATED ? silu_f(a[e]) * u[e] : gelu_f(a[e]);
  store4<Tout>(out + mat_index(r, col0 + c, ld, kmajor, rows_alloc), v);   // 4 columns within one k-tile
}

template <typename Tres, typename Tout, bool LN, int NT>
hipError_t run_norm_nt(const void *resid, const float *part, int splits, float *sum_out, void *sum_lo,
                       const float *g, const float *b, void *out, int H, int rows, int rows_alloc,
                       float eps, int kmajor_rows, int kmajor_shift, hipStream_t s) {
  hipLaunchKernelGGL((norm_rows<Tres, Tout, LN, NT>), dim3(rows_alloc), dim3(NT), 0, s,
                     static_cast<const Tres *>(resid), part, splits, sum_out,
                     static_cast<Tout *>(sum_lo), g, b, static_cast<Tout *>(out), H, rows, eps,
                     kmajor_rows, kmajor_shift);
  return hipGetLastError();
}

template <typename Tres, typename Tout>
hipError_t run_norm(bool ln, const void *resid, const float *part, int splits, float *sum_out,
                    void *sum_lo, const float *g, const float *b, void *out, int H, int rows,
                    int rows_alloc, float eps, int kmajor_rows, int kmajor_shift, hipStream_t s) {
  const bool wide = rows_alloc <= kNormWideRows;
#define SARATHI_NORM(LN, NT)                                                                    \
  return run_norm_nt<Tres, Tout, LN, NT>(resid, part, splits, sum_out, sum_lo, g, b, out, H, rows, \
                                         rows_alloc, eps, kmajor_rows, kmajor_shift, s)
  if (ln) {
    if (wide) SARATHI_NORM(true, 1024); else SARATHI_NORM(true, 512);
  } else {
    if (wide) SARATHI_NORM(false, 1024); else SARATHI_NORM(false, 512);
  }
#undef SARATHI_NORM
}

}  // namespace

hipError_t launch_norm_rows(int res_type, int out_type, bool layernorm, const void *resid,
                            const float *part, int splits, float *sum_out, void *sum_lo,
                            const float *g, const float *b, void *out, int H, int rows,
                            int rows_alloc, float eps, int kmajor, hipStream_t s) {
  if (rows_alloc <= 0) return hipSuccess;
  if (splits > kMaxSplits || H > kMaxHidden || H % 4) return hipErrorInvalidValue;
  if (kmajor != 0 && kmajor != 32 && kmajor != 64) return hipErrorInvalidValue;
  if (kmajor && H % 64) return hipErrorInvalidValue;
  if (sum_out && sum_lo) return hipErrorInvalidValue;
  const int km = kmajor ? rows_alloc : 0, ks = kmajor == 32 ? 5 : 6;
#define SARATHI_RUN_NORM(TR, TO) \
  return run_norm<TR, TO>(layernorm, resid, part, splits, sum_out, sum_lo, g, b, out, H, rows, rows_alloc, \
                          eps, km, ks, s)
  if (res_type == kF32 && out_type == kF32) SARATHI_RUN_NORM(float, float);
  if (res_type == kBF16 && out_type == kBF16) SARATHI_RUN_NORM(bf16_t, bf16_t);
  if (res_type == kF32 && out_type == kBF16) SARATHI_RUN_NORM(float, bf16_t);
#undef SARATHI_RUN_NORM
  return hipErrorInvalidValue;
}

hipError_t launch_ffn_act(int out_type, bool gated, const float *part, int splits, void *out,
                          int rows, int F, int col0, int ld, int kmajor, int rows_alloc, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (splits > kMaxSplits || F % 4 || col0 % 4 || col0 < 0 || col0 + F > ld) return hipErrorInvalidValue;
  if (kmajor && ((kmajor != 32 && kmajor != 64) || F % kmajor || col0 % kmajor || ld % kmajor ||
                 rows > rows_alloc))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(((size_t)rows * F / 4 + kThreads - 1) / kThreads));
#define SARATHI_ACT(T, GT) \
  hipLaunchKernelGGL((ffn_act<T, GT>), grid, dim3(kThreads), 0, s, part, splits, static_cast<T *>(out), \
                     rows, F, col0, ld, kmajor, rows_alloc)
  if (out_type == kF32) {
    if (gated) SARATHI_ACT(float, true); else SARATHI_ACT(float, false);
  } else {
    if (gated) SARATHI_ACT(bf16_t, true); else SARATHI_ACT(bf16_t, false);
  }
#undef SARATHI_ACT
  return hipGetLastError();
}

hipError_t launch_resid_sum(int out_type, const float *resid, const float *part, int splits,
                            void *out, int rows, int cols, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (splits > kMaxSplits) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(((size_t)rows * cols / 4 + kThreads - 1) / kThreads));
  if (out_type == kF32)
    hipLaunchKernelGGL(resid_sum<float>, grid, dim3(kThreads), 0, s, resid, part, splits,
                       static_cast<float *>(out), rows, cols);
  else
    hipLaunchKernelGGL(resid_sum<bf16_t>, grid, dim3(kThreads), 0, s, resid, part, splits,
                       static_cast<bf16_t *>(out), rows, cols);
  return hipGetLastError();
}

}  // namespace sarathi
