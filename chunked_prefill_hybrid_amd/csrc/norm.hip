// Token-wise norms of the hybrid batch (run on the flattened C+B rows, like every non-attention op of
// a hybrid iteration: junupark.xyz notes on Sarathi-Serve, "The effect of mixed batching", step 1).
// RMSNorm: x / sqrt(mean(x^2) + eps) * g.  LayerNorm: (x - mean) / sqrt(var + eps) * g + b with the
// biased variance.  One workgroup per row, 16-byte packets, float32 sums; rows past the batch are
// written as zeros so the GEMM that consumes them computes on zeros.
#include "kernels.h"

namespace sarathi {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) t += red[w];
  return t;
}

template <typename Tin, typename Tout, bool LN>
__global__ __launch_bounds__(kThreads) void norm_rows(const Tin *x, const float *g, const float *b,
                                                      Tout *out, int H, int rows, float eps) {
  __shared__ float red[kThreads / 64];
  const int r = blockIdx.x;
  constexpr int Ei = Packet<Tin>::E, Eo = Packet<Tout>::E;
  Tout *o = out + (size_t)r * H;
  if (r >= rows) {
    for (int c = threadIdx.x * Eo; c < H; c += kThreads * Eo) st16(o + c, make_uint4(0, 0, 0, 0));
    return;
  }
  const Tin *xr = x + (size_t)r * H;
  float s = 0.f;
  for (int c = threadIdx.x * Ei; c < H; c += kThreads * Ei) {
    float v[Ei];
    unpack<Tin>(ld16(xr + c), v);
#pragma unroll
    for (int e = 0; e < Ei; ++e) s += LN ? v[e] : v[e] * v[e];
  }
  s = block_sum(s, red);
  float mean = 0.f, ms;
  if (LN) {
    mean = s / (float)H;
    float q = 0.f;
    for (int c = threadIdx.x * Ei; c < H; c += kThreads * Ei) {
      float v[Ei];
      unpack<Tin>(ld16(xr + c), v);
#pragma unroll
      for (int e = 0; e < Ei; ++e) q += (v[e] - mean) * (v[e] - mean);
    }
    ms = block_sum(q, red) / (float)H;
  } else {
    ms = s / (float)H;
  }
  const float rstd = 1.0f / sqrtf(ms + eps);
  for (int c = threadIdx.x * Eo; c < H; c += kThreads * Eo) {
    float v[Eo];
#pragma unroll
    for (int e0 = 0; e0 < Eo; e0 += Ei) unpack<Tin>(ld16(xr + c + e0), v + e0);
#pragma unroll
    for (int e = 0; e < Eo; ++e) {
      v[e] = (v[e] - mean) * rstd * g[c + e];
      if (LN) v[e] += b[c + e];
    }
    st16(o + c, pack<Tout>(v));
  }
}

template <typename Tin, typename Tout>
hipError_t run(bool ln, const void *x, const float *g, const float *b, void *out, int H, int rows,
               int rows_alloc, float eps, hipStream_t s) {
  if (ln)
    hipLaunchKernelGGL((norm_rows<Tin, Tout, true>), dim3(rows_alloc), dim3(kThreads), 0, s,
                       static_cast<const Tin *>(x), g, b, static_cast<Tout *>(out), H, rows, eps);
  else
    hipLaunchKernelGGL((norm_rows<Tin, Tout, false>), dim3(rows_alloc), dim3(kThreads), 0, s,
                       static_cast<const Tin *>(x), g, b, static_cast<Tout *>(out), H, rows, eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norm(int in_type, int out_type, bool layernorm, const void *x, const float *g,
                       const float *b, void *out, int H, int rows, int rows_alloc, float eps,
                       hipStream_t s) {
  if (rows_alloc <= 0) return hipSuccess;
  if (in_type == kF32 && out_type == kF32)
    return run<float, float>(layernorm, x, g, b, out, H, rows, rows_alloc, eps, s);
  if (in_type == kBF16 && out_type == kBF16)
    return run<bf16_t, bf16_t>(layernorm, x, g, b, out, H, rows, rows_alloc, eps, s);
  if (in_type == kF32 && out_type == kBF16)
    return run<float, bf16_t>(layernorm, x, g, b, out, H, rows, rows_alloc, eps, s);
  return hipErrorInvalidValue;
}

}  // namespace sarathi
