// Small utility kernels: zero-filling rows of a matrix, and widening a storage matrix to float32
// (used to hand intermediates to callers that inspect them).
#include "kernels.h"

namespace sarathi {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void zero_rows(T *p, int ld, int cols, int row0) {
  T *row = p + (size_t)(row0 + blockIdx.x) * ld;
  for (int c = threadIdx.x; c < cols; c += blockDim.x) row[c] = from_f32<T>(0.f);
}

template <typename T>
__global__ __launch_bounds__(256) void widen_rows(const T *src, int ld_src, float *dst, int ld_dst,
                                              int cols) {
  const T *s = src + (size_t)blockIdx.x * ld_src;
  float *d = dst + (size_t)blockIdx.x * ld_dst;
  for (int c = threadIdx.x; c < cols; c += blockDim.x) d[c] = to_f32(s[c]);
}

template <typename T>
__global__ __launch_bounds__(256) void widen_kmajor_rows(const T *src, int w, int rows_alloc,
                                                     float *dst, int ld_dst, int cols) {
  const int r = blockIdx.x;
  float *d = dst + (size_t)r * ld_dst;
  for (int c = threadIdx.x; c < cols; c += blockDim.x)
    d[c] = to_f32(src[((size_t)(c / w) * rows_alloc + r) * w + (c % w)]);
}

__global__ __launch_bounds__(64) void clock_sample(uint64_t *out) {
  if (threadIdx.x == 0) {
    out[0] = __builtin_amdgcn_s_memtime();
    out[1] = __builtin_amdgcn_s_memrealtime();
  }
}

}  // namespace

hipError_t launch_clock_sample(uint64_t *out, hipStream_t s) {
  hipLaunchKernelGGL(clock_sample, dim3(1), dim3(64), 0, s, out);
  return hipGetLastError();
}

hipError_t launch_zero_rows(int type, void *p, int ld, int cols, int row0, int row1, hipStream_t s) {
  if (row1 <= row0) return hipSuccess;
  if (type == kF32)
    hipLaunchKernelGGL(zero_rows<float>, dim3(row1 - row0), dim3(256), 0, s,
                       static_cast<float *>(p), ld, cols, row0);
  else
    hipLaunchKernelGGL(zero_rows<bf16_t>, dim3(row1 - row0), dim3(256), 0, s,
                       static_cast<bf16_t *>(p), ld, cols, row0);
  return hipGetLastError();
}

hipError_t launch_to_f32(int type, const void *src, int ld_src, float *dst, int ld_dst, int rows,
                         int cols, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (type == kF32)
    hipLaunchKernelGGL(widen_rows<float>, dim3(rows), dim3(256), 0, s, static_cast<const float *>(src),
                       ld_src, dst, ld_dst, cols);
  else
    hipLaunchKernelGGL(widen_rows<bf16_t>, dim3(rows), dim3(256), 0, s,
                       static_cast<const bf16_t *>(src), ld_src, dst, ld_dst, cols);
  return hipGetLastError();
}

hipError_t launch_kmajor_to_f32(int type, const void *src, int w, int rows_alloc, float *dst,
                                int ld_dst, int rows, int cols, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (rows > rows_alloc || (w != 32 && w != 64) || cols % w) return hipErrorInvalidValue;
  if (type == kF32)
    hipLaunchKernelGGL(widen_kmajor_rows<float>, dim3(rows), dim3(256), 0, s,
                       static_cast<const float *>(src), w, rows_alloc, dst, ld_dst, cols);
  else
    hipLaunchKernelGGL(widen_kmajor_rows<bf16_t>, dim3(rows), dim3(256), 0, s,
                       static_cast<const bf16_t *>(src), w, rows_alloc, dst, ld_dst, cols);
  return hipGetLastError();
}

}  // namespace sarathi
