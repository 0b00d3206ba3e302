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

// The shader-clock counter is not common to a chip, nor to an XCD (pairs taken on different compute
// units of one XCD measured 2.0 to 3.4 GHz over the same few milliseconds), so a sample holds one
// (s_memtime, s_memrealtime) pair per compute unit: kClockWorkgroups single-wave workgroups spread
// over the units, each writing its pair to the slot of the unit it runs on, from the XCC_ID hardware
// register (hwreg 20, bits 3:0) and bits 15:8 of HW_ID (hwreg 4: compute unit, shader array and
// shader engine).  Workgroups that share a unit write the same slot; either pair serves.
__global__ __launch_bounds__(64) void clock_sample(uint64_t *out) {
  if (threadIdx.x == 0) {
    const int xcc = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 7;
    const int unit = (__builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4) >> 8) & 255;
    const uint64_t t = __builtin_amdgcn_s_memtime();
    const uint64_t r = __builtin_amdgcn_s_memrealtime();
    *reinterpret_cast<ulonglong2 *>(&out[2 * (xcc * 256 + unit)]) = make_ulonglong2(t, r);
  }
}

}  // namespace

hipError_t launch_clock_sample(uint64_t *out, hipStream_t s) {
  hipLaunchKernelGGL(clock_sample, dim3(kClockWorkgroups), dim3(64), 0, s, out);
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
