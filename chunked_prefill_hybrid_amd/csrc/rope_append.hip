// RoPE on the queries and keys of every batch row, and the in-place KV-cache append.
//
// Each row's new K and V go into its request's cache at the row's position: chunk row t of a chunk at
// offset o writes slot o+t of the chunk request's cache; decode i writes slot decode_len[i] of its
// own cache.  Caches are allocated by the caller at maximum length and updated in place (SARATHI:
// Efficient LLM Inference by Piggybacking Decodes with Chunked Prefills, section 3,
// "Implementation", KV cache pre-allocation).  The rotation pairs adjacent elements (2j, 2j+1) with
// angle pos * base^(-2j/d); cos/sin come from a float32 table built on the host in float64.
// The q|k|v row is the sum of the QKV GEMM's float32 split partials, taken in split order; it is
// rounded to the storage type only once, after the rotation.
// Every thread moves 4 consecutive elements of one row's q, k and v.  With a page pool the row's K/V
// go to the pool page its request's block table names for the row's position.
#include "kernels.h"

namespace sarathi {
namespace {

// Stores go through global-memory views: the cache pointers arrive as integers in the request
// descriptors.
template <typename T> __device__ __forceinline__ void put4(T *p, const float *v);
template <> __device__ __forceinline__ void put4<float>(float *p, const float *v) {
  *as_global(reinterpret_cast<f32x4_t *>(p)) = f32x4_t{v[0], v[1], v[2], v[3]};
}
template <> __device__ __forceinline__ void put4<bf16_t>(bf16_t *p, const float *v) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 u = {(uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                   (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16)};
  *as_global(reinterpret_cast<u32x2 *>(p)) = u;
}

constexpr int kMaxSplits = 8;

// v = sum_s part[s][off..off+3] in split order (all loads issued before the adds).
__device__ __forceinline__ void sum4(const float *part, int splits, size_t slice, size_t off,
                                     float *v) {
  float4 a[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < splits) a[s] = *reinterpret_cast<const float4 *>(part + s * slice + off);
  v[0] = a[0].x; v[1] = a[0].y; v[2] = a[0].z; v[3] = a[0].w;
#pragma unroll
  for (int s = 1; s < kMaxSplits; ++s)
    if (s < splits) {
      v[0] += a[s].x; v[1] += a[s].y; v[2] += a[s].z; v[3] += a[s].w;
    }
}

// grid: (rows, column blocks of 1024); one 4-element chunk of q, k and v per thread.
template <typename T, bool kChunkRows, bool kPaged>
__global__ __launch_bounds__(256) void rope_append(const float *part, int splits, int rows_total,
                                                   T *q_out, int ld_q, float *qkv_dump,
                                                   const float2 *tab, int use_rope, int nh, int d,
                                                   int row0, ChunkSet cs, DecodeGroup dg,
                                                   PagePool pool) {
  const int r = row0 + blockIdx.x;
  const int A = nh * d;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= A) return;
  const RowRef rr = row_ref<kChunkRows>(r, cs, dg);
  T *kc = reinterpret_cast<T *>(rr.k);
  T *vc = reinterpret_cast<T *>(rr.v);
  const size_t slice = (size_t)rows_total * 3 * A, src = (size_t)r * 3 * A;
  const int h = c / d, e0 = c - h * d;
  float q[4], k[4], v[4];
  sum4(part, splits, slice, src + c, q);
  sum4(part, splits, slice, src + A + c, k);
  sum4(part, splits, slice, src + 2 * A + c, v);
  if (qkv_dump) {
    float *dr = qkv_dump + src;
    *reinterpret_cast<float4 *>(dr + c) = make_float4(q[0], q[1], q[2], q[3]);
    *reinterpret_cast<float4 *>(dr + A + c) = make_float4(k[0], k[1], k[2], k[3]);
    *reinterpret_cast<float4 *>(dr + 2 * A + c) = make_float4(v[0], v[1], v[2], v[3]);
  }
  if (use_rope) {
    const float2 *t = tab + (size_t)rr.pos * (d / 2) + e0 / 2;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // Explicit fused multiply-adds: every instantiation of the kernel rounds the rotation the
      // same way, so a row's result does not depend on which launch variant served it.
      const float2 cz = t[u];
      const float q0 = q[2 * u], q1 = q[2 * u + 1], k0 = k[2 * u], k1 = k[2 * u + 1];
      q[2 * u] = fmaf(q0, cz.x, -(q1 * cz.y));
      q[2 * u + 1] = fmaf(q0, cz.y, q1 * cz.x);
      k[2 * u] = fmaf(k0, cz.x, -(k1 * cz.y));
      k[2 * u + 1] = fmaf(k0, cz.y, k1 * cz.x);
    }
  }
  put4<T>(q_out + (size_t)r * ld_q + c, q);
  if (kPaged) {
    const int page = pool_page(reinterpret_cast<const int32_t *>(rr.k), rr.pos >> pool.shift, pool.n_pages);
    const size_t slot = paged_off(page, h, rr.pos, nh, pool.shift, d) + e0;
    put4<T>(reinterpret_cast<T *>(pool.k) + slot, k);
    put4<T>(reinterpret_cast<T *>(pool.v) + slot, v);
  } else {
    const size_t slot = ((size_t)h * rr.cap + rr.pos) * d + e0;
    put4<T>(kc + slot, k);
    put4<T>(vc + slot, v);
  }
}

}  // namespace

hipError_t launch_rope_append(int type, const float *part, int splits, int rows_total, void *q_out,
                              int ld_q, float *qkv_dump, const float2 *tab, int use_rope, int nh,
                              int d, int row0, int n_rows, const ChunkSet &cs, const DecodeGroup &dg,
                              const PagePool &pool, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  if (splits < 1 || splits > kMaxSplits) return hipErrorInvalidValue;
  const dim3 grid(n_rows, (nh * d / 4 + 255) / 256);
#define SARATHI_ROPE(T, CR, PG)                                                                        \
  hipLaunchKernelGGL((rope_append<T, CR, PG>), grid, dim3(256), 0, s, part, splits, rows_total,        \
                     static_cast<T *>(q_out), ld_q, qkv_dump, tab, use_rope, nh, d, row0, cs, dg, pool)
#define SARATHI_ROPE_T(T)                                                                              \
  if (chunk_rows) {                                                                                    \
    if (paged) SARATHI_ROPE(T, true, true); else SARATHI_ROPE(T, true, false);                         \
  } else {                                                                                             \
    if (paged) SARATHI_ROPE(T, false, true); else SARATHI_ROPE(T, false, false);                       \
  }
  const bool chunk_rows = row0 < cs.rows, paged = pool.k != 0;
  if (type == kF32) {
    SARATHI_ROPE_T(float)
  } else {
    SARATHI_ROPE_T(bf16_t)
  }
#undef SARATHI_ROPE_T
#undef SARATHI_ROPE
  return hipGetLastError();
}

}  // namespace sarathi
