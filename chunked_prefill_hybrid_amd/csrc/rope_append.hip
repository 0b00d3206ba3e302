// RoPE on the queries and keys of every batch row, and the in-place KV-cache append.
//
// Each row's new K and V go into its request's cache at the row's position: chunk row t of a chunk at
// offset o writes slot o+t of the chunk request's cache; decode i writes slot decode_len[i] of its
// own cache.  Caches are allocated by the caller at maximum length and updated in place (SARATHI:
// Efficient LLM Inference by Piggybacking Decodes with Chunked Prefills, section 3,
// "Implementation", KV cache pre-allocation).  The rotation pairs adjacent elements (2j, 2j+1) with
// angle pos * base^(-2j/d); cos/sin come from a float32 table built on the host in float64.
// One workgroup per row; every thread moves one 16-byte packet of q, k and v.
#include "kernels.h"

namespace sarathi {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void rope_append(const T *qkv, int ld_qkv, T *q_out, int ld_q,
                                                   const float2 *tab, int use_rope, int nh, int d,
                                                   int row0, ChunkRef ch, DecodeGroup dg) {
  constexpr int E = Packet<T>::E;
  const int r = row0 + blockIdx.x;
  const int A = nh * d;
  const RowRef rr = row_ref(r, ch, dg);
  T *kc = reinterpret_cast<T *>(rr.k);
  T *vc = reinterpret_cast<T *>(rr.v);
  const T *src = qkv + (size_t)r * ld_qkv;
  for (int c = threadIdx.x * E; c < A; c += blockDim.x * E) {
    const int h = c / d, e0 = c - h * d;
    float q[E], k[E], v[E];
    unpack<T>(ld16(src + c), q);
    unpack<T>(ld16(src + A + c), k);
    unpack<T>(ld16(src + 2 * A + c), v);
    if (use_rope) {
      const float2 *t = tab + (size_t)rr.pos * (d / 2) + e0 / 2;
#pragma unroll
      for (int u = 0; u < E / 2; ++u) {
        const float2 cs = t[u];
        const float q0 = q[2 * u], q1 = q[2 * u + 1], k0 = k[2 * u], k1 = k[2 * u + 1];
        q[2 * u] = q0 * cs.x - q1 * cs.y;
        q[2 * u + 1] = q0 * cs.y + q1 * cs.x;
        k[2 * u] = k0 * cs.x - k1 * cs.y;
        k[2 * u + 1] = k0 * cs.y + k1 * cs.x;
      }
    }
    st16(q_out + (size_t)r * ld_q + c, pack<T>(q));
    const size_t slot = ((size_t)h * rr.cap + rr.pos) * d + e0;
    st16(kc + slot, pack<T>(k));
    st16(vc + slot, pack<T>(v));
  }
}

}  // namespace

hipError_t launch_rope_append(int type, const void *qkv, int ld_qkv, void *q_out, int ld_q,
                              const float2 *tab, int use_rope, int nh, int d, int row0, int n_rows,
                              const ChunkRef &ch, const DecodeGroup &dg, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  if (type == kF32)
    hipLaunchKernelGGL(rope_append<float>, dim3(n_rows), dim3(256), 0, s,
                       static_cast<const float *>(qkv), ld_qkv, static_cast<float *>(q_out), ld_q,
                       tab, use_rope, nh, d, row0, ch, dg);
  else
    hipLaunchKernelGGL(rope_append<bf16_t>, dim3(n_rows), dim3(256), 0, s,
                       static_cast<const bf16_t *>(qkv), ld_qkv, static_cast<bf16_t *>(q_out), ld_q,
                       tab, use_rope, nh, d, row0, ch, dg);
  return hipGetLastError();
}

}  // namespace sarathi
