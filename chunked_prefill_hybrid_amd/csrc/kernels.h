// Host-side launchers of the gfx950 kernels (implemented in the .hip files of this directory).
// Every launcher only enqueues on the given stream and returns hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace sarathi {

enum StorageType { kF32 = 0, kBF16 = 1 };

// ---------------------------------------------------------------------------------------------
// Row norms: out[r] = RMSNorm(x[r]) * g  or  LayerNorm(x[r]) * g + b, for r < rows; rows
// rows..rows_alloc-1 of out are zero-filled.  x is `in_type` storage [rows, H]; out is `out_type`.
hipError_t launch_norm(int in_type, int out_type, bool layernorm, const void *x, const float *g,
                       const float *b, void *out, int H, int rows, int rows_alloc, float eps,
                       hipStream_t s);

// ---------------------------------------------------------------------------------------------
// GEMM  out[m, n] = epilogue( sum_k a[m, k] * w[n, k] )  over the concatenated batch rows.
enum Epilogue {
  kEpiStore = 0,     // out (storage) = acc
  kEpiResidF32 = 1,  // out (float32) = acc + resid (storage)          [x + attn W_o^T]
  kEpiResidOut = 2,  // out (storage) = acc + resid (float32)          [h1 + act W_down^T]
  kEpiSwiGLU = 3,    // out (storage) = silu(a w0^T) * (a w1^T)         [gate, up]
  kEpiGelu = 4,      // out (storage) = gelu(acc)                      [GPT MLP up]
};

struct GemmArgs {
  const void *a;      // [m_alloc, k], row stride lda (elements)
  const void *w0;     // [n, k] row stride ldw
  const void *w1;     // second weight of SwiGLU (up), else null
  void *out;          // row stride ldo
  const void *resid;  // residual input for kEpiResid*, row stride ldr
  int lda, ldw, ldo, ldr;
  int m_alloc;        // rows of a that may be read
  int m_store;        // rows of out that are written (m_store <= m_alloc)
  int n;              // output columns
  int k;
};

hipError_t launch_gemm(int type, int epi, const GemmArgs &g, hipStream_t s);

// Planned bf16 tile shape for a GEMM (exposed for tests and reports).
struct GemmPlan { int bm, bn, m_tiles, n_tiles, grid; };
GemmPlan plan_gemm(int type, int epi, int m, int n, int k);

// ---------------------------------------------------------------------------------------------
// RoPE + KV append: for rows [row0, row0+n_rows) of the batch, reads q, k, v from qkv
// [rows, 3A] (row stride ld_qkv), rotates q and k at the row's position (if use_rope) with the
// float32 cos/sin table tab[pos * d/2 + j], writes q to q_out (row stride ld_q) and k, v into the
// row's caches at slot pos.
hipError_t launch_rope_append(int type, const void *qkv, int ld_qkv, void *q_out, int ld_q,
                              const float2 *tab, int use_rope, int nh, int d, int row0, int n_rows,
                              const ChunkRef &ch, const DecodeGroup &dg, hipStream_t s);

// ---------------------------------------------------------------------------------------------
// Split-KV single-query attention for rows [row0, row0+n_rows): each (row, head) attends over keys
// 0..pos of its cache in balanced splits of at most kAttnSplit keys; each split writes its partial
// (running max m and sum l in the log2 domain, unnormalised output o) to part_ml / part_o.
constexpr int kAttnSplit = 256;
__host__ __device__ inline int attn_splits(int n_keys) {
  return (n_keys + kAttnSplit - 1) / kAttnSplit;
}
hipError_t launch_attn_rows(int type, int d, const void *q, int ld_q, int nh, int row0, int n_rows,
                            const ChunkRef &ch, const DecodeGroup &dg, int max_splits,
                            float *part_o, float *part_ml, hipStream_t s);

// Merges the split partials of rows [row0, row0+n_rows) into out[row, h*d + e] (storage type,
// row stride ld_out).
hipError_t launch_attn_combine(int type, int d, int nh, int row0, int n_rows, int max_splits,
                               const float *part_o, const float *part_ml, void *out, int ld_out,
                               hipStream_t s);

// Flash-style causal chunk attention (bf16, MFMA): chunk rows [0, ch.len) attend to chunk keys
// 0..ch.off+t.  q rows are the chunk rows of q (row stride ld_q); out likewise.
hipError_t launch_attn_chunk(int d, const void *q, int ld_q, int nh, const ChunkRef &ch, void *out,
                             int ld_out, hipStream_t s);

// Zero-fill rows [row0, row1) of a [*, cols] storage matrix (row stride ld).
hipError_t launch_zero_rows(int type, void *p, int ld, int cols, int row0, int row1, hipStream_t s);

// Convert a [rows, cols] storage matrix (row stride ld_src) to float32 (row stride ld_dst).
hipError_t launch_to_f32(int type, const void *src, int ld_src, float *dst, int ld_dst, int rows,
                         int cols, hipStream_t s);

}  // namespace sarathi
