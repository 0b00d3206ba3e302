// Host-side launchers of the gfx950 kernels (implemented in the .hip files of this directory).
// Every launcher only enqueues on the given stream and returns hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace sarathi {

enum StorageType { kF32 = 0, kBF16 = 1 };

// ---------------------------------------------------------------------------------------------
// Row norms.  v[r] = resid[r] + sum_{s < splits} part[s][r]  (resid in `res_type` storage, the
// split partials of a GEMM in float32 with slice stride rows*H; splits may be 0).  If sum_out is
// non-null it receives v (float32); if sum_lo is non-null (and sum_out null) v is rounded to the
// out type, stored there row-major [rows, H], and normalised as rounded.  out[r] = RMSNorm(v) * g
// or LayerNorm(v) * g + b for r < rows; rows rows..rows_alloc-1 of out are zero-filled.  out is
// row-major [rows_alloc, H] (kmajor = 0), or k-tile-major [H/w][rows_alloc][w] with w = kmajor, 32
// or 64 (the layout the bf16 GEMM reads fastest: w = its stage depth; H % 64 == 0).  Type pairs
// (resid, out): (f32, f32), (bf16, bf16), (f32, bf16).
constexpr int kMaxHidden = 16384;   // widest row a norm workgroup holds (1024 threads x 16 elements)
hipError_t launch_norm_rows(int res_type, int out_type, bool layernorm, const void *resid,
                            const float *part, int splits, float *sum_out, void *sum_lo,
                            const float *g, const float *b, void *out, int H, int rows,
                            int rows_alloc, float eps, int kmajor, hipStream_t s);

// FFN activation from split partials ([splits][rows][n_part] float32): gated (n_part = 2F):
// a[r, j] = silu(sum_s part[s][r][j]) * sum_s part[s][r][F + j];  else (n_part = F):
// a[r, j] = gelu(sum_s part[s][r][j]); a[r, j] is stored as column col0 + j of out, a storage-type
// matrix of ld columns (col0 + F <= ld), row-major (kmajor = 0) or k-tile-major [ld/w][rows_alloc][w]
// with w = kmajor (32 or 64; ld, col0 and F multiples of w).
hipError_t launch_ffn_act(int out_type, bool gated, const float *part, int splits, void *out,
                          int rows, int F, int col0, int ld, int kmajor, int rows_alloc, hipStream_t s);

// out[r, c] = resid[r, c] + sum_{s < splits} part[s][r][c]  (resid float32, out storage type).
hipError_t launch_resid_sum(int out_type, const float *resid, const float *part, int splits,
                            void *out, int rows, int cols, hipStream_t s);

// ---------------------------------------------------------------------------------------------
// GEMM  epilogue( sum_k a[m, k] * w[n, k] )  over the concatenated batch rows.
enum Epilogue {
  kEpiStore = 0,     // out (storage) = acc
  kEpiPartial = 1,   // part[split][m][n] (float32) = acc over the split's k range
  kEpiSwiGLU = 2,    // out (storage) = silu(a w0^T) * (a w1^T)         [gate, up]
  kEpiGelu = 3,      // out (storage) = gelu(acc)                      [GPT MLP up]
};

struct GemmArgs {
  const void *a;      // [m_alloc, k], row stride lda (elements)
  const void *w0;     // [n, k] row stride ldw (rows 0..n_w0-1 when w1 continues it)
  const void *w1;     // SwiGLU: the up weight.  kEpiPartial: rows n_w0..n-1 of the product's
                      // weight (the up half of a gate|up product), else null
  void *out;          // row stride ldo (kEpiStore / kEpiSwiGLU / kEpiGelu); with out_kmajor = w
                      // (32 or 64; kEpiSwiGLU / kEpiGelu only) k-tile-major [n/w][m_alloc][w]
  float *part;        // [splits][m_store][n] (kEpiPartial)
  int lda, ldw, ldo;
  int m_alloc;        // rows of a that may be read
  int m_store;        // rows of the product that are written (m_store <= m_alloc)
  int n;              // output columns
  int k;              // multiple of 64 in bf16 mode
  int n_w0;           // kEpiPartial with w1: rows of the product taken from w0
  int out_kmajor;     // 0 or the k-tile width of out (see out)
  int a_kmajor;       // 0: a is row-major.  bf16 only, w = 32 or 64 (the plan's stage depth): a is
                      // k-tile-major, [k/w][m_alloc][w] (lda unused).  A k-tile of 1024 / (2 w) rows
                      // is then 1 KiB of consecutive bytes, which the LDS DMA fetches faster
  int w_kmajor;       // 0: w0 / w1 are row-major (row stride ldw).  bf16 only, w = the plan's stage
                      // depth: each is k-tile-major, [k/w][rows][w] (ldw unused), and k-tile j of
                      // row r of w0 is at w0 + j * w_slab0 + r * w (w1: w_slab1); with w = 32 two
                      // weight rows of one k-tile then fill one 128-byte line instead of half of two
  int w_slab0, w_slab1;   // with w_kmajor: elements between consecutive k-tiles of w0 / w1
};

// Launch shape of one GEMM: m_tiles x n_tiles output tiles, each k range cut into `splits`;
// mbw = 16-row blocks per wave row; wn = wave columns (4: 8 waves, 2: 4 waves); bn = product
// columns per tile (128, or 256 for the wide tiles of batches of more than 288 rows); the grid is
// 8 * per_xcd workgroups.
struct GemmPlan { int epi, m_tiles, n_tiles, splits, mbw, wn, per_xcd, grid, bn; };
// Plans a GEMM with epilogue `epi` (kEpiSwiGLU / kEpiGelu may come back as kEpiPartial when a split
// product plus a separate activation pass is estimated faster; n is then the product width:
// 2F for SwiGLU).  n_out is the output width of the epilogue (F for the FFN up products).
GemmPlan plan_gemm(int type, int epi, int m, int n_out, int k, int cus);
// A fused-activation FFN product (kEpiSwiGLU / kEpiGelu, bf16) whose fused plan needs more than one
// round of `cus` weight stripes runs as two parts: the first cus stripes as one round of fused tiles
// (*main, over the first n_main output columns), the remaining output columns as a split product
// (*tail, kEpiPartial over their gate|up or up weight rows) whose partials an activation pass sums.
// Returns n_main, or 0 (main and tail untouched) when the product runs whole.  Depends on the
// weight shape only, never on m beyond the row tiles, which the tail takes from the main part (one
// input layout serves both).
int plan_gemm_tail(int type, int epi, int m, int n_out, int k, int cus, GemmPlan *main, GemmPlan *tail);
// k depth of one LDS stage of a bf16 plan (32 or 64): the k-tile width of a k-tile-major A.
int gemm_stage_depth(const GemmPlan &p);
hipError_t launch_gemm(int type, int epi, const GemmArgs &g, const GemmPlan &p, hipStream_t s);
// Repacks a bf16 weight [rows, k] (row stride ld elements) into k-tile-major [k/w][rows][w]
// (w = 32 or 64, k a multiple of w, rows * k < 2^31): element (r, c) moves to ((c / w) * rows + r) * w
// + c % w.  dst must not overlap src.
hipError_t launch_pack_kmajor(const void *src, int rows, int k, int ld, int w, void *dst, hipStream_t s);

// ---------------------------------------------------------------------------------------------
// RoPE + KV append: for rows [row0, row0+n_rows) of the batch, sums the QKV GEMM's split partials
// (float32 [splits][rows_total][3A]), rotates q and k at the row's position (if use_rope) with the
// float32 cos/sin table tab[pos * d/2 + j], writes q to q_out (storage, row stride ld_q) and k, v
// into the row's caches at slot pos (with a page pool: into the pool page of the row's block table).  If qkv_dump is non-null it receives the summed, unrotated
// q|k|v row (float32 [rows, 3A]).
hipError_t launch_rope_append(int type, const float *part, int splits, int rows_total, void *q_out,
                              int ld_q, float *qkv_dump, const float2 *tab, int use_rope, int nh,
                              int d, int row0, int n_rows, const ChunkSet &cs, const DecodeGroup &dg,
                              const PagePool &pool, hipStream_t s);

// ---------------------------------------------------------------------------------------------
// Split-KV single-query attention for rows [row0, row0+n_rows): each (row, head) attends over keys
// 0..pos of its cache in balanced splits of at most attn_split_keys(pos + 1) keys; each split writes
// its partial (running max m and sum l in the log2 domain, unnormalised output o) to part_ml /
// part_o, at slot ((r - prow0) * nh + h) * stride + s (stride >= the row's split count; splits past
// a row's count are written as empty partials).  A split's four waves walk its keys in passes of
// kAttnSplit keys (64 per wave).  Rows with more than kAttnLongKeys keys take splits of
// kAttnLongPasses passes (1024 keys): their workgroups then stream four times the bytes each, and
// write and merge a quarter of the partials.  The split size depends only on the row's own length,
// so a row's result does not depend on the batch it is in.
#ifndef SARATHI_DECODE_LONG_KEYS
#define SARATHI_DECODE_LONG_KEYS 2048
#endif
#ifndef SARATHI_DECODE_LONG_PASSES
#define SARATHI_DECODE_LONG_PASSES 4
#endif
constexpr int kAttnSplit = 256;
constexpr int kAttnLongKeys = SARATHI_DECODE_LONG_KEYS;
constexpr int kAttnLongPasses = SARATHI_DECODE_LONG_PASSES;
constexpr int kMaxKeySplits = 256;   // split partials per (row, head): keys up to 65536
__host__ __device__ inline int attn_split_keys(int n_keys) {
  return n_keys > kAttnLongKeys ? kAttnSplit * kAttnLongPasses : kAttnSplit;
}
__host__ __device__ inline int attn_splits(int n_keys) {
  const int sk = attn_split_keys(n_keys);
  return (n_keys + sk - 1) / sk;
}
hipError_t launch_attn_rows(int type, int d, const void *q, int ld_q, int nh, int row0, int n_rows,
                            const ChunkSet &cs, const DecodeGroup &dg, const PagePool &pool,
                            int stride, int prow0, float *part_o, float *part_ml, hipStream_t s);

// Where the attention split partials of a forward live: chunk rows (batch rows below the merge's
// chunk_rows) in region c, `stride_c` partials per (row, head), slot (r * nh + h) * stride_c + s;
// decode rows in region d, slot ((r - chunk_rows) * nh + h) * stride_d + s.
struct AttnParts {
  float *o_c, *ml_c;   // [chunk rows][nh][stride_c] x (D floats | (m, l)), or null without chunk partials
  float *o_d, *ml_d;   // [decode rows][nh][stride_d] x (D floats | (m, l))
  int stride_c, stride_d;
};

// Partial counts of the chunk rows for the merge: chunk i owns rows row0[i].. (up to the next
// chunk's first row) and left split[i] partials per row and head; split[i] == 1 means the chunk
// kernel wrote those rows itself.
struct ChunkSplits {
  int32_t row0[kMaxChunks];
  int32_t split[kMaxChunks];
  int32_t n;
};
// Merges the split partials of rows [row0, row0+n_rows) into out[row, h*d + e] (storage type, laid
// out as olay says).  Rows at or past chunk_rows merge their stride_d partials of region d.  Rows
// below it merge chunk_splits partials of region c when chunk_splits > 0; with chunk_splits == 0
// they merge their chunk's count from `table`, and the rows of chunks with one split are left as
// they are.
hipError_t launch_attn_combine(int type, int d, int nh, int row0, int n_rows, int chunk_rows,
                               int chunk_splits, const ChunkSplits &table, const AttnParts &parts,
                               void *out, OutLayout olay, hipStream_t s);

// Flash-style causal chunk attention (bf16, MFMA) over every chunk of the set: row row0[j] + t of
// chunk j attends to keys 0..off[j]+t of chunk j's cache.  q and out are batch-row indexed (q row
// stride ld_q; out laid out as olay says).  Chunk j's query blocks (64 queries; 128 with cs.qblocks = 2, two 16-query
// blocks per wave, contiguous caches only) split their key tiles cs.split[j] ways; n_split is the
// largest of these.  A chunk with cs.split[j] > 1 writes partials (stride `stride` splits per row and
// head) for launch_attn_combine instead of out.
constexpr int kChunkResident = 512;           // chunk-kernel workgroups resident at once (two per CU)
constexpr int kFusedChunkResident = 512;      // fused-kernel workgroups resident at once (two per CU)
// Time of one key tile of a chunk-kernel item with two 16-query blocks per wave, in units of the
// one-block item's tile time (measured on the llama-13b shape over an 8K-key prefix: 2.44 against
// 1.51 microseconds per tile).
constexpr double kTwoBlockTileCost = 1.62;
constexpr int kMinSplitTiles = 4;             // a split keeps at least 4 key tiles
constexpr int kMaxChunkSplits = 16;
constexpr int kSplitCostTiles = 3;            // makespan cost of one more split, in key-tile times
int chunk_attn_splits(ChunkSet &cs, int nh, int bq, int resident, long long *cost);
int chunk_attn_plan(ChunkSet &cs, int nh, bool paged);
hipError_t launch_attn_chunk(int d, const void *q, int ld_q, int nh, const ChunkSet &cs,
                             const PagePool &pool, void *out, OutLayout olay, int n_split, int stride,
                             float *part_o, float *part_ml, hipStream_t s);

// The chunk attention of every chunk of the set and the split-KV attention of decode rows
// [dec_row0, dec_row0 + dec_rows) (one decode group, dg) in one launch (bf16).  Chunk rows are
// handled as by launch_attn_chunk with n_split key splits (partials in region c of `parts` when
// n_split > 1, stride_c = n_split) and cs.qblocks 16-query blocks per wave (2: contiguous caches
// only); decode rows write split partials to region d as launch_attn_rows does (stride_d, first row
// of the region = cs.rows).
hipError_t launch_attn_fused(int d, const void *q, int ld_q, int nh, const ChunkSet &cs,
                             const PagePool &pool, void *out, OutLayout olay, int n_split,
                             const AttnParts &parts, const DecodeGroup &dg, int dec_row0,
                             int dec_rows, hipStream_t s);

// Device address of the current device's copy of the library's fixed scratch (kNoAllocScratchBytes,
// 256-byte aligned), the workspace of the no-allocation forward.  Looked up once per device (the
// device must be the current one then) and cached; later calls return the cached address.
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
hipError_t noalloc_scratch(int device, void **out);

// kClockWorkgroups single-wave workgroups; one running on compute unit u (slot u = XCD * 256 + bits
// 15:8 of its HW_ID) writes the unit's shader-clock timestamp (s_memtime) and the 100 MHz real-time
// counter (s_memrealtime) to out[2u], out[2u + 1] (out: kClockSlots pairs).
constexpr int kClockSlots = 2048;
constexpr int kClockWorkgroups = 4096;
hipError_t launch_clock_sample(uint64_t *out, hipStream_t s);

// Zero-fill rows [row0, row1) of a [*, cols] storage matrix (row stride ld).
hipError_t launch_zero_rows(int type, void *p, int ld, int cols, int row0, int row1, hipStream_t s);

// Convert a [rows, cols] storage matrix (row stride ld_src) to float32 (row stride ld_dst).
hipError_t launch_to_f32(int type, const void *src, int ld_src, float *dst, int ld_dst, int rows,
                         int cols, hipStream_t s);
// The same from a k-tile-major [cols/w][rows_alloc][w] matrix (w = 32 or 64).
hipError_t launch_kmajor_to_f32(int type, const void *src, int w, int rows_alloc, float *dst,
                                int ld_dst, int rows, int cols, hipStream_t s);

}  // namespace sarathi
