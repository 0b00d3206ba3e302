// Host side of the C ABI declared in include/sarathi.h: validation, workspace planning, the RoPE
// table, and the launch sequence of one hybrid-batch layer forward.
//
// Launch sequence (all on the caller's stream, no host synchronisation):
//   norm1 -> QKV GEMM over the C+B rows -> RoPE + KV append -> attention (chunk rows and decode rows
//   split per request) -> O GEMM + residual -> norm2 -> gate/up GEMM + SiLU*mul (or up + GELU) ->
//   down GEMM + residual.
// This is the hybrid iteration of SARATHI: Efficient LLM Inference by Piggybacking Decodes with
// Chunked Prefills, section 3, "Decode-Maximal Batching": linear ops fused over the concatenated
// chunk and decode tokens, attention computed separately per request.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/sarathi.h"
#include "kernels.h"

using namespace sarathi;

struct sarathi_layer {
  sarathi_layer_desc desc;
  sarathi_weights w;   // bf16: the projection weights point into wpack
  float2 *rope_tab;  // device [max_pos, head_dim/2] (LLAMA), else null
  void *wpack;       // bf16: device copy of the projection weights, each k-tile-major [k/wk][rows][wk]
  int wk;            // k-tile width of the packed weights (bf16), 0: row-major caller weights (f32)
  int device;
};

struct sarathi_timer {
  int capacity;
  int used;                       // forwards recorded since the last read
  uint32_t mask;                  // timed stages
  int slot[SARATHI_N_STAGES];     // index of a timed stage among the timed ones, else -1
  int n_timed;
  std::vector<hipEvent_t> ev;     // [capacity][n_timed][2]: before, after
  std::vector<uint32_t> ran;      // per recorded forward: bit s set if stage s launched work
};

namespace {

thread_local std::string g_last_error;

sarathi_status fail(sarathi_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

size_t elem_size(int dtype) { return dtype == SARATHI_BF16 ? 2 : 4; }
size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
int round_up(int v, int m) { return (v + m - 1) / m * m; }

sarathi_status check_desc(const sarathi_layer_desc *d) {
  if (!d) return fail(SARATHI_ERR_INVALID, "layer description is null");
  if (d->hidden <= 0 || d->n_heads <= 0 || d->head_dim <= 0 || d->ffn <= 0)
    return fail(SARATHI_ERR_INVALID, "hidden, n_heads, head_dim and ffn must be positive");
  if (d->max_tokens <= 0 || d->max_pos <= 0)
    return fail(SARATHI_ERR_INVALID, "max_tokens and max_pos must be positive");
  if (d->max_pos > kMaxKeySplits * kAttnSplit)
    return fail(SARATHI_ERR_UNSUPPORTED, "max_pos %d > %d (attention key-range limit)", d->max_pos,
                kMaxKeySplits * kAttnSplit);
  if (d->arch != SARATHI_ARCH_LLAMA && d->arch != SARATHI_ARCH_GPT)
    return fail(SARATHI_ERR_INVALID, "unknown arch %d", d->arch);
  if (d->dtype != SARATHI_F32 && d->dtype != SARATHI_BF16)
    return fail(SARATHI_ERR_INVALID, "unknown dtype %d", d->dtype);
  if (!(d->norm_eps >= 0.f) || !std::isfinite(d->norm_eps))
    return fail(SARATHI_ERR_INVALID, "norm_eps must be finite and >= 0");
  if (d->arch == SARATHI_ARCH_LLAMA && !(d->rope_base > 0.f))
    return fail(SARATHI_ERR_INVALID, "rope_base must be > 0");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(SARATHI_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
  if (d->hidden % 64 || (d->n_heads * d->head_dim) % 64)
    return fail(SARATHI_ERR_UNSUPPORTED, "hidden and n_heads*head_dim must be multiples of 64");
  if (d->dtype == SARATHI_BF16 && d->ffn % 64)
    return fail(SARATHI_ERR_UNSUPPORTED, "ffn must be a multiple of 64 in bf16 mode");
  if (d->dtype == SARATHI_F32 && d->ffn % 16)
    return fail(SARATHI_ERR_UNSUPPORTED, "ffn must be a multiple of 16 in f32 mode");
  if (d->hidden > kMaxHidden)
    return fail(SARATHI_ERR_UNSUPPORTED, "hidden %d > %d (a norm row is held by one workgroup)",
                d->hidden, kMaxHidden);
  if ((long long)d->max_tokens * 3 * d->n_heads * d->head_dim > (1ll << 31))
    return fail(SARATHI_ERR_UNSUPPORTED, "max_tokens too large");
  // the packed bf16 weights and the GEMM's k-tile steps through them use 32-bit element offsets
  const long long A = (long long)d->n_heads * d->head_dim;
  if (d->dtype == SARATHI_BF16 &&
      (3 * A * d->hidden >= (1ll << 31) || (long long)d->ffn * d->hidden >= (1ll << 31)))
    return fail(SARATHI_ERR_UNSUPPORTED, "a weight matrix of 2^31 or more elements");
  return SARATHI_OK;
}

struct Range {
  uintptr_t lo, hi;
  const char *what;
  int idx;
};

// The batch as the forward sees it, whichever entry point passed it: prefill chunks (rows first, in
// order), then decodes.
// With a page pool (paged == true), a chunk's kv.k holds its block table, kv.v is null and
// kv.capacity is the table's token capacity; the decodes' tables are in decode_tables.
struct BatchView {
  int n_chunks;
  sarathi_chunk chunks[kMaxChunks];
  int C;   // total chunk rows
  int B;
  const sarathi_kv *decode_kv;
  const int32_t *decode_len;
  const void *x;
  void *y;
  bool paged;
  sarathi_page_pool pool;
  int page_shift;
  const sarathi_page_table *decode_tables;
};

int log2_exact(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return (1 << s) == v ? s : -1;
}

// Shape fields of a one-chunk batch; the rest is checked on the view.
sarathi_status view_batch(const sarathi_batch *b, BatchView *v) {
  if (!b) return fail(SARATHI_ERR_INVALID, "batch is null");
  if (b->chunk_len < 0 || b->n_decodes < 0)
    return fail(SARATHI_ERR_INVALID, "chunk_len and n_decodes must be >= 0");
  if (b->reserved != 0) return fail(SARATHI_ERR_INVALID, "batch.reserved must be 0");
  v->paged = false;
  v->decode_tables = nullptr;
  v->n_chunks = b->chunk_len > 0 ? 1 : 0;
  if (v->n_chunks) {
    v->chunks[0].len = b->chunk_len;
    v->chunks[0].offset = b->chunk_offset;
    v->chunks[0].kv = b->chunk_kv;
  }
  v->C = b->chunk_len;
  v->B = b->n_decodes;
  v->decode_kv = b->decode_kv;
  v->decode_len = b->decode_len;
  v->x = b->x;
  v->y = b->y;
  return SARATHI_OK;
}

sarathi_status view_multi(const sarathi_multi_batch *b, BatchView *v) {
  if (!b) return fail(SARATHI_ERR_INVALID, "batch is null");
  if (b->n_chunks < 0 || b->n_chunks > kMaxChunks)
    return fail(SARATHI_ERR_INVALID, "n_chunks %d outside [0, %d]", b->n_chunks, kMaxChunks);
  if (b->n_decodes < 0) return fail(SARATHI_ERR_INVALID, "n_decodes must be >= 0");
  if (b->reserved != 0 || b->reserved2 != 0) return fail(SARATHI_ERR_INVALID, "reserved fields must be 0");
  if (b->n_chunks > 0 && !b->chunks) return fail(SARATHI_ERR_INVALID, "chunks is null");
  v->paged = false;
  v->decode_tables = nullptr;
  v->n_chunks = b->n_chunks;
  long long rows = 0;
  for (int j = 0; j < b->n_chunks; ++j) {
    if (b->chunks[j].len < 1) return fail(SARATHI_ERR_INVALID, "chunk %d has len %d < 1", j, b->chunks[j].len);
    v->chunks[j] = b->chunks[j];
    rows += b->chunks[j].len;
  }
  if (rows > (1 << 30)) return fail(SARATHI_ERR_INVALID, "too many chunk rows");
  v->C = (int)rows;
  v->B = b->n_decodes;
  v->decode_kv = b->decode_kv;
  v->decode_len = b->decode_len;
  v->x = b->x;
  v->y = b->y;
  return SARATHI_OK;
}

sarathi_status view_paged(const sarathi_paged_batch *b, BatchView *v) {
  if (!b) return fail(SARATHI_ERR_INVALID, "batch is null");
  if (b->n_chunks < 0 || b->n_chunks > kMaxChunks)
    return fail(SARATHI_ERR_INVALID, "n_chunks %d outside [0, %d]", b->n_chunks, kMaxChunks);
  if (b->n_decodes < 0) return fail(SARATHI_ERR_INVALID, "n_decodes must be >= 0");
  if (b->reserved != 0 || b->reserved2 != 0) return fail(SARATHI_ERR_INVALID, "reserved fields must be 0");
  if (b->n_chunks > 0 && !b->chunks) return fail(SARATHI_ERR_INVALID, "chunks is null");
  const sarathi_page_pool &pl = b->pool;
  if (!pl.k_pool || !pl.v_pool) return fail(SARATHI_ERR_INVALID, "page pool pointers are null");
  if (pl.n_pages < 1) return fail(SARATHI_ERR_INVALID, "page pool has no pages");
  const int shift = log2_exact(pl.page_size);
  if (pl.page_size < 1 || pl.page_size > 65536 || shift < 0)
    return fail(SARATHI_ERR_INVALID, "page_size %d is not a power of two in [1, 65536]", pl.page_size);
  v->paged = true;
  v->pool = pl;
  v->page_shift = shift;
  auto table_cap = [&](const sarathi_page_table &t, const char *what, int idx, int *cap) {
    if (!t.pages) return fail(SARATHI_ERR_INVALID, "%s %d: block table is null", what, idx);
    if (t.reserved != 0) return fail(SARATHI_ERR_INVALID, "%s %d: table.reserved must be 0", what, idx);
    if (t.n_entries < 1 || (long long)t.n_entries << shift > (1ll << 30))
      return fail(SARATHI_ERR_INVALID, "%s %d: block table size %d out of range", what, idx, t.n_entries);
    *cap = t.n_entries << shift;
    return SARATHI_OK;
  };
  v->n_chunks = b->n_chunks;
  long long rows = 0;
  for (int j = 0; j < b->n_chunks; ++j) {
    const sarathi_paged_chunk &c = b->chunks[j];
    if (c.len < 1) return fail(SARATHI_ERR_INVALID, "chunk %d has len %d < 1", j, c.len);
    int cap = 0;
    const sarathi_status st = table_cap(c.table, "chunk", j, &cap);
    if (st != SARATHI_OK) return st;
    v->chunks[j].len = c.len;
    v->chunks[j].offset = c.offset;
    v->chunks[j].kv.k = const_cast<int32_t *>(c.table.pages);
    v->chunks[j].kv.v = nullptr;
    v->chunks[j].kv.capacity = cap;
    v->chunks[j].kv.reserved = 0;
    rows += c.len;
  }
  if (b->n_decodes > 0 && (!b->decode_tables || !b->decode_len))
    return fail(SARATHI_ERR_INVALID, "decode_tables and decode_len must be non-null when n_decodes > 0");
  for (int i = 0; i < b->n_decodes; ++i) {
    int cap = 0;
    const sarathi_status st = table_cap(b->decode_tables[i], "decode", i, &cap);
    if (st != SARATHI_OK) return st;
  }
  if (rows > (1 << 30)) return fail(SARATHI_ERR_INVALID, "too many chunk rows");
  v->C = (int)rows;
  v->B = b->n_decodes;
  v->decode_kv = nullptr;
  v->decode_tables = b->decode_tables;
  v->decode_len = b->decode_len;
  v->x = b->x;
  v->y = b->y;
  return SARATHI_OK;
}

// need_xy: forward requires x and y; the attention-only entry does not.
sarathi_status check_view(const sarathi_layer_desc *d, const BatchView &b, bool need_xy) {
  sarathi_status st = check_desc(d);
  if (st != SARATHI_OK) return st;
  const int C = b.C, B = b.B;
  if (C + B < 1) return fail(SARATHI_ERR_INVALID, "empty batch (no chunk rows and no decodes)");
  if ((long long)C + B > d->max_tokens)
    return fail(SARATHI_ERR_INVALID, "C+B = %lld exceeds max_tokens %d", (long long)C + B, d->max_tokens);
  if (need_xy && (!b.x || !b.y)) return fail(SARATHI_ERR_INVALID, "x and y must be non-null");
  const size_t el = elem_size(d->dtype);
  const size_t per_slot = (size_t)d->n_heads * d->head_dim * el;
  std::vector<Range> ranges;
  std::vector<uintptr_t> tables;   // paged: every request's block table, to reject shared ones
  for (int j = 0; j < b.n_chunks; ++j) {
    const sarathi_chunk &c = b.chunks[j];
    const sarathi_kv &kv = c.kv;
    if (!b.paged) {
      if (!kv.k || !kv.v) return fail(SARATHI_ERR_INVALID, "chunk %d cache pointers are null", j);
      if (kv.reserved != 0) return fail(SARATHI_ERR_INVALID, "chunk %d kv.reserved must be 0", j);
    }
    if (c.offset < 0) return fail(SARATHI_ERR_INVALID, "chunk %d offset must be >= 0", j);
    if (kv.capacity <= 0 || (long long)c.offset + c.len > kv.capacity)
      return fail(SARATHI_ERR_CAPACITY, "chunk %d: offset %d + len %d exceeds cache capacity %d", j,
                  c.offset, c.len, kv.capacity);
    if ((long long)c.offset + c.len > d->max_pos)
      return fail(SARATHI_ERR_CAPACITY, "chunk %d positions reach %lld >= max_pos %d", j,
                  (long long)c.offset + c.len - 1, d->max_pos);
    if (b.paged) {
      tables.push_back((uintptr_t)kv.k);
    } else {
      ranges.push_back({(uintptr_t)kv.k, (uintptr_t)kv.k + per_slot * kv.capacity, "chunk K", j});
      ranges.push_back({(uintptr_t)kv.v, (uintptr_t)kv.v + per_slot * kv.capacity, "chunk V", j});
    }
  }
  if (B > 0) {
    if ((!b.paged && !b.decode_kv) || !b.decode_len)
      return fail(SARATHI_ERR_INVALID, "decode_kv and decode_len must be non-null when n_decodes > 0");
    for (int i = 0; i < B; ++i) {
      const int L = b.decode_len[i];
      int cap;
      if (b.paged) {
        cap = b.decode_tables[i].n_entries << b.page_shift;
        tables.push_back((uintptr_t)b.decode_tables[i].pages);
      } else {
        const sarathi_kv &kv = b.decode_kv[i];
        if (!kv.k || !kv.v) return fail(SARATHI_ERR_INVALID, "decode %d cache pointers are null", i);
        if (kv.reserved != 0) return fail(SARATHI_ERR_INVALID, "decode_kv[%d].reserved must be 0", i);
        cap = kv.capacity;
        ranges.push_back({(uintptr_t)kv.k, (uintptr_t)kv.k + per_slot * kv.capacity, "decode K", i});
        ranges.push_back({(uintptr_t)kv.v, (uintptr_t)kv.v + per_slot * kv.capacity, "decode V", i});
      }
      if (L < 0) return fail(SARATHI_ERR_INVALID, "decode_len[%d] = %d < 0", i, L);
      if ((long long)L + 1 > cap)
        return fail(SARATHI_ERR_CAPACITY, "decode %d: slot %d does not fit capacity %d", i, L, cap);
      if (L >= d->max_pos)
        return fail(SARATHI_ERR_CAPACITY, "decode %d: position %d >= max_pos %d", i, L, d->max_pos);
    }
  }
  if (b.paged) {
    std::sort(tables.begin(), tables.end());
    for (size_t i = 1; i < tables.size(); ++i)
      if (tables[i] == tables[i - 1])
        return fail(SARATHI_ERR_INVALID, "two requests share one block table");
    const size_t pool_bytes = (size_t)b.pool.n_pages * d->n_heads * b.pool.page_size * d->head_dim * el;
    ranges.push_back({(uintptr_t)b.pool.k_pool, (uintptr_t)b.pool.k_pool + pool_bytes, "K pool", -1});
    ranges.push_back({(uintptr_t)b.pool.v_pool, (uintptr_t)b.pool.v_pool + pool_bytes, "V pool", -1});
  }
  if (need_xy) {
    const size_t rows = (size_t)(C + B) * d->hidden * el;
    ranges.push_back({(uintptr_t)b.y, (uintptr_t)b.y + rows, "y", -1});
    const uintptr_t xl = (uintptr_t)b.x, xh = xl + rows;
    const uintptr_t yl = (uintptr_t)b.y, yh = yl + rows;
    if (xl < yh && yl < xh) return fail(SARATHI_ERR_INVALID, "y overlaps x");
  }
  std::sort(ranges.begin(), ranges.end(),
            [](const Range &a, const Range &c) { return a.lo < c.lo; });
  for (size_t i = 1; i < ranges.size(); ++i)
    if (ranges[i].lo < ranges[i - 1].hi)
      return fail(SARATHI_ERR_INVALID, "%s (%d) overlaps %s (%d): requests must not share caches",
                  ranges[i].what, ranges[i].idx, ranges[i - 1].what, ranges[i - 1].idx);
  return SARATHI_OK;
}


// Workspace layout of one forward.  The GEMM plans are fixed by the shapes alone (planned for the
// 256 compute units of an MI355X), so the workspace size depends only on the description and batch.
constexpr int kPlanCUs = 256;

struct Plan {
  int T, T_alloc, max_splits;   // max_splits: the most key splits of any row (reported by plan_describe)
  int chunk_splits;   // key-range splits of the MFMA chunk kernel (1: it writes the output itself)
  int stride_c;       // attention partials per (chunk row, head): 0 when no chunk row leaves partials
  int stride_d;       // attention partials per (decode row, head)
  GemmPlan qkv, o, up, down;
  GemmPlan up_tail;   // with up_main > 0: the split product of the FFN up columns past up_main
  int up_main;        // 0, or the FFN up columns of the fused part `up` (plan_gemm_tail)
  size_t n1, q, attn, h1, n2, act, part, part_o_c, part_ml_c, part_o_d, part_ml_d, total;
};

#ifndef SARATHI_FUSED_ATTN
#define SARATHI_FUSED_ATTN 1
#endif
constexpr bool kFusedAttention = SARATHI_FUSED_ATTN != 0;

// bf16 chunk rows run the flash-style MFMA kernel; the split-KV kernel (and its partials) serves the
// decode rows, and the chunk rows too in float32 mode.
bool chunk_uses_split(const sarathi_layer_desc *d) { return d->dtype != SARATHI_BF16; }

ChunkSet chunk_set(const BatchView &b) {
  ChunkSet cs{};
  cs.n = b.n_chunks;
  int row = 0;
  for (int j = 0; j < b.n_chunks; ++j) {
    const sarathi_chunk &c = b.chunks[j];
    cs.k[j] = (uint64_t)c.kv.k;
    cs.v[j] = (uint64_t)c.kv.v;
    cs.cap[j] = c.kv.capacity;
    cs.len[j] = c.len;
    cs.off[j] = c.offset;
    cs.row0[j] = row;
    cs.split[j] = 1;
    row += c.len;
  }
  cs.rows = row;
  cs.qblocks = 1;
  return cs;
}

// Attention split partials per (row, head) of the chunk rows: with the split-KV kernel serving them
// (float32) the most splits of any chunk row; with the MFMA kernel the chunk splits when there are
// several, else none (the chunk kernel writes its rows itself).
int chunk_partial_stride(const sarathi_layer_desc *d, const BatchView &b, int chunk_splits) {
  if (!chunk_uses_split(d)) return chunk_splits > 1 ? chunk_splits : 0;
  int ms = 0;
  for (int j = 0; j < b.n_chunks; ++j) ms = std::max(ms, attn_splits(b.chunks[j].offset + b.chunks[j].len));
  return ms;
}

// ... and of the decode rows: the most splits of any decode.
int decode_partial_stride(const BatchView &b) {
  int ms = 1;
  for (int i = 0; i < b.B; ++i) ms = std::max(ms, attn_splits(b.decode_len[i] + 1));
  return ms;
}

// Whether a batch runs its chunk and decode attention in one fused launch: bf16, both kinds of rows,
// and at most one 64-query chunk block per compute unit and head with unsplit key ranges.  With more
// chunk items the shared launch's register and LDS footprint (that of the chunk work) lowers the
// decode splits' occupancy by more than the overlap gains (measured).
bool fused_attention(const sarathi_layer_desc *d, const BatchView &b, const ChunkSet &cs) {
  if (!kFusedAttention || chunk_uses_split(d) || b.C <= 0 || b.B <= 0) return false;
  int work = 0;
  for (int j = 0; j < cs.n; ++j) work += (cs.len[j] + 63) / 64 * d->n_heads;
  return work <= kPlanCUs;
}

// Key-range splits of every chunk for the MFMA chunk kernel, written to cs.split; returns the
// largest.  A fused launch takes them only while its chunk items stay within one per compute unit;
// otherwise its chunks run unsplit.  A fused launch with at least kFusedTwoBlockItems 64-query items
// (contiguous caches) gives each wave two 16-query blocks: half as many items, each sharing its K/V
// tile reads between two blocks, leave more slots to the decode splits (measured +1.5% on the
// llama-13b batch with 160 items; with 48 items the longer items cost 0.8%).
constexpr int kFusedTwoBlockItems = 128;
int plan_chunk_splits(const sarathi_layer_desc *d, const BatchView &b, ChunkSet &cs) {
  for (int j = 0; j < cs.n; ++j) cs.split[j] = 1;
  if (chunk_uses_split(d) || cs.n <= 0) return 1;
  const bool fused = fused_attention(d, b, cs);
  long long cost;
  const int most = fused ? chunk_attn_splits(cs, d->n_heads, 64, kFusedChunkResident, &cost)
                         : chunk_attn_plan(cs, d->n_heads, b.paged);
  if (fused) {
    int items = 0;
    for (int j = 0; j < cs.n; ++j) items += (cs.len[j] + 63) / 64 * cs.split[j] * d->n_heads;
    int result = most;
    if (items > kPlanCUs) {
      for (int j = 0; j < cs.n; ++j) cs.split[j] = 1;
      items = 0;
      for (int j = 0; j < cs.n; ++j) items += (cs.len[j] + 63) / 64 * d->n_heads;
      result = 1;
    }
    cs.qblocks = !b.paged && items >= kFusedTwoBlockItems ? 2 : 1;
    return result;
  }
  return most;
}

Plan make_plan(const sarathi_layer_desc *d, const BatchView &b) {
  Plan p{};
  p.T = b.C + b.B;
  p.T_alloc = round_up(p.T, 64);
  ChunkSet cs = chunk_set(b);
  p.chunk_splits = plan_chunk_splits(d, b, cs);
  p.stride_c = chunk_partial_stride(d, b, p.chunk_splits);
  p.stride_d = decode_partial_stride(b);
  p.max_splits = std::max({p.chunk_splits, p.stride_c, b.B > 0 ? p.stride_d : 1});
  const int ty = d->dtype;
  const size_t el = elem_size(ty), R = p.T_alloc;
  const int H = d->hidden, A = d->n_heads * d->head_dim, F = d->ffn;
  const bool llama = d->arch == SARATHI_ARCH_LLAMA;
  p.qkv = plan_gemm(ty, kEpiPartial, p.T, 3 * A, H, kPlanCUs);
  p.o = plan_gemm(ty, kEpiPartial, p.T, H, A, kPlanCUs);
  p.up = plan_gemm(ty, llama ? kEpiSwiGLU : kEpiGelu, p.T, F, H, kPlanCUs);
  p.up_main = plan_gemm_tail(ty, llama ? kEpiSwiGLU : kEpiGelu, p.T, F, H, kPlanCUs, &p.up, &p.up_tail);
  p.down = plan_gemm(ty, kEpiPartial, p.T, H, F, kPlanCUs);
  const size_t up_cols = p.up.epi == kEpiPartial ? (llama ? 2 * (size_t)F : F) : 0;
  const size_t tail_cols = p.up_main > 0 ? (llama ? 2 : 1) * (size_t)(F - p.up_main) : 0;
  const size_t part_elems = std::max({(size_t)p.qkv.splits * p.T * 3 * A, (size_t)p.o.splits * p.T * H,
                                      (size_t)p.down.splits * p.T * H,
                                      (size_t)p.up.splits * p.T * up_cols,
                                      p.up_main > 0 ? (size_t)p.up_tail.splits * p.T * tail_cols : 0});
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  p.n1 = take(R * H * el);
  p.q = take(R * A * el);
  p.attn = take(R * A * el);
  p.h1 = take(R * H * 4);
  p.n2 = take(R * H * el);
  p.act = take(R * F * el);
  p.part = take(part_elems * 4);
  // attention split partials: only the rows the merge reads (decode rows, and chunk rows when they
  // leave partials)
  const size_t slots_c = (size_t)b.C * d->n_heads * p.stride_c;
  const size_t slots_d = (size_t)b.B * d->n_heads * p.stride_d;
  p.part_o_c = take(slots_c * d->head_dim * 4);
  p.part_ml_c = take(slots_c * 2 * 4);
  p.part_o_d = take(slots_d * d->head_dim * 4);
  p.part_ml_d = take(slots_d * 2 * 4);
  p.total = off;
  return p;
}

PagePool page_pool(const BatchView &b) {
  PagePool p{};
  if (b.paged) {
    p.k = (uint64_t)b.pool.k_pool;
    p.v = (uint64_t)b.pool.v_pool;
    p.n_pages = b.pool.n_pages;
    p.shift = b.page_shift;
  }
  return p;
}

DecodeGroup decode_group(const BatchView &b, int base) {
  DecodeGroup g{};
  g.base = base;
  g.n = std::min(kMaxDecodesPerLaunch, b.B - base);
  if (g.n < 0) g.n = 0;
  for (int i = 0; i < g.n; ++i) {
    if (b.paged) {
      const sarathi_page_table &t = b.decode_tables[base + i];
      g.k[i] = (uint64_t)t.pages;
      g.v[i] = 0;
      g.cap[i] = t.n_entries << b.page_shift;
    } else {
      g.k[i] = (uint64_t)b.decode_kv[base + i].k;
      g.v[i] = (uint64_t)b.decode_kv[base + i].v;
      g.cap[i] = b.decode_kv[base + i].capacity;
    }
    g.len[i] = b.decode_len[base + i];
  }
  return g;
}

// A bf16 layer's projection weights, copied once into one device buffer, each k-tile-major
// [k/32][rows][32]: the GEMM's 32-deep k-tiles of a weight stripe are then whole 128-byte lines
// (two rows per line) instead of half lines of row-major rows, and a stripe's k-tile is 8 KiB of
// consecutive bytes.  The caller's weight buffers are not read after this.
constexpr int kWeightTile = 32;
sarathi_status pack_weights(sarathi_layer *L) {
  const sarathi_layer_desc *d = &L->desc;
  const int H = d->hidden, A = d->n_heads * d->head_dim, F = d->ffn;
  struct Mat {
    const void **w;
    int rows, k;
  } mats[5] = {{&L->w.w_qkv, 3 * A, H}, {&L->w.w_o, H, A}, {&L->w.w_gate, F, H}, {&L->w.w_up, F, H},
               {&L->w.w_down, H, F}};
  size_t ofs[5], total = 0;
  for (int i = 0; i < 5; ++i) {
    ofs[i] = total;
    if (*mats[i].w) total += ((size_t)mats[i].rows * mats[i].k * 2 + 255) / 256 * 256;
  }
  hipError_t e = hipMalloc(&L->wpack, total);
  if (e != hipSuccess) {
    L->wpack = nullptr;
    return fail(SARATHI_ERR_NOMEM, "hipMalloc of %zu bytes of packed weights failed: %s", total,
                hipGetErrorString(e));
  }
  for (int i = 0; i < 5; ++i) {
    if (!*mats[i].w) continue;
    void *dst = static_cast<char *>(L->wpack) + ofs[i];
    e = launch_pack_kmajor(*mats[i].w, mats[i].rows, mats[i].k, mats[i].k, kWeightTile, dst, nullptr);
    if (e != hipSuccess) return fail(SARATHI_ERR_HIP, "packing weight %d failed: %s", i, hipGetErrorString(e));
    *mats[i].w = dst;
  }
  e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) return fail(SARATHI_ERR_HIP, "packing the weights failed: %s", hipGetErrorString(e));
  L->wk = kWeightTile;
  return SARATHI_OK;
}

// Weight operands of a GEMM of layer L: w0 with rows0 rows, w1 (or null) with rows1; each [rows, k]
// row-major (f32 layers) or packed (bf16 layers).
void set_weights(GemmArgs &g, const sarathi_layer *L, const void *w0, int rows0, const void *w1, int rows1,
                 int k) {
  g.w0 = w0;
  g.w1 = w1;
  g.ldw = k;
  g.w_kmajor = L->wk;
  g.w_slab0 = rows0 * L->wk;
  g.w_slab1 = w1 ? rows1 * L->wk : 0;
}

#define HIP_TRY(expr)                                                                     \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess)                                                                 \
      return fail(SARATHI_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));        \
  } while (0)

// Records the timer's events around the timed stages (nothing when there is no timer).
struct Marker {
  sarathi_timer *t = nullptr;
  hipStream_t s = nullptr;
  int f = 0;
  hipEvent_t ev(int stage, int which) const {
    return t->ev[((size_t)f * t->n_timed + t->slot[stage]) * 2 + which];
  }
  void begin() {
    if (t) {
      f = t->used;
      t->ran[f] = 0;
    }
  }
  hipError_t start(int stage) {
    if (!t || !(t->mask >> stage & 1u)) return hipSuccess;
    return hipEventRecord(ev(stage, 0), s);
  }
  hipError_t end(int stage, bool ran) {
    if (!t || !(t->mask >> stage & 1u)) return hipSuccess;
    if (ran) t->ran[f] |= 1u << stage;
    return hipEventRecord(ev(stage, 1), s);
  }
  void commit() {
    if (t) t->used++;
  }
};

// Attention of all batch rows, split per request: chunk rows (all chunks in one launch), then
// decode rows (64 per launch group), then one merge of the split partials; writes out [T, A]
// (storage type).
sarathi_status run_attention(const sarathi_layer_desc *d, const BatchView &b, const Plan &p,
                             const void *q, void *out, const OutLayout &olay, char *ws, hipStream_t s,
                             Marker &mk) {
  const int A = d->n_heads * d->head_dim;
  const int C = b.C, B = b.B;
  ChunkSet cs = chunk_set(b);
  plan_chunk_splits(d, b, cs);   // the same counts as p.chunk_splits (their largest)
  const PagePool pool = page_pool(b);
  AttnParts parts{};
  if (p.stride_c > 0) {
    parts.o_c = reinterpret_cast<float *>(ws + p.part_o_c);
    parts.ml_c = reinterpret_cast<float *>(ws + p.part_ml_c);
    parts.stride_c = p.stride_c;
  }
  parts.o_d = reinterpret_cast<float *>(ws + p.part_o_d);
  parts.ml_d = reinterpret_cast<float *>(ws + p.part_ml_d);
  parts.stride_d = p.stride_d;
  const bool split_chunk = chunk_uses_split(d);
  // Batches with chunk rows and decode rows run both attentions in one launch when fused_attention
  // says so (few chunk items): the decode splits then fill the units the latency-bound chunk work
  // leaves idle.  The fused launch's time is recorded as the decode stage.
  const bool fused = fused_attention(d, b, cs);
  HIP_TRY(mk.start(SARATHI_STAGE_ATTN_CHUNK));
  if (C > 0 && !fused) {
    if (split_chunk) {
      const DecodeGroup none = decode_group(b, B);   // empty group
      HIP_TRY(launch_attn_rows(d->dtype, d->head_dim, q, A, d->n_heads, 0, C, cs, none, pool,
                               p.stride_c, 0, parts.o_c, parts.ml_c, s));
    } else {
      HIP_TRY(launch_attn_chunk(d->head_dim, q, A, d->n_heads, cs, pool, out, olay, p.chunk_splits,
                                std::max(p.stride_c, 1), parts.o_c, parts.ml_c, s));
    }
  }
  HIP_TRY(mk.end(SARATHI_STAGE_ATTN_CHUNK, C > 0 && !fused));
  HIP_TRY(mk.start(SARATHI_STAGE_ATTN_DECODE));
  for (int base = 0; base < B; base += kMaxDecodesPerLaunch) {
    const DecodeGroup g = decode_group(b, base);
    if (fused && base == 0)
      HIP_TRY(launch_attn_fused(d->head_dim, q, A, d->n_heads, cs, pool, out, olay, p.chunk_splits, parts,
                                g, C, g.n, s));
    else
      HIP_TRY(launch_attn_rows(d->dtype, d->head_dim, q, A, d->n_heads, C + base, g.n, cs, g, pool,
                               p.stride_d, C, parts.o_d, parts.ml_d, s));
  }
  HIP_TRY(mk.end(SARATHI_STAGE_ATTN_DECODE, B > 0));
  HIP_TRY(mk.start(SARATHI_STAGE_ATTN_MERGE));
  // Chunk rows need merging when the split-KV kernel served them (all their splits) or their chunk
  // was split by the MFMA kernel (the merge reads each chunk's count from the table and leaves the
  // rows of unsplit chunks alone).
  const bool merge_chunk = p.stride_c > 0;
  const int merge_row0 = merge_chunk ? 0 : C;
  const int chunk_splits = split_chunk ? p.stride_c : 0;
  ChunkSplits table{};
  table.n = cs.n;
  for (int j = 0; j < cs.n; ++j) {
    table.row0[j] = cs.row0[j];
    table.split[j] = cs.split[j];
  }
  if (C + B > merge_row0)
    HIP_TRY(launch_attn_combine(d->dtype, d->head_dim, d->n_heads, merge_row0, C + B - merge_row0, C,
                                chunk_splits, table, parts, out, olay, s));
  HIP_TRY(mk.end(SARATHI_STAGE_ATTN_MERGE, C + B > merge_row0));
  return SARATHI_OK;
}

// n1_ready: norm 1 of x is already in the n1 region (written by the previous layer of a stack);
// next: the following layer of a stack, whose norm 1 this forward then computes with its own output.
sarathi_status forward_impl(sarathi_layer *L, const BatchView &b, void *workspace, size_t ws_bytes,
                            void *stream, const sarathi_debug_dump *dump, sarathi_timer *timer,
                            bool n1_ready = false, const sarathi_layer *next = nullptr) {
  if (!L) return fail(SARATHI_ERR_INVALID, "layer is null");
  const sarathi_layer_desc *d = &L->desc;
  sarathi_status st = check_view(d, b, true);
  if (st != SARATHI_OK) return st;
  const Plan p = make_plan(d, b);
  if (!workspace) return fail(SARATHI_ERR_WORKSPACE, "workspace is null");
  if ((uintptr_t)workspace % 256) return fail(SARATHI_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (ws_bytes < p.total)
    return fail(SARATHI_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, p.total);
  if (timer && timer->used >= timer->capacity)
    return fail(SARATHI_ERR_INVALID, "timer is full (%d unread forwards)", timer->used);

  hipStream_t s = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  Marker mk;
  mk.t = timer;
  mk.s = s;
  mk.begin();
  const int ty = d->dtype, T = p.T, R = p.T_alloc;
  const int H = d->hidden, A = d->n_heads * d->head_dim, F = d->ffn;
  const bool llama = d->arch == SARATHI_ARCH_LLAMA;
  void *n1 = ws + p.n1, *q = ws + p.q, *attn = ws + p.attn;
  float *h1 = reinterpret_cast<float *>(ws + p.h1);
  float *part = reinterpret_cast<float *>(ws + p.part);
  void *n2 = ws + p.n2, *act = ws + p.act;
  // bf16: the norms write the QKV and gate/up GEMMs' inputs k-tile-major ([H/w][R][w], w = the
  // consuming GEMM's stage depth)
  const int kmajor1 = ty == kBF16 ? gemm_stage_depth(p.qkv) : 0;
  const int kmajor2 = ty == kBF16 ? gemm_stage_depth(p.up) : 0;
  // ... and the FFN activation k-tile-major for a down GEMM with 32-deep stages (its rows are then
  // whole 64-byte blocks; with 64-deep stages row-major rows are whole 128-byte lines already)
  const int kmajor_act = ty == kBF16 && gemm_stage_depth(p.down) == 32 ? 32 : 0;
  const int kmajor_attn = ty == kBF16 && gemm_stage_depth(p.o) == 32 ? 32 : 0;   // same, O GEMM input

  // 1. norm 1 over the C+B rows (pad rows zeroed)
  HIP_TRY(mk.start(SARATHI_STAGE_NORM1));
  if (!n1_ready)
    HIP_TRY(launch_norm_rows(ty, ty, !llama, b.x, nullptr, 0, nullptr, nullptr, L->w.norm1_w,
                             L->w.norm1_b, n1, H, T, R, d->norm_eps, kmajor1, s));
  HIP_TRY(mk.end(SARATHI_STAGE_NORM1, true));
  // 2. QKV projection: one GEMM over chunk and decode rows (float32 split partials)
  HIP_TRY(mk.start(SARATHI_STAGE_QKV));
  GemmArgs g{};
  g.a = n1; g.lda = H; g.a_kmajor = kmajor1; g.part = part;
  set_weights(g, L, L->w.w_qkv, 3 * A, nullptr, 0, H);
  g.m_alloc = R; g.m_store = T; g.n = 3 * A; g.k = H;
  HIP_TRY(launch_gemm(ty, kEpiPartial, g, p.qkv, s));
  HIP_TRY(mk.end(SARATHI_STAGE_QKV, true));
  // 3. sum of the partials + RoPE + KV append: the chunk rows with the first decode group, then the
  // other decode groups
  const ChunkSet cs = chunk_set(b);
  const PagePool pool = page_pool(b);
  HIP_TRY(mk.start(SARATHI_STAGE_ROPE_APPEND));
  {
    int base = 0;
    do {
      const DecodeGroup dg = decode_group(b, base);
      const int row0 = base == 0 ? 0 : b.C + base;
      const int n_rows = (base == 0 ? b.C : 0) + dg.n;
      HIP_TRY(launch_rope_append(ty, part, p.qkv.splits, T, q, A, dump ? dump->qkv : nullptr,
                                 L->rope_tab, llama ? 1 : 0, d->n_heads, d->head_dim, row0, n_rows,
                                 cs, dg, pool, s));
      base += kMaxDecodesPerLaunch;
    } while (base < b.B);
  }
  HIP_TRY(mk.end(SARATHI_STAGE_ROPE_APPEND, true));
  // 4. attention, split per request
  st = run_attention(d, b, p, q, attn, OutLayout{A, kmajor_attn, R}, ws, s, mk);
  if (st != SARATHI_OK) return st;
  // 5. O projection (float32 split partials)
  HIP_TRY(mk.start(SARATHI_STAGE_O));
  g = GemmArgs{};
  g.a = attn; g.lda = A; g.a_kmajor = kmajor_attn; g.part = part;
  set_weights(g, L, L->w.w_o, H, nullptr, 0, A);
  g.m_alloc = R; g.m_store = T; g.n = H; g.k = A;
  HIP_TRY(launch_gemm(ty, kEpiPartial, g, p.o, s));
  HIP_TRY(mk.end(SARATHI_STAGE_O, true));
  // 6. h1 = x + sum of the O partials (kept in float32), then norm 2
  HIP_TRY(mk.start(SARATHI_STAGE_NORM2));
  HIP_TRY(launch_norm_rows(ty, ty, !llama, b.x, part, p.o.splits, h1, nullptr, L->w.norm2_w,
                           L->w.norm2_b, n2, H, T, R, d->norm_eps, kmajor2, s));
  HIP_TRY(mk.end(SARATHI_STAGE_NORM2, true));
  // 7. FFN up (+gate): activation fused into the GEMM, or split product + activation pass
  HIP_TRY(mk.start(SARATHI_STAGE_FFN_UP));
  g = GemmArgs{};
  g.a = n2; g.lda = H; g.a_kmajor = kmajor2; g.m_alloc = R; g.m_store = T; g.k = H;
  set_weights(g, L, llama ? L->w.w_gate : L->w.w_up, F, llama ? L->w.w_up : nullptr, F, H);
  if (p.up.epi == kEpiPartial) {
    g.part = part; g.n = llama ? 2 * F : F; g.n_w0 = F;
    HIP_TRY(launch_gemm(ty, kEpiPartial, g, p.up, s));
    HIP_TRY(launch_ffn_act(ty, llama, part, p.up.splits, act, T, F, 0, F, kmajor_act, R, s));
  } else {
    g.out = act; g.ldo = F; g.n = p.up_main > 0 ? p.up_main : F; g.out_kmajor = kmajor_act;
    HIP_TRY(launch_gemm(ty, p.up.epi, g, p.up, s));
    if (p.up_main > 0) {
      // the columns past up_main: split product of their weight rows, then the activation pass
      const int n_tail = F - p.up_main;
      // row up_main of a weight: a row offset within each k-tile when packed
      const size_t wofs = (size_t)p.up_main * (L->wk ? L->wk : H) * elem_size(ty);
      GemmArgs t = g;
      t.out = nullptr; t.ldo = 0; t.out_kmajor = 0;
      t.w0 = static_cast<const char *>(g.w0) + wofs;
      t.w1 = g.w1 ? static_cast<const char *>(g.w1) + wofs : nullptr;
      t.part = part; t.n = llama ? 2 * n_tail : n_tail; t.n_w0 = n_tail;
      HIP_TRY(launch_gemm(ty, kEpiPartial, t, p.up_tail, s));
      HIP_TRY(launch_ffn_act(ty, llama, part, p.up_tail.splits, act, T, n_tail, p.up_main, F, kmajor_act,
                             R, s));
    }
  }
  HIP_TRY(mk.end(SARATHI_STAGE_FFN_UP, true));
  // 8. down projection (split partials), y = h1 + sum of the partials
  HIP_TRY(mk.start(SARATHI_STAGE_FFN_DOWN));
  g = GemmArgs{};
  g.a = act; g.lda = F; g.a_kmajor = kmajor_act; g.part = part;
  set_weights(g, L, L->w.w_down, H, nullptr, 0, F);
  g.m_alloc = R; g.m_store = T; g.n = H; g.k = F;
  HIP_TRY(launch_gemm(ty, kEpiPartial, g, p.down, s));
  if (next) {
    // y = h1 + sum of the partials, stored, and the next layer's norm 1 of y into the n1 region
    // (offset 0 of every layer's plan, the same size for layers of one hidden size)
    const sarathi_layer_desc *dn = &next->desc;
    const int A_next = dn->n_heads * dn->head_dim;
    const int kmajor1_next = ty == kBF16 ? gemm_stage_depth(plan_gemm(ty, kEpiPartial, T, 3 * A_next, H, kPlanCUs)) : 0;
    HIP_TRY(launch_norm_rows(kF32, ty, dn->arch != SARATHI_ARCH_LLAMA, h1, part, p.down.splits, nullptr,
                             b.y, next->w.norm1_w, next->w.norm1_b, n1, H, T, R, dn->norm_eps,
                             kmajor1_next, s));
  } else {
    HIP_TRY(launch_resid_sum(ty, h1, part, p.down.splits, b.y, T, H, s));
  }
  HIP_TRY(mk.end(SARATHI_STAGE_FFN_DOWN, true));
  mk.commit();

  if (dump) {
    if (dump->n1)
      HIP_TRY(kmajor1 ? launch_kmajor_to_f32(ty, n1, kmajor1, R, dump->n1, H, T, H, s)
                     : launch_to_f32(ty, n1, H, dump->n1, H, T, H, s));
    if (dump->q_rot) HIP_TRY(launch_to_f32(ty, q, A, dump->q_rot, A, T, A, s));
    if (dump->attn)
      HIP_TRY(kmajor_attn ? launch_kmajor_to_f32(ty, attn, kmajor_attn, R, dump->attn, A, T, A, s)
                          : launch_to_f32(ty, attn, A, dump->attn, A, T, A, s));
    if (dump->h1) HIP_TRY(launch_to_f32(kF32, h1, H, dump->h1, H, T, H, s));
    if (dump->n2)
      HIP_TRY(kmajor2 ? launch_kmajor_to_f32(ty, n2, kmajor2, R, dump->n2, H, T, H, s)
                     : launch_to_f32(ty, n2, H, dump->n2, H, T, H, s));
    if (dump->act)
      HIP_TRY(kmajor_act ? launch_kmajor_to_f32(ty, act, kmajor_act, R, dump->act, F, T, F, s)
                         : launch_to_f32(ty, act, F, dump->act, F, T, F, s));
  }
  return SARATHI_OK;
}

sarathi_status make_view(const sarathi_batch *b, BatchView *v) { return view_batch(b, v); }
sarathi_status make_view(const sarathi_multi_batch *b, BatchView *v) { return view_multi(b, v); }
sarathi_status make_view(const sarathi_paged_batch *b, BatchView *v) { return view_paged(b, v); }

// Validation of a batch of either kind: the description first, then the batch.
template <typename Batch>
sarathi_status checked_view(const sarathi_layer_desc *d, const Batch *b, bool need_xy, BatchView *v) {
  sarathi_status st = check_desc(d);
  if (st != SARATHI_OK) return st;
  st = make_view(b, v);
  if (st != SARATHI_OK) return st;
  return check_view(d, *v, need_xy);
}

template <typename Batch>
size_t workspace_bytes(const sarathi_layer_desc *d, const Batch *b) {
  BatchView v;
  if (checked_view(d, b, false, &v) != SARATHI_OK) return 0;
  return make_plan(d, v).total;
}

sarathi_gemm_plan gemm_info(const GemmPlan &g) {
  sarathi_gemm_plan out{};
  out.epilogue = g.epi;
  out.row_tiles = g.m_tiles;
  out.col_tiles = g.n_tiles;
  out.k_splits = g.splits;
  out.tile_cols = g.epi == kEpiSwiGLU ? g.bn / 2 : g.bn;
  return out;
}

template <typename Batch>
sarathi_status describe_entry(const sarathi_layer_desc *d, const Batch *b, sarathi_plan_info *info) {
  if (!info) return fail(SARATHI_ERR_INVALID, "info is null");
  BatchView v;
  const sarathi_status st = checked_view(d, b, false, &v);
  if (st != SARATHI_OK) return st;
  const Plan p = make_plan(d, v);
  ChunkSet cs = chunk_set(v);
  plan_chunk_splits(d, v, cs);
  sarathi_plan_info out{};
  out.rows = p.T;
  out.rows_alloc = p.T_alloc;
  out.n_chunks = cs.n;
  out.fused_attention = fused_attention(d, v, cs) ? 1 : 0;
  for (int j = 0; j < cs.n; ++j) out.chunk_splits[j] = cs.split[j];
  out.max_key_splits = p.max_splits;
  out.chunk_query_blocks = cs.qblocks;
  out.qkv = gemm_info(p.qkv);
  out.o = gemm_info(p.o);
  out.up = gemm_info(p.up);
  out.down = gemm_info(p.down);
  if (p.up_main > 0) out.up_tail = gemm_info(p.up_tail);
  out.workspace_bytes = p.total;
  *info = out;
  return SARATHI_OK;
}

template <typename Batch>
sarathi_status forward_entry(sarathi_layer *L, const Batch *b, void *workspace, size_t ws_bytes,
                             void *stream, const sarathi_debug_dump *dump, sarathi_timer *timer) {
  if (!L) return fail(SARATHI_ERR_INVALID, "layer is null");
  BatchView v;
  const sarathi_status st = checked_view(&L->desc, b, true, &v);
  if (st != SARATHI_OK) return st;
  return forward_impl(L, v, workspace, ws_bytes, stream, dump, timer);
}

static_assert(SARATHI_MAX_CHUNKS == kMaxChunks, "chunk table size");


}  // namespace

extern "C" {

sarathi_status sarathi_layer_create(const sarathi_layer_desc *desc, const sarathi_weights *weights,
                                    sarathi_layer **out) {
  if (!out) return fail(SARATHI_ERR_INVALID, "out is null");
  *out = nullptr;
  sarathi_status st = check_desc(desc);
  if (st != SARATHI_OK) return st;
  if (!weights) return fail(SARATHI_ERR_INVALID, "weights is null");
  const bool llama = desc->arch == SARATHI_ARCH_LLAMA;
  if (!weights->w_qkv || !weights->w_o || !weights->w_up || !weights->w_down || !weights->norm1_w ||
      !weights->norm2_w)
    return fail(SARATHI_ERR_INVALID, "a required weight pointer is null");
  if (llama && !weights->w_gate) return fail(SARATHI_ERR_INVALID, "w_gate is required for LLAMA");
  if (!llama && (!weights->norm1_b || !weights->norm2_b))
    return fail(SARATHI_ERR_INVALID, "LayerNorm biases are required for GPT");
  // every weight is read in 16-byte pieces (the packing copy, the GEMM, the norms)
  const void *all[9] = {weights->w_qkv, weights->w_o, llama ? weights->w_gate : nullptr, weights->w_up,
                        weights->w_down, weights->norm1_w, weights->norm2_w,
                        llama ? nullptr : weights->norm1_b, llama ? nullptr : weights->norm2_b};
  for (const void *w : all)
    if ((uintptr_t)w % 16) return fail(SARATHI_ERR_INVALID, "weight pointer %p is not 16-byte aligned", w);
  sarathi_layer *L = new (std::nothrow) sarathi_layer();
  if (!L) return fail(SARATHI_ERR_NOMEM, "host allocation failed");
  L->desc = *desc;
  L->w = *weights;
  if (!llama) L->w.w_gate = nullptr;
  L->rope_tab = nullptr;
  L->wpack = nullptr;
  L->wk = 0;
  if (hipGetDevice(&L->device) != hipSuccess) {
    delete L;
    return fail(SARATHI_ERR_HIP, "hipGetDevice failed");
  }
  if (desc->dtype == SARATHI_BF16) {
    st = pack_weights(L);
    if (st != SARATHI_OK) {
      if (L->wpack) (void)hipFree(L->wpack);
      delete L;
      return st;
    }
  }
  if (llama) {
    const int half = desc->head_dim / 2;
    std::vector<float2> tab((size_t)desc->max_pos * half);
    for (int pos = 0; pos < desc->max_pos; ++pos)
      for (int j = 0; j < half; ++j) {
        const double inv = std::pow((double)desc->rope_base, -2.0 * j / desc->head_dim);
        const double ang = (double)pos * inv;
        tab[(size_t)pos * half + j] = make_float2((float)std::cos(ang), (float)std::sin(ang));
      }
    const size_t bytes = tab.size() * sizeof(float2);
    hipError_t e = hipMalloc(&L->rope_tab, bytes);
    if (e != hipSuccess) {
      delete L;
      return fail(SARATHI_ERR_NOMEM, "hipMalloc of the RoPE table failed: %s", hipGetErrorString(e));
    }
    e = hipMemcpy(L->rope_tab, tab.data(), bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(L->rope_tab);
      delete L;
      return fail(SARATHI_ERR_HIP, "copying the RoPE table failed: %s", hipGetErrorString(e));
    }
  }
  // Set-up of the no-allocation forward: find this device's copy of the fixed scratch now, with the
  // device current.  A failure here only matters to that entry point, which looks it up again.
  void *scratch = nullptr;
  (void)noalloc_scratch(L->device, &scratch);
  *out = L;
  return SARATHI_OK;
}

void sarathi_layer_destroy(sarathi_layer *layer) {
  if (!layer) return;
  if (layer->rope_tab) (void)hipFree(layer->rope_tab);
  if (layer->wpack) (void)hipFree(layer->wpack);
  delete layer;
}

sarathi_status sarathi_batch_check(const sarathi_layer_desc *desc, const sarathi_batch *batch) {
  BatchView v;
  return checked_view(desc, batch, true, &v);
}

size_t sarathi_workspace_size(const sarathi_layer_desc *desc, const sarathi_batch *batch) {
  return workspace_bytes(desc, batch);
}

sarathi_status sarathi_layer_forward(sarathi_layer *layer, const sarathi_batch *batch,
                                     void *workspace, size_t ws_bytes, void *stream) {
  return forward_entry(layer, batch, workspace, ws_bytes, stream, nullptr, nullptr);
}

sarathi_status sarathi_layer_forward_noalloc(sarathi_layer *layer, const sarathi_batch *batch,
                                             void *stream) {
  if (!layer) return fail(SARATHI_ERR_INVALID, "layer is null");
  BatchView v;
  const sarathi_status st = checked_view(&layer->desc, batch, true, &v);
  if (st != SARATHI_OK) return st;
  const size_t need = make_plan(&layer->desc, v).total;
  if (need > kNoAllocScratchBytes)
    return fail(SARATHI_ERR_WORKSPACE,
                "batch needs %zu bytes of workspace, more than the %zu-byte fixed scratch of the "
                "no-allocation forward (use sarathi_layer_forward with a workspace)",
                need, kNoAllocScratchBytes);
  int device = -1;
  HIP_TRY(hipGetDevice(&device));
  if (device != layer->device)
    return fail(SARATHI_ERR_INVALID, "current device %d is not the layer's device %d", device,
                layer->device);
  void *scratch = nullptr;
  HIP_TRY(noalloc_scratch(device, &scratch));
  return forward_impl(layer, v, scratch, kNoAllocScratchBytes, stream, nullptr, nullptr);
}

sarathi_status sarathi_layer_forward_debug(sarathi_layer *layer, const sarathi_batch *batch,
                                           void *workspace, size_t ws_bytes, void *stream,
                                           const sarathi_debug_dump *dump) {
  return forward_entry(layer, batch, workspace, ws_bytes, stream, dump, nullptr);
}

sarathi_status sarathi_multi_batch_check(const sarathi_layer_desc *desc,
                                         const sarathi_multi_batch *batch) {
  BatchView v;
  return checked_view(desc, batch, true, &v);
}

size_t sarathi_multi_workspace_size(const sarathi_layer_desc *desc, const sarathi_multi_batch *batch) {
  return workspace_bytes(desc, batch);
}

sarathi_status sarathi_multi_forward(sarathi_layer *layer, const sarathi_multi_batch *batch,
                                     void *workspace, size_t ws_bytes, void *stream) {
  return forward_entry(layer, batch, workspace, ws_bytes, stream, nullptr, nullptr);
}

sarathi_status sarathi_multi_forward_debug(sarathi_layer *layer, const sarathi_multi_batch *batch,
                                           void *workspace, size_t ws_bytes, void *stream,
                                           const sarathi_debug_dump *dump) {
  return forward_entry(layer, batch, workspace, ws_bytes, stream, dump, nullptr);
}

sarathi_status sarathi_paged_batch_check(const sarathi_layer_desc *desc,
                                         const sarathi_paged_batch *batch) {
  BatchView v;
  return checked_view(desc, batch, true, &v);
}

size_t sarathi_paged_workspace_size(const sarathi_layer_desc *desc, const sarathi_paged_batch *batch) {
  return workspace_bytes(desc, batch);
}

sarathi_status sarathi_paged_forward(sarathi_layer *layer, const sarathi_paged_batch *batch,
                                     void *workspace, size_t ws_bytes, void *stream) {
  return forward_entry(layer, batch, workspace, ws_bytes, stream, nullptr, nullptr);
}

sarathi_status sarathi_paged_forward_debug(sarathi_layer *layer, const sarathi_paged_batch *batch,
                                           void *workspace, size_t ws_bytes, void *stream,
                                           const sarathi_debug_dump *dump) {
  return forward_entry(layer, batch, workspace, ws_bytes, stream, dump, nullptr);
}

sarathi_status sarathi_gemm(int32_t dtype, int32_t m, int32_t n, int32_t k, const void *a,
                            const void *w, void *out, void *stream) {
  if (dtype != SARATHI_F32 && dtype != SARATHI_BF16)
    return fail(SARATHI_ERR_INVALID, "unknown dtype %d", dtype);
  if (m <= 0 || n <= 0 || k <= 0) return fail(SARATHI_ERR_INVALID, "m, n, k must be positive");
  if (!a || !w || !out) return fail(SARATHI_ERR_INVALID, "null pointer");
  if (dtype == SARATHI_BF16 && k % 64)
    return fail(SARATHI_ERR_UNSUPPORTED, "bf16 GEMM needs k %% 64 == 0 (k = %d)", k);
  GemmArgs g{};
  g.a = a; g.lda = k; g.w0 = w; g.ldw = k; g.out = out; g.ldo = n;
  g.m_alloc = m; g.m_store = m; g.n = n; g.k = k;
  const GemmPlan plan = plan_gemm(dtype, kEpiStore, m, n, k, kPlanCUs);
  HIP_TRY(launch_gemm(dtype, kEpiStore, g, plan, static_cast<hipStream_t>(stream)));
  return SARATHI_OK;
}

// ---------------------------------------------------------------------------------------------
// Stack of layers: layer l's batch is the stack batch with its own caches and with x / y chained
// through two activation buffers placed after the (largest) per-layer workspace.

namespace {

sarathi_batch stack_layer_batch(const sarathi_stack_batch *b, int l, const void *x, void *y) {
  sarathi_batch bl{};
  bl.chunk_len = b->chunk_len;
  bl.chunk_offset = b->chunk_offset;
  if (b->chunk_len > 0 && b->chunk_kv) bl.chunk_kv = b->chunk_kv[l];
  bl.n_decodes = b->n_decodes;
  bl.reserved = b->reserved;
  bl.decode_kv = b->n_decodes > 0 && b->decode_kv ? b->decode_kv + (size_t)l * b->n_decodes : nullptr;
  bl.decode_len = b->decode_len;
  bl.x = x;
  bl.y = y;
  return bl;
}

struct StackPlan {
  size_t layer_ws, act_bytes, total;
};

// Validates every layer's batch (before anything is launched) and sizes the workspace.
sarathi_status stack_plan(sarathi_layer *const *layers, int n, const sarathi_stack_batch *b,
                          bool report, StackPlan *out) {
  auto bad = [&](sarathi_status st, const char *msg) { return report ? fail(st, "%s", msg) : st; };
  if (!layers || n < 1) return bad(SARATHI_ERR_INVALID, "no layers");
  if (!b) return bad(SARATHI_ERR_INVALID, "batch is null");
  if (b->chunk_len > 0 && !b->chunk_kv) return bad(SARATHI_ERR_INVALID, "chunk_kv is null");
  if (b->n_decodes > 0 && !b->decode_kv) return bad(SARATHI_ERR_INVALID, "decode_kv is null");
  for (int l = 0; l < n; ++l)
    if (!layers[l]) return bad(SARATHI_ERR_INVALID, "a layer handle is null");
  const sarathi_layer_desc &d0 = layers[0]->desc;
  StackPlan p{};
  for (int l = 0; l < n; ++l) {
    const sarathi_layer_desc &d = layers[l]->desc;
    if (d.hidden != d0.hidden || d.dtype != d0.dtype)
      return report ? fail(SARATHI_ERR_INVALID, "layer %d: hidden size or storage type differs from layer 0", l)
                    : SARATHI_ERR_INVALID;
    const sarathi_batch bl = stack_layer_batch(b, l, b->x, b->y);
    BatchView v;
    const sarathi_status st = checked_view(&d, &bl, true, &v);
    if (st != SARATHI_OK) return st;
    p.layer_ws = std::max(p.layer_ws, make_plan(&d, v).total);
  }
  const size_t T = (size_t)b->chunk_len + b->n_decodes;
  p.act_bytes = n > 1 ? align256(T * d0.hidden * elem_size(d0.dtype)) : 0;
  p.total = align256(p.layer_ws) + 2 * p.act_bytes;
  *out = p;
  return SARATHI_OK;
}

}  // namespace

size_t sarathi_stack_workspace_size(sarathi_layer *const *layers, int32_t n_layers,
                                    const sarathi_stack_batch *batch) {
  StackPlan p;
  if (stack_plan(layers, n_layers, batch, false, &p) != SARATHI_OK) return 0;
  return p.total;
}

sarathi_status sarathi_stack_forward(sarathi_layer *const *layers, int32_t n_layers,
                                     const sarathi_stack_batch *batch, void *workspace,
                                     size_t ws_bytes, void *stream) {
  StackPlan p;
  sarathi_status st = stack_plan(layers, n_layers, batch, true, &p);
  if (st != SARATHI_OK) return st;
  if (!workspace) return fail(SARATHI_ERR_WORKSPACE, "workspace is null");
  if ((uintptr_t)workspace % 256) return fail(SARATHI_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (ws_bytes < p.total)
    return fail(SARATHI_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, p.total);
  char *ws = static_cast<char *>(workspace);
  void *act[2] = {ws + align256(p.layer_ws), ws + align256(p.layer_ws) + p.act_bytes};
  for (int l = 0; l < n_layers; ++l) {
    const void *x = l == 0 ? batch->x : act[(l - 1) & 1];
    void *y = l == n_layers - 1 ? batch->y : act[l & 1];
    const sarathi_batch bl = stack_layer_batch(batch, l, x, y);
    // Each layer but the last ends with the next layer's norm 1 (fused with its output sum), so
    // each layer but the first starts at its QKV GEMM.
    BatchView v;
    st = checked_view(&layers[l]->desc, &bl, true, &v);
    if (st != SARATHI_OK) return st;
    st = forward_impl(layers[l], v, ws, p.layer_ws, stream, nullptr, nullptr, l > 0,
                      l + 1 < n_layers ? layers[l + 1] : nullptr);
    if (st != SARATHI_OK) return st;
  }
  return SARATHI_OK;
}

sarathi_status sarathi_attention(const sarathi_layer_desc *desc, const sarathi_batch *batch,
                                 const void *q, void *out, void *workspace, size_t ws_bytes,
                                 void *stream) {
  BatchView v;
  sarathi_status st = checked_view(desc, batch, false, &v);
  if (st != SARATHI_OK) return st;
  if (!q || !out) return fail(SARATHI_ERR_INVALID, "q and out must be non-null");
  const Plan p = make_plan(desc, v);
  if (!workspace) return fail(SARATHI_ERR_WORKSPACE, "workspace is null");
  if ((uintptr_t)workspace % 256) return fail(SARATHI_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (ws_bytes < p.total)
    return fail(SARATHI_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, p.total);
  Marker none;
  const int A = desc->n_heads * desc->head_dim;
  return run_attention(desc, v, p, q, out, OutLayout{A, 0, p.T}, static_cast<char *>(workspace),
                       static_cast<hipStream_t>(stream), none);
}

sarathi_status sarathi_timer_create(int32_t capacity, uint32_t stage_mask, sarathi_timer **out) {
  if (!out) return fail(SARATHI_ERR_INVALID, "out is null");
  *out = nullptr;
  if (capacity <= 0 || capacity > (1 << 20)) return fail(SARATHI_ERR_INVALID, "bad timer capacity");
  stage_mask &= (1u << SARATHI_N_STAGES) - 1u;
  if (!stage_mask) return fail(SARATHI_ERR_INVALID, "timer stage mask selects no stage");
  sarathi_timer *t = new (std::nothrow) sarathi_timer();
  if (!t) return fail(SARATHI_ERR_NOMEM, "host allocation failed");
  t->capacity = capacity;
  t->used = 0;
  t->mask = stage_mask;
  t->n_timed = 0;
  for (int st = 0; st < SARATHI_N_STAGES; ++st) t->slot[st] = (stage_mask >> st & 1u) ? t->n_timed++ : -1;
  t->ran.assign(capacity, 0);
  const size_t n_ev = (size_t)capacity * t->n_timed * 2;
  t->ev.reserve(n_ev);
  for (size_t i = 0; i < n_ev; ++i) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) {
      sarathi_timer_destroy(t);
      return fail(SARATHI_ERR_HIP, "hipEventCreate failed");
    }
    t->ev.push_back(e);
  }
  *out = t;
  return SARATHI_OK;
}

void sarathi_timer_destroy(sarathi_timer *timer) {
  if (!timer) return;
  for (hipEvent_t e : timer->ev) (void)hipEventDestroy(e);
  delete timer;
}

sarathi_status sarathi_layer_forward_timed(sarathi_layer *layer, const sarathi_batch *batch,
                                           void *workspace, size_t ws_bytes, void *stream,
                                           sarathi_timer *timer) {
  if (!timer) return fail(SARATHI_ERR_INVALID, "timer is null");
  return forward_entry(layer, batch, workspace, ws_bytes, stream, nullptr, timer);
}

sarathi_status sarathi_multi_forward_timed(sarathi_layer *layer, const sarathi_multi_batch *batch,
                                           void *workspace, size_t ws_bytes, void *stream,
                                           sarathi_timer *timer) {
  if (!timer) return fail(SARATHI_ERR_INVALID, "timer is null");
  return forward_entry(layer, batch, workspace, ws_bytes, stream, nullptr, timer);
}

sarathi_status sarathi_paged_forward_timed(sarathi_layer *layer, const sarathi_paged_batch *batch,
                                           void *workspace, size_t ws_bytes, void *stream,
                                           sarathi_timer *timer) {
  if (!timer) return fail(SARATHI_ERR_INVALID, "timer is null");
  return forward_entry(layer, batch, workspace, ws_bytes, stream, nullptr, timer);
}

sarathi_status sarathi_timer_read(sarathi_timer *timer, double *total_ms, int32_t *count) {
  if (!timer || !total_ms || !count) return fail(SARATHI_ERR_INVALID, "null argument");
  for (int st = 0; st < SARATHI_N_STAGES; ++st) {
    total_ms[st] = 0.0;
    count[st] = 0;
  }
  const int n = timer->used;
  timer->used = 0;
  for (int f = 0; f < n; ++f) {
    for (int st = 0; st < SARATHI_N_STAGES; ++st) {
      if (timer->slot[st] < 0 || !(timer->ran[f] >> st & 1u)) continue;
      const size_t base = ((size_t)f * timer->n_timed + timer->slot[st]) * 2;
      HIP_TRY(hipEventSynchronize(timer->ev[base + 1]));
      float ms = 0.f;
      HIP_TRY(hipEventElapsedTime(&ms, timer->ev[base], timer->ev[base + 1]));
      total_ms[st] += ms;
      count[st] += 1;
    }
  }
  return SARATHI_OK;
}

sarathi_status sarathi_clock_sample(uint64_t *out, void *stream) {
  if (!out) return fail(SARATHI_ERR_INVALID, "out is null");
  HIP_TRY(launch_clock_sample(out, static_cast<hipStream_t>(stream)));
  return SARATHI_OK;
}

const char *sarathi_status_str(sarathi_status status) {
  switch (status) {
    case SARATHI_OK: return "ok";
    case SARATHI_ERR_INVALID: return "invalid argument";
    case SARATHI_ERR_UNSUPPORTED: return "unsupported shape";
    case SARATHI_ERR_CAPACITY: return "cache or position capacity exceeded";
    case SARATHI_ERR_HIP: return "HIP runtime error";
    case SARATHI_ERR_NOMEM: return "out of memory";
    case SARATHI_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case SARATHI_ERR_INTERNAL: return "internal error";
  }
  return "unknown status";
}

const char *sarathi_last_error(void) { return g_last_error.c_str(); }

sarathi_status sarathi_plan_describe(const sarathi_layer_desc *desc, const sarathi_batch *batch,
                                     sarathi_plan_info *info) {
  return describe_entry(desc, batch, info);
}

sarathi_status sarathi_multi_plan_describe(const sarathi_layer_desc *desc,
                                           const sarathi_multi_batch *batch, sarathi_plan_info *info) {
  return describe_entry(desc, batch, info);
}

sarathi_status sarathi_paged_plan_describe(const sarathi_layer_desc *desc,
                                           const sarathi_paged_batch *batch, sarathi_plan_info *info) {
  return describe_entry(desc, batch, info);
}

}  // extern "C"
