// The chunk attention kernel and its launcher; the work of a chunk work item is in attn_chunk_body.h,
// shared with the fused attention kernel of attn_rows.hip.
#include "attn_chunk_body.h"

namespace sarathi {
namespace {

template <int D, bool kPaged, int RB>
__global__ __launch_bounds__(256) void attn_chunk_mfma(const bf16_t *q, int ld_q, int nh,
                                                       ChunkSet cs, PagePool pool, bf16_t *out, OutLayout olay,
                                                       float qscale_log2, int n_split, int stride,
                                                       float *part_o, float *part_ml, int per_xcd) {
  SARATHI_CHUNK_LDS(D);
  chunk_attn_item<D, kPaged, RB>(chunk_item_of(blockIdx.x, per_xcd), q, ld_q, nh, cs, pool, out, olay,
                                 qscale_log2, n_split, stride, part_o, part_ml, k0s, v0s, k1s, v1s, k2s,
                                 v2s);
}

template <int D, bool kPaged, int RB>
hipError_t run_chunk(const void *q, int ld_q, int nh, const ChunkSet &cs, const PagePool &pool, void *out,
                     OutLayout olay, int n_split, int stride, float *part_o, float *part_ml, hipStream_t s) {
  int items = 0;
  for (int j = 0; j < cs.n; ++j) items += chunk_items(cs.len[j], cs.split[j], nh, kBQ * RB);
  const int per_xcd = (items + 7) / 8;
  const float qscale = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL((attn_chunk_mfma<D, kPaged, RB>), dim3(8 * per_xcd), dim3(256), 0, s,
                     static_cast<const bf16_t *>(q), ld_q, nh, cs, pool, static_cast<bf16_t *>(out), olay,
                     qscale, n_split, stride, part_o, part_ml, per_xcd);
  return hipGetLastError();
}

}  // namespace

// Splits of each chunk's query-block key ranges, chosen per chunk and written to cs.split; returns
// the largest; *cost is the estimated makespan in key-tile times.  Query blocks have bq queries (64,
// or 128 in the chunk kernel with two blocks per wave) and the work items run in rounds of `resident`
// workgroups (as many as the compute units hold at once).  A round lasts about as long as its longest item walks its key tiles,
// and each split beyond the first costs about kSplitCostTiles tile times (its partial is written and merged).  For a target item
// length of T tiles every chunk takes the splits that bring its longest block under T, within its
// limit: splits of at least kMinSplitTiles tiles, and never more than its first block has tiles (so
// no split is empty).  The T with the shortest estimated makespan wins.  Two cases this serves: a
// long prefix chunk next to short new prompts in a token-budget batch is split while the short ones
// are not, so it stops setting the makespan alone; and with 8 query blocks x 40 heads over an
// 8K-key prefix, two splits make 640 items (a full round and a quarter of one, no faster than one
// split) while three make 960 in two full rounds.
int chunk_attn_splits(ChunkSet &cs, int nh, int bq, int resident, long long *cost) {
  int cap[kMaxChunks], tiles[kMaxChunks], blocks[kMaxChunks];
  int max_tiles = 1;
  for (int j = 0; j < cs.n; ++j) {
    const int C = cs.len[j], off = cs.off[j];
    blocks[j] = (C + bq - 1) / bq;
    tiles[j] = (off + C + kBKV - 1) / kBKV;
    const int first_tiles = (off + min(C, bq) + kBKV - 1) / kBKV;
    const int avg_tiles = (off + (C + 1) / 2 + kBKV - 1) / kBKV;
    cap[j] = max(1, min(kMaxChunkSplits, min(first_tiles, avg_tiles / kMinSplitTiles)));
    max_tiles = max(max_tiles, tiles[j]);
    cs.split[j] = 1;
  }
  long long best_t = -1;
  int best_T = max_tiles;
  for (int T = max_tiles; T >= 1; --T) {
    long long items = 0;
    int longest = 0, most = 1;
    for (int j = 0; j < cs.n; ++j) {
      const int sp = min(cap[j], (tiles[j] + T - 1) / T);
      items += (long long)blocks[j] * sp * nh;
      longest = max(longest, (tiles[j] + sp - 1) / sp);
      most = max(most, sp);
    }
    const long long rounds = (items + resident - 1) / resident;
    const long long t = rounds * longest + (long long)kSplitCostTiles * (most - 1);
    if (best_t < 0 || t < best_t) {
      best_t = t;
      best_T = T;
    }
  }
  int most = 1;
  for (int j = 0; j < cs.n; ++j) {
    cs.split[j] = min(cap[j], (tiles[j] + best_T - 1) / best_T);
    most = max(most, cs.split[j]);
  }
  *cost = best_t;
  return most;
}

// Query blocks per wave and key splits for the chunk kernel.  Two 16-query blocks per wave halve the
// LDS reads per score and double each wave's independent MFMA chains, so a key tile of a 128-query
// item costs kTwoBlockTileCost (not 2) tiles of a 64-query item; but the items are then half as many,
// which leaves compute units idle when a batch's chunks are short.  The plan with the shorter
// estimated makespan wins.  Paged caches keep one block per wave: with the block-table lookups the
// two-block item's registers exceed half a SIMD's, and one workgroup per compute unit loses to two.
int chunk_attn_plan(ChunkSet &cs, int nh, bool paged) {
  ChunkSet two = cs;
  long long c1 = 0, c2 = 0;
  const int m1 = chunk_attn_splits(cs, nh, kBQ, kChunkResident, &c1);
  cs.qblocks = 1;
  if (paged) return m1;
  const int m2 = chunk_attn_splits(two, nh, 2 * kBQ, kChunkResident, &c2);
  if (kTwoBlockTileCost * (double)c2 < (double)c1) {
    cs = two;
    cs.qblocks = 2;
    return m2;
  }
  return m1;
}

hipError_t launch_attn_chunk(int d, const void *q, int ld_q, int nh, const ChunkSet &cs,
                             const PagePool &pool, void *out, OutLayout olay, int n_split, int stride,
                             float *part_o, float *part_ml, hipStream_t s) {
  if (cs.n <= 0 || cs.rows <= 0) return hipSuccess;
  if (cs.n > kMaxChunks) return hipErrorInvalidValue;
  if (n_split < 1 || n_split > stride || (n_split > 1 && (!part_o || !part_ml)))
    return hipErrorInvalidValue;
  for (int j = 0; j < cs.n; ++j)
    if (cs.split[j] < 1 || cs.split[j] > n_split) return hipErrorInvalidValue;
  // two 16-query blocks per wave: contiguous caches only
  if (cs.qblocks != 1 && !(cs.qblocks == 2 && !pool.k)) return hipErrorInvalidValue;
#define SARATHI_RUN_CHUNK(D, P, RB) \
  run_chunk<D, P, RB>(q, ld_q, nh, cs, pool, out, olay, n_split, stride, part_o, part_ml, s)
  if (d == 128)
    return pool.k ? SARATHI_RUN_CHUNK(128, true, 1)
                  : cs.qblocks == 2 ? SARATHI_RUN_CHUNK(128, false, 2) : SARATHI_RUN_CHUNK(128, false, 1);
  if (d == 64)
    return pool.k ? SARATHI_RUN_CHUNK(64, true, 1)
                  : cs.qblocks == 2 ? SARATHI_RUN_CHUNK(64, false, 2) : SARATHI_RUN_CHUNK(64, false, 1);
#undef SARATHI_RUN_CHUNK
  return hipErrorInvalidValue;
}

}  // namespace sarathi
