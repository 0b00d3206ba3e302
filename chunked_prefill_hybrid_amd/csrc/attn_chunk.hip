// The chunk attention kernel and its launcher; the work of a chunk work item is in attn_chunk_body.h,
// shared with the fused attention kernel of attn_rows.hip.
#include "attn_chunk_body.h"

namespace sarathi {
namespace {

template <int D, bool kPaged>
__global__ __launch_bounds__(256) void attn_chunk_mfma(const bf16_t *q, int ld_q, int nh,
                                                       ChunkSet cs, PagePool pool, bf16_t *out, int ld_out,
                                                       float qscale_log2, int n_split, int stride,
                                                       float *part_o, float *part_ml, int per_xcd) {
  SARATHI_CHUNK_LDS(D);
  chunk_attn_item<D, kPaged>(chunk_item_of(blockIdx.x, per_xcd), q, ld_q, nh, cs, pool, out, ld_out,
                             qscale_log2, n_split, stride, part_o, part_ml, k0s, v0s, k1s, v1s, k2s, v2s);
}

template <int D>
hipError_t run_chunk(const void *q, int ld_q, int nh, const ChunkSet &cs, const PagePool &pool, void *out,
                     int ld_out, int n_split, int stride, float *part_o, float *part_ml, hipStream_t s) {
  int items = 0;
  for (int j = 0; j < cs.n; ++j) items += chunk_items(cs.len[j], n_split, nh);
  const int per_xcd = (items + 7) / 8;
  const float qscale = 1.4426950408889634f / sqrtf((float)D);
  if (pool.k)
    hipLaunchKernelGGL((attn_chunk_mfma<D, true>), dim3(8 * per_xcd), dim3(256), 0, s,
                       static_cast<const bf16_t *>(q), ld_q, nh, cs, pool, static_cast<bf16_t *>(out),
                       ld_out, qscale, n_split, stride, part_o, part_ml, per_xcd);
  else
    hipLaunchKernelGGL((attn_chunk_mfma<D, false>), dim3(8 * per_xcd), dim3(256), 0, s,
                       static_cast<const bf16_t *>(q), ld_q, nh, cs, pool, static_cast<bf16_t *>(out),
                       ld_out, qscale, n_split, stride, part_o, part_ml, per_xcd);
  return hipGetLastError();
}

}  // namespace

// Splits of each query block's key range, one count for every chunk of the set.  The work items run
// in rounds of kChunkTargetWorkgroups (two per compute unit); a round lasts about as long as its
// longest item walks its key tiles, and each split beyond the first costs about kSplitCostTiles tile
// times (its partial is written and merged).  The count with the shortest estimated makespan wins,
// among those that keep every split at least kMinSplitTiles tiles long and never exceed the tiles of
// any chunk's first block (so no split is empty).  Items that leave the last round mostly idle are
// what this avoids: with 8 query blocks x 40 heads over an 8K-key prefix, two splits make 640 items,
// a full round and a quarter of one, no faster than one split; three make 960 in two full rounds.
int chunk_attn_splits(const ChunkSet &cs, int nh) {
  if (cs.n <= 0) return 1;
  int q_blocks = 0, first_tiles = 1 << 30, by_length = 1 << 30, max_tiles = 0;
  for (int j = 0; j < cs.n; ++j) {
    const int C = cs.len[j], off = cs.off[j];
    q_blocks += (C + kBQ - 1) / kBQ;
    first_tiles = min(first_tiles, (off + min(C, kBQ) + kBKV - 1) / kBKV);
    const int avg_tiles = (off + (C + 1) / 2 + kBKV - 1) / kBKV;
    by_length = min(by_length, max(1, avg_tiles / kMinSplitTiles));
    max_tiles = max(max_tiles, (off + C + kBKV - 1) / kBKV);
  }
  const int s_max = max(1, min(kMaxChunkSplits, min(by_length, first_tiles)));
  int best = 1;
  long long best_t = -1;
  for (int sp = 1; sp <= s_max; ++sp) {
    const long long items = (long long)q_blocks * nh * sp;
    const long long rounds = (items + kChunkTargetWorkgroups - 1) / kChunkTargetWorkgroups;
    const long long t = rounds * ((max_tiles + sp - 1) / sp) + (long long)kSplitCostTiles * (sp - 1);
    if (best_t < 0 || t < best_t) {
      best_t = t;
      best = sp;
    }
  }
  return best;
}

hipError_t launch_attn_chunk(int d, const void *q, int ld_q, int nh, const ChunkSet &cs,
                             const PagePool &pool, void *out, int ld_out, int n_split, int stride,
                             float *part_o, float *part_ml, hipStream_t s) {
  if (cs.n <= 0 || cs.rows <= 0) return hipSuccess;
  if (cs.n > kMaxChunks) return hipErrorInvalidValue;
  if (n_split < 1 || n_split > stride || (n_split > 1 && (!part_o || !part_ml)))
    return hipErrorInvalidValue;
  if (d == 128) return run_chunk<128>(q, ld_q, nh, cs, pool, out, ld_out, n_split, stride, part_o, part_ml, s);
  if (d == 64) return run_chunk<64>(q, ld_q, nh, cs, pool, out, ld_out, n_split, stride, part_o, part_ml, s);
  return hipErrorInvalidValue;
}

}  // namespace sarathi
