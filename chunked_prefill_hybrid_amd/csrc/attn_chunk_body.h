// Causal attention of a prefill chunk over its request's cached prefix plus itself (bf16, MFMA).
//
// Chunk query t sits at absolute position off+t and attends to keys 0..off+t: the whole cached
// prefix and the causal part of its own chunk, whose K/V rows were appended to the same cache just
// before (SARATHI: Efficient LLM Inference by Piggybacking Decodes with Chunked Prefills, section 3,
// "Chunked-Prefills", attention mask construction and Figure 6).  The prefix is re-read from HBM by
// every chunk of the request, the overhead the same page discusses under "Overhead 2".
//
// Flash-style design for gfx950.  A workgroup takes one head and 64 RB queries (16 RB per wave, in RB
// blocks of 16) and streams a range of the request's keys in tiles of 64 through a 2- or 3-stage LDS ring filled by LDS DMA
// (global_load_lds_dwordx4: no staging registers, no LDS store instructions).  Per wave and tile:
//   S^T = K Q^T   (16 x v_mfma_f32_16x16x32_bf16 per block for d = 128): lane l then holds the
//                 scores of query l % 16 of each block for 16 of the tile's keys, so a query's row
//                 max / sum need only in-lane work and two butterfly steps;
//   online softmax in float32 (log2 domain, scale folded into the exponent);
//   O^T += V^T P^T (16 more MFMAs): P^T is taken straight from the S^T registers, and V^T's operand
//                 comes from the row-major V tile through transposing LDS reads (ds_read_b64_tr_b16:
//                 in each group of 16 lanes, lane j addresses row j/4, columns 4(j%4)..4(j%4)+3, and
//                 lane i receives column i of those 4 rows), so the keys of a lane's k-slots match
//                 the keys of its P^T values without any register shuffling.
// Each K and V fragment read from LDS feeds the MFMAs of all RB query blocks of the wave, so RB = 2
// halves the LDS reads per score and doubles the independent MFMA chains per wave.
// K rows are stored with their 16-byte chunks permuted (slot = chunk ^ f(row)) so the 16 rows of a
// fragment read hit distinct banks; V rows likewise for the transposing reads.  Only tiles that cross
// the diagonal are masked.  Rows past the last key any query of the block needs are loaded as copies
// of that key (finite values whose probability is 0 after the mask), never from unwritten slots.
//
// The key range of each 64-query block can be split over several workgroups so that short chunks
// still fill the GPU; a split writes (m, l, unnormalised O) partials for attn_combine.
//
// Paged KV caches (a pool of fixed-size pages per layer and a block table per request) change only
// the DMA source addresses: each lane's key row is looked up in the chunk's block table, one tile
// ahead of its loads.
//
// One launch serves every prefill chunk of the batch.  A batch may carry several partial prefills of
// different requests next to its decodes, as in token-budget ("stall-free") batching (junupark.xyz
// notes on Sarathi-Serve, "Stall Free Batching"); each chunk attends only to its own request's cache,
// so a work item names its chunk, and the items of all chunks share one grid.
#pragma once
#include <math.h>

#include "kernels.h"

namespace sarathi {
namespace {

constexpr int kBQ = 64;         // queries per workgroup at one 16-query block per wave
constexpr int kBKV = 64;        // keys per tile
#ifndef SARATHI_CHUNK_STAGES
#define SARATHI_CHUNK_STAGES 2
#endif
constexpr int kChunkStages = SARATHI_CHUNK_STAGES;   // LDS ring depth (2 or 3)
static_assert(kChunkStages == 2 || kChunkStages == 3, "ring depth");

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

// 2^x for x <= 0 with the hardware exponential alone: results below the normal range flush to 0,
// which is what a probability that small contributes anyway.
__device__ __forceinline__ float exp2_nonpos(float x) { return __builtin_amdgcn_exp2f(x); }
// Largest log2 gap between a tile's score maximum and the running exponent base before the base moves.
constexpr float kRebase = 8.0f;

template <int D> struct TileGeom {
  static constexpr int kChunks = D / 8;            // 16-byte chunks per row
  static constexpr int kRPL = 1024 / (2 * D);      // rows per DMA load (64 lanes x 16 bytes)
  static constexpr int kLoadsPerWave = kBKV / kRPL / 4;
  static constexpr int kElems = kBKV * D;
};
// Chunk slot of K row r (row within the tile): 16 rows at one logical chunk land in 16 distinct
// 4-bank groups (256-byte rows: slot = c ^ (r & 15); 128-byte rows: slot = c ^ ((r >> 1) & 7)).
template <int D> __device__ __forceinline__ int k_slot(int r, int c) {
  return D == 128 ? c ^ (r & 15) : c ^ ((r >> 1) & 7);
}
// Chunk slot of V row r: a transposing read by 32 lanes covers 8 consecutive rows x 2 adjacent
// chunks; for 256-byte rows slot = c ^ 2 (r & 7) spreads those 16 (row, chunk) pairs over all 64
// banks; 128-byte rows already fall in distinct banks.
template <int D> __device__ __forceinline__ int v_slot(int r, int c) {
  return D == 128 ? c ^ ((r & 7) << 1) : c;
}

// Work items of a chunk of `len` rows: bq-query blocks x key splits x heads.
__host__ __device__ inline int chunk_items(int len, int n_split, int nh, int bq) {
  return (len + bq - 1) / bq * n_split * nh;
}

// The work of one chunk work item (chunk, head, key split, 64-query block), for the chunk kernel and
// for the chunk part of the fused attention kernel.  The LDS stages are the caller's
// shared-memory arrays (separate arrays, so the compiler can tell the stages apart).
template <int D, bool kPaged, int RB>
__device__ __forceinline__ void chunk_attn_item(int item, const bf16_t *q, int ld_q, int nh,
                                                const ChunkSet &cs, const PagePool &pool, bf16_t *out,
                                                OutLayout olay, float qscale_log2, int n_split, int stride,
                                                float *part_o, float *part_ml, bf16_t *k0s, bf16_t *v0s,
                                                bf16_t *k1s, bf16_t *v1s, bf16_t *k2s, bf16_t *v2s) {
  using G = TileGeom<D>;
  constexpr int KS = D / 32;             // k-steps of the score MFMA
  constexpr int DB = D / 16;             // 16-row blocks of O^T
  constexpr int BQ = kBQ * RB;           // queries of the workgroup
  static_assert(RB == 1 || RB == 2, "query blocks per wave");
  auto kst = [&](int u) -> bf16_t * { return u == 0 ? k0s : u == 1 ? k1s : k2s; };
  auto vst = [&](int u) -> bf16_t * { return u == 0 ? v0s : u == 1 ? v1s : v2s; };

  // Items are numbered chunk by chunk; the scan over the chunks is uniform across the workgroup.
  int cj = 0, first_item = 0;
  for (; cj < cs.n; ++cj) {
    const int n_items = chunk_items(cs.len[cj], cs.split[cj], nh, BQ);
    if (item < first_item + n_items) break;
    first_item += n_items;
  }
  if (cj >= cs.n) return;
  const int C = cs.len[cj], off = cs.off[cj], row0 = cs.row0[cj], cap = cs.cap[cj];
  const int q_blocks = (C + BQ - 1) / BQ;
  const int local = item - first_item;
  const int ns = cs.split[cj];   // this chunk's splits (n_split is the largest of the set)
  const int qb = local % q_blocks, split = (local / q_blocks) % ns, h = local / (q_blocks * ns);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int q_first = qb * BQ;
  const int q_last = min(C, q_first + BQ) - 1;           // last query of the workgroup
  const int q_wave = q_first + wave * 16 * RB;            // first query of this wave
  const int n_keys = off + q_last + 1;                    // keys any of its queries sees
  const int nt = (n_keys + kBKV - 1) / kBKV;
  const int t_begin = (int)((long long)split * nt / ns);
  const int t_end = (int)((long long)(split + 1) * nt / ns);
  // Contiguous caches: this head's [cap, D] slab.  Paged caches: the pools, addressed per key row
  // through the chunk's block table.
  const bf16_t *Kh = kPaged ? reinterpret_cast<const bf16_t *>(pool.k)
                            : reinterpret_cast<const bf16_t *>(cs.k[cj]) + (size_t)h * cap * D;
  const bf16_t *Vh = kPaged ? reinterpret_cast<const bf16_t *>(pool.v)
                            : reinterpret_cast<const bf16_t *>(cs.v[cj]) + (size_t)h * cap * D;
  const int32_t *table = reinterpret_cast<const int32_t *>(cs.k[cj]);

  // This lane's query in each of the wave's blocks (row c16 of block rb) and its fragments of q
  // (B operand of S^T = K Q^T).
  int my_q[RB], my_pos[RB];
  bf16x8_t qf[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    my_q[rb] = q_wave + rb * 16 + c16;
    my_pos[rb] = off + min(my_q[rb], C - 1);
    const bf16_t *qr = q + (size_t)(row0 + min(my_q[rb], C - 1)) * ld_q + h * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[rb][ks] = *reinterpret_cast<const bf16x8_t *>(qr + ks * 32 + g * 8);
  }

  // DMA sources: load i of this wave fills tile rows kRPL (wave + 4 i) .. + kRPL - 1; lane l lands
  // in row kRPL (wave + 4 i) + l / kChunks, slot l % kChunks, so it fetches the chunk stored there.
  int lr[G::kLoadsPerWave], kc[G::kLoadsPerWave], vc[G::kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < G::kLoadsPerWave; ++i) {
    const int r = G::kRPL * (wave + 4 * i) + lane / G::kChunks, sl = lane % G::kChunks;
    lr[i] = r;
    kc[i] = k_slot<D>(r, sl);   // the slot permutation is an involution
    vc[i] = v_slot<D>(r, sl);
  }
  // Paged caches: pool pages of the rows this lane loads for a tile.  They are fetched one tile ahead
  // (pages_of for the next tile is issued right after the current tile's DMA), so the table's latency
  // hides behind a tile of work.
  int pg_next[G::kLoadsPerWave] = {};
  auto pages_of = [&](int t) {
    if (!kPaged) return;
    const int k0 = min(t, t_end - 1) * kBKV;
#pragma unroll
    for (int i = 0; i < G::kLoadsPerWave; ++i)
      pg_next[i] = pool_page(table, min(k0 + lr[i], n_keys - 1) >> pool.shift, pool.n_pages);
  };
  // Tile t (clamped to the split's last tile, so every step issues the same loads) into stage u.
  auto issue = [&](int u, int t) {
    const int k0 = min(t, t_end - 1) * kBKV;
#pragma unroll
    for (int i = 0; i < G::kLoadsPerWave; ++i) {
      const int key = min(k0 + lr[i], n_keys - 1);
      const size_t ro = kPaged ? paged_off(pg_next[i], h, key, nh, pool.shift, D) : (size_t)key * D;
      const int dst = G::kRPL * (wave + 4 * i) * D;
      dma16(Kh + ro + kc[i] * 8, kst(u) + dst);
      dma16(Vh + ro + vc[i] * 8, vst(u) + dst);
    }
  };

  f32x4_t o[RB][DB];
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
  }

  auto compute = [&](int u, int t) {
    const bf16_t *Ks = kst(u), *Vs = vst(u);
    // S^T for the tile: 4 key blocks of 16, each K fragment shared by the wave's query blocks.
    f32x4_t sacc[RB][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sacc[rb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int r = kb * 16 + c16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t *>(&Ks[r * D + k_slot<D>(r, ks * 4 + g) * 8]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sacc[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rb][ks], sacc[rb][kb], 0, 0, 0);
      }
    }
    // Raw scores, masked past each query's position; only tiles that reach past the wave's first
    // query need the mask (a wave-uniform test).  The log2-domain scale (positive) is applied to the
    // maximum and inside each exponent's multiply-add.
    const int k0 = t * kBKV;
    const bool diag = k0 + kBKV - 1 > off + q_wave;
    bf16x8_t pf[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float sc[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[kb][i] = sacc[rb][kb][i];
      if (diag) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (k0 + kb * 16 + g * 4 + i > my_pos[rb]) sc[kb][i] = -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sc[kb][i]);
      tmax = max_xor(max_xor(tmax, 16), 32);
      // The exponent base m_run moves only when a tile's maximum exceeds it by more than kRebase (in
      // log2 units): probabilities then stay below 2^kRebase, well inside float32 and bfloat16
      // range, and the running sums are rescaled on a few tiles instead of on every tile with a new
      // maximum.  Any base gives the same softmax, since O and l share it.  A split that starts past
      // a query's position leaves its row fully masked (m_run stays -inf): the exponent base is then
      // 0, every p is 0 and the row's partial stays empty (l = 0).
      const float m_tile = tmax * qscale_log2;
      const bool rebase = m_tile > m_run[rb] + kRebase;
      if (__any(rebase)) {
        const float m_new = rebase ? m_tile : m_run[rb];
        // 1 for a query whose base stays, 0 for one whose sums are still empty (m_run = -inf)
        const float corr = exp2_nonpos(m_run[rb] - (m_new == -INFINITY ? 0.f : m_new));
        l_run[rb] *= corr;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rb][db] *= corr;
        m_run[rb] = m_new;
      }
      const float m_base = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
      // P^T operands: k-step s holds keys s*32 + 4g + i (slots 0..3) and s*32 + 16 + 4g + i (4..7).
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sc[2 * s + hb][i], qscale_log2, -m_base));
            l_run[rb] += p;
            pf[rb][s][hb * 4 + i] = (__bf16)p;
          }
    }
    // O^T += V^T P^T; V^T fragments by transposing reads of rows s*32 + 4g + (0..3) and + 16, each
    // shared by the wave's query blocks.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = db * 16 + 4 * (c16 & 3);          // this lane's 4 addressed columns
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        s16x4_t half[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int r = s * 32 + hh * 16 + 4 * g + (c16 >> 2);
          const bf16_t *a = &Vs[r * D + v_slot<D>(r, col >> 3) * 8 + (col & 7)];
          half[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t *)(a));
        }
        const s16x8_t vv = {half[0][0], half[0][1], half[0][2], half[0][3],
                            half[1][0], half[1][1], half[1][2], half[1][3]};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vv), pf[rb][s],
                                                              o[rb][db], 0, 0, 0);
      }
    }
  };

  if (t_begin < t_end) {   // workgroup-uniform: an empty split only writes its empty partial
    constexpr int kL = 2 * G::kLoadsPerWave;   // loads per wave per tile
    constexpr int kNSt = kChunkStages;
    auto step = [&](int u, int t) {
      issue((u + kNSt - 1) % kNSt, t + kNSt - 1);
      pages_of(t + kNSt);
      compute(u, t);
      wait_vm_lgkm0<(kNSt - 2) * kL>();   // this wave's loads of tile t + 1 have landed
      stage_barrier();                    // ... and everyone's; stage u is free again
    };
#pragma unroll
    for (int u = 0; u < kNSt - 1; ++u) {
      pages_of(t_begin + u);
      issue(u, t_begin + u);
    }
    pages_of(t_begin + kNSt - 1);
    wait_vm_lgkm0<(kNSt - 2) * kL>();
    stage_barrier();
    int t0 = t_begin;
    for (; t0 + kNSt <= t_end; t0 += kNSt) {
#pragma unroll
      for (int u = 0; u < kNSt; ++u) step(u, t0 + u);
    }
#pragma unroll
    for (int u = 0; u < kNSt; ++u)
      if (t0 + u < t_end) step(u, t0 + u);
    wait_vm_lgkm0<0>();   // the clamped loads past the last tile land before the workgroup ends
  }

  // Row sums over the four lane groups of the query, then O[q][d] = O^T[d][q] / l.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float l = l_run[rb];
    l = sum_xor(sum_xor(l, 16), 32);
    const int qr = my_q[rb];
    if (ns > 1) {   // a split chunk: partials for attn_combine (an unsplit one writes its rows)
      if (qr < C) {
        const size_t pidx = ((size_t)(row0 + qr) * nh + h) * stride + split;
        if (g == 0) {
          part_ml[2 * pidx] = m_run[rb];
          part_ml[2 * pidx + 1] = l;
        }
        float *po = part_o + pidx * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          *reinterpret_cast<float4 *>(&po[db * 16 + g * 4]) =
              make_float4(o[rb][db][0], o[rb][db][1], o[rb][db][2], o[rb][db][3]);
      }
    } else if (qr < C) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        uint2 u;
        u.x = (uint32_t)f32_to_bf16(o[rb][db][0] * inv) | ((uint32_t)f32_to_bf16(o[rb][db][1] * inv) << 16);
        u.y = (uint32_t)f32_to_bf16(o[rb][db][2] * inv) | ((uint32_t)f32_to_bf16(o[rb][db][3] * inv) << 16);
        // 4 consecutive columns, within one k-tile of a k-tile-major output
        *reinterpret_cast<uint2 *>(&out[out_index(olay, row0 + qr, h * D + db * 16 + g * 4)]) = u;
      }
    }
  }
}

// LDS stages of the chunk attention, declared by each kernel that runs chunk work items.
#define SARATHI_CHUNK_LDS(D)                                                                          \
  __shared__ __attribute__((aligned(1024))) bf16_t k0s[TileGeom<D>::kElems], v0s[TileGeom<D>::kElems]; \
  __shared__ __attribute__((aligned(1024))) bf16_t k1s[TileGeom<D>::kElems], v1s[TileGeom<D>::kElems]; \
  __shared__ __attribute__((aligned(1024))) bf16_t k2s[kChunkStages > 2 ? TileGeom<D>::kElems : 8];    \
  __shared__ __attribute__((aligned(1024))) bf16_t v2s[kChunkStages > 2 ? TileGeom<D>::kElems : 8]


// Chunk work item of workgroup b: XCD-aware, workgroup b runs on XCD b % 8 and the items of XCD x are
// the consecutive range [x per_xcd, (x + 1) per_xcd), so the query blocks and splits of a head share
// one XCD's L2 and its K/V crosses HBM about once.
__device__ __forceinline__ int chunk_item_of(int b, int per_xcd) { return (b & 7) * per_xcd + (b >> 3); }

}  // namespace
}  // namespace sarathi
