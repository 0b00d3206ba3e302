// Single-query attention per (row, head) with the key range split across workgroups, plus the merge
// of the split partials.
//
// A decode query attends over its request's cached entries plus its own new entry, i.e. keys
// 0..pos with pos = the decode's cached length (Sarathi-Serve Guide: Chunked-Prefills & LLM Serving,
// "Deep Dive", "Attention Complexity Across Mixed Batches"); each decode reads only its own cache
// because decode attention is not fused across requests (SARATHI: Efficient LLM Inference by
// Piggybacking Decodes with Chunked Prefills, section 3, "Decode-Maximal Batching").  The same kernel
// serves chunk rows (keys 0..offset+t, Figure 6 of that page) in float32 mode.
//
// Memory-bound design: the head-major cache makes each (request, head) key stream contiguous; a key
// row of d elements is read by d*size/16 lanes with 16-byte loads, so one wave load instruction covers
// 4 bf16 keys of d=128 (1 KiB).  Each wave streams its keys in steps of 8 loads of K and 8 of V per
// lane (an online softmax across steps; the next step's K loads go out once a step's scores are
// taken and its V loads once the step's accumulation is done, so loads are always in flight), the
// four waves of a workgroup merge through LDS, and each workgroup writes one split partial (max m
// and sum l in the log2 domain, unnormalised output).
// With a paged cache a key row is located through the request's block table (one table entry per
// page, held in a lane of the wave and shuffled to the lanes reading that page); a page's
// [page_size, d] slab per head is contiguous, so each 16-byte load stays a full-row read.
#include <math.h>

#include <type_traits>

#include "attn_chunk_body.h"
#include "kernels.h"

namespace sarathi {
namespace {

constexpr int kUnroll = 8;       // keys per lane and online-softmax step

// c + a.lo * b.lo + a.hi * b.hi for two packed bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}
// f(integral_constant<int, I>) for I = B .. E - 1, in order.
template <int B, int E, typename F> __device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}
// Steps whose K/V loads the fused kernel issues together.  Its occupancy is set by the chunk work's
// registers and LDS, so its decode waves are fewer; each keeps two steps of loads in flight.  The
// arithmetic is the same step by step, so a decode row's result does not depend on which kernel
// served it.
constexpr int kPrefetchFused = 2;

// The work of one (row r, key split s, head h) item: the split's partial of row r's attention.  sm,
// sl (4 floats each) and so (4 x D floats) are the caller's shared-memory arrays for the merge of the
// four waves.
template <typename T, int D, bool kChunkRows, bool kPaged, int kPre = 1>
__device__ __forceinline__ void split_attn_item(int r, int s, int h, const T *q, int ld_q, int nh,
                                                const ChunkSet &cs, const DecodeGroup &dg,
                                                const PagePool &pool, int stride, int prow0,
                                                float *part_o, float *part_ml, float qscale, float *sm,
                                                float *sl, float *so) {
  // No contraction of separate operations into fused multiply-adds (only the explicit fmaf calls
  // fuse): the two walks below order the same operations differently, and a row's result must not
  // depend on which walk, kernel or batch served it.
#pragma clang fp contract(off)
  constexpr int E = Packet<T>::E;      // elements per 16-byte packet
  constexpr int LPK = D / E;           // lanes per key row
  constexpr int KPI = kWave / LPK;     // keys per wave load step
  constexpr int KPW = kAttnSplit / 4;  // keys per wave per pass
  constexpr int NIT = KPW / KPI;
  static_assert(NIT % kUnroll == 0, "whole unrolled steps");
  constexpr int P = (kPre * kUnroll <= NIT && NIT % (kPre * kUnroll) == 0) ? kPre : 1;
  constexpr int U = P * kUnroll;   // loads per lane issued together
  const RowRef rr = row_ref<kChunkRows>(r, cs, dg);
  const int n_keys = rr.pos + 1;
  const int nsp = attn_splits(n_keys);
  const size_t pidx = ((size_t)(r - prow0) * nh + h) * stride + s;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (s >= nsp) {  // no keys for this split: an empty partial
    if (tid == 0) {
      part_ml[2 * pidx] = -INFINITY;
      part_ml[2 * pidx + 1] = 0.f;
    }
    return;
  }
  const int per = (n_keys + nsp - 1) / nsp;
  const int k_begin = s * per, k_end = min(n_keys, k_begin + per);
  const int npass = (per + kAttnSplit - 1) / kAttnSplit;   // 1 .. kAttnLongPasses
  const int sub = lane % LPK, grp = lane / LPK;

  // bf16: q stays packed and a lane's part of a score is four bf16-pair dot products (exact
  // products, float32 sums), scaled once; float32: q scaled, one multiply-add per element.
  constexpr bool kBf16 = sizeof(T) == 2;
  const uint4 q_raw = ld16(q + (size_t)r * ld_q + h * D + sub * E);
  float qv[E];
  if constexpr (!kBf16) {
    unpack<T>(q_raw, qv);
#pragma unroll
    for (int e = 0; e < E; ++e) qv[e] *= qscale;
  }
  const T *Kh = kPaged ? reinterpret_cast<const T *>(pool.k) + sub * E
                      : reinterpret_cast<const T *>(rr.k) + (size_t)h * rr.cap * D + sub * E;
  const T *Vh = kPaged ? reinterpret_cast<const T *>(pool.v) + sub * E
                      : reinterpret_cast<const T *>(rr.v) + (size_t)h * rr.cap * D + sub * E;
  // Pass p of wave w covers keys wbeg(p) .. wbeg(p) + KPW - 1, wbeg(p) = k_begin + (4p + w) KPW.
  // Paged caches: lane i of tbl[p] holds the pool page of the pass's i-th page (its KPW keys span at
  // most KPW / page_size + 1 pages); a key's page is then one lane shuffle away.  All passes' tables
  // are read before the first key.
  int tbl[kAttnLongPasses] = {}, pg0[kAttnLongPasses] = {};
  if (kPaged) {
    const int n_ent = rr.cap >> pool.shift;
#pragma unroll
    for (int p = 0; p < kAttnLongPasses; ++p)
      if (p < npass) {
        pg0[p] = (k_begin + (4 * p + wave) * KPW) >> pool.shift;
        tbl[p] = pool_page(reinterpret_cast<const int32_t *>(rr.k), min(pg0[p] + lane, n_ent - 1),
                           pool.n_pages);
      }
  }

  float m_run = -INFINITY, l_run = 0.f, o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;

  // Element offset of key j in this wave's K or V stream; `pass` (a compile-time index) names the
  // page-table register of the pass that key j belongs to.
  auto key_off = [&](auto pass_, int j) -> size_t {
    constexpr int pass = decltype(pass_)::value;
    if (!kPaged) return (size_t)j * D;
    const int page = __shfl(tbl[pass], min((j >> pool.shift) - pg0[pass], kWave - 1), kWave);
    return paged_off(page, h, j, nh, pool.shift, D);
  };
  // One online-softmax step over kUnroll loads of keys (ok[u]: load u holds a key of the split): the
  // scores from the step's K registers, then the rescale and the V accumulation.
  float sc[kUnroll], m_new = 0.f;
  auto scores = [&](const uint4 *kw, const bool *ok) {
    float cmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float dot = 0.f;
      if constexpr (kBf16) {
        dot = dot2_bf16(kw[u].x, q_raw.x, dot);
        dot = dot2_bf16(kw[u].y, q_raw.y, dot);
        dot = dot2_bf16(kw[u].z, q_raw.z, dot);
        dot = dot2_bf16(kw[u].w, q_raw.w, dot);
      } else {
        float kv[E];
        unpack<T>(kw[u], kv);
#pragma unroll
        for (int e = 0; e < E; ++e) dot = fmaf(qv[e], kv[e], dot);
      }
#pragma unroll
      for (int m = LPK / 2; m >= 1; m >>= 1) dot += __shfl_xor(dot, m, kWave);
      if constexpr (kBf16) dot *= qscale;
      sc[u] = ok[u] ? dot : -INFINITY;
      cmax = fmaxf(cmax, sc[u]);
    }
    cmax = wave_max(cmax, LPK);
    m_new = fmaxf(m_run, cmax);
  };
  auto accumulate = [&](const uint4 *vw, const bool *ok) {
    const float corr = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
    l_run *= corr;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= corr;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float p = ok[u] ? exp2f(sc[u] - m_new) : 0.f;
      l_run += p;
      float vv[E];
      unpack<T>(vw[u], vv);
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = fmaf(p, vv[e], o[e]);
      if constexpr (P == 1 && !kPaged) __builtin_amdgcn_sched_barrier(0);   // one key's values at a time
    }
    m_run = m_new;
  };

  if constexpr (P == 1 && !kPaged) {
    // Software-pipelined walk: the wave's steps in key order (pass by pass), the K loads of step
    // t + 1 issued as soon as step t's scores are taken and its V loads as soon as step t's
    // accumulation is done, so some of the wave's loads are always in flight.  (Paged caches take
    // the walk below: their page lookups would need more registers than four workgroups per compute
    // unit leave.)
    constexpr int SPP = NIT / kUnroll;               // steps per pass
    constexpr int kSteps = kAttnLongPasses * SPP;
    auto step_key = [&](int t) {
      const int pass = t / SPP;
      return k_begin + (4 * pass + wave) * KPW + (t - pass * SPP) * kUnroll * KPI;
    };
    int n_steps = 0;   // first keys rise with t, so the non-empty steps are a prefix
#pragma unroll
    for (int t = 0; t < kSteps; ++t) n_steps += (t < npass * SPP && step_key(t) < k_end) ? 1 : 0;
    uint4 kr[kUnroll], vr[kUnroll];
    // Loads of step t into dst from the K or V stream.  Every load is issued, so the wait before a
    // step's use can count the loads issued after it: a key past the split's end reads the split's
    // last key instead (its score is masked), and a step past the wave's last (t >= n_steps) reads
    // this lane's q piece, a cache hit (the values are not used).
    const T *q_lane = q + (size_t)r * ld_q + h * D + sub * E;
    auto load = [&](auto t_, uint4 *dst, const T *base) {
      constexpr int t = decltype(t_)::value;
      const bool real = t < n_steps;
      int j0 = step_key(t) + grp;
      // An opaque copy: the V loads recompute their offsets instead of holding the K loads' offsets
      // in registers across the accumulation.
      asm volatile("" : "+v"(j0));
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int j = min(j0 + u * KPI, k_end - 1);
        dst[u] = ld16_stream(real ? base + (size_t)j * D : q_lane);
      }
    };
    // The walk is unrolled (steps past n_steps are skipped); the scheduling barriers keep each step's
    // four phases in order, since the compiler would otherwise hoist the next step's loads above the
    // arithmetic and hold two steps in registers.
    load(std::integral_constant<int, 0>{}, kr, Kh);
    load(std::integral_constant<int, 0>{}, vr, Vh);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, kSteps>([&](auto t_) {
      constexpr int t = decltype(t_)::value;
      if (t < n_steps) {
        bool ok[kUnroll];
        const int j0 = step_key(t) + grp;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) ok[u] = j0 + u * KPI < k_end;
        scores(kr, ok);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (t + 1 < kSteps) load(std::integral_constant<int, t + 1>{}, kr, Kh);
        __builtin_amdgcn_sched_barrier(0);
        accumulate(vr, ok);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (t + 1 < kSteps) load(std::integral_constant<int, t + 1>{}, vr, Vh);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  } else {
    // P steps of loads issued together, then the steps one at a time.
    static_for<0, kAttnLongPasses>([&](auto pass_) {
      constexpr int pass = decltype(pass_)::value;
      if (pass >= npass) return;
      const int wbeg = k_begin + (4 * pass + wave) * KPW;
      for (int c0 = 0; c0 < NIT; c0 += U) {
        if (wbeg + c0 * KPI >= k_end) break;
        uint4 kr[U], vr[U];
        bool ok[U];
        size_t ko[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {   // a key past the split's end reads its last key (masked)
          const int j = wbeg + (c0 + u) * KPI + grp;
          ok[u] = j < k_end;
          ko[u] = key_off(pass_, min(j, k_end - 1));
          kr[u] = ld16_stream(Kh + ko[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) vr[u] = ld16_stream(Vh + ko[u]);
#pragma unroll
        for (int st = 0; st < P; ++st) {
          if (st > 0 && wbeg + (c0 + st * kUnroll) * KPI >= k_end) break;   // the steps one at a time
          scores(kr + st * kUnroll, ok + st * kUnroll);
          accumulate(vr + st * kUnroll, ok + st * kUnroll);
        }
      }
    });
  }
  // Sum over the key groups of the wave (lanes with equal `sub`); scores were replicated per group.
  l_run = wave_sum(l_run, LPK);
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = wave_sum(o[e], LPK);

  if (grp == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) so[wave * D + sub * E + e] = o[e];
  }
  if (lane == 0) {
    sm[wave] = m_run;
    sl[wave] = l_run;
  }
  __syncthreads();
  if (wave == 0) {
    float M = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
    float w[4], L = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[i] = (sm[i] == -INFINITY) ? 0.f : exp2f(sm[i] - M);
      L = fmaf(sl[i], w[i], L);
    }
    // Lane l writes columns CPL l .. CPL l + CPL - 1 with one store.  A long split's partial is
    // stored non-temporally: written back from the L2 at random times, partials slow the cache
    // stream around them (a load-only replay of the long-context grid: 688 us without the partial
    // writes, 710 us with plain stores, 697 us with non-temporal ones), while short splits' partials
    // are better kept in the L2 for the merge that follows.
    constexpr int CPL = D / kWave;
    typedef float cvec_t __attribute__((ext_vector_type(CPL)));
    cvec_t acc;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane * CPL + j;
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) a = (w[i] != 0.f) ? fmaf(so[i * D + c], w[i], a) : a;
      acc[j] = a;
    }
    cvec_t *dst = reinterpret_cast<cvec_t *>(&part_o[pidx * D + lane * CPL]);
    if (npass > 1) {
      __builtin_nontemporal_store(acc, dst);
      if (lane == 0) {
        __builtin_nontemporal_store(M, &part_ml[2 * pidx]);
        __builtin_nontemporal_store(L, &part_ml[2 * pidx + 1]);
      }
    } else {
      // (The empty asm statements keep the compiler from merging these stores with the
      // non-temporal ones above, which would drop the non-temporal hint.)
      asm volatile("" ::: "memory");
      *dst = acc;
      if (lane == 0) {
        part_ml[2 * pidx] = M;
        part_ml[2 * pidx + 1] = L;
      }
      asm volatile("" ::: "memory");
    }
  }
}

template <typename T, int D, bool kChunkRows, bool kPaged>
__global__ __launch_bounds__(256) void attn_rows_split(const T *q, int ld_q, int nh, int row0,
                                                       ChunkSet cs, DecodeGroup dg, PagePool pool,
                                                       int stride, int prow0,
                                                       float *part_o, float *part_ml, float qscale) {
  __shared__ float sm[4], sl[4], so[4 * D];
  // Decode rows (at most kMaxDecodesPerLaunch): grid (heads, rows, splits), so a row's heads run
  // together and the splits come last; chunk rows (any number): grid (rows, splits, heads).
  const int r = kChunkRows ? blockIdx.x : blockIdx.y, s = kChunkRows ? blockIdx.y : blockIdx.z,
            h = kChunkRows ? blockIdx.z : blockIdx.x;
  split_attn_item<T, D, kChunkRows, kPaged>(row0 + r, s, h, q, ld_q, nh, cs, dg, pool, stride, prow0,
                                            part_o, part_ml, qscale, sm, sl, so);
}

// Chunk and decode attention in one launch.  Workgroups [0, chunk_grid) run the chunk work items
// (attn_chunk_body.h), the others the key splits of the decode rows [dec_row0, dec_row0 + dec_rows).
// The chunk items are few and latency-bound (one 64-query block each, walking its key range tile by
// tile) and leave most compute units idle; the memory-bound decode splits fill them, so the two kinds
// of attention of a hybrid batch overlap instead of running one after the other.
template <int D, bool kPaged, int RB>
__global__ __launch_bounds__(256) void attn_fused(const bf16_t *q, int ld_q, int nh, ChunkSet cs,
                                                  PagePool pool, bf16_t *out, OutLayout olay,
                                                  float chunk_qscale, int n_split, AttnParts parts,
                                                  int per_xcd, int chunk_grid, DecodeGroup dg,
                                                  int dec_row0, int dec_rows, float dec_qscale) {
  SARATHI_CHUNK_LDS(D);
  __shared__ float sm[4], sl[4], so[4 * D];
  const int b = blockIdx.x;
  if (b < chunk_grid) {
    chunk_attn_item<D, kPaged, RB>(chunk_item_of(b, per_xcd), q, ld_q, nh, cs, pool, out, olay,
                               chunk_qscale, n_split, parts.stride_c, parts.o_c, parts.ml_c, k0s, v0s,
                               k1s, v1s, k2s, v2s);
  } else {
    const int d = b - chunk_grid;   // heads fastest, then rows, then splits
    const int hd = d % nh, rest = d / nh;
    split_attn_item<bf16_t, D, false, kPaged, kPrefetchFused>(
        dec_row0 + rest % dec_rows, rest / dec_rows, hd, q, ld_q, nh, cs, dg, pool,
        parts.stride_d, cs.rows, parts.o_d, parts.ml_d, dec_qscale, sm, sl, so);
  }
}

template <int D, bool kPaged, int RB>
hipError_t run_fused(const void *q, int ld_q, int nh, const ChunkSet &cs, const PagePool &pool, void *out,
                     OutLayout olay, int n_split, const AttnParts &parts, const DecodeGroup &dg, int dec_row0,
                     int dec_rows, hipStream_t s) {
  int items = 0;
  for (int j = 0; j < cs.n; ++j) items += chunk_items(cs.len[j], cs.split[j], nh, kBQ * RB);
  const int per_xcd = (items + 7) / 8;
  const int chunk_grid = 8 * per_xcd;
  const int grid = chunk_grid + dec_rows * parts.stride_d * nh;
  const float qscale = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL((attn_fused<D, kPaged, RB>), dim3(grid), dim3(256), 0, s,
                     static_cast<const bf16_t *>(q), ld_q, nh, cs, pool, static_cast<bf16_t *>(out),
                     olay, qscale, n_split, parts, per_xcd, chunk_grid, dg, dec_row0, dec_rows,
                     qscale);
  return hipGetLastError();
}

// Merge of the split partials, four waves per workgroup.  Pairs with at most kFewSplits splits are
// merged by D / 4 lanes each (several per wave) or a whole wave (combine_few); the general merge
// takes a whole wave per pair: lane l holds the (m, l) of splits l, l + 64, ...; the wave max M and
// the weights w_s = 2^(m_s - M) (0 for empty splits) come from lane shuffles, then each lane
// accumulates its D / 64 output elements over the splits, all loads of a group of splits issued
// before their adds.
constexpr int kCombineWaves = 4;
constexpr int kCombineSlots = kMaxKeySplits / kWave;   // splits per lane
constexpr int kFewSplits = 8;

// The merge of ns <= kFewSplits partials of one (row, head).  Every (m, l) pair is written (l = 0
// for a split with no keys of the row), but a split with l = 0 may have left its o slot unwritten,
// so such a split is skipped rather than multiplied by 0.  Every load is issued at once: each lane
// reads all (m, l) pairs and one 4-column piece of o from each of its splits; the wave's lanes form
// SPL groups of D / 4, group g taking splits g, g + SPL, ... (summed in that order, then the groups
// in order g = 0, 1, ...).
template <typename T, int D>
__device__ __forceinline__ void combine_few(int ns, size_t base, int r, int h, const float *part_o,
                                            const float *part_ml, T *out, OutLayout olay) {
  constexpr int LPS = D / 4;            // lanes per split (4 columns each)
  constexpr int SPL = kWave / LPS;      // splits per wave load
  constexpr int NJ = (kFewSplits + SPL - 1) / SPL;
  const int lane = threadIdx.x & 63, grp = lane / LPS, col = (lane % LPS) * 4;
  float2 ml[kFewSplits];
#pragma unroll
  for (int s = 0; s < kFewSplits; ++s)
    ml[s] = s < ns ? *reinterpret_cast<const float2 *>(&part_ml[2 * (base + s)]) : make_float2(-INFINITY, 0.f);
  float4 ov[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int sp = j * SPL + grp;
    ov[j] = sp < ns ? *reinterpret_cast<const float4 *>(&part_o[(base + sp) * D + col])
                    : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kFewSplits; ++s)
    if (ml[s].y > 0.f) M = fmaxf(M, ml[s].x);
  float L = 0.f, w[kFewSplits];
#pragma unroll
  for (int s = 0; s < kFewSplits; ++s) {
    w[s] = ml[s].y > 0.f ? exp2f(ml[s].x - M) : 0.f;
    L = fmaf(ml[s].y, w[s], L);
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    float ws = 0.f;
#pragma unroll
    for (int s = 0; s < kFewSplits; ++s) ws = (s == j * SPL + grp) ? w[s] : ws;
    if (ws != 0.f) {
      acc[0] = fmaf(ws, ov[j].x, acc[0]);
      acc[1] = fmaf(ws, ov[j].y, acc[1]);
      acc[2] = fmaf(ws, ov[j].z, acc[2]);
      acc[3] = fmaf(ws, ov[j].w, acc[3]);
    }
  }
  // Groups in order: after step m, group 0 holds the sum of groups 0 .. 2^(m+1) - 1 (each step adds
  // the group LPS 2^m lanes up, through sum_xor: the same sum as a shuffle down).
#pragma unroll
  for (int o = LPS; o < kWave; o <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = sum_xor(acc[e], o);
  }
  if (grp == 0) {   // 4 consecutive columns, within one k-tile of a k-tile-major output
    const float inv = 1.0f / L;
    T *dst = &out[out_index(olay, r, h * D + col)];
    if constexpr (sizeof(T) == 2) {
      uint2 u;
      u.x = (uint32_t)from_f32<T>(acc[0] * inv) | ((uint32_t)from_f32<T>(acc[1] * inv) << 16);
      u.y = (uint32_t)from_f32<T>(acc[2] * inv) | ((uint32_t)from_f32<T>(acc[3] * inv) << 16);
      *reinterpret_cast<uint2 *>(dst) = u;
    } else {
      *reinterpret_cast<float4 *>(dst) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    }
  }
}

// The same merge with D / 4 lanes per (row, head) pair, so a wave merges kWave / (D / 4) pairs: each
// lane reads the (m, l) of all its pair's splits and its 4 columns of o from every split, all loads
// issued at once.  The sum runs in combine_few's order (per group g the splits g, g + SPL, ..., then
// the groups' sums as combine_few's lane tree adds them), so a pair gets the same bits from either.
template <typename T, int D>
__device__ __forceinline__ void combine_lanes(int ns, size_t base, int r, int h, const float *part_o,
                                              const float *part_ml, T *out, OutLayout olay) {
#pragma clang fp contract(off)
  constexpr int LPS = D / 4;
  constexpr int SPL = kWave / LPS;
  const int col = (threadIdx.x % LPS) * 4;
  float2 ml[kFewSplits];
  float4 ov[kFewSplits];
#pragma unroll
  for (int s = 0; s < kFewSplits; ++s) {
    ml[s] = s < ns ? *reinterpret_cast<const float2 *>(&part_ml[2 * (base + s)]) : make_float2(-INFINITY, 0.f);
    ov[s] = s < ns ? *reinterpret_cast<const float4 *>(&part_o[(base + s) * D + col])
                   : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kFewSplits; ++s)
    if (ml[s].y > 0.f) M = fmaxf(M, ml[s].x);
  float L = 0.f, acc[SPL][4] = {};
#pragma unroll
  for (int s = 0; s < kFewSplits; ++s) {
    const float w = ml[s].y > 0.f ? exp2f(ml[s].x - M) : 0.f;
    L = fmaf(ml[s].y, w, L);
    if (w != 0.f) {
      float *a = acc[s % SPL];
      a[0] = fmaf(w, ov[s].x, a[0]);
      a[1] = fmaf(w, ov[s].y, a[1]);
      a[2] = fmaf(w, ov[s].z, a[2]);
      a[3] = fmaf(w, ov[s].w, a[3]);
    }
  }
#pragma unroll
  for (int st = 1; st < SPL; st <<= 1)
#pragma unroll
    for (int g = 0; g < SPL; g += 2 * st)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[g][e] = acc[g][e] + acc[g + st][e];
  const float inv = 1.0f / L;
  T *dst = &out[out_index(olay, r, h * D + col)];
  if constexpr (sizeof(T) == 2) {
    uint2 u;
    u.x = (uint32_t)from_f32<T>(acc[0][0] * inv) | ((uint32_t)from_f32<T>(acc[0][1] * inv) << 16);
    u.y = (uint32_t)from_f32<T>(acc[0][2] * inv) | ((uint32_t)from_f32<T>(acc[0][3] * inv) << 16);
    *reinterpret_cast<uint2 *>(dst) = u;
  } else {
    *reinterpret_cast<float4 *>(dst) =
        make_float4(acc[0][0] * inv, acc[0][1] * inv, acc[0][2] * inv, acc[0][3] * inv);
  }
}

// Where a (row, head) pair's partials are, and how it is merged: kind 0 leaves it alone (a row of
// an unsplit chunk, written by the chunk kernel), 1 takes the few-split merge over ns splits, 2 the
// general one over n_used slots.
struct PairMerge {
  size_t base;
  const float *o, *ml;
  int n, kind;
};
__device__ __forceinline__ PairMerge pair_merge(int r, int h, int nh, int chunk_rows, int chunk_splits,
                                                const ChunkSplits &table, const AttnParts &parts) {
  PairMerge p;
  if (r < chunk_rows) {
    p.base = ((size_t)r * nh + h) * parts.stride_c;
    p.o = parts.o_c;
    p.ml = parts.ml_c;
    p.n = chunk_splits;
    p.kind = 2;
    if (chunk_splits == 0) {
      // The row's chunk, found with constant-index selects (the table is a by-value argument).
      int ns = table.split[0];
#pragma unroll
      for (int i = 1; i < kMaxChunks; ++i)
        if (i < table.n && r >= table.row0[i]) ns = table.split[i];
      p.n = ns;
      p.kind = ns <= 1 ? 0 : ns <= kFewSplits ? 1 : 2;
    }
  } else {
    p.base = ((size_t)(r - chunk_rows) * nh + h) * parts.stride_d;
    p.o = parts.o_d;
    p.ml = parts.ml_d;
    p.n = parts.stride_d;   // every decode of the group has at most this many splits
    p.kind = parts.stride_d <= kFewSplits ? 1 : 2;
  }
  return p;
}

// The general merge of one (row, head) pair's n_used split slots by a whole wave.
template <typename T, int D>
__device__ __forceinline__ void combine_general(int n_used, size_t base, int r, int h,
                                                const float *part_o, const float *part_ml, T *out,
                                                OutLayout olay) {
  const int lane = threadIdx.x & 63;
  float m[kCombineSlots], l[kCombineSlots], w[kCombineSlots];
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kCombineSlots; ++k) {
    const int sp = lane + k * kWave;
    m[k] = -INFINITY;
    l[k] = 0.f;
    if (sp < n_used) {
      const float2 ml = *reinterpret_cast<const float2 *>(&part_ml[2 * (base + sp)]);
      if (ml.y > 0.f) {
        m[k] = ml.x;
        l[k] = ml.y;
      }
    }
    M = fmaxf(M, m[k]);
  }
  M = wave_max(M);
  // A row's non-empty splits come first (l >= 1 for each: its largest score contributes 2^0); the
  // empty ones after them hold no output, so only the leading non-empty splits are read.
  int n_keyed = 0;
#pragma unroll
  for (int k = 0; k < kCombineSlots; ++k)
    if (l[k] > 0.f) n_keyed = lane + k * kWave + 1;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) n_keyed = max(n_keyed, __shfl_xor(n_keyed, o, kWave));
  n_used = n_keyed;
  float L = 0.f;
#pragma unroll
  for (int k = 0; k < kCombineSlots; ++k) {
    w[k] = l[k] > 0.f ? exp2f(m[k] - M) : 0.f;
    L = fmaf(l[k], w[k], L);
  }
  L = wave_sum(L);
  constexpr int PER = D / kWave;
  float acc[PER] = {};
  constexpr int kGroup = 4;
  for (int s0 = 0; s0 < n_used; s0 += kGroup) {
    float v[kGroup][PER], ws[kGroup];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const int sp = min(s0 + u, n_used - 1);
      float wk = w[0];
#pragma unroll
      for (int k = 1; k < kCombineSlots; ++k) wk = sp / kWave == k ? w[k] : wk;   // wave-uniform
      ws[u] = s0 + u < n_used ? __shfl(wk, sp % kWave, kWave) : 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i) v[u][i] = part_o[(base + sp) * D + lane + i * kWave];
    }
    // A split with weight 0 (no keys, or a padding slot of the group) adds nothing; its o slot may
    // never have been written, so it is skipped rather than multiplied by 0.
#pragma unroll
    for (int u = 0; u < kGroup; ++u)
      if (ws[u] != 0.f) {
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] = fmaf(ws[u], v[u][i], acc[i]);
      }
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    out[out_index(olay, r, h * D + lane + i * kWave)] = from_f32<T>(acc[i] * inv);
}

// One launch merges every split row of the batch.  A wave takes kWave / (D / 4) consecutive (row, head)
// pairs; when none of them needs the general merge, each pair gets D / 4 lanes (combine_lanes),
// otherwise the wave merges them one after the other with all its lanes.
template <typename T, int D>
__global__ __launch_bounds__(64 * kCombineWaves) void attn_combine(int nh, int row0, int n_rows,
                                                                   int chunk_rows, int chunk_splits,
                                                                   ChunkSplits table,
                                                                   AttnParts parts, T *out,
                                                                   OutLayout olay) {
  constexpr int LPS = D / 4, PPW = kWave / LPS;   // lanes per pair, pairs per wave
  const int wave = blockIdx.x * kCombineWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_pairs = n_rows * nh;
  {
    const int pair = wave * PPW + (threadIdx.x & 63) / LPS;
    PairMerge p{0, nullptr, nullptr, 0, 0};
    int r = 0, h = 0;
    if (pair < n_pairs) {
      r = row0 + pair / nh;
      h = pair % nh;
      p = pair_merge(r, h, nh, chunk_rows, chunk_splits, table, parts);
    }
    if (!__any(p.kind == 2)) {
      if (p.kind == 1) combine_lanes<T, D>(p.n, p.base, r, h, p.o, p.ml, out, olay);
      return;
    }
  }
#pragma unroll 1
  for (int i = 0; i < PPW; ++i) {
    const int pair = wave * PPW + i;   // wave-uniform
    if (pair >= n_pairs) return;
    const int r = row0 + pair / nh, h = pair % nh;
    const PairMerge p = pair_merge(r, h, nh, chunk_rows, chunk_splits, table, parts);
    if (p.kind == 1)
      combine_few<T, D>(p.n, p.base, r, h, p.o, p.ml, out, olay);
    else if (p.kind == 2)
      combine_general<T, D>(p.n, p.base, r, h, p.o, p.ml, out, olay);
  }
}

template <typename T, int D>
hipError_t run_split(const void *q, int ld_q, int nh, int row0, int n_rows, const ChunkSet &cs,
                     const DecodeGroup &dg, const PagePool &pool, int stride, int prow0, float *po,
                     float *pml, hipStream_t s) {
  const float qscale = 1.4426950408889634f / sqrtf((float)D);
#define SARATHI_SPLIT(CR, PG)                                                                   \
  hipLaunchKernelGGL((attn_rows_split<T, D, CR, PG>), CR ? dim3(n_rows, stride, nh) : dim3(nh, n_rows, stride), \
                     dim3(256), 0, s,                                                            \
                     static_cast<const T *>(q), ld_q, nh, row0, cs, dg, pool, stride, prow0, po, pml, qscale)
  const bool chunk_rows = row0 < cs.rows, paged = pool.k != 0;
  if (chunk_rows) {
    if (paged) SARATHI_SPLIT(true, true); else SARATHI_SPLIT(true, false);
  } else {
    if (paged) SARATHI_SPLIT(false, true); else SARATHI_SPLIT(false, false);
  }
#undef SARATHI_SPLIT
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_combine(int nh, int row0, int n_rows, int chunk_rows, int chunk_splits,
                       const ChunkSplits &table, const AttnParts &parts, void *out, OutLayout olay,
                       hipStream_t s) {
  const int waves = (n_rows * nh + kWave / (D / 4) - 1) / (kWave / (D / 4));
  hipLaunchKernelGGL((attn_combine<T, D>), dim3((waves + kCombineWaves - 1) / kCombineWaves),
                     dim3(64 * kCombineWaves), 0, s, nh, row0, n_rows, chunk_rows, chunk_splits,
                     table, parts, static_cast<T *>(out), olay);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_rows(int type, int d, const void *q, int ld_q, int nh, int row0, int n_rows,
                            const ChunkSet &cs, const DecodeGroup &dg, const PagePool &pool,
                            int stride, int prow0, float *part_o, float *part_ml, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  if (stride < 1 || stride > kMaxKeySplits || prow0 > row0 || !part_o || !part_ml) return hipErrorInvalidValue;
#define SARATHI_ROWS(T, D) \
  return run_split<T, D>(q, ld_q, nh, row0, n_rows, cs, dg, pool, stride, prow0, part_o, part_ml, s)
  if (type == kF32 && d == 64) SARATHI_ROWS(float, 64);
  if (type == kF32 && d == 128) SARATHI_ROWS(float, 128);
  if (type == kBF16 && d == 64) SARATHI_ROWS(bf16_t, 64);
  if (type == kBF16 && d == 128) SARATHI_ROWS(bf16_t, 128);
#undef SARATHI_ROWS
  return hipErrorInvalidValue;
}

hipError_t launch_attn_combine(int type, int d, int nh, int row0, int n_rows, int chunk_rows,
                               int chunk_splits, const ChunkSplits &table, const AttnParts &parts,
                               void *out, OutLayout olay, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  if (row0 + n_rows > chunk_rows &&
      (parts.stride_d < 1 || parts.stride_d > kMaxKeySplits || !parts.o_d || !parts.ml_d))
    return hipErrorInvalidValue;
  if (row0 < chunk_rows) {   // some merged rows are chunk rows
    if (parts.stride_c < 1 || parts.stride_c > kMaxKeySplits || !parts.o_c || !parts.ml_c)
      return hipErrorInvalidValue;
    if (chunk_splits < 0 || chunk_splits > parts.stride_c) return hipErrorInvalidValue;
    if (chunk_splits == 0) {   // the table serves
      if (table.n < 1 || table.n > kMaxChunks) return hipErrorInvalidValue;
      for (int j = 0; j < table.n; ++j)
        if (table.split[j] < 1 || table.split[j] > parts.stride_c) return hipErrorInvalidValue;
    }
  }
#define SARATHI_COMBINE(T, D) \
  return run_combine<T, D>(nh, row0, n_rows, chunk_rows, chunk_splits, table, parts, out, olay, s)
  if (type == kF32 && d == 64) SARATHI_COMBINE(float, 64);
  if (type == kF32 && d == 128) SARATHI_COMBINE(float, 128);
  if (type == kBF16 && d == 64) SARATHI_COMBINE(bf16_t, 64);
  if (type == kBF16 && d == 128) SARATHI_COMBINE(bf16_t, 128);
#undef SARATHI_COMBINE
  return hipErrorInvalidValue;
}

hipError_t launch_attn_fused(int d, const void *q, int ld_q, int nh, const ChunkSet &cs,
                             const PagePool &pool, void *out, OutLayout olay, int n_split,
                             const AttnParts &parts, const DecodeGroup &dg, int dec_row0,
                             int dec_rows, hipStream_t s) {
  if (cs.n <= 0 || cs.n > kMaxChunks || dec_rows <= 0 || dec_rows > kMaxDecodesPerLaunch)
    return hipErrorInvalidValue;
  if (dec_row0 < cs.rows || parts.stride_d < 1 || parts.stride_d > kMaxKeySplits || !parts.o_d || !parts.ml_d)
    return hipErrorInvalidValue;
  if (n_split < 1 || (n_split > 1 && (parts.stride_c != n_split || !parts.o_c || !parts.ml_c)))
    return hipErrorInvalidValue;
  for (int j = 0; j < cs.n; ++j)
    if (cs.split[j] < 1 || cs.split[j] > n_split) return hipErrorInvalidValue;
  const bool paged = pool.k != 0;
  // two 16-query blocks per wave: contiguous caches only
  if (cs.qblocks != 1 && !(cs.qblocks == 2 && !paged)) return hipErrorInvalidValue;
#define SARATHI_FUSED(D, P, RB) \
  return run_fused<D, P, RB>(q, ld_q, nh, cs, pool, out, olay, n_split, parts, dg, dec_row0, dec_rows, s)
  if (d == 128) {
    if (paged) SARATHI_FUSED(128, true, 1);
    if (cs.qblocks == 2) SARATHI_FUSED(128, false, 2);
    SARATHI_FUSED(128, false, 1);
  }
  if (d == 64) {
    if (paged) SARATHI_FUSED(64, true, 1);
    if (cs.qblocks == 2) SARATHI_FUSED(64, false, 2);
    SARATHI_FUSED(64, false, 1);
  }
#undef SARATHI_FUSED
  return hipErrorInvalidValue;
}

}  // namespace sarathi
