// Fused linear ops of the hybrid batch: out = epilogue(a w^T) over the C+B concatenated rows.
//
// Every projection of the layer (QKV, O, gate/up, down) runs as ONE GEMM over the chunk rows and the
// decode rows together, so each weight tile crosses HBM once for the whole batch and the decodes
// share the chunk's weight fetches (SARATHI: Efficient LLM Inference by Piggybacking Decodes with
// Chunked Prefills, section 3, "Decode-Maximal Batching", "How fusion works").  The token dimension
// is padded only to 32 rows; rows past C+B are never stored (the tile-quantization point of the same
// page, "Identifying the Ideal Chunk Size", Figure 7, restated for 16-row MFMA blocks).
//
// bf16 path.  One workgroup (8 waves as 2 x 4) owns ALL rows of the batch (up to 320; larger batches
// take a few row tiles) and a 128-column stripe of the weights, so a weight tile is read once for
// the whole batch.  v_mfma_f32_16x16x32_bf16; a wave computes up to 160 rows x 32 columns.  A and W
// k-tiles (64 wide) are staged through LDS (swizzled rows, no bank conflicts) with double buffering.  When the weight stripes alone do
// not fill the 256 compute units, the k range is split: each split writes a float32 partial and the
// kernel that consumes the product sums the partials in a fixed order (deterministic, no atomics).
// Workgroup b runs on XCD b % 8; consecutive workgroups of one XCD share a weight stripe.
// fp32 path: a plain FMA tile kernel (exact float32 products, used by the float32 layer mode).
#include <math.h>

#include "kernels.h"

namespace sarathi {
namespace {

constexpr int kBK = 64;         // k extent of one LDS stage (bf16 elements)
constexpr int kLdsK = kBK;      // LDS row: 128 bytes = 8 chunks of 16 bytes, stored swizzled
// Chunk c of LDS row r is stored in slot c ^ ((r >> 1) & 7).  A 16-byte store of two consecutive
// rows then covers the two halves of the 64 banks once each, and the 16 rows a fragment read touches
// at one chunk fall in 16 distinct 4-bank groups: both directions are free of bank conflicts.
__device__ __forceinline__ int swz(int row, int chunk) { return (chunk ^ ((row >> 1) & 7)) * 8; }
#ifndef SARATHI_GEMM_W_RING
#define SARATHI_GEMM_W_RING 2     // weight k-tiles in flight in registers
#endif
#ifndef SARATHI_GEMM_A_RING
#define SARATHI_GEMM_A_RING 1     // activation k-tiles in flight in registers
#endif
#ifndef SARATHI_GEMM_WAVE_COLS
#define SARATHI_GEMM_WAVE_COLS 4   // 4: 8 waves per workgroup, 2: 4 waves
#endif
constexpr int kPlanWaveCols = SARATHI_GEMM_WAVE_COLS;
constexpr int kWM = 2;          // wave rows of a workgroup
constexpr int kMBW = 10;        // max 16-row blocks per wave row: 320 rows per tile
#ifndef SARATHI_GEMM_BN
#define SARATHI_GEMM_BN 128
#endif
constexpr int kBN = SARATHI_GEMM_BN;   // columns per tile (weight rows per stripe)
constexpr int kBMX = 16 * kMBW * kWM;

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }
__device__ __forceinline__ float gelu_f(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

// WN wave columns: WN = 4 gives 8 waves with 144x32 wave tiles (two waves per SIMD); WN = 2 gives
// 4 waves with 144x64 wave tiles (one wave per SIMD, whose 512 registers hold the larger
// accumulator tile), which halves the LDS bytes read per MFMA.
template <int WN, int MB, int EPI>
__global__ __launch_bounds__(64 * kWM * WN) __attribute__((amdgpu_waves_per_eu(WN == 2 ? 1 : 2, WN == 2 ? 1 : 2)))
void gemm_bf16_rows(GemmArgs g, GemmPlan p) {
  static_assert(MB >= 1 && MB <= kMBW, "16-row blocks per wave row");
  constexpr int kThreads = 64 * kWM * WN;
  constexpr int kNB = kBN / (16 * WN);  // 16-column blocks per wave
  constexpr bool kGlu = EPI == kEpiSwiGLU;
  constexpr int A_CH = (kBMX * (kBK / 8) + kThreads - 1) / kThreads;   // 16-B A chunks per thread
  constexpr int B_CH = kBN * (kBK / 8) / kThreads;
  constexpr int kStage = (kBMX + kBN) * kLdsK;
  extern __shared__ __attribute__((aligned(16))) bf16_t lds[];

  // Tile of this workgroup (XCD-aware order: slot s of XCD x takes tile x * per_xcd + s).
  const int bid = blockIdx.x;
  const int t = (bid & 7) * p.per_xcd + (bid >> 3);
  if (t >= p.m_tiles * p.n_tiles * p.splits) return;
  const int m_tile = t % p.m_tiles;
  const int rest = t / p.m_tiles;
  const int split = rest % p.splits;
  const int n_tile = rest / p.splits;
  constexpr int mbw = MB;                   // 16-row blocks per wave row
  constexpr int rows = 32 * MB;             // rows of the tile
  const int m0 = m_tile * rows;
  const int n0 = n_tile * (kGlu ? kBN / 2 : kBN);
  const int nk = g.k / kBK;
  const int kb = (int)((long long)split * nk / p.splits);
  const int ke = (int)((long long)(split + 1) * nk / p.splits);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const bf16_t *A = static_cast<const bf16_t *>(g.a);
  const bf16_t *W0 = static_cast<const bf16_t *>(g.w0);
  const bf16_t *W1 = static_cast<const bf16_t *>(g.w1);

  // Every thread always loads its chunks (rows clamped into the matrix): rows past the tile land in
  // LDS rows no wave reads, and branch-free loads keep the load counters exact across the k loop.
  static_assert(A_CH * kThreads == kBMX * (kBK / 8), "A chunks cover the LDS rows exactly");
  const bf16_t *a_src[A_CH];
  int a_dst[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + i * kThreads, row = c >> 3, kc = c & 7;
    const int gr = min(m0 + row, g.m_alloc - 1);
    a_src[i] = A + (size_t)gr * g.lda + kc * 8 + (size_t)kb * kBK;
    a_dst[i] = row * kLdsK + swz(row, kc);
  }
  const bf16_t *b_src[B_CH];
  int b_dst[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + i * kThreads, row = c >> 3, kc = c & 7;
    int src_row;
    const bf16_t *Wp = W0;
    if (kGlu) {
      // LDS rows of wave column wv: its gate block(s), then the up block(s) of the same columns.
      const int wv = row / (16 * kNB), bb = (row >> 4) % kNB, rl = row & 15;
      const int cb = wv * (kNB / 2) + bb % (kNB / 2);
      src_row = n0 + cb * 16 + rl;
      Wp = (bb >= kNB / 2) ? W1 : W0;
    } else {
      src_row = min(n0 + row, g.n - 1);
      if (g.w1 && src_row >= g.n_w0) {   // the second weight continues the product's rows
        Wp = W1;
        src_row -= g.n_w0;
      }
    }
    src_row = kGlu ? min(src_row, g.n - 1) : src_row;
    b_src[i] = Wp + (size_t)src_row * g.ldw + kc * 8 + (size_t)kb * kBK;
    b_dst[i] = (kBMX + row) * kLdsK + swz(row, kc);   // kBMX is a multiple of 16: same swizzle
  }

  f32x4_t acc[MB][kNB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Register rings: weight k-tiles are fetched kDW tiles ahead of their use (they come from HBM),
  // activation k-tiles kDA ahead (they are shared by every workgroup and mostly hit L2).  Two LDS
  // stages: tile j is computed from stage j&1 while tile j+1 is written into the other stage.
  // Tile indices past the end are clamped (a few redundant loads) so that the steady-state loop body
  // has no branches around its loads.
  constexpr int kDW = SARATHI_GEMM_W_RING, kDA = SARATHI_GEMM_A_RING;
  constexpr int kUnrollK = kDW * kDA;             // a multiple of both ring depths
  uint4 ra[kDA][A_CH], rb[kDW][B_CH];
  const int ntiles = ke - kb;
  auto tile = [&](int j) { return min(j, ntiles - 1) * kBK; };
  auto load_a = [&](int slot, int j) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) ra[slot][i] = ld16(a_src[i] + tile(j));
  };
  auto load_b = [&](int slot, int j) {
#pragma unroll
    for (int i = 0; i < B_CH; ++i) rb[slot][i] = ld16(b_src[i] + tile(j));
  };
  auto store_tile = [&](int aslot, int bslot, int stage) {
    bf16_t *Ls = lds + stage * kStage;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) st16(&Ls[a_dst[i]], ra[aslot][i]);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) st16(&Ls[b_dst[i]], rb[bslot][i]);
  };
  // Fragment rows start at multiples of 16, so a lane's swizzle term is ((lane & 15) >> 1).
  const int frag_row = lane & 15;
  const int frag_k0 = (((lane >> 4) + 0) ^ (frag_row >> 1)) * 8;   // k-step 0: chunks 0..3
  const int frag_k1 = (((lane >> 4) + 4) ^ (frag_row >> 1)) * 8;   // k-step 1: chunks 4..7
  const int a_row0 = wm * 16 * mbw;
  // Fragment reads are grouped ahead of the MFMAs that use them, so each MFMA waits only for its
  // own operands (descending LDS counters) rather than a read round trip every two MFMAs.  With
  // narrow wave tiles both k-steps' fragments fit in registers at once (the MFMAs of k-step 0 then
  // run while k-step 1's reads are in flight); wide wave tiles read one k-step at a time.
  constexpr bool kAllK = kNB <= 2;
  auto compute = [&](int stage) {
    const bf16_t *L = lds + stage * kStage;
    bf16x8_t bw[kAllK ? 2 : 1][kNB], af[kAllK ? 2 : 1][MB];
    auto read = [&](int ks, int slot) {
      const int fk = ks == 0 ? frag_k0 : frag_k1;
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        bw[slot][nb] = *reinterpret_cast<const bf16x8_t *>(
            &L[(kBMX + wn * 16 * kNB + nb * 16 + frag_row) * kLdsK + fk]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        af[slot][mb] = *reinterpret_cast<const bf16x8_t *>(
            &L[(a_row0 + mb * 16 + frag_row) * kLdsK + fk]);
    };
    auto mfma = [&](int slot) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          acc[mb][nb] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[slot][mb], bw[slot][nb], acc[mb][nb], 0, 0, 0);
    };
    if (kAllK) {
      read(0, 0);
      read(1, kAllK ? 1 : 0);
      __builtin_amdgcn_sched_barrier(0);
      mfma(0);
      mfma(kAllK ? 1 : 0);
    } else {
#pragma unroll
      for (int ks = 0; ks < kBK / 32; ++ks) {
        read(ks, 0);
        __builtin_amdgcn_sched_barrier(0);
        mfma(0);
      }
    }
  };

  // One step: compute tile j (ring position u = j mod kUnrollK), stage tile j+1 into the other LDS
  // buffer, refill the freed ring slots, barrier.
  auto step = [&](int u, int j) {
    compute(u & 1);
    const int as = (u + 1) % kDA, bs = (u + 1) % kDW;   // ring slots of tile j+1
    store_tile(as, bs, (u + 1) & 1);
    load_a(as, j + 1 + kDA);
    load_b(bs, j + 1 + kDW);
    __syncthreads();
  };

#pragma unroll
  for (int j = 0; j < kDW; ++j) load_b(j, j);
#pragma unroll
  for (int j = 0; j < kDA; ++j) load_a(j, j);
  store_tile(0, 0, 0);
  load_a(0, kDA);
  load_b(0, kDW);
  __syncthreads();

  const int nsteps = ntiles - 1;   // tiles followed by another tile
  int j0 = 0;
  for (; j0 + kUnrollK <= nsteps; j0 += kUnrollK) {
#pragma unroll
    for (int u = 0; u < kUnrollK; ++u) step(u, j0 + u);
  }
#pragma unroll
  for (int u = 0; u < kUnrollK; ++u) {
    if (j0 + u < nsteps) step(u, j0 + u);
    else if (j0 + u == nsteps) compute(u & 1);   // the last tile
  }

  // Epilogue.  Lane l of a 16x16 block holds rows 4*(l/16)+i, column l%16.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + a_row0 + mb * 16 + (lane >> 4) * 4 + i;
      if (m >= g.m_store) continue;
#pragma unroll
      for (int nb = 0; nb < (kGlu ? kNB / 2 : kNB); ++nb) {
        if (kGlu) {
          const int n = n0 + (wn * (kNB / 2) + nb) * 16 + (lane & 15);
          if (n >= g.n) continue;
          const float gt = acc[mb][nb][i], up = acc[mb][nb + kNB / 2][i];
          static_cast<bf16_t *>(g.out)[(size_t)m * g.ldo + n] = f32_to_bf16(silu_f(gt) * up);
        } else {
          const int n = n0 + wn * 16 * kNB + nb * 16 + (lane & 15);
          if (n >= g.n) continue;
          const float v = acc[mb][nb][i];
          if (EPI == kEpiPartial) {
            g.part[((size_t)split * g.m_store + m) * g.n + n] = v;
          } else if (EPI == kEpiStore) {
            static_cast<bf16_t *>(g.out)[(size_t)m * g.ldo + n] = f32_to_bf16(v);
          } else {  // kEpiGelu
            static_cast<bf16_t *>(g.out)[(size_t)m * g.ldo + n] = f32_to_bf16(gelu_f(v));
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// float32: 64x64 output tile, 16x16 threads with 4x4 outputs each, k staged 16 at a time.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_fma(GemmArgs g) {
  constexpr int TM = 64, TN = 64, TK = 16;
  constexpr bool kGlu = EPI == kEpiSwiGLU;
  __shared__ float As[TK][TM + 1];
  __shared__ float Bs[kGlu ? 2 : 1][TK][TN + 1];
  const float *A = static_cast<const float *>(g.a);
  const float *W0 = static_cast<const float *>(g.w0);
  const float *W1 = static_cast<const float *>(g.w1);
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {}, acc2[4][4] = {};
  for (int k0 = 0; k0 < g.k; k0 += TK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + i * 256, row = idx >> 4, kk = idx & 15;
      const int m = m0 + row, n = n0 + row, k = k0 + kk;
      As[kk][row] = (m < g.m_alloc && k < g.k) ? A[(size_t)m * g.lda + k] : 0.f;
      Bs[0][kk][row] = (n < g.n && k < g.k) ? W0[(size_t)n * g.ldw + k] : 0.f;
      if (kGlu) Bs[kGlu ? 1 : 0][kk][row] = (n < g.n && k < g.k) ? W1[(size_t)n * g.ldw + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4], b2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b[j] = Bs[0][kk][tx + 16 * j];
        if (kGlu) b2[j] = Bs[kGlu ? 1 : 0][kk][tx + 16 * j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if (kGlu) acc2[i][j] = fmaf(a[i], b2[j], acc2[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty + 16 * i;
    if (m >= g.m_store) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n >= g.n) continue;
      const float v = acc[i][j];
      if (EPI == kEpiPartial) g.part[(size_t)m * g.n + n] = v;   // one split in float32 mode
      else {
        float *o = static_cast<float *>(g.out) + (size_t)m * g.ldo + n;
        if (EPI == kEpiStore) *o = v;
        else if (EPI == kEpiSwiGLU) *o = silu_f(v) * acc2[i][j];
        else *o = gelu_f(v);
      }
    }
  }
}

constexpr size_t kLdsBytes = 2 * (size_t)(kBMX + kBN) * kLdsK * sizeof(bf16_t);

template <int WN, int MB, int EPI>
hipError_t run_bf16_mb(const GemmArgs &g, const GemmPlan &p, hipStream_t s) {
  static bool attr_set = false;   // one LDS opt-in per instantiation (host-side, idempotent)
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_bf16_rows<WN, MB, EPI>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((gemm_bf16_rows<WN, MB, EPI>), dim3(p.grid), dim3(64 * kWM * WN), kLdsBytes, s,
                     g, p);
  return hipGetLastError();
}

template <int WN, int EPI>
hipError_t run_bf16_wn(const GemmArgs &g, const GemmPlan &p, hipStream_t s) {
  switch (p.mbw) {
    case 1: return run_bf16_mb<WN, 1, EPI>(g, p, s);
    case 2: return run_bf16_mb<WN, 2, EPI>(g, p, s);
    case 3: return run_bf16_mb<WN, 3, EPI>(g, p, s);
    case 4: return run_bf16_mb<WN, 4, EPI>(g, p, s);
    case 5: return run_bf16_mb<WN, 5, EPI>(g, p, s);
    case 6: return run_bf16_mb<WN, 6, EPI>(g, p, s);
    case 7: return run_bf16_mb<WN, 7, EPI>(g, p, s);
    case 8: return run_bf16_mb<WN, 8, EPI>(g, p, s);
    case 9: return run_bf16_mb<WN, 9, EPI>(g, p, s);
    case 10: return run_bf16_mb<WN, 10, EPI>(g, p, s);
  }
  return hipErrorInvalidValue;
}

template <int EPI>
hipError_t run_bf16(const GemmArgs &g, const GemmPlan &p, hipStream_t s) {
  if (p.wn != kPlanWaveCols) return hipErrorInvalidValue;
  return run_bf16_wn<kPlanWaveCols, EPI>(g, p, s);
}

template <int EPI>
hipError_t run_f32(const GemmArgs &g, hipStream_t s) {
  dim3 grid((g.n + 63) / 64, (g.m_store + 63) / 64);
  hipLaunchKernelGGL(gemm_f32_fma<EPI>, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

GemmPlan plan_gemm(int type, int epi, int m, int n_out, int k, int cus) {
  GemmPlan p{};
  p.epi = epi;
  if (type == kF32) {
    p.m_tiles = (m + 63) / 64;
    p.n_tiles = (n_out + 63) / 64;
    p.splits = 1;
    p.grid = p.m_tiles * p.n_tiles;
    return p;
  }
  p.m_tiles = (m + kBMX - 1) / kBMX;
  const int rows = (m + p.m_tiles - 1) / p.m_tiles;
  p.mbw = (rows + 31) / 32;
  p.wn = kPlanWaveCols;
  const int nk = k / kBK;
  // The split count and the epilogue form depend on the weight shape only, never on the number of
  // batch rows: a row's k-sum is then cut at the same points whatever else is in the batch, so a
  // decode run alone and the same decode inside a hybrid batch give bitwise-equal results.
  // Time model for one 256-row tile: whole rounds of `cus` workgroups, each k-tile at ~half of a
  // CU's MFMA rate, plus the float32 partials written and read back at ~5 TB/s.
  const double m_ref = 256.0;
  const double t_k = 2.0 * m_ref * kBN * kBK / 5.0e12;
  auto est = [&](int tiles, int sp, double part_cols) {
    const int rounds = (tiles * sp + cus - 1) / cus;
    return rounds * (double)((nk + sp - 1) / sp) * t_k + (double)sp * m_ref * part_cols * 8.0 / 5.0e12;
  };
  auto best_split = [&](int tiles, double part_cols, double *t) {
    int bs = 1;
    double bt = 1e30;
    for (int sp = 1; sp <= 8 && sp <= nk; ++sp) {
      const double v = est(tiles, sp, part_cols);
      if (v < bt * 0.98) { bt = v; bs = sp; }
    }
    *t = bt;
    return bs;
  };
  if (epi == kEpiPartial || epi == kEpiStore) {
    p.n_tiles = (n_out + kBN - 1) / kBN;
    double t;
    p.splits = epi == kEpiPartial ? best_split(p.n_tiles, n_out, &t) : 1;
  } else {
    // Fused activation (one pass, no partials) vs split product + activation pass.
    const int n_prod = epi == kEpiSwiGLU ? 2 * n_out : n_out;
    const int fcols = epi == kEpiSwiGLU ? kBN / 2 : kBN;
    const int fused_tiles = (n_out + fcols - 1) / fcols;
    const double t_fused = est(fused_tiles, 1, 0.0);
    double t_split;
    const int tiles_p = (n_prod + kBN - 1) / kBN;
    const int sp = best_split(tiles_p, n_prod, &t_split);
    if (t_split < 0.9 * t_fused) {
      p.epi = kEpiPartial;
      p.n_tiles = tiles_p;
      p.splits = sp;
    } else {
      p.n_tiles = fused_tiles;
      p.splits = 1;
    }
  }
  const int total = p.m_tiles * p.n_tiles * p.splits;
  p.per_xcd = (total + 7) / 8;
  p.grid = 8 * p.per_xcd;
  return p;
}

hipError_t launch_gemm(int type, int epi, const GemmArgs &g, const GemmPlan &p, hipStream_t s) {
  if (type == kF32) {
    switch (epi) {
      case kEpiStore: return run_f32<kEpiStore>(g, s);
      case kEpiPartial: return run_f32<kEpiPartial>(g, s);
      case kEpiSwiGLU: return run_f32<kEpiSwiGLU>(g, s);
      case kEpiGelu: return run_f32<kEpiGelu>(g, s);
    }
  } else {
    switch (epi) {
      case kEpiStore: return run_bf16<kEpiStore>(g, p, s);
      case kEpiPartial: return run_bf16<kEpiPartial>(g, p, s);
      case kEpiSwiGLU: return run_bf16<kEpiSwiGLU>(g, p, s);
      case kEpiGelu: return run_bf16<kEpiGelu>(g, p, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace sarathi
