// Fused linear ops of the hybrid batch: out = epilogue(a w^T) over the C+B concatenated rows.
//
// Every projection of the layer (QKV, O, gate/up, down) runs as ONE GEMM over the chunk rows and the
// decode rows together, so each weight tile crosses HBM once for the whole batch and the decodes
// share the chunk's weight fetches (SARATHI: Efficient LLM Inference by Piggybacking Decodes with
// Chunked Prefills, section 3, "Decode-Maximal Batching", "How fusion works").  The token dimension
// is padded only to 32 rows; rows past C+B are never stored (the tile-quantization point of the same
// page, "Identifying the Ideal Chunk Size", Figure 7, restated for 16-row MFMA blocks).
//
// bf16 path.  One workgroup (8 waves as 2 x 4) owns ALL rows of the batch (up to 576; larger batches
// take a few row tiles) and a 128-column stripe of the weights, so a weight tile is read once for
// the whole batch.  v_mfma_f32_16x16x32_bf16; a wave computes up to 288 rows x 32 columns.  A and W
// k-tiles, 32 deep, travel from global memory straight into LDS (global_load_lds_dwordx4: no staging
// registers, no LDS store instructions) through a ring of as many stages as fit (up to 6), so the
// loads of the next tiles are in flight while tile j is multiplied.  Both operands are k-tile-major,
// [k/32][rows][32] (the norms write A that way, the layer packs its weights that way once), so the
// 32-deep rows of one 1 KiB load are 1 KiB of consecutive bytes in whole 128-byte lines.  The loads
// are what bounds this kernel: a compute unit keeps only ~10 KB of reads in flight, so its fetch rate
// is set by memory latency and by how many requests the tiles cost, and the A tile is fetched by
// every workgroup.
// When the weight stripes alone do not fill the 256 compute units, the k range is split: each split
// writes a float32 partial and the kernel that consumes the product sums the partials in a fixed
// order (deterministic, no atomics); a fused-activation product with more stripes than one round
// runs its first 256 stripes fused and the rest split (plan_gemm_tail).  Workgroup b runs on XCD
// b % 8; consecutive workgroups of one XCD share a weight stripe.
// fp32 path: a plain FMA tile kernel (exact float32 products, used by the float32 layer mode).
#include <math.h>

#include <type_traits>

#include "kernels.h"

namespace sarathi {
namespace {

// Stage depth.  Every tile takes 32-deep k-tiles (64-byte LDS rows, one MFMA k-step per stage): six
// stages of a 288 x 128 tile, four of a 288 x 256 one, three of a 576 x 128 one (the row tiles of
// products whose width is not a whole number of 256-column stripes) fit in LDS.  Against 64-deep stages (128-byte LDS rows, two k-steps) for tiles of up
// to 288 rows, with the weights k-tile-major in both: gate/up at 274 rows 95.6 -> 84.3 us, QKV 52.4
// -> 50.3 us, O and down within 1 us (same box, five interleaved runs each).  64-deep stages stay
// selectable at build time (SARATHI_GEMM_MBW64 = 9) for tiles of up to 288 rows.
template <int BK> struct KGeom {
  static_assert(BK == 32 || BK == 64, "stage depth");
  static constexpr int kChunks = BK / 8;          // 16-byte chunks per LDS row
  static constexpr int kRPL = 1024 / (BK * 2);    // LDS rows per 1 KiB load
  static constexpr int kSteps = BK / 32;          // MFMA k-steps per stage
};
// Chunk c of LDS row r is stored in slot c ^ f(r).  A fragment read takes one chunk of 16 consecutive
// rows (rows 16q .. 16q + 15).  f = (r >> 1) & 7 with 128-byte rows and f = (r >> 1) & 3 with 64-byte
// rows make those reads free of bank conflicts (both measured with the LDS bank-conflict counter on
// this access pattern; with 64-byte rows, f = (r >> 2) & 3, r & 3, (r >> 3) & 3 or no swizzle give
// four conflict cycles per read).
template <int BK> __device__ __forceinline__ int swz_slot(int row, int chunk) {
  return BK == 64 ? chunk ^ ((row >> 1) & 7) : chunk ^ ((row >> 1) & 3);
}
#ifndef SARATHI_GEMM_MAX_STAGES
#define SARATHI_GEMM_MAX_STAGES 6
#endif
constexpr int kMaxStages = SARATHI_GEMM_MAX_STAGES;
constexpr int kPlanWaveCols = 4;   // wave columns of a workgroup (8 waves: 2 rows x 4 columns)
constexpr int kWM = 2;             // wave rows of a workgroup
constexpr int kWaves = kWM * kPlanWaveCols;
// 16-row blocks per wave row: up to 18 (576-row tiles); tiles of up to kMBW64 blocks per wave row
// would take 64-deep stages (0: none do).
#ifndef SARATHI_GEMM_MBW64
#define SARATHI_GEMM_MBW64 0
#endif
constexpr int kMBW64 = SARATHI_GEMM_MBW64;
#ifndef SARATHI_GEMM_MBW
#define SARATHI_GEMM_MBW 18
#endif
constexpr int kMBW = SARATHI_GEMM_MBW;
#ifndef SARATHI_GEMM_BN
#define SARATHI_GEMM_BN 128
#endif
constexpr int kBN = SARATHI_GEMM_BN;   // columns per tile (weight rows per stripe)
// Wide tiles for batches of more than 288 rows: two row tiles of at most 288 rows and 256 columns
// instead of one of 289..576 rows and 128 columns, the same number of workgroups and k-splits.  A
// workgroup then fetches half the activation rows per k-tile and twice the weight rows (the two row
// tiles of a stripe run side by side on one XCD, so the second fetch of a weight line mostly hits its
// L2), reads 13 instead of 20 LDS fragments per 36 MFMAs a wave, and keeps four LDS stages in flight
// instead of three.
#ifndef SARATHI_GEMM_WIDE
#define SARATHI_GEMM_WIDE 1
#endif
constexpr bool kWideTiles = SARATHI_GEMM_WIDE != 0;
constexpr int kBNWide = 256;
constexpr int kMBWide = 9;   // 16-row blocks per wave row of a wide tile: 288 rows
constexpr int kBMX = 16 * kMBW * kWM;
constexpr int kLdsBudget = 160 * 1024;
// Split-K boundaries lie on multiples of 64 k whatever a tile's stage depth, so a row's k-sum is cut
// at the same points in a 288-row tile and in a 576-row one.
constexpr int kSplitK = 64;

__host__ __device__ constexpr int stage_depth(int mb) { return mb > kMBW64 ? 32 : 64; }

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }
// SiLU for the bf16 epilogue: z / (1 + 2^(-z log2 e)) with the hardware exponential and reciprocal,
// each within about one float32 ulp, far below the bfloat16 rounding that follows; the limits hold
// (2^(+large) = inf gives 0, 2^(-large) = 0 gives z).  The libm forms cost the epilogue, which every
// workgroup runs at the same time at the end of the GEMM, about 4 us at 274 rows.
__device__ __forceinline__ float silu_bf16_epilogue(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}
__device__ __forceinline__ float gelu_f(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

// Stage geometry for MB 16-row blocks per wave row.  One global_load_lds_dwordx4 moves 64 lanes x
// 16 bytes = 1 KiB, i.e. kRPL LDS rows; the A rows of a stage take kRowsA / kRPL such loads, the
// weight rows kBN / kRPL, dealt round-robin to the 8 waves.  As many stages as fit in LDS (up to
// kMaxStages) are kept in flight: the loads of a tile are issued that many steps before its use,
// which is what hides the memory latency.
template <int MB, int BN> struct StageGeom {
  static constexpr int kBK = stage_depth(MB);
  using K = KGeom<kBK>;
  static constexpr int kRowsA = 32 * MB;
  static constexpr int kElems = (kRowsA + BN) * kBK;
  static constexpr int kFit = kLdsBudget / (kElems * 2);
  static constexpr int kStages = kFit < kMaxStages ? kFit : kMaxStages;
  static_assert(kStages >= 2, "two stages fit in LDS");
  static constexpr int kLoadsA = kRowsA / K::kRPL;
  static constexpr int kAI = (kLoadsA + kWaves - 1) / kWaves;   // A loads of waves 0 .. kARem - 1
  static constexpr int kARem = kLoadsA % kWaves;                // (the others issue kAI - 1 if > 0)
  static constexpr int kBI = BN / K::kRPL / kWaves;             // weight loads per wave
  static_assert(kRowsA % K::kRPL == 0, "whole loads of A rows");
  static_assert(BN % (K::kRPL * kWaves) == 0, "weight rows split evenly over the waves");
  static_assert((kStages - 2) * (kAI + kBI) < 64, "loads in flight fit the wait counter");
};

template <int MB, int EPI, int BN>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_rows(GemmArgs g, GemmPlan p) {
  static_assert(MB >= 1 && MB <= kMBW, "16-row blocks per wave row");
  static_assert(BN == kBN || (BN == kBNWide && MB <= kMBWide), "tile shape");
  using G = StageGeom<MB, BN>;
  constexpr int BK = G::kBK;
  using K = KGeom<BK>;
  constexpr int WN = kPlanWaveCols;
  constexpr int kNB = BN / (16 * WN);   // 16-column blocks per wave
  constexpr bool kGlu = EPI == kEpiSwiGLU;
  constexpr int kNSt = G::kStages;
  // One array per stage: the compiler then knows that reading one stage does not depend on the
  // loads still landing in the others.
  __shared__ __attribute__((aligned(1024))) bf16_t st0[G::kElems];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[G::kElems];
  __shared__ __attribute__((aligned(1024))) bf16_t st2[kNSt > 2 ? G::kElems : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t st3[kNSt > 3 ? G::kElems : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t st4[kNSt > 4 ? G::kElems : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t st5[kNSt > 5 ? G::kElems : 8];
  static_assert(kNSt <= 6, "stage arrays");
  auto stage = [&](int u) -> bf16_t * {
    return u == 0 ? st0 : u == 1 ? st1 : u == 2 ? st2 : u == 3 ? st3 : u == 4 ? st4 : st5;
  };

  // Tile of this workgroup (XCD-aware order: slot s of XCD x takes tile x * per_xcd + s).
  const int bid = blockIdx.x;
  const int t = (bid & 7) * p.per_xcd + (bid >> 3);
  if (t >= p.m_tiles * p.n_tiles * p.splits) return;
  const int m_tile = t % p.m_tiles;
  const int rest = t / p.m_tiles;
  const int split = rest % p.splits;
  const int n_tile = rest / p.splits;
  const int m0 = m_tile * G::kRowsA;
  const int n0 = n_tile * (kGlu ? BN / 2 : BN);
  const int nk = g.k / kSplitK;
  const int kb = (int)((long long)split * nk / p.splits) * (kSplitK / BK);   // in BK-deep k-tiles
  const int ke = (int)((long long)(split + 1) * nk / p.splits) * (kSplitK / BK);
  const int ntiles = ke - kb;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const bf16_t *A = static_cast<const bf16_t *>(g.a);
  const bf16_t *W0 = static_cast<const bf16_t *>(g.w0);
  const bf16_t *W1 = static_cast<const bf16_t *>(g.w1);

  // Per-lane sources of this wave's loads.  Load q fills LDS rows kRPL q .. kRPL q + kRPL - 1; lane
  // l lands in row kRPL q + l / kChunks, slot l % kChunks, so it fetches the chunk that the swizzle
  // stores in that slot.  The A loads are dealt round-robin, so waves kARem .. 7 issue one fewer per
  // stage than the first kARem (every request a compute unit keeps in flight counts: the loads are
  // this kernel's bound); each wave waits on its own count.  Rows are clamped into the matrices:
  // rows past the batch fill LDS rows whose products are never stored.
  const int lrow = lane / K::kChunks, lslot = lane % K::kChunks;
  const bf16_t *a_src[G::kAI];
  int a_lds[G::kAI];
#pragma unroll
  for (int i = 0; i < G::kAI; ++i) {
    const int q = min(wave + kWaves * i, G::kLoadsA - 1);
    const int row = K::kRPL * q + lrow;
    const int gr = min(m0 + row, g.m_alloc - 1);
    const size_t a_row = g.a_kmajor ? ((size_t)kb * g.m_alloc + gr) * BK : (size_t)gr * g.lda + (size_t)kb * BK;
    a_src[i] = A + a_row + swz_slot<BK>(row, lslot) * 8;
    a_lds[i] = K::kRPL * q * BK;
  }
  const bf16_t *b_src[G::kBI];
  int b_step[G::kBI];   // elements from one k-tile of a lane's weight row to the next
#pragma unroll
  for (int i = 0; i < G::kBI; ++i) {
    const int row = K::kRPL * (wave + kWaves * i) + lrow;   // weight row within the stripe's LDS block
    int src_row;
    bool second = false;
    if (kGlu) {
      // LDS rows of wave column wv: its gate block(s), then the up block(s) of the same columns.
      const int wv = row / (16 * kNB), bb = (row >> 4) % kNB, rl = row & 15;
      const int cb = wv * (kNB / 2) + bb % (kNB / 2);
      src_row = min(n0 + cb * 16 + rl, g.n - 1);
      second = bb >= kNB / 2;
    } else {
      src_row = min(n0 + row, g.n - 1);
      if (g.w1 && src_row >= g.n_w0) {   // the second weight continues the product's rows
        second = true;
        src_row -= g.n_w0;
      }
    }
    const bf16_t *Wp = second ? W1 : W0;
    // kRowsA is a multiple of 16, so the weight block's rows swizzle like rows 0..BN-1
    const int chunk = swz_slot<BK>(row, lslot) * 8;
    if (g.w_kmajor) {
      const int slab = second ? g.w_slab1 : g.w_slab0;
      b_src[i] = Wp + (size_t)kb * slab + (size_t)src_row * BK + chunk;
      b_step[i] = slab;
    } else {
      b_src[i] = Wp + (size_t)src_row * g.ldw + (size_t)kb * BK + chunk;
      b_step[i] = BK;
    }
  }

  // Loads of k-tile j (clamped to the last tile, so every wave issues the same loads every step)
  // into LDS stage `st`.  A k-tile of a k-tile-major A lies m_alloc * BK elements after the previous.
  const int a_kstep = g.a_kmajor ? g.m_alloc * BK : BK;
  // kX: this wave issues the extra A load (a template constant, so each form of the k loop below is
  // straight-line code; a run-time test per load measured 10-35% slower).
  auto issue = [&](auto kX, bf16_t *st, int j) {
    const int jj = min(j, ntiles - 1);
    const int a_kofs = jj * a_kstep;
#pragma unroll
    for (int i = 0; i < G::kAI; ++i)
      if (i < G::kAI - 1 || decltype(kX)::value) dma16(a_src[i] + a_kofs, st + a_lds[i]);
#pragma unroll
    for (int i = 0; i < G::kBI; ++i) {
      const int q = wave + kWaves * i;
      dma16(b_src[i] + jj * b_step[i], st + (G::kRowsA + K::kRPL * q) * BK);
    }
  };

  f32x4_t acc[MB][kNB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Fragment rows start at multiples of 16, so a lane's swizzle term depends on lane & 15 only.
  // Both k-steps' fragments of a 64-deep tile are read before its MFMAs, so the MFMAs of k-step 0
  // run while the reads of k-step 1 are in flight; a 32-deep tile of a tall workgroup tile (one
  // k-step, up to 18 A fragments per wave) leaves the read order to the compiler's scheduler.
  const int frag_row = lane & 15;
  int frag_k[K::kSteps];
#pragma unroll
  for (int ks = 0; ks < K::kSteps; ++ks) frag_k[ks] = swz_slot<BK>(frag_row, (lane >> 4) + 4 * ks) * 8;
  const int a_row0 = wm * 16 * MB;
  auto compute = [&](const bf16_t *L) {
    bf16x8_t fa[K::kSteps][MB], fb[K::kSteps][kNB];
#pragma unroll
    for (int ks = 0; ks < K::kSteps; ++ks) {
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        fb[ks][nb] = *reinterpret_cast<const bf16x8_t *>(
            &L[(G::kRowsA + wn * 16 * kNB + nb * 16 + frag_row) * BK + frag_k[ks]]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        fa[ks][mb] = *reinterpret_cast<const bf16x8_t *>(&L[(a_row0 + mb * 16 + frag_row) * BK + frag_k[ks]]);
    }
    if (K::kSteps > 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < K::kSteps; ++ks)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[ks][mb], fb[ks][nb], acc[mb][nb], 0, 0, 0);
  };

  // Step j (stage u = j mod kNSt): start the loads of tile j + kNSt - 1 into the stage that step j - 1
  // finished reading, multiply tile j, then wait until this wave's loads of tile j + 1 have landed
  // (at most kNSt - 2 tiles' loads outstanding) and meet the other waves: tile j + 1 is then complete
  // in LDS and nobody reads stage u any more.
  auto k_loop = [&](auto kX) {
    constexpr int kLoads = G::kAI - 1 + (decltype(kX)::value ? 1 : 0) + G::kBI;   // per stage
    auto step = [&](int u, int j) {
      issue(kX, stage((u + kNSt - 1) % kNSt), j + kNSt - 1);
      compute(stage(u));
      wait_vm_lgkm0<(kNSt - 2) * kLoads>();
      stage_barrier();
    };
#pragma unroll
    for (int u = 0; u < kNSt - 1; ++u) issue(kX, stage(u), u);
    wait_vm_lgkm0<(kNSt - 2) * kLoads>();   // tile 0 landed
    stage_barrier();
    int j0 = 0;
    for (; j0 + kNSt <= ntiles; j0 += kNSt) {
#pragma unroll
      for (int u = 0; u < kNSt; ++u) step(u, j0 + u);
    }
#pragma unroll
    for (int u = 0; u < kNSt; ++u)
      if (j0 + u < ntiles) step(u, j0 + u);
    wait_vm_lgkm0<0>();   // the clamped loads past the last tile land before the workgroup ends
  };
  if (G::kARem == 0 || wave < G::kARem) k_loop(std::true_type{});
  else k_loop(std::false_type{});

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
          static_cast<bf16_t *>(g.out)[mat_index(m, n, g.ldo, g.out_kmajor, g.m_alloc)] =
              f32_to_bf16(silu_bf16_epilogue(gt) * up);
        } else {
          const int n = n0 + wn * 16 * kNB + nb * 16 + (lane & 15);
          if (n >= g.n) continue;
          const float v = acc[mb][nb][i];
          if (EPI == kEpiPartial) {
            g.part[((size_t)split * g.m_store + m) * g.n + n] = v;
          } else if (EPI == kEpiStore) {
            static_cast<bf16_t *>(g.out)[(size_t)m * g.ldo + n] = f32_to_bf16(v);
          } else {  // kEpiGelu
            static_cast<bf16_t *>(g.out)[mat_index(m, n, g.ldo, g.out_kmajor, g.m_alloc)] =
                f32_to_bf16(gelu_f(v));
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

// k-tile-major repack of a weight: thread i moves the 16-byte piece i of the source (8 elements of
// one row, k fastest), so the reads are coalesced; the writes land as 16-byte pieces of the
// destination's w-element rows.
__global__ __launch_bounds__(256) void pack_kmajor(const bf16_t *__restrict__ src, int rows, int k, int ld,
                                                   int w, bf16_t *__restrict__ dst) {
  const int per_row = k / 8;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)rows * per_row) return;
  const int r = (int)(i / per_row), c = (int)(i % per_row) * 8;
  const uint4 v = *reinterpret_cast<const uint4 *>(src + (size_t)r * ld + c);
  *reinterpret_cast<uint4 *>(dst + ((size_t)(c / w) * rows + r) * w + c % w) = v;
}

template <int MB, int EPI, int BN>
hipError_t run_bf16_mb(const GemmArgs &g, const GemmPlan &p, hipStream_t s) {
  hipLaunchKernelGGL((gemm_bf16_rows<MB, EPI, BN>), dim3(p.grid), dim3(64 * kWaves), 0, s, g, p);
  return hipGetLastError();
}

// The kernel instance for the plan's 16-row blocks per wave row (1 .. kMBW).
template <int EPI, int MB = 1>
hipError_t run_bf16(const GemmArgs &g, const GemmPlan &p, hipStream_t s) {
  if constexpr (MB > kMBW) {
    return hipErrorInvalidValue;
  } else {
    if (p.wn != kPlanWaveCols) return hipErrorInvalidValue;
    if (p.mbw == MB) {
      if (p.bn == kBN) return run_bf16_mb<MB, EPI, kBN>(g, p, s);
      if constexpr (kWideTiles && MB >= (kMBWide + 1) / 2 && MB <= kMBWide) {
        if (p.bn == kBNWide) return run_bf16_mb<MB, EPI, kBNWide>(g, p, s);
      }
      return hipErrorInvalidValue;
    }
    return run_bf16<EPI, MB + 1>(g, p, s);
  }
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
  p.wn = kPlanWaveCols;
  p.bn = kBN;
  const int nk = k / kSplitK;
  // The split count and the epilogue form depend on the weight shape only, never on the number of
  // batch rows: a row's k-sum is then cut at the same points whatever else is in the batch, so a
  // decode run alone and the same decode inside a hybrid batch give bitwise-equal results.
  // Time model for one 256-row tile: whole rounds of `cus` workgroups, each k-tile at ~half of a
  // CU's MFMA rate, plus the float32 partials written and read back at ~5 TB/s.
  const double m_ref = 256.0;
  const double t_k = 2.0 * m_ref * kBN * kSplitK / 5.0e12;
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
  // Row tiles: as few 576-row tiles as hold the batch (then made wide, below).  (In a build with 64-deep stages for tiles of
  // up to 288 rows, those are the alternative, and the shorter estimate of whole rounds of `cus`
  // workgroups times one workgroup's time wins: a workgroup's time grows with its rows from its
  // weight stream, about 0.55 of a 288-row workgroup at 1 row, up to 1.0 at 288 rows with 64-deep
  // stages and 1.6 at 576 rows, measured on the llama-13b gate/up product with row-major weights.)
  // The rows of a batch never change its split count, so every choice gives a row the same k-sum.
  auto wg_time = [](int rows) {
    return stage_depth((rows + 31) / 32) == 64 ? 0.55 + 0.45 * rows / 288.0 : 0.55 + 0.525 * rows / 288.0;
  };
  auto plan_rows = [&](int tile_rows, int *m_tiles, int *mbw) {
    *m_tiles = (m + tile_rows - 1) / tile_rows;
    const int rows = (m + *m_tiles - 1) / *m_tiles;
    *mbw = (rows + 31) / 32;
    const int wgs = *m_tiles * p.n_tiles * p.splits;
    return (double)((wgs + cus - 1) / cus) * wg_time(rows);
  };
  int mt_tall, mb_tall, mt_short = 0, mb_short = 0;
  const double t_tall = plan_rows(kBMX, &mt_tall, &mb_tall);
  const double t_short = kMBW64 > 0 ? plan_rows(16 * kMBW64 * kWM, &mt_short, &mb_short) : 1e30;
  if (t_tall <= t_short) {
    p.m_tiles = mt_tall;
    p.mbw = mb_tall;
  } else {
    p.m_tiles = mt_short;
    p.mbw = mb_short;
  }
  // Wide tiles: row tiles of 289..576 rows, for a product width that is a whole number of
  // 256-column stripes (128 output columns of a fused gate|up tile), become twice as many row tiles
  // of at most 288 rows and twice the columns: the same workgroups, k-splits and k-sum order.
  const int tile_cols = p.epi == kEpiSwiGLU ? kBN / 2 : kBN;
  const int width = p.epi == kEpiPartial && epi == kEpiSwiGLU ? 2 * n_out : n_out;
  const int tile_rows = (m + p.m_tiles - 1) / p.m_tiles;
  if (kWideTiles && tile_rows > 16 * kMBWide * kWM && width % (2 * tile_cols) == 0) {
    p.bn = kBNWide;
    p.n_tiles /= 2;
    p.m_tiles *= 2;
    p.mbw = ((m + p.m_tiles - 1) / p.m_tiles + 31) / 32;
  }
  const int total = p.m_tiles * p.n_tiles * p.splits;
  p.per_xcd = (total + 7) / 8;
  p.grid = 8 * p.per_xcd;
  return p;
}

int plan_gemm_tail(int type, int epi, int m, int n_out, int k, int cus, GemmPlan *main, GemmPlan *tail) {
  if (type != kBF16 || (epi != kEpiSwiGLU && epi != kEpiGelu)) return 0;
  const GemmPlan whole = plan_gemm(type, epi, m, n_out, k, cus);
  // (counted in 128-column stripes: a wide tile covers two)
  if (whole.epi == kEpiPartial || whole.n_tiles * (whole.bn / kBN) <= cus) return 0;
  const int n_main = cus * (epi == kEpiSwiGLU ? kBN / 2 : kBN);
  if (n_main >= n_out) return 0;
  const GemmPlan mp = plan_gemm(type, epi, m, n_main, k, cus);
  if (mp.epi == kEpiPartial) return 0;
  const int n_tail = n_out - n_main;
  const GemmPlan tp = plan_gemm(type, kEpiPartial, m, epi == kEpiSwiGLU ? 2 * n_tail : n_tail, k, cus);
  // Both parts read the one input, k-tile-major at their (common) stage depth.
  if (stage_depth(tp.mbw) != stage_depth(mp.mbw)) return 0;
  *main = mp;
  *tail = tp;
  return n_main;
}

int gemm_stage_depth(const GemmPlan &p) { return stage_depth(p.mbw); }

hipError_t launch_pack_kmajor(const void *src, int rows, int k, int ld, int w, void *dst, hipStream_t s) {
  if (!src || !dst || rows <= 0 || k <= 0 || (w != 32 && w != 64) || k % w || ld < k || ld % 8 ||
      (long long)rows * k >= (1ll << 31))
    return hipErrorInvalidValue;
  const long long n = (long long)rows * (k / 8);
  hipLaunchKernelGGL(pack_kmajor, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     static_cast<const bf16_t *>(src), rows, k, ld, w, static_cast<bf16_t *>(dst));
  return hipGetLastError();
}

hipError_t launch_gemm(int type, int epi, const GemmArgs &g, const GemmPlan &p, hipStream_t s) {
  // k-tile-major A: bf16 only, tiles as wide as the plan's stage depth, and its whole extent
  // addressable with 32-bit offsets
  if (g.a_kmajor && (type == kF32 || g.a_kmajor != stage_depth(p.mbw) ||
                     (long long)g.m_alloc * g.k >= (1ll << 31)))
    return hipErrorInvalidValue;
  // k-tile-major weights: the same, with each k-tile step of either weight a 32-bit offset that
  // covers at least the product's rows taken from it
  if (g.w_kmajor) {
    const long long rows0 = g.w1 && epi != kEpiSwiGLU ? g.n_w0 : g.n;
    const long long rows1 = g.w1 ? (epi == kEpiSwiGLU ? g.n : g.n - g.n_w0) : 0;
    if (type == kF32 || g.w_kmajor != stage_depth(p.mbw) || g.w_slab0 < rows0 * g.w_kmajor ||
        (g.w1 && g.w_slab1 < rows1 * g.w_kmajor) || (long long)g.w_slab0 * (g.k / g.w_kmajor) >= (1ll << 31) ||
        (long long)g.w_slab1 * (g.k / g.w_kmajor) >= (1ll << 31))
      return hipErrorInvalidValue;
  }
  if (type == kBF16 && (g.k % kSplitK || p.mbw < 1 || p.mbw > kMBW)) return hipErrorInvalidValue;
  if (g.out_kmajor && (type == kF32 || (epi != kEpiSwiGLU && epi != kEpiGelu) ||
                       (g.out_kmajor != 32 && g.out_kmajor != 64) || g.n % g.out_kmajor))
    return hipErrorInvalidValue;
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
