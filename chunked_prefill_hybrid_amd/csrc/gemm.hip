// Fused linear ops of the hybrid batch: out = epilogue(a w^T) over the C+B concatenated rows.
//
// Every projection of the layer (QKV, O, gate/up, down) runs as ONE GEMM over the chunk rows and the
// decode rows together, so each weight tile crosses HBM once for the whole batch and the decodes
// share the chunk's weight fetches (SARATHI: Efficient LLM Inference by Piggybacking Decodes with
// Chunked Prefills, section 3, "Decode-Maximal Batching", "How fusion works").  The token dimension
// is padded only to the tile height; rows past C+B are never stored (the tile-quantization point of
// the same page, "Identifying the Ideal Chunk Size", Figure 7).
//
// bf16 path: v_mfma_f32_16x16x32_bf16, 4 waves per workgroup, A and W tiles staged through LDS with
// double buffering, BK = 64.  Workgroup b runs on XCD b % 8; the tiles of one weight stripe (all its
// row tiles) are given to workgroups of the same XCD so that the stripe's re-reads hit that XCD's L2.
// fp32 path: a plain FMA tile kernel (exact float32 products, used by the float32 layer mode).
#include <math.h>

#include "kernels.h"

namespace sarathi {
namespace {

constexpr int kBK = 64;         // k extent of one LDS stage (bf16 elements)
constexpr int kLdsK = kBK + 8;  // padded LDS row: 144 bytes keeps the 16-byte fragment reads spread

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }
__device__ __forceinline__ float gelu_f(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_mfma(GemmArgs g, int m_tiles, int n_tiles,
                                                       int n_per_xcd) {
  static_assert(WM * WN == 4, "four waves per workgroup");
  constexpr int WTM = BM / WM, WTN = BN / WN;       // wave tile
  constexpr int MB = WTM / 16, NB = WTN / 16;       // 16x16 MFMA blocks per wave
  constexpr bool kGlu = EPI == kEpiSwiGLU;
  static_assert(!kGlu || NB % 2 == 0, "SwiGLU pairs gate and up blocks inside a wave");
  constexpr int A_LD = BM * (kBK / 8) / 256, B_LD = BN * (kBK / 8) / 256;
  static_assert(A_LD * 256 == BM * (kBK / 8) && B_LD * 256 == BN * (kBK / 8), "whole 16-B loads");
  constexpr int kStage = (BM + BN) * kLdsK;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * kStage];

  // XCD-aware tile order: consecutive slots of one XCD walk the row tiles of one weight stripe.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int n_tile = xcd * n_per_xcd + slot / m_tiles;
  const int m_tile = slot % m_tiles;
  if (n_tile >= n_tiles) return;
  const int m0 = m_tile * BM;
  const int n0 = n_tile * (kGlu ? BN / 2 : BN);      // first output column of the tile

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const bf16_t *A = static_cast<const bf16_t *>(g.a);
  const bf16_t *W0 = static_cast<const bf16_t *>(g.w0);
  const bf16_t *W1 = static_cast<const bf16_t *>(g.w1);

  const bf16_t *a_src[A_LD];
  int a_dst[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int c = tid + i * 256, row = c >> 3, kc = c & 7;
    const int gr = min(m0 + row, g.m_alloc - 1);
    a_src[i] = A + (size_t)gr * g.lda + kc * 8;
    a_dst[i] = row * kLdsK + kc * 8;
  }
  const bf16_t *b_src[B_LD];
  int b_dst[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int c = tid + i * 256, row = c >> 3, kc = c & 7;
    int src_row;
    const bf16_t *Wp = W0;
    if (kGlu) {
      // LDS rows of wave wv: NB/2 gate blocks then the NB/2 up blocks of the same columns.
      const int wv = row / WTN, bb = (row % WTN) >> 4, rl = row & 15;
      const int cb = wv * (NB / 2) + bb % (NB / 2);
      src_row = n0 + cb * 16 + rl;
      Wp = (bb >= NB / 2) ? W1 : W0;
    } else {
      src_row = n0 + row;
    }
    src_row = min(src_row, g.n - 1);
    b_src[i] = Wp + (size_t)src_row * g.ldw + kc * 8;
    b_dst[i] = (BM + row) * kLdsK + kc * 8;
  }

  f32x4_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 ra[A_LD], rb[B_LD];
  const int nk = g.k / kBK;
#pragma unroll
  for (int i = 0; i < A_LD; ++i) ra[i] = ld16(a_src[i]);
#pragma unroll
  for (int i = 0; i < B_LD; ++i) rb[i] = ld16(b_src[i]);
#pragma unroll
  for (int i = 0; i < A_LD; ++i) st16(&lds[a_dst[i]], ra[i]);
#pragma unroll
  for (int i = 0; i < B_LD; ++i) st16(&lds[b_dst[i]], rb[i]);
  __syncthreads();

  const int frag_row = lane & 15, frag_k = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const bf16_t *L = lds + (kt & 1) * kStage;
    if (kt + 1 < nk) {
      const int ko = (kt + 1) * kBK;
#pragma unroll
      for (int i = 0; i < A_LD; ++i) ra[i] = ld16(a_src[i] + ko);
#pragma unroll
      for (int i = 0; i < B_LD; ++i) rb[i] = ld16(b_src[i] + ko);
    }
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      bf16x8_t af[MB], bw[NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        af[mb] = *reinterpret_cast<const bf16x8_t *>(
            &L[(wm * WTM + mb * 16 + frag_row) * kLdsK + ks * 32 + frag_k]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        bw[nb] = *reinterpret_cast<const bf16x8_t *>(
            &L[(BM + wn * WTN + nb * 16 + frag_row) * kLdsK + ks * 32 + frag_k]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb], bw[nb], acc[mb][nb], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      bf16_t *Ln = lds + ((kt + 1) & 1) * kStage;
#pragma unroll
      for (int i = 0; i < A_LD; ++i) st16(&Ln[a_dst[i]], ra[i]);
#pragma unroll
      for (int i = 0; i < B_LD; ++i) st16(&Ln[b_dst[i]], rb[i]);
    }
    __syncthreads();
  }

  // Epilogue.  Lane l of a 16x16 block holds rows 4*(l/16)+i, column l%16.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * WTM + mb * 16 + (lane >> 4) * 4 + i;
      if (m >= g.m_store) continue;
#pragma unroll
      for (int nb = 0; nb < (kGlu ? NB / 2 : NB); ++nb) {
        if (kGlu) {
          const int n = n0 + (wn * (NB / 2) + nb) * 16 + (lane & 15);
          if (n >= g.n) continue;
          const float gt = acc[mb][nb][i], up = acc[mb][nb + NB / 2][i];
          static_cast<bf16_t *>(g.out)[(size_t)m * g.ldo + n] = f32_to_bf16(silu_f(gt) * up);
        } else {
          const int n = n0 + wn * WTN + nb * 16 + (lane & 15);
          if (n >= g.n) continue;
          const float v = acc[mb][nb][i];
          if (EPI == kEpiStore) {
            static_cast<bf16_t *>(g.out)[(size_t)m * g.ldo + n] = f32_to_bf16(v);
          } else if (EPI == kEpiResidF32) {
            const float r = to_f32(static_cast<const bf16_t *>(g.resid)[(size_t)m * g.ldr + n]);
            static_cast<float *>(g.out)[(size_t)m * g.ldo + n] = v + r;
          } else if (EPI == kEpiResidOut) {
            const float r = static_cast<const float *>(g.resid)[(size_t)m * g.ldr + n];
            static_cast<bf16_t *>(g.out)[(size_t)m * g.ldo + n] = f32_to_bf16(v + r);
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
      float *o = static_cast<float *>(g.out) + (size_t)m * g.ldo + n;
      if (EPI == kEpiStore) *o = v;
      else if (EPI == kEpiResidF32 || EPI == kEpiResidOut)
        *o = v + static_cast<const float *>(g.resid)[(size_t)m * g.ldr + n];
      else if (EPI == kEpiSwiGLU) *o = silu_f(v) * acc2[i][j];
      else *o = gelu_f(v);
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI>
hipError_t run_bf16(const GemmArgs &g, hipStream_t s) {
  const int m_tiles = (g.m_store + BM - 1) / BM;
  const int cols_per_tile = EPI == kEpiSwiGLU ? BN / 2 : BN;
  const int n_tiles = (g.n + cols_per_tile - 1) / cols_per_tile;
  const int n_per_xcd = (n_tiles + 7) / 8;
  const int grid = 8 * n_per_xcd * m_tiles;
  hipLaunchKernelGGL((gemm_bf16_mfma<BM, BN, WM, WN, EPI>), dim3(grid), dim3(256), 0, s, g, m_tiles,
                     n_tiles, n_per_xcd);
  return hipGetLastError();
}

template <int EPI>
hipError_t dispatch_bf16(const GemmArgs &g, hipStream_t s) {
  if (g.m_store <= 32) return run_bf16<32, 128, 1, 4, EPI>(g, s);
  return run_bf16<64, 128, 2, 2, EPI>(g, s);
}

template <int EPI>
hipError_t run_f32(const GemmArgs &g, hipStream_t s) {
  dim3 grid((g.n + 63) / 64, (g.m_store + 63) / 64);
  hipLaunchKernelGGL(gemm_f32_fma<EPI>, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

GemmPlan plan_gemm(int type, int epi, int m, int n, int /*k*/) {
  GemmPlan p{};
  if (type == kF32) {
    p.bm = 64; p.bn = 64;
    p.m_tiles = (m + 63) / 64; p.n_tiles = (n + 63) / 64;
    p.grid = p.m_tiles * p.n_tiles;
    return p;
  }
  p.bm = m <= 32 ? 32 : 64;
  p.bn = 128;
  const int cols = epi == kEpiSwiGLU ? p.bn / 2 : p.bn;
  p.m_tiles = (m + p.bm - 1) / p.bm;
  p.n_tiles = (n + cols - 1) / cols;
  p.grid = 8 * ((p.n_tiles + 7) / 8) * p.m_tiles;
  return p;
}

hipError_t launch_gemm(int type, int epi, const GemmArgs &g, hipStream_t s) {
  if (type == kF32) {
    switch (epi) {
      case kEpiStore: return run_f32<kEpiStore>(g, s);
      case kEpiResidF32: return run_f32<kEpiResidF32>(g, s);
      case kEpiResidOut: return run_f32<kEpiResidOut>(g, s);
      case kEpiSwiGLU: return run_f32<kEpiSwiGLU>(g, s);
      case kEpiGelu: return run_f32<kEpiGelu>(g, s);
    }
  } else {
    switch (epi) {
      case kEpiStore: return dispatch_bf16<kEpiStore>(g, s);
      case kEpiResidF32: return dispatch_bf16<kEpiResidF32>(g, s);
      case kEpiResidOut: return dispatch_bf16<kEpiResidOut>(g, s);
      case kEpiSwiGLU: return dispatch_bf16<kEpiSwiGLU>(g, s);
      case kEpiGelu: return dispatch_bf16<kEpiGelu>(g, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace sarathi
