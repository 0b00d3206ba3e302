// Causal attention of a prefill chunk over its request's cached prefix plus itself (bf16, MFMA).
//
// Chunk query t sits at absolute position off+t and attends to keys 0..off+t: the whole cached
// prefix and the causal part of its own chunk, whose K/V rows were appended to the same cache just
// before (SARATHI: Efficient LLM Inference by Piggybacking Decodes with Chunked Prefills, section 3,
// "Chunked-Prefills", attention mask construction and Figure 6).  The prefix is re-read from HBM by
// every chunk of the request, the overhead the same page discusses under "Overhead 2".
//
// Flash-style design for gfx950.  A workgroup takes one head and 64 queries (16 per wave) and streams
// the request's keys in tiles of 64 through LDS with double buffering.  Per wave and tile:
//   S^T = K Q^T   (16 x v_mfma_f32_16x16x32_bf16 for d = 128): lane l then holds the scores of query
//                 l % 16 for 16 of the tile's keys, so a query's row max / sum need only in-lane work
//                 and two butterfly steps;
//   online softmax in float32 (log2 domain, scale folded into the exponent);
//   O^T += V^T P^T (16 more MFMAs): P^T is taken straight from the S^T registers (the MFMA's k order
//                 is the same free permutation of the 32 keys on both operands), V^T comes from a
//                 transposed copy of the V tile in LDS.
// Only tiles that cross the diagonal are masked.  Keys at or past the chunk's end are zero-filled in
// LDS (never loaded), so a masked probability of 0 never meets an unwritten cache slot.
#include <math.h>

#include "kernels.h"

namespace sarathi {
namespace {

constexpr int kBQ = 64;         // queries per workgroup (16 per wave)
constexpr int kBKV = 64;        // keys per tile
constexpr int kKPad = 8;        // K tile row padding (elements)
constexpr int kVtPad = 4;       // transposed V tile row padding (elements)

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const bf16_t gbf16_t;   // global memory

// 2^x for x <= 0 with the hardware exponential alone: results below the normal range flush to 0,
// which is what a probability that small contributes anyway.
__device__ __forceinline__ float exp2_nonpos(float x) { return __builtin_amdgcn_exp2f(x); }

// Split s of S covers key tiles [s nt / S, (s + 1) nt / S) of the workgroup's nt tiles.  With S = 1 the
// workgroup writes the normalised output; otherwise it writes its split partial (running max m and
// sum l in the log2 domain, unnormalised output) at ((row * nh + h) * stride + s), for the combine
// kernel to merge.
template <int D>
__global__ __launch_bounds__(256) void attn_chunk_mfma(const bf16_t *q, int ld_q, int nh,
                                                       ChunkRef ch, bf16_t *out, int ld_out,
                                                       float qscale_log2, int n_split, int stride,
                                                       float *part_o, float *part_ml) {
  constexpr int KS = D / 32;             // k-steps of the score MFMA
  constexpr int DB = D / 16;             // 16-row blocks of O^T
  constexpr int kKRow = D + kKPad;       // K tile LDS row (keys x d)
  constexpr int kVtRow = kBKV + kVtPad;  // V^T tile LDS row (d x keys)
  constexpr int kStage = kBKV * kKRow + D * kVtRow;
  extern __shared__ __attribute__((aligned(16))) bf16_t lds[];   // 2 * kStage elements

  const int qb = blockIdx.x, h = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int C = ch.len, off = ch.off;
  const int q_first = qb * kBQ;
  const int q_last = min(C, q_first + kBQ) - 1;          // last query of the workgroup
  const int n_keys = off + q_last + 1;                    // keys any of its queries sees
  const int nt = (n_keys + kBKV - 1) / kBKV;
  const int t_begin = (int)((long long)split * nt / n_split);
  const int t_end = (int)((long long)(split + 1) * nt / n_split);
  gbf16_t *Kh = reinterpret_cast<gbf16_t *>(ch.k) + (size_t)h * ch.cap * D;
  gbf16_t *Vh = reinterpret_cast<gbf16_t *>(ch.v) + (size_t)h * ch.cap * D;
  auto gld16 = [](gbf16_t *p) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = *reinterpret_cast<const __attribute__((address_space(1))) u32x4 *>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
  };

  // This lane's query (row of the wave's 16) and its fragments of q (B operand of S^T = K Q^T).
  const int my_q = q_first + wave * 16 + c16;
  const int my_pos = off + min(my_q, C - 1);
  bf16x8_t qf[KS];
  {
    const bf16_t *qr = q + (size_t)min(my_q, C - 1) * ld_q + h * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8_t *>(qr + ks * 32 + g * 8);
  }

  // Tile loads: K as [key][d] rows of 16-byte chunks; V as key pairs x 16 d, written transposed.
  constexpr int K_CH = kBKV * D / 8 / 256;                // 16-byte K chunks per thread
  uint4 rk[K_CH], rv[4];
  auto load_tile = [&](int t) {
    const int k0 = t * kBKV;
#pragma unroll
    for (int i = 0; i < K_CH; ++i) {
      const int c = tid + i * 256, key = c / (D / 8), dc = c % (D / 8);
      const int kg = k0 + key;
      rk[i] = kg < n_keys ? gld16(Kh + (size_t)kg * D + dc * 8) : make_uint4(0, 0, 0, 0);
    }
    // V: thread -> key pair kp (32 pairs) x d chunk of 16 (D/16 chunks); 256 threads cover it when
    // D == 128; for D == 64 each thread takes half as many d.
    const int kp = tid & 31, dch = tid >> 5;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kg = k0 + 2 * kp + j;
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const int d0 = (D == 128 ? dch * 16 : (dch >> 1) * 16) + hlf * 8;
        const bool use = (D == 128 || (dch & 1) == hlf) && kg < n_keys;
        rv[j * 2 + hlf] = use ? gld16(Vh + (size_t)kg * D + d0) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int stage) {
    bf16_t *Ks = lds + stage * kStage;
    bf16_t *Vt = Ks + kBKV * kKRow;
#pragma unroll
    for (int i = 0; i < K_CH; ++i) {
      const int c = tid + i * 256, key = c / (D / 8), dc = c % (D / 8);
      st16(&Ks[key * kKRow + dc * 8], rk[i]);
    }
    const int kp = tid & 31, dch = tid >> 5;
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf) {
      if (D == 64 && (dch & 1) != hlf) continue;
      const int d0 = (D == 128 ? dch * 16 : (dch >> 1) * 16) + hlf * 8;
      const uint4 a = rv[hlf], b = rv[2 + hlf];          // keys 2kp and 2kp+1, d0..d0+7
      const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (wa[e] & 0xffffu) | (wb[e] << 16);          // d0+2e   : keys 2kp, 2kp+1
        const uint32_t hi = (wa[e] >> 16) | (wb[e] & 0xffff0000u);      // d0+2e+1
        *reinterpret_cast<uint32_t *>(&Vt[(d0 + 2 * e) * kVtRow + 2 * kp]) = lo;
        *reinterpret_cast<uint32_t *>(&Vt[(d0 + 2 * e + 1) * kVtRow + 2 * kp]) = hi;
      }
    }
  };

  f32x4_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  if (t_begin < t_end) {   // workgroup-uniform
    load_tile(t_begin);
    store_tile(0);
  }
  __syncthreads();
  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const bf16_t *Ks = lds + buf * kStage;
    const bf16_t *Vt = Ks + kBKV * kKRow;
    if (t + 1 < t_end) load_tile(t + 1);

    // S^T for the tile: 4 key blocks of 16.
    f32x4_t sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t *>(
            &Ks[(kb * 16 + c16) * kKRow + ks * 32 + g * 8]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], sacc[kb], 0, 0, 0);
      }
    }
    // Scores in the log2 domain, masked past each query's position (and past the chunk's keys);
    // only tiles that reach past the wave's first query need the mask (a wave-uniform test).
    const int k0 = t * kBKV;
    const bool diag = k0 + kBKV - 1 > off + q_first + wave * 16;
    float sc[4][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[kb][i] = sacc[kb][i] * qscale_log2;
    if (diag) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (k0 + kb * 16 + g * 4 + i > my_pos) sc[kb][i] = -INFINITY;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sc[kb][i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    // A split that starts past a query's position leaves its row fully masked (m_new = -inf): then
    // the exponent base is 0, every p is 0 and the row's partial stays empty (l = 0).
    const float m_new = fmaxf(m_run, tmax);
    const float m_base = m_new == -INFINITY ? 0.f : m_new;
    // Rescale the running sums only when some query of the wave found a larger maximum (after the
    // first tiles this is rare); otherwise the factor is exactly 1 for every lane.
    if (__any(m_new > m_run)) {
      const float corr = exp2_nonpos(m_run - m_base);
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= corr;
    }
    m_run = m_new;
    // P^T operands: k-step s covers key blocks 2s and 2s+1.
    bf16x8_t pf[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2_nonpos(sc[2 * s + hb][i] - m_base);
          l_run += p;
          pf[s][hb * 4 + i] = (__bf16)p;
        }
    }
    // O^T += V^T P^T.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16_t *vr = &Vt[(db * 16 + c16) * kVtRow + s * 32 + g * 4];
        const bf16x4_t lo = *reinterpret_cast<const bf16x4_t *>(vr);
        const bf16x4_t hi = *reinterpret_cast<const bf16x4_t *>(vr + 16);
        const bf16x8_t vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[s], o[db], 0, 0, 0);
      }
    }
    if (t + 1 < t_end) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Row sums over the four lane groups of the query, then O[q][d] = O^T[d][q] / l.
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  if (n_split > 1) {
    if (my_q < C) {
      const size_t pidx = ((size_t)my_q * nh + h) * stride + split;
      if (g == 0) {
        part_ml[2 * pidx] = m_run;
        part_ml[2 * pidx + 1] = l_run;
      }
      float *po = part_o + pidx * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<float4 *>(&po[db * 16 + g * 4]) = make_float4(o[db][0], o[db][1], o[db][2], o[db][3]);
    }
  } else if (my_q < C) {
    const float inv = 1.0f / l_run;
    bf16_t *orow = out + (size_t)my_q * ld_out + h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      uint2 u;
      u.x = (uint32_t)f32_to_bf16(o[db][0] * inv) | ((uint32_t)f32_to_bf16(o[db][1] * inv) << 16);
      u.y = (uint32_t)f32_to_bf16(o[db][2] * inv) | ((uint32_t)f32_to_bf16(o[db][3] * inv) << 16);
      *reinterpret_cast<uint2 *>(&orow[db * 16 + g * 4]) = u;
    }
  }
}

template <int D>
hipError_t run_chunk(const void *q, int ld_q, int nh, const ChunkRef &ch, void *out, int ld_out,
                     int n_split, int stride, float *part_o, float *part_ml, hipStream_t s) {
  constexpr size_t bytes = 2 * sizeof(bf16_t) * ((size_t)kBKV * (D + kKPad) + (size_t)D * (kBKV + kVtPad));
  static bool attr_set = false;   // one LDS opt-in per instantiation (host-side, idempotent)
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_chunk_mfma<D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const dim3 grid((ch.len + kBQ - 1) / kBQ, nh, n_split);
  const float qscale = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL(attn_chunk_mfma<D>, grid, dim3(256), bytes, s, static_cast<const bf16_t *>(q),
                     ld_q, nh, ch, static_cast<bf16_t *>(out), ld_out, qscale, n_split, stride,
                     part_o, part_ml);
  return hipGetLastError();
}

}  // namespace

int chunk_attn_splits(int chunk_len, int chunk_offset, int nh) {
  if (chunk_len <= 0) return 1;
  const int q_blocks = (chunk_len + kBQ - 1) / kBQ;
  const int min_tiles = (chunk_offset + min(chunk_len, kBQ) + kBKV - 1) / kBKV;   // first block's
  const int want = (kChunkTargetWorkgroups + q_blocks * nh - 1) / (q_blocks * nh);
  return max(1, min(min(want, kMaxChunkSplits), max(min_tiles, 1)));
}

hipError_t launch_attn_chunk(int d, const void *q, int ld_q, int nh, const ChunkRef &ch, void *out,
                             int ld_out, int n_split, int stride, float *part_o, float *part_ml,
                             hipStream_t s) {
  if (ch.len <= 0) return hipSuccess;
  if (n_split < 1 || n_split > stride || (n_split > 1 && (!part_o || !part_ml)))
    return hipErrorInvalidValue;
  if (d == 128) return run_chunk<128>(q, ld_q, nh, ch, out, ld_out, n_split, stride, part_o, part_ml, s);
  if (d == 64) return run_chunk<64>(q, ld_q, nh, ch, out, ld_out, n_split, stride, part_o, part_ml, s);
  return hipErrorInvalidValue;
}

}  // namespace sarathi
