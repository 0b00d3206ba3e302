// Device helpers shared by the gfx950 kernels: bfloat16 storage, 16-byte packets, wave64 reductions,
// MFMA operand types, and the per-launch request descriptors passed by value as kernel arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sarathi {

typedef uint16_t bf16_t;  // bfloat16 storage (upper half of an IEEE float32)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// float32 -> bfloat16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// A 16-byte packet of storage elements: 4 floats or 8 bfloat16.
template <typename T> struct Packet { static constexpr int E = 16 / (int)sizeof(T); };

template <typename T> __device__ __forceinline__ void unpack(const uint4 &v, float *out);
template <> __device__ __forceinline__ void unpack<float>(const uint4 &v, float *out) {
  out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
}
template <> __device__ __forceinline__ void unpack<bf16_t>(const uint4 &v, float *out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <typename T> __device__ __forceinline__ uint4 pack(const float *in);
template <> __device__ __forceinline__ uint4 pack<float>(const float *in) {
  return make_uint4(__float_as_uint(in[0]), __float_as_uint(in[1]), __float_as_uint(in[2]),
                    __float_as_uint(in[3]));
}
template <> __device__ __forceinline__ uint4 pack<bf16_t>(const float *in) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)f32_to_bf16(in[2 * i]) | ((uint32_t)f32_to_bf16(in[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st16(void *p, const uint4 &v) { *reinterpret_cast<uint4 *>(p) = v; }

// ---------------------------------------------------------------------------------------------
// Global -> LDS streaming (gfx950 LDS DMA), shared by the GEMM and the chunk attention kernels.
// A kernel keeps several LDS stages, one __shared__ array each (the compiler then knows a read of one
// stage does not depend on loads still landing in another), issues the loads of a later tile,
// computes the current one, waits for its own loads of the next tile and meets the other waves.

// global -> LDS, 16 bytes per lane: lane l writes bytes [16 l, 16 l + 16) after the wave-uniform LDS
// address `lds`.
__device__ __forceinline__ void dma16(const bf16_t *src, bf16_t *lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}
// Global-memory view of a pointer.  Request descriptors carry cache pointers as integers, so the
// compiler cannot tell which memory they point to and would emit flat_* accesses through them; a
// flat access also counts against the LDS wait counter and checks the address space per lane.
// Accesses through this view compile to global_* instructions.
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T *as_global(T *p) {
  return (__attribute__((address_space(1))) T *)p;
}

// 16-byte load of data read once per forward (KV caches in decode attention): non-temporal, which
// streams from HBM measurably faster (6.3 vs 5.6 TB/s in a plain read) than loads that allocate in
// the caches.
__device__ __forceinline__ uint4 ld16_stream(const void *p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(as_global(reinterpret_cast<const u32x4 *>(p)));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Wait until at most N of this wave's global loads are outstanding and all its LDS operations are
// done (s_waitcnt with vmcnt = N, lgkmcnt = 0, expcnt left open).
template <int N> __device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// Workgroup barrier without a memory fence (a fence would also wait for the loads still in flight
// into the other stages); the empty asm statements keep the compiler from moving memory accesses
// across it.  Visibility of the LDS stage that the next step reads comes from the explicit wait that
// precedes each barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Element (r, c) of a [rows, cols] matrix stored row-major (kw = 0, row stride ld) or k-tile-major,
// [cols / kw][rows_alloc][kw] with kw = 32 or 64 (the layout a GEMM with kw-deep LDS stages reads as
// contiguous blocks).
__host__ __device__ __forceinline__ size_t mat_index(int r, int c, int ld, int kw, int rows_alloc) {
  return kw ? ((size_t)(c / kw) * rows_alloc + r) * kw + (c % kw) : (size_t)r * ld + c;
}

// Where a kernel writes element (r, c) of its [rows, cols] output: row-major with row stride ld
// (kw = 0), or k-tile-major over rows_alloc rows (kw = 32 or 64), as mat_index.
struct OutLayout {
  int ld, kw, rows_alloc;
};
__host__ __device__ __forceinline__ size_t out_index(const OutLayout &o, int r, int c) {
  return mat_index(r, c, o.ld, o.kw, o.rows_alloc);
}

// This lane's value and that of lane l ^ 32 (swap32) or l ^ 16 (swap16), through gfx950's permlane
// swaps: VALU instructions, where a shuffle through ds_bpermute takes an LDS round trip.  The pair
// comes back in a lane-dependent order (measured with an in-bounds probe: with both operands v,
// permlane32_swap gives lanes 0..31 (v[l], v[l + 32]) and lanes 32..63 (v[l - 32], v[l]);
// permlane16_swap gives the even 16-lane rows (v[l], v[l + 16]) and the odd ones (v[l - 16], v[l])),
// so only commutative merges use them: the sum or maximum is then the same as own op partner.
struct LanePair {
  float a, b;
};
__device__ __forceinline__ LanePair swap32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(p[0]), __uint_as_float(p[1])};
}
__device__ __forceinline__ LanePair swap16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(p[0]), __uint_as_float(p[1])};
}
__device__ __forceinline__ float sum_xor(float v, int m) {
  if (m == 32) { const LanePair p = swap32(v); return p.a + p.b; }
  if (m == 16) { const LanePair p = swap16(v); return p.a + p.b; }
  return v + __shfl_xor(v, m, kWave);
}
__device__ __forceinline__ float max_xor(float v, int m) {
  if (m == 32) { const LanePair p = swap32(v); return fmaxf(p.a, p.b); }
  if (m == 16) { const LanePair p = swap16(v); return fmaxf(p.a, p.b); }
  return fmaxf(v, __shfl_xor(v, m, kWave));
}

// Butterfly reductions over the lanes whose index differs only in the bits of [from, 32].
__device__ __forceinline__ float wave_sum(float v, int from = 1) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1)
    if (m >= from) v = sum_xor(v, m);
  return v;
}
__device__ __forceinline__ float wave_max(float v, int from = 1) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1)
    if (m >= from) v = max_xor(v, m);
  return v;
}

// Request descriptors, passed by value as kernel arguments.  A launch covers rows
// [row0, row0 + n_rows) of the batch.  The batch's prefill chunks come first, in chunk order: chunk j
// owns rows [row0[j], row0[j] + len[j]) at positions off[j] .. off[j] + len[j] - 1 of its request;
// `rows` is the number of chunk rows.  Batch row rows + i is decode i, which must lie in
// [dec.base, dec.base + dec.n).
constexpr int kMaxDecodesPerLaunch = 64;
constexpr int kMaxChunks = 16;

struct ChunkSet {
  uint64_t k[kMaxChunks], v[kMaxChunks];   // device [nh, cap, d] each
  int32_t cap[kMaxChunks];
  int32_t len[kMaxChunks];                 // chunk rows (>= 1)
  int32_t off[kMaxChunks];                 // entries already cached = position of the first row
  int32_t row0[kMaxChunks];                // first batch row
  int32_t split[kMaxChunks];               // key-range splits of the chunk's query blocks (>= 1)
  int32_t n, rows;                         // chunks; total chunk rows
  int32_t qblocks;                         // chunk kernel: 16-query blocks per wave (1 or 2)
};

struct DecodeGroup {
  uint64_t k[kMaxDecodesPerLaunch];
  uint64_t v[kMaxDecodesPerLaunch];
  int32_t len[kMaxDecodesPerLaunch];   // cached entries before this step = the new token's slot
  int32_t cap[kMaxDecodesPerLaunch];
  int32_t n, base;                      // decodes base .. base+n-1 of the batch
};

// Paged KV caches: every request's K (and V) rows live in fixed-size pages of one pool per layer,
// each pool [n_pages, nh, page_size, d] (a (page, head) slab of page_size rows is contiguous), and the
// request's block table maps its logical page i (tokens i*page_size ...) to a pool page.  With a pool,
// the k field of a request descriptor holds its block table (device int32 [cap / page_size]) and cap
// is the request's capacity in tokens.  Table entries are clamped into [0, n_pages) before use, so a
// bad entry can give wrong values but never an access outside the pool.
struct PagePool {
  uint64_t k, v;        // device pools (0: the requests use contiguous caches)
  int32_t n_pages;
  int32_t shift;        // page_size = 1 << shift
};

__device__ __forceinline__ int pool_page(const int32_t *table, int entry, int n_pages) {
  return min(max(as_global(table)[entry], 0), n_pages - 1);
}

// Element offset of (head h, key j) in a paged pool, given key j's pool page.
__device__ __forceinline__ size_t paged_off(int page, int h, int j, int nh, int shift, int d) {
  return (((size_t)page * nh + h) << shift | (size_t)(j & ((1 << shift) - 1))) * d;
}

// Position, cache and key count of batch row r (keys 0..pos are attended; pos is the write slot).
struct RowRef {
  uint64_t k, v;
  int32_t cap, pos;
};

// Position, cache and key count of batch row r.  The chunk table is read at constant indices only
// (a select per entry), which keeps the argument block out of per-lane scratch memory.
// kChunkRows = false: the launch covers decode rows only, and the chunk table is never read.
template <bool kChunkRows = true>
__device__ __forceinline__ RowRef row_ref(int r, const ChunkSet &cs, const DecodeGroup &dg) {
  RowRef rr;
  if (kChunkRows && r < cs.rows) {
    uint64_t k = cs.k[0], v = cs.v[0];
    int cap = cs.cap[0], pos = cs.off[0] + r;
#pragma unroll
    for (int i = 1; i < kMaxChunks; ++i)
      if (i < cs.n && r >= cs.row0[i]) {
        k = cs.k[i]; v = cs.v[i]; cap = cs.cap[i]; pos = cs.off[i] + (r - cs.row0[i]);
      }
    rr.k = k; rr.v = v; rr.cap = cap; rr.pos = pos;
  } else {
    const int i = r - cs.rows - dg.base;
    rr.k = dg.k[i]; rr.v = dg.v[i]; rr.cap = dg.cap[i]; rr.pos = dg.len[i];
  }
  return rr;
}

}  // namespace sarathi
