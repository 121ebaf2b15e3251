// Shared device helpers for the CSA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ------------------------------------------------------ LDS transpose read

typedef short i16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 (gfx950).  Within each group of 16 lanes, with M[L]
// the four 16-bit values at lane L's address, lane j receives element e =
// M[4e + j/4][j % 4]: four lanes per row of 4 x 4 values come back
// transposed.  `p` must point into LDS and be 8-byte aligned.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<uint8_t*>(p)));
  return __builtin_bit_cast(u32x2, v);
}

// ------------------------------------------------- lane-group reductions

// Combine each lane's value with that of lane ^ 16 (resp. lane ^ 32) using
// the gfx950 VALU lane swaps instead of an LDS permute: with both operands
// set to x, the swap leaves every lane's own value in one result and its
// partner's in the other, so their sum (or max) is the same in both lanes
// of a pair.
__device__ __forceinline__ float sum_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// ---------------------------------------------------------------- bfloat16

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ----------------------------------------------------------------- fp8 e4m3

// fp32 -> OCP E4M3FN code, round to nearest even, saturating at 448.
__device__ __forceinline__ uint8_t f32_to_e4m3(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fabsf(v);
  uint32_t mag;
  if (a >= 448.0f) {
    mag = 0x7eu;  // every value >= 448 rounds (or saturates) to 448
  } else if (a < 0.015625f) {
    // subnormal range: value = f * 2^-9, f = 0..7; 2^-6 itself is code 8
    mag = static_cast<uint32_t>(rintf(a * 512.0f));
  } else {
    uint32_t u = __float_as_uint(a);
    u += 0x7ffffu + ((u >> 20) & 1u);  // round to 3 fraction bits, ties even
    uint32_t e = (u >> 23) - 127u + 7u;
    mag = (e << 3) | ((u >> 20) & 7u);
    if (mag > 0x7eu) mag = 0x7eu;
  }
  return static_cast<uint8_t>(sign | mag);
}

// max(x, 0) for finite x as one integer max on the bit pattern: negative
// floats (and -0.0) have the sign bit set, so they compare below integer 0
// and become +0.0; non-negative floats are unchanged.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// ----------------------------------------------------- range-checked stores

// Cache-policy operand of the raw buffer stores: sc1 makes a store
// device-scope, written through the XCD's L2 to memory.
constexpr int kCachePolicySc1 = 16;

// Raw buffer descriptor over [base, base + nbytes): stores at byte offsets
// >= nbytes are dropped by the hardware range check.  The caller passes
// wave-uniform values; they are moved to scalar registers explicitly so the
// descriptor is never treated as per-lane (a per-lane descriptor makes every
// store a loop over the distinct descriptors of the wave).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t store_rsrc(const void* base, int nbytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  void* up = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(up, 0, __builtin_amdgcn_readfirstlane(nbytes),
                                           0x00020000);
}

// ------------------------------------------------------- order-preserving key

// Map a finite float to a uint32 whose unsigned order is the float order;
// -0.0 and +0.0 map to the same key.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) return 0x80000000u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Smallest float whose score_key is >= key (inverse of score_key on the
// first key of a bucket).  Valid for keys of finite floats: 0x00800000
// (-FLT_MAX) .. 0xff800000 (+inf); 0x80000000 gives +0.0, which compares
// equal to -0.0 as the keys do.
__device__ __forceinline__ float key_floor_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// ---------------------------------------------------------- wave reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ------------------------------------------------------------- MFMA wrappers
//
// 16x16 output tiles.  In every flavour lane l holds column (l % 16) of B
// and row (l % 16) of A, and lane group g = l / 16 holds one quarter of the
// reduction (k) dimension; A and B lanes with the same (g, element) meet in
// the same product, so any consistent assignment of k to (g, element) gives
// the same sum.  The accumulator holds D[4*g + i][l % 16], i = 0..3.

__device__ __forceinline__ f32x4 mma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16x16x128 FP8 (E4M3 x E4M3), fp32 accumulate, unit block scales.
__device__ __forceinline__ f32x4 mma_fp8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Sequence index of query row `row` (row = b * T + i).  The row count is a
// grid dimension, so 32-bit arithmetic is exact; the result is moved to a
// scalar register (wave-uniform), so per-sequence loads go through the
// scalar cache and values derived from it stay scalar.
__device__ __forceinline__ int64_t seq_of_row(int64_t row, int64_t T) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<int>(static_cast<uint32_t>(row) / static_cast<uint32_t>(T)));
}

// Grids of `items` workgroups for each of `rows` rows whose workgroups share
// per-row data (a query row, a histogram, lists): the hardware hands
// consecutive workgroups to the 8 XCDs in turn, so with a 1-D grid of
// xcd_grid_size() workgroups, workgroup id goes to row id % 8 + 8 (id / 8 /
// items) and item id / 8 % items, which keeps all of a row's workgroups on
// one XCD and its shared data in one L2.  Used for rows >= 8 (xcd_mappable;
// with fewer rows, measured no better than the 2-D grid); xcd_row_item
// returns false for the padding workgroups.
constexpr int kXcds = 8;
inline bool xcd_mappable(int64_t rows) { return rows >= kXcds; }
inline int64_t xcd_grid_size(int64_t rows, int64_t items) {
  return kXcds * ((rows + kXcds - 1) / kXcds) * items;
}
__device__ __forceinline__ bool xcd_row_item(int64_t id, int items, int64_t rows, int64_t* row,
                                             int* item) {
  const int64_t k = id / kXcds;
  *row = (id % kXcds) + kXcds * (k / items);
  *item = static_cast<int>(k % items);
  return *row < rows;
}

// A wave-uniform 64-bit value moved to scalar registers (so loop bounds and
// addresses derived from it stay scalar).
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// MXFP4 x MXFP4: each lane's 16 bytes are the 32 E2M1 codes of one
// 32-element block of its row (A) or column (B), and byte 0 of sa / sb is
// that block's E8M0 scale.
__device__ __forceinline__ f32x4 mma_fp4(u32x4 a, u32x4 b, f32x4 c, uint32_t sa, uint32_t sb) {
  const i32x8 av = {static_cast<int>(a[0]), static_cast<int>(a[1]), static_cast<int>(a[2]),
                    static_cast<int>(a[3]), 0, 0, 0, 0};
  const i32x8 bv = {static_cast<int>(b[0]), static_cast<int>(b[1]), static_cast<int>(b[2]),
                    static_cast<int>(b[3]), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0,
                                                          static_cast<int>(sa), 0,
                                                          static_cast<int>(sb));
}

// ------------------------------------------------------------- compressor

template <typename T>
__device__ __forceinline__ float load_elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

constexpr int kCompressBatch = 8;

// The m tokens of one channel of a block with m <= NB, loaded together
// (indices clamped to the last token; the repeats are never used).
template <int NB, typename T>
__device__ __forceinline__ void compress_load(const T* x, const float* z, int64_t stride, int m,
                                              float (&zz)[NB], float (&xx)[NB]) {
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int64_t o = static_cast<int64_t>(min(j, m - 1)) * stride;
    zz[j] = z[o];
    xx[j] = load_elem<T>(x, o);
  }
}

// The entry value from loaded tokens (m <= NB): softmax over the m logits
// weights the m values, accumulated in token order.  The result does not
// depend on NB.
template <int NB>
__device__ __forceinline__ float compress_loaded(const float (&zz)[NB], const float (&xx)[NB],
                                                 int m) {
  float zmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < NB; ++j) zmax = fmaxf(zmax, zz[j]);  // repeats change nothing
  float num = 0.f, den = 0.f;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if (j < m) {
      const float a = expf(zz[j] - zmax);
      den += a;
      num = fmaf(a, xx[j], num);
    }
  }
  return num / den;
}

// One channel of one compressed entry: the softmax over the block's m
// tokens of their logits z weights the tokens' values x ("DeepSeek V4
// technical review", takeshell.com, section 2.1: each block of m tokens is
// aggregated into one entry).  x and z step by `stride` elements per
// token.  The compressor kernel and the decode indexer's fused block
// compression compute entries with these functions, so the two give the
// same bits.  Longer blocks are read in batches of kCompressBatch tokens
// (every load of a batch in flight at once), in the same arithmetic order.
template <typename T>
__device__ __forceinline__ float compress_channel(const T* x, const float* z, int64_t stride,
                                                  int m) {
  constexpr int kB = kCompressBatch;
  if (m <= kB) {
    float zz[kB], xx[kB];
    compress_load<kB>(x, z, stride, m, zz, xx);
    return compress_loaded<kB>(zz, xx, m);
  }
  float zmax = -INFINITY;
  for (int i0 = 0; i0 < m; i0 += kB) {
    float zz[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) zz[j] = z[static_cast<int64_t>(min(i0 + j, m - 1)) * stride];
#pragma unroll
    for (int j = 0; j < kB; ++j) zmax = fmaxf(zmax, zz[j]);
  }
  float num = 0.f, den = 0.f;
  for (int i0 = 0; i0 < m; i0 += kB) {
    float zz[kB], xx[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int64_t o = static_cast<int64_t>(min(i0 + j, m - 1)) * stride;
      zz[j] = z[o];
      xx[j] = load_elem<T>(x, o);
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      if (i0 + j < m) {
        const float a = expf(zz[j] - zmax);
        den += a;
        num = fmaf(a, xx[j], num);
      }
    }
  }
  return num / den;
}

__device__ __forceinline__ int64_t visible_entries(int64_t t, int m, int64_t n_cap) {
  int64_t v = (t + 1) / m;
  if (v < 0) v = 0;
  return v < n_cap ? v : n_cap;
}

}  // namespace csa
