// Token-level compressor and FP8 row quantizer.
//
// Compressor: every m tokens of K (or V) become one cache entry, a weighted
// aggregation over the block ("DeepSeek V4 technical review", takeshell.com,
// section 2.1 CSA; octagono.org "Hybrid Attention: CSA and HCA" calls it a
// learned token-level compressor).  The weights are a softmax over the m
// tokens of caller-supplied logits, independently per channel.
//
// Layout: one thread per (entry, channel).  Consecutive lanes take
// consecutive channels, so every token row of x and of the logits is read
// with fully coalesced loads; the m-token loop is the only serial part.
#include "common.h"
#include "kernels.h"

namespace csa {

template <typename T>
__device__ __forceinline__ void store_elem(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_elem<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t* p, int64_t i, float v) {
  p[i] = f32_to_bf16(v);
}

template <typename T>
__global__ __launch_bounds__(256) void compress_kernel(
    const T* __restrict__ x, const float* __restrict__ z, T* __restrict__ cache,
    int64_t n_blocks, int64_t d, int m, int64_t x_sb, int64_t z_sb, int64_t n_cap,
    int64_t first_entry) {
  const int64_t b = blockIdx.y;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= n_blocks * d) return;
  const int64_t j = e / d;
  const int64_t c = e - j * d;
  const T* xb = x + b * x_sb + (j * m) * d + c;
  const float* zb = z + b * z_sb + (j * m) * d + c;
  store_elem<T>(cache, b * n_cap * d + (first_entry + j) * d + c, compress_channel(xb, zb, d, m));
}

// Gradients of the compressor for one (block, channel) per thread: with
// w_i = softmax_i(z) and c = sum_i w_i x_i (the forward's arithmetic),
// dx_i = w_i dc and dz_i = w_i (x_i - c) dc.
template <typename T>
__global__ __launch_bounds__(256) void compress_bwd_kernel(
    const T* __restrict__ x, const float* __restrict__ z, const float* __restrict__ dc,
    float* __restrict__ dx, float* __restrict__ dz, int64_t n_blocks, int64_t d, int m,
    int64_t x_sb, int64_t z_sb) {
  const int64_t b = blockIdx.y;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= n_blocks * d) return;
  const int64_t j = e / d;
  const int64_t ch = e - j * d;
  const T* xb = x + b * x_sb + (j * m) * d + ch;
  const float* zb = z + b * z_sb + (j * m) * d + ch;
  const float c = compress_channel(xb, zb, d, m);
  float zmax = -INFINITY;
  for (int i = 0; i < m; ++i) zmax = fmaxf(zmax, zb[static_cast<int64_t>(i) * d]);
  float den = 0.f;
  for (int i = 0; i < m; ++i) den += expf(zb[static_cast<int64_t>(i) * d] - zmax);
  const float g = dc[(b * n_blocks + j) * d + ch];
  const int64_t o = b * n_blocks * m * d + (j * m) * d + ch;
  for (int i = 0; i < m; ++i) {
    const int64_t off = static_cast<int64_t>(i) * d;
    const float w = expf(zb[off] - zmax) / den;
    dx[o + off] = w * g;
    dz[o + off] = w * (load_elem<T>(xb, off) - c) * g;
  }
}

int launch_compress_bwd(const void* x, int dtype, const float* z, const float* dc, int64_t B,
                        int64_t n_tok, int64_t d, int m, int64_t x_sb, int64_t z_sb, float* dx,
                        float* dz, hipStream_t s) {
  const int64_t nb = n_tok / m;
  dim3 grid(static_cast<unsigned>((nb * d + 255) / 256), static_cast<unsigned>(B));
  if (dtype == 0)
    launch_kernel(compress_bwd_kernel<float>, grid, 256, s, static_cast<const float*>(x), z, dc, dx, dz,
                                                    nb, d, m, x_sb, z_sb);
  else
    launch_kernel(compress_bwd_kernel<uint16_t>, grid, 256, s, static_cast<const uint16_t*>(x), z, dc,
                                                       dx, dz, nb, d, m, x_sb, z_sb);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_compress(const void* x, int dtype, const float* z, int64_t B, int64_t n_tok,
                    int64_t d, int m, int64_t x_sb, int64_t z_sb, void* cache,
                    int64_t n_cap, int64_t first_entry, hipStream_t s) {
  const int64_t nb = n_tok / m;
  const int64_t total = nb * d;
  dim3 grid(static_cast<unsigned>((total + 255) / 256), static_cast<unsigned>(B));
  if (dtype == 0) {
    launch_kernel(compress_kernel<float>, grid, 256, s, static_cast<const float*>(x), z,
                                                static_cast<float*>(cache), nb, d, m, x_sb,
                                                z_sb, n_cap, first_entry);
  } else {
    launch_kernel(compress_kernel<uint16_t>, grid, 256, s, static_cast<const uint16_t*>(x), z,
                                                   static_cast<uint16_t*>(cache), nb, d, m,
                                                   x_sb, z_sb, n_cap, first_entry);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// FP8 row quantizer: one wave per row.  scale = amax / 448 and the code
// quotient x / scale are correctly rounded fp32 divisions (the default HIP
// division), then rounded to E4M3 (nearest even, saturating).
template <typename T>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const T* __restrict__ x,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales,
                                                            int64_t rows, int d) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const T* xr = x + r * d;
  float amax = 0.f;
  for (int c = lane; c < d; c += 64) amax = fmaxf(amax, fabsf(load_elem<T>(xr, c)));
  amax = wave_max(amax);
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
  for (int c = lane; c < d; c += 64) codes[r * d + c] = f32_to_e4m3(load_elem<T>(xr, c) / scale);
  if (lane == 0) scales[r] = scale;
}

// MXFP4 row quantizer (OCP MX: E2M1 elements, one E8M0 scale per block of
// 32): one wave per row, lane l taking elements 2l and 2l+1 of each group of
// 128 (one output byte; a block is 16 lanes).  Block scale exponent
// s = floor(log2 amax) - 2 (clamped to [-127, 127]; code 0 for a zero
// block); element code = E2M1 rounding of x * 2^-s (exact), nearest with
// ties to even and saturation at 6, as a sum of threshold tests; the sign
// bit is the sign of x.
__device__ __forceinline__ uint32_t f32_to_e2m1(float v) {
  const float a = fabsf(v);
  const uint32_t mag = (a > 0.25f ? 1u : 0u) + (a >= 0.75f ? 1u : 0u) + (a > 1.25f ? 1u : 0u) +
                       (a >= 1.75f ? 1u : 0u) + (a > 2.5f ? 1u : 0u) + (a >= 3.5f ? 1u : 0u) +
                       (a > 5.0f ? 1u : 0u);
  return mag | ((__float_as_uint(v) >> 28) & 8u);
}

template <typename T>
__global__ __launch_bounds__(256) void quantize_mxfp4_rows_kernel(const T* __restrict__ x,
                                                                  uint8_t* __restrict__ codes,
                                                                  uint8_t* __restrict__ scales,
                                                                  int64_t rows, int d) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const T* xr = x + r * d;
  for (int c0 = 0; c0 < d; c0 += 128) {
    const int c = c0 + 2 * lane;
    const bool live = c < d;  // d % 32 == 0: whole 16-lane blocks are live or not
    const float x0 = live ? load_elem<T>(xr, c) : 0.f;
    const float x1 = live ? load_elem<T>(xr, c + 1) : 0.f;
    float a = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
    int s = -127;
    if (a > 0.f) {
      s = __builtin_amdgcn_frexp_expf(a) - 1 - 2;  // a = f * 2^e, f in [0.5, 1)
      s = s < -127 ? -127 : (s > 127 ? 127 : s);
    }
    const uint32_t q = f32_to_e2m1(ldexpf(x0, -s)) | (f32_to_e2m1(ldexpf(x1, -s)) << 4);
    if (live) {
      codes[r * (d / 2) + c / 2] = static_cast<uint8_t>(q);
      if ((lane & 15) == 0) scales[r * (d / 32) + c / 32] = static_cast<uint8_t>(a > 0.f ? s + 127 : 0);
    }
  }
}

int launch_quantize_mxfp4_rows(const void* x, int dtype, int64_t rows, int64_t d, uint8_t* codes,
                               uint8_t* scales, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  if (dtype == 0) {
    launch_kernel(quantize_mxfp4_rows_kernel<float>, grid, 256, s, static_cast<const float*>(x), codes,
                                                           scales, rows, static_cast<int>(d));
  } else {
    launch_kernel(quantize_mxfp4_rows_kernel<uint16_t>, grid, 256, s, 
        static_cast<const uint16_t*>(x), codes, scales, rows, static_cast<int>(d));
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_quantize_fp8_rows(const void* x, int dtype, int64_t rows, int64_t d,
                             uint8_t* codes, float* scales, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  if (dtype == 0) {
    launch_kernel(quantize_rows_kernel<float>, grid, 256, s, static_cast<const float*>(x), codes,
                                                     scales, rows, static_cast<int>(d));
  } else {
    launch_kernel(quantize_rows_kernel<uint16_t>, grid, 256, s, static_cast<const uint16_t*>(x),
                                                        codes, scales, rows,
                                                        static_cast<int>(d));
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
