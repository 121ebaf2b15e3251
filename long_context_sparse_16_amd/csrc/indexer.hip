// Lightning Indexer scores ("DeepSeek V4 technical review", takeshell.com,
// section 2.1: indexer queries per query token scored against every
// compressed entry; 64 heads x 128 dims for V4-Pro.  The QK path runs in
// low precision: takeshell.com section 5, dataforcee.us "Muon Optimizer and
// FP4 QAT").
//
//   S[t, j] = ki_scale[j] * sum_h w'[t, h] * phi(qi[t, h, :] . ki[j, :])
//
// The per-query product [H_I x d_I] x [d_I x entries] is a dense
// contraction, so it runs on MFMA: the query heads are the A rows (held in
// registers for the whole kernel), 16 compressed entries form one B column
// tile streamed straight from HBM, and the ReLU / head-weight / cross-head
// sum is fused into the epilogue so only one fp32 score per entry is
// written.
//
// Each lane owns one contiguous quarter of a d_I row (lane group g = l/16
// takes elements [g*d_I/4, (g+1)*d_I/4)), so one entry row is read by four
// lanes as 16-byte vector loads.  The same k assignment is used for the A
// operand, which is all the MFMA needs (see common.h).
#include "common.h"
#include "kernels.h"

namespace csa {

// Element traits: bytes each lane loads per row quarter, and how those
// bytes split into MFMA operand fragments.
template <int DTYPE, int DI>
struct IdxTraits;

template <int DI>
struct IdxTraits<0, DI> {  // fp32, v_mfma_f32_16x16x4_f32
  static constexpr int kElemBytes = 4;
  static constexpr int kLaneBytes = DI * 4 / 4;
  static constexpr int kSteps = DI / 4;
  using Frag = float;
  __device__ static f32x4 mma(const u32x4* a, const u32x4* b, int s, f32x4 c) {
    const float av = __uint_as_float(a[s >> 2][s & 3]);
    const float bv = __uint_as_float(b[s >> 2][s & 3]);
    return mma_f32(av, bv, c);
  }
};

template <int DI>
struct IdxTraits<1, DI> {  // bf16, v_mfma_f32_16x16x32_bf16
  static constexpr int kElemBytes = 2;
  static constexpr int kLaneBytes = DI * 2 / 4;
  static constexpr int kSteps = DI / 32;
  __device__ static f32x4 mma(const u32x4* a, const u32x4* b, int s, f32x4 c) {
    return mma_bf16(__builtin_bit_cast(bf16x8, a[s]), __builtin_bit_cast(bf16x8, b[s]), c);
  }
};

template <int DI>
struct IdxTraits<2, DI> {  // fp8 e4m3, v_mfma_f32_16x16x128_f8f6f4
  static constexpr int kElemBytes = 1;
  static constexpr int kLaneBytes = DI / 4;
  static constexpr int kSteps = DI / 128;
  __device__ static f32x4 mma(const u32x4* a, const u32x4* b, int s, f32x4 c) {
    i32x8 av, bv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      av[i] = static_cast<int>(a[2 * s][i]);
      av[4 + i] = static_cast<int>(a[2 * s + 1][i]);
      bv[i] = static_cast<int>(b[2 * s][i]);
      bv[4 + i] = static_cast<int>(b[2 * s + 1][i]);
    }
    return mma_fp8(av, bv, c);
  }
};

constexpr int kIdxWaves = 4;
constexpr int kIdxTile = 16;  // entries per MFMA column tile

// grid: x = entry chunk, y = query row (b * T + i).  block: 4 waves.
// Wave w of chunk c handles the 16-entry tiles c*tiles_per_wg + w + 4*n.
template <int DTYPE, int DI, bool RELU>
__global__ __launch_bounds__(256) void indexer_kernel(
    const uint8_t* __restrict__ qi, const float* __restrict__ qi_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ ki,
    const float* __restrict__ ki_scale, const int64_t* __restrict__ pos0, int64_t T,
    int H_I, int64_t n_cap, int m, int tiles_per_wg, float* __restrict__ scores) {
  using Tr = IdxTraits<DTYPE, DI>;
  constexpr int kVec = Tr::kLaneBytes / 16;  // 16-byte loads per lane per row
  constexpr int kRowBytes = DI * Tr::kElemBytes;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int64_t row = blockIdx.y;
  const int64_t b = row / T;
  const int64_t t = pos0[b] + (row - b * T);
  const int64_t V = visible_entries(t, m, n_cap);
  const int64_t tile0 = static_cast<int64_t>(blockIdx.x) * tiles_per_wg;
  const int64_t e_begin = tile0 * kIdxTile;
  if (e_begin >= V) return;
  const int64_t ntiles = min(static_cast<int64_t>(tiles_per_wg), (V - e_begin + kIdxTile - 1) / kIdxTile);

  // A operand: 4 head tiles of 16 query heads, kept in registers.
  u32x4 a[4][kVec];
  float wq[4][4];
  const int n_ht = (H_I + 15) >> 4;
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const int h = ht * 16 + col;
#pragma unroll
    for (int v = 0; v < kVec; ++v) a[ht][v] = u32x4{0u, 0u, 0u, 0u};
    if (ht < n_ht && h < H_I) {
      const u32x4* src = reinterpret_cast<const u32x4*>(
          qi + (row * H_I + h) * kRowBytes + g * Tr::kLaneBytes);
#pragma unroll
      for (int v = 0; v < kVec; ++v) a[ht][v] = src[v];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = ht * 16 + g * 4 + i;
      float wv = 0.f;
      if (hh < H_I) {
        wv = w[row * H_I + hh];
        if (DTYPE == 2) wv *= qi_scale[row * H_I + hh];
      }
      wq[ht][i] = wv;
    }
  }

  const uint8_t* kib = ki + b * n_cap * kRowBytes;
  float* srow = scores + row * n_cap;

  auto load_tile = [&](int64_t tile, u32x4* dst) {
    const int64_t e = (tile0 + tile) * kIdxTile + col;
    if (e < V) {
      const u32x4* src = reinterpret_cast<const u32x4*>(kib + e * kRowBytes + g * Tr::kLaneBytes);
#pragma unroll
      for (int v = 0; v < kVec; ++v) dst[v] = src[v];
    } else {
#pragma unroll
      for (int v = 0; v < kVec; ++v) dst[v] = u32x4{0u, 0u, 0u, 0u};
    }
  };

  u32x4 bcur[kVec], bnext[kVec];
  int64_t tile = wave;
  if (tile < ntiles) load_tile(tile, bcur);
  for (; tile < ntiles; tile += kIdxWaves) {
    if (tile + kIdxWaves < ntiles) load_tile(tile + kIdxWaves, bnext);
    f32x4 acc[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < Tr::kSteps; ++s) {
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        if (ht < n_ht) acc[ht] = Tr::mma(a[ht], bcur, s, acc[ht]);
      }
    }
    float v = 0.f;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = RELU ? fmaxf(acc[ht][i], 0.f) : acc[ht][i];
        v = fmaf(wq[ht][i], x, v);
      }
    }
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    const int64_t e = (tile0 + tile) * kIdxTile + col;
    if (lane < 16 && e < V) {
      if (DTYPE == 2) v *= ki_scale[b * n_cap + e];
      srow[e] = v;
    }
#pragma unroll
    for (int k = 0; k < kVec; ++k) bcur[k] = bnext[k];
  }
}

template <int DTYPE, int DI>
static void launch_idx_t(const void* qi, const float* qs, const float* w, const void* ki,
                         const float* ks, const int64_t* pos0, int64_t B, int64_t T, int H_I,
                         int64_t n_cap, int m, bool relu, float* scores, hipStream_t s) {
  // 2048 entries per workgroup (32 tiles per wave) unless the cache is small.
  const int64_t tiles = (n_cap + kIdxTile - 1) / kIdxTile;
  const int tiles_per_wg = static_cast<int>(tiles < 128 ? tiles : 128);
  dim3 grid(static_cast<unsigned>((tiles + tiles_per_wg - 1) / tiles_per_wg),
            static_cast<unsigned>(B * T));
  auto q8 = static_cast<const uint8_t*>(qi);
  auto k8 = static_cast<const uint8_t*>(ki);
  if (relu)
    indexer_kernel<DTYPE, DI, true><<<grid, 256, 0, s>>>(q8, qs, w, k8, ks, pos0, T, H_I, n_cap,
                                                         m, tiles_per_wg, scores);
  else
    indexer_kernel<DTYPE, DI, false><<<grid, 256, 0, s>>>(q8, qs, w, k8, ks, pos0, T, H_I,
                                                          n_cap, m, tiles_per_wg, scores);
}

int launch_index_scores(const void* qi, int dtype, const float* qs, const float* w,
                        const void* ki, const float* ks, const int64_t* pos0, int64_t B,
                        int64_t T, int64_t H_I, int64_t d_I, int64_t n_cap, int m, int act,
                        float* scores, hipStream_t s) {
  const bool relu = act == 0;
  const int H = static_cast<int>(H_I);
#define CSA_IDX_CASE(DT, DI)                                                             \
  if (dtype == DT && d_I == DI) {                                                        \
    launch_idx_t<DT, DI>(qi, qs, w, ki, ks, pos0, B, T, H, n_cap, m, relu, scores, s);   \
    return hipGetLastError() == hipSuccess ? 0 : -1;                                     \
  }
  CSA_IDX_CASE(0, 64)
  CSA_IDX_CASE(0, 128)
  CSA_IDX_CASE(1, 64)
  CSA_IDX_CASE(1, 128)
  CSA_IDX_CASE(1, 256)
  CSA_IDX_CASE(2, 128)
#undef CSA_IDX_CASE
  return -2;
}

}  // namespace csa
