// Per-query top-k selection over indexer scores ("DeepSeek V4 technical
// review", takeshell.com, section 2.1: the indexer keeps the top-k most
// relevant compressed blocks; k = 1024 for V4-Pro).
//
// Order: larger score first, equal scores to the lower entry index.  Output:
// the selected entry indices in ascending order, padded with -1.
//
// Algorithm (exact radix select on order-preserving 32-bit keys):
//   1. 4096-bin histogram of the top 12 key bits over the visible entries;
//      the bucket b1 holding the k-th largest key splits the row into
//      entries that are surely selected (bucket > b1) and candidates
//      (bucket == b1).
//   2. The candidates are resolved in LDS by two more digit passes (10 + 10
//      bits) that give the exact k-th key, and -- only when several entries
//      share it -- three digit passes over the entry index that keep the
//      lowest indices.
//   3. The k winners are sorted ascending with a bitonic network in LDS.
// If the candidate bucket is larger than the LDS buffer (e.g. a row of equal
// scores) the same digit passes run directly over the row in global memory.
//
// Two drivers share the resolution code:
//   * "row" path for many rows: one 1024-thread workgroup per row reads its
//     score row twice (histogram, then sure/candidate split).
//   * "split" path for few long rows (decode): the histogram and the split
//     are spread over many workgroups per row (global integer atomics, whose
//     final counts are order independent), then one workgroup per row
//     resolves the candidates.
#include "common.h"
#include "kernels.h"

namespace csa {

constexpr int kTopkThreads = 1024;
constexpr int kHistBins = 4096;  // top 12 key bits
constexpr int kCandCap = 12288;  // candidates resolved in LDS
constexpr int kMaxK = 4096;
constexpr int kSliceThreads = 256;
constexpr int kSliceEntries = 2048;  // entries per workgroup in the split path

struct TopkShared {
  uint32_t hist[kHistBins];
  uint32_t ckey[kCandCap];
  int32_t cidx[kCandCap];
  int32_t sel[kMaxK];
  uint32_t scan[32];
  uint32_t misc[8];
};

// ------------------------------------------------------------ block helpers

template <int NT>
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* sm) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  constexpr int NW = NT / 64;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sm[wv] = x;
  __syncthreads();
  if (wv == 0) {
    uint32_t s = lane < NW ? sm[lane] : 0u;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
      const uint32_t y = __shfl_up(s, o);
      if (lane >= o) s += y;
    }
    if (lane < NW) sm[lane] = s;
  }
  __syncthreads();
  const uint32_t base = wv > 0 ? sm[wv - 1] : 0u;
  __syncthreads();
  return base + x - v;
}

// Given a histogram in LDS, find the bin holding the r-th largest element
// (1-based) and the number of elements in higher bins.  Results land in
// out[0] (bin) and out[1] (count above).  Requires r <= total.
template <int NT>
__device__ void block_find_top(const uint32_t* hist, int nb, uint32_t r, uint32_t* scan_sm,
                               uint32_t* out) {
  const int tid = threadIdx.x;
  const int per = nb / NT > 0 ? nb / NT : 1;
  const int hi = nb - tid * per;  // this thread covers bins [hi-per, hi)
  uint32_t local = 0;
  if (hi > 0)
    for (int q = 0; q < per; ++q) local += hist[hi - 1 - q];
  const uint32_t excl = block_excl_scan<NT>(local, scan_sm);
  if (hi > 0 && excl < r && r <= excl + local) {
    uint32_t acc = excl;
    for (int q = 0; q < per; ++q) {
      const int bin = hi - 1 - q;
      if (acc + hist[bin] >= r) {
        out[0] = static_cast<uint32_t>(bin);
        out[1] = acc;
        break;
      }
      acc += hist[bin];
    }
  }
  __syncthreads();
}

template <int NT>
__device__ void block_clear(uint32_t* a, int n) {
  for (int i = threadIdx.x; i < n; i += NT) a[i] = 0u;
  __syncthreads();
}

// One digit pass over a set of (key, index) items: histogram of
// (key >> shift) & (nb-1) over the items accepted by `match`, then the bin
// of the r-th largest.  `visit(f)` calls f(key, index) for every item.
template <int NT, typename Visit>
__device__ void digit_pass(TopkShared& sm, Visit visit, int shift, int nb, uint32_t r) {
  block_clear<NT>(sm.hist, nb);
  visit([&](uint32_t key, int32_t) {
    atomicAdd(&sm.hist[(key >> shift) & (nb - 1)], 1u);
  });
  __syncthreads();
  block_find_top<NT>(sm.hist, nb, r, sm.scan, sm.misc);
}

// Resolve the exact selection among the items (all in bucket b1 of the
// first digit) given by `visit_all`, needing r of them, and append the
// winners to sm.sel starting at the current sm.misc[4] count.
template <int NT, typename Visit>
__device__ void resolve_candidates(TopkShared& sm, Visit visit_all, uint32_t r) {
  // digit 2: key bits 19..10
  digit_pass<NT>(sm, visit_all, 10, 1024, r);
  const uint32_t b2 = sm.misc[0];
  const uint32_t r2 = r - sm.misc[1];
  __syncthreads();
  auto visit_b2 = [&](auto f) {
    visit_all([&](uint32_t key, int32_t j) {
      if (((key >> 10) & 1023u) == b2) f(key, j);
    });
  };
  // digit 3: key bits 9..0 among bits 19..10 == b2
  digit_pass<NT>(sm, visit_b2, 0, 1024, r2);
  const uint32_t b3 = sm.misc[0];
  const uint32_t r3 = r2 - sm.misc[1];   // ties needed at the exact key
  const uint32_t n_eq = sm.hist[b3];
  const uint32_t low20 = (b2 << 10) | b3;  // the k-th key's low 20 bits
  __syncthreads();
  int32_t jmax = 0x7fffffff;
  if (n_eq > r3) {
    // keep the r3 lowest indices among the ties: select the top r3 of
    // 0x7fffffff - j, three digits of 11 / 10 / 10 bits
    auto visit_eq = [&](auto f) {
      visit_all([&](uint32_t key, int32_t j) {
        if ((key & 0xfffffu) == low20) f(0x7fffffffu - static_cast<uint32_t>(j), j);
      });
    };
    digit_pass<NT>(sm, visit_eq, 20, 2048, r3);
    const uint32_t c1 = sm.misc[0];
    const uint32_t q1 = r3 - sm.misc[1];
    __syncthreads();
    auto visit_c1 = [&](auto f) {
      visit_eq([&](uint32_t k2, int32_t j) {
        if ((k2 >> 20) == c1) f(k2, j);
      });
    };
    digit_pass<NT>(sm, visit_c1, 10, 1024, q1);
    const uint32_t c2 = sm.misc[0];
    const uint32_t q2 = q1 - sm.misc[1];
    __syncthreads();
    auto visit_c2 = [&](auto f) {
      visit_c1([&](uint32_t k2, int32_t j) {
        if (((k2 >> 10) & 1023u) == c2) f(k2, j);
      });
    };
    digit_pass<NT>(sm, visit_c2, 0, 1024, q2);
    const uint32_t c3 = sm.misc[0];
    __syncthreads();
    const uint32_t k2star = (c1 << 20) | (c2 << 10) | c3;
    jmax = static_cast<int32_t>(0x7fffffffu - k2star);
  }
  visit_all([&](uint32_t key, int32_t j) {
    const uint32_t lo = key & 0xfffffu;
    if (lo > low20 || (lo == low20 && j <= jmax)) {
      const uint32_t p = atomicAdd(&sm.misc[4], 1u);
      if (p < kMaxK) sm.sel[p] = j;
    }
  });
  __syncthreads();
}

// Sort sm.sel[0..k) ascending and write it out.
template <int NT>
__device__ void sort_and_store(TopkShared& sm, int k, int32_t* out) {
  int k2 = 1;
  while (k2 < k) k2 <<= 1;
  for (int i = threadIdx.x + k; i < k2; i += NT) sm.sel[i] = 0x7fffffff;
  __syncthreads();
  for (int size = 2; size <= k2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < k2; i += NT) {
        const int p = i ^ stride;
        if (p > i) {
          const int32_t a = sm.sel[i], b = sm.sel[p];
          const bool up = (i & size) == 0;
          if ((a > b) == up) {
            sm.sel[i] = b;
            sm.sel[p] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < k; i += NT) out[i] = sm.sel[i];
}

__device__ __forceinline__ void write_iota(int32_t* out, int64_t V, int k) {
  for (int i = threadIdx.x; i < k; i += blockDim.x) out[i] = i < V ? i : -1;
}

// Candidates either in LDS (nc <= cap) or re-derived from the score row.
template <int NT>
__device__ void finish_row(TopkShared& sm, const float* srow, int64_t V, uint32_t b1,
                           uint32_t r, uint32_t nc, int k, int32_t* out) {
  if (nc <= static_cast<uint32_t>(kCandCap)) {
    auto visit = [&](auto f) {
      for (uint32_t i = threadIdx.x; i < nc; i += NT) f(sm.ckey[i], sm.cidx[i]);
    };
    resolve_candidates<NT>(sm, visit, r);
  } else {
    auto visit = [&](auto f) {
      for (int64_t j = threadIdx.x; j < V; j += NT) {
        const uint32_t key = score_key(srow[j]);
        if ((key >> 20) == b1) f(key, static_cast<int32_t>(j));
      }
    };
    resolve_candidates<NT>(sm, visit, r);
  }
  sort_and_store<NT>(sm, k, out);
}

// ------------------------------------------------------------- row path

__global__ __launch_bounds__(kTopkThreads) void topk_row_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ pos0, int64_t T,
    int64_t n_cap, int m, int k, int32_t* __restrict__ idx) {
  __shared__ TopkShared sm;
  const int64_t row = blockIdx.x;
  const int64_t b = row / T;
  const int64_t t = pos0[b] + (row - b * T);
  const int64_t V = visible_entries(t, m, n_cap);
  int32_t* out = idx + row * k;
  if (V <= k) {
    write_iota(out, V, k);
    return;
  }
  const float* srow = scores + row * n_cap;
  block_clear<kTopkThreads>(sm.hist, kHistBins);
  for (int64_t j = threadIdx.x; j < V; j += kTopkThreads)
    atomicAdd(&sm.hist[score_key(srow[j]) >> 20], 1u);
  __syncthreads();
  block_find_top<kTopkThreads>(sm.hist, kHistBins, static_cast<uint32_t>(k), sm.scan, sm.misc);
  const uint32_t b1 = sm.misc[0];
  const uint32_t above = sm.misc[1];
  __syncthreads();
  if (threadIdx.x == 0) {
    sm.misc[4] = 0;  // selected so far
    sm.misc[5] = 0;  // candidates
  }
  __syncthreads();
  for (int64_t j = threadIdx.x; j < V; j += kTopkThreads) {
    const uint32_t key = score_key(srow[j]);
    const uint32_t bk = key >> 20;
    if (bk > b1) {
      sm.sel[atomicAdd(&sm.misc[4], 1u)] = static_cast<int32_t>(j);
    } else if (bk == b1) {
      const uint32_t p = atomicAdd(&sm.misc[5], 1u);
      if (p < kCandCap) {
        sm.ckey[p] = key;
        sm.cidx[p] = static_cast<int32_t>(j);
      }
    }
  }
  __syncthreads();
  const uint32_t nc = sm.misc[5];
  finish_row<kTopkThreads>(sm, srow, V, b1, static_cast<uint32_t>(k) - above, nc, k, out);
}

// ------------------------------------------------------------ split path
//
// Workspace per row: hist[4096] u32, counters[4] u32 (sure, candidates),
// sure[kMaxK] i32, ckey[kCandCap] u32, cidx[kCandCap] i32.

struct SplitWs {
  uint32_t* hist;
  uint32_t* cnt;
  int32_t* sure;
  uint32_t* ckey;
  int32_t* cidx;
};

__host__ __device__ inline size_t split_ws_bytes(int64_t rows) {
  return static_cast<size_t>(rows) *
         (sizeof(uint32_t) * (kHistBins + 4) + sizeof(int32_t) * kMaxK +
          (sizeof(uint32_t) + sizeof(int32_t)) * kCandCap);
}

__host__ __device__ inline SplitWs split_ws(void* base, int64_t rows) {
  SplitWs w;
  char* p = static_cast<char*>(base);
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * kHistBins * rows;
  w.cnt = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * 4 * rows;
  w.sure = reinterpret_cast<int32_t*>(p);
  p += sizeof(int32_t) * kMaxK * rows;
  w.ckey = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * kCandCap * rows;
  w.cidx = reinterpret_cast<int32_t*>(p);
  return w;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0u;
}

__global__ __launch_bounds__(kSliceThreads) void topk_hist_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ pos0, int64_t T,
    int64_t n_cap, int m, int k, SplitWs ws) {
  __shared__ uint32_t hist[kHistBins];
  const int64_t row = blockIdx.y;
  const int64_t b = row / T;
  const int64_t t = pos0[b] + (row - b * T);
  const int64_t V = visible_entries(t, m, n_cap);
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * kSliceEntries;
  if (V <= k || j0 >= V) return;
  const int64_t j1 = min(V, j0 + kSliceEntries);
  for (int i = threadIdx.x; i < kHistBins; i += kSliceThreads) hist[i] = 0u;
  __syncthreads();
  const float* srow = scores + row * n_cap;
  for (int64_t j = j0 + threadIdx.x; j < j1; j += kSliceThreads)
    atomicAdd(&hist[score_key(srow[j]) >> 20], 1u);
  __syncthreads();
  uint32_t* gh = ws.hist + row * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kSliceThreads) {
    const uint32_t c = hist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

__global__ __launch_bounds__(kSliceThreads) void topk_split_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ pos0, int64_t T,
    int64_t n_cap, int m, int k, SplitWs ws) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t scan_sm[32];
  __shared__ uint32_t res[8];
  __shared__ int32_t l_sure[kSliceEntries];
  __shared__ uint32_t l_ckey[kSliceEntries];
  __shared__ int32_t l_cidx[kSliceEntries];
  const int64_t row = blockIdx.y;
  const int64_t b = row / T;
  const int64_t t = pos0[b] + (row - b * T);
  const int64_t V = visible_entries(t, m, n_cap);
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * kSliceEntries;
  if (V <= k || j0 >= V) return;
  const int64_t j1 = min(V, j0 + kSliceEntries);
  const uint32_t* gh = ws.hist + row * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kSliceThreads) hist[i] = gh[i];
  if (threadIdx.x < 8) res[threadIdx.x] = 0u;
  __syncthreads();
  block_find_top<kSliceThreads>(hist, kHistBins, static_cast<uint32_t>(k), scan_sm, res);
  const uint32_t b1 = res[0];
  const float* srow = scores + row * n_cap;
  for (int64_t j = j0 + threadIdx.x; j < j1; j += kSliceThreads) {
    const uint32_t key = score_key(srow[j]);
    const uint32_t bk = key >> 20;
    if (bk > b1) {
      l_sure[atomicAdd(&res[2], 1u)] = static_cast<int32_t>(j);
    } else if (bk == b1) {
      const uint32_t p = atomicAdd(&res[3], 1u);
      l_ckey[p] = key;
      l_cidx[p] = static_cast<int32_t>(j);
    }
  }
  __syncthreads();
  const uint32_t ns = res[2], nc = res[3];
  if (threadIdx.x == 0) {
    res[4] = ns ? atomicAdd(&ws.cnt[row * 4 + 0], ns) : 0u;
    res[5] = nc ? atomicAdd(&ws.cnt[row * 4 + 1], nc) : 0u;
  }
  __syncthreads();
  const uint32_t sbase = res[4], cbase = res[5];
  int32_t* gs = ws.sure + row * kMaxK;
  for (uint32_t i = threadIdx.x; i < ns; i += kSliceThreads)
    if (sbase + i < static_cast<uint32_t>(kMaxK)) gs[sbase + i] = l_sure[i];
  uint32_t* gk = ws.ckey + row * kCandCap;
  int32_t* gi = ws.cidx + row * kCandCap;
  for (uint32_t i = threadIdx.x; i < nc; i += kSliceThreads) {
    if (cbase + i < static_cast<uint32_t>(kCandCap)) {
      gk[cbase + i] = l_ckey[i];
      gi[cbase + i] = l_cidx[i];
    }
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_finish_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ pos0, int64_t T,
    int64_t n_cap, int m, int k, SplitWs ws, int32_t* __restrict__ idx) {
  __shared__ TopkShared sm;
  const int64_t row = blockIdx.x;
  const int64_t b = row / T;
  const int64_t t = pos0[b] + (row - b * T);
  const int64_t V = visible_entries(t, m, n_cap);
  int32_t* out = idx + row * k;
  if (V <= k) {
    write_iota(out, V, k);
    return;
  }
  const uint32_t* gh = ws.hist + row * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kTopkThreads) sm.hist[i] = gh[i];
  __syncthreads();
  block_find_top<kTopkThreads>(sm.hist, kHistBins, static_cast<uint32_t>(k), sm.scan, sm.misc);
  const uint32_t b1 = sm.misc[0];
  const uint32_t above = sm.misc[1];
  const uint32_t ns = min(ws.cnt[row * 4 + 0], static_cast<uint32_t>(kMaxK));
  const uint32_t nc = ws.cnt[row * 4 + 1];
  __syncthreads();
  const int32_t* gs = ws.sure + row * kMaxK;
  for (uint32_t i = threadIdx.x; i < ns; i += kTopkThreads) sm.sel[i] = gs[i];
  if (nc <= static_cast<uint32_t>(kCandCap)) {
    const uint32_t* gk = ws.ckey + row * kCandCap;
    const int32_t* gi = ws.cidx + row * kCandCap;
    for (uint32_t i = threadIdx.x; i < nc; i += kTopkThreads) {
      sm.ckey[i] = gk[i];
      sm.cidx[i] = gi[i];
    }
  }
  if (threadIdx.x == 0) sm.misc[4] = ns;
  __syncthreads();
  (void)above;
  const float* srow = scores + row * n_cap;
  finish_row<kTopkThreads>(sm, srow, V, b1, static_cast<uint32_t>(k) - ns, nc, k, out);
}

// ----------------------------------------------------------------- host side

size_t topk_workspace_bytes(int64_t B, int64_t T, int64_t n_cap, int k) {
  (void)n_cap;
  (void)k;
  const int64_t rows = B * T;
  return rows <= kTopkSplitMaxRows ? split_ws_bytes(rows) : 0;
}

int launch_topk(const float* scores, const int64_t* pos0, int64_t B, int64_t T, int64_t n_cap,
                int m, int k, int32_t* idx, void* ws, hipStream_t s) {
  const int64_t rows = B * T;
  if (rows <= kTopkSplitMaxRows) {
    SplitWs w = split_ws(ws, rows);
    const int64_t n_zero = rows * (kHistBins + 4);  // hist and counters are adjacent
    fill_zero_kernel<<<static_cast<unsigned>((n_zero + 255) / 256 < 1024 ? (n_zero + 255) / 256 : 1024), 256, 0,
                       s>>>(w.hist, n_zero);
    dim3 grid(static_cast<unsigned>((n_cap + kSliceEntries - 1) / kSliceEntries),
              static_cast<unsigned>(rows));
    topk_hist_kernel<<<grid, kSliceThreads, 0, s>>>(scores, pos0, T, n_cap, m, k, w);
    topk_split_kernel<<<grid, kSliceThreads, 0, s>>>(scores, pos0, T, n_cap, m, k, w);
    topk_finish_kernel<<<static_cast<unsigned>(rows), kTopkThreads, 0, s>>>(scores, pos0, T,
                                                                            n_cap, m, k, w, idx);
  } else {
    topk_row_kernel<<<static_cast<unsigned>(rows), kTopkThreads, 0, s>>>(scores, pos0, T, n_cap,
                                                                         m, k, idx);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
