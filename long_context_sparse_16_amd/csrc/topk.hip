// Per-query top-k selection over indexer scores ("DeepSeek V4 technical
// review", takeshell.com, section 2.1: the indexer keeps the top-k most
// relevant compressed blocks; k = 1024 for V4-Pro).
//
// Order: larger score first, equal scores to the lower entry index.  Output:
// the selected entry indices in ascending order, padded with -1.
//
// Exact radix select on order-preserving 32-bit keys:
//   1. 4096-bin histogram of the top 12 key bits over the visible entries
//      (fused into the indexer epilogue on the decode path).  The bucket b1
//      holding the k-th largest key splits the row into entries that are
//      surely selected (bucket > b1) and candidates (bucket == b1).
//   2. The candidates are resolved in LDS by two more digit passes (10 + 10
//      bits) that give the exact k-th key and, only when several entries
//      share it, three digit passes over the entry index that keep the
//      lowest indices.  A candidate bucket larger than the LDS buffer (a row
//      of equal scores, say) is resolved by the same passes reading the row
//      from global memory.
//   3. The winners are marked in an LDS bitmap over the row and emitted in
//      ascending order by a prefix sum of per-word popcounts.
//
// Drivers:
//   * split path (few long rows, decode): many workgroups per row classify
//     a 4096-entry slice each and append sure entries / candidates to
//     per-row lists with one atomic per wave; a second kernel resolves each
//     row in one workgroup and returns the row's workspace to all-zero.
//     (A kernel boundary is the cheap way to make the lists visible: a
//     last-workgroup hand-off would need device-scope fences, which write
//     back and invalidate a whole XCD's L2.)
//   * row path (many rows, prefill): one workgroup per row reads its score
//     row twice (histogram, then classification) and resolves in LDS.
#include "common.h"
#include "kernels.h"

namespace csa {

constexpr int kHistBins = kTopkHistBins;        // 4096
constexpr int kCandCap = 8192;                  // candidates resolved in LDS
constexpr int kMaxK = 4096;
constexpr int kBitmapMaxEntries = 262144;       // bitmap output up to this V
constexpr int kSelThreads = 256;
constexpr int kSelEntries = 4096;               // entries per select workgroup
constexpr int kRowThreads = 1024;
constexpr int64_t kRowDirectMaxEntries = 65536;  // few-row cut-over to the row kernel

struct FinishShared {
  uint32_t hist[2048];                    // digit passes 2.. (<= 2048 bins)
  uint32_t ckey[kCandCap];
  int32_t cidx[kCandCap];
  int32_t sel[kMaxK];
  uint32_t bitmap[kBitmapMaxEntries / 32];  // also the 4096-bin first digit
  uint32_t scan[32];
  uint32_t misc[8];  // [0] bin [1] above [4] selected [5] candidates [7] flag
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

// Find the bin holding the r-th largest element (1-based) of a histogram in
// LDS and the number of elements in higher bins: out[0] = bin, out[1] =
// count above.  Requires 1 <= r <= total and nb a multiple of NT (or <= NT).
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

// One digit pass over a set of (key, index) items: histogram of
// (key >> shift) & (nb-1), then the bin of the r-th largest.  visit(f)
// calls f(key, index) for every item.
template <int NT, typename Visit>
__device__ void digit_pass(FinishShared& sm, Visit visit, int shift, int nb, uint32_t r) {
  for (int i = threadIdx.x; i < nb; i += NT) sm.hist[i] = 0u;
  __syncthreads();
  visit([&](uint32_t key, int32_t) { atomicAdd(&sm.hist[(key >> shift) & (nb - 1)], 1u); });
  __syncthreads();
  block_find_top<NT>(sm.hist, nb, r, sm.scan, sm.misc);
}

// Resolve the exact selection among items that all share the first digit,
// needing r of them; winners are appended to sm.sel at sm.misc[4].
template <int NT, typename Visit>
__device__ void resolve_candidates(FinishShared& sm, Visit visit_all, uint32_t r) {
  digit_pass<NT>(sm, visit_all, 10, 1024, r);  // key bits 19..10
  const uint32_t b2 = sm.misc[0];
  const uint32_t r2 = r - sm.misc[1];
  __syncthreads();
  auto visit_b2 = [&](auto f) {
    visit_all([&](uint32_t key, int32_t j) {
      if (((key >> 10) & 1023u) == b2) f(key, j);
    });
  };
  digit_pass<NT>(sm, visit_b2, 0, 1024, r2);   // key bits 9..0
  const uint32_t b3 = sm.misc[0];
  const uint32_t r3 = r2 - sm.misc[1];        // entries needed at the exact key
  const uint32_t n_eq = sm.hist[b3];
  const uint32_t low20 = (b2 << 10) | b3;
  __syncthreads();
  int32_t jmax = 0x7fffffff;
  if (n_eq > r3) {
    // keep the r3 lowest indices among the ties: the top r3 of
    // 0x7fffffff - j, in digits of 11 / 10 / 10 bits
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
    jmax = static_cast<int32_t>(0x7fffffffu - ((c1 << 20) | (c2 << 10) | c3));
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

// Emit sm.sel[0..k) in ascending order to out[0..k).  Rows up to
// kBitmapMaxEntries long use a bitmap over the row and a prefix sum of
// popcounts; longer rows sort with a bitonic network.
template <int NT>
__device__ void emit_sorted(FinishShared& sm, int k, int64_t V, int32_t* out) {
  const int tid = threadIdx.x;
  if (V <= kBitmapMaxEntries) {
    const int nw = static_cast<int>((V + 31) >> 5);
    for (int i = tid; i < nw; i += NT) sm.bitmap[i] = 0u;
    __syncthreads();
    for (int i = tid; i < k; i += NT) {
      const int32_t j = sm.sel[i];
      if (j >= 0 && j < V) atomicOr(&sm.bitmap[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    const int per = (nw + NT - 1) / NT;
    const int w0 = tid * per;
    const int w1 = min(nw, w0 + per);
    uint32_t cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(sm.bitmap[w]);
    uint32_t pos = block_excl_scan<NT>(cnt, sm.scan);
    if (tid == NT - 1) sm.misc[6] = pos + cnt;  // number of marked entries
    for (int w = w0; w < w1; ++w) {
      uint32_t bits = sm.bitmap[w];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        if (pos < static_cast<uint32_t>(k)) out[pos] = w * 32 + bit;
        ++pos;
        bits &= bits - 1;
      }
    }
    __syncthreads();
    for (int i = static_cast<int>(sm.misc[6]) + tid; i < k; i += NT) out[i] = -1;
  } else {
    int k2 = 1;
    while (k2 < k) k2 <<= 1;
    for (int i = tid + k; i < k2; i += NT) sm.sel[i] = 0x7fffffff;
    __syncthreads();
    for (int size = 2; size <= k2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < k2; i += NT) {
          const int p = i ^ stride;
          if (p > i) {
            const int32_t a = sm.sel[i], b = sm.sel[p];
            if ((a > b) == ((i & size) == 0)) {
              sm.sel[i] = b;
              sm.sel[p] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < k; i += NT) out[i] = sm.sel[i];
  }
}

__device__ __forceinline__ void write_iota(int32_t* out, int64_t V, int k) {
  for (int i = threadIdx.x; i < k; i += blockDim.x) out[i] = i < V ? i : -1;
}

// Resolve r winners among the candidates (first digit == b1), either from
// LDS (nc <= kCandCap) or from the score row, then emit the row.
template <int NT>
__device__ void finish_row(FinishShared& sm, const float* srow, int64_t V, uint32_t b1,
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
        if ((key >> kTopkDigit1Shift) == b1) f(key, static_cast<int32_t>(j));
      }
    };
    resolve_candidates<NT>(sm, visit, r);
  }
  emit_sorted<NT>(sm, k, V, out);
}

// ------------------------------------------------------------- row path

// The row is read twice (histogram, then classification); each pass takes
// the row in batches of kRowBatch independent loads per thread that are all
// in flight before any is used.
constexpr int kRowBatch = 16;

// hist_io (nullable): the rows' first-digit histograms built by the
// indexer; used instead of the first pass and returned to zero.
__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ pos0, int64_t T,
    int64_t n_cap, int m, int k, int32_t* __restrict__ idx, uint32_t* __restrict__ hist_io) {
  __shared__ FinishShared sm;
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
  uint32_t* h1 = sm.bitmap;  // first-digit histogram (the bitmap is used later)
  uint32_t* gh = hist_io ? hist_io + row * kHistBins : nullptr;
  for (int i = threadIdx.x; i < kHistBins; i += kRowThreads) h1[i] = gh ? gh[i] : 0u;
  if (threadIdx.x < 8) sm.misc[threadIdx.x] = 0u;
  __syncthreads();
  // visit(f): f(key, j) for every visible entry, batched loads
  auto visit_row = [&](auto f) {
    for (int64_t base = threadIdx.x; base < V; base += static_cast<int64_t>(kRowThreads) * kRowBatch) {
      float v[kRowBatch];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        const int64_t j = base + static_cast<int64_t>(u) * kRowThreads;
        v[u] = srow[j < V ? j : V - 1];
      }
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        const int64_t j = base + static_cast<int64_t>(u) * kRowThreads;
        if (j < V) f(score_key(v[u]), j);
      }
    }
  };
  if (!gh) {
    visit_row([&](uint32_t key, int64_t) { atomicAdd(&h1[key >> kTopkDigit1Shift], 1u); });
    __syncthreads();
  } else {
    for (int i = threadIdx.x; i < kHistBins; i += kRowThreads) gh[i] = 0u;
  }
  block_find_top<kRowThreads>(h1, kHistBins, static_cast<uint32_t>(k), sm.scan, sm.misc);
  const uint32_t b1 = sm.misc[0];
  visit_row([&](uint32_t key, int64_t j) {
    const uint32_t bk = key >> kTopkDigit1Shift;
    if (bk > b1) {
      const uint32_t p = atomicAdd(&sm.misc[4], 1u);
      if (p < kMaxK) sm.sel[p] = static_cast<int32_t>(j);
    } else if (bk == b1) {
      const uint32_t p = atomicAdd(&sm.misc[5], 1u);
      if (p < kCandCap) {
        sm.ckey[p] = key;
        sm.cidx[p] = static_cast<int32_t>(j);
      }
    }
  });
  const uint32_t above = sm.misc[1];
  __syncthreads();
  const uint32_t nc = sm.misc[5];
  finish_row<kRowThreads>(sm, srow, V, b1, static_cast<uint32_t>(k) - above, nc, k, out);
}

// ------------------------------------------------------------ split path
//
// Workspace per row, all-zero between calls: hist[4096] u32, ctrl[4] u32
// (sure count, candidate count, first-digit bucket, count above it); then
// the per-row lists
// sure[kMaxK] i32, ckey[kCandCap] u32, cidx[kCandCap] i32, whose contents
// never matter on entry.

struct SplitWs {
  uint32_t* hist;
  uint32_t* ctrl;
  int32_t* sure;
  uint32_t* ckey;
  int32_t* cidx;
};

inline size_t split_ws_bytes(int64_t rows) {
  return static_cast<size_t>(rows) *
         (sizeof(uint32_t) * (kHistBins + 4) + sizeof(int32_t) * kMaxK +
          (sizeof(uint32_t) + sizeof(int32_t)) * kCandCap);
}

inline SplitWs split_ws(void* base, int64_t rows) {
  SplitWs w;
  char* p = static_cast<char*>(base);
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * kHistBins * rows;
  w.ctrl = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * 4 * rows;
  w.sure = reinterpret_cast<int32_t*>(p);
  p += sizeof(int32_t) * kMaxK * rows;
  w.ckey = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * kCandCap * rows;
  w.cidx = reinterpret_cast<int32_t*>(p);
  return w;
}

// First-digit histogram of each row (when the indexer did not build it).
__global__ __launch_bounds__(kSelThreads) void topk_hist_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ pos0, int64_t T,
    int64_t n_cap, int m, int k, SplitWs ws) {
  __shared__ uint32_t hist[kHistBins];
  const int64_t row = blockIdx.y;
  const int64_t b = row / T;
  const int64_t t = pos0[b] + (row - b * T);
  const int64_t V = visible_entries(t, m, n_cap);
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * kSelEntries;
  if (V <= k || j0 >= V) return;
  const int64_t j1 = min(V, j0 + kSelEntries);
  for (int i = threadIdx.x; i < kHistBins; i += kSelThreads) hist[i] = 0u;
  __syncthreads();
  const float* srow = scores + row * n_cap;
  for (int64_t j = j0 + threadIdx.x; j < j1; j += kSelThreads)
    atomicAdd(&hist[score_key(srow[j]) >> kTopkDigit1Shift], 1u);
  __syncthreads();
  uint32_t* gh = ws.hist + row * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kSelThreads) {
    const uint32_t c = hist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// Append the lanes whose flag is set to an LDS list with one LDS atomic per
// wave; positions within the wave follow lane order.
__device__ __forceinline__ void wave_append_lds(bool flag, uint32_t* counter, int32_t* list_idx,
                                                uint32_t* list_key, int32_t j, uint32_t key) {
  const unsigned long long mask = __ballot(flag);
  if (mask == 0ull) return;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll(static_cast<long long>(mask)) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, static_cast<uint32_t>(__popcll(mask)));
  base = __shfl(base, leader);
  if (flag) {
    const uint32_t p = base + static_cast<uint32_t>(__popcll(mask & ((1ull << lane) - 1ull)));
    list_idx[p] = j;
    if (list_key) list_key[p] = key;
  }
}

// Classify one 4096-entry slice of a row: entries above the bucket of the
// k-th largest key go to the row's "sure" list, entries in that bucket to
// its candidate list.  Each workgroup collects its slice's entries in LDS
// and reserves its range of the row's lists with one global atomic per
// list.  The bucket and the count above it are also recorded for the
// finishing kernel.
__global__ __launch_bounds__(kSelThreads) void topk_classify_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ pos0, int64_t T,
    int64_t n_cap, int m, int k, SplitWs ws) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t scan[32];
  __shared__ uint32_t res[8];
  __shared__ int32_t l_sure[kSelEntries];
  __shared__ int32_t l_cidx[kSelEntries];
  __shared__ uint32_t l_ckey[kSelEntries];
  const int64_t row = blockIdx.y;
  const int64_t b = row / T;
  const int64_t t = pos0[b] + (row - b * T);
  const int64_t V = visible_entries(t, m, n_cap);
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * kSelEntries;
  if (V <= k || j0 >= V) return;
  const uint32_t* gh = ws.hist + row * kHistBins;
  uint32_t* ctrl = ws.ctrl + row * 4;
  for (int i = threadIdx.x; i < kHistBins; i += kSelThreads) hist[i] = gh[i];
  if (threadIdx.x < 8) res[threadIdx.x] = 0u;
  __syncthreads();
  block_find_top<kSelThreads>(hist, kHistBins, static_cast<uint32_t>(k), scan, res);
  const uint32_t b1 = res[0];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ctrl[2] = b1;
    ctrl[3] = res[1];
  }
  const float* srow = scores + row * n_cap;
  const int64_t j1 = min(V, j0 + kSelEntries);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // all of this thread's scores are loaded before any is classified
  constexpr int kIters = kSelEntries / kSelThreads;
  float sv[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    int64_t j = j0 + it * kSelThreads + wave * 64 + lane;
    sv[it] = srow[j < j1 ? j : j1 - 1];
  }
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int64_t j = j0 + it * kSelThreads + wave * 64 + lane;
    const bool valid = j < j1;
    const uint32_t key = score_key(sv[it]);
    const uint32_t bk = key >> kTopkDigit1Shift;
    wave_append_lds(valid && bk > b1, &res[4], l_sure, nullptr, static_cast<int32_t>(j), key);
    wave_append_lds(valid && bk == b1, &res[5], l_cidx, l_ckey, static_cast<int32_t>(j), key);
  }
  __syncthreads();
  const uint32_t ns = res[4], nc = res[5];
  if (threadIdx.x == 0) {
    res[6] = ns ? atomicAdd(&ctrl[0], ns) : 0u;
    res[7] = nc ? atomicAdd(&ctrl[1], nc) : 0u;
  }
  __syncthreads();
  const uint32_t sb = res[6], cb = res[7];
  int32_t* gs = ws.sure + row * kMaxK;
  for (uint32_t i = threadIdx.x; i < ns; i += kSelThreads)
    if (sb + i < static_cast<uint32_t>(kMaxK)) gs[sb + i] = l_sure[i];
  int32_t* gi = ws.cidx + row * kCandCap;
  uint32_t* gk = ws.ckey + row * kCandCap;
  for (uint32_t i = threadIdx.x; i < nc; i += kSelThreads) {
    if (cb + i < static_cast<uint32_t>(kCandCap)) {
      gi[cb + i] = l_cidx[i];
      gk[cb + i] = l_ckey[i];
    }
  }
}

// Resolve one row from its sure list and candidates, then return the row's
// histogram and counters to zero for the next call.
__global__ __launch_bounds__(kSelThreads) void topk_finish_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ pos0, int64_t T,
    int64_t n_cap, int m, int k, SplitWs ws, int32_t* __restrict__ idx) {
  __shared__ FinishShared sm;
  const int64_t row = blockIdx.x;
  const int64_t b = row / T;
  const int64_t t = pos0[b] + (row - b * T);
  const int64_t V = visible_entries(t, m, n_cap);
  int32_t* out = idx + row * k;
  if (V <= k) {
    write_iota(out, V, k);
    return;
  }
  uint32_t* gh = ws.hist + row * kHistBins;
  uint32_t* ctrl = ws.ctrl + row * 4;
  const u32x4 cv = *reinterpret_cast<const u32x4*>(ctrl);  // sure, candidates, bucket, above
  const uint32_t ns = min(cv[0], static_cast<uint32_t>(k));
  const uint32_t nc = cv[1];
  const uint32_t b1 = cv[2];
  if (threadIdx.x < 8) sm.misc[threadIdx.x] = 0u;
  const int32_t* gs = ws.sure + row * kMaxK;
  for (uint32_t i = threadIdx.x; i < ns; i += kSelThreads) sm.sel[i] = gs[i];  // ns <= k
  if (nc <= static_cast<uint32_t>(kCandCap)) {
    const uint32_t* gk = ws.ckey + row * kCandCap;
    const int32_t* gi = ws.cidx + row * kCandCap;
    for (uint32_t i = threadIdx.x; i < nc; i += kSelThreads) {
      sm.ckey[i] = gk[i];
      sm.cidx[i] = gi[i];
    }
  }
  if (threadIdx.x == 0) sm.misc[4] = ns;
  __syncthreads();
  finish_row<kSelThreads>(sm, scores + row * n_cap, V, b1, static_cast<uint32_t>(k) - ns, nc, k,
                          out);
  for (int i = threadIdx.x; i < kHistBins; i += kSelThreads) gh[i] = 0u;
  if (threadIdx.x < 4) ctrl[threadIdx.x] = 0u;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0u;
}

// ----------------------------------------------------------------- host side

size_t topk_workspace_bytes(int64_t B, int64_t T, int64_t n_cap, int k) {
  (void)n_cap;
  (void)k;
  const int64_t rows = B * T;
  return rows <= kTopkSplitMaxRows ? split_ws_bytes(rows) : 0;
}

uint32_t* topk_hist_ptr(void* ws, int64_t B, int64_t T) {
  return B * T <= kTopkSplitMaxRows ? split_ws(ws, B * T).hist : nullptr;
}

int launch_topk(const float* scores, const int64_t* pos0, int64_t B, int64_t T, int64_t n_cap,
                int m, int k, int32_t* idx, void* ws, bool hist_ready, hipStream_t s) {
  const int64_t rows = B * T;
  if (rows <= kTopkSplitMaxRows && n_cap <= kRowDirectMaxEntries) {
    // few rows short enough for one workgroup each: one pass over the row
    // using the indexer's histogram when it built one
    uint32_t* h = hist_ready ? split_ws(ws, rows).hist : nullptr;
    topk_row_kernel<<<static_cast<unsigned>(rows), kRowThreads, 0, s>>>(scores, pos0, T, n_cap, m,
                                                                        k, idx, h);
  } else if (rows <= kTopkSplitMaxRows) {
    SplitWs w = split_ws(ws, rows);
    dim3 grid(static_cast<unsigned>((n_cap + kSelEntries - 1) / kSelEntries),
              static_cast<unsigned>(rows));
    if (!hist_ready) topk_hist_kernel<<<grid, kSelThreads, 0, s>>>(scores, pos0, T, n_cap, m, k, w);
    topk_classify_kernel<<<grid, kSelThreads, 0, s>>>(scores, pos0, T, n_cap, m, k, w);
    topk_finish_kernel<<<static_cast<unsigned>(rows), kSelThreads, 0, s>>>(scores, pos0, T, n_cap,
                                                                           m, k, w, idx);
  } else {
    topk_row_kernel<<<static_cast<unsigned>(rows), kRowThreads, 0, s>>>(scores, pos0, T, n_cap, m,
                                                                        k, idx, nullptr);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_clear(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(bytes / 4);
  if (n == 0) return 0;
  const int64_t blocks = (n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048;
  fill_zero_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(static_cast<uint32_t*>(p), n);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
