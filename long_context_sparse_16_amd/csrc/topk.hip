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
//   * split path (few long rows, decode): one workgroup per 4096-entry
//     slice finds the bucket from the row's histogram and writes the
//     slice's sure entries and candidates to its own workspace region; a
//     second kernel, one workgroup per row, gathers them, resolves the row
//     and returns the row's histogram to zero.  (A kernel boundary is the
//     cheap way to make the lists visible: a last-workgroup hand-off needs
//     device-scope fences, which write back and invalidate a whole XCD's
//     L2; measured on the 32 x 32768 decode rows, such a fused kernel took
//     three times as long as the two launches.)
//   * row path (many rows, prefill; short rows): one workgroup per row;
//     rows of up to 32768 entries are held in registers and read once;
//     rows of up to 16384, and rows read in batches, run two 512-thread
//     workgroups per CU.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "select.h"

namespace csa {

constexpr int kHistBins = kTopkHistBins;        // 4096
constexpr int kCandCap = 8192;                  // candidates resolved in LDS
constexpr int kMaxK = 4096;
constexpr int kBitmapMaxEntries = 262144;       // bitmap output up to this V
constexpr int kSelThreads = 256;
constexpr int kSelEntries = 4096;               // entries per select workgroup
constexpr int kRowThreads = 1024;
constexpr int64_t kRowSplitMinEntries = 8192;  // few rows longer than this take the split path

// LDS of the finishing and row kernels: CAND candidates resolved in LDS,
// bitmap output for rows of up to BM entries.
template <int CAND, int BM>
struct FinishSharedT {
  static constexpr int kCand = CAND;
  static constexpr int kBitmapEntries = BM;
  uint32_t hist[2048];                    // digit passes 2.. (<= 2048 bins)
  uint32_t ckey[CAND];
  int32_t cidx[CAND];
  int32_t sel[kMaxK];
  // row bitmap, one pad word after every 32 (see bm_slot); also holds the
  // 4096-bin first-digit histogram in the row kernel
  uint32_t bitmap[BM / 32 + BM / 1024];
  uint32_t scan[32];
  uint32_t misc[8];  // [0] bin [1] above [2] [3] cut [4] selected [5] candidates [6] flag [7] count
};
using FinishShared = FinishSharedT<kCandCap, kBitmapMaxEntries>;
// The 512-thread row kernel, two workgroups per CU: 74,400 bytes of LDS
// (4096 candidates; the bitmap area still holds the 4096-bin histogram).
using RowShared2 = FinishSharedT<4096, 131072>;
static_assert(131072 / 32 >= kHistBins, "the bitmap area holds the first-digit histogram");

// resolve_cut, then append the winners to sm.sel at sm.misc[4].
template <int NT, typename SM, typename Visit>
__device__ void resolve_candidates(SM& sm, Visit visit_all, uint32_t r) {
  const Cut c = resolve_cut<NT>(sm, visit_all, r);
  visit_all([&](uint32_t key, int32_t j) {
    if (cut_wins(c, key, j)) {
      const uint32_t p = atomicAdd(&sm.misc[4], 1u);
      if (p < kMaxK) sm.sel[p] = j;
    }
  });
  __syncthreads();
}

// LDS slot of bitmap word w: one pad word after every 32, so that threads
// reading 32 consecutive words each hit distinct banks.
__device__ __forceinline__ int bm_slot(int w) { return w + (w >> 5); }

// Emit sm.sel[0..k) in ascending order to out[0..k).  Rows up to
// SM::kBitmapEntries long use a bitmap over the row: each thread owns a run
// of consecutive words, counts their bits, takes its output position from
// a block prefix sum and writes its entries in order.  Longer rows sort
// with a bitonic network.
template <int NT, typename SM>
__device__ void emit_sorted(SM& sm, int k, int64_t V, int32_t* out) {
  const int tid = threadIdx.x;
  if (V <= SM::kBitmapEntries) {
    const int nw = static_cast<int>((V + 31) >> 5);
    for (int i = tid; i < bm_slot(nw); i += NT) sm.bitmap[i] = 0u;
    __syncthreads();
    for (int i = tid; i < k; i += NT) {
      const int32_t j = sm.sel[i];
      if (j >= 0 && j < V) atomicOr(&sm.bitmap[bm_slot(j >> 5)], 1u << (j & 31));
    }
    __syncthreads();
    const int per = (nw + NT - 1) / NT;
    const int w0 = tid * per;
    const int w1 = min(nw, w0 + per);
    uint32_t cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(sm.bitmap[bm_slot(w)]);
    uint32_t pos = block_excl_scan<NT>(cnt, sm.scan);
    if (tid == NT - 1) sm.misc[6] = pos + cnt;  // number of marked entries
    for (int w = w0; w < w1; ++w) {
      uint32_t bits = sm.bitmap[bm_slot(w)];
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
// LDS (nc <= SM::kCand) or from the score row, then emit the row.
template <int NT, typename SM>
__device__ void finish_row(SM& sm, const float* srow, int64_t V, uint32_t b1,
                           uint32_t r, uint32_t nc, int k, int32_t* out) {
  if (nc <= static_cast<uint32_t>(SM::kCand)) {
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

// Rows of up to NT * REGS entries are held in registers (REGS > 0):
// the histogram loads go out first, then the row's, so the histogram is
// usable before the row has arrived, and the row is read once.  Longer rows
// (REGS == 0) are read in batches of kRowBatch independent loads per thread
// (twice when the histogram is built here).  Register rows are classified
// by counting each thread's sure entries and candidates, one block prefix
// sum of the packed counts and writes without atomics; batched rows take
// their list slots with one LDS atomic per thread, list and batch.
constexpr int kRowBatch = 32;
// Batched rows run 512-thread workgroups with the small LDS layout, two per
// CU, so one row's cut and output phases overlap the other's reads.
constexpr int kRowBatchedThreads = 512;
// register-resident rows: 32 per thread, V <= 16384 at 512 threads and
// V <= 32768 at 1024
constexpr int kRowRegs = 32;

// LDS layout of the row kernel by workgroup size: 1024 threads (one
// workgroup per CU) use the full layout, 512 threads (two per CU) the small
// one.
template <int NT> struct RowShm { using T = FinishShared; };
template <> struct RowShm<512> { using T = RowShared2; };

// hist_io (nullable): the rows' first-digit histograms built by the
// indexer; used instead of a histogram pass and returned to zero.
// COARSE: the rows' 2048-bin histograms of the top 11 key bits from the
// prefill indexer instead (each used when its flag says this call wrote it;
// every flag is cleared).  The row is then classified against the coarse
// bucket in its one pass, which also counts the bucket's upper half; that
// count decides which half holds the k-th key, and the candidates in LDS
// are narrowed to it (the upper half joining the sure entries when the cut
// is in the lower one).  Should the coarse candidates overflow the LDS
// list, the row is classified again against the exact 12-bit bucket.
template <int REGS, bool COARSE, int NT>
__global__ __launch_bounds__(NT) void topk_row_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ pos0, int64_t T,
    int64_t n_cap, int m, int k, int32_t* __restrict__ idx, uint32_t* __restrict__ hist_io,
    CoarseHist coarse) {
  using SM = typename RowShm<NT>::T;
  __shared__ SM sm;
  constexpr int kHistPer = kHistBins / NT;
  constexpr int kCoarsePer = kTopkCoarseBins / NT;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t b = seq_of_row(row, T);
  const int64_t t = pos0[b] + (row - b * T);
  const int64_t V = uniform64(visible_entries(t, m, n_cap));
  int32_t* out = idx + row * k;
  if (V <= k) {
    if (COARSE && tid == 0) coarse.flag[row] = 0u;
    write_iota(out, V, k);
    return;
  }
  const float* srow = scores + row * n_cap;
  uint32_t* h1 = sm.bitmap;  // first-digit histogram (the bitmap is used later)
  uint32_t* gh = !COARSE && hist_io ? hist_io + row * kHistBins : nullptr;
  // (all threads read the flag before thread 0 clears it, after the barrier)
  const bool use_coarse = COARSE && coarse.flag[row] != 0u;
  uint32_t hv[kHistPer];
#pragma unroll
  for (int q = 0; q < kHistPer; ++q) {
    if (COARSE)
      hv[q] = q < kCoarsePer && use_coarse
                  ? coarse.hist[row * kTopkCoarseBins + tid + q * NT]
                  : 0u;
    else
      hv[q] = gh ? gh[tid + q * NT] : 0u;
  }
  float rv[REGS > 0 ? REGS : 1];
  if (REGS > 0) {
#pragma unroll
    for (int u = 0; u < REGS; ++u) {
      const int64_t j = tid + static_cast<int64_t>(u) * NT;
      rv[u] = srow[j < V ? j : V - 1];
    }
  }
#pragma unroll
  for (int q = 0; q < kHistPer; ++q) h1[tid + q * NT] = hv[q];
  if (tid < 8) sm.misc[tid] = 0u;
  __syncthreads();
  if (COARSE && tid == 0) coarse.flag[row] = 0u;
  const bool have_hist = use_coarse || gh != nullptr;
  if (!have_hist) {
    if (REGS > 0) {
#pragma unroll
      for (int u = 0; u < REGS; ++u) {
        const int64_t j = tid + static_cast<int64_t>(u) * NT;
        if (j < V) atomicAdd(&h1[score_key(rv[u]) >> kTopkDigit1Shift], 1u);
      }
    } else {
      for (int64_t base = 0; base < V; base += static_cast<int64_t>(NT) * kRowBatch) {
        float v[kRowBatch];
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
          const int64_t j = base + tid + static_cast<int64_t>(u) * NT;
          v[u] = srow[j < V ? j : V - 1];
        }
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
          const int64_t j = base + tid + static_cast<int64_t>(u) * NT;
          if (j < V) atomicAdd(&h1[score_key(v[u]) >> kTopkDigit1Shift], 1u);
        }
      }
    }
    __syncthreads();
  } else if (gh) {
#pragma unroll
    for (int q = 0; q < kHistPer; ++q) gh[tid + q * NT] = 0u;
  }
  const int shift = use_coarse ? kTopkCoarseShift : kTopkDigit1Shift;
  block_find_top<NT>(h1, use_coarse ? kTopkCoarseBins : kHistBins,
                              static_cast<uint32_t>(k), sm.scan, sm.misc);
  const uint32_t bk0 = sm.misc[0];
  const uint32_t above0 = sm.misc[1];
  if (REGS > 0) {
#pragma unroll
    for (int u = 0; u < REGS; ++u)
      if (tid + static_cast<int64_t>(u) * NT >= V) rv[u] = -INFINITY;
  }
  // One classification of the row against bucket bk of the digit at
  // `shift`: sure entries (higher buckets) to sm.sel, candidates to the LDS
  // list; with count_up, also the candidates in the upper half of the
  // bucket (misc[6]).
  auto classify = [&](int sh, uint32_t bk, bool count_up) __attribute__((always_inline)) {
    if (REGS > 0) {
      // The bucket test runs on the floats: bucket(v) > bk iff v >= hi and
      // bucket(v) == bk iff lo <= v < hi, with lo / hi the smallest floats
      // of buckets bk and bk + 1 (finite scores keep both proper floats).
      // Slots past V hold -inf, below every bucket of a finite score.
      // Count, one packed prefix sum, then write at the thread's positions;
      // only hits compute their key.  Packing: sure entries in the low 12
      // bits (fewer than k <= 4096 in the whole row), candidates above them
      // (at most V <= 32768).
      const float lo = key_floor_float(bk << sh);
      const float hi = key_floor_float((bk + 1u) << sh);
      const float mid = key_floor_float(((2u * bk + 1u) << (sh - 1)));
      uint32_t ns = 0, nc = 0, nup = 0;
#pragma unroll
      for (int u = 0; u < REGS; ++u) {
        ns += rv[u] >= hi ? 1u : 0u;
        nc += rv[u] >= lo ? 1u : 0u;
        nup += rv[u] >= mid ? 1u : 0u;
      }
      nup -= ns;
      nc -= ns;
      if (count_up) {
        for (int o = 1; o < 64; o <<= 1) nup += __shfl_xor(nup, o);
        if ((tid & 63) == 0) atomicAdd(&sm.misc[6], nup);
      }
      const uint32_t packed = block_excl_scan<NT>(ns | (nc << 12), sm.scan);
      uint32_t ps = packed & 0xfffu, pcand = packed >> 12;
      if (tid == NT - 1) sm.misc[5] = pcand + nc;  // total candidates
#pragma unroll
      for (int u = 0; u < REGS; ++u) {
        if (rv[u] >= lo) {
          const int32_t j = tid + u * NT;
          if (rv[u] >= hi) {
            if (ps < static_cast<uint32_t>(kMaxK)) sm.sel[ps] = j;
            ++ps;
          } else {
            if (pcand < static_cast<uint32_t>(SM::kCand)) {
              sm.ckey[pcand] = score_key(rv[u]);
              sm.cidx[pcand] = j;
            }
            ++pcand;
          }
        }
      }
      if (tid == NT - 1) sm.misc[4] = ps;  // sure entries (== above)
    } else {
      // The same float bucket tests batch by batch: each thread counts its
      // batch's sure entries and candidates and takes its slots in the two
      // lists with one atomic each (wave-aggregated: one LDS atomic per wave
      // and list per batch), then writes; the lists' order is free (the
      // output is sorted through the row bitmap, the cut is order-free).
      const float lo = key_floor_float(bk << sh);
      const float hi = key_floor_float((bk + 1u) << sh);
      const float mid = key_floor_float(((2u * bk + 1u) << (sh - 1)));
      uint32_t nup = 0;  // entries at or above mid, less the sure ones
      constexpr int64_t kStep = static_cast<int64_t>(NT) * kRowBatch;
      // (the loads are unconditional: past the row's end a lane reads entry
      // V - 1, and its value is replaced; 32-bit indices, V < 2^31)
      // Full batches need no bounds: only the last one is clamped and masked.
      const int V32 = static_cast<int>(V);
      const __amdgpu_buffer_rsrc_t rs = store_rsrc(srow, V32 * 4);
      auto batch = [&](int64_t base, auto tail) __attribute__((always_inline)) {
        constexpr bool TAIL = decltype(tail)::value;
        const int j0 = static_cast<int>(base) + tid;
        float v[kRowBatch];
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) v[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, j0 * 4, u * NT * 4, 0));
        uint32_t ns = 0, nc = 0;
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
          if (TAIL && j0 + u * NT >= V32) v[u] = -INFINITY;  // below every finite bucket
          ns += v[u] >= hi ? 1u : 0u;
          nc += v[u] >= lo ? 1u : 0u;
          nup += v[u] >= mid ? 1u : 0u;
        }
        nc -= ns;
        nup -= ns;
        uint32_t ps = atomicAdd(&sm.misc[4], ns);
        uint32_t pc = atomicAdd(&sm.misc[5], nc);
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
          if (v[u] >= lo) {
            const int32_t j = j0 + u * NT;
            if (v[u] >= hi) {
              if (ps < static_cast<uint32_t>(kMaxK)) sm.sel[ps] = j;
              ++ps;
            } else {
              if (pc < static_cast<uint32_t>(SM::kCand)) {
                sm.ckey[pc] = score_key(v[u]);
                sm.cidx[pc] = j;
              }
              ++pc;
            }
          }
        }
      };
      int64_t base = 0;
      for (; base + kStep <= V; base += kStep) batch(base, std::false_type{});
      if (base < V) batch(base, std::true_type{});
      if (count_up) {
        for (int o = 1; o < 64; o <<= 1) nup += __shfl_xor(nup, o);
        if ((tid & 63) == 0) atomicAdd(&sm.misc[6], nup);
      }
    }
    __syncthreads();
  };
  classify(shift, bk0, use_coarse);
  uint32_t b1 = bk0, above = above0;
  uint32_t nc = sm.misc[5];
  if (use_coarse) {
    // the exact 12-bit bucket: the upper half of the coarse one when it
    // holds the k-th key
    const uint32_t n_up = sm.misc[6];
    const bool up = above0 + n_up >= static_cast<uint32_t>(k);
    b1 = 2u * bk0 + (up ? 1u : 0u);
    above = up ? above0 : above0 + n_up;
    if (nc <= static_cast<uint32_t>(SM::kCand)) {
      // narrow the LDS candidates to bucket b1 (in place: every thread
      // reads its run, then the barrier, then the kept ones are written
      // at their compacted positions); the other half is dropped or, when
      // the cut lies in the lower half, joins the sure entries
      constexpr int kRun = SM::kCand / NT;
      const uint32_t c0 = min(nc, static_cast<uint32_t>(tid * kRun));
      const uint32_t c1 = min(nc, c0 + kRun);
      uint32_t rk[kRun];
      int32_t rj[kRun];
      uint32_t kept = 0;
#pragma unroll
      for (int u = 0; u < kRun; ++u) {
        const uint32_t i = c0 + u;
        rk[u] = i < c1 ? sm.ckey[i] : 0u;
        rj[u] = i < c1 ? sm.cidx[i] : 0;
        kept += i < c1 && (rk[u] >> kTopkDigit1Shift) == b1 ? 1u : 0u;
      }
      uint32_t pos = block_excl_scan<NT>(kept, sm.scan);
      if (tid == NT - 1) sm.misc[5] = pos + kept;
#pragma unroll
      for (int u = 0; u < kRun; ++u) {
        if (c0 + u >= c1) continue;
        if ((rk[u] >> kTopkDigit1Shift) == b1) {
          sm.ckey[pos] = rk[u];
          sm.cidx[pos] = rj[u];
          ++pos;
        } else if (!up) {
          const uint32_t p = atomicAdd(&sm.misc[4], 1u);
          if (p < kMaxK) sm.sel[p] = rj[u];
        }
      }
      __syncthreads();
      nc = sm.misc[5];
    } else {
      // the coarse candidates did not fit: classify again, exactly
      if (tid < 8) sm.misc[tid] = 0u;
      __syncthreads();
      classify(kTopkDigit1Shift, b1, false);
      nc = sm.misc[5];
    }
  }
  finish_row<NT>(sm, srow, V, b1, static_cast<uint32_t>(k) - above, nc, k, out);
}

// ------------------------------------------------------------ split path
//
// Workspace per row: hist[4096] u32 (zero between calls; the indexer or
// topk_hist_kernel accumulates into it and the finishing kernel, or the
// attention launch that selects from the lists, clears it), ctrl[4] u32
// (first-digit bucket, count above it: written by classify before it is
// read; the finishing kernel clears it), then
// per 4096-entry slice: cnt[2] u32 (listed entries, candidates among them)
// and the slice's list lidx[4096] i32, lkey[4096] u32: every entry whose
// first digit is >= the row's bucket (the sure entries and the
// candidates), in entry order, with its key.  cnt and the lists are written
// before they are read in the same call.

struct SplitWs {
  uint32_t* hist;   // [rows][kHistBins]
  uint32_t* ctrl;   // [rows][4]
  uint32_t* cnt;    // [rows][n_sl][2]
  int32_t* lidx;    // [rows][n_sl][kSelEntries]
  uint32_t* lkey;   // [rows][n_sl][kSelEntries]
  int64_t n_sl;     // slices per row
};

// Rows of the split path hold at most this many slices (the finishing
// kernel keeps a 4-word record per slice in its bitmap area).
constexpr int64_t kMaxSlices = 2048;
static_assert(4 * kMaxSlices <= kBitmapMaxEntries / 32, "slice table must fit the bitmap area");

inline int64_t n_slices(int64_t n_cap) { return (n_cap + kSelEntries - 1) / kSelEntries; }

inline size_t split_ws_bytes(int64_t rows, int64_t n_cap) {
  const int64_t ns = n_slices(n_cap);
  return static_cast<size_t>(rows) *
         (sizeof(uint32_t) * (kHistBins + 4) +
          static_cast<size_t>(ns) * (sizeof(uint32_t) * 2 + sizeof(int32_t) * kSelEntries * 2));
}

inline SplitWs split_ws(void* base, int64_t rows, int64_t n_cap) {
  SplitWs w;
  w.n_sl = n_slices(n_cap);
  char* p = static_cast<char*>(base);
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * kHistBins * rows;
  w.ctrl = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * 4 * rows;
  w.cnt = reinterpret_cast<uint32_t*>(p);
  p += sizeof(uint32_t) * 2 * w.n_sl * rows;
  w.lidx = reinterpret_cast<int32_t*>(p);
  p += sizeof(int32_t) * kSelEntries * w.n_sl * rows;
  w.lkey = reinterpret_cast<uint32_t*>(p);
  return w;
}

// First-digit histogram of each row (when the indexer did not build it).
__global__ __launch_bounds__(kSelThreads) void topk_hist_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ pos0, int64_t T,
    int64_t n_cap, int m, int k, SplitWs ws) {
  __shared__ uint32_t hist[kHistBins];
  const int64_t row = blockIdx.y;
  const int64_t b = seq_of_row(row, T);
  const int64_t t = pos0[b] + (row - b * T);
  const int64_t V = uniform64(visible_entries(t, m, n_cap));
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

// Classify one 4096-entry slice of a row: entries above the bucket of the
// k-th largest key are "sure", entries in that bucket candidates.  The
// slice's scores and the row's histogram are loaded together; each thread
// keeps 16 consecutive bins (thread 0 the highest) and one block prefix sum
// of their totals gives the bucket.  Pass `it` of wave w covers the 64
// consecutive entries j0 + 256 it + 64 w + lane, so the slice's lists come
// out in ascending entry order from per-(pass, wave) ballot counts, one
// prefix sum over those 64 counts and each lane's rank in its ballot.  The
// list (sure entries and candidates together, with their keys) goes to the
// slice's own workspace region (no atomics) with its length and candidate
// count in cnt; slice 0 also records the bucket.
constexpr int kSelPer = kSelEntries / kSelThreads;   // 16 passes
constexpr int kHistPerSel = kHistBins / kSelThreads;  // 16 bins per thread
constexpr int kSelWaves = kSelThreads / 64;

struct ClassifyShared {
  uint32_t scan[32];
  uint32_t res[2];
  uint32_t tab[kSelPer * kSelWaves];  // (pass, wave) counts, sure | cand << 16
};

// The slice's histogram and score loads (issued by classify_load before
// the row's length is known: scores past the row's end are read from
// clamped, in-bounds addresses and never used).
struct ClassifyLoads {
  u32x4 hq[kHistPerSel / 4];
  float sv[kSelPer];
};

__device__ __forceinline__ void classify_load(ClassifyLoads& ld, const float* __restrict__ srow,
                                              int64_t row, int64_t j0, int64_t n_cap,
                                              const SplitWs& ws) {
  const int tid = threadIdx.x;
  // bins [kHistBins - 16 (tid + 1), kHistBins - 16 tid), 64-byte aligned
  const uint32_t* gh = ws.hist + row * kHistBins + (kHistBins - kHistPerSel * (tid + 1));
#pragma unroll
  for (int q = 0; q < kHistPerSel / 4; ++q) ld.hq[q] = reinterpret_cast<const u32x4*>(gh)[q];
#pragma unroll
  for (int it = 0; it < kSelPer; ++it) {
    const int64_t j = j0 + it * kSelThreads + tid;
    ld.sv[it] = srow[j < n_cap ? j : n_cap - 1];
  }
}

// Classify slice sl of row `row` (entries [j0, j1), j0 < V, V > k) from its
// loads: writes the slice's lists and counts and returns the bucket b1.
__device__ uint32_t classify_slice(ClassifyShared& cs, const ClassifyLoads& ld, int64_t row,
                                   int sl, int64_t j0, int64_t j1, int k, SplitWs ws) {
  uint32_t* scan = cs.scan;
  uint32_t* res = cs.res;
  uint32_t* tab = cs.tab;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const auto& hq = ld.hq;
  const auto& sv = ld.sv;
  uint32_t local = 0;
#pragma unroll
  for (int q = 0; q < kHistPerSel / 4; ++q) local += hq[q][0] + hq[q][1] + hq[q][2] + hq[q][3];
  const uint32_t excl = block_excl_scan<kSelThreads>(local, scan);
  const uint32_t r = static_cast<uint32_t>(k);
  if (excl < r && r <= excl + local) {
    uint32_t acc = excl;
#pragma unroll
    for (int q = kHistPerSel - 1; q >= 0; --q) {  // highest bin first
      const uint32_t c = hq[q >> 2][q & 3];
      if (acc < r && r <= acc + c) {
        res[0] = static_cast<uint32_t>(kHistBins - kHistPerSel * (tid + 1) + q);
        res[1] = acc;
      }
      acc += c;
    }
  }
  __syncthreads();
  const uint32_t b1 = res[0];
  // per (pass, wave) counts of listed entries (bucket >= b1) and of
  // candidates among them (bucket == b1); at most 64 of each, packed
#pragma unroll
  for (int it = 0; it < kSelPer; ++it) {
    const int64_t j = j0 + it * kSelThreads + tid;
    const uint32_t bk = score_key(sv[it]) >> kTopkDigit1Shift;
    const unsigned long long ml = __ballot(j < j1 && bk >= b1);
    const unsigned long long mc = __ballot(j < j1 && bk == b1);
    if (lane == 0)
      tab[it * kSelWaves + wv] =
          static_cast<uint32_t>(__popcll(ml)) | (static_cast<uint32_t>(__popcll(mc)) << 16);
  }
  __syncthreads();
  static_assert(kSelPer * kSelWaves == 64, "one wave scans the (pass, wave) table");
  if (wv == 0) {
    // exclusive prefix over the 64 entries in (pass, wave) order; totals fit
    // 16 bits each (<= 4096 per slice)
    const uint32_t c = tab[lane];
    uint32_t x = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    tab[lane] = x - c;
    if (lane == 63) {
      const int64_t slot = row * ws.n_sl + sl;
      ws.cnt[slot * 2] = x & 0xffffu;
      ws.cnt[slot * 2 + 1] = x >> 16;
      if (sl == 0) {
        ws.ctrl[row * 4] = b1;
        ws.ctrl[row * 4 + 1] = res[1];
      }
    }
  }
  __syncthreads();
  const int64_t slot = row * ws.n_sl + sl;
  int32_t* gi = ws.lidx + slot * kSelEntries;
  uint32_t* gk = ws.lkey + slot * kSelEntries;
#pragma unroll
  for (int it = 0; it < kSelPer; ++it) {
    const int64_t j = j0 + it * kSelThreads + tid;
    const uint32_t key = score_key(sv[it]);
    const bool listed = j < j1 && (key >> kTopkDigit1Shift) >= b1;
    const unsigned long long ml = __ballot(listed);
    if (listed) {
      const uint32_t pl = (tab[it * kSelWaves + wv] & 0xffffu) + lanes_below(ml);
      gi[pl] = static_cast<int32_t>(j);
      gk[pl] = key;
    }
  }
  return b1;
}

// xcd_rows > 0: a 1-D grid in XCD row order (the slices of a row share its
// histogram in one L2); else the grid is (slices, rows).
__global__ __launch_bounds__(kSelThreads) void topk_classify_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ pos0, int64_t T,
    int64_t n_cap, int m, int k, SplitWs ws, int64_t xcd_rows) {
  __shared__ ClassifyShared cs;
  int64_t row;
  int sl;
  if (xcd_rows > 0) {
    if (!xcd_row_item(blockIdx.x, static_cast<int>(ws.n_sl), xcd_rows, &row, &sl)) return;
  } else {
    row = blockIdx.y;
    sl = blockIdx.x;
  }
  const int64_t b = seq_of_row(row, T);
  const int64_t j0 = static_cast<int64_t>(sl) * kSelEntries;
  // the slice's loads go out before the row's position arrives
  ClassifyLoads ld;
  if (j0 < n_cap) classify_load(ld, scores + row * n_cap, row, j0, n_cap, ws);
  const int64_t t = pos0[b] + (row - b * T);
  const int64_t V = uniform64(visible_entries(t, m, n_cap));
  if (V <= k || j0 >= V) return;
  classify_slice(cs, ld, row, sl, j0, min(V, j0 + kSelEntries), k, ws);
}

static void launch_classify(const float* scores, const int64_t* pos0, int64_t T, int64_t n_cap,
                            int m, int k, const SplitWs& w, int64_t rows, hipStream_t s) {
  if (xcd_mappable(rows))
    launch_kernel(topk_classify_kernel, dim3(static_cast<unsigned>(xcd_grid_size(rows, w.n_sl))), kSelThreads, s, scores, pos0, T, n_cap, m, k, w, rows);
  else
    launch_kernel(topk_classify_kernel, dim3(static_cast<unsigned>(w.n_sl), static_cast<unsigned>(rows)), kSelThreads, s, scores, pos0, T, n_cap, m, k, w, 0);
}

// Resolve one row from its slices' lists and return its histogram and
// counters to zero.  The slice counts and a prefix of every slice's list
// (P entries each, P a power of two sized so that all of them take kFinPre
// loads per thread) are loaded together, before the row's position is
// known; the counts' prefix sum places the prefetched entries, and any
// entries past P are fetched afterwards.  The
// LDS list is then the row's sure entries and candidates in entry order:
// the cut among the candidates is found and one order-preserving
// compaction (sure entries and winning candidates) writes the output.  A
// list longer than the LDS buffer is finished as in the row path
// (candidates re-read from the scores, bitmap emit).
constexpr int kFinThreads = 1024;
constexpr int kFinPre = 8;  // prefetched list entries per thread
constexpr int kFinBatch = 8;  // loads in flight per thread for list entries past the prefix

__global__ __launch_bounds__(kFinThreads) void topk_finish_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ pos0, int64_t T,
    int64_t n_cap, int m, int k, SplitWs ws, int32_t* __restrict__ idx) {
  constexpr int NT = kFinThreads;
  __shared__ FinishShared sm;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t slot0 = row * ws.n_sl;
  const int n_alloc = static_cast<int>(ws.n_sl);  // slices per row in the workspace
  // Everything that does not depend on the row's length is loaded first:
  // the slice counts, a prefix of every slice's list (slot q = tid + NT i
  // is entry q % P of slice q / P; addresses clamped to the workspace's
  // slices, entries past a count unused), the bucket and the position.
  constexpr int kPer = static_cast<int>(kMaxSlices / NT);  // slices per thread
  uint32_t cl[kPer], cc[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int sl = tid * kPer + q;
    const int64_t sc = slot0 + (sl < n_alloc ? sl : n_alloc - 1);
    cl[q] = ws.cnt[sc * 2];
    cc[q] = ws.cnt[sc * 2 + 1];
  }
  int lp = 0;  // log2 P (P <= 512: lists are a few hundred entries long)
  while (lp < 9 && (n_alloc << (lp + 1)) <= NT * kFinPre) ++lp;
  int32_t pi[kFinPre];
  uint32_t pk[kFinPre];
#pragma unroll
  for (int i = 0; i < kFinPre; ++i) {
    const int q = tid + NT * i;
    const int sl = q >> lp;
    const int64_t at =
        (slot0 + (sl < n_alloc ? sl : n_alloc - 1)) * kSelEntries + (q & ((1 << lp) - 1));
    pi[i] = ws.lidx[at];
    pk[i] = ws.lkey[at];
  }
  const uint32_t b1 = ws.ctrl[row * 4];
  const int64_t b = seq_of_row(row, T);
  const int64_t t = pos0[b] + (row - b * T);
  const int64_t V = uniform64(visible_entries(t, m, n_cap));
  int32_t* out = idx + row * k;
  if (V <= k) {
    write_iota(out, V, k);
    return;
  }
  const float* srow = scores + row * n_cap;
  const int n_sl = static_cast<int>((V + kSelEntries - 1) / kSelEntries);

  uint32_t ll = 0, lc = 0, lmax = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    if (tid * kPer + q < n_sl) {
      ll += cl[q];
      lc += cc[q];
      lmax = max(lmax, cl[q]);
    }
  }
  uint32_t ol = block_excl_scan<NT>(ll, sm.scan);
  const uint32_t oc = block_excl_scan<NT>(lc, sm.scan);
  uint32_t* table = sm.bitmap;  // [slice][2]: list offset, list length
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int sl = tid * kPer + q;
    if (sl < n_sl) {
      table[sl * 2] = ol;
      table[sl * 2 + 1] = cl[q];
      ol += cl[q];
    }
  }
  if (tid == NT - 1) {
    sm.misc[4] = ol;       // listed entries
    sm.misc[5] = oc + lc;  // candidates among them
  }
  if (tid < 4) sm.misc[tid] = 0u;
  if (tid == 0) sm.misc[6] = sm.misc[7] = 0u;
  __syncthreads();
  if (lmax > (1u << lp)) sm.misc[6] = 1u;  // some list is longer than its prefix
  const uint32_t n_list = sm.misc[4], nc = sm.misc[5];
  const uint32_t ns = n_list - nc;                   // sure entries (fewer than k)
  const uint32_t r = static_cast<uint32_t>(k) - ns;  // winners needed among the candidates
  const bool fits = n_list <= static_cast<uint32_t>(kCandCap);
  if (fits) {
#pragma unroll
    for (int i = 0; i < kFinPre; ++i) {
      const int q = tid + NT * i;
      const int sl = q >> lp;
      const uint32_t pos = static_cast<uint32_t>(q & ((1 << lp) - 1));
      if (sl < n_sl && pos < table[sl * 2 + 1]) {
        const uint32_t at = table[sl * 2] + pos;
        sm.cidx[at] = pi[i];
        sm.ckey[at] = pk[i];
      }
    }
  }
  __syncthreads();
  if (fits && sm.misc[6] != 0u) {
    // entries past the prefixes: 2^lt threads per slice, kFinBatch loads
    // in flight per thread
    int lt = 0;
    while ((n_sl << (lt + 1)) <= NT) ++lt;
    const uint32_t step = 1u << lt;
    for (int base = 0; base < (n_sl << lt); base += NT) {
      const int q = base + tid;
      const int sl = q >> lt;
      if (sl < n_sl) {
        const uint32_t o = table[sl * 2], c = table[sl * 2 + 1];
        const int64_t g0 = (slot0 + sl) * kSelEntries;
        for (uint32_t p0 = (1u << lp) + static_cast<uint32_t>(q & (step - 1)); p0 < c;
             p0 += step * kFinBatch) {
          int32_t vi[kFinBatch];
          uint32_t vk[kFinBatch];
#pragma unroll
          for (int u = 0; u < kFinBatch; ++u) {
            const uint32_t pos = p0 + u * step;
            const int64_t at = g0 + (pos < c ? pos : c - 1);
            vi[u] = ws.lidx[at];
            vk[u] = ws.lkey[at];
          }
#pragma unroll
          for (int u = 0; u < kFinBatch; ++u) {
            const uint32_t pos = p0 + u * step;
            if (pos < c) {
              sm.cidx[o + pos] = vi[u];
              sm.ckey[o + pos] = vk[u];
            }
          }
        }
      }
    }
    __syncthreads();
  }
  if (!fits) {
    // the sure entries into sel (any order: the bitmap emit sorts), then
    // the row path's resolution from the scores
    for (int sl = 0; sl < n_sl; ++sl) {
      const uint32_t c = table[sl * 2 + 1];
      for (uint32_t pos = tid; pos < c; pos += NT) {
        const int64_t at = (slot0 + sl) * kSelEntries + pos;
        if ((ws.lkey[at] >> kTopkDigit1Shift) > b1) {
          const uint32_t p = atomicAdd(&sm.misc[7], 1u);
          if (p < static_cast<uint32_t>(kMaxK)) sm.sel[p] = ws.lidx[at];
        }
      }
    }
    __syncthreads();
    if (tid == 0) sm.misc[4] = ns;
    __syncthreads();
    // (the candidates are not in LDS: a count above kCandCap makes
    // finish_row read them from the scores)
    finish_row<NT>(sm, srow, V, b1, r, static_cast<uint32_t>(kCandCap) + 1u, k, out);
  } else {
    Cut c{0u, 0x7fffffff};  // r == nc: every candidate wins
    if (r < nc) {
      auto visit = [&](auto f) {
        for (uint32_t i = tid; i < n_list; i += NT) {
          const uint32_t key = sm.ckey[i];
          if ((key >> kTopkDigit1Shift) == b1) f(key, sm.cidx[i]);
        }
      };
      c = resolve_cut<NT>(sm, visit, r);
    }
    // sure entries and winning candidates, in entry order
    auto keep = [&](uint32_t i) {
      const uint32_t key = sm.ckey[i];
      return (key >> kTopkDigit1Shift) > b1 || r >= nc || cut_wins(c, key, sm.cidx[i]);
    };
    const uint32_t per = (n_list + NT - 1) / NT;
    const uint32_t i0 = min(n_list, tid * per), i1 = min(n_list, i0 + per);
    uint32_t cnt = 0;
    for (uint32_t i = i0; i < i1; ++i) cnt += keep(i) ? 1u : 0u;
    uint32_t pos = block_excl_scan<NT>(cnt, sm.scan);
    for (uint32_t i = i0; i < i1; ++i)
      if (keep(i)) {
        if (pos < static_cast<uint32_t>(k)) out[pos] = sm.cidx[i];
        ++pos;
      }
  }
  uint32_t* gh = ws.hist + row * kHistBins;
  for (int i = tid; i < kHistBins; i += NT) gh[i] = 0u;
  if (tid < 4) ws.ctrl[row * 4 + tid] = 0u;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0u;
}

// ----------------------------------------------------------------- host side

size_t topk_workspace_bytes(int64_t B, int64_t T, int64_t n_cap, int k) {
  (void)k;
  const int64_t rows = B * T;
  return rows <= kTopkSplitMaxRows
             ? split_ws_bytes(rows, n_cap)
             : static_cast<size_t>(rows) * (kTopkCoarseBins + 1) * sizeof(uint32_t);
}

CoarseHist topk_coarse_hist(void* ws, int64_t B, int64_t T) {
  const int64_t rows = B * T;
  if (rows <= kTopkSplitMaxRows || ws == nullptr) return CoarseHist{nullptr, nullptr};
  uint32_t* h = static_cast<uint32_t*>(ws);
  return CoarseHist{h, h + rows * kTopkCoarseBins};
}

size_t topk_zero_state_bytes(int64_t B, int64_t T) {
  // hist then ctrl lead the split workspace; the many-row one ends with the
  // coarse histograms' flags
  const int64_t rows = B * T;
  return rows <= kTopkSplitMaxRows
             ? static_cast<size_t>(rows) * (kHistBins + 4) * sizeof(uint32_t)
             : static_cast<size_t>(rows) * (kTopkCoarseBins + 1) * sizeof(uint32_t);
}

uint32_t* topk_hist_ptr(void* ws, int64_t B, int64_t T) {
  // the histogram leads the workspace whatever n_cap is
  return B * T <= kTopkSplitMaxRows ? static_cast<uint32_t*>(ws) : nullptr;
}

// One workgroup per row; rows that fit are held in registers.
static void launch_row_kernel(const float* scores, const int64_t* pos0, int64_t T, int64_t n_cap,
                              int m, int k, int32_t* idx, uint32_t* hist, const CoarseHist& ch,
                              int64_t rows, hipStream_t s) {
  const unsigned g = static_cast<unsigned>(rows);
  // register rows of up to 512 x 32 entries also run two 512-thread
  // workgroups per CU; up to 1024 x 32, one 1024-thread workgroup
  const bool regs = n_cap <= static_cast<int64_t>(kRowThreads) * kRowRegs;
  const bool regs_small = n_cap <= static_cast<int64_t>(kRowBatchedThreads) * kRowRegs;
#define CSA_ROW_GO(R, C, NT) \
  launch_kernel(topk_row_kernel<R, C, NT>, g, NT, s, scores, pos0, T, n_cap, m, k, idx, hist, ch)
#define CSA_ROW_CASE(C)                                                  \
  do {                                                                   \
    if (regs_small) CSA_ROW_GO(kRowRegs, C, kRowBatchedThreads);         \
    else if (regs) CSA_ROW_GO(kRowRegs, C, kRowThreads);                 \
    else CSA_ROW_GO(0, C, kRowBatchedThreads);                           \
  } while (0)
  if (ch.flag) CSA_ROW_CASE(true);
  else CSA_ROW_CASE(false);
#undef CSA_ROW_CASE
#undef CSA_ROW_GO
}

int launch_topk(const float* scores, const int64_t* pos0, int64_t B, int64_t T, int64_t n_cap,
                int m, int k, int32_t* idx, void* ws, bool hist_ready, hipStream_t s) {
  const int64_t rows = B * T;
  if (rows <= kTopkSplitMaxRows && n_cap > kRowSplitMinEntries &&
      n_slices(n_cap) <= kMaxSlices) {
    // few long rows: many workgroups per row classify slices, one per row
    // finishes
    SplitWs w = split_ws(ws, rows, n_cap);
    dim3 grid(static_cast<unsigned>(w.n_sl), static_cast<unsigned>(rows));
    if (!hist_ready) launch_kernel(topk_hist_kernel, grid, kSelThreads, s, scores, pos0, T, n_cap, m, k, w);
    launch_classify(scores, pos0, T, n_cap, m, k, w, rows, s);
    launch_kernel(topk_finish_kernel, static_cast<unsigned>(rows), kFinThreads, s, scores, pos0, T, n_cap,
                                                                           m, k, w, idx);
  } else {
    // one workgroup per row, using the indexer's histogram when it built
    // one (the coarse ones are checked, and their flags cleared, per row)
    uint32_t* h = rows <= kTopkSplitMaxRows && hist_ready ? static_cast<uint32_t*>(ws) : nullptr;
    launch_row_kernel(scores, pos0, T, n_cap, m, k, idx, h, topk_coarse_hist(ws, B, T), rows, s);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_topk_lists(const float* scores, const int64_t* pos0, int64_t B, int64_t T,
                      int64_t n_cap, int m, int k, void* ws, bool hist_ready, TopkLists* lists,
                      hipStream_t s) {
  const int64_t rows = B * T;
  if (!(rows <= kTopkSplitMaxRows && n_cap > kRowSplitMinEntries &&
        n_slices(n_cap) <= kSelMaxSlices))
    return 1;
  SplitWs w = split_ws(ws, rows, n_cap);
  dim3 grid(static_cast<unsigned>(w.n_sl), static_cast<unsigned>(rows));
  if (!hist_ready) launch_kernel(topk_hist_kernel, grid, kSelThreads, s, scores, pos0, T, n_cap, m, k, w);
  // rows that fit the attention workgroup's registers need no lists
  lists->regs = n_cap <= kSelRegEntries && n_cap % 4 == 0 &&
                (reinterpret_cast<uintptr_t>(scores) & 15u) == 0;
  lists->scores = scores;
  if (!lists->regs) launch_classify(scores, pos0, T, n_cap, m, k, w, rows, s);
  lists->cnt = w.cnt;
  lists->lidx = w.lidx;
  lists->lkey = w.lkey;
  lists->ctrl = w.ctrl;
  lists->hist = w.hist;
  lists->n_sl = w.n_sl;
  lists->m = m;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_clear(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(bytes / 4);
  if (n == 0) return 0;
  const int64_t blocks = (n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048;
  launch_kernel(fill_zero_kernel, static_cast<unsigned>(blocks), 256, s, static_cast<uint32_t*>(p), n);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
