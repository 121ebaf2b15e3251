// Core attention over selected compressed entries plus the sliding window
// (octagono.org "Hybrid Attention: CSA and HCA": attend only to the
// selected entries, with a window of recent tokens for local context;
// dataforcee.us "Hybrid Attention: CSA and HCA": both CSA and HCA carry the
// window branch; HCA attends densely to every compressed entry,
// "DeepSeek V4 technical review" section 2.2).
//
// One query token per workgroup row; every query head shares the single KV
// head, so the gathered key/value rows are staged in LDS once and used by
// all heads.  Eight waves: four tiles of 16 heads times the two 32-key
// halves of each chunk, so two waves share a SIMD and one's softmax hides
// the other's MFMA and LDS latency; each wave keeps its own softmax state
// for its half, and the halves of a head are combined once at the end.  The logical key list of a query is
//   slots [0, n_entries)            -> compressed entry (idx list or 0..V-1)
//   slots [n_entries, n_entries+W)  -> raw window position t-W+1+w
// and is cut into 64-key chunks; long lists are split over several
// workgroups whose (max, sum, O) partials are merged in a fixed order.
//
// MFMA orientation: S^T = K . Q^T puts keys on rows and heads on columns,
// so each lane ends up holding the probabilities of its own head for 4 keys
// per tile -- exactly the B operand layout of O^T = V^T . P^T (the key order
// inside the reduction is free as long as V^T uses the same one).  K and V
// are both staged row-major ([key][dim]) in LDS; the bf16 V^T operand is
// read with the LDS transpose read (4 keys x 4 dims per 4 lanes), and the
// fp32 one (one key per lane group) needs no transpose.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "select.h"

namespace csa {

constexpr int kAttChunk = 64;  // keys per LDS chunk
constexpr int kAttThreads = 512;  // 8 waves: 4 head tiles x 2 key halves
// Grids of at least this many workgroups (two per CU of the 256) take the
// two-per-CU build where it exists.
constexpr int64_t kAttWideGroups = 512;
// CSA: a split's slice of the top-k list is staged in LDS, so a split spans
// at most this many chunks.
constexpr int kAttMaxSplitChunks = 32;
constexpr int kMergeMaxSplits = 64;  // most partials per row (bounds the workspace)
constexpr float kLog2e = 1.4426950408889634f;
// The running softmax reference only moves up when a chunk's maximum exceeds
// it by more than this (log2 domain), so probabilities stay <= 2^8 and the
// accumulators are rescaled only on the rare large jumps; the final
// normalisation makes the result independent of the reference.
constexpr float kAttMaxSlack = 8.0f;

template <int DTYPE, int D>
struct AttTraits;

// LDS row strides (bytes): K rows are read 16 rows x 16 bytes at a time
// (stride = 4 banks mod 64); bf16 V rows are read 8 rows x 32 bytes per half
// wave by the transpose read (stride = 8 banks mod 64), fp32 V rows 4 rows x
// 64 bytes (stride = 4 banks mod 64).
template <int D>
struct AttTraits<0, D> {  // fp32 storage, v_mfma_f32_16x16x4_f32
  static constexpr int kElem = 4;
  static constexpr int kRowBytes = D * 4;
  static constexpr int kKSteps = D / 4;       // QK steps (1 element per lane)
  static constexpr int kVsStride = kRowBytes + 16;
};

template <int D>
struct AttTraits<1, D> {  // bf16 storage, v_mfma_f32_16x16x32_bf16
  static constexpr int kElem = 2;
  static constexpr int kRowBytes = D * 2;
  static constexpr int kKSteps = D / 32;
  static constexpr int kVsStride = kRowBytes + 32;
};

struct AttParams {
  const uint8_t* q;
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* idx;
  const uint8_t* kr;
  const uint8_t* vr;
  const int64_t* raw_pos0;
  const int64_t* pos0;
  float* out;
  float* lse;
  float* po;  // partial O   [rows][splits][H][D]
  float* pm;  // partial max [rows][splits][H] (log2 domain)
  float* pl;  // partial sum [rows][splits][H]
  int64_t T, H, n_cap, R;
  int k, W, m;
  int splits, chunks_per_split;
  int64_t xcd_rows;  // > 0: 1-D grid in XCD row order (xcd_row_item), else (splits, rows)
  float scale_log2;  // scale * log2(e)
  TopkLists sel;     // the selection's lists or scores (SEL variants)
  uint32_t* hist_zero;  // [rows][kTopkHistBins] histograms the merge launch zeroes, or NULL
};

// ---- the top-k selection made inside the launch from lists (CSA, SEL 1)
//
// Every workgroup of a row reads the row's classified lists (sure entries
// and candidates, a few thousand entries for decode rows) into LDS, finds
// the cut among the candidates, and keeps the slots of the sorted
// selection that its split attends; each split writes its own range of the
// index output, and split 0 returns the row's first-digit histogram
// (consumed by the classify launch) to zero.  The selection is the one the
// top-k finishing kernel makes: the r best candidates by (key, lower index
// first).  A histogram of the candidates' second digit gives the cut's
// 20-bit prefix, and the few candidates sharing it (at most 64) are ranked
// by all waves; more go through the general digit passes, and lists longer
// than the LDS space are read from global memory (only with very many
// ties).
struct AttSelShared {
  uint32_t hist[2048];  // digit passes; the packed candidates on the ranking path
  uint32_t scan[32];
  uint32_t misc[8];
  uint64_t scan64[8];
  uint32_t table[2 * kSelMaxSlices];  // per slice: list offset, length
};
constexpr int kAttSelPre = 8;    // prefetched list entries per thread
constexpr int kAttSelBatch = 8;  // loads in flight per thread past the prefix

// Exclusive prefix sum of v over the workgroup, and its total, with one
// barrier: per-wave scans, the wave totals through sm[0 .. NT / 64), each
// thread adding those of the waves before its own.  sm must not be written
// again before the caller's next barrier.
template <int NT, typename U>
__device__ __forceinline__ U block_scan_1b(U v, U* sm, U* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  U x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const U y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sm[wv] = x;
  __syncthreads();
  U base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const U c = sm[w];
    base += w < wv ? c : U(0);
    tot += c;
  }
  *total = tot;
  return base + x - v;
}

template <int NT, int CAP>
__device__ __forceinline__ void attend_select(const TopkLists& sel, int64_t row, int64_t t,
                                              int64_t n_cap, int k, int64_t s_begin,
                                              int64_t s_end, int split, int32_t* s_ent,
                                              uint32_t* ck, int32_t* ci, AttSelShared& ss) {
  static_assert(NT >= kSelMaxSlices, "one slice count per thread");
  constexpr int kEnt = 4096;  // entries per classified slice
  const int tid = threadIdx.x;
  const int64_t slot0 = row * sel.n_sl;
  const int n_alloc = static_cast<int>(sel.n_sl);
  // Loaded before the row's length is known: the slice counts, a prefix of
  // every slice's list (P entries each, slot q = tid + NT i is entry q % P
  // of slice q / P; slices clamped to the workspace's), the bucket.
  const int64_t my_slot = slot0 + (tid < n_alloc ? tid : n_alloc - 1);
  const uint32_t cl0 = sel.cnt[my_slot * 2];
  const uint32_t cc0 = sel.cnt[my_slot * 2 + 1];
  int lp = 0;
  while (lp < 9 && (n_alloc << (lp + 1)) <= NT * kAttSelPre) ++lp;
  int32_t pi[kAttSelPre];
  uint32_t pk[kAttSelPre];
#pragma unroll
  for (int i = 0; i < kAttSelPre; ++i) {
    const int q = tid + NT * i;
    const int sl = q >> lp;
    const int64_t at = (slot0 + (sl < n_alloc ? sl : n_alloc - 1)) * kEnt + (q & ((1 << lp) - 1));
    pi[i] = sel.lidx[at];
    pk[i] = sel.lkey[at];
  }
  const uint32_t b1 = sel.ctrl[row * 4];
  const int64_t V = uniform64(visible_entries(t, sel.m, n_cap));
  int32_t* out = sel.idx + row * k;
  if (split == 0)
    for (int i = tid; i < kTopkHistBins; i += NT) sel.hist[row * kTopkHistBins + i] = 0u;
  if (V <= k) {  // every visible entry, then -1
    for (int64_t i = s_begin + tid; i < s_end; i += NT) {
      const int32_t e = i < V ? static_cast<int32_t>(i) : -1;
      s_ent[i - s_begin] = e;
      out[i] = e;
    }
    return;
  }
  // list offsets of the slices (listed and candidate counts in one scan)
  const int n_sl = static_cast<int>((V + kEnt - 1) / kEnt);
  const uint32_t cl = tid < n_sl ? cl0 : 0u, cc = tid < n_sl ? cc0 : 0u;
  uint64_t tot;
  const uint64_t ex = block_scan_1b<NT>(static_cast<uint64_t>(cl) | (static_cast<uint64_t>(cc) << 32),
                                        ss.scan64, &tot);
  const uint32_t n_list = static_cast<uint32_t>(tot), nc = static_cast<uint32_t>(tot >> 32);
  if (tid < n_sl) {
    ss.table[2 * tid] = static_cast<uint32_t>(ex);
    ss.table[2 * tid + 1] = cl;
  }
  const bool more = __syncthreads_or(tid < n_sl && cl > (1u << lp));  // a list past its prefix
  const uint32_t r = static_cast<uint32_t>(k) - (n_list - nc);  // winners among candidates
  const bool fits = n_list <= static_cast<uint32_t>(CAP);
  if (fits) {
#pragma unroll
    for (int i = 0; i < kAttSelPre; ++i) {
      const int q = tid + NT * i;
      const int sl = q >> lp;
      const uint32_t pos = static_cast<uint32_t>(q & ((1 << lp) - 1));
      if (sl < n_sl && pos < ss.table[2 * sl + 1]) {
        const uint32_t at = ss.table[2 * sl] + pos;
        ck[at] = pk[i];
        ci[at] = pi[i];
      }
    }
    if (more) {
      // entries past the prefixes: 2^lt threads per slice, kAttSelBatch
      // loads in flight per thread
      int lt = 0;
      while ((n_sl << (lt + 1)) <= NT) ++lt;
      const uint32_t step = 1u << lt;
      for (int base = 0; base < (n_sl << lt); base += NT) {
        const int q = base + tid;
        const int sl = q >> lt;
        if (sl < n_sl) {
          const uint32_t o = ss.table[2 * sl], c = ss.table[2 * sl + 1];
          const int64_t g0 = (slot0 + sl) * kEnt;
          for (uint32_t p0 = (1u << lp) + static_cast<uint32_t>(q & (step - 1)); p0 < c;
               p0 += step * kAttSelBatch) {
            int32_t vi[kAttSelBatch];
            uint32_t vk[kAttSelBatch];
#pragma unroll
            for (int u = 0; u < kAttSelBatch; ++u) {
              const uint32_t pos = p0 + u * step;
              const int64_t at = g0 + (pos < c ? pos : c - 1);
              vi[u] = sel.lidx[at];
              vk[u] = sel.lkey[at];
            }
#pragma unroll
            for (int u = 0; u < kAttSelBatch; ++u) {
              const uint32_t pos = p0 + u * step;
              if (pos < c) {
                ck[o + pos] = vk[u];
                ci[o + pos] = vi[u];
              }
            }
          }
        }
      }
    }
  }
  // second-digit histogram of the candidates (key bits 19..10), cleared
  // before the barrier that publishes the list; bin b at word b + b / 16,
  // so the 16 consecutive bins each lane reads below sit 17 words from the
  // next lane's (no bank conflicts)
  uint32_t* h2 = ss.hist;
  auto h2_at = [](uint32_t b) __attribute__((always_inline)) { return b + (b >> 4); };
  uint64_t* tmp = reinterpret_cast<uint64_t*>(h2 + 1152);  // 64 prefix candidates
  uint32_t* rank = h2 + 1280;                               // their ranks
  for (int i = tid; i < 1344; i += NT) h2[i] = 0u;
  if (tid == 0) ss.misc[6] = 0u;  // candidates collected at the cut's prefix
  __syncthreads();  // the list is in LDS
  // list entry i (sure entries and candidates of all slices, in entry
  // order): from LDS, or found in its slice's global list
  auto entry = [&](uint32_t i, uint32_t& key, int32_t& j) __attribute__((always_inline)) {
    if (fits) {
      key = ck[i];
      j = ci[i];
      return;
    }
    int lo = 0, hi = n_sl - 1;  // the last slice whose list starts at or before i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ss.table[2 * mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    const int64_t at = (slot0 + lo) * kEnt + (i - ss.table[2 * lo]);
    key = sel.lkey[at];
    j = sel.lidx[at];
  };
  // this thread's run of the list
  const uint32_t per = (n_list + NT - 1) / NT;
  const uint32_t i0 = min(n_list, tid * per), i1 = min(n_list, i0 + per);
  Cut c{0u, 0x7fffffff};  // r == nc: every candidate wins
  bool general = r < nc && !fits;
  if (r < nc && fits) {
    // a histogram of the candidates' second digits gives the 20-bit prefix
    // of the cut; the few candidates that share it are ranked by all waves
    for (uint32_t i = i0; i < i1; ++i) {
      const uint32_t key = ck[i];
      if ((key >> kTopkDigit1Shift) == b1) atomicAdd(&h2[h2_at((key >> 10) & 1023u)], 1u);
    }
    __syncthreads();
    // every wave finds the bucket b2 of the r-th best candidate's second
    // digit (lane l holds bins 1023 - 16 l - q, q = 0..15, highest first)
    const int lane = tid & 63;
    uint32_t hb[16];
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      hb[q] = h2[h2_at(1023u - 16u * lane - q)];
      sum += hb[q];
    }
    uint32_t incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const uint32_t excl = incl - sum;
    const bool mine = excl < r && r <= incl;
    uint32_t b2 = 0, above = 0;
    if (mine) {
      uint32_t acc = excl;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (acc < r && r <= acc + hb[q]) {
          b2 = 1023u - 16u * lane - q;
          above = acc;
        }
        acc += hb[q];
      }
    }
    const int owner = __ffsll(static_cast<long long>(__ballot(mine))) - 1;
    b2 = __shfl(b2, owner);
    above = __shfl(above, owner);
    const uint32_t n2 = h2[h2_at(b2)];
    general = n2 > 64u;  // too many share the cut's prefix: the digit passes
    if (!general) {
      // the n2 candidates with prefix (b1, b2), any order
      const uint32_t prefix = (b1 << 10) | b2;
      for (uint32_t i = i0; i < i1; ++i) {
        const uint32_t key = ck[i];
        if ((key >> 10) == prefix)
          tmp[atomicAdd(&ss.misc[6], 1u)] =
              (static_cast<uint64_t>(key & 0xfffffu) << 32) | static_cast<uint32_t>(ci[i]);
      }
    }
    __syncthreads();
    // their ranks by (key desc, index asc), every wave comparing all of
    // them with its share (LDS broadcast reads, all in flight at once)
    constexpr int NW = NT / 64;
    const int wvu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool have = !general && static_cast<uint32_t>(lane) < n2;
    const uint64_t v = tmp[lane];
    const uint32_t lo20 = static_cast<uint32_t>(v >> 32);
    const int32_t jj = static_cast<int32_t>(static_cast<uint32_t>(v));
    if (!general) {
      uint64_t u[64 / NW];
#pragma unroll
      for (int i = 0; i < 64 / NW; ++i) u[i] = tmp[wvu + NW * i];
      uint32_t part = 0;
#pragma unroll
      for (int i = 0; i < 64 / NW; ++i) {
        const uint32_t lo_q = static_cast<uint32_t>(u[i] >> 32);
        const int32_t j_q = static_cast<int32_t>(static_cast<uint32_t>(u[i]));
        const bool before = lo_q > lo20 || (lo_q == lo20 && j_q < jj);
        part += static_cast<uint32_t>(wvu + NW * i) < n2 && before ? 1u : 0u;
      }
      if (have && part) atomicAdd(&rank[lane], part);
    }
    __syncthreads();
    // the (r - above)-th of them is the cut (every wave finds it)
    const int who =
        __ffsll(static_cast<long long>(__ballot(have && rank[lane] == r - above - 1u))) - 1;
    c = Cut{static_cast<uint32_t>(__builtin_amdgcn_readlane(lo20, who & 63)),
            static_cast<int32_t>(__builtin_amdgcn_readlane(static_cast<uint32_t>(jj), who & 63))};
  }
  if (general) {
    auto visit = [&](auto f) {
      for (uint32_t i = tid; i < n_list; i += NT) {
        uint32_t key;
        int32_t j;
        entry(i, key, j);
        if ((key >> kTopkDigit1Shift) == b1) f(key, j);
      }
    };
    c = resolve_cut<NT>(ss, visit, r);
  }
  // sure entries and winning candidates in entry order: this split's
  // positions [s_begin, s_end) of the sorted list
  auto keep = [&](uint32_t key, int32_t j) __attribute__((always_inline)) {
    return (key >> kTopkDigit1Shift) > b1 || r >= nc || cut_wins(c, key, j);
  };
  uint32_t cnt = 0;
  for (uint32_t i = i0; i < i1; ++i) {
    uint32_t key;
    int32_t j;
    entry(i, key, j);
    cnt += keep(key, j) ? 1u : 0u;
  }
  uint32_t unused;
  int64_t pos = block_scan_1b<NT>(cnt, ss.scan + 8, &unused);
  for (uint32_t i = i0; i < i1 && pos < s_end; ++i) {
    uint32_t key;
    int32_t j;
    entry(i, key, j);
    if (keep(key, j)) {
      if (pos >= s_begin) {
        s_ent[pos - s_begin] = j;
        out[pos] = j;
      }
      ++pos;
    }
  }
}

// ---- the top-k selection from the row's scores held in registers (SEL 2)
//
// For rows of at most kSelRegEntries entries no classify launch precedes
// the attention: every workgroup of the row loads the row's first-digit
// histogram (8 bins per thread, thread 0 the highest) and then the whole
// row of scores (64 per thread: float4 q of wave w covers entries 4096 w +
// 256 q + 4 lane .. + 3).  One block scan of the bin totals gives the
// bucket b1 of the k-th key, the count above it and the number nc of
// candidates (first digit b1).  Every workgroup of a row redoes this work,
// and with two waves per SIMD each instruction of it costs the workgroup
// about 8 cycles, so the pass over the registers is one max and one
// compare per float4 against the bucket's lower bound (slots past V hold
// -inf; finite scores assumed, as in the row top-k): a float4 holding a
// listed score (in bucket b1 or above) goes, with its first entry number,
// to its wave's region of an LDS group list (slot numbered by ballot).
// Each wave then splits its own groups' listed scores, without a barrier:
// sure entries (above b1) are set in an LDS bitmap of the row in entry
// order, candidates go with their keys to the wave's region of a candidate
// list (numbered by ballot) while their second digits are counted.  The
// cut among the candidates is found (the 20-bit prefix from that
// histogram, the few candidates sharing it ranked by all waves, else the
// general digit passes) and the winners are set in the bitmap.  Each
// thread then owns 64 consecutive bits of it: one block scan of their
// counts numbers the kept entries in entry order, and each split keeps,
// and writes out, the slots it attends.  A wave region that overflows
// (clustered scores) sends the selection to passes over the scores in
// memory.  The row's histogram goes back to zero in the merge launch, or
// here when the row has one split (each thread clears the bins it read).
constexpr int kAttSelRegs = 64;     // scores per thread
constexpr int kAttSelGroups = 384;  // listed float4 groups per wave region
static_assert(kAttThreads * kAttSelRegs == kSelRegEntries, "a row's scores fill the registers");
static_assert(kAttThreads * 8 == kTopkHistBins, "8 histogram bins per thread");

// The entries of float4 q of a thread: e0 + 256 q + 0..3.
__device__ __forceinline__ f32x4 sel_regs_load(const float* srow, int64_t n_cap, int e0, int q) {
  const int64_t e = e0 + 256 * q;
  return *reinterpret_cast<const f32x4*>(srow + (e + 4 <= n_cap ? e : n_cap - 4));
}

template <int NT>
__device__ __forceinline__ void attend_select_regs(const TopkLists& sel, int64_t row, int64_t t,
                                                   int64_t n_cap, int k, int64_t s_begin,
                                                   int64_t s_end, bool zero_hist,
                                                   int32_t* s_ent, AttSelShared& ss, f32x4* gx,
                                                   uint32_t* gj, uint32_t* kept, uint32_t* lst,
                                                   int lwcap) {
  constexpr int kQ = kAttSelRegs / 4;  // float4 loads per thread
  constexpr int NW = NT / 64;
  constexpr int gcap = kAttSelGroups;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int e0 = wv * (64 * kAttSelRegs) + 4 * lane;
  const float* srow = sel.scores + row * n_cap;
  // the histogram first: loads complete in order, so the bucket is found
  // while the scores are still arriving
  u32x4* gh = reinterpret_cast<u32x4*>(sel.hist + row * kTopkHistBins +
                                       (kTopkHistBins - 8 * (tid + 1)));
  const u32x4 h0 = gh[0], h1 = gh[1];  // bins base .. base + 7
  f32x4 sv[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) sv[q] = sel_regs_load(srow, n_cap, e0, q);
  // second-digit histogram (bin b at word b + b / 16: the 16 consecutive
  // bins each lane reads below sit 17 words from the next lane's), the
  // prefix candidates' counter and ranks, the overflow flag and the kept
  // bitmap (entry j at bit j % 32 of word j / 32), cleared before the first
  // barrier
  uint32_t* h2 = ss.hist;
  auto h2_at = [](uint32_t b) __attribute__((always_inline)) { return b + (b >> 4); };
  uint64_t* tmp = reinterpret_cast<uint64_t*>(h2 + 1152);  // 64 prefix candidates
  uint32_t* rank = h2 + 1280;                               // their ranks
  for (int i = tid; i < 1344; i += NT) h2[i] = 0u;
  for (int i = tid; i < kSelRegEntries / 32; i += NT) kept[i] = 0u;
  if (tid == 0) ss.misc[5] = ss.misc[6] = 0u;
  const uint32_t hb[8] = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) local += hb[i];
  const uint32_t kk = static_cast<uint32_t>(k);
  uint32_t total;
  const uint32_t excl = block_scan_1b<NT>(local, ss.scan, &total);
  if (excl < kk && kk <= excl + local) {
    uint32_t acc = excl;
#pragma unroll
    for (int i = 7; i >= 0; --i) {  // highest bin first
      if (acc < kk && kk <= acc + hb[i]) {
        ss.misc[0] = static_cast<uint32_t>(kTopkHistBins - 8 * (tid + 1) + i);
        ss.misc[1] = acc;
        ss.misc[4] = hb[i];
      }
      acc += hb[i];
    }
  }
  // the bins were summed above, so their loads are complete
  if (zero_hist) gh[0] = gh[1] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  const int64_t V = uniform64(visible_entries(t, sel.m, n_cap));
  int32_t* out = sel.idx + row * k;
  if (V <= k) {  // every visible entry, then -1
    for (int64_t i = s_begin + tid; i < s_end; i += NT) {
      const int32_t e = i < V ? static_cast<int32_t>(i) : -1;
      s_ent[i - s_begin] = e;
      out[i] = e;
    }
    return;
  }
  const int V32 = static_cast<int>(V);  // V <= n_cap <= kSelRegEntries
  const uint32_t b1 = ss.misc[0];
  const uint32_t nc = ss.misc[4];
  const uint32_t r = kk - ss.misc[1];  // winners among the candidates
  const bool all_win = r >= nc;
  // bucket(v) > b1 iff v >= hi, bucket(v) == b1 iff lo <= v < hi (finite
  // scores; hi is NaN for the top bucket, which nothing is above)
  const float lo = key_floor_float(b1 << kTopkDigit1Shift);
  const float hi = key_floor_float((b1 + 1u) << kTopkDigit1Shift);
  auto set_kept = [&](int j) __attribute__((always_inline)) {
    atomicOr(&kept[j >> 5], 1u << (j & 31));
  };
  // the pass over the registers: float4 groups holding a listed score
  f32x4* wgx = gx + wvu * gcap;
  uint32_t* wgj = gj + wvu * gcap;
  uint32_t gcount = 0;  // this wave's groups (wave-uniform)
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    f32x4 x = sv[q];
    if (wvu * (64 * kAttSelRegs) + 256 * (q + 1) > V32) {  // part of this group lies past V
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e0 + 256 * q + e >= V32) x[e] = -INFINITY;
    }
    const bool listed = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])) >= lo;
    const unsigned long long m = __ballot(listed);
    if (listed) {
      const uint32_t at = gcount + lanes_below(m);
      if (at < static_cast<uint32_t>(gcap)) {
        wgx[at] = x;
        wgj[at] = static_cast<uint32_t>(e0 + 256 * q);
      }
    }
    gcount += static_cast<uint32_t>(__popcll(m));
  }
  // this wave's groups: sure entries into the bitmap, candidates into the
  // wave's list region and the second-digit histogram
  uint32_t* lkey = lst + wvu * lwcap;
  int32_t* lidx = reinterpret_cast<int32_t*>(lst + NW * lwcap) + wvu * lwcap;
  uint32_t lcount = 0;  // this wave's candidates (wave-uniform)
  const uint32_t gn = min(gcount, static_cast<uint32_t>(gcap));
  for (uint32_t g0 = 0; g0 < gn; g0 += 64) {
    const uint32_t g = g0 + lane;
    const bool have = g < gn;
    const f32x4 x = wgx[have ? g : 0];
    const int j0 = static_cast<int>(wgj[have ? g : 0]);
    uint32_t sn = 0, cn = 0;  // sure and candidate entries of the group
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool su = x[e] >= hi;
      sn |= su ? 1u << e : 0u;
      cn |= !su && x[e] >= lo ? 1u << e : 0u;
    }
    if (!have) sn = cn = 0u;
    if (all_win) {
      sn |= cn;
      cn = 0u;
    }
    // the group's 4 entries share a bitmap word
    if (sn) atomicOr(&kept[j0 >> 5], sn << (j0 & 31));
    // the lane's candidates at the wave's next slots (a prefix over the
    // lanes of counts 0..4, from their three bits)
    const uint32_t nl = static_cast<uint32_t>(__popc(cn));
    const unsigned long long c0 = __ballot(nl & 1u), c1 = __ballot(nl & 2u),
                             c2 = __ballot(nl & 4u);
    uint32_t at = lcount + lanes_below(c0) + 2u * lanes_below(c1) + 4u * lanes_below(c2);
    lcount += static_cast<uint32_t>(__popcll(c0) + 2 * __popcll(c1) + 4 * __popcll(c2));
    while (cn) {
      const int e = __builtin_ctz(cn);
      cn &= cn - 1u;
      const float v = e == 0 ? x[0] : e == 1 ? x[1] : e == 2 ? x[2] : x[3];
      const uint32_t ky = score_key(v);
      atomicAdd(&h2[h2_at((ky >> 10) & 1023u)], 1u);
      if (at < static_cast<uint32_t>(lwcap)) {
        lkey[at] = ky;
        lidx[at] = j0 + e;
      }
      ++at;
    }
  }
  if (lane == 0 && (gcount > static_cast<uint32_t>(gcap) || lcount > static_cast<uint32_t>(lwcap)))
    ss.misc[5] = 1u;  // a wave region overflowed
  __syncthreads();  // the bitmap's sure entries, the lists and the histogram
  if (ss.misc[5] == 0u) {
    if (!all_win) {
      // every wave finds the bucket b2 of the r-th best candidate's second
      // digit (lane l holds bins 1023 - 16 l - q, q = 0..15, highest first)
      uint32_t hq[16];
      uint32_t sum = 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        hq[q] = h2[h2_at(1023u - 16u * lane - q)];
        sum += hq[q];
      }
      uint32_t incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      const uint32_t ex2 = incl - sum;
      const bool mine = ex2 < r && r <= incl;
      uint32_t b2 = 0, above = 0;
      if (mine) {
        uint32_t acc = ex2;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          if (acc < r && r <= acc + hq[q]) {
            b2 = 1023u - 16u * lane - q;
            above = acc;
          }
          acc += hq[q];
        }
      }
      const int owner = __ffsll(static_cast<long long>(__ballot(mine))) - 1;
      b2 = __builtin_amdgcn_readlane(b2, owner & 63);
      above = __builtin_amdgcn_readlane(above, owner & 63);
      const uint32_t n2 = h2[h2_at(b2)];
      Cut c;
      if (n2 <= 64u) {
        const uint32_t prefix = (b1 << 10) | b2;
        for (uint32_t i = lane; i < lcount; i += 64) {
          const uint32_t ky = lkey[i];
          if ((ky >> 10) == prefix) {
            const uint32_t at = atomicAdd(&ss.misc[6], 1u);
            if (at < 64u)
              tmp[at] = (static_cast<uint64_t>(ky & 0xfffffu) << 32) |
                        static_cast<uint32_t>(lidx[i]);
          }
        }
        __syncthreads();
        // their ranks by (key desc, index asc), every wave comparing all of
        // them with its eighth (LDS broadcast reads, all in flight at once)
        const bool have = static_cast<uint32_t>(lane) < n2;
        const uint64_t v = tmp[lane];
        const uint32_t lo20 = static_cast<uint32_t>(v >> 32);
        const int32_t jj = static_cast<int32_t>(static_cast<uint32_t>(v));
        uint64_t u[64 / NW];
#pragma unroll
        for (int i = 0; i < 64 / NW; ++i) u[i] = tmp[wvu + NW * i];
        uint32_t part = 0;
#pragma unroll
        for (int i = 0; i < 64 / NW; ++i) {
          const uint32_t lo_q = static_cast<uint32_t>(u[i] >> 32);
          const int32_t j_q = static_cast<int32_t>(static_cast<uint32_t>(u[i]));
          const bool before = lo_q > lo20 || (lo_q == lo20 && j_q < jj);
          part += static_cast<uint32_t>(wvu + NW * i) < n2 && before ? 1u : 0u;
        }
        if (have && part) atomicAdd(&rank[lane], part);
        __syncthreads();
        // the (r - above)-th of them is the cut (every wave finds it)
        const int who =
            __ffsll(static_cast<long long>(__ballot(have && rank[lane] == r - above - 1u))) - 1;
        c = Cut{static_cast<uint32_t>(__builtin_amdgcn_readlane(lo20, who & 63)),
                static_cast<int32_t>(__builtin_amdgcn_readlane(static_cast<uint32_t>(jj),
                                                               who & 63))};
      } else {
        // every candidate, visited by the threads of the wave that listed it
        auto visit = [&](auto f) {
          for (uint32_t i = lane; i < lcount; i += 64) f(lkey[i], lidx[i]);
        };
        // (every wave took this branch; the digit passes clear the
        // histogram the others may still be reading)
        __syncthreads();
        c = resolve_cut<NT>(ss, visit, r);
      }
      // the winning candidates into the bitmap
      for (uint32_t i = lane; i < lcount; i += 64) {
        const int32_t j = lidx[i];
        if (cut_wins(c, lkey[i], j)) set_kept(j);
      }
    }
  } else {
    // a wave region overflowed: the same over the scores in memory
    auto visit_mem = [&](auto f) {
      for (int q = 0; q < kQ; ++q) {
        const f32x4 v = sel_regs_load(srow, n_cap, e0, q);
#pragma unroll
        for (int x = 0; x < 4; ++x)
          if (e0 + 256 * q + x < V32 && v[x] >= lo) f(v[x], e0 + 256 * q + x);
      }
    };
    Cut c{0u, 0x7fffffff};
    if (!all_win) {
      auto visit = [&](auto f) {
        visit_mem([&](float v, int j) {
          if (!(v >= hi)) f(score_key(v), j);
        });
      };
      c = resolve_cut<NT>(ss, visit, r);
    }
    visit_mem([&](float v, int j) {
      if (v >= hi || all_win || cut_wins(c, score_key(v), j)) set_kept(j);
    });
  }
  __syncthreads();  // the kept bitmap
  // thread t: entries 64 t .. 64 t + 63, numbered by one block scan
  uint64_t bits = kept[2 * tid] | (static_cast<uint64_t>(kept[2 * tid + 1]) << 32);
  uint32_t unused;
  int at = static_cast<int>(block_scan_1b<NT>(static_cast<uint32_t>(__popcll(bits)),
                                              ss.scan + 16, &unused));
  const int sb0 = static_cast<int>(s_begin), se0 = static_cast<int>(s_end);
  while (bits && at < se0) {
    const int i = __builtin_ctzll(bits);
    bits &= bits - 1;
    if (at >= sb0) {
      const int32_t j = 64 * tid + i;
      s_ent[at - sb0] = j;
      out[at] = j;
    }
    ++at;
  }
}

// SEL: 0 the selection is given (idx), 1 made from the classified lists,
// 2 made from the scores held in registers.
template <int DTYPE, int D, bool HCA, int SEL>
__device__ __forceinline__ void attend_body(const AttParams& p) {
  using Tr = AttTraits<DTYPE, D>;
  constexpr int RB = Tr::kRowBytes;
  constexpr int kPieces = RB / 16;             // 16-byte pieces per row
  constexpr int kPerThread = kAttChunk * kPieces / kAttThreads;
  static_assert(kPerThread >= 1 && kPerThread * kAttThreads == kAttChunk * kPieces,
                "a chunk must split evenly over the threads");
  constexpr int kKsStride = RB + 16;
  constexpr int kVsStride = Tr::kVsStride;
  // Two LDS buffers: chunk i+1 is staged into one while chunk i is computed
  // from the other, with one barrier per chunk.
  __shared__ __attribute__((aligned(16))) uint8_t ks[2][kAttChunk * kKsStride];
  __shared__ __attribute__((aligned(16))) uint8_t vs[2][kAttChunk * kVsStride];
  __shared__ int valid[2][kAttChunk];
  // 1 + (split-relative) index of the last chunk staged into the buffer that
  // had absent keys, so no flag ever has to be cleared
  __shared__ int s_partial[2];
  __shared__ int32_t s_ent[HCA ? 1 : kAttMaxSplitChunks * kAttChunk];
  // SEL 2: the float4 groups of listed scores, per wave region, in the K
  // buffers when they are large enough (fp32 rows), else in LDS of their own
  constexpr int kSelGroupSlots = kAttSelGroups * (kAttThreads / 64);
  constexpr bool kGroupsInKs = sizeof(ks) >= 20 * kSelGroupSlots;
  constexpr int kOwnSlots = SEL == 2 && !kGroupsInKs ? kSelGroupSlots : 1;
  __shared__ f32x4 s_gx[kOwnSlots];
  __shared__ uint32_t s_ginfo[kOwnSlots];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ht = wave & 3;  // head tile
  const int kh = wave >> 2;  // key half of every chunk
  const int col = lane & 15;
  const int g = lane >> 4;
  int64_t row;
  int split;
  if (p.xcd_rows > 0) {  // a row's splits on one XCD (shared q, lists)
    if (!xcd_row_item(blockIdx.x, p.splits, p.xcd_rows, &row, &split)) return;
  } else {
    row = blockIdx.y;
    split = blockIdx.x;
  }
  const int64_t b = seq_of_row(row, p.T);
  // both position loads are unconditional, so they are in flight together
  // (raw_pos0 may be NULL when W == 0; its value is then unused)
  const int64_t t = p.pos0[b] + (row - b * p.T);
  const int64_t rp0 = (p.W > 0 ? p.raw_pos0 : p.pos0)[b];
  // the register slots of the chunk gathers (see below)
  const uint8_t* kc_b = p.kc + b * p.n_cap * RB;
  const uint8_t* vc_b = p.vc + b * p.n_cap * RB;
  const int pc = tid % kPieces;
  const int key0 = tid / kPieces;
  struct Slot {
    u32x4 k[kPerThread], v[kPerThread];
    bool ok[kPerThread];
  };
  Slot ring0, ring1;
  auto pick = [&](auto slot) __attribute__((always_inline)) -> Slot& {
    if constexpr (decltype(slot)::value == 0) return ring0;
    else return ring1;
  };
  if constexpr (HCA) {
    // HCA: the split's first two chunks are loaded before the row's
    // position arrives, as if every slot were a visible entry (addresses
    // clamped into the cache, so always in bounds); kept when that holds
    // (spec_ok), which saves the position's round trip to memory
    const int64_t sc0 = static_cast<int64_t>(split) * p.chunks_per_split;
    auto spec = [&](Slot& S, int64_t chunk) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < kPerThread; ++r) {
        const int64_t e =
            min(chunk * kAttChunk + key0 + r * (kAttThreads / kPieces), p.n_cap - 1);
        S.ok[r] = true;
        S.k[r] = *reinterpret_cast<const u32x4*>(kc_b + e * RB + pc * 16);
        S.v[r] = *reinterpret_cast<const u32x4*>(vc_b + e * RB + pc * 16);
      }
    };
    spec(ring0, sc0);
    spec(ring1, sc0 + 1);
  }
  const int64_t n_ent =
      HCA ? uniform64(visible_entries(t, p.m, p.n_cap)) : static_cast<int64_t>(p.k);
  const int64_t n_slots = n_ent + p.W;
  const int64_t c_begin = static_cast<int64_t>(split) * p.chunks_per_split;
  const int64_t c_end = min(c_begin + p.chunks_per_split, (n_slots + kAttChunk - 1) / kAttChunk);
  const int n_ht = static_cast<int>((p.H + 15) >> 4);
  const bool has_heads = ht < n_ht;
  const int head = ht * 16 + col;

  // Q^T fragments: this lane's head, one contiguous quarter of the row.
  // Lanes past the last head load it again (unconditional loads); their
  // columns are never written out.
  constexpr int kQVec = RB / 4 / 16;
  u32x4 qf[kQVec];
  {
    const int64_t hq = head < p.H ? head : p.H - 1;
    const u32x4* src = reinterpret_cast<const u32x4*>(p.q + (row * p.H + hq) * RB + g * (RB / 4));
#pragma unroll
    for (int v = 0; v < kQVec; ++v) qf[v] = src[v];
  }

  // CSA: the split's slice of the top-k list is copied to LDS once, so the
  // gathers never wait on index loads.
  const int64_t s_begin = c_begin * kAttChunk;
  const int64_t idx_row = row * p.k;
  if constexpr (SEL == 2) {
    // the listed groups in the K buffers when they are large enough (fp32
    // rows; the candidate lists then after the shared state and the kept
    // bitmap in vs), else in LDS of their own (the lists in ks); ks and vs
    // are free until the first chunk is staged
    constexpr int kVsUsed = static_cast<int>(sizeof(AttSelShared)) + kSelRegEntries / 8;
    constexpr int kListBytes =
        kGroupsInKs ? static_cast<int>(sizeof(vs)) - kVsUsed : static_cast<int>(sizeof(ks));
    constexpr int kListWaveCap = kListBytes / (8 * (kAttThreads / 64));
    static_assert(kVsUsed <= static_cast<int>(sizeof(vs)) && kListWaveCap >= 256,
                  "selection LDS");
    attend_select_regs<kAttThreads>(
        p.sel, row, t, p.n_cap, p.k, s_begin, min(c_end * kAttChunk, n_ent), p.splits == 1,
        s_ent, *reinterpret_cast<AttSelShared*>(&vs[0][0]),
        kGroupsInKs ? reinterpret_cast<f32x4*>(&ks[0][0]) : s_gx,
        kGroupsInKs ? reinterpret_cast<uint32_t*>(&ks[0][0] + 16 * kSelGroupSlots) : s_ginfo,
        reinterpret_cast<uint32_t*>(&vs[0][0] + sizeof(AttSelShared)),
        reinterpret_cast<uint32_t*>(kGroupsInKs ? &vs[0][0] + kVsUsed : &ks[0][0]), kListWaveCap);
  } else if constexpr (SEL == 1) {
    // the selection itself: keys in ks, then the shared state and the
    // indices in vs (both free until the first chunk is staged)
    constexpr int kCapK = static_cast<int>(sizeof(ks) / 4);
    constexpr int kCapI = static_cast<int>((sizeof(vs) - sizeof(AttSelShared)) / 4);
    constexpr int kCap = kCapK < kCapI ? kCapK : kCapI;
    static_assert(sizeof(AttSelShared) % 16 == 0 && kCap >= 2048, "selection LDS");
    AttSelShared& ss = *reinterpret_cast<AttSelShared*>(&vs[0][0]);
    attend_select<kAttThreads, kCap>(
        p.sel, row, t, p.n_cap, p.k, s_begin, min(c_end * kAttChunk, n_ent), split, s_ent,
        reinterpret_cast<uint32_t*>(&ks[0][0]),
        reinterpret_cast<int32_t*>(&vs[0][0] + sizeof(AttSelShared)), ss);
  } else if (!HCA) {
    const int64_t n_list = min(c_end * kAttChunk, n_ent) - s_begin;
    for (int64_t i = tid; i < n_list; i += kAttThreads) s_ent[i] = p.idx[idx_row + s_begin + i];
  }
  if (tid == 0) s_partial[0] = s_partial[1] = 0;

  // Every thread gathers kPerThread 16-byte pieces of K and of V per chunk
  // (piece r: key (tid + 512 r) / kPieces, same column pc), into one of two
  // register slots: while chunk i is computed, the loads of chunks i+2 and
  // i+3 are in flight.  Absent slots (padding, positions outside the raw
  // buffer) read row 0 of the sequence's cache instead, and chunks past the
  // split's end re-read its last chunk, so every load is issued
  // unconditionally (which keeps the compiler's wait counts partial); absent
  // keys are masked out of the softmax.
  auto gather = [&](auto slot, int64_t chunk) __attribute__((always_inline)) {
    Slot& S = pick(slot);
    const int64_t s0 = chunk * kAttChunk;
    int64_t koff[kPerThread], voff[kPerThread];  // byte offsets from kc_b / vc_b
    if (s0 + kAttChunk <= n_ent) {
      // uniform fast path: every slot of the chunk is a compressed entry
#pragma unroll
      for (int r = 0; r < kPerThread; ++r) {
        const int key = key0 + r * (kAttThreads / kPieces);
        int64_t e;
        if (HCA) {
          e = s0 + key;
          S.ok[r] = true;
        } else {
          const int32_t ei = s_ent[s0 + key - s_begin];
          S.ok[r] = ei >= 0 && ei < p.n_cap;
          e = S.ok[r] ? ei : 0;
        }
        koff[r] = voff[r] = e * RB + pc * 16;
      }
    } else {
      // window slots, the split's tail, padding
      const int64_t raw_k = p.kr - kc_b, raw_v = p.vr - vc_b;
#pragma unroll
      for (int r = 0; r < kPerThread; ++r) {
        const int64_t s = s0 + key0 + r * (kAttThreads / kPieces);
        int64_t ko = pc * 16, vo = pc * 16;
        bool ok = false;
        if (s < n_ent) {
          const int64_t e = HCA ? s : static_cast<int64_t>(s_ent[s - s_begin]);
          ok = e >= 0 && e < p.n_cap;
          if (ok) ko = vo = e * RB + pc * 16;
        } else {
          const int64_t pos = t - p.W + 1 + (s - n_ent);
          const int64_t rr = pos - rp0;
          ok = s < n_slots && pos >= 0 && rr >= 0 && rr < p.R;
          if (ok) {
            ko = raw_k + (b * p.R + rr) * RB + pc * 16;
            vo = raw_v + (b * p.R + rr) * RB + pc * 16;
          }
        }
        S.ok[r] = ok;
        koff[r] = ko;
        voff[r] = vo;
      }
    }
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      S.k[r] = *reinterpret_cast<const u32x4*>(kc_b + koff[r]);
      S.v[r] = *reinterpret_cast<const u32x4*>(vc_b + voff[r]);
    }
  };
  auto stage = [&](auto slot, auto buf, int i) __attribute__((always_inline)) {
    const Slot& S = pick(slot);
    constexpr int bf = decltype(buf)::value;
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int key = key0 + r * (kAttThreads / kPieces);
      *reinterpret_cast<u32x4*>(&ks[bf][key * kKsStride + pc * 16]) = S.k[r];
      *reinterpret_cast<u32x4*>(&vs[bf][key * kVsStride + pc * 16]) = S.v[r];
      if (pc == 0) {
        valid[bf][key] = S.ok[r] ? 1 : 0;
        if (!S.ok[r]) s_partial[bf] = i + 1;
      }
    }
  };

  constexpr int kDT = D / 16;  // output dim tiles
  f32x4 o[kDT];
#pragma unroll
  for (int i = 0; i < kDT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // softmax reference (log2 domain), uniform per head
  float l_run = 0.f;        // this lane's partial sum of exp

  // Chunk i from LDS buffer `buf`: scores, online softmax update,
  // O^T += V^T . P^T.
  auto compute = [&](auto buf, int i) __attribute__((always_inline)) {
    constexpr int bf = decltype(buf)::value;
    if (!has_heads) return;
    const bool masked = s_partial[bf] == i + 1;
    const uint8_t* kb = ks[bf];
    const uint8_t* vb = vs[bf];
    // S^T tiles: this wave's 2 tiles of 16 keys x 16 heads (keys 32 kh ..)
    f32x4 s[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kt = 2 * kh + j;
      s[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint8_t* arow = kb + (kt * 16 + col) * kKsStride + g * (RB / 4);
      if (DTYPE == 1) {
#pragma unroll
        for (int st = 0; st < Tr::kKSteps; ++st) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(arow + st * 16);
          s[j] = mma_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[st]), s[j]);
        }
      } else {
#pragma unroll
        for (int st = 0; st < Tr::kKSteps; ++st) {
          const float a = *reinterpret_cast<const float*>(arow + st * 4);
          s[j] = mma_f32(a, __uint_as_float(qf[st >> 2][st & 3]), s[j]);
        }
      }
    }
    // scale (log2 domain), mask, chunk maximum.  The scaled score is
    // rounded once and the maximum taken over those values, so the largest
    // key gets exactly exp2(0) = 1 (no contraction into the exponent's FMA).
    {
#pragma clang fp contract(off)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[j][i] *= p.scale_log2;
    }
    if (masked) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!valid[bf][(2 * kh + j) * 16 + g * 4 + i]) s[j][i] = -INFINITY;
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, s[j][i]);
    mloc = max_xor32(max_xor16(mloc));
    const float m_new = mloc > m_run + kAttMaxSlack ? mloc : m_run;
    if (m_new == -INFINITY) return;  // nothing valid so far (uniform per head)
    if (__any(m_new != m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first update
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < kDT; ++i) o[i] *= alpha;
    }
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(s[j][i] - m_new);
        s[j][i] = e;
        lsum += e;
      }
    }
    l_run += lsum;

    // O^T += V^T . P^T
    if (DTYPE == 1) {
      // lane (dim col, group g) needs V[32kh + 4g + i][dim] (lo) and
      // V[32kh + 16 + 4g + i][dim] (hi), i = 0..3
      const uint8_t* vbase = vb + (32 * kh + 4 * g + (col >> 2)) * kVsStride + (col & 3) * 8;
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = static_cast<__bf16>(s[0][i]);
        pb[4 + i] = static_cast<__bf16>(s[1][i]);
      }
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        const u32x2 lo = lds_read_tr16(vbase + dt * 32);
        const u32x2 hi = lds_read_tr16(vbase + 16 * kVsStride + dt * 32);
        const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
        o[dt] = mma_bf16(__builtin_bit_cast(bf16x8, a), pb, o[dt]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float* vrow = reinterpret_cast<const float*>(
              vb + ((2 * kh + j) * 16 + 4 * g + i) * kVsStride);
#pragma unroll
          for (int dt = 0; dt < kDT; ++dt) o[dt] = mma_f32(vrow[dt * 16 + col], s[j][i], o[dt]);
        }
      }
    }
  };

  // Chunk i (split-relative) lives in register slot i % 2 and LDS buffer
  // i % 2.  Step i stages chunk i+1, refills its register slot with chunk
  // i+3, computes chunk i and ends with the barrier that publishes chunk i+1
  // and releases buffer i % 2.  The loop is unrolled by two so every slot
  // and buffer index is static and the order of loads in flight is the same
  // on every path.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  const int n_chunks = c_end > c_begin ? static_cast<int>(c_end - c_begin) : 0;
  auto clamp_chunk = [&](int i) __attribute__((always_inline)) {
    return c_begin + min(i, n_chunks - 1);
  };
  // the speculative HCA chunk i is what gather() would load: every slot a
  // visible entry and the chunk one of the split's
  auto spec_ok = [&](int i) __attribute__((always_inline)) {
    return i < n_chunks && (c_begin + i + 1) * kAttChunk <= n_ent;
  };
  if (n_chunks > 0) {
    // HCA gathers need nothing from LDS: their first loads go out before the
    // barrier that publishes s_ent / s_partial.  The two speculative chunks
    // loaded at the top are kept when they hold only visible entries of
    // this split (the usual case); otherwise they are gathered again now
    // that the row's position is known.
    if (HCA) {
      if (!spec_ok(0)) gather(I0{}, clamp_chunk(0));
      if (!spec_ok(1)) gather(I1{}, clamp_chunk(1));
    }
    __syncthreads();
    if (!HCA) {
      gather(I0{}, clamp_chunk(0));
      gather(I1{}, clamp_chunk(1));
    }
    stage(I0{}, I0{}, 0);
    gather(I0{}, clamp_chunk(2));
    __syncthreads();
    int i = 0;
    for (; i + 1 < n_chunks; i += 2) {
      stage(I1{}, I1{}, i + 1);
      gather(I1{}, clamp_chunk(i + 3));
      compute(I0{}, i);
      __syncthreads();
      stage(I0{}, I0{}, i + 2);
      gather(I0{}, clamp_chunk(i + 4));
      compute(I1{}, i + 1);
      __syncthreads();
    }
    if (i < n_chunks) compute(I0{}, i);
  }

  float l_tot = sum_xor32(sum_xor16(l_run));
  // Combine the two key halves of each head: the second-half waves leave
  // (O, max, sum) in the (now free) chunk buffers, the first-half waves fold
  // them in and write the result.
  {
    static_assert(sizeof(ks) >= 4 * kDT * 64 * sizeof(f32x4), "combine buffer");
    static_assert(sizeof(vs) >= 128 * sizeof(float), "combine buffer");
    f32x4* xo = reinterpret_cast<f32x4*>(&ks[0][0]);  // [head tile][dim tile][lane]
    float* xm = reinterpret_cast<float*>(&vs[0][0]);  // max [64], sum [64] per head slot
    __syncthreads();  // every wave is done with the chunk buffers
    if (kh == 1 && has_heads) {
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) xo[(ht * kDT + dt) * 64 + lane] = o[dt];
      if (g == 0) {
        xm[ht * 16 + col] = m_run;
        xm[64 + ht * 16 + col] = l_tot;
      }
    }
    __syncthreads();
    if (kh == 1 || !has_heads) return;
    const float m1 = xm[ht * 16 + col];
    const float l1 = xm[64 + ht * 16 + col];
    const float mm = fmaxf(m_run, m1);
    if (mm != -INFINITY) {  // both halves empty: O and the sum stay 0
      const float f0 = exp2f(m_run - mm), f1 = exp2f(m1 - mm);
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) o[dt] = o[dt] * f0 + xo[(ht * kDT + dt) * 64 + lane] * f1;
      l_tot = l_tot * f0 + l1 * f1;
      m_run = mm;
    }
  }
  const bool writer = head < p.H;
  if (p.splits == 1) {
    if (!writer) return;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    float* orow = p.out + (row * p.H + head) * D;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
      *reinterpret_cast<f32x4*>(orow + dt * 16 + 4 * g) = o[dt] * inv;
    if (p.lse && g == 0)
      p.lse[row * p.H + head] = l_tot > 0.f ? (m_run + log2f(l_tot)) / kLog2e : -INFINITY;
    return;
  }
  if (writer) {
    // the partial output is written through to memory (device-scope
    // stores, sc1): the merge launch reads it from there, and the end of
    // this launch has no dirty lines of it to write back (HCA 1M decode
    // 26.7 -> 26.0 us)
    const int64_t pr = (row * p.splits + split) * p.H + head;
    const __amdgpu_buffer_rsrc_t prs =
        store_rsrc(p.po + (row * p.splits + split) * p.H * D, static_cast<int>(p.H * D * 4));
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[dt]), prs,
                                             static_cast<uint32_t>((head * D + dt * 16 + 4 * g) * 4),
                                             0, kCachePolicySc1);
    if (g == 0) {
      p.pm[pr] = m_run;
      p.pl[pr] = l_tot;
    }
  }
}

template <int DTYPE, int D, bool HCA, int SEL>
__global__ __launch_bounds__(kAttThreads) void attend_kernel(AttParams p) {
  attend_body<DTYPE, D, HCA, SEL>(p);
}

// The same kernel held to 128 VGPRs (at least 4 waves per SIMD), so that two
// workgroups share a CU when their LDS fits twice: each hides the other's
// gather latency.  Used for grids of many rows (the chunked prefill); the
// decode grids, about one workgroup per CU, keep the unconstrained build.
template <int DTYPE, int D, bool HCA, int SEL>
__global__ __launch_bounds__(kAttThreads, 4) void attend_wide_kernel(AttParams p) {
  attend_body<DTYPE, D, HCA, SEL>(p);
}

// Merge the split partials of one query row: each thread owns 4 output dims
// of one head.  Splits are taken in batches of MB (8, 16 or 32: the
// smallest that holds a row's splits, so up to 32 splits cost one round
// trip to memory and few splits issue few redundant loads): every load of a
// batch (maxima, sums, partial outputs; indices clamped so none is
// conditional) is issued before any is used, and the batch is folded into a
// running (max, sum, O) in split order, so the result does not depend on
// scheduling.  Workgroups of NT threads: 256, or one wave when rows x
// head tiles of 256 threads would leave CUs idle (few rows), so that the
// loads of a row's partials are issued from more CUs.
constexpr int kMergeThreads = 256;
constexpr int kMergeThreadsSmall = 64;

template <int D, int MB, int NT>
__global__ __launch_bounds__(NT) void attend_merge_kernel(AttParams p) {
  constexpr int kTPH = D / 4;  // threads per head
  constexpr int kHPB = NT / kTPH;
  const int n_tiles = static_cast<int>((p.H + kHPB - 1) / kHPB);
  int64_t row;
  int tile;
  if (p.xcd_rows > 0) {  // a row's tiles on the XCD whose L2 holds its partials
    if (!xcd_row_item(blockIdx.x, n_tiles, p.xcd_rows, &row, &tile)) return;
  } else {
    row = blockIdx.y;
    tile = blockIdx.x;
  }
  const int64_t h = static_cast<int64_t>(tile) * kHPB + threadIdx.x / kTPH;
  const int d4 = threadIdx.x % kTPH;
  if (p.hist_zero) {  // the row's top-k histogram, read by every split of the attention launch
    uint32_t* hz = p.hist_zero + row * kTopkHistBins;
    for (int i = tile * NT + threadIdx.x; i < kTopkHistBins; i += n_tiles * NT)
      hz[i] = 0u;
  }
  if (h >= p.H) return;
  const int64_t base = row * p.splits * p.H + h;  // partial (row, split 0, head h)
  float M = -INFINITY, L = 0.f;
  f32x4 O = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < p.splits; s0 += MB) {
    float pm[MB], pl[MB];
    f32x4 po[MB];
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int64_t sp = min(s0 + j, p.splits - 1);
      pm[j] = p.pm[base + sp * p.H];
      pl[j] = p.pl[base + sp * p.H];
      po[j] = *reinterpret_cast<const f32x4*>(p.po + (base + sp * p.H) * D + 4 * d4);
    }
    float mb = -INFINITY;
#pragma unroll
    for (int j = 0; j < MB; ++j)
      if (s0 + j < p.splits) mb = fmaxf(mb, pm[j]);
    const float m_new = fmaxf(M, mb);
    if (m_new == -INFINITY) continue;  // every split so far is empty
    const float f = exp2f(M - m_new);  // 0 while M is -inf
    L *= f;
    O *= f;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const float w = s0 + j < p.splits ? exp2f(pm[j] - m_new) : 0.f;  // 0 for empty splits
      L = fmaf(pl[j], w, L);
      O += po[j] * w;
    }
    M = m_new;
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  *reinterpret_cast<f32x4*>(p.out + (row * p.H + h) * D + 4 * d4) = O * inv;
  if (p.lse && d4 == 0) p.lse[row * p.H + h] = L > 0.f ? (M + log2f(L)) / kLog2e : -INFINITY;
}

// ----------------------------------------------------------------- host side

AttSplit attend_split(int64_t rows, int64_t n_slots_max, bool hca) {
  // A split's partial result (H x D fp32) is as large as 64 gathered K/V
  // rows, so splits are kept at >= 4 chunks (256 keys) unless the batch is
  // too small to occupy the GPU otherwise; enough splits are made to give
  // roughly 256 workgroups.  CSA splits span at most kAttMaxSplitChunks
  // chunks (k <= 65536 and W <= 4096 keep that within the merge's
  // kMergeMaxSplits).
  AttSplit s;
  int64_t chunks = (n_slots_max + kAttChunk - 1) / kAttChunk;
  if (chunks < 1) chunks = 1;
  int64_t target = rows >= 256 ? 1 : (256 + rows - 1) / rows;
  int64_t min_cps = rows >= 64 ? 4 : rows >= 16 ? 2 : 1;
  if (target > chunks) target = chunks;
  int64_t cps = (chunks + target - 1) / target;
  if (cps < min_cps) cps = min_cps;
  // at most kMergeMaxSplits partials per row
  if (cps < (chunks + kMergeMaxSplits - 1) / kMergeMaxSplits)
    cps = (chunks + kMergeMaxSplits - 1) / kMergeMaxSplits;
  if (!hca && cps > kAttMaxSplitChunks) cps = kAttMaxSplitChunks;
  if (cps > chunks) cps = chunks;
  s.chunks_per_split = static_cast<int>(cps);
  s.splits = static_cast<int>((chunks + cps - 1) / cps);
  return s;
}

// Workspace: the split partials (O, max, sum); nothing in it is read before
// being written in the same call.
size_t attend_workspace_bytes(int64_t rows, int64_t H, int64_t D, int64_t n_slots_max, bool hca) {
  const AttSplit s = attend_split(rows, n_slots_max, hca);
  if (s.splits == 1) return 0;
  return static_cast<size_t>(rows) * s.splits * H * (D + 2) * sizeof(float);
}

template <int D>
void launch_merge(int splits, bool small, dim3 grid, const AttParams& p, hipStream_t stream) {
  // the smallest batch that holds the row's splits
  if (small) {
    if (splits > 16) launch_kernel(attend_merge_kernel<D, 32, kMergeThreadsSmall>, grid, kMergeThreadsSmall, stream, p);
    else if (splits > 8) launch_kernel(attend_merge_kernel<D, 16, kMergeThreadsSmall>, grid, kMergeThreadsSmall, stream, p);
    else launch_kernel(attend_merge_kernel<D, 8, kMergeThreadsSmall>, grid, kMergeThreadsSmall, stream, p);
  } else {
    if (splits > 16) launch_kernel(attend_merge_kernel<D, 32, kMergeThreads>, grid, kMergeThreads, stream, p);
    else if (splits > 8) launch_kernel(attend_merge_kernel<D, 16, kMergeThreads>, grid, kMergeThreads, stream, p);
    else launch_kernel(attend_merge_kernel<D, 8, kMergeThreads>, grid, kMergeThreads, stream, p);
  }
}

int launch_attend(const void* q, int dtype, const void* kc, const void* vc, const int32_t* idx,
                  int k, int hca_m, const void* kr, const void* vr, const int64_t* raw_pos0,
                  int64_t R, const int64_t* pos0, int64_t B, int64_t T, int64_t H, int64_t D,
                  int64_t n_cap, int W, float scale, float* out, float* lse, void* ws,
                  hipStream_t stream, const TopkLists* sel) {
  const bool hca = hca_m > 0;
  if (sel != nullptr && hca) return -2;
  const int64_t rows = B * T;
  const int64_t n_slots_max = (hca ? n_cap : k) + W;
  const AttSplit sp = attend_split(rows, n_slots_max, hca);
  if (sp.splits > kMergeMaxSplits || (!hca && sp.chunks_per_split > kAttMaxSplitChunks))
    return -2;
  AttParams p;
  p.q = static_cast<const uint8_t*>(q);
  p.kc = static_cast<const uint8_t*>(kc);
  p.vc = static_cast<const uint8_t*>(vc);
  p.idx = idx;
  p.kr = static_cast<const uint8_t*>(kr);
  p.vr = static_cast<const uint8_t*>(vr);
  p.raw_pos0 = raw_pos0;
  p.pos0 = pos0;
  p.out = out;
  p.lse = lse;
  p.T = T;
  p.H = H;
  p.n_cap = n_cap;
  p.R = R;
  p.k = k;
  p.W = W;
  p.m = hca ? hca_m : 1;
  p.splits = sp.splits;
  p.chunks_per_split = sp.chunks_per_split;
  p.scale_log2 = scale * kLog2e;
  p.po = p.pm = p.pl = nullptr;
  p.sel = sel ? *sel : TopkLists{};
  p.hist_zero = sel && sel->regs && sp.splits > 1 ? sel->hist : nullptr;
  if (sp.splits > 1) {
    float* base = static_cast<float*>(ws);
    p.po = base;
    p.pm = base + rows * sp.splits * H * D;
    p.pl = p.pm + rows * sp.splits * H;
  }
  p.xcd_rows = xcd_mappable(rows) ? rows : 0;
  const dim3 grid = p.xcd_rows ? dim3(static_cast<unsigned>(xcd_grid_size(rows, sp.splits)))
                               : dim3(static_cast<unsigned>(sp.splits), static_cast<unsigned>(rows));
  // (bf16 keys, d 128, given indices: its LDS fits twice in a CU)
  const bool wide = static_cast<int64_t>(grid.x) * grid.y >= kAttWideGroups;
  const bool m_small = rows * ((H + kMergeThreads / (D / 4) - 1) / (kMergeThreads / (D / 4))) < 256;
  const int m_nt = m_small ? kMergeThreadsSmall : kMergeThreads;
  const int64_t m_tiles = (H + m_nt / (D / 4) - 1) / (m_nt / (D / 4));
  const dim3 mgrid = p.xcd_rows ? dim3(static_cast<unsigned>(xcd_grid_size(rows, m_tiles)))
                                : dim3(static_cast<unsigned>(m_tiles), static_cast<unsigned>(rows));
#define CSA_ATT_CASE(DT, DD)                                                        \
  if (dtype == DT && D == DD) {                                                     \
    if (hca)                                                                        \
      launch_kernel(attend_kernel<DT, DD, true, 0>, grid, kAttThreads, stream, p);          \
    else if (sel && sel->regs)                                                      \
      launch_kernel(attend_kernel<DT, DD, false, 2>, grid, kAttThreads, stream, p);         \
    else if (sel)                                                                   \
      launch_kernel(attend_kernel<DT, DD, false, 1>, grid, kAttThreads, stream, p);         \
    else if (DT == 1 && DD == 128 && wide)                                          \
      launch_kernel(attend_wide_kernel<1, 128, false, 0>, grid, kAttThreads, stream, p);    \
    else                                                                            \
      launch_kernel(attend_kernel<DT, DD, false, 0>, grid, kAttThreads, stream, p);         \
    if (sp.splits > 1) launch_merge<DD>(sp.splits, m_small, mgrid, p, stream);      \
    return hipGetLastError() == hipSuccess ? 0 : -1;                                \
  }
  CSA_ATT_CASE(0, 64)
  CSA_ATT_CASE(0, 128)
  CSA_ATT_CASE(1, 64)
  CSA_ATT_CASE(1, 128)
#undef CSA_ATT_CASE
  return -2;
}

}  // namespace csa
