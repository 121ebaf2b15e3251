// Block-wide pieces of the exact radix top-k selection (larger score key
// first, ties to the lower index), shared by the top-k kernels and the
// attention kernel that selects its own keys.  Keys are the order-preserving
// 32-bit images of fp32 scores; the first digit is the top 12 bits.
// Functions taking an `sm` need its members hist (at least 2048 words), scan
// (32 words) and misc (8 words) in LDS.  Every function is called by all NT
// threads of the workgroup (they contain barriers).
#pragma once

#include "common.h"

namespace csa {

// Number of lanes below this one whose bit is set in a wave mask.
__device__ __forceinline__ uint32_t lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

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
template <int NT, typename SM, typename Visit>
__device__ void digit_pass(SM& sm, Visit visit, int shift, int nb, uint32_t r) {
  for (int i = threadIdx.x; i < nb; i += NT) sm.hist[i] = 0u;
  __syncthreads();
  visit([&](uint32_t key, int32_t) { atomicAdd(&sm.hist[(key >> shift) & (nb - 1)], 1u); });
  __syncthreads();
  block_find_top<NT>(sm.hist, nb, r, sm.scan, sm.misc);
}

// The exact selection among items that all share the first digit, needing
// r of them: an item (key, j) wins iff (key & 0xfffff) > low20, or it equals
// low20 and j <= jmax.  Returns {low20, jmax}.
struct Cut {
  uint32_t low20;
  int32_t jmax;
};

template <int NT, typename SM, typename Visit>
__device__ Cut resolve_cut(SM& sm, Visit visit_all, uint32_t r) {
  digit_pass<NT>(sm, visit_all, 10, 1024, r);  // key bits 19..10
  const uint32_t b2 = sm.misc[0];
  const uint32_t r2 = r - sm.misc[1];
  const uint32_t n2 = sm.hist[b2];  // candidates sharing the cut's top 20 key bits
  __syncthreads();
  if (n2 <= 64) {
    // Few of them (the usual case): collect them in LDS and let one wave
    // rank them by (key desc, index asc); the r2-th is the cut.  Three
    // barriers instead of the further digit passes.
    uint32_t* ck = sm.hist;        // keys [64]
    uint32_t* cj = sm.hist + 64;   // indices [64]
    uint32_t* cn = sm.hist + 128;  // count
    if (threadIdx.x == 0) *cn = 0u;
    __syncthreads();
    visit_all([&](uint32_t key, int32_t j) {
      if (((key >> 10) & 1023u) == b2) {
        const uint32_t q = atomicAdd(cn, 1u);
        ck[q] = key;
        cj[q] = static_cast<uint32_t>(j);
      }
    });
    __syncthreads();
    if (threadIdx.x < 64) {
      const int l = threadIdx.x;
      const bool have = static_cast<uint32_t>(l) < n2;
      const uint32_t lo = have ? (ck[l] & 0xfffffu) : 0u;
      const int32_t jj = have ? static_cast<int32_t>(cj[l]) : 0x7fffffff;
      uint32_t rank = 0;  // candidates that come before this one
      for (uint32_t q = 0; q < n2; ++q) {
        const uint32_t lo_q = __shfl(lo, static_cast<int>(q));
        const int32_t j_q = __shfl(jj, static_cast<int>(q));
        rank += (lo_q > lo || (lo_q == lo && j_q < jj)) ? 1u : 0u;
      }
      if (have && rank == r2 - 1u) {
        sm.misc[2] = lo;
        sm.misc[3] = static_cast<uint32_t>(jj);
      }
    }
    __syncthreads();
    const Cut c{sm.misc[2], static_cast<int32_t>(sm.misc[3])};
    __syncthreads();
    return c;
  }
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
  return Cut{low20, jmax};
}

__device__ __forceinline__ bool cut_wins(Cut c, uint32_t key, int32_t j) {
  const uint32_t lo = key & 0xfffffu;
  return lo > c.low20 || (lo == c.low20 && j <= c.jmax);
}

}  // namespace csa
