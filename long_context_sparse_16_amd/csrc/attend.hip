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

namespace csa {

constexpr int kAttChunk = 64;  // keys per LDS chunk
constexpr int kAttThreads = 512;  // 8 waves: 4 head tiles x 2 key halves
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
  float scale_log2;  // scale * log2(e)
};

template <int DTYPE, int D, bool HCA>
__global__ __launch_bounds__(kAttThreads) void attend_kernel(AttParams p) {
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

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ht = wave & 3;  // head tile
  const int kh = wave >> 2;  // key half of every chunk
  const int col = lane & 15;
  const int g = lane >> 4;
  const int64_t row = blockIdx.y;
  const int split = blockIdx.x;
  const int64_t b = seq_of_row(row, p.T);
  // both position loads are unconditional, so they are in flight together
  // (raw_pos0 may be NULL when W == 0; its value is then unused)
  const int64_t t = p.pos0[b] + (row - b * p.T);
  const int64_t rp0 = (p.W > 0 ? p.raw_pos0 : p.pos0)[b];
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
  if (!HCA) {
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
  if (n_chunks > 0) {
    // HCA gathers need nothing from LDS: their first loads go out before the
    // barrier that publishes s_ent / s_partial.
    if (HCA) {
      gather(I0{}, clamp_chunk(0));
      gather(I1{}, clamp_chunk(1));
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
    const int64_t pr = (row * p.splits + split) * p.H + head;
    float* orow = p.po + pr * D;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) *reinterpret_cast<f32x4*>(orow + dt * 16 + 4 * g) = o[dt];
    if (g == 0) {
      p.pm[pr] = m_run;
      p.pl[pr] = l_tot;
    }
  }
}

// Merge the split partials of one query row: each thread owns 4 output dims
// of one head.  Splits are taken in batches of MB (8, 16 or 32: the
// smallest that holds a row's splits, so up to 32 splits cost one round
// trip to memory and few splits issue few redundant loads): every load of a
// batch (maxima, sums, partial outputs; indices clamped so none is
// conditional) is issued before any is used, and the batch is folded into a
// running (max, sum, O) in split order, so the result does not depend on
// scheduling.
constexpr int kMergeThreads = 256;

template <int D, int MB>
__global__ __launch_bounds__(kMergeThreads) void attend_merge_kernel(AttParams p) {
  constexpr int kTPH = D / 4;  // threads per head
  constexpr int kHPB = kMergeThreads / kTPH;
  const int64_t row = blockIdx.y;
  const int64_t h = static_cast<int64_t>(blockIdx.x) * kHPB + threadIdx.x / kTPH;
  const int d4 = threadIdx.x % kTPH;
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

int launch_attend(const void* q, int dtype, const void* kc, const void* vc, const int32_t* idx,
                  int k, int hca_m, const void* kr, const void* vr, const int64_t* raw_pos0,
                  int64_t R, const int64_t* pos0, int64_t B, int64_t T, int64_t H, int64_t D,
                  int64_t n_cap, int W, float scale, float* out, float* lse, void* ws,
                  hipStream_t stream) {
  const bool hca = hca_m > 0;
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
  if (sp.splits > 1) {
    float* base = static_cast<float*>(ws);
    p.po = base;
    p.pm = base + rows * sp.splits * H * D;
    p.pl = p.pm + rows * sp.splits * H;
  }
  dim3 grid(static_cast<unsigned>(sp.splits), static_cast<unsigned>(rows));
  const dim3 mgrid(static_cast<unsigned>((H + kMergeThreads / (D / 4) - 1) / (kMergeThreads / (D / 4))),
                   static_cast<unsigned>(rows));
#define CSA_ATT_CASE(DT, DD)                                                        \
  if (dtype == DT && D == DD) {                                                     \
    if (hca)                                                                        \
      attend_kernel<DT, DD, true><<<grid, kAttThreads, 0, stream>>>(p);             \
    else                                                                            \
      attend_kernel<DT, DD, false><<<grid, kAttThreads, 0, stream>>>(p);            \
    if (sp.splits > 16)                                                             \
      attend_merge_kernel<DD, 32><<<mgrid, kMergeThreads, 0, stream>>>(p);          \
    else if (sp.splits > 8)                                                         \
      attend_merge_kernel<DD, 16><<<mgrid, kMergeThreads, 0, stream>>>(p);          \
    else if (sp.splits > 1)                                                         \
      attend_merge_kernel<DD, 8><<<mgrid, kMergeThreads, 0, stream>>>(p);           \
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
