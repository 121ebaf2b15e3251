// Core attention over selected compressed entries plus the sliding window
// (octagono.org "Hybrid Attention: CSA and HCA": attend only to the
// selected entries, with a window of recent tokens for local context;
// dataforcee.us "Hybrid Attention: CSA and HCA": both CSA and HCA carry the
// window branch; HCA attends densely to every compressed entry,
// "DeepSeek V4 technical review" section 2.2).
//
// One query token per workgroup row; every query head shares the single KV
// head, so the gathered key/value rows are staged in LDS once and used by
// all heads (4 waves x 16 heads).  The logical key list of a query is
//   slots [0, n_entries)            -> compressed entry (idx list or 0..V-1)
//   slots [n_entries, n_entries+W)  -> raw window position t-W+1+w
// and is cut into 64-key chunks; long lists are split over several
// workgroups whose (max, sum, O) partials are merged in a fixed order.
//
// MFMA orientation: S^T = K . Q^T puts keys on rows and heads on columns,
// so each lane ends up holding the probabilities of its own head for 4 keys
// per tile -- exactly the B operand layout of O^T = V^T . P^T (the key order
// inside the reduction is free as long as V^T uses the same one).  V is
// therefore staged transposed ([dim][key]) in LDS.
#include "common.h"
#include "kernels.h"

namespace csa {

constexpr int kAttChunk = 64;  // keys per LDS chunk
constexpr int kMergeMaxSplits = 64;  // partials merged per row
constexpr float kLog2e = 1.4426950408889634f;

template <int DTYPE, int D>
struct AttTraits;

template <int D>
struct AttTraits<0, D> {  // fp32 storage, v_mfma_f32_16x16x4_f32
  static constexpr int kElem = 4;
  static constexpr int kRowBytes = D * 4;
  static constexpr int kKSteps = D / 4;       // QK steps (1 element per lane)
  static constexpr int kVtStride = kAttChunk * 4 + 16;  // bytes per dim row
};

template <int D>
struct AttTraits<1, D> {  // bf16 storage, v_mfma_f32_16x16x32_bf16
  static constexpr int kElem = 2;
  static constexpr int kRowBytes = D * 2;
  static constexpr int kKSteps = D / 32;
  static constexpr int kVtStride = kAttChunk * 2 + 8;
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
__global__ __launch_bounds__(256) void attend_kernel(AttParams p) {
  using Tr = AttTraits<DTYPE, D>;
  constexpr int RB = Tr::kRowBytes;
  constexpr int kPieces = RB / 16;             // 16-byte pieces per row
  constexpr int kPerThread = kAttChunk * kPieces / 256;
  constexpr int kKsStride = RB + 16;
  __shared__ __attribute__((aligned(16))) uint8_t ks[kAttChunk * kKsStride];
  __shared__ __attribute__((aligned(16))) uint8_t vt[D * Tr::kVtStride];
  __shared__ int valid[kAttChunk];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int g = lane >> 4;
  const int64_t row = blockIdx.y;
  const int split = blockIdx.x;
  const int64_t b = row / p.T;
  const int64_t t = p.pos0[b] + (row - b * p.T);
  const int64_t rp0 = p.W > 0 ? p.raw_pos0[b] : 0;
  const int64_t n_ent = HCA ? visible_entries(t, p.m, p.n_cap) : static_cast<int64_t>(p.k);
  const int64_t n_slots = n_ent + p.W;
  const int64_t c_begin = static_cast<int64_t>(split) * p.chunks_per_split;
  const int64_t c_end = min(c_begin + p.chunks_per_split, (n_slots + kAttChunk - 1) / kAttChunk);
  const int n_ht = static_cast<int>((p.H + 15) >> 4);
  const bool has_heads = wave < n_ht;
  const int head = wave * 16 + col;

  // Q^T fragments: this lane's head, one contiguous quarter of the row.
  constexpr int kQVec = RB / 4 / 16;
  u32x4 qf[kQVec];
#pragma unroll
  for (int v = 0; v < kQVec; ++v) qf[v] = u32x4{0u, 0u, 0u, 0u};
  if (has_heads && head < p.H) {
    const u32x4* src =
        reinterpret_cast<const u32x4*>(p.q + (row * p.H + head) * RB + g * (RB / 4));
#pragma unroll
    for (int v = 0; v < kQVec; ++v) qf[v] = src[v];
  }

  // Every thread gathers kPerThread 16-byte pieces of K and of V per chunk.
  // Absent slots (padding, positions outside the raw buffer) read row 0 of
  // the sequence's cache instead, so every load is issued unconditionally;
  // they are masked out of the softmax and their values get weight 0.
  const uint8_t* kc_b = p.kc + b * p.n_cap * RB;
  const uint8_t* vc_b = p.vc + b * p.n_cap * RB;
  const int64_t idx_row = row * p.k;
  int32_t ent[kPerThread];  // the chunk's entry index per piece (CSA)
  auto fetch_idx = [&](int64_t chunk) {
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int64_t s = chunk * kAttChunk + (tid + 256 * r) / kPieces;
      if (HCA) {
        ent[r] = static_cast<int32_t>(s);
      } else {
        const int64_t sc = s < n_ent ? s : n_ent - 1;
        ent[r] = n_ent > 0 ? p.idx[idx_row + sc] : -1;
      }
    }
  };
  u32x4 kreg[kPerThread], vreg[kPerThread];
  bool vld[kPerThread];
  auto gather = [&](int64_t chunk) {
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int id = tid + 256 * r;
      const int key = id / kPieces;
      const int pc = id - key * kPieces;
      const int64_t s = chunk * kAttChunk + key;
      const uint8_t* krow = kc_b;
      const uint8_t* vrow = vc_b;
      bool ok = false;
      if (s < n_ent) {
        const int64_t e = ent[r];
        ok = e >= 0 && e < p.n_cap;
        if (ok) {
          krow = kc_b + e * RB;
          vrow = vc_b + e * RB;
        }
      } else {
        const int64_t pos = t - p.W + 1 + (s - n_ent);
        const int64_t rr = pos - rp0;
        ok = s < n_slots && pos >= 0 && rr >= 0 && rr < p.R;
        if (ok) {
          krow = p.kr + (b * p.R + rr) * RB;
          vrow = p.vr + (b * p.R + rr) * RB;
        }
      }
      vld[r] = ok;
      kreg[r] = *reinterpret_cast<const u32x4*>(krow + pc * 16);
      vreg[r] = *reinterpret_cast<const u32x4*>(vrow + pc * 16);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int id = tid + 256 * r;
      const int key = id / kPieces;
      const int pc = id - key * kPieces;
      *reinterpret_cast<u32x4*>(ks + key * kKsStride + pc * 16) = kreg[r];
      if (pc == 0) valid[key] = vld[r] ? 1 : 0;
      if (DTYPE == 1) {
        // 8 bf16 values: dims pc*8 .. pc*8+7 of this key
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t word = vreg[r][e >> 1];
          const uint16_t h = static_cast<uint16_t>((e & 1) ? (word >> 16) : (word & 0xffffu));
          *reinterpret_cast<uint16_t*>(vt + (pc * 8 + e) * Tr::kVtStride + key * 2) = h;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<uint32_t*>(vt + (pc * 4 + e) * Tr::kVtStride + key * 4) = vreg[r][e];
      }
    }
  };

  constexpr int kDT = D / 16;  // output dim tiles
  f32x4 o[kDT];
#pragma unroll
  for (int i = 0; i < kDT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max (log2 domain), uniform per head
  float l_run = 0.f;        // this lane's partial sum of exp

  if (c_begin < c_end) {
    fetch_idx(c_begin);
    gather(c_begin);
    if (c_begin + 1 < c_end) fetch_idx(c_begin + 1);
  }
  for (int64_t c = c_begin; c < c_end; ++c) {
    __syncthreads();
    stage();
    __syncthreads();
    if (c + 1 < c_end) {
      gather(c + 1);
      if (c + 2 < c_end) fetch_idx(c + 2);
    }
    if (!has_heads) continue;

    // S^T tiles: 4 tiles of 16 keys x 16 heads
    f32x4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint8_t* arow = ks + (kt * 16 + col) * kKsStride + g * (RB / 4);
      if (DTYPE == 1) {
#pragma unroll
        for (int st = 0; st < Tr::kKSteps; ++st) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(arow + st * 16);
          s[kt] = mma_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[st]), s[kt]);
        }
      } else {
#pragma unroll
        for (int st = 0; st < Tr::kKSteps; ++st) {
          const float a = *reinterpret_cast<const float*>(arow + st * 4);
          s[kt] = mma_f32(a, __uint_as_float(qf[st >> 2][st & 3]), s[kt]);
        }
      }
    }
    // scale, mask, running max
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = valid[kt * 16 + g * 4 + i] ? s[kt][i] * p.scale_log2 : -INFINITY;
        s[kt][i] = x;
        mloc = fmaxf(mloc, x);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    if (m_new == -INFINITY) continue;  // nothing valid so far (uniform per head)
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = exp2f(s[kt][i] - m_new);
        s[kt][i] = e;
        lsum += e;
      }
    }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int i = 0; i < kDT; ++i) o[i] *= alpha;

    // O^T += V^T . P^T
    if (DTYPE == 1) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[i] = static_cast<__bf16>(s[2 * kk][i]);
          pb[4 + i] = static_cast<__bf16>(s[2 * kk + 1][i]);
        }
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          const uint8_t* vrow = vt + (dt * 16 + col) * Tr::kVtStride;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + (32 * kk + 4 * g) * 2);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + (32 * kk + 16 + 4 * g) * 2);
          const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
          o[dt] = mma_bf16(__builtin_bit_cast(bf16x8, a), pb, o[dt]);
        }
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int dt = 0; dt < kDT; ++dt) {
            const float a = *reinterpret_cast<const float*>(
                vt + (dt * 16 + col) * Tr::kVtStride + (kt * 16 + 4 * g + i) * 4);
            o[dt] = mma_f32(a, s[kt][i], o[dt]);
          }
        }
      }
    }
  }

  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const bool writer = has_heads && head < p.H;
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

// Merge the split partials of one (query row, head): one thread per output
// dim.  All split maxima and sums are fetched at once into LDS, the merge
// weights follow from them, and each thread then issues its partial-output
// loads for every split before using any (fixed split order, so the result
// does not depend on scheduling).
template <int D>
__global__ __launch_bounds__(D) void attend_merge_kernel(AttParams p) {
  __shared__ float s_w[kMergeMaxSplits];
  __shared__ float s_inv[2];
  const int64_t row = blockIdx.y;
  const int64_t h = blockIdx.x;
  const int dd = threadIdx.x;
  const int64_t base = row * p.splits * p.H + h;  // partial (row, split 0, head h)
  if (dd < 64) {
    // one wave: per-split weights exp2(m_s - M) and the merged normaliser
    const bool on = dd < p.splits;
    const float pm = on ? p.pm[base + dd * p.H] : -INFINITY;
    const float pl = on ? p.pl[base + dd * p.H] : 0.f;
    const float M = wave_max(pm);
    const float wgt = (M == -INFINITY || pm == -INFINITY) ? 0.f : exp2f(pm - M);
    const float L = wave_sum(pl * wgt);
    if (on) s_w[dd] = wgt;
    if (dd == 0) {
      s_inv[0] = L > 0.f ? 1.0f / L : 0.f;
      s_inv[1] = L > 0.f ? (M + log2f(L)) / kLog2e : -INFINITY;
    }
  }
  __syncthreads();
  float po[kMergeMaxSplits];
#pragma unroll
  for (int s = 0; s < kMergeMaxSplits; ++s)
    po[s] = s < p.splits ? p.po[(base + s * p.H) * D + dd] : 0.f;
  float O = 0.f;
#pragma unroll
  for (int s = 0; s < kMergeMaxSplits; ++s)
    if (s < p.splits) O = fmaf(po[s], s_w[s], O);
  p.out[(row * p.H + h) * D + dd] = O * s_inv[0];
  if (p.lse && dd == 0) p.lse[row * p.H + h] = s_inv[1];
}

// ----------------------------------------------------------------- host side

AttSplit attend_split(int64_t rows, int64_t n_slots_max) {
  // A split's partial result (H x D fp32) is as large as 64 gathered K/V
  // rows, so splits are kept at >= 4 chunks (256 keys) unless the batch is
  // too small to occupy the GPU otherwise; enough splits are made to give
  // roughly 256 workgroups.
  AttSplit s;
  int64_t chunks = (n_slots_max + kAttChunk - 1) / kAttChunk;
  if (chunks < 1) chunks = 1;
  int64_t target = rows >= 256 ? 1 : (256 + rows - 1) / rows;
  int64_t min_cps = rows >= 64 ? 4 : rows >= 16 ? 2 : 1;
  if (target > chunks) target = chunks;
  int64_t cps = (chunks + target - 1) / target;
  if (cps < min_cps) cps = min_cps;
  // the merge handles at most kMergeMaxSplits partials per row
  if (cps < (chunks + kMergeMaxSplits - 1) / kMergeMaxSplits)
    cps = (chunks + kMergeMaxSplits - 1) / kMergeMaxSplits;
  if (cps > chunks) cps = chunks;
  s.chunks_per_split = static_cast<int>(cps);
  s.splits = static_cast<int>((chunks + cps - 1) / cps);
  return s;
}

// Workspace: the split partials (O, max, sum); nothing in it is read before
// being written in the same call.
size_t attend_workspace_bytes(int64_t rows, int64_t H, int64_t D, int64_t n_slots_max) {
  const AttSplit s = attend_split(rows, n_slots_max);
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
  const AttSplit sp = attend_split(rows, n_slots_max);
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
#define CSA_ATT_CASE(DT, DD)                                                        \
  if (dtype == DT && D == DD) {                                                     \
    if (hca)                                                                        \
      attend_kernel<DT, DD, true><<<grid, 256, 0, stream>>>(p);                     \
    else                                                                            \
      attend_kernel<DT, DD, false><<<grid, 256, 0, stream>>>(p);                    \
    if (sp.splits > 1)                                                              \
      attend_merge_kernel<DD><<<dim3(static_cast<unsigned>(H), static_cast<unsigned>(rows)), \
                                DD, 0, stream>>>(p);                                \
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
