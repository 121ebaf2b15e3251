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
#include <atomic>
#include <type_traits>

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
  static constexpr int kRowBytes = DI * 4;
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
  static constexpr int kRowBytes = DI * 2;
  static constexpr int kLaneBytes = DI * 2 / 4;
  static constexpr int kSteps = DI / 32;
  __device__ static f32x4 mma(const u32x4* a, const u32x4* b, int s, f32x4 c) {
    return mma_bf16(__builtin_bit_cast(bf16x8, a[s]), __builtin_bit_cast(bf16x8, b[s]), c);
  }
};

template <int DI>
struct IdxTraits<2, DI> {  // fp8 e4m3, v_mfma_f32_16x16x128_f8f6f4
  static constexpr int kElemBytes = 1;
  static constexpr int kRowBytes = DI;
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

// MXFP4 (OCP MX: E2M1 codes two per byte, one E8M0 scale per 32 elements),
// v_mfma_scale_f32_16x16x128_f8f6f4: a lane's 16 bytes are exactly one
// 32-element block, so the block scales ride along as one byte per lane
// (see mma_fp4); the kernel passes them.
template <int DI>
struct IdxTraits<3, DI> {
  static constexpr int kRowBytes = DI / 2;
  static constexpr int kLaneBytes = DI / 8;
  static constexpr int kSteps = DI / 128;
};

// A fragments (4 tiles of 16 query heads, this lane's quarter of each head
// row) and per-head weights (times the query scale for fp8) of query row
// `row`.  issue() starts every load unconditionally from clamped addresses
// (heads >= H_I read head H_I - 1), so they are in flight together;
// finish() then zeroes the weights of heads >= H_I, and of every head when
// !ok, which removes those heads from the score (their A rows need no
// masking).  Callers put their first key loads between the two.
template <int DTYPE, int DI>
struct QueryFrags {
  using Tr = IdxTraits<DTYPE, DI>;
  static constexpr int kVec = Tr::kLaneBytes / 16;
  static constexpr int kRowBytes = Tr::kRowBytes;
  u32x4 a[4][kVec];
  float wq[4][4];
  float ws[4][4];
  uint32_t sa[4];  // MXFP4: E8M0 scale of this lane's block of each head tile's row

  __device__ __forceinline__ void issue(const uint8_t* __restrict__ qi,
                                        const float* __restrict__ qi_scale,
                                        const float* __restrict__ w, int64_t row, int H_I,
                                        int col, int g) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const int h = ht * 16 + col;
      const int64_t hrow = row * H_I + (h < H_I ? h : H_I - 1);
      const u32x4* src =
          reinterpret_cast<const u32x4*>(qi + hrow * kRowBytes + g * Tr::kLaneBytes);
#pragma unroll
      for (int v = 0; v < kVec; ++v) a[ht][v] = src[v];
      if (DTYPE == 3) sa[ht] = reinterpret_cast<const uint8_t*>(qi_scale)[hrow * (DI / 32) + g];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = ht * 16 + g * 4 + i;
        const int64_t off = row * H_I + (hh < H_I ? hh : H_I - 1);
        wq[ht][i] = w[off];
        ws[ht][i] = DTYPE == 2 ? qi_scale[off] : 1.f;
      }
    }
  }

  __device__ __forceinline__ void finish(int H_I, bool ok, int g) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool live = ok && ht * 16 + g * 4 + i < H_I;
        wq[ht][i] = live ? (DTYPE == 2 ? wq[ht][i] * ws[ht][i] : wq[ht][i]) : 0.f;
      }
    }
  }
};

constexpr int kIdxWaves = 4;
constexpr int kIdxTile = 16;        // entries per MFMA column tile
constexpr int kIdxGroupLoads = 8;   // 16-byte key loads per lane per group

// Tiles per load group: 8 KiB of keys per wave (MXFP4: 4 KiB, measured
// best there, where the per-entry epilogue is the larger share of the work).
template <int DTYPE, int DI>
constexpr int idx_group_tiles() {
  constexpr int loads = DTYPE == 3 ? kIdxGroupLoads / 2 : kIdxGroupLoads;
  return loads / (IdxTraits<DTYPE, DI>::kLaneBytes / 16) > 0
             ? loads / (IdxTraits<DTYPE, DI>::kLaneBytes / 16)
             : 1;
}

// grid: x = entry chunk, y = query row (b * T + i).  block: 4 waves.
// The chunk's tiles are taken in groups of kGroup tiles; wave w handles
// groups w, w+4, ...  While one group is multiplied, the next group's loads
// are already in flight (two register buffers, statically indexed so they
// stay in VGPRs).  The host sizes the chunks so that the grid is about one
// workgroup per compute unit.
template <int DTYPE, int DI, bool RELU, bool HIST, bool FUSED>
__global__ __launch_bounds__(256) void indexer_kernel(
    const uint8_t* __restrict__ qi, const float* __restrict__ qi_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ ki,
    const float* __restrict__ ki_scale, const int64_t* __restrict__ pos0, int64_t T,
    int H_I, int64_t n_cap, int m, int tiles_per_wg, float* __restrict__ scores,
    uint32_t* __restrict__ hist, int topk_k, FusedCompress fc) {
  using Tr = IdxTraits<DTYPE, DI>;
  constexpr int kVec = Tr::kLaneBytes / 16;  // 16-byte loads per lane per row
  constexpr int kRowBytes = Tr::kRowBytes;
  constexpr int kGroup = idx_group_tiles<DTYPE, DI>();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int col = lane & 15;
  const int g = lane >> 4;
  // first-digit histogram, then one dummy word per lane (see below)
  __shared__ uint32_t s_hist[HIST ? kTopkHistBins + 64 : 1];
  const int64_t row = blockIdx.y;
  // A operand: 4 head tiles of 16 query heads, kept in registers (issued
  // first: it does not depend on the row's position).
  QueryFrags<DTYPE, DI> qf;
  qf.issue(qi, qi_scale, w, row, H_I, col, g);
  const auto& a = qf.a;
  const auto& wq = qf.wq;

  const int64_t b = seq_of_row(row, T);
  // FP8: each lane also fetches the fp32 scale of its column's entry with
  // the group's keys; MXFP4: the entry's four E8M0 block scales as one
  // word, whose byte g the MFMA step shifts into place.  (KScale holds
  // either.)
  using KScale = std::conditional_t<DTYPE == 3, uint32_t, float>;
  constexpr int kGroupEnt = kGroup * kIdxTile;
  u32x4 buf0[kGroup][kVec], buf1[kGroup][kVec];
  KScale ks0[kGroup], ks1[kGroup];
  {
    // This wave's first group is loaded before the row's position arrives,
    // as if every entry of the workgroup's range were visible (addresses
    // clamped into the cache, so always in bounds): kept when the group is
    // full (the same addresses), which takes the position's round trip to
    // memory off the start of the scan.
    const int64_t e_first = static_cast<int64_t>(blockIdx.x) * tiles_per_wg * kIdxTile +
                            static_cast<int64_t>(wave) * kGroupEnt;
#pragma unroll
    for (int tt = 0; tt < kGroup; ++tt) {
      const int64_t e = min(e_first + tt * kIdxTile + col, n_cap - 1);
      const u32x4* src = reinterpret_cast<const u32x4*>(ki + (b * n_cap + e) * kRowBytes +
                                                        g * Tr::kLaneBytes);
#pragma unroll
      for (int v = 0; v < kVec; ++v) buf0[tt][v] = src[v];
      if constexpr (DTYPE == 2) ks0[tt] = ki_scale[b * n_cap + e];
      if constexpr (DTYPE == 3) ks0[tt] = reinterpret_cast<const uint32_t*>(ki_scale)[b * n_cap + e];
    }
  }
  const int64_t t = pos0[b] + (row - b * T);
  const int64_t V = uniform64(visible_entries(t, m, n_cap));
  const int64_t tile0 = static_cast<int64_t>(blockIdx.x) * tiles_per_wg;
  const int64_t e_begin = tile0 * kIdxTile;
  if (e_begin >= V) return;

  const uint8_t* kib = ki + b * n_cap * kRowBytes;
  float* srow = scores + row * n_cap;

  // Loads are issued unconditionally (past-the-end entries read the last
  // visible row instead) so that the wait counts stay static and the next
  // group's loads really overlap the current group's MFMAs.  A column only
  // depends on its own key row, and past-the-end columns are never stored.
  // Groups that lie entirely below V are loaded from a wave-uniform base
  // pointer plus a constant per-lane offset, with no per-lane clamping, so
  // the loop needs no address temporaries and its loads stay in flight
  // across the previous group's MFMAs.  The prefetch of the next group is
  // unconditional (the last full group re-reads itself, from cache) so the
  // loop body is straight-line code with static wait counts.  A trailing
  // partial group is loaded once with clamped addresses (past-the-end
  // columns are computed from a valid row and never stored).
  const int n_ent_wg =
      static_cast<int>(min<int64_t>(V - e_begin, static_cast<int64_t>(tiles_per_wg) * kIdxTile));
  const int n_full = n_ent_wg / kGroupEnt;
  const int n_grp = (n_ent_wg + kGroupEnt - 1) / kGroupEnt;
  const uint8_t* kwg = kib + e_begin * kRowBytes;          // wave-uniform
  const uint32_t lane_off = static_cast<uint32_t>(col * kRowBytes + g * Tr::kLaneBytes);

  // Fused block compression (bf16, one query per sequence): the workgroup
  // whose entries include the block completed by the new token (entry
  // V - 1, its last) forms that entry, K and V, from the raw rows.  The
  // wave that scores the last group (the one holding entry V - 1) issues
  // the raw loads first, and just before scoring that group computes the
  // entry, stores it to kc / vc and puts the key into the loaded group
  // through its own LDS slot, so nothing waits for the global stores and
  // no other wave is involved.  A block whose raw rows are not all in the
  // raw buffer is left unwritten (and entry V - 1 is scored as stored).
  bool comp_ok = false;
  int64_t comp_src = 0;
  const int comp_grp = n_grp - 1;
  const int comp_wave = comp_grp & (kIdxWaves - 1);
  if constexpr (DTYPE == 1 && FUSED) {
    if (fc.kr != nullptr && T == 1 && (t + 1) % m == 0 && (t + 1) / m <= n_cap &&
        V - 1 >= e_begin && V - 1 < e_begin + n_ent_wg) {
      const int64_t r0 = t - m + 1 - fc.raw_pos0[b];
      comp_ok = r0 >= 0 && r0 + m <= fc.R;
      comp_src = (b * fc.R + r0) * DI;
    }
  }
  // The block's tokens (m <= kFusedMaxM) are preloaded into registers.
  constexpr int kCh = (DI + 63) / 64;  // channels per lane of the fused compression
  constexpr int kPre = kFusedMaxM;
  float ckz[kCh][kPre], ckx[kCh][kPre], cvz[kCh][kPre], cvx[kCh][kPre];
  __shared__ __attribute__((aligned(16))) uint16_t s_newk[DTYPE == 1 && FUSED ? DI : 1];
  if constexpr (DTYPE == 1 && FUSED) {
    if (comp_ok && wave == comp_wave) {
#pragma unroll
      for (int i = 0; i < kCh; ++i) {
        const int64_t o = comp_src + min(lane + 64 * i, DI - 1);
        compress_load<kPre>(fc.kr + o, fc.zk + o, DI, m, ckz[i], ckx[i]);
        compress_load<kPre>(fc.vr + o, fc.zv + o, DI, m, cvz[i], cvx[i]);
      }
    }
  }

  const float* ksc = DTYPE == 2 ? ki_scale + b * n_cap + e_begin : nullptr;
  const uint32_t* ksw =
      DTYPE == 3 ? reinterpret_cast<const uint32_t*>(ki_scale) + b * n_cap + e_begin : nullptr;
  auto load_scale = [&](int e, KScale& kd) __attribute__((always_inline)) {
    if constexpr (DTYPE == 2) kd = ksc[e];
    if constexpr (DTYPE == 3) kd = ksw[e];
  };
  auto load_full = [&](int grp, u32x4 (&dst)[kGroup][kVec], KScale (&kd)[kGroup]) {
    const uint8_t* gb = kwg + static_cast<int64_t>(grp) * (kGroupEnt * kRowBytes);
#pragma unroll
    for (int tt = 0; tt < kGroup; ++tt) {
      const u32x4* src = reinterpret_cast<const u32x4*>(gb + tt * (kIdxTile * kRowBytes) + lane_off);
#pragma unroll
      for (int v = 0; v < kVec; ++v) dst[tt][v] = src[v];
      load_scale(grp * kGroupEnt + tt * kIdxTile + col, kd[tt]);
    }
  };
  auto load_tail = [&](int grp, u32x4 (&dst)[kGroup][kVec], KScale (&kd)[kGroup]) {
#pragma unroll
    for (int tt = 0; tt < kGroup; ++tt) {
      int e = (grp * kGroup + tt) * kIdxTile + col;
      e = e < n_ent_wg - 1 ? e : n_ent_wg - 1;
      const u32x4* src = reinterpret_cast<const u32x4*>(
          kwg + static_cast<uint32_t>(e) * kRowBytes + g * Tr::kLaneBytes);
#pragma unroll
      for (int v = 0; v < kVec; ++v) dst[tt][v] = src[v];
      load_scale(e, kd[tt]);
    }
  };

  // Scores go straight out, one 16-entry tile at a time from lane group 0,
  // through a buffer descriptor whose range is this workgroup's entries (so
  // past-the-end columns are dropped by the range check), and with HIST the
  // first-digit histogram of the top-k selection is accumulated in LDS on
  // the way (rows that keep every visible entry need none).
  const __amdgpu_buffer_rsrc_t srsrc = store_rsrc(srow + e_begin, n_ent_wg * 4);
  const bool do_hist = HIST && V > topk_k;
  auto compute_group = [&](int grp, const u32x4 (&bt)[kGroup][kVec], const KScale (&kd)[kGroup]) {
    float vv[kGroup];  // the tiles' 16 scores (every lane group holds all of them)
#pragma unroll
    for (int tt = 0; tt < kGroup; ++tt) {
      f32x4 acc[4];
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (DTYPE == 3) {
        static_assert(DI == 128, "MXFP4 indexer: one 128-element MFMA step");
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
          acc[ht] = mma_fp4(a[ht][0], bt[tt][0], acc[ht], qf.sa[ht], kd[tt] >> (8 * g));
      } else {
#pragma unroll
        for (int st = 0; st < Tr::kSteps; ++st) {
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) acc[ht] = Tr::mma(a[ht], bt[tt], st, acc[ht]);
        }
      }
      float v = 0.f;
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = RELU ? relu(acc[ht][i]) : acc[ht][i];
          v = fmaf(wq[ht][i], x, v);
        }
      }
      v = sum_xor32(sum_xor16(v));
      if constexpr (DTYPE == 2) v *= kd[tt];
      vv[tt] = v;
    }
    // Write-out and histogram, up to four tiles per instruction: lane group
    // g takes tile 4r + g.  Lanes without a tile in the round, and
    // past-the-end columns, store to an offset past the descriptor's range
    // (dropped) and count into a word of their own past the bins, so every
    // lane executes both without a branch.  The bin is the top of the
    // order-preserving key: flip all bits of a negative score, set the sign
    // bit of a positive one; adding +0.0 first makes -0.0 count as +0.0.
#pragma unroll
    for (int r = 0; r < (kGroup + 3) / 4; ++r) {
      float my = vv[4 * r];
#pragma unroll
      for (int t = 1; t < 4; ++t)
        if (4 * r + t < kGroup) my = g == t ? vv[4 * r + t] : my;
      const bool live = 4 * r + g < kGroup;
      const int e = (grp * kGroup + 4 * r + g) * kIdxTile + col;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(my), srsrc,
                                            live ? static_cast<uint32_t>(e) * 4u : 0x80000000u,
                                            0, 0);
      if (HIST && do_hist) {
        const uint32_t u = __float_as_uint(my + 0.0f);
        const uint32_t bin = (u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u)) >>
                             kTopkDigit1Shift;
        const bool mine = live & (e < n_ent_wg);
        atomicAdd(&s_hist[mine ? bin : static_cast<uint32_t>(kTopkHistBins + lane)], 1u);
      }
    }
  };

  // compute_group, with the fused compression's new key put into the
  // group that holds entry V - 1 (the lanes of that column, and the
  // clamped past-the-end ones of a tail group, hold its row)
  auto compute_last = [&](int grp, u32x4 (&bt)[kGroup][kVec], const KScale (&kd)[kGroup])
      __attribute__((always_inline)) {
    if constexpr (DTYPE == 1 && FUSED) {
      if (comp_ok && grp == comp_grp) {
        const int64_t dst = (b * n_cap + V - 1) * DI;
#pragma unroll
        for (int i = 0; i < kCh; ++i) {
          const int c = lane + 64 * i;
          const float kv = compress_loaded<kPre>(ckz[i], ckx[i], m);
          const float vv = compress_loaded<kPre>(cvz[i], cvx[i], m);
          if (c < DI) {
            const uint16_t kb = f32_to_bf16(kv);
            s_newk[c] = kb;
            fc.kc[dst + c] = kb;
            fc.vc[dst + c] = f32_to_bf16(vv);
          }
        }
        // this wave's LDS writes are done before its reads below
        __builtin_amdgcn_wave_barrier();
        const int e_last = n_ent_wg - 1 - grp * kGroupEnt;  // entry V - 1 within the group
        const u32x4* nk = reinterpret_cast<const u32x4*>(
            reinterpret_cast<const uint8_t*>(s_newk) + g * Tr::kLaneBytes);
#pragma unroll
        for (int tt = 0; tt < kGroup; ++tt) {
          if (tt * kIdxTile + col >= e_last) {
#pragma unroll
            for (int v = 0; v < kVec; ++v) bt[tt][v] = nk[v];
          }
        }
      }
    }
    compute_group(grp, bt, kd);
  };

  if (do_hist) {
    for (int i = threadIdx.x; i < kTopkHistBins; i += 256) s_hist[i] = 0u;
    __syncthreads();
  }
  // This wave's full groups are wave, wave + 4, ...: n_my of them, taken in
  // pairs (one per buffer) with a single trailing group when n_my is odd.
  // Every loop iteration runs both halves, so the body is straight-line.
  const int n_my = wave < n_full ? (n_full - 1 - wave) / kIdxWaves + 1 : 0;
  // (the first group was loaded speculatively at the top; a group that is
  // not full, or past the end, is loaded again through clamped addresses)
  if (wave >= n_full) load_tail(wave, buf0, ks0);
  qf.finish(H_I, true, g);
  int j = 0;
  for (; j + 2 <= n_my; j += 2) {
    load_full(wave + (j + 1) * kIdxWaves, buf1, ks1);
    compute_group(wave + j * kIdxWaves, buf0, ks0);
    // (past the end this re-reads this wave's last group, from cache)
    load_full(wave + min(j + 2, n_my - 1) * kIdxWaves, buf0, ks0);
    compute_last(wave + (j + 1) * kIdxWaves, buf1, ks1);
  }
  if (j < n_my) compute_last(wave + j * kIdxWaves, buf0, ks0);
  if (n_full < n_grp && (n_full & (kIdxWaves - 1)) == wave) {
    load_tail(n_full, buf0, ks0);
    compute_last(n_full, buf0, ks0);
  }
  if (do_hist) {
    __syncthreads();
    uint32_t* gh = hist + row * kTopkHistBins;
    for (int i = threadIdx.x; i < kTopkHistBins; i += 256) {
      const uint32_t c = s_hist[i];
      if (c) atomicAdd(&gh[i], c);
    }
  }
}

// ------------------------------------------------------------------ prefill
//
// Many query tokens per sequence (chunked prefill): the key matrix is
// shared by every token, so it is the B operand streamed once per group of
// 8 tokens, while each wave keeps one token's queries (64 heads x 128 dims)
// in registers as A fragments.  Each 64-entry key tile is loaded
// cooperatively into double-buffered LDS (the next tile's loads are in
// flight during the current tile's 64 MFMAs per wave); B fragments are read
// from LDS with a padded row stride (no bank conflicts).
//
// The epilogue of a 16-entry column tile (ReLU, head weights, the 64-head
// sum in lane plus two lane swaps) runs while the next column tile's MFMAs
// are in flight: two accumulator sets alternate, so the matrix cores and
// the vector ALUs of a wave overlap even though the per-tile barrier keeps
// the waves in step.  Scores go out through a buffer descriptor whose range is
// the token's visible entries, so stores past V(t) are dropped by the range
// check rather than branched around.
constexpr int kPfTok = 8;        // query tokens per workgroup (one per wave)
#ifndef CSA_PF_TILE
#define CSA_PF_TILE 128
#endif
constexpr int kPfTile = CSA_PF_TILE;  // entries per LDS tile
constexpr int kPfCt = kPfTile / 16;   // column tiles per LDS tile
constexpr int kPfThreads = 64 * kPfTok;
// Score rows of the prefill path are addressed with 32-bit byte offsets.
constexpr int64_t kPfMaxEntries = int64_t(1) << 28;

//
// HIST: each wave also counts its token's scores into a 2048-bin histogram
// of their top 11 key bits in LDS (one atomic per lane for every 4 column
// tiles), then writes it whole to the top-k workspace with the row's flag.
template <int DTYPE, bool RELU, bool HIST>
__global__ __launch_bounds__(kPfThreads) void indexer_prefill_kernel(
    const uint8_t* __restrict__ qi, const float* __restrict__ qi_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ ki,
    const float* __restrict__ ki_scale, const int64_t* __restrict__ pos0, int64_t T,
    int H_I, int64_t n_cap, int m, float* __restrict__ scores, CoarseHist coarse) {
  constexpr int DI = 128;
  using Tr = IdxTraits<DTYPE, DI>;
  constexpr int kVec = Tr::kLaneBytes / 16;
  constexpr int RB = DI * Tr::kElemBytes;             // key row bytes
  constexpr int kStride = RB + 16;                    // padded LDS row
  constexpr int kLoads = kPfTile * RB / 16 / kPfThreads;  // 16-byte loads per thread per tile
  __shared__ __attribute__((aligned(16))) uint8_t bt[2][kPfTile * kStride];
  __shared__ float s_ksc[2][DTYPE == 2 ? kPfTile : 1];  // fp8 key scales of the staged tiles
  __shared__ uint32_t s_hist[HIST ? kPfTok * kTopkCoarseBins : 1];  // per wave (token)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int g = lane >> 4;
  const int64_t b = blockIdx.y;
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * kPfTok;
  const int64_t tok_last = min(tok0 + kPfTok, T) - 1;
  const int64_t p0 = pos0[b];
  const int64_t V_max = uniform64(visible_entries(p0 + tok_last, m, n_cap));
  if (V_max <= 0) return;

  // this wave's token: A fragments, head weights, score-row descriptor
  const int64_t tok = tok0 + wave;
  const bool tok_ok = tok < T;
  const int64_t row = b * T + (tok_ok ? tok : 0);
  const int64_t Vt = uniform64(tok_ok ? visible_entries(p0 + tok, m, n_cap) : 0);
  const __amdgpu_buffer_rsrc_t srsrc = store_rsrc(scores + row * n_cap, static_cast<int>(Vt * 4));
  uint32_t* my_hist = s_hist + (HIST ? wave * kTopkCoarseBins : 0);
  if (HIST)  // (only this wave touches its token's bins: no barrier)
    for (int i = lane; i < kTopkCoarseBins; i += 64) my_hist[i] = 0u;
  QueryFrags<DTYPE, DI> qf;
  qf.issue(qi, qi_scale, w, row, H_I, col, g);
  const auto& a = qf.a;
  const auto& wq = qf.wq;

  const uint8_t* kib = ki + b * n_cap * RB;
  const int ntiles = static_cast<int>((V_max + kPfTile - 1) / kPfTile);
  u32x4 breg[kLoads];
  float kreg = 0.f;  // fp8: one key scale per thread (threads < kPfTile)
  // A tile is addressed from a wave-uniform base with 32-bit per-lane
  // offsets: piece r of this thread is byte ent * RB + pc * 16 of the tile,
  // and entries past V_max are clamped to the last visible one (one min).
  auto load_tile = [&](int tile) __attribute__((always_inline)) {
    const int64_t e0 = static_cast<int64_t>(tile) * kPfTile;  // uniform
    const uint8_t* tb = kib + e0 * RB;
    const int last = static_cast<int>(min<int64_t>(kPfTile, V_max - e0)) - 1;  // >= 0
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int id = tid + kPfThreads * r;
      const int ent = id / (RB / 16);
      const int pc = id - ent * (RB / 16);
      const uint32_t off = static_cast<uint32_t>(min(ent, last) * RB + pc * 16);
      breg[r] = *reinterpret_cast<const u32x4*>(tb + off);
    }
    if (DTYPE == 2) kreg = ki_scale[b * n_cap + e0 + min(tid & (kPfTile - 1), last)];
  };
  auto store_tile = [&](auto buf) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int id = tid + kPfThreads * r;
      const int ent = id / (RB / 16);
      const int pc = id - ent * (RB / 16);
      *reinterpret_cast<u32x4*>(&bt[decltype(buf)::value][ent * kStride + pc * 16]) = breg[r];
    }
    if (DTYPE == 2 && tid < kPfTile) s_ksc[decltype(buf)::value][tid] = kreg;
  };
  // One column tile (16 entries) at a time: its 4 x kSteps MFMAs go into
  // one of two accumulator sets while the other set's epilogue runs.
  using Acc = f32x4[4];  // [head tile]
  auto mfma_ct = [&](auto buf, int ct, Acc& acc) __attribute__((always_inline)) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint8_t* src = &bt[decltype(buf)::value][(ct * 16 + col) * kStride + g * Tr::kLaneBytes];
#pragma unroll
    for (int st = 0; st < Tr::kSteps; ++st) {
      u32x4 bf[kVec / Tr::kSteps > 0 ? kVec / Tr::kSteps : 1];
#pragma unroll
      for (int v = 0; v < kVec / Tr::kSteps; ++v)
        bf[v] = *reinterpret_cast<const u32x4*>(src + (st * (kVec / Tr::kSteps) + v) * 16);
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        if (DTYPE == 1) {
          acc[ht] = mma_bf16(__builtin_bit_cast(bf16x8, a[ht][st]), __builtin_bit_cast(bf16x8, bf[0]),
                             acc[ht]);
        } else {
          i32x8 av, bv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            av[i] = static_cast<int>(a[ht][0][i]);
            av[4 + i] = static_cast<int>(a[ht][1][i]);
            bv[i] = static_cast<int>(bf[0][i]);
            bv[4 + i] = static_cast<int>(bf[1][i]);
          }
          acc[ht] = mma_fp8(av, bv, acc[ht]);
        }
      }
    }
  };
  // sum_h w_h phi(acc) for one column tile (all 64 heads: in lane, then two
  // lane swaps, after which every lane group holds the 16 column sums)
  // store offsets: lane group ct % 4 writes column ct's 16 sums; the other
  // lanes' offsets start at 2^31, past the descriptor's range (the entry
  // part added to them stays below 2^30), so their stores are dropped
  float x_own = 0.f;  // this lane group's column sum of the current group of 4 (HIST)
  uint32_t lane_off[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) lane_off[c] = g == c ? static_cast<uint32_t>(col) * 4u : 0x80000000u;
  auto epi_ct = [&](int tile, int ct, const Acc& acc) __attribute__((always_inline)) {
    float x = 0.f;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y = RELU ? relu(acc[ht][i]) : acc[ht][i];
        x = fmaf(wq[ht][i], y, x);
      }
    x = sum_xor32(sum_xor16(x));
    if (DTYPE == 2) x *= s_ksc[tile & 1][ct * 16 + col];
    const uint32_t off = lane_off[ct & 3] + static_cast<uint32_t>(tile * kPfTile + ct * 16) * 4u;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), srsrc, off, 0, 0);
    if (HIST) {
      // lane group g keeps the sum of column tile 4q + g; after every
      // fourth column tile all 64 lanes count theirs in one LDS atomic
      if (g == (ct & 3)) x_own = x;
      if ((ct & 3) == 3 && tile * kPfTile + (ct - 3 + g) * 16 + col < Vt)
        atomicAdd(&my_hist[score_key(x_own) >> kTopkCoarseShift], 1u);
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  Acc acc0, acc1;
  // Tile t: stage it, then its column tiles alternate acc0 / acc1; the
  // epilogue of each column tile runs under the next one's MFMAs (the last
  // column tile's under the next tile's first).
  static_assert(kPfCt % 2 == 0, "column tiles alternate two accumulator sets");
  static_assert(kPfCt % 4 == 0, "histogram groups of 4 column tiles stay within a tile");
  auto do_tile = [&](auto buf, int t) __attribute__((always_inline)) {
    store_tile(buf);
    __syncthreads();
    load_tile(t + 1 < ntiles ? t + 1 : t);
    mfma_ct(buf, 0, acc0);
    if (t > 0) epi_ct(t - 1, kPfCt - 1, acc1);
#pragma unroll
    for (int ct = 1; ct < kPfCt; ct += 2) {
      mfma_ct(buf, ct, acc1);
      epi_ct(t, ct - 1, acc0);
      if (ct + 1 < kPfCt) {
        mfma_ct(buf, ct + 1, acc0);
        epi_ct(t, ct, acc1);
      }
    }
  };
  load_tile(0);
  qf.finish(H_I, tok_ok, g);
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    do_tile(I0{}, t);
    do_tile(I1{}, t + 1);
  }
  if (t < ntiles) {
    do_tile(I0{}, t);
    ++t;
  }
  epi_ct(t - 1, kPfCt - 1, acc1);
  if (HIST && tok_ok) {
    uint32_t* gh = coarse.hist + row * kTopkCoarseBins;
    for (int i = lane; i < kTopkCoarseBins; i += 64) gh[i] = my_hist[i];
    if (lane == 0) coarse.flag[row] = 1u;
  }
}

// Compute units of the current device (cached per device).
static int device_cu_count() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int DTYPE, int DI>
static void launch_idx_t(const void* qi, const float* qs, const float* w, const void* ki,
                         const float* ks, const int64_t* pos0, int64_t B, int64_t T, int H_I,
                         int64_t n_cap, int m, bool relu, float* scores, uint32_t* hist, int k,
                         const FusedCompress& fc, hipStream_t s, const CoarseHist* coarse) {
  // Chunk size: about one workgroup per compute unit over the whole grid
  // (measured best for this streaming kernel), in whole rounds of load
  // groups for the 4 waves, and no more than a row.
  const int64_t tiles = (n_cap + kIdxTile - 1) / kIdxTile;
  constexpr int64_t kRound = static_cast<int64_t>(idx_group_tiles<DTYPE, DI>()) * kIdxWaves;
  int64_t tpw = (B * T * tiles + device_cu_count() - 1) / device_cu_count();
  tpw = (tpw + kRound - 1) / kRound * kRound;
  if (tpw > tiles) tpw = tiles;
  // (the workgroup's score range is a 32-bit byte count)
  if (tpw > (int64_t(1) << 24)) tpw = int64_t(1) << 24;
  const int tiles_per_wg = static_cast<int>(tpw);
  dim3 grid(static_cast<unsigned>((tiles + tiles_per_wg - 1) / tiles_per_wg),
            static_cast<unsigned>(B * T));
  auto q8 = static_cast<const uint8_t*>(qi);
  auto k8 = static_cast<const uint8_t*>(ki);
  if ((DTYPE == 1 || DTYPE == 2) && DI == 128 && T >= kPfTok && hist == nullptr &&
      n_cap <= kPfMaxEntries && fc.kr == nullptr) {
    constexpr int DT = DTYPE == 2 ? 2 : 1;
    dim3 pgrid(static_cast<unsigned>((T + kPfTok - 1) / kPfTok), static_cast<unsigned>(B));
    const CoarseHist ch = coarse ? *coarse : CoarseHist{nullptr, nullptr};
#define CSA_PF_GO(R, H)                                                                        \
  launch_kernel(indexer_prefill_kernel<DT, R, H>, pgrid, kPfThreads, s, q8, qs, w, k8, ks, pos0, T, H_I, \
                                                                n_cap, m, scores, ch)
    if (ch.hist) {
      if (relu) CSA_PF_GO(true, true); else CSA_PF_GO(false, true);
    } else {
      if (relu) CSA_PF_GO(true, false); else CSA_PF_GO(false, false);
    }
#undef CSA_PF_GO
    return;
  }
  // no coarse histograms from this path: clear their flags, so the top-k
  // reads its rows instead
  if (coarse != nullptr && coarse->flag != nullptr)
    launch_clear(coarse->flag, static_cast<size_t>(B * T) * sizeof(uint32_t), s);
  // (the fused block compression has kernels of its own, so the plain
  // decode kernels keep their register allocation)
#define CSA_IDX_GO(R, HST)                                                                   \
  do {                                                                                       \
    if (DTYPE == 1 && fc.kr != nullptr)                                                      \
      launch_kernel(indexer_kernel<DTYPE, DI, R, HST, DTYPE == 1>, grid, 256, s,                     \
          q8, qs, w, k8, ks, pos0, T, H_I, n_cap, m, tiles_per_wg, scores, hist, k, fc);     \
    else                                                                                     \
      launch_kernel(indexer_kernel<DTYPE, DI, R, HST, false>, grid, 256, s,                          \
          q8, qs, w, k8, ks, pos0, T, H_I, n_cap, m, tiles_per_wg, scores, hist, k, fc);     \
  } while (0)
  if (relu) {
    if (hist) CSA_IDX_GO(true, true); else CSA_IDX_GO(true, false);
  } else {
    if (hist) CSA_IDX_GO(false, true); else CSA_IDX_GO(false, false);
  }
#undef CSA_IDX_GO
}

int launch_index_scores(const void* qi, int dtype, const void* qs_v, const float* w,
                        const void* ki, const void* ks_v, const int64_t* pos0, int64_t B,
                        int64_t T, int64_t H_I, int64_t d_I, int64_t n_cap, int m, int act,
                        float* scores, uint32_t* hist, int k, const FusedCompress* fc,
                        hipStream_t s, const CoarseHist* coarse) {
  const bool relu = act == 0;
  const FusedCompress none{};
  const FusedCompress& fcr = fc ? *fc : none;
  const int H = static_cast<int>(H_I);
  // (fp32 scales for FP8; for MXFP4 the kernel reads them as E8M0 bytes)
  const float* qs = static_cast<const float*>(qs_v);
  const float* ks = static_cast<const float*>(ks_v);
#define CSA_IDX_CASE(DT, DI)                                                                  \
  if (dtype == DT && d_I == DI) {                                                             \
    launch_idx_t<DT, DI>(qi, qs, w, ki, ks, pos0, B, T, H, n_cap, m, relu, scores, hist, k,    \
                         fcr, s, coarse);                                                     \
    return hipGetLastError() == hipSuccess ? 0 : -1;                                          \
  }
  CSA_IDX_CASE(0, 64)
  CSA_IDX_CASE(0, 128)
  CSA_IDX_CASE(1, 64)
  CSA_IDX_CASE(1, 128)
  CSA_IDX_CASE(1, 256)
  CSA_IDX_CASE(2, 128)
  CSA_IDX_CASE(3, 128)
#undef CSA_IDX_CASE
  return -2;
}

}  // namespace csa
