// Backward pass of core attention and of the compressor.
//
// The pages describe a model trained end to end (a learned token-level
// compressor, octagono.org "Hybrid Attention: CSA and HCA"; the indexer's
// QK path trained quantization-aware, dataforcee.us "Muon Optimizer and FP4
// QAT") but give no formula for the backward pass; these kernels compute the
// derivatives of the forward definitions.  For one query row t and head h
// over its key list (logits s = scale K q, p = softmax(s) = exp(s - lse),
// o = p V, upstream gradient dout):
//   dp = V dout,  D = dout . o,  ds = p (dp - D)
//   dq = scale ds K,  dK += scale ds q,  dV += p dout
// with the key/value gradients summed over heads and over every query that
// attends the row.  No gradient flows through the top-k selection.
//
// Determinism (no float atomics): the row kernel writes each query row's
// per-slot key/value gradients (already summed over the row's heads) to a
// staging buffer; the reduction kernels then give every compressed entry
// and raw row one workgroup that finds the query rows referencing it and
// sums their contributions in ascending row order.  Every result is
// bitwise reproducible.
//
// Arithmetic: fp32 storage on the 16x16x4 fp32 MFMA; bf16 storage on the
// 16x16x32 bf16 MFMA, the fp32 operands (dout, P, dS) as bf16 hi + lo pairs
// (attend_bwd_rows_bf16_kernel).  Accumulation is fp32 either way.  The
// per-row contributions (B*T x slots x d x 8 bytes; 9.7 GB for 8192 query
// rows of 1152 slots at d = 128) are the dominant HBM traffic.
#include "common.h"
#include "kernels.h"

namespace csa {

struct BwdParams {
  const uint8_t* q;
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* idx;
  const uint8_t* kr;
  const uint8_t* vr;
  const int64_t* raw_pos0;
  const int64_t* pos0;
  const float* out;
  const float* lse;
  const float* dout;
  float* dq;
  float* gk;  // [rows][n_ent_max + W][D] key-gradient contributions
  float* gv;  // [rows][n_ent_max + W][D] value-gradient contributions
  float* dkc;
  float* dvc;
  float* dkr;
  float* dvr;
  // CSA: the query-row references of every entry, by counting sort
  uint32_t* cnt;   // [B][n_cap] references per entry (zero on entry)
  uint32_t* off;   // [B][n_cap] first reference of each entry in lst
  uint32_t* lst;   // [B][T * k] packed references, grouped by entry
  // [B * T][k] arrival rank of each reference within its entry's count;
  // lives in the (not yet written) gk staging area: the counting sort runs
  // before the row kernel
  uint32_t* rank;
  int64_t T, H, n_cap, R;
  int k, W, m;
  int n_ent_max;  // entry slots per staging row: k (CSA) or n_cap (HCA)
  float scale;
};

constexpr int kBwdChunk = 32;   // keys per chunk
constexpr float kLog2eBwd = 1.4426950408889634f;
constexpr int kBwdHeads = 64;   // head slots (4 tiles of 16)
constexpr int kBwdThreads = 512;  // row kernel: 8 waves = 4 head tiles x 2 key tiles
constexpr int kBwdMaxK = 4096;  // longest index list (staged in LDS)
// A reference (query row within the sequence, list slot) is packed as
// row << kBwdSlotBits | slot: ascending references are rows in ascending
// order, and unpacking needs no division.
constexpr int kBwdSlotBits = 12;
static_assert((1 << kBwdSlotBits) == kBwdMaxK, "slot field holds every list slot");
static_assert(kBwdMaxRows << kBwdSlotBits <= (int64_t(1) << 32),
              "packed references fit 32 bits");

template <int DTYPE>
__device__ __forceinline__ void load_row_f32(const uint8_t* src, int e0, float* dst, int n);

// n consecutive elements of a storage row starting at element e0, as fp32
// (bf16: 8 per 16-byte load; fp32: 4 per load); n is 8 (bf16) or 4 (fp32).
template <>
__device__ __forceinline__ void load_row_f32<1>(const uint8_t* src, int e0, float* dst, int) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(src + e0 * 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dst[2 * i] = __uint_as_float(v[i] << 16);
    dst[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load_row_f32<0>(const uint8_t* src, int e0, float* dst, int) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(src + e0 * 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = v[i];
}

template <int DTYPE, int D, bool HCA>
__global__ __launch_bounds__(kBwdThreads) void attend_bwd_rows_kernel(BwdParams p) {
  constexpr int NT = kBwdThreads;
  constexpr int kEb = DTYPE == 1 ? 2 : 4;     // bytes per stored element
  constexpr int kPer = 16 / kEb;              // elements per 16-byte load
  constexpr int kPieces = D / kPer;           // 16-byte pieces per row
  constexpr int kKs = D / 4;                  // fp32 k-steps over the dims
  constexpr int kDT = D / 16;                 // dim tiles
  constexpr int kS = D + 4;                   // padded fp32 row stride
  constexpr int kHs = kBwdHeads + 4;          // padded [key][head] stride
  // q and dout transposed ([dim][head]): the key / value phase reads a
  // lane's 16 heads of one dim as contiguous 16-byte pieces; the score
  // phase keeps its lane's share of its head's row in registers
  __shared__ __attribute__((aligned(16))) float sQt[D][kHs];
  __shared__ __attribute__((aligned(16))) float sdOt[D][kHs];
  __shared__ __attribute__((aligned(16))) float sK[kBwdChunk][kS];
  __shared__ __attribute__((aligned(16))) float sV[kBwdChunk][kS];
  __shared__ __attribute__((aligned(16))) float sP[kBwdChunk][kHs];
  __shared__ __attribute__((aligned(16))) float sdS[kBwdChunk][kHs];
  __shared__ float sD[kBwdHeads];
  __shared__ int s_valid[kBwdChunk];
  __shared__ int s_gslot[kBwdChunk];
  __shared__ int32_t s_ent[HCA ? 1 : kBwdMaxK];  // the row's index list

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int g = lane >> 4;
  const int64_t row = blockIdx.x;
  const int64_t b = seq_of_row(row, p.T);
  const int64_t t = p.pos0[b] + (row - b * p.T);
  const int64_t rp0 = (p.W > 0 ? p.raw_pos0 : p.pos0)[b];
  const int64_t n_ent =
      HCA ? uniform64(visible_entries(t, p.m, p.n_cap)) : static_cast<int64_t>(p.k);
  const int64_t n_slots = n_ent + p.W;
  const int64_t H = p.H;

  // q and dout rows (fp32) of all heads; head slots past H hold zeros, so
  // their probabilities and gradients are zero (lse = +inf below).
  for (int i = tid; i < kBwdHeads * kPieces; i += NT) {
    const int h = i / kPieces, pc = i % kPieces;
    float v[kPer];
    if (h < H) {
      load_row_f32<DTYPE>(p.q + ((row * H + h) * D) * kEb, pc * kPer, v, kPer);
    } else {
#pragma unroll
      for (int e = 0; e < kPer; ++e) v[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) sQt[pc * kPer + e][h] = v[e];
  }
  for (int i = tid; i < kBwdHeads * (D / 4); i += NT) {
    const int h = i / (D / 4), c4 = i % (D / 4);
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    if (h < H) v = *reinterpret_cast<const f32x4*>(p.dout + (row * H + h) * D + c4 * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) sdOt[c4 * 4 + e][h] = v[e];
  }
  // D[h] = dout . o: eight threads per head, an eighth of the dims each
  {
    static_assert(NT == 8 * kBwdHeads, "eight threads per head slot");
    const int h = tid >> 3, qd = tid & 7;
    float acc = 0.f;
    if (h < H) {
      const float* orow = p.out + (row * H + h) * D + qd * (D / 8);
      const float* grow = p.dout + (row * H + h) * D + qd * (D / 8);
      for (int c = 0; c < D / 8; ++c) acc = fmaf(grow[c], orow[c], acc);
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (qd == 0) sD[h] = acc;
  }
  // wave = (key tile kh of each 32-key chunk, head tile ht)
  const int ht = wave & 3;
  const int kh = wave >> 2;
  const int head = ht * 16 + col;
  const float lse2 = head < H ? p.lse[row * H + head] * kLog2eBwd : INFINITY;
  const float scale_log2 = p.scale * kLog2eBwd;

  f32x4 dq[kDT];
#pragma unroll
  for (int i = 0; i < kDT; ++i) dq[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint8_t* kc_b = p.kc + b * p.n_cap * D * kEb;
  const uint8_t* vc_b = p.vc + b * p.n_cap * D * kEb;
  const int n_chunks = static_cast<int>((n_slots + kBwdChunk - 1) / kBwdChunk);
  if (!HCA)
    for (int i = tid; i < p.k; i += NT) s_ent[i] = p.idx[row * p.k + i];
  __syncthreads();
  const float Dh = sD[head];
  // this lane's dims g kKs .. g kKs + kKs - 1 of its head's q and dout rows
  float qreg[kKs], oreg[kKs];
#pragma unroll
  for (int k = 0; k < kKs; ++k) {
    qreg[k] = sQt[g * kKs + k][head];
    oreg[k] = sdOt[g * kKs + k][head];
  }

  // Slot s of the key list -> its K / V rows (absent keys: row 0, masked)
  auto slot_rows = [&](int64_t s, const uint8_t*& ksrc, const uint8_t*& vsrc,
                       int& ok) __attribute__((always_inline)) {
    ksrc = kc_b;
    vsrc = vc_b;
    ok = 0;
    if (s < n_ent) {
      const int64_t e = HCA ? s : static_cast<int64_t>(s_ent[s]);
      if (e >= 0 && e < p.n_cap) {
        ksrc = kc_b + e * D * kEb;
        vsrc = vc_b + e * D * kEb;
        ok = 1;
      }
    } else if (s < n_slots) {
      const int64_t pos = t - p.W + 1 + (s - n_ent);
      const int64_t rr = pos - rp0;
      if (pos >= 0 && rr >= 0 && rr < p.R) {
        ksrc = p.kr + (b * p.R + rr) * D * kEb;
        vsrc = p.vr + (b * p.R + rr) * D * kEb;
        ok = 1;
      }
    }
  };
  // The next chunk's rows are loaded into registers while a chunk is
  // computed: piece i = tid + NT u is row i / kPieces, 16 bytes at i %
  // kPieces.  (d = 64, bf16: 256 pieces for 512 threads; the upper half
  // loads the lower half's pieces again and does not stage them.)
  constexpr int kChunkPieces = kBwdChunk * kPieces;
  constexpr int kIters = (kChunkPieces + NT - 1) / NT;
  static_assert(kChunkPieces % NT == 0 || NT % kChunkPieces == 0,
                "pieces split evenly over the threads");
  u32x4 pk[kIters], pv[kIters];
  auto fetch = [&](int c) __attribute__((always_inline)) {
    const int64_t s0 = static_cast<int64_t>(min(c, n_chunks - 1)) * kBwdChunk;
#pragma unroll
    for (int u = 0; u < kIters; ++u) {
      const int i = (tid + NT * u) % kChunkPieces;
      const uint8_t *ks, *vs;
      int ok;
      slot_rows(s0 + i / kPieces, ks, vs, ok);
      pk[u] = *reinterpret_cast<const u32x4*>(ks + (i % kPieces) * 16);
      pv[u] = *reinterpret_cast<const u32x4*>(vs + (i % kPieces) * 16);
    }
  };
  auto put = [&](float* dst, u32x4 v) __attribute__((always_inline)) {
    if (DTYPE == 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dst[2 * e] = __uint_as_float(v[e] << 16);
        dst[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = __uint_as_float(v[e]);
    }
  };
  if (n_chunks > 0) fetch(0);

  for (int c = 0; c < n_chunks; ++c) {
    // ---- stage the chunk's key / value rows (fp32) and slot table
    const int64_t s0 = static_cast<int64_t>(c) * kBwdChunk;
    if (tid < kBwdChunk) {
      const int64_t s = s0 + tid;
      const uint8_t *ks, *vs;
      int ok;
      slot_rows(s, ks, vs, ok);
      s_valid[tid] = ok;
      s_gslot[tid] = s < n_ent ? static_cast<int>(s) : p.n_ent_max + static_cast<int>(s - n_ent);
    }
#pragma unroll
    for (int u = 0; u < kIters; ++u) {
      const int i = tid + NT * u;
      if (i < kChunkPieces) {
        const int key = i / kPieces, e0 = (i % kPieces) * kPer;
        put(&sK[key][e0], pk[u]);
        put(&sV[key][e0], pv[u]);
      }
    }
    __syncthreads();
    fetch(c + 1);  // (past the end: the last chunk again, from cache)

    // ---- phase A (wave = 16 heads x the 16 keys of key tile kh): S^T,
    // dP^T, P, dS, and this key tile's share of dq
    // (the dims are summed in the order lane group g takes dims
    // g kKs .. g kKs + kKs - 1, so each lane reads its K, V, q and dout
    // values as contiguous 16-byte pieces)
    f32x4 sT, dpT;
    {
      f32x4 as = f32x4{0.f, 0.f, 0.f, 0.f}, ad = f32x4{0.f, 0.f, 0.f, 0.f};
      const float* krow = &sK[kh * 16 + col][g * kKs];
      const float* vrow = &sV[kh * 16 + col][g * kKs];
#pragma unroll
      for (int k4 = 0; k4 < kKs / 4; ++k4) {
        const f32x4 kq = *reinterpret_cast<const f32x4*>(krow + 4 * k4);
        const f32x4 vq = *reinterpret_cast<const f32x4*>(vrow + 4 * k4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          as = mma_f32(kq[j], qreg[4 * k4 + j], as);
          ad = mma_f32(vq[j], oreg[4 * k4 + j], ad);
        }
      }
      sT = as;
      dpT = ad;
    }
    float dss[4];
    {
#pragma clang fp contract(off)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kh * 16 + g * 4 + i;
        const float pr = s_valid[key] ? exp2f(sT[i] * scale_log2 - lse2) : 0.f;
        dss[i] = pr * (dpT[i] - Dh) * p.scale;
        sP[key][head] = pr;
        sdS[key][head] = dss[i];
      }
    }
    // dq^T[dim][head] += sum_key K[key][dim] dS[head][key] (scale folded)
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dq[dt] = mma_f32(sK[kh * 16 + g * 4 + i][dt * 16 + col], dss[i], dq[dt]);
    __syncthreads();

    // ---- phase B (wave = one 16-dim tile, all keys, all heads): the
    // chunk's key and value gradient contributions, summed over heads
    for (int dd = wave; dd < D / 16; dd += NT / 64) {
      const int dim0 = dd * 16;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 ak = f32x4{0.f, 0.f, 0.f, 0.f}, av = f32x4{0.f, 0.f, 0.f, 0.f};
        // (heads summed in the order lane group g takes heads 16 g ..
        // 16 g + 15: a lane's dS and P values are contiguous)
        const float* dsrow = &sdS[kt * 16 + col][g * (kBwdHeads / 4)];
        const float* prow = &sP[kt * 16 + col][g * (kBwdHeads / 4)];
        const float* qtrow = &sQt[dim0 + col][g * (kBwdHeads / 4)];
        const float* otrow = &sdOt[dim0 + col][g * (kBwdHeads / 4)];
#pragma unroll
        for (int k4 = 0; k4 < kBwdHeads / 16; ++k4) {
          const f32x4 dsv = *reinterpret_cast<const f32x4*>(dsrow + 4 * k4);
          const f32x4 pv4 = *reinterpret_cast<const f32x4*>(prow + 4 * k4);
          const f32x4 qv = *reinterpret_cast<const f32x4*>(qtrow + 4 * k4);
          const f32x4 ov = *reinterpret_cast<const f32x4*>(otrow + 4 * k4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            ak = mma_f32(qv[j], dsv[j], ak);
            av = mma_f32(ov[j], pv4[j], av);
          }
        }
        // lane (key col, g) holds dims dim0 + 4 g .. + 3 of key kt*16 + col
        const int key = kt * 16 + col;
        if (s_valid[key]) {
          const int64_t gi = (row * (p.n_ent_max + p.W) + s_gslot[key]) * D + dim0 + g * 4;
          *reinterpret_cast<f32x4*>(p.gk + gi) = ak;
          *reinterpret_cast<f32x4*>(p.gv + gi) = av;
        }
      }
    }
    __syncthreads();
  }
  // dq: the two key tiles' shares of each head, added in a fixed order
  // through the (now free) query buffer
  static_assert(sizeof(sQt) >= 4 * kDT * 64 * sizeof(f32x4), "dq exchange buffer");
  f32x4* xq = reinterpret_cast<f32x4*>(&sQt[0][0]);  // [head tile][dim tile][lane]
  if (kh == 1) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) xq[(ht * kDT + dt) * 64 + lane] = dq[dt];
  }
  __syncthreads();
  if (kh == 0 && head < H) {
    float* dst = p.dq + (row * H + head) * D;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
      *reinterpret_cast<f32x4*>(dst + dt * 16 + g * 4) = dq[dt] + xq[(ht * kDT + dt) * 64 + lane];
  }
}

// bf16 storage: every product on the 16x16x32 bf16 MFMA.  q, K and V are
// bf16 values; the fp32 operands (dout, and the probabilities P and score
// gradients dS formed here) enter as two bf16 values hi + lo (hi the
// rounded value, lo the rounded remainder: 16 significant bits, relative
// error <= 2^-17), so x y = hi_x y + lo_x y for a bf16 y and x y ~ hi_x hi_y
// + hi_x lo_y + lo_x hi_y for two such operands; accumulation is fp32.
// Per 32-key chunk:
//   phase A (wave = head tile ht x dim half dh): S^T = K q^T and dP^T =
//     V dout^T for both 16-key tiles (each head tile's two waves compute
//     them alike), P, dS, and dq^T = K^T dS for the wave's half of the
//     dims (K^T through the LDS transpose read, keys in the order of the
//     lane's P / dS registers); the dh = 0 waves store P and dS (hi, lo) in
//     LDS as [key][head];
//   phase B (wave = one 16-dim tile): dK^T = q^T dS and dV^T = dout^T P
//     over all heads, written to the staging buffer as the fp32 kernel
//     does, so the same reductions follow.
template <int D, bool HCA>
__global__ __launch_bounds__(kBwdThreads) void attend_bwd_rows_bf16_kernel(BwdParams p) {
  constexpr int NT = kBwdThreads;
  constexpr int RB = D * 2;            // bytes of a bf16 row
  constexpr int kPieces = RB / 16;     // 16-byte pieces per row
  constexpr int kSteps = D / 32;       // MFMA k-steps over the dims
  constexpr int kSpan = D / 4;         // dims of one lane group (kSteps x 8)
  constexpr int kDT = D / 16;          // dim tiles
  constexpr int kHalfDT = kDT / 2;     // dim tiles of a phase A wave
  constexpr int kRs = RB + 32;         // K / V LDS row stride (bytes)
  constexpr int kHp = kBwdHeads + 8;   // [x][head] bf16 LDS row stride (elements)
  __shared__ __attribute__((aligned(16))) uint16_t sQt[D][kHp];   // q^T
  __shared__ __attribute__((aligned(16))) uint16_t sOtH[D][kHp];  // dout^T, hi
  __shared__ __attribute__((aligned(16))) uint16_t sOtL[D][kHp];  // dout^T, lo
  __shared__ __attribute__((aligned(16))) uint8_t sK[kBwdChunk * kRs];
  __shared__ __attribute__((aligned(16))) uint8_t sV[kBwdChunk * kRs];
  __shared__ __attribute__((aligned(16))) uint16_t sPH[kBwdChunk][kHp];
  __shared__ __attribute__((aligned(16))) uint16_t sPL[kBwdChunk][kHp];
  __shared__ __attribute__((aligned(16))) uint16_t sSH[kBwdChunk][kHp];
  __shared__ __attribute__((aligned(16))) uint16_t sSL[kBwdChunk][kHp];
  __shared__ float sD[kBwdHeads];
  __shared__ int s_valid[kBwdChunk];
  __shared__ int s_gslot[kBwdChunk];
  __shared__ int32_t s_ent[HCA ? 1 : kBwdMaxK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int g = lane >> 4;
  const int64_t row = blockIdx.x;
  const int64_t b = seq_of_row(row, p.T);
  const int64_t t = p.pos0[b] + (row - b * p.T);
  const int64_t rp0 = (p.W > 0 ? p.raw_pos0 : p.pos0)[b];
  const int64_t n_ent =
      HCA ? uniform64(visible_entries(t, p.m, p.n_cap)) : static_cast<int64_t>(p.k);
  const int64_t n_slots = n_ent + p.W;
  const int64_t H = p.H;
  auto split = [](float x, uint16_t& hi, uint16_t& lo) __attribute__((always_inline)) {
    hi = f32_to_bf16(x);
    lo = f32_to_bf16(x - bf16_to_f32(hi));
  };

  // q^T and dout^T (hi, lo) of all heads in LDS; head slots past H hold
  // zeros (their probabilities and gradients are zero: lse = +inf below)
  for (int i = tid; i < kBwdHeads * kPieces; i += NT) {
    const int h = i / kPieces, pc = i % kPieces;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (h < H) v = *reinterpret_cast<const u32x4*>(p.q + ((row * H + h) * D + pc * 8) * 2);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sQt[pc * 8 + 2 * e][h] = static_cast<uint16_t>(v[e] & 0xffffu);
      sQt[pc * 8 + 2 * e + 1][h] = static_cast<uint16_t>(v[e] >> 16);
    }
  }
  for (int i = tid; i < kBwdHeads * (D / 4); i += NT) {
    const int h = i / (D / 4), c4 = i % (D / 4);
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    if (h < H) v = *reinterpret_cast<const f32x4*>(p.dout + (row * H + h) * D + c4 * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) split(v[e], sOtH[c4 * 4 + e][h], sOtL[c4 * 4 + e][h]);
  }
  // D[h] = dout . o: eight threads per head, an eighth of the dims each
  {
    static_assert(NT == 8 * kBwdHeads, "eight threads per head slot");
    const int h = tid >> 3, qd = tid & 7;
    float acc = 0.f;
    if (h < H) {
      const float* orow = p.out + (row * H + h) * D + qd * (D / 8);
      const float* grow = p.dout + (row * H + h) * D + qd * (D / 8);
      for (int c = 0; c < D / 8; ++c) acc = fmaf(grow[c], orow[c], acc);
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (qd == 0) sD[h] = acc;
  }
  // phase A roles
  const int ht = wave & 3;
  const int dh = wave >> 2;
  const int head = ht * 16 + col;
  const float lse2 = head < H ? p.lse[row * H + head] * kLog2eBwd : INFINITY;
  const float scale_log2 = p.scale * kLog2eBwd;
  // this lane's B operands of S^T and dP^T: its head's q and dout (hi, lo)
  // at dims g kSpan + 8 st .. + 8 (the K / V A operands use the same dims)
  bf16x8 qf[kSteps], ofh[kSteps], ofl[kSteps];
  {
    const int64_t hq = head < H ? head : 0;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int d0 = g * kSpan + st * 8;
      u32x4 v = *reinterpret_cast<const u32x4*>(p.q + ((row * H + hq) * D + d0) * 2);
      if (head >= H) v = u32x4{0u, 0u, 0u, 0u};
      qf[st] = __builtin_bit_cast(bf16x8, v);
      const float* dr = p.dout + (row * H + hq) * D + d0;
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(dr);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(dr + 4);
      uint16_t h8[8], l8[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        split(head < H ? x0[e] : 0.f, h8[e], l8[e]);
        split(head < H ? x1[e] : 0.f, h8[4 + e], l8[4 + e]);
      }
      u32x4 ph, pl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ph[e] = static_cast<uint32_t>(h8[2 * e]) | (static_cast<uint32_t>(h8[2 * e + 1]) << 16);
        pl[e] = static_cast<uint32_t>(l8[2 * e]) | (static_cast<uint32_t>(l8[2 * e + 1]) << 16);
      }
      ofh[st] = __builtin_bit_cast(bf16x8, ph);
      ofl[st] = __builtin_bit_cast(bf16x8, pl);
    }
  }

  f32x4 dq[kHalfDT];
#pragma unroll
  for (int i = 0; i < kHalfDT; ++i) dq[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint8_t* kc_b = p.kc + b * p.n_cap * RB;
  const uint8_t* vc_b = p.vc + b * p.n_cap * RB;
  const int n_chunks = static_cast<int>((n_slots + kBwdChunk - 1) / kBwdChunk);
  if (!HCA)
    for (int i = tid; i < p.k; i += NT) s_ent[i] = p.idx[row * p.k + i];
  __syncthreads();
  const float Dh = sD[head];

  // Slot s of the key list -> its K / V rows (absent keys: row 0, masked)
  auto slot_rows = [&](int64_t s, const uint8_t*& ksrc, const uint8_t*& vsrc,
                       int& ok) __attribute__((always_inline)) {
    ksrc = kc_b;
    vsrc = vc_b;
    ok = 0;
    if (s < n_ent) {
      const int64_t e = HCA ? s : static_cast<int64_t>(s_ent[s]);
      if (e >= 0 && e < p.n_cap) {
        ksrc = kc_b + e * RB;
        vsrc = vc_b + e * RB;
        ok = 1;
      }
    } else if (s < n_slots) {
      const int64_t pos = t - p.W + 1 + (s - n_ent);
      const int64_t rr = pos - rp0;
      if (pos >= 0 && rr >= 0 && rr < p.R) {
        ksrc = p.kr + (b * p.R + rr) * RB;
        vsrc = p.vr + (b * p.R + rr) * RB;
        ok = 1;
      }
    }
  };
  // the next chunk's rows are loaded into registers while a chunk is
  // computed: piece i = tid + NT u is row i / kPieces, 16 bytes at i %
  // kPieces (d = 64: the upper half of the threads repeats the lower's)
  constexpr int kChunkPieces = kBwdChunk * kPieces;
  constexpr int kIters = (kChunkPieces + NT - 1) / NT;
  static_assert(kChunkPieces % NT == 0 || NT % kChunkPieces == 0,
                "pieces split evenly over the threads");
  u32x4 pk[kIters], pv[kIters];
  auto fetch = [&](int c) __attribute__((always_inline)) {
    const int64_t s0 = static_cast<int64_t>(min(c, n_chunks - 1)) * kBwdChunk;
#pragma unroll
    for (int u = 0; u < kIters; ++u) {
      const int i = (tid + NT * u) % kChunkPieces;
      const uint8_t *ks, *vs;
      int ok;
      slot_rows(s0 + i / kPieces, ks, vs, ok);
      pk[u] = *reinterpret_cast<const u32x4*>(ks + (i % kPieces) * 16);
      pv[u] = *reinterpret_cast<const u32x4*>(vs + (i % kPieces) * 16);
    }
  };
  if (n_chunks > 0) fetch(0);

  for (int c = 0; c < n_chunks; ++c) {
    // ---- stage the chunk's key / value rows and slot table
    const int64_t s0 = static_cast<int64_t>(c) * kBwdChunk;
    if (tid < kBwdChunk) {
      const int64_t s = s0 + tid;
      const uint8_t *ks, *vs;
      int ok;
      slot_rows(s, ks, vs, ok);
      s_valid[tid] = ok;
      s_gslot[tid] = s < n_ent ? static_cast<int>(s) : p.n_ent_max + static_cast<int>(s - n_ent);
    }
#pragma unroll
    for (int u = 0; u < kIters; ++u) {
      const int i = tid + NT * u;
      if (i < kChunkPieces) {
        const int key = i / kPieces, pc = i % kPieces;
        *reinterpret_cast<u32x4*>(&sK[key * kRs + pc * 16]) = pk[u];
        *reinterpret_cast<u32x4*>(&sV[key * kRs + pc * 16]) = pv[u];
      }
    }
    __syncthreads();
    fetch(c + 1);  // (past the end: the last chunk again, from cache)

    // ---- phase A: S^T, dP^T for both key tiles (rows 16 j + 4 g + i of
    // this lane's head column), P, dS
    uint16_t ph8[8], pl8[8], sh8[8], sl8[8];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x4 sT = f32x4{0.f, 0.f, 0.f, 0.f}, dpT = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint8_t* krow = &sK[(j * 16 + col) * kRs + g * kSpan * 2];
      const uint8_t* vrow = &sV[(j * 16 + col) * kRs + g * kSpan * 2];
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        const bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + st * 16));
        const bf16x8 va = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vrow + st * 16));
        sT = mma_bf16(ka, qf[st], sT);
        dpT = mma_bf16(va, ofh[st], dpT);
        dpT = mma_bf16(va, ofl[st], dpT);
      }
      {
#pragma clang fp contract(off)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = j * 16 + g * 4 + i;
          const float pr = s_valid[key] ? exp2f(sT[i] * scale_log2 - lse2) : 0.f;
          const float ds = pr * (dpT[i] - Dh) * p.scale;
          split(pr, ph8[j * 4 + i], pl8[j * 4 + i]);
          split(ds, sh8[j * 4 + i], sl8[j * 4 + i]);
        }
      }
    }
    if (dh == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = j * 16 + g * 4 + i;
          sPH[key][head] = ph8[j * 4 + i];
          sPL[key][head] = pl8[j * 4 + i];
          sSH[key][head] = sh8[j * 4 + i];
          sSL[key][head] = sl8[j * 4 + i];
        }
    }
    // dq^T[dim][head] += sum_key K[key][dim] dS[head][key] (scale folded):
    // A = K^T read transposed, keys 4 g .. 4 g + 3 and 16 + 4 g .. + 3 in the
    // order of the lane's dS values
    {
      u32x4 bh, bl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bh[e] = static_cast<uint32_t>(sh8[2 * e]) | (static_cast<uint32_t>(sh8[2 * e + 1]) << 16);
        bl[e] = static_cast<uint32_t>(sl8[2 * e]) | (static_cast<uint32_t>(sl8[2 * e + 1]) << 16);
      }
      const bf16x8 dsh = __builtin_bit_cast(bf16x8, bh), dsl = __builtin_bit_cast(bf16x8, bl);
      const uint8_t* kbase = sK + (4 * g + (col >> 2)) * kRs + (col & 3) * 8;
#pragma unroll
      for (int d = 0; d < kHalfDT; ++d) {
        const int dt = dh * kHalfDT + d;
        const u32x2 lo = lds_read_tr16(kbase + dt * 32);
        const u32x2 hi = lds_read_tr16(kbase + 16 * kRs + dt * 32);
        const bf16x8 ka = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        dq[d] = mma_bf16(ka, dsh, dq[d]);
        dq[d] = mma_bf16(ka, dsl, dq[d]);
      }
    }
    __syncthreads();

    // ---- phase B (wave = one 16-dim tile, both key tiles, all heads):
    // dK^T = q^T dS and dV^T = dout^T P; lane (key col, g) ends with dims
    // 4 g .. 4 g + 3 of its key
    for (int dd = wave; dd < kDT; dd += NT / 64) {
      const int dim = dd * 16 + col;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int key = kt * 16 + col;
        f32x4 ak = f32x4{0.f, 0.f, 0.f, 0.f}, av = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hb = 0; hb < kBwdHeads / 32; ++hb) {
          const int h0 = hb * 32 + g * 8;
          const bf16x8 qa = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sQt[dim][h0]));
          const bf16x8 oah = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sOtH[dim][h0]));
          const bf16x8 oal = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sOtL[dim][h0]));
          const bf16x8 sbh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sSH[key][h0]));
          const bf16x8 sbl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sSL[key][h0]));
          const bf16x8 pbh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sPH[key][h0]));
          const bf16x8 pbl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sPL[key][h0]));
          ak = mma_bf16(qa, sbh, ak);
          ak = mma_bf16(qa, sbl, ak);
          av = mma_bf16(oah, pbh, av);
          av = mma_bf16(oah, pbl, av);
          av = mma_bf16(oal, pbh, av);
        }
        if (s_valid[key]) {
          const int64_t gi = (row * (p.n_ent_max + p.W) + s_gslot[key]) * D + dd * 16 + g * 4;
          *reinterpret_cast<f32x4*>(p.gk + gi) = ak;
          *reinterpret_cast<f32x4*>(p.gv + gi) = av;
        }
      }
    }
    __syncthreads();
  }
  // dq: each dim half from its own wave
  if (head < H) {
    float* dst = p.dq + (row * H + head) * D;
#pragma unroll
    for (int d = 0; d < kHalfDT; ++d)
      *reinterpret_cast<f32x4*>(dst + (dh * kHalfDT + d) * 16 + g * 4) = dq[d];
  }
}

// HCA: key / value gradients of compressed entry j of sequence b, the sum
// of the contributions of every query row that sees it (all of them attend
// it), in ascending row order.
template <int D, bool HCA>
__global__ __launch_bounds__(256) void attend_bwd_entries_kernel(BwdParams p) {
  __shared__ int s_row[256];
  __shared__ int s_slot[256];
  __shared__ int s_cnt[5];
  const int tid = threadIdx.x;
  const int64_t j = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t pos0 = p.pos0[b];
  // HCA: the rows whose position sees entry j, t >= (j + 1) m - 1; CSA:
  // every row is searched (its list says whether it selected j)
  int64_t i0 = HCA ? (j + 1) * p.m - 1 - pos0 : 0;
  if (i0 < 0) i0 = 0;
  const int64_t n_slots_row = p.n_ent_max + p.W;
  const int dim = tid % D;
  const bool is_v = tid >= D;  // threads D .. 2D-1 sum values (D = 128); D = 64: both halves
  float acc_k = 0.f, acc_v = 0.f;
  for (int64_t base = i0; base < p.T; base += 256) {
    const int64_t i = base + tid;
    int slot = -1;
    if (i < p.T) {
      const int64_t rowi = b * p.T + i;
      (void)rowi;
      slot = static_cast<int>(j);
    }
    // compact the hits in row order (one block prefix over the flags)
    const unsigned long long bal = __ballot(slot >= 0);
    const int w = tid >> 6;
    if ((tid & 63) == 0) s_cnt[w] = __popcll(bal);
    __syncthreads();
    if (tid == 0) {
      int a = 0;
      for (int x = 0; x < 4; ++x) { const int c = s_cnt[x]; s_cnt[x] = a; a += c; }
      s_cnt[4] = a;
    }
    __syncthreads();
    if (slot >= 0) {
      const int r = s_cnt[w] + static_cast<int>(__popcll(bal & ((1ull << (tid & 63)) - 1ull)));
      s_row[r] = static_cast<int>(i);
      s_slot[r] = slot;
    }
    __syncthreads();
    const int n_hit = s_cnt[4];
    for (int r = 0; r < n_hit; ++r) {
      const int64_t gi = ((b * p.T + s_row[r]) * n_slots_row + s_slot[r]) * D + dim;
      if (D == 128) {
        if (is_v) acc_v += p.gv[gi]; else acc_k += p.gk[gi];
      } else {
        acc_k += p.gk[gi];
        acc_v += p.gv[gi];
      }
    }
    __syncthreads();
  }
  const int64_t o = (b * p.n_cap + j) * D + dim;
  if (D == 128) {
    if (is_v) p.dvc[o] = acc_v; else p.dkc[o] = acc_k;
  } else if (tid < D) {
    p.dkc[o] = acc_k;
    p.dvc[o] = acc_v;
  }
}

// ---- CSA: inverse of the index lists (which rows attended each entry)

constexpr int kBwdMaxRefs = 16384;  // references of one entry kept in LDS (= rows per sequence)
// A row's index list is strictly ascending (the ABI's contract, which
// csa_topk's output meets), so an entry has at most one reference per query
// row and at most kBwdMaxRows per sequence: the largest list fits.
static_assert(kBwdMaxRefs >= kBwdMaxRows, "an entry's references must fit the reduction's LDS");

__device__ __forceinline__ bool bwd_entry_ok(int32_t e, int64_t n_cap) {
  return e >= 0 && e < n_cap;
}

// cnt[b][j] = number of (row, slot) pairs of sequence b that hold entry j.
__global__ __launch_bounds__(256) void attend_bwd_count_kernel(BwdParams p) {
  const int64_t row = blockIdx.x;
  const int64_t b = row / p.T;
  for (int s = threadIdx.x; s < p.k; s += 256) {
    const int32_t e = p.idx[row * p.k + s];
    if (bwd_entry_ok(e, p.n_cap)) p.rank[row * p.k + s] = atomicAdd(&p.cnt[b * p.n_cap + e], 1u);
  }
}

// off[b][:] = exclusive prefix sum of cnt[b][:] (one workgroup per sequence,
// a contiguous run of entries per thread).
__global__ __launch_bounds__(256) void attend_bwd_scan_kernel(BwdParams p) {
  __shared__ uint32_t part[256];
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t per = (p.n_cap + 255) / 256;
  const int64_t j0 = min(p.n_cap, tid * per), j1 = min(p.n_cap, j0 + per);
  const uint32_t* c = p.cnt + b * p.n_cap;
  uint32_t sum = 0;
  for (int64_t j = j0; j < j1; ++j) sum += c[j];
  part[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    uint32_t a = 0;
    for (int i = 0; i < 256; ++i) { const uint32_t v = part[i]; part[i] = a; a += v; }
  }
  __syncthreads();
  uint32_t a = part[tid] + static_cast<uint32_t>(b * p.T * p.k);
  uint32_t* o = p.off + b * p.n_cap;
  for (int64_t j = j0; j < j1; ++j) { o[j] = a; a += c[j]; }
}

// lst[off[j] + i] = the packed (row, slot) of the reference to entry j that
// arrived i-th in the count kernel (its rank, so no atomics here; the
// reduction sorts each entry's references).
__global__ __launch_bounds__(256) void attend_bwd_fill_kernel(BwdParams p) {
  const int64_t row = blockIdx.x;
  const int64_t b = row / p.T;
  const int64_t rl = row - b * p.T;
  for (int s = threadIdx.x; s < p.k; s += 256) {
    const int32_t e = p.idx[row * p.k + s];
    if (bwd_entry_ok(e, p.n_cap)) {
      const uint32_t at = p.off[b * p.n_cap + e] + p.rank[row * p.k + s];
      p.lst[at] = static_cast<uint32_t>((rl << kBwdSlotBits) | s);
    }
  }
}

// Key / value gradients of entry j of sequence b: its references sorted
// ascending (row order; a row holds an entry at most once), then the
// contributions summed in that order, kBwdSumBatch loads in flight.  Lists
// of up to CAP references are sorted in LDS by this kernel; the BIG variant
// (CAP = kBwdMaxRefs) takes only the entries whose list is longer.
constexpr int kBwdSmallRefs = 2048;
constexpr int kBwdSumBatch = 16;

template <int D, int CAP, bool BIG>
__global__ __launch_bounds__(256) void attend_bwd_entries_csr_kernel(BwdParams p) {
  __shared__ uint32_t refs[CAP];
  const int tid = threadIdx.x;
  const int64_t j = blockIdx.x;
  const int64_t b = blockIdx.y;
  // (at most one reference per row, since index rows are strictly
  // ascending; the clamp only keeps lists that break that contract inside
  // the buffer)
  const int n_all = static_cast<int>(p.cnt[b * p.n_cap + j]);
  if (BIG != (n_all > kBwdSmallRefs)) return;  // the other variant's entry
  const int n = min(n_all, CAP);
  const uint32_t o = p.off[b * p.n_cap + j];
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  for (int i = tid; i < n2; i += 256) refs[i] = i < n ? p.lst[o + i] : 0xffffffffu;
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n2; i += 256) {
        const int q = i ^ stride;
        if (q > i) {
          const uint32_t a = refs[i], c = refs[q];
          if ((a > c) == ((i & size) == 0)) {
            refs[i] = c;
            refs[q] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  const int64_t n_slots_row = p.n_ent_max + p.W;
  const int dim = tid % D;
  const bool is_v = D == 128 && tid >= D;
  const float* src = is_v ? p.gv : p.gk;
  float acc_k = 0.f, acc_v = 0.f;
  for (int r0 = 0; r0 < n; r0 += kBwdSumBatch) {
    float vk[kBwdSumBatch], vv[kBwdSumBatch];
#pragma unroll
    for (int u = 0; u < kBwdSumBatch; ++u) {
      const uint32_t ref = refs[min(r0 + u, n - 1)];
      const int64_t rl = ref >> kBwdSlotBits, slot = ref & (kBwdMaxK - 1);
      const int64_t gi = ((b * p.T + rl) * n_slots_row + slot) * D + dim;
      vk[u] = src[gi];
      vv[u] = D == 128 ? 0.f : p.gv[gi];
    }
#pragma unroll
    for (int u = 0; u < kBwdSumBatch; ++u) {
      if (r0 + u < n) {
        acc_k += vk[u];
        acc_v += vv[u];
      }
    }
  }
  const int64_t oo = (b * p.n_cap + j) * D + dim;
  if (D == 128) {
    (is_v ? p.dvc : p.dkc)[oo] = acc_k;
  } else if (tid < D) {
    p.dkc[oo] = acc_k;
    p.dvc[oo] = acc_v;
  }
}

// Key / value gradients of raw row r of sequence b (position raw_pos0 + r):
// the rows whose window holds it, t in [pos, pos + W - 1], in row order.
template <int D>
__global__ __launch_bounds__(256) void attend_bwd_raw_kernel(BwdParams p) {
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t pos = p.raw_pos0[b] + r;
  const int64_t pos0 = p.pos0[b];
  const int64_t n_slots_row = p.n_ent_max + p.W;
  const int dim = tid % D;
  const bool is_v = tid >= D;
  float acc_k = 0.f, acc_v = 0.f;
  int64_t i0 = pos - pos0, i1 = pos - pos0 + p.W;  // rows [i0, i1)
  if (i0 < 0) i0 = 0;
  if (i1 > p.T) i1 = p.T;
  if (pos >= 0) {
    for (int64_t i = i0; i < i1; ++i) {
      const int64_t t = pos0 + i;
      const int64_t slot = p.n_ent_max + (pos - (t - p.W + 1));
      const int64_t gi = ((b * p.T + i) * n_slots_row + slot) * D + dim;
      if (D == 128) {
        if (is_v) acc_v += p.gv[gi]; else acc_k += p.gk[gi];
      } else {
        acc_k += p.gk[gi];
        acc_v += p.gv[gi];
      }
    }
  }
  const int64_t o = (b * p.R + r) * D + dim;
  if (D == 128) {
    if (is_v) p.dvr[o] = acc_v; else p.dkr[o] = acc_k;
  } else if (tid < D) {
    p.dkr[o] = acc_k;
    p.dvr[o] = acc_v;
  }
}

static size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// Workspace: the key / value contributions [B*T][n_ent_max + W][D] fp32,
// then (CSA) cnt, off [B][n_cap] and the reference list [B*T*k].
size_t attend_bwd_workspace_bytes(int64_t B, int64_t T, int64_t D, int64_t n_ent_max, int W,
                                  int64_t n_cap, bool csa) {
  size_t bytes = align256(static_cast<size_t>(B * T) * (n_ent_max + W) * D * sizeof(float) * 2);
  if (csa)
    bytes += 2 * align256(static_cast<size_t>(B * n_cap) * 4) +
             align256(static_cast<size_t>(B * T) * n_ent_max * 4);
  return bytes;
}

int launch_attend_bwd(const void* q, int dtype, const void* kc, const void* vc,
                      const int32_t* idx, int k, int hca_m, const void* kr, const void* vr,
                      const int64_t* raw_pos0, int64_t R, const int64_t* pos0, int64_t B,
                      int64_t T, int64_t H, int64_t D, int64_t n_cap, int W, float scale,
                      const float* out, const float* lse, const float* dout, float* dq,
                      float* dkc, float* dvc, float* dkr, float* dvr, void* ws,
                      hipStream_t stream) {
  const bool hca = hca_m > 0;
  BwdParams p;
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
  p.dout = dout;
  p.dq = dq;
  p.dkc = dkc;
  p.dvc = dvc;
  p.dkr = dkr;
  p.dvr = dvr;
  p.T = T;
  p.H = H;
  p.n_cap = n_cap;
  p.R = R;
  p.k = k;
  p.W = W;
  p.m = hca ? hca_m : 1;
  p.n_ent_max = hca ? static_cast<int>(n_cap) : k;
  p.scale = scale;
  const int64_t rows = B * T;
  float* base = static_cast<float*>(ws);
  p.gk = base;
  p.gv = base + rows * (p.n_ent_max + W) * D;
  p.cnt = p.off = p.lst = p.rank = nullptr;
  if (!hca) {
    char* c = static_cast<char*>(ws) +
              align256(static_cast<size_t>(rows) * (p.n_ent_max + W) * D * sizeof(float) * 2);
    const size_t nb = align256(static_cast<size_t>(B * n_cap) * 4);
    p.cnt = reinterpret_cast<uint32_t*>(c);
    p.off = reinterpret_cast<uint32_t*>(c + nb);
    p.lst = reinterpret_cast<uint32_t*>(c + 2 * nb);
    p.rank = reinterpret_cast<uint32_t*>(p.gk);  // rows * k words <= the gk area
    if (launch_clear(p.cnt, nb, stream)) return -1;
  }
#define CSA_BWD_CASE(DT, DD)                                                                  \
  if (dtype == DT && D == DD) {                                                               \
    if (hca) {                                                                                \
      if (DT == 1)                                                                            \
        attend_bwd_rows_bf16_kernel<DD, true><<<dim3(rows), kBwdThreads, 0, stream>>>(p);      \
      else                                                                                    \
        attend_bwd_rows_kernel<DT, DD, true><<<dim3(rows), kBwdThreads, 0, stream>>>(p);       \
      attend_bwd_entries_kernel<DD, true><<<dim3(n_cap, B), 256, 0, stream>>>(p);              \
    } else {                                                                                  \
      /* the counting sort needs only the index lists; its ranks use the */                   \
      /* staging area before the row kernel fills it */                                       \
      attend_bwd_count_kernel<<<dim3(rows), 256, 0, stream>>>(p);                              \
      attend_bwd_scan_kernel<<<dim3(B), 256, 0, stream>>>(p);                                  \
      attend_bwd_fill_kernel<<<dim3(rows), 256, 0, stream>>>(p);                               \
      if (DT == 1)                                                                            \
        attend_bwd_rows_bf16_kernel<DD, false><<<dim3(rows), kBwdThreads, 0, stream>>>(p);     \
      else                                                                                    \
        attend_bwd_rows_kernel<DT, DD, false><<<dim3(rows), kBwdThreads, 0, stream>>>(p);      \
      attend_bwd_entries_csr_kernel<DD, kBwdSmallRefs, false>                                  \
          <<<dim3(n_cap, B), 256, 0, stream>>>(p);                                             \
      attend_bwd_entries_csr_kernel<DD, kBwdMaxRefs, true>                                     \
          <<<dim3(n_cap, B), 256, 0, stream>>>(p);                                             \
    }                                                                                         \
    if (R > 0) attend_bwd_raw_kernel<DD><<<dim3(R, B), 256, 0, stream>>>(p);                   \
    return hipGetLastError() == hipSuccess ? 0 : -1;                                          \
  }
  CSA_BWD_CASE(0, 64)
  CSA_BWD_CASE(0, 128)
  CSA_BWD_CASE(1, 64)
  CSA_BWD_CASE(1, 128)
#undef CSA_BWD_CASE
  return -2;
}

}  // namespace csa
