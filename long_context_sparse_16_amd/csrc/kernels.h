// Internal launchers of the CSA kernels (not part of the public ABI).
// Each returns 0 on success, -1 if the HIP runtime reported a launch error,
// -2 if no kernel variant matches the (already validated) arguments.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

// Kernel timing (csa_time_next_kernels): the events a launch records
// around itself, taken from the calling host thread's pending request;
// both null when there is none.
struct LaunchEvents {
  hipEvent_t start;  // recorded when the kernel starts
  hipEvent_t stop;   // recorded when the kernel ends
};
LaunchEvents take_launch_events();

// Every kernel of the forward calls is launched through here: a plain
// launch, or, when a timing request is pending, hipExtLaunchKernelGGL with
// the request's events (the kernel's own start / end, without the dispatch
// around it).  Arguments are converted to the kernel's parameter types.
template <typename... P, typename... A>
inline void launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s,
                          A... args) {
  const LaunchEvents ev = take_launch_events();
  if (ev.start != nullptr || ev.stop != nullptr)
    hipExtLaunchKernelGGL(kernel, grid, block, 0u, s, ev.start, ev.stop, 0u,
                          static_cast<P>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0u, s, static_cast<P>(args)...);
}

// Block compression fused into the decode indexer (bf16 caches): when the
// new token at t completes a block ((t + 1) % m == 0), the block's K and V
// entries are formed from the raw rows of positions t - m + 1 .. t and
// written to entry (t + 1) / m - 1 of kc / vc before that entry is scored.
// kr == nullptr disables it.  Blocks of at most kFusedMaxM tokens.
constexpr int kFusedMaxM = 4;
struct FusedCompress {
  const uint16_t* kr;        // [B][R][d] raw keys; row r holds position raw_pos0[b] + r
  const uint16_t* vr;        // [B][R][d] raw values
  const float* zk;           // [B][R][d] compressor logits of the raw keys
  const float* zv;           // [B][R][d] compressor logits of the raw values
  const int64_t* raw_pos0;   // [B]
  uint16_t* kc;              // [B][n_cap][d] compressed keys (the indexer keys)
  uint16_t* vc;              // [B][n_cap][d] compressed values
  int64_t R;
};

int launch_compress(const void* x, int dtype, const float* z, int64_t B, int64_t n_tok, int64_t d,
                    int m, int64_t x_sb, int64_t z_sb, void* cache, int64_t n_cap,
                    int64_t first_entry, hipStream_t s);

int launch_quantize_fp8_rows(const void* x, int dtype, int64_t rows, int64_t d, uint8_t* codes,
                             float* scales, hipStream_t s);
int launch_quantize_mxfp4_rows(const void* x, int dtype, int64_t rows, int64_t d, uint8_t* codes,
                               uint8_t* scales, hipStream_t s);

// Top-k first digit: the 12 most significant bits of the order-preserving
// score key (4096 bins).
constexpr int kTopkDigit1Shift = 20;
constexpr int kTopkHistBins = 1 << (32 - kTopkDigit1Shift);

// Coarse first-digit histograms of the many-row top-k (the top 11 key
// bits, 2048 bins per row), each written whole by the prefill indexer
// together with a per-row flag that the top-k clears after use.
constexpr int kTopkCoarseShift = 21;
constexpr int kTopkCoarseBins = 1 << (32 - kTopkCoarseShift);
struct CoarseHist {
  uint32_t* hist;  // [rows][kTopkCoarseBins]
  uint32_t* flag;  // [rows]: 1 when hist holds this call's row
};

// hist (nullable): per-row first-digit histogram accumulated for csa_topk
// (rows with V <= k are skipped).  It must be zero on entry.  coarse
// (nullable): the many-row histograms, written when the prefill kernel
// runs.  qs / ks are fp32 row scales (dtype 2, FP8) or E8M0 block-scale
// bytes (dtype 3, MXFP4).  fc (nullable): block compression fused into the
// launch (bf16, T == 1).
int launch_index_scores(const void* qi, int dtype, const void* qs, const float* w,
                        const void* ki, const void* ks, const int64_t* pos0, int64_t B,
                        int64_t T, int64_t H_I, int64_t d_I, int64_t n_cap, int m, int act,
                        float* scores, uint32_t* hist, int k, const FusedCompress* fc,
                        hipStream_t s, const CoarseHist* coarse = nullptr);

// Rows (B*T) up to this count use the multi-workgroup split top-k, which
// needs a workspace; more rows use one workgroup per row, whose workspace
// (optional) holds the coarse histograms.
constexpr int64_t kTopkSplitMaxRows = 256;
size_t topk_workspace_bytes(int64_t B, int64_t T, int64_t n_cap, int k);
// The first-digit histogram inside a top-k workspace (nullptr when the row
// path, which keeps its histogram in LDS, will be used).
uint32_t* topk_hist_ptr(void* ws, int64_t B, int64_t T);
// Bytes at the start of a top-k workspace that must be zero on entry (the
// histograms and counters; the rest is written before it is read).
size_t topk_zero_state_bytes(int64_t B, int64_t T);
// The coarse histograms inside a many-row top-k workspace ({nullptr,
// nullptr} for B*T <= kTopkSplitMaxRows or no workspace).
CoarseHist topk_coarse_hist(void* ws, int64_t B, int64_t T);
int launch_topk(const float* scores, const int64_t* pos0, int64_t B, int64_t T, int64_t n_cap,
                int m, int k, int32_t* idx, void* ws, bool hist_ready, hipStream_t s);

// What the attention launch needs to make the top-k selection itself: the
// split top-k's per-slice lists (every entry whose first digit is at or
// above the row's cut bucket, in entry order, with its key), or, for rows
// of at most kSelRegEntries entries (regs != 0), only the scores and the
// first-digit histograms (each workgroup then holds its row's scores in
// registers and no classify launch precedes it).
constexpr int64_t kSelMaxSlices = 256;      // rows of up to 2^20 entries
constexpr int64_t kSelRegEntries = 32768;   // 64 scores per thread of a 512-thread workgroup
struct TopkLists {
  const uint32_t* cnt;   // [rows][n_sl][2]: listed entries, candidates among them
  const int32_t* lidx;   // [rows][n_sl][4096]
  const uint32_t* lkey;  // [rows][n_sl][4096]
  const uint32_t* ctrl;  // [rows][4]: [0] the cut bucket b1
  uint32_t* hist;        // [rows][4096]: first-digit histograms, zeroed by the consumer
  int64_t n_sl;          // slices allocated per row
  int m;                 // compression ratio (visible entries V(t))
  int regs;              // select from the scores (n_cap <= kSelRegEntries, n_cap % 4 == 0)
  const float* scores;   // [rows][n_cap], 16-byte aligned (regs only)
  int32_t* idx;          // [rows][k] output: the selection, ascending, -1 padded
};
// Only the first half of the split top-k (classify; nothing but the
// histograms, when the indexer did not build them, for rows the attention
// launch selects from registers); returns 1 (nothing launched) when the
// split path does not apply to these sizes or the row needs more than
// kSelMaxSlices slices.
int launch_topk_lists(const float* scores, const int64_t* pos0, int64_t B, int64_t T,
                      int64_t n_cap, int m, int k, void* ws, bool hist_ready, TopkLists* lists,
                      hipStream_t s);
// Zero-fill (a kernel, so it may be captured in a graph).
int launch_clear(void* p, size_t bytes, hipStream_t s);

// The fixed per-device scratch of the allocation-free entry points.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
// The current device's scratch address for a call with `rows` query rows
// over n_cap entries whose first zero_bytes bytes must be zero on entry.
// The whole array is zeroed (on stream s) at its first use on the device
// and after a failed call marked it dirty; otherwise the first zero_bytes
// are zeroed when (rows, n_cap) differ from the previous call's, since a
// call of the same sizes leaves that part zero.  Returns 0, or -1 when the
// HIP runtime reported an error.
int static_scratch(hipStream_t s, int64_t rows, int64_t n_cap, size_t zero_bytes, void** out);
// A call that launched work and then failed may leave the zero-state parts
// of the scratch (the top-k histograms) dirty: clear all of it next time.
void static_scratch_mark_dirty();

struct AttSplit {
  int splits;
  int chunks_per_split;
};
AttSplit attend_split(int64_t rows, int64_t n_slots_max, bool hca);
size_t attend_workspace_bytes(int64_t rows, int64_t H, int64_t D, int64_t n_slots_max, bool hca);
// hca_m > 0 selects HCA (all visible entries, idx ignored).  sel
// (nullable, CSA): make the top-k selection from these lists inside the
// launch (writing sel->idx) instead of reading idx.
int launch_attend(const void* q, int dtype, const void* kc, const void* vc, const int32_t* idx,
                  int k, int hca_m, const void* kr, const void* vr, const int64_t* raw_pos0,
                  int64_t R, const int64_t* pos0, int64_t B, int64_t T, int64_t H, int64_t D,
                  int64_t n_cap, int W, float scale, float* out, float* lse, void* ws,
                  hipStream_t stream, const TopkLists* sel = nullptr);

// Backward pass (fp32 gradients).  The workspace holds the per-row key /
// value gradient contributions: attend_bwd_workspace_bytes() bytes.
size_t attend_bwd_workspace_bytes(int64_t B, int64_t T, int64_t D, int64_t n_ent_max, int W,
                                  int64_t n_cap, bool csa);
constexpr int64_t kBwdMaxRows = 16384;  // CSA backward: query rows per sequence
int launch_attend_bwd(const void* q, int dtype, const void* kc, const void* vc,
                      const int32_t* idx, int k, int hca_m, const void* kr, const void* vr,
                      const int64_t* raw_pos0, int64_t R, const int64_t* pos0, int64_t B,
                      int64_t T, int64_t H, int64_t D, int64_t n_cap, int W, float scale,
                      const float* out, const float* lse, const float* dout, float* dq,
                      float* dkc, float* dvc, float* dkr, float* dvr, void* ws,
                      hipStream_t stream);
int launch_compress_bwd(const void* x, int dtype, const float* z, const float* dc, int64_t B,
                        int64_t n_tok, int64_t d, int m, int64_t x_sb, int64_t z_sb, float* dx,
                        float* dz, hipStream_t s);

}  // namespace csa
