// Internal launchers of the CSA kernels (not part of the public ABI).
// Each returns 0 on success, -1 if the HIP runtime reported a launch error,
// -2 if no kernel variant matches the (already validated) arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

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

// hist (nullable): per-row first-digit histogram accumulated for csa_topk
// (rows with V <= k are skipped).  It must be zero on entry.  qs / ks are
// fp32 row scales (dtype 2, FP8) or E8M0 block-scale bytes (dtype 3, MXFP4).
// fc (nullable): block compression fused into the launch (bf16, T == 1).
int launch_index_scores(const void* qi, int dtype, const void* qs, const float* w,
                        const void* ki, const void* ks, const int64_t* pos0, int64_t B,
                        int64_t T, int64_t H_I, int64_t d_I, int64_t n_cap, int m, int act,
                        float* scores, uint32_t* hist, int k, const FusedCompress* fc,
                        hipStream_t s);

// Rows (B*T) up to this count use the multi-workgroup split top-k, which
// needs a workspace; more rows use one workgroup per row and none.
constexpr int64_t kTopkSplitMaxRows = 256;
size_t topk_workspace_bytes(int64_t B, int64_t T, int64_t n_cap, int k);
// The first-digit histogram inside a top-k workspace (nullptr when the row
// path, which keeps its histogram in LDS, will be used).
uint32_t* topk_hist_ptr(void* ws, int64_t B, int64_t T);
int launch_topk(const float* scores, const int64_t* pos0, int64_t B, int64_t T, int64_t n_cap,
                int m, int k, int32_t* idx, void* ws, bool hist_ready, hipStream_t s);
// Zero-fill (a kernel, so it may be captured in a graph).
int launch_clear(void* p, size_t bytes, hipStream_t s);

struct AttSplit {
  int splits;
  int chunks_per_split;
};
AttSplit attend_split(int64_t rows, int64_t n_slots_max, bool hca);
size_t attend_workspace_bytes(int64_t rows, int64_t H, int64_t D, int64_t n_slots_max, bool hca);
// hca_m > 0 selects HCA (all visible entries, idx ignored).
int launch_attend(const void* q, int dtype, const void* kc, const void* vc, const int32_t* idx,
                  int k, int hca_m, const void* kr, const void* vr, const int64_t* raw_pos0,
                  int64_t R, const int64_t* pos0, int64_t B, int64_t T, int64_t H, int64_t D,
                  int64_t n_cap, int W, float scale, float* out, float* lse, void* ws,
                  hipStream_t stream);

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
