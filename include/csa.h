/*
 * csa.h -- C ABI of the Compressed Sparse Attention (CSA) hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (DeepSeek-V4's CSA and HCA) as the source pages describe it:
 *   - "DeepSeek V4 technical review" (takeshell.com), section 2.1 "CSA":
 *     every m tokens' KV become one entry by weighted aggregation; a
 *     Lightning Indexer scores each query against the compressed entries and
 *     keeps the top-k; core attention runs over the selected entries only.
 *     Section 2.2 "HCA": m' = 128, dense attention over all entries.
 *   - "DeepSeek V4: Compressed Sparse Attention and the Million-Token
 *     Context" (octagono.org), "Hybrid Attention: CSA and HCA": top-1024,
 *     a sliding window of 128 recent tokens, HCA has no selection.
 *   - dataforcee.us "Hybrid Attention: CSA and HCA": both CSA and HCA carry
 *     a sliding-window branch over the most recent raw tokens.
 *   - takeshell.com section 5 and dataforcee.us "Muon Optimizer and FP4
 *     QAT": the indexer's query-key path runs in low precision.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor pointers are DEVICE pointers, row-major and contiguous in the
 *   stated shape unless a batch stride argument says otherwise.  The caller
 *   owns every buffer; no call allocates or frees device memory.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   Every call is asynchronous on that stream: it only enqueues kernels.
 * - Arguments are validated on the host before anything is enqueued.  A
 *   failed validation returns a negative status and enqueues nothing;
 *   csa_last_error() then describes the problem (thread-local).  Nothing
 *   aborts or throws across this ABI.  A launch failure reported by the HIP
 *   runtime returns CSA_ERR_HIP.  Faults inside kernels surface at the
 *   caller's next synchronisation of the stream.
 * - Query token i (0 <= i < T) of sequence b sits at absolute position
 *   t = pos0[b] + i (pos0 is a DEVICE array of B int64).  The compressed
 *   entries visible to position t are j < V(t) = floor((t + 1) / m): block
 *   j covers raw positions j*m .. j*m+m-1 and is visible once it is
 *   complete.  Kernels clamp V(t) to n_cap so that no access leaves the
 *   buffers; positions with V(t) > n_cap are a caller error.
 * - Scores must be finite; -0.0 is ranked equal to +0.0.
 * - Workspaces (`ws`): device memory owned by the caller, sized by the
 *   matching *_workspace_size() query.  Top-k workspaces must be zero
 *   before first use (a zero-filled allocation, or csa_workspace_clear);
 *   every call leaves them ready for the next call with the same B, T and
 *   n_cap (the parts read before being written -- histograms and counters
 *   -- are returned to zero), so they are reused call after call without
 *   clearing; their layout depends on those sizes, so a workspace reused
 *   for other sizes must be cleared first.  Attention workspaces
 *   hold per-call partial results and may contain anything on entry.
 *   Calls that share a workspace must be ordered (same stream); concurrent
 *   calls on one workspace race.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define CSA_F32 0      /* IEEE binary32 */
#define CSA_BF16 1     /* bfloat16, stored as 16-bit words */
#define CSA_FP8_E4M3 2 /* OCP FP8 E4M3FN byte codes (max 448, no inf) */
/* OCP MX FP4: E2M1 codes two per byte (element 2i in the low nibble, 2i+1
 * in the high nibble; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) with one E8M0
 * scale byte (2^(byte - 127)) per block of 32 consecutive elements.  A row
 * of d elements is d/2 code bytes plus d/32 scale bytes, in two arrays. */
#define CSA_MXFP4 3

/* indexer nonlinearity */
#define CSA_ACT_RELU 0
#define CSA_ACT_IDENTITY 1

/* status codes */
#define CSA_OK 0
#define CSA_ERR_NULL (-1)        /* a required pointer is NULL */
#define CSA_ERR_SHAPE (-2)       /* a size or position argument is invalid */
#define CSA_ERR_DTYPE (-3)       /* unsupported element type or combination */
#define CSA_ERR_UNSUPPORTED (-4) /* valid, but outside what the kernels support */
#define CSA_ERR_WORKSPACE (-5)   /* workspace missing or too small */
#define CSA_ERR_HIP (-6)         /* the HIP runtime reported an error */

/* Human-readable name of a status code (static string). */
const char* csa_status_string(int status);
/* Message describing the last failed call on this thread ("" if none). */
const char* csa_last_error(void);
/* ABI version of this library (incremented on incompatible changes). */
int csa_abi_version(void);
/* sha256 (64 hex digits) of the sources, headers and flags the library was
 * built from; callers compare it with the tree to refuse a stale build. */
const char* csa_build_digest(void);

/* Zero `ws_bytes` bytes of a device workspace on `stream` (a kernel, so it
 * may be captured in a HIP graph).  ws 16-byte aligned, ws_bytes % 4 == 0. */
int csa_workspace_clear(void* ws, size_t ws_bytes, void* stream);

/* Kernel timing, for callers that measure one kernel of a call rather than
 * the call with the dispatch around it.  The next n kernels that library
 * calls made on the calling host thread launch (the kernels of csa_compress,
 * the quantizers, csa_index_scores / csa_topk / csa_index_topk,
 * csa_decode_index_topk, csa_select_attend, csa_decode, csa_decode_noalloc,
 * csa_attend and hca_attend; the backward calls' kernels and
 * csa_workspace_clear do not count) are launched with hipExtLaunchKernelGGL:
 * the first records start_event when it starts, the n-th records stop_event
 * when it ends, so hipEventElapsedTime(start_event, stop_event) is the time
 * from the first kernel's start to the n-th kernel's end.  start_event and
 * stop_event are hipEvent_t created by the caller (non-NULL when n > 0), not
 * owned by the library.  n = 0 cancels a pending request; a request stays
 * pending until n kernels have been launched.  Returns CSA_OK, or
 * CSA_ERR_NULL / CSA_ERR_SHAPE for missing events or n < 0. */
int csa_time_next_kernels(void* start_event, void* stop_event, int n);

/*
 * csa_compress -- the token-level compressor (takeshell.com 2.1: every m
 * tokens' KV entries are compressed into one entry by weighted
 * aggregation; octagono.org: a learned token-level compressor).
 *
 * For sequence b, block j < n_tok/m and channel c:
 *   w_i = softmax over i < m of logits[b, j*m + i, c]
 *   cache[b, first_entry + j, c] = sum_i w_i * x[b, j*m + i, c]
 * computed in fp32 and rounded to nearest-even when the cache is bf16.
 *
 *   x       [B][x_batch_stride] elements; row i (i < n_tok) of sequence b
 *           starts at x + b*x_batch_stride + i*d.  dtype x_dtype.
 *   logits  fp32, same indexing with z_batch_stride.
 *   cache   [B][n_cap][d] of cache_dtype (must equal x_dtype); entries
 *           first_entry .. first_entry + n_tok/m - 1 are written, nothing
 *           else is touched.
 * Requirements: n_tok % m == 0 (only complete blocks), m >= 1, d >= 1,
 * first_entry >= 0, first_entry + n_tok/m <= n_cap, strides >= n_tok*d.
 * dtypes: (F32 -> F32), (BF16 -> BF16).  n_tok == 0 is a no-op.
 */
int csa_compress(const void* x, int x_dtype, const float* logits,
                 int64_t B, int64_t n_tok, int64_t d, int m,
                 int64_t x_batch_stride, int64_t z_batch_stride,
                 void* cache, int cache_dtype, int64_t n_cap,
                 int64_t first_entry, void* stream);

/*
 * csa_quantize_fp8_rows -- FP8 storage of indexer keys and queries (the
 * pages quantize the indexer's QK path; takeshell.com section 5).  For each
 * row r of x [rows][d]:
 *   scale[r] = max_c |x[r,c]| / 448   (correctly rounded fp32; 1 if zero)
 *   codes[r,c] = E4M3FN(x[r,c] / scale[r])  (correctly rounded fp32
 *                quotient, round to nearest even, saturate to +-448)
 * dequantized value = decode(code) * scale.  x_dtype F32 or BF16;
 * 1 <= d <= 1024.  rows == 0 is a no-op.
 */
int csa_quantize_fp8_rows(const void* x, int x_dtype, int64_t rows, int64_t d,
                          uint8_t* codes, float* scales, void* stream);

/*
 * csa_quantize_mxfp4_rows -- MXFP4 storage of indexer keys and queries, the
 * pages' own precision for the indexer's query-key path (takeshell.com
 * section 5; dataforcee.us "Muon Optimizer and FP4 QAT": MXFP4 QAT of the
 * Lightning Indexer's QK path, FP4 E2M1 dequantizing losslessly to FP8).
 * The scale rule is the OCP MX v1.0 one.  For each block of 32 consecutive
 * elements of each row r of x [rows][d]:
 *   amax = max |x|;  s = floor(log2(amax)) - 2, clamped to [-127, 127]
 *   scales[r, blk] = s + 127   (0 for an all-zero block)
 *   code = E2M1(x * 2^-s): nearest, ties to the even code, saturating at
 *          +-6; the sign bit is the sign of x
 * codes [rows][d/2] (two codes per byte, low nibble first), scales
 * [rows][d/32].  Dequantized value = e2m1(code) * 2^(scale - 127).  x_dtype
 * F32 or BF16; d a multiple of 32 in [32, 4096].  rows == 0 is a no-op.
 */
int csa_quantize_mxfp4_rows(const void* x, int x_dtype, int64_t rows, int64_t d,
                            uint8_t* codes, uint8_t* scales, void* stream);

/*
 * csa_index_scores -- the Lightning Indexer (takeshell.com 2.1: indexer
 * queries per query token, scored against the compressed entries; 64 heads
 * x 128 dims for V4-Pro).  For query (b, i) at position t and j < V(t):
 *   scores[b,i,j] = sum_h w[b,i,h] * phi( qi[b,i,h,:] . ki[b,j,:] )
 * phi = ReLU (act = CSA_ACT_RELU) or identity (CSA_ACT_IDENTITY).  With
 * FP8 inputs the operands are decode(code) * scale, i.e.
 *   scores = ki_scale[b,j] * sum_h (w * qi_scale[b,i,h]) * phi(q~ . k~);
 * with MXFP4 inputs they are the dequantized MXFP4 rows (each 32-element
 * block times its own scale, inside the dot product).
 * Entries j >= V(t) of a score row are not written.
 *
 * Optional fusion with csa_topk: when topk_ws is non-NULL, the call also
 * accumulates into topk_ws the first-digit histogram of the top-k
 * selection with this k (saves csa_topk one pass over the scores); the
 * next call must then be csa_topk(..., topk_ws, ..., hist_ready = 1) with
 * the same B, T, n_cap, m, k, which consumes it.  topk_ws must follow the
 * top-k workspace protocol above and be at least csa_topk_workspace_size()
 * bytes.  With
 * topk_ws == NULL, k is ignored.
 *
 *   qi        [B][T][H_I][d_I]      qi_dtype (MXFP4: [B][T][H_I][d_I/2] bytes)
 *   qi_scale  FP8: [B][T][H_I] fp32; MXFP4: [B][T][H_I][d_I/32] E8M0
 *             bytes; other dtypes: ignored, may be NULL
 *   w         [B][T][H_I] fp32
 *   ki        [B][n_cap][d_I]       ki_dtype (== qi_dtype; MXFP4: d_I/2 bytes)
 *   ki_scale  FP8: [B][n_cap] fp32; MXFP4: [B][n_cap][d_I/32] E8M0 bytes,
 *             4-byte aligned; other dtypes: ignored, may be NULL
 *   pos0      [B] int64 (device)
 *   scores    [B][T][n_cap] fp32
 * Supported: dtypes F32, BF16 (d_I % 32 == 0, d_I <= 256), FP8_E4M3 and
 * MXFP4 (d_I == 128); 1 <= H_I <= 64; m >= 1; T >= 1, B >= 1.
 */
int csa_index_scores(const void* qi, int qi_dtype, const void* qi_scale,
                     const float* w, const void* ki, int ki_dtype,
                     const void* ki_scale, const int64_t* pos0,
                     int64_t B, int64_t T, int64_t H_I, int64_t d_I,
                     int64_t n_cap, int m, int act, float* scores, int k,
                     void* topk_ws, size_t topk_ws_bytes, void* stream);

/*
 * csa_topk -- per-query top-k selection (takeshell.com 2.1: the k most
 * relevant compressed blocks are kept; k = 1024 for V4-Pro).  For query
 * (b, i) at position t the min(k, V(t)) visible entries with the largest
 * score are kept; equal scores go to the lower entry index.  idx[b,i,:]
 * lists them in ascending index order, padded with -1 to length k.
 *
 *   scores [B][T][n_cap] fp32 (only j < V(t) is read)
 *   idx    [B][T][k] int32
 *   ws     device workspace of csa_topk_workspace_size() bytes (top-k
 *          workspace protocol above).  For B*T <= 256 it is required.  For
 *          more query rows (one workgroup per row) it is optional: it
 *          holds per row a 2048-bin histogram of the scores' top 11 key
 *          bits and a flag, which csa_index_scores writes when its
 *          many-token kernel runs (BF16 / FP8, d_I = 128, T >= 8) and this
 *          call uses instead of a histogram pass over the row; every flag
 *          is cleared here, and csa_index_scores clears them when it
 *          writes no histograms.
 *   hist_ready  1 if the directly preceding csa_index_scores was given
 *          this ws (and k) and so already built the first-digit
 *          histogram; 0 otherwise (for more than 256 rows the flags
 *          decide).
 * 1 <= k <= 4096.
 */
size_t csa_topk_workspace_size(int64_t B, int64_t T, int64_t n_cap, int k);
int csa_topk(const float* scores, const int64_t* pos0, int64_t B, int64_t T,
             int64_t n_cap, int m, int k, int32_t* idx, void* ws,
             size_t ws_bytes, int hist_ready, void* stream);

/*
 * csa_index_topk -- csa_index_scores followed by csa_topk on the same
 * stream, with the top-k histogram fused into the indexer.  scores may be
 * NULL, in which case the score matrix lives in the workspace
 * (csa_index_topk_workspace_size accounts for it).  Same top-k workspace
 * protocol.
 */
size_t csa_index_topk_workspace_size(int64_t B, int64_t T, int64_t n_cap,
                                     int k, int scores_in_workspace);
int csa_index_topk(const void* qi, int qi_dtype, const void* qi_scale,
                   const float* w, const void* ki, int ki_dtype,
                   const void* ki_scale, const int64_t* pos0,
                   int64_t B, int64_t T, int64_t H_I, int64_t d_I,
                   int64_t n_cap, int m, int act, int k, float* scores,
                   int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * csa_decode_index_topk -- the selection half of a decode step, one new
 * query token per sequence, with the block compression folded into the
 * indexer launch (takeshell.com 2.1: every m tokens become one entry by
 * weighted aggregation, then the indexer scores the query against every
 * visible entry and keeps the top-k).  For sequence b the query sits at
 * t = pos0[b].  When t completes a block ((t + 1) % m == 0 and
 * (t + 1) / m <= n_cap), entry j = (t + 1) / m - 1 of kc and vc is first
 * written as in csa_compress from the raw rows of positions t-m+1 .. t
 * (bit-identical to csa_compress on those rows), and is then scored with
 * the rest; otherwise kc and vc are not written.  The indexer keys are the
 * compressed keys kc themselves.  Results are those of csa_compress (K and
 * V) followed by csa_index_topk, in one indexer launch plus the top-k.
 *
 *   qi     [B][H_I][d] bf16;  w [B][H_I] fp32
 *   kc,vc  [B][n_cap][d] bf16 (read; entry j written as above)
 *   kr,vr  [B][R][d] bf16; row r holds position raw_pos0[b] + r.  A block
 *          whose raw rows are not all inside the buffer is not written
 *          (a caller error).
 *   zk,zv  [B][R][d] fp32 compressor logits of the raw rows (may be equal)
 *   raw_pos0, pos0 [B] int64 (device)
 *   scores [B][n_cap] fp32 or NULL (then kept in the workspace), idx
 *          [B][k] int32, ws: as csa_index_topk with T = 1.
 * Supported: d in {64, 128, 256}; 1 <= H_I <= 64; 1 <= m <= 4 (CSA's
 * compression ratio; larger m: csa_compress then csa_index_topk); R >= m;
 * 1 <= k <= 4096.
 */
int csa_decode_index_topk(const void* qi, const float* w, void* kc, void* vc,
                          const void* kr, const void* vr, const float* zk,
                          const float* zv, const int64_t* raw_pos0, int64_t R,
                          const int64_t* pos0, int64_t B, int64_t H_I,
                          int64_t d, int64_t n_cap, int m, int act, int k,
                          float* scores, int32_t* idx, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * csa_attend -- core attention over the selected compressed entries plus
 * the sliding window, in one softmax (octagono.org "Hybrid Attention":
 * attend only to the selected entries, with a 128-token window for local
 * context; dataforcee.us: the window branch covers the most recent raw
 * tokens).  One KV head is shared by all H query heads.  For query (b, i)
 * at position t and head h the key set is
 *   { kc[b, j] : j = idx[b,i,s] >= 0 }  followed by
 *   { kr[b, p - raw_pos0[b]] : max(0, t-W+1) <= p <= t }
 * (the window is not de-duplicated against the selected entries), with
 * values from vc / vr at the same rows:
 *   out[b,i,h,:] = softmax_keys(scale * q[b,i,h,:] . key) @ values
 *   lse[b,i,h]   = natural-log sum of exp(scale * q . key)
 *
 *   q     [B][T][H][d]         q_dtype (== kv_dtype)
 *   kc,vc [B][n_cap][d]        kv_dtype
 *   idx   [B][T][k] int32      entries < 0 or >= n_cap are skipped
 *   kr,vr [B][R][d]            kv_dtype; row r holds position raw_pos0[b]+r
 *   raw_pos0 [B] int64 (device); window positions outside the raw buffer
 *          are a caller error and are skipped (never read out of bounds)
 *   out   [B][T][H][d] fp32;  lse [B][T][H] fp32 or NULL
 *   ws    device workspace of csa_attend_workspace_size() bytes (contents
 *         on entry do not matter; size 0 and ws may be NULL when each query
 *         fits one workgroup)
 * Supported: dtypes F32, BF16; d in {64, 128}; 1 <= H <= 64;
 * 0 <= W <= 4096; 0 <= k <= 65536; k + W >= 1; scale finite and > 0
 * (else CSA_ERR_SHAPE).  A query whose key set is empty gets out = 0 and
 * lse = -inf.
 */
size_t csa_attend_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d,
                                 int k, int W);
int csa_attend(const void* q, int q_dtype, const void* kc, const void* vc,
               int kv_dtype, const int32_t* idx, int k, const void* kr,
               const void* vr, const int64_t* raw_pos0, int64_t R,
               const int64_t* pos0, int64_t B, int64_t T, int64_t H,
               int64_t d, int64_t n_cap, int W, float scale, float* out,
               float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * csa_select_attend -- the top-k selection and the core attention of a CSA
 * step ("DeepSeek V4 technical review", takeshell.com, section 2.1: the
 * indexer's top-k entries, then attention over them only; octagono.org:
 * top-1,024 plus a 128-token window), from csa_index_scores' scores.
 * Computes exactly what csa_topk (same ws, same hist_ready) followed by
 * csa_attend compute: idx receives csa_topk's selection, out / lse the
 * attention over it.  For up to 256 query rows over n_cap <= 2^20 entries
 * (n_cap > 8192) the selection is made inside the attention launch: from
 * the scores themselves when n_cap <= 32768, n_cap is a multiple of 4 and
 * scores is 16-byte aligned (no top-k launch when hist_ready), else from
 * the top-k's classified lists (one launch fewer); other sizes run
 * csa_topk's kernels first.  Scores are taken to be finite (the bucket
 * tests run on the floats, as in csa_topk's row kernel).
 *
 *   scores, topk_ws, topk_ws_bytes, hist_ready, pos0, m, k   as csa_topk
 *   q, kc, vc, kv_dtype, kr, vr, raw_pos0, R, W, scale, out, lse, ws,
 *   ws_bytes   as csa_attend (the query has kv_dtype; attention workspace
 *              of csa_attend_workspace_size(B, T, H, d, k, W) bytes)
 *   idx        [B][T][k] int32 output
 * Errors: those of csa_topk's and csa_attend's checks, in that order.
 */
int csa_select_attend(const float* scores, void* topk_ws, size_t topk_ws_bytes,
                      int hist_ready, const int64_t* pos0, int m, int k,
                      const void* q, const void* kc, const void* vc,
                      int kv_dtype, const void* kr, const void* vr,
                      const int64_t* raw_pos0, int64_t R, int64_t B, int64_t T,
                      int64_t H, int64_t d, int64_t n_cap, int W, float scale,
                      int32_t* idx, float* out, float* lse, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * csa_decode -- one whole CSA step for a batch of queries in one call
 * ("DeepSeek V4 technical review", takeshell.com, section 2.1: compress,
 * index, select, attend): the Lightning Indexer's scores (csa_index_scores,
 * which also builds the top-k histogram), then the top-k selection and the
 * attention over the selected entries plus the window (csa_select_attend),
 * and -- when zk and zv are given -- the compression of the block that the
 * query token completes, done inside the indexer launch as in
 * csa_decode_index_topk.  Outputs are bit-identical to those calls made one
 * after another; the query q has kv_dtype.
 *
 *   qi .. ki_scale   the indexer inputs of csa_index_scores (act, H_I, d_I)
 *   q, kc, vc, kv_dtype, kr, vr, raw_pos0, R   the attention inputs of
 *                    csa_attend; kc / vc are written only by the block
 *                    compression
 *   zk, zv           NULL, or the compressor logits [B][R][d] fp32 of the
 *                    raw rows (block compression: needs T == 1, ki == kc,
 *                    bf16, R >= m, m <= 4)
 *   scores           [B][T][n_cap] fp32 output, or NULL to keep the scores in
 *                    the workspace
 *   idx, out, lse    outputs as csa_topk / csa_attend
 *   ws               device workspace of csa_decode_workspace_size(B, T, H,
 *                    d, n_cap, k, W, scores == NULL) bytes, 16-byte aligned,
 *                    zero before first use and left zero (workspace protocol
 *                    above)
 * Errors: CSA_ERR_WORKSPACE for a missing or short workspace, then the
 * argument checks of csa_index_scores, csa_topk and csa_attend in that
 * order; CSA_ERR_UNSUPPORTED for a block compression outside the limits
 * above.  Nothing is launched when a check fails.
 */
size_t csa_decode_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d,
                                 int64_t n_cap, int k, int W,
                                 int scores_in_workspace);
int csa_decode(const void* qi, int qi_dtype, const void* qi_scale,
               const float* w, const void* ki, int ki_dtype,
               const void* ki_scale, const void* q, void* kc, void* vc,
               int kv_dtype, const void* kr, const void* vr, const float* zk,
               const float* zv, const int64_t* raw_pos0, int64_t R,
               const int64_t* pos0, int64_t B, int64_t T, int64_t H_I,
               int64_t d_I, int64_t H, int64_t d, int64_t n_cap, int m,
               int act, int k, int W, float scale, float* scores,
               int32_t* idx, float* out, float* lse, void* ws,
               size_t ws_bytes, void* stream);

/*
 * csa_decode_noalloc -- csa_decode without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  It
 * computes exactly what csa_decode computes, with the same arguments minus
 * ws / ws_bytes, and allocates nothing: its workspace is a fixed array of
 * csa_decode_noalloc_max_bytes() bytes (64 MiB) inside the library, one
 * per GPU, held until the process ends.  Sizes whose
 * csa_decode_workspace_size(..., scores == NULL) exceeds it return
 * CSA_ERR_UNSUPPORTED; other errors as csa_decode.
 * The array is zeroed by a fill kernel on the caller's stream at its first
 * use on a device, after a call that failed once kernels were enqueued,
 * and in its leading histogram part whenever B*T or n_cap differ from the
 * previous call's.  Every call on a GPU shares that GPU's array: calls
 * that may overlap on one GPU (other streams, other threads) race and must
 * be ordered by the caller.
 */
size_t csa_decode_noalloc_max_bytes(void);
int csa_decode_noalloc(const void* qi, int qi_dtype, const void* qi_scale,
                       const float* w, const void* ki, int ki_dtype,
                       const void* ki_scale, const void* q, void* kc,
                       void* vc, int kv_dtype, const void* kr,
                       const void* vr, const float* zk, const float* zv,
                       const int64_t* raw_pos0, int64_t R,
                       const int64_t* pos0, int64_t B, int64_t T,
                       int64_t H_I, int64_t d_I, int64_t H, int64_t d,
                       int64_t n_cap, int m, int act, int k, int W,
                       float scale, float* scores, int32_t* idx,
                       float* out, float* lse, void* stream);

/*
 * hca_attend -- Heavily Compressed Attention (takeshell.com 2.2: m' = 128;
 * octagono.org: dense attention over the heavily compressed entries, no
 * sparse selection), with the same sliding-window branch.  Identical to
 * csa_attend with idx[b,i] = 0 .. V(t)-1, V(t) = floor((t+1)/m), clamped
 * to n_cap.  Same layouts and support limits as csa_attend.
 */
size_t hca_attend_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d,
                                 int64_t n_cap, int W);
int hca_attend(const void* q, int q_dtype, const void* kc, const void* vc,
               int kv_dtype, int m, const void* kr, const void* vr,
               const int64_t* raw_pos0, int64_t R, const int64_t* pos0,
               int64_t B, int64_t T, int64_t H, int64_t d, int64_t n_cap,
               int W, float scale, float* out, float* lse, void* ws,
               size_t ws_bytes, void* stream);

/*
 * Backward pass (fp32 gradients).  The pages describe a model trained end
 * to end -- a learned token-level compressor (octagono.org "Hybrid
 * Attention: CSA and HCA"), an indexer QK path trained quantization-aware
 * (dataforcee.us "Muon Optimizer and FP4 QAT") -- without a formula for
 * the backward pass; these calls compute the derivatives of csa_attend /
 * hca_attend / csa_compress.  No gradient flows through the top-k
 * selection.  All reductions are deterministic (no float atomics): two
 * runs give identical bits.
 *
 * csa_attend_backward -- for csa_attend's inputs, its outputs out / lse and
 * the upstream gradient dout (d loss / d out), writes
 *   dq    [B][T][H][d] fp32
 *   dkc, dvc [B][n_cap][d] fp32: every entry; the sum over all query rows
 *         and heads that attended it (0 for entries nobody selected)
 *   dkr, dvr [B][R][d] fp32: every raw row, the same over the windows
 * (with one query row t, head h over its key list, p = exp(scale q.K - lse),
 * dp = V dout, D = dout . out, ds = p (dp - D): dq = scale ds K,
 * dK += scale ds q, dV += p dout).  idx rows must be strictly ascending
 * then -1 padded (as csa_topk emits them): a row never repeats an entry,
 * so an entry is referenced at most T times; rows that break this give
 * undefined dkc / dvc (not detected).  ws: device workspace of
 * csa_attend_backward_workspace_size() bytes (the per-row key/value
 * contributions, B*T*(k+W)*d*8 bytes, and each entry's list of the rows
 * that attended it; contents on entry do not matter).
 * Supported: q/kv dtypes F32 or BF16 (equal), d in {64, 128}, H <= 64,
 * k <= 4096, T <= 16384, B*T*k < 2^32.
 */
size_t csa_attend_backward_workspace_size(int64_t B, int64_t T, int64_t d,
                                          int64_t n_cap, int k, int W);
int csa_attend_backward(const void* q, int q_dtype, const void* kc,
                        const void* vc, int kv_dtype, const int32_t* idx,
                        int k, const void* kr, const void* vr,
                        const int64_t* raw_pos0, int64_t R,
                        const int64_t* pos0, int64_t B, int64_t T,
                        int64_t H, int64_t d, int64_t n_cap, int W,
                        float scale, const float* out, const float* lse,
                        const float* dout, float* dq, float* dkc, float* dvc,
                        float* dkr, float* dvr, void* ws, size_t ws_bytes,
                        void* stream);

/* hca_attend_backward -- the same for hca_attend (every visible entry
 * attended, compression ratio m); n_cap <= 65536; workspace of
 * hca_attend_backward_workspace_size() bytes. */
size_t hca_attend_backward_workspace_size(int64_t B, int64_t T, int64_t d,
                                          int64_t n_cap, int W);
int hca_attend_backward(const void* q, int q_dtype, const void* kc,
                        const void* vc, int kv_dtype, int m, const void* kr,
                        const void* vr, const int64_t* raw_pos0, int64_t R,
                        const int64_t* pos0, int64_t B, int64_t T,
                        int64_t H, int64_t d, int64_t n_cap, int W,
                        float scale, const float* out, const float* lse,
                        const float* dout, float* dq, float* dkc, float* dvc,
                        float* dkr, float* dvr, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * csa_compress_backward -- gradients of csa_compress with respect to its
 * tokens and logits: for block j, channel c, w_i = softmax_i(logits) and
 * c_j = sum_i w_i x_i,
 *   dx[jm+i, c]      = w_i dc[j, c]
 *   dlogits[jm+i, c] = w_i (x[jm+i, c] - c_j) dc[j, c]
 *   x       [B][n_tok][d] x_dtype (F32 or BF16), batch stride x_sb elements
 *   logits  [B][n_tok][d] fp32, batch stride z_sb elements
 *   dc      [B][n_tok/m][d] fp32 (gradient of the n_tok/m compressed rows)
 *   dx, dlogits [B][n_tok][d] fp32
 * n_tok % m == 0.
 */
int csa_compress_backward(const void* x, int x_dtype, const float* logits,
                          const float* dc, int64_t B, int64_t n_tok,
                          int64_t d, int m, int64_t x_sb, int64_t z_sb,
                          float* dx, float* dlogits, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
