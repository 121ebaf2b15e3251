// C ABI of the CSA hot path: argument validation (pure host code, runs
// before anything is enqueued) and dispatch to the HIP kernels.  The
// contract of every call is documented in include/csa.h.
#include "../../include/csa.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return CSA_OK;
}

int hip_result(int rc, const char* what) {
  if (rc == 0) return ok();
  if (rc == -2) return fail(CSA_ERR_UNSUPPORTED, "%s: no kernel variant for these arguments", what);
  return fail(CSA_ERR_HIP, "%s: kernel launch failed: %s", what,
              hipGetErrorString(hipGetLastError()));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxGridY = 65535;
constexpr int64_t kMaxIndex = 0x7fffffffLL;

size_t round_up(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

#define CSA_REQUIRE(cond, code, ...) \
  do {                               \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

int check_index_args(const void* qi, int qi_dtype, const void* qi_scale, const float* w,
                     const void* ki, int ki_dtype, const void* ki_scale, const int64_t* pos0,
                     int64_t B, int64_t T, int64_t H_I, int64_t d_I, int64_t n_cap, int m, int act,
                     const float* scores, const char* fn) {
  CSA_REQUIRE(qi && w && ki && pos0 && scores, CSA_ERR_NULL,
              "%s: qi, w, ki, pos0 and scores must be non-NULL", fn);
  CSA_REQUIRE(qi_dtype == ki_dtype, CSA_ERR_DTYPE, "%s: qi_dtype (%d) must equal ki_dtype (%d)", fn,
              qi_dtype, ki_dtype);
  CSA_REQUIRE(qi_dtype == CSA_F32 || qi_dtype == CSA_BF16 || qi_dtype == CSA_FP8_E4M3 ||
                  qi_dtype == CSA_MXFP4,
              CSA_ERR_DTYPE, "%s: unknown dtype %d", fn, qi_dtype);
  if (qi_dtype == CSA_FP8_E4M3)
    CSA_REQUIRE(qi_scale && ki_scale, CSA_ERR_NULL, "%s: FP8 inputs need qi_scale and ki_scale", fn);
  if (qi_dtype == CSA_MXFP4) {
    CSA_REQUIRE(qi_scale && ki_scale, CSA_ERR_NULL,
                "%s: MXFP4 inputs need qi_scale and ki_scale (E8M0 block scales)", fn);
    CSA_REQUIRE((reinterpret_cast<uintptr_t>(ki_scale) & 3) == 0, CSA_ERR_SHAPE,
                "%s: MXFP4 ki_scale must be 4-byte aligned", fn);
  }
  CSA_REQUIRE(act == CSA_ACT_RELU || act == CSA_ACT_IDENTITY, CSA_ERR_SHAPE, "%s: unknown act %d",
              fn, act);
  CSA_REQUIRE(B >= 1 && T >= 1, CSA_ERR_SHAPE, "%s: B and T must be >= 1", fn);
  CSA_REQUIRE(B * T <= kMaxGridY, CSA_ERR_UNSUPPORTED, "%s: B*T must be <= %lld", fn,
              static_cast<long long>(kMaxGridY));
  CSA_REQUIRE(m >= 1, CSA_ERR_SHAPE, "%s: m must be >= 1", fn);
  CSA_REQUIRE(n_cap >= 1 && n_cap <= kMaxIndex, CSA_ERR_SHAPE, "%s: n_cap must be in [1, 2^31)",
              fn);
  CSA_REQUIRE(H_I >= 1 && H_I <= 64, CSA_ERR_UNSUPPORTED, "%s: H_I must be in [1, 64]", fn);
  if (qi_dtype == CSA_F32)
    CSA_REQUIRE(d_I == 64 || d_I == 128, CSA_ERR_UNSUPPORTED, "%s: fp32 needs d_I in {64, 128}", fn);
  else if (qi_dtype == CSA_BF16)
    CSA_REQUIRE(d_I == 64 || d_I == 128 || d_I == 256, CSA_ERR_UNSUPPORTED,
                "%s: bf16 needs d_I in {64, 128, 256}", fn);
  else
    CSA_REQUIRE(d_I == 128, CSA_ERR_UNSUPPORTED, "%s: fp8 and mxfp4 need d_I == 128", fn);
  CSA_REQUIRE(aligned16(qi) && aligned16(ki), CSA_ERR_SHAPE, "%s: qi and ki must be 16-byte aligned",
              fn);
  return CSA_OK;
}

int check_topk_args(const float* scores, const int64_t* pos0, int64_t B, int64_t T, int64_t n_cap,
                    int m, int k, const int32_t* idx, const char* fn) {
  CSA_REQUIRE(scores && pos0 && idx, CSA_ERR_NULL, "%s: scores, pos0 and idx must be non-NULL", fn);
  CSA_REQUIRE(B >= 1 && T >= 1, CSA_ERR_SHAPE, "%s: B and T must be >= 1", fn);
  CSA_REQUIRE(B * T <= kMaxGridY, CSA_ERR_UNSUPPORTED, "%s: B*T must be <= %lld", fn,
              static_cast<long long>(kMaxGridY));
  CSA_REQUIRE(m >= 1, CSA_ERR_SHAPE, "%s: m must be >= 1", fn);
  CSA_REQUIRE(n_cap >= 1 && n_cap <= kMaxIndex, CSA_ERR_SHAPE, "%s: n_cap must be in [1, 2^31)",
              fn);
  CSA_REQUIRE(k >= 1 && k <= 4096, CSA_ERR_UNSUPPORTED, "%s: k must be in [1, 4096]", fn);
  return CSA_OK;
}

int check_attend_args(const void* q, int q_dtype, const void* kc, const void* vc, int kv_dtype,
                      const void* kr, const void* vr, const int64_t* raw_pos0, int64_t R,
                      const int64_t* pos0, int64_t B, int64_t T, int64_t H, int64_t d,
                      int64_t n_cap, int W, float scale, const float* out, const char* fn) {
  CSA_REQUIRE(q && kc && vc && pos0 && out, CSA_ERR_NULL,
              "%s: q, kc, vc, pos0 and out must be non-NULL", fn);
  CSA_REQUIRE(W == 0 || (kr && vr && raw_pos0), CSA_ERR_NULL,
              "%s: kr, vr and raw_pos0 must be non-NULL when W > 0", fn);
  CSA_REQUIRE(q_dtype == kv_dtype, CSA_ERR_DTYPE, "%s: q_dtype (%d) must equal kv_dtype (%d)", fn,
              q_dtype, kv_dtype);
  CSA_REQUIRE(q_dtype == CSA_F32 || q_dtype == CSA_BF16, CSA_ERR_DTYPE,
              "%s: dtype must be F32 or BF16, got %d", fn, q_dtype);
  CSA_REQUIRE(B >= 1 && T >= 1, CSA_ERR_SHAPE, "%s: B and T must be >= 1", fn);
  CSA_REQUIRE(B * T <= kMaxGridY, CSA_ERR_UNSUPPORTED, "%s: B*T must be <= %lld", fn,
              static_cast<long long>(kMaxGridY));
  CSA_REQUIRE(H >= 1 && H <= 64, CSA_ERR_UNSUPPORTED, "%s: H must be in [1, 64]", fn);
  CSA_REQUIRE(d == 64 || d == 128, CSA_ERR_UNSUPPORTED, "%s: d must be 64 or 128", fn);
  CSA_REQUIRE(n_cap >= 1 && n_cap <= kMaxIndex, CSA_ERR_SHAPE, "%s: n_cap must be in [1, 2^31)",
              fn);
  CSA_REQUIRE(W >= 0 && W <= 4096, CSA_ERR_UNSUPPORTED, "%s: W must be in [0, 4096]", fn);
  CSA_REQUIRE(scale > 0.f && scale <= 3.4e38f, CSA_ERR_SHAPE, "%s: scale must be finite and > 0",
              fn);
  CSA_REQUIRE(R >= 0 && (W == 0 || R >= 1), CSA_ERR_SHAPE, "%s: R must be >= 1 when W > 0", fn);
  CSA_REQUIRE(aligned16(q) && aligned16(kc) && aligned16(vc) && aligned16(out) &&
                  (W == 0 || (aligned16(kr) && aligned16(vr))),
              CSA_ERR_SHAPE, "%s: q, kc, vc, kr, vr and out must be 16-byte aligned", fn);
  return CSA_OK;
}

}  // namespace

namespace csa {

// The calling thread's pending kernel-timing request (csa_time_next_kernels).
struct TimingRequest {
  hipEvent_t start = nullptr, stop = nullptr;
  int remaining = 0, total = 0;
};
thread_local TimingRequest g_timing;

LaunchEvents take_launch_events() {
  TimingRequest& r = g_timing;
  LaunchEvents ev{nullptr, nullptr};
  if (r.remaining <= 0) return ev;
  if (r.remaining == r.total) ev.start = r.start;
  if (r.remaining == 1) ev.stop = r.stop;
  if (--r.remaining == 0) r = TimingRequest{};
  return ev;
}

}  // namespace csa

extern "C" {

const char* csa_status_string(int status) {
  switch (status) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_NULL: return "CSA_ERR_NULL";
    case CSA_ERR_SHAPE: return "CSA_ERR_SHAPE";
    case CSA_ERR_DTYPE: return "CSA_ERR_DTYPE";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE";
    case CSA_ERR_HIP: return "CSA_ERR_HIP";
    default: return "CSA_ERR_UNKNOWN";
  }
}

const char* csa_last_error(void) { return g_last_error; }

int csa_abi_version(void) { return 4; }

#ifndef CSA_SOURCE_DIGEST
#define CSA_SOURCE_DIGEST "unknown"
#endif
// The build embeds the sha256 of the sources it compiled; the tag lets the
// build scripts read it from the file without loading the library.
static const char kSourceDigest[] = "csa-source-digest:" CSA_SOURCE_DIGEST;

const char* csa_build_digest(void) { return kSourceDigest + sizeof("csa-source-digest:") - 1; }

int csa_time_next_kernels(void* start_event, void* stop_event, int n) {
  const char* fn = "csa_time_next_kernels";
  CSA_REQUIRE(n >= 0, CSA_ERR_SHAPE, "%s: n must be >= 0", fn);
  CSA_REQUIRE(n == 0 || (start_event && stop_event), CSA_ERR_NULL,
              "%s: start_event and stop_event must be non-NULL", fn);
  csa::g_timing = csa::TimingRequest{static_cast<hipEvent_t>(start_event),
                                     static_cast<hipEvent_t>(stop_event), n, n};
  return ok();
}

int csa_workspace_clear(void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "csa_workspace_clear";
  if (ws_bytes == 0) return ok();
  CSA_REQUIRE(ws, CSA_ERR_NULL, "%s: ws must be non-NULL", fn);
  CSA_REQUIRE(aligned16(ws) && ws_bytes % 4 == 0, CSA_ERR_WORKSPACE,
              "%s: ws must be 16-byte aligned and a multiple of 4 bytes", fn);
  return hip_result(csa::launch_clear(ws, ws_bytes, static_cast<hipStream_t>(stream)), fn);
}

int csa_compress(const void* x, int x_dtype, const float* logits, int64_t B, int64_t n_tok,
                 int64_t d, int m, int64_t x_batch_stride, int64_t z_batch_stride, void* cache,
                 int cache_dtype, int64_t n_cap, int64_t first_entry, void* stream) {
  const char* fn = "csa_compress";
  CSA_REQUIRE(x && logits && cache, CSA_ERR_NULL, "%s: x, logits and cache must be non-NULL", fn);
  CSA_REQUIRE(x_dtype == cache_dtype, CSA_ERR_DTYPE, "%s: x_dtype must equal cache_dtype", fn);
  CSA_REQUIRE(x_dtype == CSA_F32 || x_dtype == CSA_BF16, CSA_ERR_DTYPE,
              "%s: dtype must be F32 or BF16, got %d", fn, x_dtype);
  CSA_REQUIRE(B >= 1 && B <= kMaxGridY, CSA_ERR_SHAPE, "%s: B must be in [1, 65535]", fn);
  CSA_REQUIRE(m >= 1, CSA_ERR_SHAPE, "%s: m must be >= 1", fn);
  CSA_REQUIRE(d >= 1, CSA_ERR_SHAPE, "%s: d must be >= 1", fn);
  CSA_REQUIRE(n_tok >= 0 && n_tok % m == 0, CSA_ERR_SHAPE,
              "%s: n_tok (%lld) must be a non-negative multiple of m (%d)", fn,
              static_cast<long long>(n_tok), m);
  CSA_REQUIRE(x_batch_stride >= n_tok * d && z_batch_stride >= n_tok * d, CSA_ERR_SHAPE,
              "%s: batch strides must be >= n_tok*d", fn);
  CSA_REQUIRE(first_entry >= 0 && n_cap >= 1 && first_entry + n_tok / m <= n_cap, CSA_ERR_SHAPE,
              "%s: entries [%lld, %lld) do not fit n_cap=%lld", fn,
              static_cast<long long>(first_entry), static_cast<long long>(first_entry + n_tok / m),
              static_cast<long long>(n_cap));
  CSA_REQUIRE((n_tok / m) * d <= 0x7fffffffLL * 256, CSA_ERR_UNSUPPORTED, "%s: too many entries",
              fn);
  if (n_tok == 0) return ok();
  return hip_result(csa::launch_compress(x, x_dtype, logits, B, n_tok, d, m, x_batch_stride,
                                         z_batch_stride, cache, n_cap, first_entry,
                                         static_cast<hipStream_t>(stream)),
                    fn);
}

int csa_quantize_fp8_rows(const void* x, int x_dtype, int64_t rows, int64_t d, uint8_t* codes,
                          float* scales, void* stream) {
  const char* fn = "csa_quantize_fp8_rows";
  CSA_REQUIRE(x && codes && scales, CSA_ERR_NULL, "%s: x, codes and scales must be non-NULL", fn);
  CSA_REQUIRE(x_dtype == CSA_F32 || x_dtype == CSA_BF16, CSA_ERR_DTYPE,
              "%s: dtype must be F32 or BF16, got %d", fn, x_dtype);
  CSA_REQUIRE(rows >= 0, CSA_ERR_SHAPE, "%s: rows must be >= 0", fn);
  CSA_REQUIRE(d >= 1 && d <= 1024, CSA_ERR_UNSUPPORTED, "%s: d must be in [1, 1024]", fn);
  CSA_REQUIRE(rows / 4 < 0x7fffffffLL, CSA_ERR_UNSUPPORTED, "%s: too many rows", fn);
  if (rows == 0) return ok();
  return hip_result(csa::launch_quantize_fp8_rows(x, x_dtype, rows, d, codes, scales,
                                                  static_cast<hipStream_t>(stream)),
                    fn);
}

int csa_quantize_mxfp4_rows(const void* x, int x_dtype, int64_t rows, int64_t d, uint8_t* codes,
                            uint8_t* scales, void* stream) {
  const char* fn = "csa_quantize_mxfp4_rows";
  CSA_REQUIRE(x && codes && scales, CSA_ERR_NULL, "%s: x, codes and scales must be non-NULL", fn);
  CSA_REQUIRE(x_dtype == CSA_F32 || x_dtype == CSA_BF16, CSA_ERR_DTYPE,
              "%s: dtype must be F32 or BF16, got %d", fn, x_dtype);
  CSA_REQUIRE(rows >= 0, CSA_ERR_SHAPE, "%s: rows must be >= 0", fn);
  CSA_REQUIRE(d >= 32 && d <= 4096 && d % 32 == 0, CSA_ERR_UNSUPPORTED,
              "%s: d must be a multiple of 32 in [32, 4096]", fn);
  CSA_REQUIRE(rows / 4 < 0x7fffffffLL, CSA_ERR_UNSUPPORTED, "%s: too many rows", fn);
  if (rows == 0) return ok();
  return hip_result(csa::launch_quantize_mxfp4_rows(x, x_dtype, rows, d, codes, scales,
                                                    static_cast<hipStream_t>(stream)),
                    fn);
}

int csa_index_scores(const void* qi, int qi_dtype, const void* qi_scale, const float* w,
                     const void* ki, int ki_dtype, const void* ki_scale, const int64_t* pos0,
                     int64_t B, int64_t T, int64_t H_I, int64_t d_I, int64_t n_cap, int m, int act,
                     float* scores, int k, void* topk_ws, size_t topk_ws_bytes, void* stream) {
  const char* fn = "csa_index_scores";
  int rc = check_index_args(qi, qi_dtype, qi_scale, w, ki, ki_dtype, ki_scale, pos0, B, T, H_I,
                            d_I, n_cap, m, act, scores, fn);
  if (rc) return rc;
  uint32_t* hist = nullptr;
  csa::CoarseHist coarse{nullptr, nullptr};
  if (topk_ws) {
    CSA_REQUIRE(k >= 1 && k <= 4096, CSA_ERR_UNSUPPORTED, "%s: k must be in [1, 4096]", fn);
    const size_t need = csa_topk_workspace_size(B, T, n_cap, k);
    CSA_REQUIRE(topk_ws_bytes >= need, CSA_ERR_WORKSPACE,
                "%s: top-k workspace of %zu bytes needed, got %zu", fn, need, topk_ws_bytes);
    CSA_REQUIRE(aligned16(topk_ws), CSA_ERR_WORKSPACE, "%s: ws must be 16-byte aligned", fn);
    hist = need ? csa::topk_hist_ptr(topk_ws, B, T) : nullptr;
    coarse = csa::topk_coarse_hist(topk_ws, B, T);
  }
  return hip_result(csa::launch_index_scores(qi, qi_dtype, qi_scale, w, ki, ki_scale, pos0, B, T,
                                             H_I, d_I, n_cap, m, act, scores, hist, k, nullptr,
                                             static_cast<hipStream_t>(stream), &coarse),
                    fn);
}

// Top-k workspaces of more than kTopkSplitMaxRows query rows only carry the
// prefill indexer's histograms: they may be omitted.
static bool topk_ws_optional(int64_t B, int64_t T) { return B * T > csa::kTopkSplitMaxRows; }

size_t csa_topk_workspace_size(int64_t B, int64_t T, int64_t n_cap, int k) {
  if (B < 1 || T < 1) return 0;
  return round_up(csa::topk_workspace_bytes(B, T, n_cap, k));
}

int csa_topk(const float* scores, const int64_t* pos0, int64_t B, int64_t T, int64_t n_cap, int m,
             int k, int32_t* idx, void* ws, size_t ws_bytes, int hist_ready, void* stream) {
  const char* fn = "csa_topk";
  int rc = check_topk_args(scores, pos0, B, T, n_cap, m, k, idx, fn);
  if (rc) return rc;
  const size_t need = csa_topk_workspace_size(B, T, n_cap, k);
  CSA_REQUIRE(need == 0 || (ws && ws_bytes >= need) || (!ws && topk_ws_optional(B, T)),
              CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, got %zu", fn, need,
              ws ? ws_bytes : 0);
  CSA_REQUIRE(ws == nullptr || aligned16(ws), CSA_ERR_WORKSPACE, "%s: ws must be 16-byte aligned",
              fn);
  return hip_result(csa::launch_topk(scores, pos0, B, T, n_cap, m, k, idx, ws, hist_ready != 0,
                                     static_cast<hipStream_t>(stream)),
                    fn);
}

size_t csa_index_topk_workspace_size(int64_t B, int64_t T, int64_t n_cap, int k,
                                     int scores_in_workspace) {
  if (B < 1 || T < 1 || n_cap < 1) return 0;
  size_t s = csa_topk_workspace_size(B, T, n_cap, k);
  if (scores_in_workspace) s += round_up(static_cast<size_t>(B * T) * n_cap * sizeof(float));
  return s;
}

int csa_index_topk(const void* qi, int qi_dtype, const void* qi_scale, const float* w,
                   const void* ki, int ki_dtype, const void* ki_scale, const int64_t* pos0,
                   int64_t B, int64_t T, int64_t H_I, int64_t d_I, int64_t n_cap, int m, int act,
                   int k, float* scores, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "csa_index_topk";
  const bool scores_in_ws = scores == nullptr;
  const size_t need = csa_index_topk_workspace_size(B, T, n_cap, k, scores_in_ws ? 1 : 0);
  CSA_REQUIRE(need == 0 || (ws && ws_bytes >= need) ||
                  (!ws && !scores_in_ws && topk_ws_optional(B, T)),
              CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, got %zu", fn, need,
              ws ? ws_bytes : 0);
  CSA_REQUIRE(ws == nullptr || aligned16(ws), CSA_ERR_WORKSPACE, "%s: ws must be 16-byte aligned",
              fn);
  float* sc = scores;
  char* topk_ws = static_cast<char*>(ws);
  if (scores_in_ws && ws) {
    sc = static_cast<float*>(ws);
    topk_ws += round_up(static_cast<size_t>(B * T) * n_cap * sizeof(float));
  }
  int rc = check_index_args(qi, qi_dtype, qi_scale, w, ki, ki_dtype, ki_scale, pos0, B, T, H_I,
                            d_I, n_cap, m, act, sc, fn);
  if (rc) return rc;
  rc = check_topk_args(sc, pos0, B, T, n_cap, m, k, idx, fn);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* hist = csa::topk_hist_ptr(topk_ws, B, T);
  const csa::CoarseHist coarse = csa::topk_coarse_hist(topk_ws, B, T);
  rc = hip_result(csa::launch_index_scores(qi, qi_dtype, qi_scale, w, ki, ki_scale, pos0, B, T,
                                           H_I, d_I, n_cap, m, act, sc, hist, k, nullptr, s,
                                           &coarse),
                  fn);
  if (rc) return rc;
  return hip_result(csa::launch_topk(sc, pos0, B, T, n_cap, m, k, idx, topk_ws, hist != nullptr, s),
                    fn);
}

int csa_decode_index_topk(const void* qi, const float* w, void* kc, void* vc, const void* kr,
                          const void* vr, const float* zk, const float* zv,
                          const int64_t* raw_pos0, int64_t R, const int64_t* pos0, int64_t B,
                          int64_t H_I, int64_t d, int64_t n_cap, int m, int act, int k,
                          float* scores, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "csa_decode_index_topk";
  CSA_REQUIRE(kc && vc && kr && vr && zk && zv && raw_pos0, CSA_ERR_NULL,
              "%s: kc, vc, kr, vr, zk, zv and raw_pos0 must be non-NULL", fn);
  CSA_REQUIRE(R >= m && m >= 1, CSA_ERR_SHAPE, "%s: the raw buffer must hold a block (R >= m >= 1)",
              fn);
  CSA_REQUIRE(m <= csa::kFusedMaxM, CSA_ERR_UNSUPPORTED, "%s: m must be <= %d", fn,
              csa::kFusedMaxM);
  CSA_REQUIRE(aligned16(vc), CSA_ERR_SHAPE, "%s: vc must be 16-byte aligned", fn);
  const int64_t T = 1;
  const bool scores_in_ws = scores == nullptr;
  const size_t need = csa_index_topk_workspace_size(B, T, n_cap, k, scores_in_ws ? 1 : 0);
  CSA_REQUIRE(need == 0 || (ws && ws_bytes >= need) ||
                  (!ws && !scores_in_ws && topk_ws_optional(B, T)),
              CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, got %zu", fn, need,
              ws ? ws_bytes : 0);
  CSA_REQUIRE(ws == nullptr || aligned16(ws), CSA_ERR_WORKSPACE, "%s: ws must be 16-byte aligned",
              fn);
  float* sc = scores;
  char* topk_ws = static_cast<char*>(ws);
  if (scores_in_ws && ws) {
    sc = static_cast<float*>(ws);
    topk_ws += round_up(static_cast<size_t>(B * T) * n_cap * sizeof(float));
  }
  int rc = check_index_args(qi, CSA_BF16, nullptr, w, kc, CSA_BF16, nullptr, pos0, B, T, H_I, d,
                            n_cap, m, act, sc, fn);
  if (rc) return rc;
  rc = check_topk_args(sc, pos0, B, T, n_cap, m, k, idx, fn);
  if (rc) return rc;
  csa::FusedCompress fc;
  fc.kr = static_cast<const uint16_t*>(kr);
  fc.vr = static_cast<const uint16_t*>(vr);
  fc.zk = zk;
  fc.zv = zv;
  fc.raw_pos0 = raw_pos0;
  fc.kc = static_cast<uint16_t*>(kc);
  fc.vc = static_cast<uint16_t*>(vc);
  fc.R = R;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* hist = csa::topk_hist_ptr(topk_ws, B, T);
  const csa::CoarseHist coarse = csa::topk_coarse_hist(topk_ws, B, T);
  rc = hip_result(csa::launch_index_scores(qi, CSA_BF16, nullptr, w, kc, nullptr, pos0, B, T, H_I,
                                           d, n_cap, m, act, sc, hist, k, &fc, s, &coarse),
                  fn);
  if (rc) return rc;
  return hip_result(csa::launch_topk(sc, pos0, B, T, n_cap, m, k, idx, topk_ws, hist != nullptr, s),
                    fn);
}

size_t csa_attend_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d, int k, int W) {
  if (B < 1 || T < 1 || H < 1 || d < 1 || k < 0 || W < 0) return 0;
  return round_up(csa::attend_workspace_bytes(B * T, H, d, static_cast<int64_t>(k) + W, false));
}

int csa_attend(const void* q, int q_dtype, const void* kc, const void* vc, int kv_dtype,
               const int32_t* idx, int k, const void* kr, const void* vr,
               const int64_t* raw_pos0, int64_t R, const int64_t* pos0, int64_t B, int64_t T,
               int64_t H, int64_t d, int64_t n_cap, int W, float scale, float* out, float* lse,
               void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "csa_attend";
  int rc = check_attend_args(q, q_dtype, kc, vc, kv_dtype, kr, vr, raw_pos0, R, pos0, B, T, H, d,
                             n_cap, W, scale, out, fn);
  if (rc) return rc;
  CSA_REQUIRE(k >= 0 && k <= 65536, CSA_ERR_UNSUPPORTED, "%s: k must be in [0, 65536]", fn);
  CSA_REQUIRE(k == 0 || idx, CSA_ERR_NULL, "%s: idx must be non-NULL when k > 0", fn);
  CSA_REQUIRE(k + W >= 1, CSA_ERR_SHAPE, "%s: k + W must be >= 1", fn);
  const size_t need = csa_attend_workspace_size(B, T, H, d, k, W);
  CSA_REQUIRE(need == 0 || (ws && ws_bytes >= need), CSA_ERR_WORKSPACE,
              "%s: workspace of %zu bytes needed, got %zu", fn, need, ws ? ws_bytes : 0);
  CSA_REQUIRE(ws == nullptr || aligned16(ws), CSA_ERR_WORKSPACE, "%s: ws must be 16-byte aligned",
              fn);
  return hip_result(csa::launch_attend(q, q_dtype, kc, vc, idx, k, 0, kr, vr, raw_pos0, R, pos0, B,
                                       T, H, d, n_cap, W, scale, out, lse, ws,
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

// ------------------------------------------------------ the decode step

size_t csa_decode_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d, int64_t n_cap, int k,
                                 int W, int scores_in_workspace) {
  if (B < 1 || T < 1 || H < 1 || d < 1 || n_cap < 1 || k < 1 || W < 0) return 0;
  size_t s = csa_topk_workspace_size(B, T, n_cap, k) + csa_attend_workspace_size(B, T, H, d, k, W);
  if (scores_in_workspace) s += round_up(static_cast<size_t>(B * T) * n_cap * sizeof(float));
  return s;
}

// Top-k selection and attention on a checked top-k workspace: for few long
// rows the classify launch, then the attention launch that makes the
// selection from its lists; otherwise csa_topk's kernels, then attention.
static int select_attend_launch(const float* scores, void* topk_ws, bool hist_ready,
                                const int64_t* pos0, int m, int k, const void* q, int kv_dtype,
                                const void* kc, const void* vc, const void* kr, const void* vr,
                                const int64_t* raw_pos0, int64_t R, int64_t B, int64_t T,
                                int64_t H, int64_t d, int64_t n_cap, int W, float scale,
                                int32_t* idx, float* out, float* lse, void* att_ws, hipStream_t s,
                                const char* fn) {
  csa::TopkLists lists{};
  int rc = csa::launch_topk_lists(scores, pos0, B, T, n_cap, m, k, topk_ws, hist_ready, &lists, s);
  if (rc < 0) return hip_result(rc, fn);
  if (rc == 0) {
    lists.idx = idx;
    return hip_result(csa::launch_attend(q, kv_dtype, kc, vc, nullptr, k, 0, kr, vr, raw_pos0, R,
                                         pos0, B, T, H, d, n_cap, W, scale, out, lse, att_ws, s,
                                         &lists),
                      fn);
  }
  rc = hip_result(csa::launch_topk(scores, pos0, B, T, n_cap, m, k, idx, topk_ws, hist_ready, s),
                  fn);
  if (rc) return rc;
  return hip_result(csa::launch_attend(q, kv_dtype, kc, vc, idx, k, 0, kr, vr, raw_pos0, R, pos0,
                                       B, T, H, d, n_cap, W, scale, out, lse, att_ws, s),
                    fn);
}

int csa_select_attend(const float* scores, void* topk_ws, size_t topk_ws_bytes, int hist_ready,
                      const int64_t* pos0, int m, int k, const void* q, const void* kc,
                      const void* vc, int kv_dtype, const void* kr, const void* vr,
                      const int64_t* raw_pos0, int64_t R, int64_t B, int64_t T, int64_t H,
                      int64_t d, int64_t n_cap, int W, float scale, int32_t* idx, float* out,
                      float* lse, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "csa_select_attend";
  int rc = check_topk_args(scores, pos0, B, T, n_cap, m, k, idx, fn);
  if (rc) return rc;
  rc = check_attend_args(q, kv_dtype, kc, vc, kv_dtype, kr, vr, raw_pos0, R, pos0, B, T, H, d,
                         n_cap, W, scale, out, fn);
  if (rc) return rc;
  const size_t need_t = csa_topk_workspace_size(B, T, n_cap, k);
  CSA_REQUIRE(need_t == 0 || (topk_ws && topk_ws_bytes >= need_t && aligned16(topk_ws)),
              CSA_ERR_WORKSPACE,
              "%s: top-k workspace of %zu bytes (16-byte aligned) needed, got %zu", fn, need_t,
              topk_ws ? topk_ws_bytes : 0);
  const size_t need = csa_attend_workspace_size(B, T, H, d, k, W);
  CSA_REQUIRE(need == 0 || (ws && ws_bytes >= need && aligned16(ws)), CSA_ERR_WORKSPACE,
              "%s: workspace of %zu bytes (16-byte aligned) needed, got %zu", fn, need,
              ws ? ws_bytes : 0);
  return select_attend_launch(scores, topk_ws, hist_ready != 0 && need_t != 0, pos0, m, k, q,
                              kv_dtype, kc, vc, kr, vr, raw_pos0, R, B, T, H, d, n_cap, W, scale,
                              idx, out, lse, ws, static_cast<hipStream_t>(stream), fn);
}

// The arguments of a decode step.
struct DecodeArgs {
  const void* qi; int qi_dtype; const void* qi_scale; const float* w; const void* ki;
  int ki_dtype; const void* ki_scale; const void* q; void* kc; void* vc; int kv_dtype;
  const void* kr; const void* vr; const float* zk; const float* zv; const int64_t* raw_pos0;
  int64_t R; const int64_t* pos0; int64_t B, T, H_I, d_I, H, d, n_cap; int m, act, k, W;
  float scale; float* scores; int32_t* idx; float* out; float* lse;
};

// Argument checks of a decode step (everything but the workspace).
static int decode_check(const DecodeArgs& a, const char* fn) {
  // scores == NULL is valid (they then live in the workspace)
  static const float kInWorkspace = 0.f;
  const float* sc = a.scores ? a.scores : &kInWorkspace;
  int rc = check_index_args(a.qi, a.qi_dtype, a.qi_scale, a.w, a.ki, a.ki_dtype, a.ki_scale,
                            a.pos0, a.B, a.T, a.H_I, a.d_I, a.n_cap, a.m, a.act, sc, fn);
  if (rc) return rc;
  rc = check_topk_args(sc, a.pos0, a.B, a.T, a.n_cap, a.m, a.k, a.idx, fn);
  if (rc) return rc;
  rc = check_attend_args(a.q, a.kv_dtype, a.kc, a.vc, a.kv_dtype, a.kr, a.vr, a.raw_pos0, a.R,
                         a.pos0, a.B, a.T, a.H, a.d, a.n_cap, a.W, a.scale, a.out, fn);
  if (rc) return rc;
  if (a.zk != nullptr || a.zv != nullptr) {
    CSA_REQUIRE(a.zk && a.zv && a.kr && a.vr && a.raw_pos0, CSA_ERR_NULL,
                "%s: block compression needs zk, zv, kr, vr and raw_pos0", fn);
    CSA_REQUIRE(a.T == 1 && a.ki == a.kc && a.ki_dtype == CSA_BF16 && a.kv_dtype == CSA_BF16,
                CSA_ERR_UNSUPPORTED,
                "%s: block compression needs T == 1 and bf16 indexer keys that are kc", fn);
    CSA_REQUIRE(a.R >= a.m && a.m <= csa::kFusedMaxM, CSA_ERR_UNSUPPORTED,
                "%s: block compression needs R >= m and m <= %d", fn, csa::kFusedMaxM);
  }
  return CSA_OK;
}

// The launches of a checked decode step on a workspace of
// csa_decode_workspace_size() bytes: the top-k workspace (whose zero-state
// part leads it) first, then the scores when they live in the workspace,
// then the attention partials.
static int decode_launch(const DecodeArgs& a, void* ws, hipStream_t s, const char* fn) {
  const int64_t B = a.B, T = a.T, n_cap = a.n_cap;
  char* p = static_cast<char*>(ws);
  void* topk_ws = p;
  p += csa_topk_workspace_size(B, T, n_cap, a.k);
  float* sc = a.scores;
  if (sc == nullptr) {
    sc = reinterpret_cast<float*>(p);
    p += round_up(static_cast<size_t>(B * T) * n_cap * sizeof(float));
  }
  void* att_ws = p;
  csa::FusedCompress fc{};
  const bool compress = a.zk != nullptr;
  if (compress) {
    fc.kr = static_cast<const uint16_t*>(a.kr);
    fc.vr = static_cast<const uint16_t*>(a.vr);
    fc.zk = a.zk;
    fc.zv = a.zv;
    fc.raw_pos0 = a.raw_pos0;
    fc.kc = static_cast<uint16_t*>(a.kc);
    fc.vc = static_cast<uint16_t*>(a.vc);
    fc.R = a.R;
  }
  uint32_t* hist = csa::topk_hist_ptr(topk_ws, B, T);
  const csa::CoarseHist coarse = csa::topk_coarse_hist(topk_ws, B, T);
  int rc = hip_result(csa::launch_index_scores(a.qi, a.qi_dtype, a.qi_scale, a.w, a.ki,
                                               a.ki_scale, a.pos0, B, T, a.H_I, a.d_I, n_cap, a.m,
                                               a.act, sc, hist, a.k, compress ? &fc : nullptr, s,
                                               &coarse),
                      fn);
  if (rc) return rc;
  return select_attend_launch(sc, topk_ws, hist != nullptr, a.pos0, a.m, a.k, a.q, a.kv_dtype,
                              a.kc, a.vc, a.kr, a.vr, a.raw_pos0, a.R, B, T, a.H, a.d, n_cap, a.W,
                              a.scale, a.idx, a.out, a.lse, att_ws, s, fn);
}

int csa_decode(const void* qi, int qi_dtype, const void* qi_scale, const float* w, const void* ki,
               int ki_dtype, const void* ki_scale, const void* q, void* kc, void* vc,
               int kv_dtype, const void* kr, const void* vr, const float* zk, const float* zv,
               const int64_t* raw_pos0, int64_t R, const int64_t* pos0, int64_t B, int64_t T,
               int64_t H_I, int64_t d_I, int64_t H, int64_t d, int64_t n_cap, int m, int act,
               int k, int W, float scale, float* scores, int32_t* idx, float* out, float* lse,
               void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "csa_decode";
  const DecodeArgs a{qi, qi_dtype, qi_scale, w, ki, ki_dtype, ki_scale, q, kc, vc, kv_dtype,
                     kr, vr, zk, zv, raw_pos0, R, pos0, B, T, H_I, d_I, H, d, n_cap, m, act, k,
                     W, scale, scores, idx, out, lse};
  int rc = decode_check(a, fn);
  if (rc) return rc;
  const size_t need = csa_decode_workspace_size(B, T, H, d, n_cap, k, W, scores == nullptr ? 1 : 0);
  CSA_REQUIRE(ws && ws_bytes >= need && aligned16(ws), CSA_ERR_WORKSPACE,
              "%s: workspace of %zu bytes (16-byte aligned) needed, got %zu", fn, need,
              ws ? ws_bytes : 0);
  return decode_launch(a, ws, static_cast<hipStream_t>(stream), fn);
}

size_t csa_decode_noalloc_max_bytes(void) { return csa::kStaticScratchBytes; }

int csa_decode_noalloc(const void* qi, int qi_dtype, const void* qi_scale, const float* w,
                       const void* ki, int ki_dtype, const void* ki_scale, const void* q, void* kc,
                       void* vc, int kv_dtype, const void* kr, const void* vr, const float* zk,
                       const float* zv, const int64_t* raw_pos0, int64_t R, const int64_t* pos0,
                       int64_t B, int64_t T, int64_t H_I, int64_t d_I, int64_t H, int64_t d,
                       int64_t n_cap, int m, int act, int k, int W, float scale, float* scores,
                       int32_t* idx, float* out, float* lse, void* stream) {
  const char* fn = "csa_decode_noalloc";
  const DecodeArgs a{qi, qi_dtype, qi_scale, w, ki, ki_dtype, ki_scale, q, kc, vc, kv_dtype,
                     kr, vr, zk, zv, raw_pos0, R, pos0, B, T, H_I, d_I, H, d, n_cap, m, act, k,
                     W, scale, scores, idx, out, lse};
  int rc = decode_check(a, fn);
  if (rc) return rc;
  const size_t need = csa_decode_workspace_size(B, T, H, d, n_cap, k, W, scores == nullptr ? 1 : 0);
  CSA_REQUIRE(need <= csa::kStaticScratchBytes, CSA_ERR_UNSUPPORTED,
              "%s: these sizes need %zu bytes of scratch; the fixed scratch holds %zu "
              "(use csa_decode with a workspace)",
              fn, need, csa::kStaticScratchBytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  CSA_REQUIRE(csa::static_scratch(s, B * T, n_cap, csa::topk_zero_state_bytes(B, T), &ws) == 0,
              CSA_ERR_HIP, "%s: the fixed scratch could not be located or cleared: %s", fn,
              hipGetErrorString(hipGetLastError()));
  rc = decode_launch(a, ws, s, fn);
  // a launch that failed part way may leave the histograms dirty
  if (rc != CSA_OK) csa::static_scratch_mark_dirty();
  return rc;
}

size_t hca_attend_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d, int64_t n_cap,
                                 int W) {
  if (B < 1 || T < 1 || H < 1 || d < 1 || n_cap < 1 || W < 0) return 0;
  return round_up(csa::attend_workspace_bytes(B * T, H, d, n_cap + W, true));
}

int hca_attend(const void* q, int q_dtype, const void* kc, const void* vc, int kv_dtype, int m,
               const void* kr, const void* vr, const int64_t* raw_pos0, int64_t R,
               const int64_t* pos0, int64_t B, int64_t T, int64_t H, int64_t d, int64_t n_cap,
               int W, float scale, float* out, float* lse, void* ws, size_t ws_bytes,
               void* stream) {
  const char* fn = "hca_attend";
  int rc = check_attend_args(q, q_dtype, kc, vc, kv_dtype, kr, vr, raw_pos0, R, pos0, B, T, H, d,
                             n_cap, W, scale, out, fn);
  if (rc) return rc;
  CSA_REQUIRE(m >= 1, CSA_ERR_SHAPE, "%s: m must be >= 1", fn);
  const size_t need = hca_attend_workspace_size(B, T, H, d, n_cap, W);
  CSA_REQUIRE(need == 0 || (ws && ws_bytes >= need), CSA_ERR_WORKSPACE,
              "%s: workspace of %zu bytes needed, got %zu", fn, need, ws ? ws_bytes : 0);
  CSA_REQUIRE(ws == nullptr || aligned16(ws), CSA_ERR_WORKSPACE, "%s: ws must be 16-byte aligned",
              fn);
  return hip_result(csa::launch_attend(q, q_dtype, kc, vc, nullptr, 0, m, kr, vr, raw_pos0, R,
                                       pos0, B, T, H, d, n_cap, W, scale, out, lse, ws,
                                       static_cast<hipStream_t>(stream)),
                    fn);
}


// ------------------------------------------------------------ backward pass

static int check_bwd_args(const float* out, const float* lse, const float* dout, float* dq,
                          float* dkc, float* dvc, float* dkr, float* dvr, int W, int64_t H,
                          int64_t d, const char* fn) {
  CSA_REQUIRE(out && lse && dout && dq && dkc && dvc, CSA_ERR_NULL,
              "%s: out, lse, dout, dq, dkc and dvc must be non-NULL", fn);
  CSA_REQUIRE(W == 0 || (dkr && dvr), CSA_ERR_NULL, "%s: dkr and dvr must be non-NULL when W > 0",
              fn);
  CSA_REQUIRE(H >= 1 && H <= 64, CSA_ERR_UNSUPPORTED, "%s: H must be in [1, 64]", fn);
  CSA_REQUIRE(d == 64 || d == 128, CSA_ERR_UNSUPPORTED, "%s: d must be 64 or 128", fn);
  CSA_REQUIRE(aligned16(out) && aligned16(dout) && aligned16(dq), CSA_ERR_SHAPE,
              "%s: out, dout and dq must be 16-byte aligned", fn);
  return CSA_OK;
}

size_t csa_attend_backward_workspace_size(int64_t B, int64_t T, int64_t d, int64_t n_cap, int k,
                                          int W) {
  if (B < 1 || T < 1 || d < 1 || n_cap < 1 || k < 0 || W < 0) return 0;
  return round_up(csa::attend_bwd_workspace_bytes(B, T, d, k, W, n_cap, true));
}

size_t hca_attend_backward_workspace_size(int64_t B, int64_t T, int64_t d, int64_t n_cap, int W) {
  if (B < 1 || T < 1 || d < 1 || n_cap < 1 || W < 0) return 0;
  return round_up(csa::attend_bwd_workspace_bytes(B, T, d, n_cap, W, n_cap, false));
}

static int attend_backward_impl(const void* q, int q_dtype, const void* kc, const void* vc,
                                int kv_dtype, const int32_t* idx, int k, int hca_m,
                                const void* kr, const void* vr, const int64_t* raw_pos0,
                                int64_t R, const int64_t* pos0, int64_t B, int64_t T, int64_t H,
                                int64_t d, int64_t n_cap, int W, float scale, const float* out,
                                const float* lse, const float* dout, float* dq, float* dkc,
                                float* dvc, float* dkr, float* dvr, void* ws, size_t ws_bytes,
                                void* stream, const char* fn) {
  int rc = check_attend_args(q, q_dtype, kc, vc, kv_dtype, kr, vr, raw_pos0, R, pos0, B, T, H, d,
                             n_cap, W, scale, out, fn);
  if (rc) return rc;
  rc = check_bwd_args(out, lse, dout, dq, dkc, dvc, dkr, dvr, W, H, d, fn);
  if (rc) return rc;
  CSA_REQUIRE(B * T <= kMaxIndex, CSA_ERR_UNSUPPORTED, "%s: B*T too large", fn);
  const size_t need = hca_m > 0 ? hca_attend_backward_workspace_size(B, T, d, n_cap, W)
                                : csa_attend_backward_workspace_size(B, T, d, n_cap, k, W);
  CSA_REQUIRE(ws && ws_bytes >= need, CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, got %zu",
              fn, need, ws ? ws_bytes : 0);
  CSA_REQUIRE(aligned16(ws), CSA_ERR_WORKSPACE, "%s: ws must be 16-byte aligned", fn);
  return hip_result(csa::launch_attend_bwd(q, q_dtype, kc, vc, idx, k, hca_m, kr, vr, raw_pos0, R,
                                           pos0, B, T, H, d, n_cap, W, scale, out, lse, dout, dq,
                                           dkc, dvc, dkr, dvr, ws,
                                           static_cast<hipStream_t>(stream)),
                    fn);
}

int csa_attend_backward(const void* q, int q_dtype, const void* kc, const void* vc, int kv_dtype,
                        const int32_t* idx, int k, const void* kr, const void* vr,
                        const int64_t* raw_pos0, int64_t R, const int64_t* pos0, int64_t B,
                        int64_t T, int64_t H, int64_t d, int64_t n_cap, int W, float scale,
                        const float* out, const float* lse, const float* dout, float* dq,
                        float* dkc, float* dvc, float* dkr, float* dvr, void* ws, size_t ws_bytes,
                        void* stream) {
  const char* fn = "csa_attend_backward";
  CSA_REQUIRE(idx, CSA_ERR_NULL, "%s: idx must be non-NULL", fn);
  CSA_REQUIRE(k >= 1 && k <= 4096, CSA_ERR_UNSUPPORTED, "%s: k must be in [1, 4096]", fn);
  CSA_REQUIRE(T <= csa::kBwdMaxRows, CSA_ERR_UNSUPPORTED, "%s: T must be <= %lld", fn,
              static_cast<long long>(csa::kBwdMaxRows));
  CSA_REQUIRE(B * T * k < (int64_t(1) << 32), CSA_ERR_UNSUPPORTED, "%s: B*T*k must be < 2^32",
              fn);
  return attend_backward_impl(q, q_dtype, kc, vc, kv_dtype, idx, k, 0, kr, vr, raw_pos0, R, pos0,
                              B, T, H, d, n_cap, W, scale, out, lse, dout, dq, dkc, dvc, dkr, dvr,
                              ws, ws_bytes, stream, fn);
}

int hca_attend_backward(const void* q, int q_dtype, const void* kc, const void* vc, int kv_dtype,
                        int m, const void* kr, const void* vr, const int64_t* raw_pos0, int64_t R,
                        const int64_t* pos0, int64_t B, int64_t T, int64_t H, int64_t d,
                        int64_t n_cap, int W, float scale, const float* out, const float* lse,
                        const float* dout, float* dq, float* dkc, float* dvc, float* dkr,
                        float* dvr, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "hca_attend_backward";
  CSA_REQUIRE(m >= 1, CSA_ERR_SHAPE, "%s: m must be >= 1", fn);
  CSA_REQUIRE(n_cap <= 65536, CSA_ERR_UNSUPPORTED, "%s: n_cap must be <= 65536", fn);
  return attend_backward_impl(q, q_dtype, kc, vc, kv_dtype, nullptr, 0, m, kr, vr, raw_pos0, R,
                              pos0, B, T, H, d, n_cap, W, scale, out, lse, dout, dq, dkc, dvc, dkr,
                              dvr, ws, ws_bytes, stream, fn);
}

int csa_compress_backward(const void* x, int x_dtype, const float* logits, const float* dc,
                          int64_t B, int64_t n_tok, int64_t d, int m, int64_t x_sb, int64_t z_sb,
                          float* dx, float* dlogits, void* stream) {
  const char* fn = "csa_compress_backward";
  CSA_REQUIRE(x && logits && dc && dx && dlogits, CSA_ERR_NULL,
              "%s: x, logits, dc, dx and dlogits must be non-NULL", fn);
  CSA_REQUIRE(x_dtype == CSA_F32 || x_dtype == CSA_BF16, CSA_ERR_DTYPE,
              "%s: x_dtype must be F32 or BF16", fn);
  CSA_REQUIRE(B >= 1 && B <= kMaxGridY && d >= 1 && m >= 1, CSA_ERR_SHAPE,
              "%s: need 1 <= B <= %lld, d >= 1, m >= 1", fn, static_cast<long long>(kMaxGridY));
  CSA_REQUIRE(n_tok >= 0 && n_tok % m == 0, CSA_ERR_SHAPE, "%s: n_tok must be a multiple of m", fn);
  CSA_REQUIRE(x_sb >= n_tok * d && z_sb >= n_tok * d, CSA_ERR_SHAPE,
              "%s: batch strides must be >= n_tok * d", fn);
  if (n_tok == 0) return CSA_OK;
  return hip_result(csa::launch_compress_bwd(x, x_dtype, logits, dc, B, n_tok, d, m, x_sb, z_sb,
                                             dx, dlogits, static_cast<hipStream_t>(stream)),
                    fn);
}

}  // extern "C"
