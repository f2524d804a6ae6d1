// extern "C" entry points of liblca: host-side validation, then launches.
// Every check runs before anything is enqueued; a failing call enqueues nothing.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <cmath>
#include <string>

#include "lca_common.h"

namespace lca {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

// launchers (lca_compress.hip, lca_indexer.hip, lca_attention.hip)
int launch_compress(const lca_compress_stream* streams, int n, const int64_t* tok_off, const int64_t* done_len,
                    int B, float eps, int dtype, hipStream_t stream);
size_t index_topk_workspace(int rows, int64_t maxN, int k);
int launch_index_score(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                       const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w, int64_t maxN,
                       float* scores, void* ws, int dtype, hipStream_t stream);
int launch_index_score_append(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                              const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w, int64_t maxN,
                              const lca_compress_stream* idx_stream, const lca_compress_stream* kv_streams, int n_kv,
                              const int64_t* tok_off, const int64_t* done_len, float eps, float* scores, void* ws,
                              int dtype, hipStream_t stream);
int launch_topk_select(const int64_t* csa_off, const int32_t* q_pos, int B, int Tq, int k, int m, int w,
                       int64_t maxN, int32_t* idx, const float* scores, void* ws, hipStream_t stream);
int launch_attention(const lca_attn_source* srcs, int n_src, const void* q, const int32_t* q_pos, int B, int Tq,
                     int H, int D, float scale, float eps, int dtype, hipStream_t stream);
int launch_attention_merge(const lca_attn_source* srcs, int n_src, const void* q, const int32_t* q_pos, int B,
                           int Tq, int H, int D, float scale, float eps, const float* sink, void* out, int dtype,
                           hipStream_t stream);

static lca_attn_source make_source(int kind, const void* kv, const int64_t* off, const int32_t* idx, int k, int m2,
                                   int w2, int W, int n_split, float* o_part, float* lse) {
  lca_attn_source s{};
  s.kind = kind; s.kv = kv; s.off = off; s.idx = idx; s.k = k; s.m2 = m2; s.w2 = w2; s.W = W;
  s.n_split = n_split; s.o_part = o_part; s.lse = lse;
  return s;
}
int launch_merge(const lca_partial* parts, int n_parts, const float* win_o, const float* win_lse,
                 const float* sink, int rows, int H, int D, void* out, int dtype, hipStream_t stream);
void diag_set_trace(uint64_t* buf, int64_t words);
size_t index_noalloc_max_bytes();
bool index_topk_stream_applies(int B, int Tq, int HI, int dI, int k, int64_t maxN, int dtype);
int launch_index_topk_stream(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                             const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w, int64_t maxN,
                             int32_t* idx, void* ws, int dtype, hipStream_t stream);
int launch_index_topk_noalloc(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                              const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w,
                              int64_t maxN, int32_t* idx, float* scores, int dtype, hipStream_t stream);
int launch_decode_front(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                        const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w, int64_t maxN,
                        const lca_compress_stream* idx_stream, const lca_compress_stream* kv_streams, int n_kv,
                        const int64_t* tok_off, const int64_t* done_len, float eps, float* scores, void* ws,
                        const lca_attn_source* srcs, int n_src, const void* q, int H, int D, float scale, int dtype,
                        hipStream_t stream);
void diag_set_topk_wait(uint32_t extra, uint32_t ticks);

static bool sync_mode() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("LCA_SYNC");
    v = (e && e[0] == '1') ? 1 : 0;
  }
  return v == 1;
}

static int finish(int rc, hipStream_t stream, const char* what) {
  if (rc != LCA_OK) {
    if (rc == LCA_ERR_HIP) set_error("%s: launch failed: %s", what, hipGetErrorString(hipGetLastError()));
    return rc;
  }
  if (sync_mode()) {
    hipError_t e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) {
      set_error("%s: %s", what, hipGetErrorString(e));
      return LCA_ERR_HIP;
    }
  }
  g_last_error.clear();
  return LCA_OK;
}

#define LCA_REQUIRE(cond, code, ...) \
  do {                               \
    if (!(cond)) {                   \
      set_error(__VA_ARGS__);        \
      return (code);                 \
    }                                \
  } while (0)

static bool valid_dtype(int d) { return d == LCA_F32 || d == LCA_BF16; }
static bool valid_head_dim(int D) { return D == 64 || D == 128 || D == 256 || D == 512; }

}  // namespace lca

using namespace lca;

extern "C" {

const char* lca_strerror(int status) {
  switch (status) {
    case LCA_OK: return "ok";
    case LCA_ERR_INVALID_ARG: return "invalid argument";
    case LCA_ERR_UNSUPPORTED: return "unsupported shape or type";
    case LCA_ERR_WORKSPACE: return "workspace missing or too small";
    case LCA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* lca_last_error(void) { return g_last_error.c_str(); }

int lca_version(void) { return 200; }

int lca_diag_trace(uint64_t* buf, int64_t n_words) {
  LCA_REQUIRE(buf == nullptr || n_words >= 0, LCA_ERR_INVALID_ARG, "diag_trace: n_words=%lld < 0",
              (long long)n_words);
  diag_set_trace(buf, n_words);
  g_last_error.clear();
  return LCA_OK;
}

int lca_diag_topk_wait(int extra_shares, int64_t max_ticks) {
  LCA_REQUIRE(extra_shares >= 0 && extra_shares <= 1024, LCA_ERR_INVALID_ARG,
              "diag_topk_wait: extra_shares=%d outside [0, 1024]", extra_shares);
  LCA_REQUIRE(max_ticks >= 0 && max_ticks <= 100000000, LCA_ERR_INVALID_ARG,
              "diag_topk_wait: max_ticks=%lld outside [0, 1e8]", (long long)max_ticks);
  diag_set_topk_wait((uint32_t)extra_shares, (uint32_t)max_ticks);
  g_last_error.clear();
  return LCA_OK;
}

static int check_streams(const lca_compress_stream* streams, int n_streams, int dtype) {
  const int VE = dtype == LCA_BF16 ? 8 : 4;
  for (int k = 0; k < n_streams; ++k) {
    const lca_compress_stream& s = streams[k];
    LCA_REQUIRE(s.src && s.logits && s.out && s.ent_off, LCA_ERR_INVALID_ARG,
                "kv_compress: stream %d has a NULL pointer", k);
    LCA_REQUIRE(s.C > 0 && s.C <= 1024 && s.C % VE == 0, LCA_ERR_INVALID_ARG,
                "kv_compress: stream %d: C=%d must be a positive multiple of %d, at most 1024", k, s.C, VE);
    const int lanes = s.C / VE;
    const bool lanes_ok = (lanes <= 64 && (64 % lanes) == 0) || (lanes % 64 == 0 && lanes / 64 <= (VE == 8 ? 2 : 4));
    LCA_REQUIRE(lanes_ok, LCA_ERR_UNSUPPORTED, "kv_compress: stream %d: C=%d is not a supported width", k, s.C);
    LCA_REQUIRE(s.m >= 1 && s.w >= s.m && s.w <= 4096, LCA_ERR_INVALID_ARG,
                "kv_compress: stream %d: need 1 <= m <= w <= 4096 (m=%d, w=%d)", k, s.m, s.w);
    LCA_REQUIRE(s.per_channel == 0 || s.per_channel == 1, LCA_ERR_INVALID_ARG, "kv_compress: per_channel");
    LCA_REQUIRE(s.rmsnorm == 0 || s.rmsnorm == 1, LCA_ERR_INVALID_ARG, "kv_compress: rmsnorm");
    LCA_REQUIRE(s.max_entries >= 0, LCA_ERR_INVALID_ARG, "kv_compress: max_entries < 0");
    LCA_REQUIRE(s.out_key >= 0 && s.out_key <= 2, LCA_ERR_INVALID_ARG, "kv_compress: out_key");
    LCA_REQUIRE(!s.out_key || (dtype == LCA_BF16 && s.C <= 512 && s.w <= 16 && (s.w == s.m || s.w == 2 * s.m)),
                LCA_ERR_UNSUPPORTED, "kv_compress: stream %d: key rows need bf16 input, C <= 512 and w = m or 2m <= 16",
                k);
    LCA_REQUIRE(s.out_key != 2 || (s.C == 32 || s.C == 64 || s.C == 128 || s.C == 256), LCA_ERR_UNSUPPORTED,
                "kv_compress: stream %d: MXFP4 rows need C in {32, 64, 128, 256}", k);
    LCA_REQUIRE(s.rope_dims >= 0 && s.rope_dims <= s.C && s.rope_dims % 2 == 0 &&
                    (s.rope_dims == 0 || (s.out_key == 0 && std::isfinite(s.rope_base) && s.rope_base > 0.f)),
                LCA_ERR_INVALID_ARG,
                "kv_compress: stream %d: rope_dims=%d must be even, <= C, on rows of the input type, with a "
                "positive rope_base", k, s.rope_dims);
    LCA_REQUIRE((s.src2 == nullptr) == (s.logits2 == nullptr), LCA_ERR_INVALID_ARG,
                "kv_compress: stream %d: src2 and logits2 are given together or not at all", k);
    LCA_REQUIRE(!s.src2 || (s.w == 2 * s.m && s.w <= 16), LCA_ERR_UNSUPPORTED,
                "kv_compress: stream %d: the dual-stream form needs w = 2m <= 16 (m=%d, w=%d)", k, s.m, s.w);
  }
  return LCA_OK;
}

int lca_kv_compress(const lca_compress_stream* streams, int n_streams, const int64_t* tok_off,
                    const int64_t* done_len, int B, float eps, int dtype, void* stream) {
  LCA_REQUIRE(streams != nullptr, LCA_ERR_INVALID_ARG, "kv_compress: streams is NULL");
  LCA_REQUIRE(n_streams >= 1 && n_streams <= 4, LCA_ERR_INVALID_ARG, "kv_compress: n_streams=%d not in [1,4]",
              n_streams);
  LCA_REQUIRE(tok_off != nullptr, LCA_ERR_INVALID_ARG, "kv_compress: tok_off is NULL");
  LCA_REQUIRE(B >= 1, LCA_ERR_INVALID_ARG, "kv_compress: B=%d", B);
  LCA_REQUIRE(valid_dtype(dtype), LCA_ERR_INVALID_ARG, "kv_compress: dtype=%d", dtype);
  LCA_REQUIRE(std::isfinite(eps) && eps >= 0.f, LCA_ERR_INVALID_ARG, "kv_compress: eps must be finite and >= 0");
  int rc = check_streams(streams, n_streams, dtype);
  if (rc != LCA_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return finish(launch_compress(streams, n_streams, tok_off, done_len, B, eps, dtype, st), st, "kv_compress");
}

size_t lca_csa_index_topk_workspace(int n_rows, int64_t max_entries, int k) {
  if (n_rows < 1 || max_entries < 1 || k < 1) return 0;
  return index_topk_workspace(n_rows, max_entries, k);
}

static int check_index(const char* what, bool need_inputs, const void* p, const float* omega, const void* ikey,
                       const int64_t* csa_off, const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int k, int m,
                       int w, int64_t max_entries, void* ws, size_t ws_bytes, int dtype) {
  if (need_inputs) {
    LCA_REQUIRE(p && omega && ikey, LCA_ERR_INVALID_ARG, "%s: a required pointer is NULL", what);
    LCA_REQUIRE(H_I >= 1 && H_I <= 16 && d_I >= 8 && d_I % 8 == 0 && H_I * d_I <= 1024, LCA_ERR_UNSUPPORTED,
                "%s: H_I=%d d_I=%d unsupported", what, H_I, d_I);
    const bool keyrows = dtype == LCA_BF16_FP8KEY || dtype == LCA_BF16_MXFP4KEY;
    LCA_REQUIRE(valid_dtype(dtype) || keyrows, LCA_ERR_INVALID_ARG, "%s: dtype=%d", what, dtype);
    LCA_REQUIRE(!keyrows || (d_I == 32 || d_I == 64 || d_I == 128 || d_I == 256), LCA_ERR_UNSUPPORTED,
                "%s: fp8 / MXFP4 key rows need d_I in {32, 64, 128, 256} (d_I=%d)", what, d_I);
  }
  LCA_REQUIRE(csa_off && q_pos, LCA_ERR_INVALID_ARG, "%s: a required pointer is NULL", what);
  LCA_REQUIRE(B >= 1 && Tq >= 1, LCA_ERR_INVALID_ARG, "%s: B=%d Tq=%d", what, B, Tq);
  LCA_REQUIRE((int64_t)B * Tq <= 65535, LCA_ERR_UNSUPPORTED, "%s: B*Tq must be <= 65535", what);
  LCA_REQUIRE(k >= 1 && k <= 4096, LCA_ERR_UNSUPPORTED, "%s: k=%d not in [1,4096]", what, k);
  LCA_REQUIRE(m >= 1 && w >= 1, LCA_ERR_INVALID_ARG, "%s: m=%d w=%d", what, m, w);
  LCA_REQUIRE(max_entries >= 1 && max_entries < (1 << 24), LCA_ERR_UNSUPPORTED,
              "%s: max_entries=%lld not in [1, 2^24)", what, (long long)max_entries);
  const size_t need = index_topk_workspace(B * Tq, max_entries, k);
  LCA_REQUIRE(ws != nullptr && ws_bytes >= need, LCA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given",
              what, need, ws ? ws_bytes : (size_t)0);
  return LCA_OK;
}

int lca_csa_index_score(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                        const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int k, int m, int w,
                        int64_t max_entries, float* scores, void* ws, size_t ws_bytes, int dtype, void* stream) {
  int rc = check_index("csa_index_score", true, p, omega, ikey, csa_off, q_pos, B, Tq, H_I, d_I, k, m, w,
                       max_entries, ws, ws_bytes, dtype);
  if (rc != LCA_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return finish(launch_index_score(p, omega, ikey, csa_off, q_pos, B, Tq, H_I, d_I, k, m, w, max_entries, scores, ws,
                                   dtype, st),
                st, "csa_index_score");
}

}  // extern "C"

static int check_score_append(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                              const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int k, int m, int w,
                              int64_t max_entries, const lca_compress_stream* idx_stream,
                              const lca_compress_stream* kv_streams, int n_kv, const int64_t* tok_off,
                              const int64_t* done_len, float eps, void* ws, size_t ws_bytes, int dtype) {
  int rc = check_index("csa_index_score_append", true, p, omega, ikey, csa_off, q_pos, B, Tq, H_I, d_I, k, m, w,
                       max_entries, ws, ws_bytes, dtype);
  if (rc != LCA_OK) return rc;
  LCA_REQUIRE(idx_stream != nullptr && tok_off != nullptr && done_len != nullptr, LCA_ERR_INVALID_ARG,
              "csa_index_score_append: idx_stream, tok_off and done_len are required");
  LCA_REQUIRE(n_kv >= 0 && n_kv <= 4 && (n_kv == 0 || kv_streams != nullptr), LCA_ERR_INVALID_ARG,
              "csa_index_score_append: n_kv=%d not in [0,4] (or kv_streams is NULL)", n_kv);
  LCA_REQUIRE(idx_stream->out == ikey && idx_stream->ent_off == csa_off && idx_stream->C == d_I &&
                  idx_stream->m == m && idx_stream->w == w,
              LCA_ERR_INVALID_ARG,
              "csa_index_score_append: idx_stream must write ikey, packed by csa_off, with C = d_I, m and w");
  LCA_REQUIRE(std::isfinite(eps) && eps >= 0.f, LCA_ERR_INVALID_ARG,
              "csa_index_score_append: eps must be finite and >= 0");
  // the streams' inputs are bf16 when the keys are written as fp8 rows
  const int want_key = dtype == LCA_BF16_FP8KEY ? 1 : dtype == LCA_BF16_MXFP4KEY ? 2 : 0;
  const int in_dtype = want_key ? LCA_BF16 : dtype;
  LCA_REQUIRE(idx_stream->out_key == want_key, LCA_ERR_INVALID_ARG,
              "csa_index_score_append: the indexer-key stream's rows (out_key) must match dtype");
  LCA_REQUIRE(idx_stream->rope_dims == 0, LCA_ERR_INVALID_ARG,
              "csa_index_score_append: indexer keys are not rotated (rope_dims must be 0)");
  for (int i = 0; i < n_kv; ++i)
    LCA_REQUIRE(kv_streams[i].out_key == 0, LCA_ERR_INVALID_ARG, "csa_index_score_append: kv stream %d writes key rows", i);
  rc = check_streams(idx_stream, 1, in_dtype);
  if (rc == LCA_OK && n_kv > 0) rc = check_streams(kv_streams, n_kv, in_dtype);
  return rc;
}

extern "C" {

int lca_csa_index_score_append(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                               const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int k, int m, int w,
                               int64_t max_entries, const lca_compress_stream* idx_stream,
                               const lca_compress_stream* kv_streams, int n_kv, const int64_t* tok_off,
                               const int64_t* done_len, float eps, float* scores, void* ws, size_t ws_bytes,
                               int dtype, void* stream) {
  const int rc = check_score_append(p, omega, ikey, csa_off, q_pos, B, Tq, H_I, d_I, k, m, w, max_entries,
                                    idx_stream, kv_streams, n_kv, tok_off, done_len, eps, ws, ws_bytes, dtype);
  if (rc != LCA_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return finish(launch_index_score_append(p, omega, ikey, csa_off, q_pos, B, Tq, H_I, d_I, k, m, w, max_entries,
                                          idx_stream, kv_streams, n_kv, tok_off, done_len, eps, scores, ws, dtype,
                                          st),
                st, "csa_index_score_append");
}

int lca_csa_topk_select(const int64_t* csa_off, const int32_t* q_pos, int B, int Tq, int k, int m, int w,
                        int64_t max_entries, int32_t* idx, const float* scores, void* ws, size_t ws_bytes,
                        void* stream) {
  int rc = check_index("csa_topk_select", false, nullptr, nullptr, nullptr, csa_off, q_pos, B, Tq, 1, 8, k, m, w,
                       max_entries, ws, ws_bytes, LCA_BF16);
  if (rc != LCA_OK) return rc;
  LCA_REQUIRE(idx != nullptr, LCA_ERR_INVALID_ARG, "csa_topk_select: idx is NULL");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return finish(launch_topk_select(csa_off, q_pos, B, Tq, k, m, w, max_entries, idx, scores, ws, st), st,
                "csa_topk_select");
}

int lca_csa_index_topk(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                       const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int k, int m, int w,
                       int64_t max_entries, int32_t* idx, float* scores, void* ws, size_t ws_bytes, int dtype,
                       void* stream) {
  LCA_REQUIRE(idx != nullptr, LCA_ERR_INVALID_ARG, "csa_index_topk: idx is NULL");
  if (!scores && index_topk_stream_applies(B, Tq, H_I, d_I, k, max_entries, dtype)) {
    // many rows per sequence: scores and selection in one launch, no score stored
    int rc = check_index("csa_index_topk", true, p, omega, ikey, csa_off, q_pos, B, Tq, H_I, d_I, k, m, w,
                         max_entries, ws, ws_bytes, dtype);
    if (rc != LCA_OK) return rc;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    return finish(launch_index_topk_stream(p, omega, ikey, csa_off, q_pos, B, Tq, H_I, d_I, k, m, w, max_entries,
                                           idx, ws, dtype, st),
                  st, "csa_index_topk");
  }
  int rc = lca_csa_index_score(p, omega, ikey, csa_off, q_pos, B, Tq, H_I, d_I, k, m, w, max_entries, scores, ws,
                               ws_bytes, dtype, stream);
  if (rc != LCA_OK) return rc;
  return lca_csa_topk_select(csa_off, q_pos, B, Tq, k, m, w, max_entries, idx, scores, ws, ws_bytes, stream);
}

size_t lca_csa_index_topk_noalloc_max_bytes(void) { return index_noalloc_max_bytes(); }

int lca_csa_index_topk_noalloc(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                               const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int k, int m, int w,
                               int64_t max_entries, int32_t* idx, float* scores, int dtype, void* stream) {
  LCA_REQUIRE(idx != nullptr, LCA_ERR_INVALID_ARG, "csa_index_topk_noalloc: idx is NULL");
  // the argument checks of lca_csa_index_topk, with a workspace that always fits them
  static char ws_standin;
  int rc = check_index("csa_index_topk_noalloc", true, p, omega, ikey, csa_off, q_pos, B, Tq, H_I, d_I, k, m, w,
                       max_entries, &ws_standin, (size_t)-1, dtype);
  if (rc != LCA_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return finish(launch_index_topk_noalloc(p, omega, ikey, csa_off, q_pos, B, Tq, H_I, d_I, k, m, w, max_entries, idx,
                                          scores, dtype, st),
                st, "csa_index_topk_noalloc");
}

static int check_attn(const char* what, const void* q, const void* kv, const void* off, const void* lst,
                      int B, int Tq, int H, int D, float scale, float eps, int n_split, const void* o,
                      const float* lse, int dtype) {
  LCA_REQUIRE(q && kv && off && lst && o && lse, LCA_ERR_INVALID_ARG, "%s: a required pointer is NULL", what);
  LCA_REQUIRE(B >= 1 && Tq >= 1 && H >= 1, LCA_ERR_INVALID_ARG, "%s: B=%d Tq=%d H=%d", what, B, Tq, H);
  LCA_REQUIRE((int64_t)B * Tq <= 65535 && H <= 65535, LCA_ERR_UNSUPPORTED, "%s: B*Tq and H must be <= 65535",
              what);
  LCA_REQUIRE(valid_head_dim(D), LCA_ERR_UNSUPPORTED, "%s: D=%d not in {64,128,256,512}", what, D);
  LCA_REQUIRE(n_split >= 1 && n_split <= 256, LCA_ERR_INVALID_ARG, "%s: n_split=%d not in [1,256]", what,
              n_split);
  LCA_REQUIRE(std::isfinite(scale) && scale > 0.f, LCA_ERR_INVALID_ARG, "%s: scale must be finite and > 0", what);
  LCA_REQUIRE(std::isfinite(eps) && eps >= 0.f, LCA_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", what);
  LCA_REQUIRE(valid_dtype(dtype), LCA_ERR_INVALID_ARG, "%s: dtype=%d", what, dtype);
  return LCA_OK;
}

int lca_csa_sparse_attn(const void* q, const void* kv_csa, const int64_t* csa_off, const int32_t* idx, int B,
                        int Tq, int H, int D, int k, float scale, float eps, int n_split, float* o_part,
                        float* lse, int dtype, void* stream) {
  int rc = check_attn("csa_sparse_attn", q, kv_csa, csa_off, idx, B, Tq, H, D, scale, eps, n_split, o_part, lse,
                      dtype);
  if (rc != LCA_OK) return rc;
  LCA_REQUIRE(k >= 1 && k <= 65536, LCA_ERR_INVALID_ARG, "csa_sparse_attn: k=%d", k);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const lca_attn_source src = make_source(LCA_SRC_GATHER, kv_csa, csa_off, idx, k, 1, 1, 0, n_split, o_part, lse);
  // q_pos is not read by the gathered source
  return finish(launch_attention(&src, 1, q, nullptr, B, Tq, H, D, scale, eps, dtype, st), st, "csa_sparse_attn");
}

int lca_hca_attn(const void* q, const void* kv_hca, const int64_t* hca_off, const int32_t* q_pos, int B, int Tq,
                 int H, int D, int m2, int w2, int64_t max_entries, float scale, float eps, int n_split,
                 float* o_part, float* lse, int dtype, void* stream) {
  int rc = check_attn("hca_attn", q, kv_hca, hca_off, q_pos, B, Tq, H, D, scale, eps, n_split, o_part, lse, dtype);
  if (rc != LCA_OK) return rc;
  LCA_REQUIRE(m2 >= 1 && w2 >= 1, LCA_ERR_INVALID_ARG, "hca_attn: m2=%d w2=%d", m2, w2);
  LCA_REQUIRE(max_entries >= 0, LCA_ERR_INVALID_ARG, "hca_attn: max_entries < 0");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const lca_attn_source src = make_source(LCA_SRC_DENSE, kv_hca, hca_off, nullptr, 0, m2, w2, 0, n_split, o_part,
                                          lse);
  return finish(launch_attention(&src, 1, q, q_pos, B, Tq, H, D, scale, eps, dtype, st), st, "hca_attn");
}

int lca_swa_attn(const void* q, const void* x, const int64_t* tok_off, const int32_t* q_pos, int B, int Tq, int H,
                 int D, int W, float scale, float eps, float* o_part, float* lse, int dtype, void* stream) {
  int rc = check_attn("swa_attn", q, x, tok_off, q_pos, B, Tq, H, D, scale, eps, 1, o_part, lse, dtype);
  if (rc != LCA_OK) return rc;
  LCA_REQUIRE(W >= 1, LCA_ERR_INVALID_ARG, "swa_attn: W=%d must be >= 1", W);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const lca_attn_source src = make_source(LCA_SRC_WINDOW, x, tok_off, nullptr, 0, 1, 1, W, 1, o_part, lse);
  return finish(launch_attention(&src, 1, q, q_pos, B, Tq, H, D, scale, eps, dtype, st), st, "swa_attn");
}

}  // extern "C"

// Argument checks of lca_hybrid_attn (and of the attention part of
// lca_hybrid_attn_merge).
static int check_hybrid(const lca_attn_source* srcs, int n_src, const void* q, const int32_t* q_pos, int B, int Tq,
                        int H, int D, float scale, float eps, int dtype) {
  LCA_REQUIRE(srcs != nullptr && n_src >= 1 && n_src <= 3, LCA_ERR_INVALID_ARG,
              "hybrid_attn: n_src=%d not in [1,3] (or srcs is NULL)", n_src);
  bool need_pos = false;
  int n_topk = 0;
  for (int i = 0; i < n_src; ++i) {
    const lca_attn_source& x = srcs[i];
    LCA_REQUIRE(x.kind == LCA_SRC_DENSE || x.kind == LCA_SRC_GATHER || x.kind == LCA_SRC_WINDOW ||
                    x.kind == LCA_SRC_TOPK,
                LCA_ERR_INVALID_ARG, "hybrid_attn: source %d has kind %d", i, x.kind);
    if (x.kind == LCA_SRC_TOPK) {
      LCA_REQUIRE(++n_topk == 1, LCA_ERR_INVALID_ARG, "hybrid_attn: more than one TOPK source");
      LCA_REQUIRE(x.idx_out != nullptr, LCA_ERR_INVALID_ARG, "hybrid_attn: source %d: idx_out is NULL", i);
      LCA_REQUIRE(q_pos != nullptr, LCA_ERR_INVALID_ARG, "hybrid_attn: q_pos is NULL");
      int rc = check_index("hybrid_attn", false, nullptr, nullptr, nullptr, x.off, q_pos, B, Tq, 1, 8, x.k, x.m2,
                           x.w2, x.max_entries, x.ws, x.ws_bytes, LCA_BF16);
      if (rc != LCA_OK) return rc;
    }
    const void* lst = x.kind == LCA_SRC_GATHER ? (const void*)x.idx : x.kind == LCA_SRC_TOPK ? (const void*)x.idx_out : q;
    int rc = check_attn("hybrid_attn", q, x.kv, x.off, lst, B, Tq, H, D, scale, eps, x.n_split, x.o_part, x.lse,
                        dtype);
    if (rc != LCA_OK) return rc;
    if (x.kind == LCA_SRC_GATHER)
      LCA_REQUIRE(x.k >= 1 && x.k <= 65536, LCA_ERR_INVALID_ARG, "hybrid_attn: source %d: k=%d", i, x.k);
    if (x.kind == LCA_SRC_DENSE)
      LCA_REQUIRE(x.m2 >= 1 && x.w2 >= 1, LCA_ERR_INVALID_ARG, "hybrid_attn: source %d: m2=%d w2=%d", i, x.m2, x.w2);
    if (x.kind == LCA_SRC_WINDOW)
      LCA_REQUIRE(x.W >= 1, LCA_ERR_INVALID_ARG, "hybrid_attn: source %d: W=%d must be >= 1", i, x.W);
    LCA_REQUIRE(x.part >= 0 && x.part <= 2 && (x.part == 0 || (x.kind == LCA_SRC_DENSE && x.done_len != nullptr)),
                LCA_ERR_INVALID_ARG, "hybrid_attn: source %d: part=%d (dense sources only, with done_len)", i,
                x.part);
    LCA_REQUIRE(x.tiles_per_split >= 0, LCA_ERR_INVALID_ARG, "hybrid_attn: source %d: tiles_per_split=%d < 0", i,
                x.tiles_per_split);
    LCA_REQUIRE(x.o_half == 0 || x.o_half == 1, LCA_ERR_INVALID_ARG, "hybrid_attn: source %d: o_half=%d", i,
                x.o_half);
    LCA_REQUIRE(x.o_half == 0 || (dtype == LCA_BF16 && H % 16 == 0), LCA_ERR_UNSUPPORTED,
                "hybrid_attn: source %d: fp16 partials need dtype bf16 and H a multiple of 16", i);
    LCA_REQUIRE(x.rope_dims == srcs[0].rope_dims && x.rope_base == srcs[0].rope_base, LCA_ERR_INVALID_ARG,
                "hybrid_attn: source %d: every source of a call gives the same rope_dims and rope_base", i);
    if (x.tiles_per_split > 0 && (x.kind == LCA_SRC_GATHER || x.kind == LCA_SRC_TOPK))
      LCA_REQUIRE((int64_t)x.n_split * x.tiles_per_split * 32 >= x.k, LCA_ERR_INVALID_ARG,
                  "hybrid_attn: source %d: n_split=%d x tiles_per_split=%d x 32 < k=%d", i, x.n_split,
                  x.tiles_per_split, x.k);
    need_pos = need_pos || x.kind != LCA_SRC_GATHER;
  }
  LCA_REQUIRE(!need_pos || q_pos != nullptr, LCA_ERR_INVALID_ARG, "hybrid_attn: q_pos is NULL");
  const int rope = srcs[0].rope_dims;
  LCA_REQUIRE(rope >= 0 && rope <= D && rope % 2 == 0 &&
                  (rope == 0 || (q_pos != nullptr && std::isfinite(srcs[0].rope_base) && srcs[0].rope_base > 0.f)),
              LCA_ERR_INVALID_ARG,
              "hybrid_attn: rope_dims=%d must be even and <= D, with q_pos and a positive rope_base", rope);
  return LCA_OK;
}

extern "C" {

int lca_hybrid_attn(const lca_attn_source* srcs, int n_src, const void* q, const int32_t* q_pos, int B, int Tq,
                    int H, int D, float scale, float eps, int dtype, void* stream) {
  const int rc = check_hybrid(srcs, n_src, q, q_pos, B, Tq, H, D, scale, eps, dtype);
  if (rc != LCA_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return finish(launch_attention(srcs, n_src, q, q_pos, B, Tq, H, D, scale, eps, dtype, st), st, "hybrid_attn");
}

int lca_hybrid_attn_merge(const lca_attn_source* srcs, int n_src, const void* q, const int32_t* q_pos, int B,
                          int Tq, int H, int D, float scale, float eps, const float* sink, void* out, int dtype,
                          void* stream) {
  const int rc = check_hybrid(srcs, n_src, q, q_pos, B, Tq, H, D, scale, eps, dtype);
  if (rc != LCA_OK) return rc;
  LCA_REQUIRE(out != nullptr, LCA_ERR_INVALID_ARG, "hybrid_attn_merge: out is NULL");
  LCA_REQUIRE((int64_t)B * Tq <= 65535 && H <= 65535, LCA_ERR_UNSUPPORTED,
              "hybrid_attn_merge: B*Tq and H must be <= 65535");
  int slots = 0;
  for (int i = 0; i < n_src; ++i) slots += srcs[i].n_split;
  LCA_REQUIRE(slots <= 512, LCA_ERR_UNSUPPORTED, "hybrid_attn_merge: %d partial slots, at most 512", slots);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return finish(launch_attention_merge(srcs, n_src, q, q_pos, B, Tq, H, D, scale, eps, sink, out, dtype, st), st,
                "hybrid_attn_merge");
}

int lca_decode_front(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                     const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int k, int m, int w, int64_t max_entries,
                     const lca_compress_stream* idx_stream, const lca_compress_stream* kv_streams, int n_kv,
                     const int64_t* tok_off, const int64_t* done_len, float eps, float* scores, void* ws,
                     size_t ws_bytes, const lca_attn_source* srcs, int n_src, const void* q, int H, int D,
                     float scale, int dtype, void* stream) {
  int rc = check_score_append(p, omega, ikey, csa_off, q_pos, B, Tq, H_I, d_I, k, m, w, max_entries, idx_stream,
                              kv_streams, n_kv, tok_off, done_len, eps, ws, ws_bytes, dtype);
  if (rc != LCA_OK) return rc;
  const int adt = dtype == LCA_F32 ? LCA_F32 : LCA_BF16;
  rc = check_hybrid(srcs, n_src, q, q_pos, B, Tq, H, D, scale, eps, adt);
  if (rc != LCA_OK) return rc;
  for (int i = 0; i < n_src; ++i) {
    const lca_attn_source& x = srcs[i];
    LCA_REQUIRE(x.kind == LCA_SRC_DENSE || x.kind == LCA_SRC_WINDOW, LCA_ERR_INVALID_ARG,
                "decode_front: source %d: only DENSE and WINDOW sources run beside the scores", i);
    // a source must not read entries the appends of the same launch write
    bool written = x.kv == idx_stream->out || (x.v && x.v == idx_stream->out);
    for (int j = 0; j < n_kv; ++j) written = written || x.kv == kv_streams[j].out || (x.v && x.v == kv_streams[j].out);
    LCA_REQUIRE(!written || (x.kind == LCA_SRC_DENSE && x.part == 1 && x.done_len == done_len), LCA_ERR_INVALID_ARG,
                "decode_front: source %d reads a cache the appends write: it must be DENSE with part = 1 and the "
                "call's done_len", i);
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return finish(launch_decode_front(p, omega, ikey, csa_off, q_pos, B, Tq, H_I, d_I, k, m, w, max_entries,
                                    idx_stream, kv_streams, n_kv, tok_off, done_len, eps, scores, ws, srcs, n_src, q,
                                    H, D, scale, dtype, st),
                st, "decode_front");
}

size_t lca_swa_merge_workspace(int n_rows, int H, int D) {
  if (n_rows < 1 || H < 1 || D < 1) return 0;
  const size_t o = ((size_t)n_rows * H * D * 4 + 255) & ~(size_t)255;
  return o + (size_t)n_rows * H * 4;
}

int lca_swa_merge(const void* q, const void* x, const int64_t* tok_off, const int32_t* q_pos, const float* sink,
                  const lca_partial* parts, int n_parts, int B, int Tq, int H, int D, int W, float scale, float eps,
                  void* out, void* ws, size_t ws_bytes, int dtype, void* stream) {
  LCA_REQUIRE(out != nullptr, LCA_ERR_INVALID_ARG, "swa_merge: out is NULL");
  LCA_REQUIRE(B >= 1 && Tq >= 1 && H >= 1, LCA_ERR_INVALID_ARG, "swa_merge: B=%d Tq=%d H=%d", B, Tq, H);
  LCA_REQUIRE((int64_t)B * Tq <= 65535 && H <= 65535, LCA_ERR_UNSUPPORTED, "swa_merge: B*Tq and H must be <= 65535");
  LCA_REQUIRE(valid_head_dim(D), LCA_ERR_UNSUPPORTED, "swa_merge: D=%d not in {64,128,256,512}", D);
  LCA_REQUIRE(valid_dtype(dtype), LCA_ERR_INVALID_ARG, "swa_merge: dtype=%d", dtype);
  LCA_REQUIRE(W >= 0, LCA_ERR_INVALID_ARG, "swa_merge: W=%d", W);
  LCA_REQUIRE(n_parts >= 0 && n_parts <= 7, LCA_ERR_UNSUPPORTED, "swa_merge: n_parts=%d not in [0,7]", n_parts);
  LCA_REQUIRE(n_parts == 0 || parts != nullptr, LCA_ERR_INVALID_ARG, "swa_merge: parts is NULL");
  int slots = W > 0 ? 1 : 0;
  for (int p = 0; p < n_parts; ++p) {
    LCA_REQUIRE(parts[p].o && parts[p].lse && parts[p].n_split >= 1 && parts[p].n_split <= 256 &&
                    (parts[p].o_half == 0 || parts[p].o_half == 1),
                LCA_ERR_INVALID_ARG, "swa_merge: part %d is invalid", p);
    slots += parts[p].n_split;
  }
  LCA_REQUIRE(slots <= 512, LCA_ERR_UNSUPPORTED, "swa_merge: %d partial slots, at most 512", slots);
  LCA_REQUIRE(std::isfinite(scale) && scale > 0.f, LCA_ERR_INVALID_ARG, "swa_merge: scale");
  LCA_REQUIRE(std::isfinite(eps) && eps >= 0.f, LCA_ERR_INVALID_ARG, "swa_merge: eps");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int rows = B * Tq;
  float* wo = nullptr;
  float* wl = nullptr;
  if (W > 0) {
    LCA_REQUIRE(q && x && tok_off && q_pos, LCA_ERR_INVALID_ARG, "swa_merge: q, x, tok_off and q_pos are required");
    const size_t need = lca_swa_merge_workspace(rows, H, D);
    LCA_REQUIRE(ws != nullptr && ws_bytes >= need, LCA_ERR_WORKSPACE,
                "swa_merge: workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    wo = reinterpret_cast<float*>(ws);
    wl = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + (((size_t)rows * H * D * 4 + 255) & ~(size_t)255));
    const lca_attn_source src = make_source(LCA_SRC_WINDOW, x, tok_off, nullptr, 0, 1, 1, W, 1, wo, wl);
    int rc = launch_attention(&src, 1, q, q_pos, B, Tq, H, D, scale, eps, dtype, st);
    if (rc != LCA_OK) return finish(rc, st, "swa_merge(window)");
  }
  LCA_REQUIRE(n_parts > 0 || W > 0 || sink != nullptr, LCA_ERR_INVALID_ARG, "swa_merge: nothing to merge");
  return finish(launch_merge(parts, n_parts, wo, wl, sink, rows, H, D, out, dtype, st), st, "swa_merge");
}

}  // extern "C"
