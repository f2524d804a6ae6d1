/*
 * lca.h -- C-ABI of the MI355X (gfx950) hybrid compressed attention library.
 *
 * DeepSeek-V4's attention stack, as the pages describe it ("Why DeepSeek V4
 * Stands Apart", Core Architectural Innovations; "DeepSeek-V4" spec sheet,
 * Design overview, Core block, Inference efficiency): the KV stream is
 * compressed into overlapping entries every 4 tokens (CSA) and into one entry
 * per 128 tokens (HCA); a lightning indexer scores the CSA entries and each
 * query attends to its top-k of them, to every HCA entry, to the most recent
 * 128 raw tokens and to an attention sink.  One KV head is shared by all query
 * heads, and a compressed entry is both key and value.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer owned by the caller; the library
 *   never allocates, frees or keeps a buffer, and keeps no state between calls
 *   except in the caller's workspace (see lca_csa_index_topk).
 * - `stream` is a hipStream_t passed as void*; every call is asynchronous on it.
 * - Every argument is validated on the host before anything is launched; a
 *   failed call launches nothing and returns a negative code.  Device faults
 *   surface at the caller's next synchronisation (HIP semantics); with the
 *   environment variable LCA_SYNC=1 every call synchronises its stream and
 *   reports a device error as LCA_ERR_HIP.
 * - Element type: LCA_BF16 (bfloat16 storage, fp32 arithmetic) or LCA_F32.
 *   Indexer head weights, sink logits, partial outputs and scores are fp32.
 * - Sequences are packed: rows of sequence b live at [off[b], off[b+1]) of a
 *   tensor; offsets are device int64 arrays of length B+1.
 * - Row-major layouts; "[a, b, c]" lists dimensions from slowest to fastest.
 * - Thread safety: concurrent calls are safe when they use different
 *   workspaces and outputs.  One case is slower, not wrong, under concurrent
 *   work: the sparse blocks of a TOPK source (lca_hybrid_attn) that filter
 *   the scores themselves wait for each other, which assumes that the whole
 *   launch is resident at once (the library checks this against the
 *   device's occupancy when nothing else runs).  Work on other streams or in
 *   other processes can keep some of those blocks from starting; a waiting
 *   block gives up after 100 us and selects the exact top-k from the row's
 *   scores alone, so the output is the same.
 */
#ifndef LCA_H_
#define LCA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum lca_status {
  LCA_OK = 0,
  LCA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, inconsistent sizes */
  LCA_ERR_UNSUPPORTED = -2, /* a shape or type the library has no kernel for */
  LCA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  LCA_ERR_HIP = -4          /* the HIP runtime reported an error */
};

enum lca_dtype { LCA_F32 = 0, LCA_BF16 = 1, LCA_BF16_FP8KEY = 2, LCA_BF16_MXFP4KEY = 3 };
/* LCA_BF16_FP8KEY (index-score calls only): indexer queries p bf16, weights
 * fp32, and the indexer-key cache in fp8 rows: d_I OCP E4M3 bytes (1 sign, 4
 * exponent bits of bias 7, 3 mantissa bits; largest finite 448), then the
 * row's fp32 scale s, then 4 zero bytes -- d_I + 8 bytes per entry.  The row
 * stands for s * q (s = max|key| / 448, q rounded to nearest even); its score
 * is the bf16 formula on that row ("DeepSeek-V4", Inference efficiency: the
 * indexer's query-key path in low precision).  Written by lca_kv_compress
 * with out_key = 1.
 * LCA_BF16_MXFP4KEY (index-score calls only): as LCA_BF16_FP8KEY with MXFP4
 * key rows (OCP microscaling FP4): d_I/2 bytes of E2M1 elements (1 sign, 2
 * exponent bits of bias 1, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6; two per
 * byte, the even channel in the low nibble), then one E8M0 scale byte per 32
 * channels (2**(byte - 127)), zero-padded -- d_I/2 + 8 bytes per entry.  A
 * block's scale is 2**(floor(log2 amax) - 2), its elements value / scale
 * rounded to nearest even and clamped to +-6 (scale 2**-127 and zero elements
 * for an all-zero block).  Written by lca_kv_compress with out_key = 2. */

/* Static text for a status code. */
const char* lca_strerror(int status);
/* Text describing the last failure on the calling thread ("" if none). */
const char* lca_last_error(void);
/* Library version, major*10000 + minor*100 + patch. */
int lca_version(void);

/* ------------------------------------------------------------------------
 * KV compression
 *
 * "Why DeepSeek V4 Stands Apart", Core Architectural Innovations (CSA
 * compresses KV entries 4x; HCA compresses 128:1) and "DeepSeek-V4", Design
 * overview (every 4 tokens into two overlapping streams; m' = 128) and
 * Provenance 17 (RMSNorm on compressed KV entries).
 *
 * Entry j of sequence b pools the raw rows t = j*m .. j*m+w-1 of that
 * sequence:  e[j, c] = sum_t softmax_t(z[t, c]) * src[t, c]  (softmax over the
 * w tokens of the window, separately per channel c; with per_channel = 0 the
 * same logit z[t] serves every channel).  With rmsnorm = 1 the entry is then
 * divided by sqrt(mean_c e[j, c]^2 + eps).  The result is rounded to the
 * storage type.  Only complete windows exist: a sequence of L tokens has
 * N(L) = L < w ? 0 : (L - w) / m + 1 entries.  CSA: m = 4, w = 8; HCA:
 * m = w = 128.
 *
 * A call writes, for every sequence b and every stream, the entries
 * N(done_len[b]) .. N(L_b) - 1, L_b = tok_off[b+1] - tok_off[b]: all of them
 * for a cache build (done_len = NULL), the ones the newest tokens complete for
 * a decode step or a prefill chunk.  Only the raw rows inside those windows
 * are read.
 * ---------------------------------------------------------------------- */
typedef struct lca_compress_stream {
  const void* src;        /* [T, C] raw rows, packed by tok_off                      */
  const void* logits;     /* [T, C] if per_channel else [T]; same element type       */
  void* out;              /* [sum_b N(L_b), C] entries, packed by ent_off             */
  const int64_t* ent_off; /* device [B+1]: first row of sequence b in `out`           */
  int32_t C;              /* channels: multiple of 8 (bf16) / 4 (f32), at most 1024   */
  int32_t m;              /* stride (>= 1)                                            */
  int32_t w;              /* window (>= m)                                            */
  int32_t per_channel;    /* 1: logits [T, C]; 0: logits [T]                          */
  int32_t rmsnorm;        /* 1: RMS-normalise each entry over its C channels          */
  int32_t max_entries;    /* host bound on entries written per sequence (>= 0)        */
  int32_t out_key;        /* 0: rows of the input type; 1: fp8 key rows (see          */
                          /* LCA_BF16_FP8KEY), 2: MXFP4 key rows (LCA_BF16_MXFP4KEY):  */
                          /* bf16 input, C <= 512 (MXFP4: C in {32,64,128,256}),       */
                          /* w = m or w = 2m <= 16                                      */
  int32_t rope_dims;      /* 0, or the rotary embedding of each entry ("DeepSeek-V4",  */
                          /* Core block and Provenance 16: partial RoPE on the last   */
                          /* 64 dims): after the norm, the last rope_dims channels    */
                          /* (even, <= C) turn pair by pair, pair p (channels         */
                          /* C - rope_dims + 2p, +1) as a complex number times        */
                          /* exp(i pos theta_p), theta_p = rope_base^(-2p/rope_dims), */
                          /* pos = j*m + w - 1 (the last token of entry j's window);  */
                          /* rows of the input type only (out_key = 0)                 */
  float rope_base;        /* > 0 when rope_dims > 0 (10000 in the benchmark layers)    */
  const void* src2;       /* NULL, or the dual-stream form ("DeepSeek-V4", Design      */
                          /* overview: every 4 tokens into two overlapping streams;  */
                          /* Core block: overlapping dual compressed streams): the   */
                          /* last m tokens of each window are read from src2 and     */
                          /* logits2 (same shapes and type as src and logits), the   */
                          /* first m from src and logits, one softmax over all w     */
                          /* logits of a channel.  Needs w = 2m <= 16                */
  const void* logits2;    /* with src2: the second-half logits; else NULL            */
} lca_compress_stream;

/* Compress up to 4 streams in one launch.
 *   streams  host array of n_streams (1..4) descriptors
 *   tok_off  device int64 [B+1]
 *   done_len device int64 [B] or NULL (0 for every sequence)
 *   eps      RMSNorm epsilon (1e-6 in the benchmark workloads)
 * Returns LCA_OK or an error; the caller must make ent_off leave room for
 * N(L_b) rows per sequence and max_entries >= N(L_b) - N(done_len[b]). */
int lca_kv_compress(const lca_compress_stream* streams, int n_streams, const int64_t* tok_off,
                    const int64_t* done_len, int B, float eps, int dtype, void* stream);

/* ------------------------------------------------------------------------
 * Lightning-indexer scores and exact top-k over the CSA entries
 *
 * "DeepSeek-V4", Design overview and Inference efficiency (V3.2's lightning
 * indexer on the compressed entries); "Why DeepSeek V4 Stands Apart", Core
 * Architectural Innovations (top-1024 for Pro, top-512 for Flash).
 *
 * For query row r = b*Tq + t at position i = q_pos[b*Tq + t], entry j of
 * sequence b is a candidate iff its window ends at or before i
 * (j*m + w - 1 <= i).  Its score is
 *     s_j = sum_h omega[r, h] * max(0, p[r, h, :] . ikey[csa_off[b] + j, :]).
 * idx[r, 0..k) receives the k candidates of largest score, ties broken toward
 * the smaller j, as local entry indices (0-based within the sequence).  When a
 * query has fewer than k candidates all are selected and the rest of its row is
 * -1.  A row lists its entries in ascending index order when the query has
 * at most 262144 candidates (a deterministic order beyond that); it is not a
 * ranking.
 *
 *   p        [B*Tq, H_I, d_I]  indexer queries (dtype)
 *   omega    [B*Tq, H_I]       fp32 head weights
 *   ikey     [sum_b N, d_I]    indexer keys (dtype), packed by csa_off; with
 *            dtype LCA_BF16_FP8KEY / LCA_BF16_MXFP4KEY: [sum_b N] key rows of
 *            d_I + 8 / d_I/2 + 8 bytes (p bf16), scored as the rows they stand for, for
 *            d_I in {32, 64, 128, 256} and H_I <= 16 (LCA_ERR_UNSUPPORTED
 *            otherwise)
 *   q_pos    device int32 [B*Tq]
 *   max_entries  host bound on the candidates of any query (>= 1)
 *   scores   optional fp32 [B*Tq, max_entries] output of every candidate's
 *            score (entry j at column j); NULL to keep them in the workspace.
 *            With NULL, many rows per sequence (Tq >= 32, max_entries <=
 *            98304), k <= 512, H_I in {1, 2, 4} and d_I a multiple of 32
 *            up to 256 (a prefill chunk), the scores and the selection run
 *            in one launch that stores no score: each block streams the
 *            keys for 16 query rows and keeps per row, in LDS, a bounded
 *            list of the entries at or above a running threshold (a key
 *            with at least k listed keys at or above it)
 *   ws       device workspace of at least lca_csa_index_topk_workspace()
 *            bytes.  It must be ZERO-FILLED before its first use; after
 *            that each score call and the selection that must follow it
 *            (lca_csa_topk_select, or a TOPK source of lca_hybrid_attn)
 *            leave it ready for the next score call.  Calls that share a
 *            workspace must be ordered on one stream.
 * Supported: H_I * d_I <= 1024, d_I multiple of 8, k in [1, 4096],
 * entries per sequence < 2^24. */
size_t lca_csa_index_topk_workspace(int n_rows, int64_t max_entries, int k);
int lca_csa_index_topk(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                       const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int k, int m, int w,
                       int64_t max_entries, int32_t* idx, float* scores, void* ws, size_t ws_bytes,
                       int dtype, void* stream);

/* lca_csa_index_topk for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments without the workspace, which is a static device array of the
 * library (lca_csa_index_topk_noalloc_max_bytes() bytes, 8 MiB; each GPU the
 * library runs on holds its own copy until the process ends).  The call
 * allocates nothing.  A call whose workspace (lca_csa_index_topk_workspace of
 * the same arguments) exceeds that size returns LCA_ERR_WORKSPACE and
 * launches nothing -- except a call that the streaming selection takes
 * (scores NULL and the many-row bounds of lca_csa_index_topk), which needs
 * no workspace at all and runs at any size.  Every call on a GPU shares that GPU's array: calls that
 * overlap on one GPU (on different streams, or from different threads) race
 * and must not be issued.  The array keeps the last call's contents; the
 * first call on a device, and every call whose (B*Tq, max_entries, k)
 * differs from the previous call's on that device, first clears it with a
 * fill kernel on `stream`.  Results are those of lca_csa_index_topk. */
size_t lca_csa_index_topk_noalloc_max_bytes(void);
int lca_csa_index_topk_noalloc(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                               const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int k, int m, int w,
                               int64_t max_entries, int32_t* idx, float* scores, int dtype, void* stream);

/* The two halves of lca_csa_index_topk, same arguments and workspace:
 * lca_csa_index_score writes the scores and the selection histogram into the
 * workspace (and the scores into `scores` when it is not NULL);
 * lca_csa_topk_select (two launches: filter, then the exact selection) must
 * follow on the same stream with the same arguments and workspace (and the
 * same `scores` pointer), or a TOPK source of lca_hybrid_attn in its place. */
int lca_csa_index_score(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                        const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int k, int m, int w,
                        int64_t max_entries, float* scores, void* ws, size_t ws_bytes, int dtype,
                        void* stream);
/* Compression + indexer scores for one decode step: the compression of the entries the newest
 * tokens complete and the index scores, in one launch.  Equivalent to
 *     lca_kv_compress({idx_stream} + kv_streams, tok_off, done_len, ...)
 *     lca_csa_index_score(..., Tq, ...)
 * with Tq query rows per sequence (1, or a few -- such as a step that checks
 * a drafted token beside the main one, the multi-token prediction of
 * "DeepSeek-V4", Inference efficiency): the new indexer keys are pooled,
 * stored and scored (for every row that sees them) by blocks of their own,
 * the entries that existed before by the scoring blocks, and the kv_streams
 * (entries only the attention reads, such as the CSA and HCA KV entries) by
 * further blocks of the same launch; no block reads what another writes.
 * With 2 <= Tq <= 4 and Tq * H_I <= 16 the rows of a sequence share one read
 * of the keys (one matrix-core product scores them all).  The caches written
 * are bit-identical to lca_kv_compress's for bf16 rows; fp8 key rows
 * (dtype LCA_BF16_FP8KEY / LCA_BF16_MXFP4KEY, idx_stream->out_key = 1 / 2)
 * agree up to the fp32
 * rounding of the pooling (the stored scale shows it); the new entries'
 * scores agree within rounding order.  Falls back to those two calls where the fused
 * launch does not apply: fp32, d_I not in {32, 64, 128, 256}, an indexer
 * window other than w = m or w = 2m <= 16, kv streams wider than 512 bf16
 * channels, Tq > 1 outside the shared-read bounds above.
 *   idx_stream  the indexer-key stream: out == ikey, ent_off == csa_off,
 *               C == d_I, same m and w
 *   kv_streams  0 to 4 further streams sharing one vector width
 *   tok_off, done_len  as lca_kv_compress (done_len required)
 * Other arguments, and the workspace, as lca_csa_index_score's. */
int lca_csa_index_score_append(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                               const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int k, int m, int w,
                               int64_t max_entries, const lca_compress_stream* idx_stream,
                               const lca_compress_stream* kv_streams, int n_kv, const int64_t* tok_off,
                               const int64_t* done_len, float eps, float* scores, void* ws, size_t ws_bytes,
                               int dtype, void* stream);

int lca_csa_topk_select(const int64_t* csa_off, const int32_t* q_pos, int B, int Tq, int k, int m, int w,
                        int64_t max_entries, int32_t* idx, const float* scores, void* ws, size_t ws_bytes,
                        void* stream);

/* ------------------------------------------------------------------------
 * Attention partials (sparse CSA, dense HCA)
 *
 * Shared-KV multi-query attention ("DeepSeek-V4", Inference efficiency): all H
 * query heads attend to the same keys, and a compressed entry is key and value.
 * Every query head is RMS-normalised over D in the kernel (RMSNorm on queries,
 * "DeepSeek-V4" Provenance 17) and rounded to the storage type; logits are
 * scale * qhat . key.  The key list of a query is cut into n_split parts; part
 * s writes the softmax-normalised output and natural-log log-sum-exp of its
 * keys:
 *     o_part[s, r, h, :]  fp32, [n_split, B*Tq, H, D]  (fp16 for an
 *                         lca_hybrid_attn source with o_half)
 *     lse[s, r, h]        fp32, [n_split, B*Tq, H]
 * An empty part writes o = 0 and lse = -inf.  lca_swa_merge combines parts.
 * Supported: D in {64, 128, 256, 512}; any H (H a multiple of 16 uses the
 * matrix cores for bf16); 1 <= n_split <= 256.
 * ---------------------------------------------------------------------- */

/* Sparse attention over the selected CSA entries ("Why DeepSeek V4
 * Stands Apart", Core Architectural Innovations: attention over the top-k
 * compressed entries of each query).
 *   q       [B*Tq, H, D] raw queries (dtype)
 *   kv_csa  [sum_b N, D] compressed, normalised KV entries, packed by csa_off
 *   idx     int32 [B*Tq, k] local entry indices, -1 = unused slot           */
int lca_csa_sparse_attn(const void* q, const void* kv_csa, const int64_t* csa_off, const int32_t* idx,
                        int B, int Tq, int H, int D, int k, float scale, float eps, int n_split,
                        float* o_part, float* lse, int dtype, void* stream);

/* Dense attention over every visible HCA entry ("Why DeepSeek V4 Stands
 * Apart", Core Architectural Innovations: dense attention over the 128:1
 * compressed representation).  Entry j of sequence b is visible to the query
 * at position i iff j*m2 + w2 - 1 <= i.
 *   kv_hca  [sum_b N2, D] packed by hca_off; q_pos device int32 [B*Tq]
 *   max_entries  host bound on the visible entries of any query            */
int lca_hca_attn(const void* q, const void* kv_hca, const int64_t* hca_off, const int32_t* q_pos,
                 int B, int Tq, int H, int D, int m2, int w2, int64_t max_entries, float scale, float eps,
                 int n_split, float* o_part, float* lse, int dtype, void* stream);

/* ------------------------------------------------------------------------
 * Sliding window + sink + merge
 *
 * "Why DeepSeek V4 Stands Apart", Core Architectural Innovations (window of
 * the most recent 128 tokens); "DeepSeek-V4", Core block (attention sinks).
 * For query row r at position i of sequence b: attends to the raw rows
 * max(0, i-W+1) .. i of x (each RMS-normalised over D and rounded to the
 * storage type on load), then combines that window with every partial of
 * `parts` and the sink logit sink[h] (zero value; NULL = no sink) into one
 * softmax:
 *     lse = log(sum_p exp(lse_p) + exp(sink))
 *     out = sum_p exp(lse_p - lse) * o_p        (rounded to dtype)
 * W = 0 skips the window.  ws: at least lca_swa_merge_workspace() bytes.
 *   x       [T, D] raw KV rows, packed by tok_off (device int64 [B+1])
 *   out     [B*Tq, H, D] (dtype)
 * ---------------------------------------------------------------------- */
/* The window branch alone, as a partial: attends to the raw rows
 * max(0, i-W+1) .. i of x (RMS-normalised over D and rounded to the storage
 * type on load) and writes o_part [1, B*Tq, H, D] and lse [1, B*Tq, H] (one
 * split), so that it can run beside the other branches and be merged by
 * lca_swa_merge with W = 0.  W >= 1. */
int lca_swa_attn(const void* q, const void* x, const int64_t* tok_off, const int32_t* q_pos, int B, int Tq, int H,
                 int D, int W, float scale, float eps, float* o_part, float* lse, int dtype, void* stream);

/* All three attention branches of a step in one launch.  Each source writes
 * its own partials, exactly as the single-branch calls above would with the
 * same n_split, so lca_swa_merge (W = 0) combines them:
 *   LCA_SRC_DENSE   HCA entries of kv (packed by off) visible under m2, w2
 *                   (as lca_hca_attn)
 *   LCA_SRC_GATHER  the k entries of kv listed in idx [B*Tq, k], -1 = unused
 *                   (as lca_csa_sparse_attn)
 *   LCA_SRC_WINDOW  raw rows max(0, i-W+1) .. i of kv packed by off, each
 *                   RMS-normalised over D on load (as lca_swa_attn, any
 *                   n_split)
 *   LCA_SRC_TOPK    the top-k selection and the sparse branch in one: after
 *                   a score call (same stream, workspace ws, scores, k slots,
 *                   m2 = m, w2 = w (the CSA entries' stride and window),
 *                   max_entries, kv's offsets as csa_off), it stands for
 *                   lca_csa_topk_select into idx_out followed by a GATHER
 *                   source over idx_out: idx_out receives exactly what
 *                   lca_csa_topk_select would write (ascending order when a
 *                   row has at most 262144 candidates).  On the bf16
 *                   matrix-core path with max_entries <= 262144 every block
 *                   of the sparse branch runs the exact selection itself;
 *                   when the whole launch fits the device at once, those
 *                   blocks also filter the scores (one launch in all; a
 *                   block whose wait for the others gives up, see the
 *                   thread-safety note above, selects from the scores
 *                   alone), else a filter launch comes first.  Elsewhere the selection's
 *                   own launches come first.  At most one TOPK source per
 *                   call.
 * The sources share q [B*Tq, H, D], q_pos (device int32 [B*Tq]; read by the
 * DENSE and WINDOW sources), scale and eps.  One launch costs one kernel
 * start and lets the branches' blocks share the machine.  The bf16
 * matrix-core path (H a multiple of 16) stages at most 2048 gathered slots
 * per split: ceil(ceil(k/32) / n_split) * 32 <= 2048, else
 * LCA_ERR_UNSUPPORTED.  1 <= n_src <= 3; 1 <= n_split <= 256 per source. */
enum { LCA_SRC_DENSE = 0, LCA_SRC_GATHER = 1, LCA_SRC_WINDOW = 2, LCA_SRC_TOPK = 3 };

typedef struct lca_attn_source {
  int32_t kind;          /* LCA_SRC_* */
  const void* kv;        /* cache rows (DENSE, GATHER) or raw rows (WINDOW), dtype */
  const int64_t* off;    /* device int64 [B+1]: row offsets of kv per sequence */
  const int32_t* idx;    /* GATHER: device int32 [B*Tq, k]; else NULL */
  int32_t k;             /* GATHER slots per row */
  int32_t m2, w2;        /* DENSE: stride and window of the entries */
  int32_t W;             /* WINDOW: window length, >= 1 */
  int32_t n_split;       /* key-range parts */
  void* o_part;          /* fp32 [n_split, B*Tq, H, D]; fp16 with o_half */
  float* lse;            /* fp32 [n_split, B*Tq, H] */
  /* LCA_SRC_TOPK only (zero otherwise): */
  void* ws;              /* index workspace of the preceding score call */
  size_t ws_bytes;
  int64_t max_entries;   /* as passed to the score call */
  const float* scores;   /* the score call's scores output, or NULL */
  int32_t* idx_out;      /* device int32 [B*Tq, k]: receives the selection */
  /* optional (zero: off) */
  const int64_t* done_len;  /* DENSE with part != 0: device int64 [B] */
  int32_t part;             /* DENSE: 0 every visible entry; 1 only the visible entries
                               complete within the first done_len[b] tokens of sequence b;
                               2 only the visible entries completed after them.  Parts
                               1 and 2 together give exactly the entries of part 0 (a
                               decode step can attend to the entries that existed before
                               it while it appends the new ones, and to those after) */
  int32_t rope_dims;        /* 0, or the rotary embedding of the call (every source of
                               a call gives the same rope_dims and rope_base): the
                               normalised query of row r turns by q_pos[r] (q_pos
                               required), a WINDOW source's raw row at token t by t
                               (DENSE and GATHER entries are stored turned, see
                               lca_compress_stream), and each partial o_part turns by
                               -q_pos[r] ("DeepSeek-V4", Provenance 16: -i RoPE on
                               the outputs; the merge of turned partials is the turned
                               merge).  Last rope_dims dims of each head, even, <= D */
  float rope_base;
  int32_t tiles_per_split;  /* > 0: split s takes the row's keys [32 t s, 32 t (s + 1)),
                               t = tiles_per_split, whatever the other rows of the call
                               (the last split also takes any keys beyond; for GATHER and
                               TOPK n_split * 32 t >= k is required); 0: each row's keys
                               are cut into n_split equal parts.  Applies to calls with
                               few query rows per sequence; the row-tiled path (many
                               rows per sequence) always cuts a block's key range into
                               n_split parts */
  const void* v;            /* NULL: the keys are the values (one shared KV vector per
                               entry, "DeepSeek-V4", Inference efficiency: shared-KV
                               MQA).  Else the values, rows laid out as kv (same dtype,
                               D wide, same row for the same key): a DENSE / GATHER /
                               TOPK source's value entries, a WINDOW source's raw value
                               tokens (RMS-normalised and turned on load as the window
                               keys).  Such calls take the per-row kernel, also with
                               many query rows per sequence */
  int32_t o_half;           /* 0: o_part is fp32.  1: o_part holds IEEE fp16 values (lse
                               stays fp32), half the bytes the partials write and the
                               merge reads.  A partial is a convex combination of value
                               rows, so each of its elements is at most the largest
                               value element in magnitude: the caller guarantees that
                               bound is below 65504 (RMS-normalised entries and window
                               tokens are at most sqrt(D) times their norm weight);
                               fp16 then rounds each element to 2^-11 of itself, a
                               quarter of a bf16 output's rounding.  Only calls of
                               dtype LCA_BF16 with H a multiple of 16 and few query rows
                               per sequence (the matrix-core kernel that writes one
                               partial per block); elsewhere LCA_ERR_UNSUPPORTED */
} lca_attn_source;

int lca_hybrid_attn(const lca_attn_source* srcs, int n_src, const void* q, const int32_t* q_pos, int B, int Tq,
                    int H, int D, float scale, float eps, int dtype, void* stream);

typedef struct lca_partial {
  const void* o;    /* [n_split, B*Tq, H, D], fp32 (fp16 with o_half) */
  const float* lse; /* [n_split, B*Tq, H]    */
  int32_t n_split;
  int32_t o_half;   /* 1: o holds fp16 values, as an lca_attn_source with o_half wrote them */
} lca_partial;

size_t lca_swa_merge_workspace(int n_rows, int H, int D);
int lca_swa_merge(const void* q, const void* x, const int64_t* tok_off, const int32_t* q_pos,
                  const float* sink, const lca_partial* parts, int n_parts, int B, int Tq, int H, int D,
                  int W, float scale, float eps, void* out, void* ws, size_t ws_bytes, int dtype,
                  void* stream);

/* ------------------------------------------------------------------------
 * Attention and merge in one call
 *
 * The output of lca_hybrid_attn(srcs, ...) followed by lca_swa_merge(q,
 * NULL, NULL, NULL, sink, the sources' partials in source order, n_src, B,
 * Tq, H, D, W = 0, ...): one softmax over every key the sources give and the
 * sink ("Why DeepSeek V4 Stands Apart", Core Architectural Innovations;
 * "DeepSeek-V4", Core block (attention sinks)), out [B*Tq, H, D] of dtype.
 * On the row-tiled path (bf16, D = 512, many query rows per sequence) with
 * one split per source it is one launch: every block attends to all sources
 * for its rows under one online softmax and writes out, and the sources'
 * o_part / lse are not written.  Otherwise it is the attention launch(es)
 * and then the merge launch, the partials written as by lca_hybrid_attn.
 * The two ways agree within rounding (one softmax over the union against a
 * log-sum-exp merge of per-source parts).
 *   sink  device fp32 [H] or NULL (no sink)
 * Errors as lca_hybrid_attn; LCA_ERR_INVALID_ARG for a NULL out;
 * LCA_ERR_UNSUPPORTED beyond 512 partial slots in all or B*Tq or H above
 * 65535. */
int lca_hybrid_attn_merge(const lca_attn_source* srcs, int n_src, const void* q, const int32_t* q_pos, int B,
                          int Tq, int H, int D, float scale, float eps, const float* sink, void* out, int dtype,
                          void* stream);

/* ------------------------------------------------------------------------
 * Decode front: the work of a decode step that does not depend on the top-k
 * selection, in one launch
 *
 * The same as
 *     lca_csa_index_score_append(p, ..., dtype, stream)
 *     lca_hybrid_attn(srcs, n_src, q, q_pos, B, Tq, H, D, scale, eps,
 *                     dtype == LCA_F32 ? LCA_F32 : LCA_BF16, stream)
 * with every argument as in those calls: the appends of the entries the
 * newest tokens complete, the lightning-indexer scores (a TOPK source of
 * lca_hybrid_attn or lca_csa_topk_select follows), and the attention over
 * DENSE and WINDOW sources ("DeepSeek-V4", Design overview and Inference
 * efficiency; "Why DeepSeek V4 Stands Apart", Core Architectural
 * Innovations: the dense attention over the 128:1 entries and the window do
 * not depend on the indexer).  On the bf16 matrix-core path (D = 512, H a
 * multiple of 16, d_I = 64, one query row per sequence or a few sharing a
 * score block, no rotary embedding, no separate values) it is one launch
 * whose attention blocks run beside the score blocks; elsewhere the two
 * launches above.
 *   srcs  DENSE or WINDOW sources only (LCA_ERR_INVALID_ARG otherwise); a
 *         source over a cache that the appends write must be DENSE with
 *         part = 1 and this call's done_len (the entries that existed
 *         before the step), so that no block reads what another writes.
 *         The entries the step completes are attended by a later call (a
 *         DENSE source with part = 2).
 * Errors as the two calls. */
int lca_decode_front(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                     const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int k, int m, int w, int64_t max_entries,
                     const lca_compress_stream* idx_stream, const lca_compress_stream* kv_streams, int n_kv,
                     const int64_t* tok_off, const int64_t* done_len, float eps, float* scores, void* ws,
                     size_t ws_bytes, const lca_attn_source* srcs, int n_src, const void* q, int H, int D,
                     float scale, int dtype, void* stream);

/* ------------------------------------------------------------------------
 * Diagnostics (process-wide settings read by every later launch; not meant
 * for production use, and not synchronised with launches in flight)
 *
 * lca_diag_trace: when buf is not NULL, every later launch of the few-row
 * attention kernel (lca_hybrid_attn / lca_csa_sparse_attn / lca_hca_attn /
 * lca_swa_attn with few query rows per sequence, and the attention blocks of
 * lca_decode_front) writes, for each block b with 16*(b+1) <= n_words, 16
 * uint64 words at buf[16*b]: the 100 MHz constant
 * clock (s_memrealtime) at 0 block start, 1 top-k filter done, 2 wait done,
 * 3 selection done, 4 prologue done, 5 key loop done, 6 partial stored (0 for
 * phases the block does not have), and word 7 = source kind (LCA_SRC_*) |
 * wait gave up << 2 | fallback selection << 3 | owns top-k slots << 4 | XCC
 * id << 8 | query row << 12 (20 bits) | the wave's HW_ID register << 32;
 * words 8-15 stamp the top-k steps of a TOPK block (8 histogram summed,
 * 9 threshold found, 10 list space reserved, 11 own share counted, 12 lists
 * loaded, 13 second-level threshold found, 14 cut found, 15 filter loads
 * issued; 0 if not reached).  buf is a device pointer the caller keeps alive while
 * tracing; NULL turns tracing off.
 *
 * lca_diag_topk_wait: the top-k wait inside the attention launch (a TOPK
 * source whose sparse blocks filter the scores themselves) waits until the
 * row's sparse blocks have all filtered their shares, for at most max_ticks
 * of the 100 MHz clock (0: the default, 10000 = 100 us).  A block whose wait
 * gives up selects the exact top-k from the row's scores alone, so the
 * result does not change, only the time.  extra_shares > 0 makes every wait
 * expect that many shares more than exist, so that every wait gives up (for
 * testing that path); 0 restores normal operation.
 * ---------------------------------------------------------------------- */
int lca_diag_trace(uint64_t* buf, int64_t n_words);
int lca_diag_topk_wait(int extra_shares, int64_t max_ticks);

#ifdef __cplusplus
}
#endif
#endif /* LCA_H_ */
