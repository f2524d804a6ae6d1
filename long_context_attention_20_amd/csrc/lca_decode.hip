// The decode front launch: the work of a decode step that does not depend on
// the top-k selection, in one grid -- the appends of the entries the new
// tokens complete, the lightning-indexer scores of every visible CSA entry
// (with the selection's histogram), and the attention over the HCA entries
// that existed before the step and over the sliding window.  The selection,
// the sparse attention over the selected CSA entries (and over an HCA entry
// the step completes) follow in the next launch.
//
// Pages: "DeepSeek-V4", Design overview (CSA entries scored by the lightning
// indexer, HCA entries attended densely), Inference efficiency (shared-KV MQA);
// "Why DeepSeek V4 Stands Apart", Core Architectural Innovations (top-k over
// the compressed entries, dense attention over the 128:1 entries, a
// 128-token window).
//
// The score stream (the indexer keys, most of a step's bytes) is bound by HBM
// bandwidth, the HCA attention by latency: in one grid the attention blocks
// overlap the score blocks' memory traffic instead of waiting for it, and the
// launch that follows holds only the selection and the sparse attention.
// Blocks, in dispatch order: the attention blocks (attn_block, XCD-aware
// numbering), the compression blocks of the KV streams, one append block per
// sequence (pools, stores and scores the new indexer keys), the score blocks.
// No block reads what another block of the grid writes: the HCA source of
// the grid covers only entries complete before the step (part 1), the score
// blocks only entries that existed before it.
#include "lca_attn_block.h"
#include "lca_score.h"

namespace lca {

struct FrontParams {
  IndexParams ip;
  AppendIdx ap;
  CompressParams cp;
  int n_attn;  // attention blocks (first in the grid; a multiple of 8)
};

template <int KS, int TQ, int KF>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_front(AttnParams a,
                                                                                                      FrontParams f) {
  __shared__ __attribute__((aligned(16))) char lds_raw[AttnLds<512, false>::kBytes];
  warm_kernargs<sizeof(AttnParams) + sizeof(FrontParams)>();
  const int bid = blockIdx.x;
  if (bid < f.n_attn) {
    attn_block<512, false, 1>(a, bid, lds_raw);
    return;
  }
  const int blk = bid - f.n_attn;
  if (blk < f.ap.ncb) {
    // 8-token batches and no prefetching keep the register budget
    compress_block<BF16, 1, 8, false>(f.cp, blk, reinterpret_cast<float*>(lds_raw));
  } else if (blk < f.ap.ncb + f.ap.B) {
    append_and_score<KF>(f.ip, f.ap, blk - f.ap.ncb);
  } else {
    const int sb = blk - f.ap.ncb - f.ap.B;
    const int b = sb / f.ap.nsx, cx = sb % f.ap.nsx;
    const int64_t lim = n_windows(f.ap.done_len[b], f.ip.m, f.ip.w);
    if constexpr (TQ == 1)
      score_chunk_mfma<KS, KF>(f.ip, b, cx, lim, reinterpret_cast<uint32_t*>(lds_raw));
    else
      score_chunk_multi<KS, TQ, KF>(f.ip, b, cx, lim, reinterpret_cast<uint32_t*>(lds_raw));
  }
}

int setup_attention_front(const lca_attn_source* srcs, int n_src, const void* q, const int32_t* q_pos, int B, int Tq,
                          int H, int D, float scale, float eps, AttnParams* a, int64_t* nblk);
bool index_append_fusable(int dtype, int Tq, int HI, int dI, int m, int w, const lca_compress_stream* idx_stream);
int setup_front_scores(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                       const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w, int64_t maxN,
                       const lca_compress_stream* idx_stream, const lca_compress_stream* kv_streams, int n_kv,
                       const int64_t* tok_off, const int64_t* done_len, float eps, float* scores, void* ws, int dtype,
                       int threads, int64_t chunk, IndexParams* a, AppendIdx* ap, CompressParams* cp,
                       size_t* lds, int64_t* blocks);
int launch_index_score_append(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                              const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w, int64_t maxN,
                              const lca_compress_stream* idx_stream, const lca_compress_stream* kv_streams, int n_kv,
                              const int64_t* tok_off, const int64_t* done_len, float eps, float* scores, void* ws,
                              int dtype, hipStream_t stream);
int launch_attention(const lca_attn_source* srcs, int n_src, const void* q, const int32_t* q_pos, int B, int Tq,
                     int H, int D, float scale, float eps, int dtype, hipStream_t stream);

// Entries per score block of the front launch: about one block per compute
// unit the attention blocks leave free (at least 1024: one pass of 8 waves x
// 8 tiles x 16 entries), at most 16384.
static int64_t front_chunk(int64_t maxN, int rows, int64_t n_attn, int cus) {
  const int64_t free_cus = cus - n_attn > cus / 4 ? cus - n_attn : cus / 4;
  int64_t want = (maxN * rows + free_cus - 1) / free_cus;
  int64_t chunk = 1024;
  while (chunk < want && chunk < 16384) chunk *= 2;
  return chunk;
}

int launch_decode_front(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                        const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w, int64_t maxN,
                        const lca_compress_stream* idx_stream, const lca_compress_stream* kv_streams, int n_kv,
                        const int64_t* tok_off, const int64_t* done_len, float eps, float* scores, void* ws,
                        const lca_attn_source* srcs, int n_src, const void* q, int H, int D, float scale, int dtype,
                        hipStream_t stream) {
  const int kf = dtype == LCA_BF16_FP8KEY ? 1 : dtype == LCA_BF16_MXFP4KEY ? 2 : 0;
  AttnParams a;
  int64_t n_attn = 0;
  int rc = LCA_ERR_UNSUPPORTED;
  // (the front's attention blocks are the plain ones: a rotary embedding or
  // separate values take the two launches)
  bool plain = true;
  for (int i = 0; i < n_src; ++i) plain = plain && srcs[i].rope_dims == 0 && srcs[i].v == nullptr;
  if (plain && dI == 64 && index_append_fusable(dtype, Tq, HI, dI, m, w, idx_stream) && (dtype != LCA_F32))
    rc = setup_attention_front(srcs, n_src, q, q_pos, B, Tq, H, D, scale, eps, &a, &n_attn);
  FrontParams f{};
  size_t lds = 0;
  int64_t nfront = 0;
  if (rc == LCA_OK) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    const int64_t chunk = front_chunk(maxN, B * Tq, n_attn, cus);
    rc = setup_front_scores(p, omega, ikey, csa_off, q_pos, B, Tq, HI, dI, k, m, w, maxN, idx_stream, kv_streams, n_kv,
                            tok_off, done_len, eps, scores, ws, dtype, kAttnThreads, chunk, &f.ip, &f.ap, &f.cp, &lds,
                            &nfront);
    if (rc == LCA_OK && lds > AttnLds<512, false>::kBytes) rc = LCA_ERR_UNSUPPORTED;
    if (rc == LCA_OK && n_attn + nfront > 0x7FFFFFFF) rc = LCA_ERR_UNSUPPORTED;
  }
  if (rc != LCA_OK) {
    // the two launches the front stands for
    rc = launch_index_score_append(p, omega, ikey, csa_off, q_pos, B, Tq, HI, dI, k, m, w, maxN, idx_stream,
                                   kv_streams, n_kv, tok_off, done_len, eps, scores, ws, dtype, stream);
    if (rc != LCA_OK) return rc;
    return launch_attention(srcs, n_src, q, q_pos, B, Tq, H, D, scale, eps, dtype == LCA_F32 ? LCA_F32 : LCA_BF16,
                            stream);
  }
  f.n_attn = (int)n_attn;
  const int tq = Tq == 1 ? 1 : Tq == 2 ? 2 : 4;
  dim3 grid((unsigned)(n_attn + nfront));
#define LCA_FRONT(TQv)                                                                                          \
  if (kf == 1) hipLaunchKernelGGL((decode_front<2, TQv, 1>), grid, dim3(kAttnThreads), 0, stream, a, f);      \
  else if (kf == 2) hipLaunchKernelGGL((decode_front<2, TQv, 2>), grid, dim3(kAttnThreads), 0, stream, a, f); \
  else hipLaunchKernelGGL((decode_front<2, TQv, 0>), grid, dim3(kAttnThreads), 0, stream, a, f);
  switch (tq) {
    case 1: LCA_FRONT(1) break;
    case 2: LCA_FRONT(2) break;
    default: LCA_FRONT(4) break;
  }
#undef LCA_FRONT
  return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
}

}  // namespace lca
