// KV compression: softmax-weighted window pooling (+ RMSNorm) of raw rows.
//
// Pages: "Why DeepSeek V4 Stands Apart", Core Architectural Innovations (CSA
// compresses KV entries 4x, HCA 128:1); "DeepSeek-V4", Design overview (every
// 4 tokens into two overlapping streams; m' = 128) and Provenance 17 (RMSNorm
// on compressed KV entries).  Design input from the same pages'
// Infrastructure section: the fused compressor reads its inputs once and
// writes its outputs once -- here every raw row is read once per stream and
// every entry is written once.
//
// Layout: one 16-byte vector per lane per row chunk; a "row group" of G lanes
// (G = C / 8 for bf16, C / 4 for f32, capped at 64) covers one row of C
// channels with fully coalesced loads.
//
// Small windows (w <= 16, w == m or w == 2m, i.e. CSA): a row group walks a
// run of consecutive entries; the statistics of each m-token segment are
// computed once and an entry combines one segment (w == m) or two adjacent
// ones (w == 2m), so each raw row is read exactly once per run.
//
// Large windows (HCA): one entry per block; the w tokens are split over the
// block's row groups, whose partial statistics meet in LDS.
//
// Per channel the pool keeps an online softmax state (max z, sum e^(z-max),
// sum e^(z-max) * x) with one exponential per token.
#include "lca_compress.h"

namespace lca {

constexpr int kCompressThreads = 512;

template <typename ET, int NV>
__global__ __launch_bounds__(kCompressThreads) void compress_kernel(CompressParams P) {
  warm_kernargs<sizeof(CompressParams)>();
  extern __shared__ float lds[];
  compress_block<ET, NV>(P, (int)blockIdx.x, lds);
}

// Host side ------------------------------------------------------------------

int setup_compress(const lca_compress_stream* streams, int n, const int64_t* tok_off, const int64_t* done_len,
                   int B, float eps, int dtype, int threads, CompressParams* Pout, int64_t* blocks_out,
                   size_t* lds_out, int* nv_out) {
  CompressParams P{};
  P.n = n;
  P.tok_off = tok_off;
  P.done_len = done_len;
  P.B = B;
  P.eps = eps;
  const int VE = dtype == LCA_BF16 ? 8 : 4;
  int nv_all = -1;
  int64_t blocks = 0;
  size_t lds_bytes = 0;
  for (int k = 0; k < n; ++k) {
    const lca_compress_stream& in = streams[k];
    CompressStreamDev& d = P.s[k];
    d.src = in.src; d.logits = in.logits; d.out = in.out; d.ent_off = in.ent_off;
    d.C = in.C; d.m = in.m; d.w = in.w; d.per_channel = in.per_channel; d.rmsnorm = in.rmsnorm;
    d.max_entries = in.max_entries;
    d.key = in.out_key;
    d.rope = make_rope_tab(in.rope_dims, in.rope_base);
    d.src2 = in.src2;
    d.logits2 = in.logits2;
    const int lanes = in.C / VE;
    d.G = lanes < 64 ? lanes : 64;
    d.NV = lanes < 64 ? 1 : lanes / 64;
    if (nv_all < 0) nv_all = d.NV;
    if (d.NV != nv_all) {
      set_error("kv_compress: all streams of one call need the same C/vector ratio (C=%d)", in.C);
      return LCA_ERR_UNSUPPORTED;
    }
    d.small = (in.w <= 16 && (in.w == in.m || in.w == 2 * in.m)) ? 1 : 0;
    const int RG = threads / d.G;
    d.epb = d.small ? RG * kRunEntries : 1;
    d.bps = in.max_entries <= 0 ? 0 : (in.max_entries + d.epb - 1) / d.epb;
    d.block_begin = (int)blocks;
    blocks += (int64_t)d.bps * B;
    if (!d.small) {
      const int VG = kLargeLayoutThreads / d.G;
      size_t need = ((size_t)VG * 3 + 1) * in.C * sizeof(float);
      if (need > lds_bytes) lds_bytes = need;
    }
  }
  if (lds_bytes > 64 * 1024) {
    set_error("kv_compress: channel count needs %zu bytes of LDS", lds_bytes);
    return LCA_ERR_UNSUPPORTED;
  }
  *Pout = P;
  *blocks_out = blocks;
  *lds_out = lds_bytes;
  *nv_out = nv_all;
  return LCA_OK;
}

int launch_compress(const lca_compress_stream* streams, int n, const int64_t* tok_off, const int64_t* done_len,
                    int B, float eps, int dtype, hipStream_t stream) {
  CompressParams P;
  int64_t blocks = 0;
  size_t lds_bytes = 0;
  int nv_all = 0;
  const int rc = setup_compress(streams, n, tok_off, done_len, B, eps, dtype, kCompressThreads, &P, &blocks,
                                &lds_bytes, &nv_all);
  if (rc != LCA_OK) return rc;
  if (blocks == 0) return LCA_OK;
  if (blocks > 0x7FFFFFFF) {
    set_error("kv_compress: grid too large (%lld blocks)", (long long)blocks);
    return LCA_ERR_UNSUPPORTED;
  }
  dim3 grid((unsigned)blocks), block(kCompressThreads);
#define LCA_COMPRESS_CASE(ETy, NVv)                                                                  \
  hipLaunchKernelGGL((compress_kernel<ETy, NVv>), grid, block, lds_bytes, stream, P);
  if (dtype == LCA_BF16) {
    switch (nv_all) {
      case 1: LCA_COMPRESS_CASE(BF16, 1); break;
      case 2: LCA_COMPRESS_CASE(BF16, 2); break;
      default: set_error("kv_compress: C too large"); return LCA_ERR_UNSUPPORTED;
    }
  } else {
    switch (nv_all) {
      case 1: LCA_COMPRESS_CASE(F32, 1); break;
      case 2: LCA_COMPRESS_CASE(F32, 2); break;
      case 4: LCA_COMPRESS_CASE(F32, 4); break;
      default: set_error("kv_compress: C too large"); return LCA_ERR_UNSUPPORTED;
    }
  }
#undef LCA_COMPRESS_CASE
  return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
}

}  // namespace lca
