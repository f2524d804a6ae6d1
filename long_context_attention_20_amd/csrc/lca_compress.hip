// a1. KV compression: softmax-weighted window pooling (+ RMSNorm) of raw rows.
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
#include "lca_common.h"

namespace lca {

constexpr int kCompressThreads = 512;
constexpr int kRunEntries = 16;  // entries per row group in small-window mode
constexpr int kPrefetchM = 4;    // small-window strides up to this use the prefetching walk

struct CompressStreamDev {
  const void* src;
  const void* logits;
  void* out;
  const int64_t* ent_off;
  int C, m, w, per_channel, rmsnorm, max_entries;
  int G;        // lanes per row
  int NV;       // 16-byte vectors per lane per row
  int small;    // 1: small-window run mode
  int epb;      // entries per block
  int bps;      // blocks per sequence
  int block_begin;
};

struct CompressParams {
  CompressStreamDev s[4];
  int n;
  const int64_t* tok_off;
  const int64_t* done_len;
  int B;
  float eps;
};

template <int VE>
struct PoolState {
  float mx[VE], se[VE], sn[VE];
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int e = 0; e < VE; ++e) { mx[e] = -INFINITY; se[e] = 0.f; sn[e] = 0.f; }
  }
  // add one token: logits z, values x
  __device__ __forceinline__ void add(const float* z, const float* x) {
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      float d = z[e] - mx[e];
      bool big = d > 0.f;
      float f = __expf(-fabsf(d));
      se[e] = big ? fmaf(se[e], f, 1.f) : se[e] + f;
      sn[e] = big ? fmaf(sn[e], f, x[e]) : fmaf(f, x[e], sn[e]);
      mx[e] = big ? z[e] : mx[e];
    }
  }
  __device__ __forceinline__ void merge(const PoolState& o) {
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      float M = fmaxf(mx[e], o.mx[e]);
      float fa = (mx[e] == -INFINITY) ? 0.f : __expf(mx[e] - M);
      float fb = (o.mx[e] == -INFINITY) ? 0.f : __expf(o.mx[e] - M);
      se[e] = se[e] * fa + o.se[e] * fb;
      sn[e] = sn[e] * fa + o.sn[e] * fb;
      mx[e] = M;
    }
  }
};

template <typename ET, int NV>
struct RowCtx {
  static constexpr int VE = ET::kVec;
  const char* src;
  const char* lg;
  int64_t row_bytes;
  int per_channel;
  int ch0[NV];  // first channel of each vector of this lane

  __device__ __forceinline__ void load(int64_t t, float (&x)[NV][VE], float (&z)[NV][VE]) const {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      uint4 xv = ldg16(src, t * row_bytes + (int64_t)ch0[v] * ET::kBytes);
      ET::unpack(xv, x[v]);
      if (per_channel) {
        uint4 zv = ldg16(lg, t * row_bytes + (int64_t)ch0[v] * ET::kBytes);
        ET::unpack(zv, z[v]);
      } else {
        float zs = ET::load1(lg, t);
#pragma unroll
        for (int e = 0; e < VE; ++e) z[v][e] = zs;
      }
    }
  }
};

template <typename ET, int NV>
__device__ __forceinline__ void finish_entry(const CompressStreamDev& s, float eps, int G,
                                             PoolState<ET::kVec> (&st)[NV], const int (&ch0)[NV],
                                             int64_t out_row, bool active) {
  constexpr int VE = ET::kVec;
  float e[NV][VE];
  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int k = 0; k < VE; ++k) {
      e[v][k] = st[v].sn[k] / st[v].se[k];
      ss = fmaf(e[v][k], e[v][k], ss);
    }
  if (s.rmsnorm) {
    ss = wave_sum(ss, G);  // all lanes of the row group take part
    float inv = 1.0f / sqrtf(ss / (float)s.C + eps);
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int k = 0; k < VE; ++k) e[v][k] *= inv;
  }
  if (active) {
    const int64_t rb = (int64_t)s.C * ET::kBytes;
#pragma unroll
    for (int v = 0; v < NV; ++v) stg16(s.out, out_row * rb + (int64_t)ch0[v] * ET::kBytes, ET::pack(e[v]));
  }
}

template <typename ET, int NV>
__device__ void compress_small(const CompressStreamDev& s, const CompressParams& P, int b, int cb) {
  constexpr int VE = ET::kVec;
  const int G = s.G;
  const int rg = threadIdx.x / G;
  const int li = threadIdx.x % G;
  const int64_t t0 = P.tok_off[b];
  const int64_t L = P.tok_off[b + 1] - t0;
  const int64_t done = P.done_len ? P.done_len[b] : 0;
  const int64_t n_lo = n_windows(done, s.m, s.w);
  const int64_t n_hi = n_windows(L, s.m, s.w);
  const int64_t j0 = n_lo + (int64_t)cb * s.epb + (int64_t)rg * kRunEntries;
  const int64_t j1 = min(j0 + kRunEntries, n_hi);
  // every lane of a row group agrees on j0/j1, so the shuffles in the norm
  // stay inside active groups
  if (j0 >= j1) return;

  RowCtx<ET, NV> rc;
  rc.row_bytes = (int64_t)s.C * ET::kBytes;
  rc.src = reinterpret_cast<const char*>(s.src) + t0 * rc.row_bytes;
  rc.per_channel = s.per_channel;
  rc.lg = reinterpret_cast<const char*>(s.logits) + (s.per_channel ? t0 * rc.row_bytes : t0 * ET::kBytes);
#pragma unroll
  for (int v = 0; v < NV; ++v) rc.ch0[v] = (v * G + li) * VE;
  const int64_t ent_base = s.ent_off[b];
  const int m = s.m;
  const bool two = (s.w == 2 * s.m);

  PoolState<VE> prev[NV], cur[NV];
  if constexpr (NV == 1) if (m <= kPrefetchM) {
    // raw rows of the next segment are requested before the current one is
    // pooled, so a run costs one memory round trip per segment at most and a
    // single entry (decode append) costs one in all
    struct Raw {
      uint4 x[kPrefetchM][NV], z[kPrefetchM][NV];
      float zs[kPrefetchM];
    };
    auto fetch = [&](int64_t q, Raw& r) {
      const int64_t tb = q * m;
#pragma unroll
      for (int t = 0; t < kPrefetchM; ++t) {
        if (t < m) {
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            r.x[t][v] = ldg16(rc.src, (tb + t) * rc.row_bytes + (int64_t)rc.ch0[v] * ET::kBytes);
            if (rc.per_channel) r.z[t][v] = ldg16(rc.lg, (tb + t) * rc.row_bytes + (int64_t)rc.ch0[v] * ET::kBytes);
          }
          if (!rc.per_channel) r.zs[t] = ET::load1(rc.lg, tb + t);
        }
      }
    };
    auto pool = [&](const Raw& r, PoolState<VE>(&st)[NV]) {
#pragma unroll
      for (int v = 0; v < NV; ++v) st[v].reset();
#pragma unroll
      for (int t = 0; t < kPrefetchM; ++t) {
        if (t < m) {
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            float x[VE], z[VE];
            ET::unpack(r.x[t][v], x);
            if (rc.per_channel) {
              ET::unpack(r.z[t][v], z);
            } else {
#pragma unroll
              for (int e = 0; e < VE; ++e) z[e] = r.zs[t];
            }
            st[v].add(z, x);
          }
        }
      }
    };
    const int64_t q_end = two ? j1 + 1 : j1;  // last segment + 1
    Raw ra, rb;
    fetch(j0, ra);
    if (j0 + 1 < q_end) fetch(j0 + 1, rb);
    if (two) {
      pool(ra, prev);
      ra = rb;
      if (j0 + 2 < q_end) fetch(j0 + 2, rb);
    }
    // ra holds the segment pooled next, rb the one after it (in flight)
    for (int64_t j = j0; j < j1; ++j) {
      pool(ra, cur);
      ra = rb;
      const int64_t nq = (two ? j + 1 : j) + 2;
      if (nq < q_end) fetch(nq, rb);
      if (two) {
        PoolState<VE> e[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) { e[v] = prev[v]; e[v].merge(cur[v]); prev[v] = cur[v]; }
        finish_entry<ET, NV>(s, P.eps, G, e, rc.ch0, ent_base + j, true);
      } else {
        finish_entry<ET, NV>(s, P.eps, G, cur, rc.ch0, ent_base + j, true);
      }
    }
    return;
  }
  auto segment = [&](int64_t q, PoolState<VE>(&st)[NV]) {
#pragma unroll
    for (int v = 0; v < NV; ++v) st[v].reset();
    const int64_t tb = q * m;
    int t = 0;
    for (; t + 4 <= m; t += 4) {
      float x[4][NV][VE], z[4][NV][VE];
#pragma unroll
      for (int u = 0; u < 4; ++u) rc.load(tb + t + u, x[u], z[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < NV; ++v) st[v].add(z[u][v], x[u][v]);
    }
    for (; t < m; ++t) {
      float x[NV][VE], z[NV][VE];
      rc.load(tb + t, x, z);
#pragma unroll
      for (int v = 0; v < NV; ++v) st[v].add(z[v], x[v]);
    }
  };

  if (two) segment(j0, prev);
  for (int64_t j = j0; j < j1; ++j) {
    if (two) {
      segment(j + 1, cur);
      PoolState<VE> e[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) { e[v] = prev[v]; e[v].merge(cur[v]); prev[v] = cur[v]; }
      finish_entry<ET, NV>(s, P.eps, G, e, rc.ch0, ent_base + j, true);
    } else {
      segment(j, cur);
      finish_entry<ET, NV>(s, P.eps, G, cur, rc.ch0, ent_base + j, true);
    }
  }
}

template <typename ET, int NV>
__device__ void compress_large(const CompressStreamDev& s, const CompressParams& P, int b, int cb,
                               float* lds) {
  constexpr int VE = ET::kVec;
  const int G = s.G;
  const int RG = kCompressThreads / G;
  const int rg = threadIdx.x / G;
  const int li = threadIdx.x % G;
  const int64_t t0 = P.tok_off[b];
  const int64_t L = P.tok_off[b + 1] - t0;
  const int64_t done = P.done_len ? P.done_len[b] : 0;
  const int64_t j = n_windows(done, s.m, s.w) + cb;  // one entry per block
  if (j >= n_windows(L, s.m, s.w)) return;           // uniform over the block

  RowCtx<ET, NV> rc;
  rc.row_bytes = (int64_t)s.C * ET::kBytes;
  rc.src = reinterpret_cast<const char*>(s.src) + t0 * rc.row_bytes;
  rc.per_channel = s.per_channel;
  rc.lg = reinterpret_cast<const char*>(s.logits) + (s.per_channel ? t0 * rc.row_bytes : t0 * ET::kBytes);
#pragma unroll
  for (int v = 0; v < NV; ++v) rc.ch0[v] = (v * G + li) * VE;

  const int chunk = (s.w + RG - 1) / RG;
  const int tb = rg * chunk;
  const int te = min(s.w, tb + chunk);
  PoolState<VE> st[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) st[v].reset();
  const int64_t base = j * s.m;
  int t = tb;
  for (; t + 8 <= te; t += 8) {
    float x[8][NV][VE], z[8][NV][VE];
#pragma unroll
    for (int u = 0; u < 8; ++u) rc.load(base + t + u, x[u], z[u]);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int v = 0; v < NV; ++v) st[v].add(z[u][v], x[u][v]);
  }
  for (; t < te; ++t) {
    float x[NV][VE], z[NV][VE];
    rc.load(base + t, x, z);
#pragma unroll
    for (int v = 0; v < NV; ++v) st[v].add(z[v], x[v]);
  }
  // partial states -> LDS [RG][3][C]
  const int C = s.C;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const int c = rc.ch0[v] + e;
      lds[(rg * 3 + 0) * C + c] = st[v].mx[e];
      lds[(rg * 3 + 1) * C + c] = st[v].se[e];
      lds[(rg * 3 + 2) * C + c] = st[v].sn[e];
    }
  __syncthreads();
  // combine the row groups' states, one channel per thread; pooled value -> LDS
  float* pooled = lds + RG * 3 * C;
  for (int c = threadIdx.x; c < C; c += kCompressThreads) {
    float M = -INFINITY;
    for (int r = 0; r < RG; ++r) M = fmaxf(M, lds[(r * 3 + 0) * C + c]);
    float se = 0.f, sn = 0.f;
    for (int r = 0; r < RG; ++r) {
      const float m = lds[(r * 3 + 0) * C + c];
      const float f = m == -INFINITY ? 0.f : __expf(m - M);
      se = fmaf(lds[(r * 3 + 1) * C + c], f, se);
      sn = fmaf(lds[(r * 3 + 2) * C + c], f, sn);
    }
    pooled[c] = sn / se;
  }
  __syncthreads();
  if (rg != 0) return;
  float e[NV][VE];
  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int k = 0; k < VE; ++k) {
      e[v][k] = pooled[rc.ch0[v] + k];
      ss = fmaf(e[v][k], e[v][k], ss);
    }
  if (s.rmsnorm) {
    ss = wave_sum(ss, G);
    const float inv = 1.0f / sqrtf(ss / (float)C + P.eps);
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int k = 0; k < VE; ++k) e[v][k] *= inv;
  }
  const int64_t rb = (int64_t)C * ET::kBytes;
  const int64_t out_row = s.ent_off[b] + j;
#pragma unroll
  for (int v = 0; v < NV; ++v) stg16(s.out, out_row * rb + (int64_t)rc.ch0[v] * ET::kBytes, ET::pack(e[v]));
}

template <typename ET, int NV>
__global__ __launch_bounds__(kCompressThreads) void compress_kernel(CompressParams P) {
  extern __shared__ float lds[];
  int si = 0;
  for (int k = 1; k < P.n; ++k)
    if ((int)blockIdx.x >= P.s[k].block_begin) si = k;
  const CompressStreamDev& s = P.s[si];
  if (s.bps <= 0) return;
  const int local = blockIdx.x - s.block_begin;
  const int b = local / s.bps;
  const int cb = local % s.bps;
  if (b >= P.B) return;
  if (s.small)
    compress_small<ET, NV>(s, P, b, cb);
  else
    compress_large<ET, NV>(s, P, b, cb, lds);
}

// Host side ------------------------------------------------------------------

int launch_compress(const lca_compress_stream* streams, int n, const int64_t* tok_off, const int64_t* done_len,
                    int B, float eps, int dtype, hipStream_t stream) {
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
    const int lanes = in.C / VE;
    d.G = lanes < 64 ? lanes : 64;
    d.NV = lanes < 64 ? 1 : lanes / 64;
    if (nv_all < 0) nv_all = d.NV;
    if (d.NV != nv_all) {
      set_error("kv_compress: all streams of one call need the same C/vector ratio (C=%d)", in.C);
      return LCA_ERR_UNSUPPORTED;
    }
    d.small = (in.w <= 16 && (in.w == in.m || in.w == 2 * in.m)) ? 1 : 0;
    const int RG = kCompressThreads / d.G;
    d.epb = d.small ? RG * kRunEntries : 1;
    d.bps = in.max_entries <= 0 ? 0 : (in.max_entries + d.epb - 1) / d.epb;
    d.block_begin = (int)blocks;
    blocks += (int64_t)d.bps * B;
    if (!d.small) {
      size_t need = ((size_t)RG * 3 + 1) * in.C * sizeof(float);
      if (need > lds_bytes) lds_bytes = need;
    }
  }
  if (blocks == 0) return LCA_OK;
  if (blocks > 0x7FFFFFFF) {
    set_error("kv_compress: grid too large (%lld blocks)", (long long)blocks);
    return LCA_ERR_UNSUPPORTED;
  }
  if (lds_bytes > 64 * 1024) {
    set_error("kv_compress: channel count needs %zu bytes of LDS", lds_bytes);
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
