// KV compression device code: the pooling state, the small-window run
// walk and the large-window block walk (see lca_compress.hip for the method
// and its sources).  Shared by the compression kernel and by the index-score
// launch that appends entries with extra blocks.  The walks take the block
// size from blockDim.x; the host setup (setup_compress) sizes the grid for it.
#pragma once
#include "lca_common.h"

namespace lca {

// The large-window walk partitions a window as a block of this many threads
// would, whatever the launch's block size.
constexpr int kLargeLayoutThreads = 512;


constexpr int kRunEntries = 16;  // entries per row group in small-window mode
constexpr int kPrefetchM = 4;    // small-window strides up to this use the prefetching walk

struct CompressStreamDev {
  const void* src;
  const void* logits;
  void* out;
  const int64_t* ent_off;
  int C, m, w, per_channel, rmsnorm, max_entries;
  RopeTab rope;  // rotated channels at the end of an entry (rope.dims, 0: none); entry j turns by j*m + w - 1
  const void* src2;     // dual-stream form (w = 2m): a window's last m tokens from src2 / logits2, or null
  const void* logits2;
  int key;      // key rows: 1 fp8 (C E4M3 bytes, fp32 scale, 4 zero bytes), 2 MXFP4 (C/2 bytes of E2M1
                // pairs, one E8M0 scale per 32 channels, zero pad to C/2 + 8); one lane group per row, NV = 1
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
      // (one fused multiply-add, written out: left to the compiler, the
      // contraction of a*b + c*d can differ between the kernels that inline
      // this, and so would the pooled entries)
      se[e] = fmaf(se[e], fa, o.se[e] * fb);
      sn[e] = fmaf(sn[e], fa, o.sn[e] * fb);
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

// Eight values as OCP E4M3 bytes of value / scale (round to nearest even,
// kept inside +-448); scale > 0.  Byte c of the result is value c.
__device__ __forceinline__ uint2 pack_fp8x8(const float (&x)[8], float scale) {
  float y[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) y[c] = fminf(fmaxf(x[c] / scale, -448.f), 448.f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}
// MXFP4: fp32 bits of the E2M1 value of nibble n (bit 3 the sign).
__device__ __forceinline__ uint32_t e2m1_bits(uint32_t n) {
  const uint32_t e = (n >> 1) & 3u, m = n & 1u;
  const uint32_t mag = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3F000000u : 0u);
  return mag | ((n & 8u) << 28);
}
// The E8M0 scale byte b as a float: 2**(b - 127).
__device__ __forceinline__ float e8m0_value(uint32_t b) {
  return __uint_as_float(b ? (b << 23) : 0x00400000u);
}
// Eight values of one 32-channel block as E2M1 nibbles (channel c at bits
// 4c): value * 2**-k rounded to nearest even on 0, .5, 1, 1.5, 2, 3, 4, 6
// (ties to the even mantissa) and clamped to 6; k = floor(log2 amax) - 2 of
// the block (its E8M0 byte k + 127 in *code), amax = 0: all zero, code 0.
__device__ __forceinline__ uint32_t pack_e2m1x8(const float (&x)[8], float amax, uint32_t* code) {
  if (!(amax > 0.f)) {
    *code = 0u;
    return 0u;
  }
  int ex;
  frexpf(amax, &ex);                       // amax = f * 2**ex, 0.5 <= f < 1
  const int k = max(-127, min(127, ex - 3));
  *code = (uint32_t)(k + 127);
  const float inv = ldexpf(1.0f, -k);      // exact
  uint32_t w = 0u;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float a = fminf(fabsf(x[c]) * inv, 6.0f);
    const uint32_t q = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                     : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
    w |= (q | (signbit(x[c]) ? 8u : 0u)) << (4 * c);
  }
  return w;
}
// The values of eight E2M1 nibbles of a block with scale s (exact in fp32).
__device__ __forceinline__ void unpack_e2m1x8(uint32_t w, float s, float (&x)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] = __uint_as_float(e2m1_bits((w >> (4 * c)) & 15u)) * s;
}
// One MXFP4 key row from its row group (G lanes x 8 channels, G >= 4): every
// lane packs its 8 channels against its block's amax (the 4 lanes of a
// 32-channel block), lane 0 writes the block scale bytes and the zero pad.
// Returns this lane's nibbles and block scale (for scoring the stored row).
__device__ __forceinline__ uint32_t store_mx_row(const float (&x)[8], int G, int li, char* row, int C, bool active,
                                                 float* scale) {
  float am = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) am = fmaxf(am, fabsf(x[c]));
  am = wave_max(am, 4);
  uint32_t code;
  const uint32_t w = pack_e2m1x8(x, am, &code);
  *scale = e8m0_value(code);
  // lane 0 of the row group gathers the block codes of lanes 0, 4, 8, ...
  const int base = ((int)threadIdx.x & 63) - li;
  uint32_t lo = 0u, hi = 0u;
  for (int b = 0; b < G / 4; ++b) {
    const uint32_t cb = (uint32_t)__shfl((int)code, base + 4 * b, 64);
    if (b < 4) lo |= cb << (8 * b); else hi |= cb << (8 * (b - 4));
  }
  if (active) {
    *reinterpret_cast<uint32_t*>(row + li * 4) = w;
    if (li == 0) *reinterpret_cast<uint2*>(row + C / 2) = make_uint2(lo, hi);
  }
  return w;
}

// The values of eight E4M3 bytes (exact in fp32).
__device__ __forceinline__ void unpack_fp8x8(uint2 v, float (&x)[8]) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, true);
  const f2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, false), d = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, true);
  x[0] = a.x; x[1] = a.y; x[2] = b.x; x[3] = b.y; x[4] = c.x; x[5] = c.y; x[6] = d.x; x[7] = d.y;
}

template <typename ET, int NV>
__device__ __forceinline__ void finish_entry(const CompressStreamDev& s, float eps, int G,
                                             PoolState<ET::kVec> (&st)[NV], const int (&ch0)[NV],
                                             int64_t out_row, bool active, int64_t j) {
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
  if (s.rope.dims)  // after the norm, before the rounding; entry j sits at the last token of its window
#pragma unroll
    for (int v = 0; v < NV; ++v) rope_turn<VE>(e[v], ch0[v], s.C, s.rope, (double)(j * s.m + s.w - 1));
  if (s.key == 2) {
    if constexpr (VE == 8) {
      char* row = reinterpret_cast<char*>(s.out) + out_row * (int64_t)(s.C / 2 + 8);
      float sc;
      store_mx_row(e[0], G, ch0[0] / 8, row, s.C, active, &sc);
    }
    return;
  }
  if (s.key == 1) {
    // one E4M3 byte per channel and the row's fp32 scale amax / 448 (the
    // row stands for scale * q; q = round-to-nearest-even of value / scale,
    // kept inside +-448).  bf16 input, C <= 512: one 8-channel vector per
    // lane (NV = 1)
    if constexpr (VE == 8) {
      float am = 0.f;
#pragma unroll
      for (int k = 0; k < VE; ++k) am = fmaxf(am, fabsf(e[0][k]));
      am = wave_max(am, G);  // all lanes of the row group take part
      const float sc = am / 448.0f;
      const uint2 q = sc > 0.f ? pack_fp8x8(e[0], sc) : make_uint2(0u, 0u);
      if (active) {
        char* row = reinterpret_cast<char*>(s.out) + out_row * (int64_t)(s.C + 8);
        *reinterpret_cast<uint2*>(row + ch0[0]) = q;
        if (ch0[0] == 0) *reinterpret_cast<uint2*>(row + s.C) = make_uint2(__float_as_uint(sc), 0u);
      }
    }
    return;
  }
  if (active) {
    const int64_t rb = (int64_t)s.C * ET::kBytes;
#pragma unroll
    for (int v = 0; v < NV; ++v) stg16(s.out, out_row * rb + (int64_t)ch0[v] * ET::kBytes, ET::pack(e[v]));
  }
}

template <typename ET, int NV, bool PF = true>
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
  if constexpr (NV == 1 && PF) if (m <= kPrefetchM && !s.src2) {
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
        finish_entry<ET, NV>(s, P.eps, G, e, rc.ch0, ent_base + j, true, j);
      } else {
        finish_entry<ET, NV>(s, P.eps, G, cur, rc.ch0, ent_base + j, true, j);
      }
    }
    return;
  }
  auto segment = [&](int64_t q, PoolState<VE>(&st)[NV], const RowCtx<ET, NV>& r) {
#pragma unroll
    for (int v = 0; v < NV; ++v) st[v].reset();
    const int64_t tb = q * m;
    int t = 0;
    for (; t + 4 <= m; t += 4) {
      float x[4][NV][VE], z[4][NV][VE];
#pragma unroll
      for (int u = 0; u < 4; ++u) r.load(tb + t + u, x[u], z[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < NV; ++v) st[v].add(z[u][v], x[u][v]);
    }
    for (; t < m; ++t) {
      float x[NV][VE], z[NV][VE];
      r.load(tb + t, x, z);
#pragma unroll
      for (int v = 0; v < NV; ++v) st[v].add(z[v], x[v]);
    }
  };

  if (s.src2) {
    // dual-stream form (w = 2m): entry j merges segment j of the first
    // stream with segment j + 1 of the second, so each segment is pooled
    // once per stream
    RowCtx<ET, NV> rc2 = rc;
    rc2.src = reinterpret_cast<const char*>(s.src2) + t0 * rc.row_bytes;
    rc2.lg = reinterpret_cast<const char*>(s.logits2) + (s.per_channel ? t0 * rc.row_bytes : t0 * ET::kBytes);
    for (int64_t j = j0; j < j1; ++j) {
      segment(j, prev, rc);
      segment(j + 1, cur, rc2);
#pragma unroll
      for (int v = 0; v < NV; ++v) prev[v].merge(cur[v]);
      finish_entry<ET, NV>(s, P.eps, G, prev, rc.ch0, ent_base + j, true, j);
    }
    return;
  }
  if (two) segment(j0, prev, rc);
  for (int64_t j = j0; j < j1; ++j) {
    if (two) {
      segment(j + 1, cur, rc);
      PoolState<VE> e[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) { e[v] = prev[v]; e[v].merge(cur[v]); prev[v] = cur[v]; }
      finish_entry<ET, NV>(s, P.eps, G, e, rc.ch0, ent_base + j, true, j);
    } else {
      segment(j, cur, rc);
      finish_entry<ET, NV>(s, P.eps, G, cur, rc.ch0, ent_base + j, true, j);
    }
  }
}

template <typename ET, int NV, int LB = (NV == 1 ? 16 : 0)>
__device__ void compress_large(const CompressStreamDev& s, const CompressParams& P, int b, int cb,
                               float* lds) {
  constexpr int VE = ET::kVec;
  const int G = s.G;
  const int RG = (int)blockDim.x / G;
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

  // the window is cut into VG groups of consecutive tokens whatever the
  // block size (the partition of a 512-thread block), so that every launch
  // configuration pools and combines in the same order; a row group walks
  // the groups rg, rg + RG, ...
  const int VG = kLargeLayoutThreads / G;
  const int chunk = (s.w + VG - 1) / VG;
  const int C = s.C;
  const int64_t base = j * s.m;
  for (int vg = rg; vg < VG; vg += RG) {
  const int tb = vg * chunk;
  const int te = min(s.w, tb + chunk);
  PoolState<VE> st[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) st[v].reset();
  int t = tb;
  // with per-channel logits a full batch of LB tokens keeps all of its raw
  // loads in flight at once (one memory round trip): an HCA window (w = 128
  // over 8 row groups, LB = 16) is one batch
  if constexpr (NV == 1 && LB > 0) {
    if (rc.per_channel) {
      for (; t + LB <= te; t += LB) {
        uint4 xr[LB], zr[LB];
#pragma unroll
        for (int u = 0; u < LB; ++u) {
          const int64_t tr = (base + t + u) * rc.row_bytes + (int64_t)rc.ch0[0] * ET::kBytes;
          xr[u] = ldg16(rc.src, tr);
          zr[u] = ldg16(rc.lg, tr);
        }
#pragma unroll
        for (int u = 0; u < LB; ++u) {
          float x[VE], z[VE];
          ET::unpack(xr[u], x);
          ET::unpack(zr[u], z);
          st[0].add(z, x);
        }
      }
    }
  }
  if (!(NV == 1 && LB > 0 && rc.per_channel)) {
    for (; t + 8 <= te; t += 8) {
      float x[8][NV][VE], z[8][NV][VE];
#pragma unroll
      for (int u = 0; u < 8; ++u) rc.load(base + t + u, x[u], z[u]);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int v = 0; v < NV; ++v) st[v].add(z[u][v], x[u][v]);
    }
  }
  for (; t < te; ++t) {
    float x[NV][VE], z[NV][VE];
    rc.load(base + t, x, z);
#pragma unroll
    for (int v = 0; v < NV; ++v) st[v].add(z[v], x[v]);
  }
  // partial states -> LDS [VG][3][C]
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const int c = rc.ch0[v] + e;
      lds[(vg * 3 + 0) * C + c] = st[v].mx[e];
      lds[(vg * 3 + 1) * C + c] = st[v].se[e];
      lds[(vg * 3 + 2) * C + c] = st[v].sn[e];
    }
  }
  __syncthreads();
  // combine the row groups' states, one channel per thread; pooled value -> LDS
  float* pooled = lds + VG * 3 * C;
  for (int c = threadIdx.x; c < C; c += (int)blockDim.x) {
    float M = -INFINITY;
    for (int r = 0; r < VG; ++r) M = fmaxf(M, lds[(r * 3 + 0) * C + c]);
    float se = 0.f, sn = 0.f;
    for (int r = 0; r < VG; ++r) {
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
  if (s.rope.dims)
#pragma unroll
    for (int v = 0; v < NV; ++v) rope_turn<VE>(e[v], rc.ch0[v], C, s.rope, (double)(j * s.m + s.w - 1));
  const int64_t rb = (int64_t)C * ET::kBytes;
  const int64_t out_row = s.ent_off[b] + j;
#pragma unroll
  for (int v = 0; v < NV; ++v) stg16(s.out, out_row * rb + (int64_t)rc.ch0[v] * ET::kBytes, ET::pack(e[v]));
}


// Block `blk` of a compression launch (any block size the setup was made
// for); LB: tokens per batch of the large-window walk (0: 8 at a time); PF:
// the small-window walk prefetches the next segment (more registers).
template <typename ET, int NV, int LB = (NV == 1 ? 16 : 0), bool PF = true>
__device__ __forceinline__ void compress_block(const CompressParams& P, int blk, float* lds) {
  int si = 0;
  for (int k = 1; k < P.n; ++k)
    if (blk >= P.s[k].block_begin) si = k;
  const CompressStreamDev& s = P.s[si];
  if (s.bps <= 0) return;
  const int local = blk - s.block_begin;
  const int b = local / s.bps;
  const int cb = local % s.bps;
  if (b >= P.B) return;
  if (s.small)
    compress_small<ET, NV, PF>(s, P, b, cb);
  else
    compress_large<ET, NV, LB>(s, P, b, cb, lds);
}

// Host: fill the stream descriptors for blocks of `threads` threads; returns
// LCA_OK and the block count and dynamic LDS bytes of the streams, or an
// error (message set) when the streams cannot share one launch.
int setup_compress(const lca_compress_stream* streams, int n, const int64_t* tok_off, const int64_t* done_len,
                   int B, float eps, int dtype, int threads, CompressParams* P, int64_t* blocks, size_t* lds_bytes,
                   int* nv);

}  // namespace lca
