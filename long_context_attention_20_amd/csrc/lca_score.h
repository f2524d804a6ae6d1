// Device side of the lightning-indexer scores (shared by the score kernels
// and the decode front launch, which runs them beside attention blocks):
// the score parameters, the key-row formats, the per-block score of an
// entry range with its histogram, and the decode append of new indexer keys.
//
// Pages: "DeepSeek-V4", Design overview and Inference efficiency (the
// lightning indexer on the compressed entries, its query-key path in low
// precision).  Score of entry j for query row r:
//     s = sum_h omega[r,h] * max(0, p[r,h,:] . key_j).
#pragma once
#include "lca_compress.h"
#include "lca_topk.h"

namespace lca {

constexpr int kIdxThreads = 256;
constexpr int kSelThreads = 256;
constexpr int kSelChunk = 4096;  // entries per select block
constexpr int kSelPerThread = kSelChunk / kSelThreads;

struct IndexParams {
  const void* p;
  const float* omega;
  const void* ikey;
  const int64_t* csa_off;
  const int32_t* q_pos;
  int Tq, HI, dI, k, m, w;
  int64_t max_entries;
  int chunk;                // entries per score block
  float* scores;            // [rows][max_entries]
  uint32_t* hist;           // [rows][nstripe][kHistBins]
  int nstripe;              // histogram copies (score blocks spread their atomics)
  unsigned long long* ctr;  // [rows]: selected count | candidate count << 32
  uint32_t* done;           // [rows]: blocks that finished filtering (in-launch filtering)
  int no_hist;              // 1: many rows per sequence, selected one block per row (no histograms)
  int32_t* sel;             // [rows][k]
  uint64_t* cand;           // [rows][max_entries]
  int32_t* idx;             // [rows][k]
};
__device__ __forceinline__ int64_t row_visible(const IndexParams& a, int r, int64_t n_seq) {
  const int i = a.q_pos[r];
  int64_t nv = n_windows((int64_t)i + 1, a.m, a.w);
  nv = nv < n_seq ? nv : n_seq;
  // never beyond the per-row capacity the workspace was sized for
  return nv < a.max_entries ? nv : a.max_entries;
}

// ------------------------------------------------------------------ fp8 key rows
// A key row of the fp8 cache: d_I OCP E4M3 bytes, the row's fp32 scale, 4 zero
// bytes.  The bytes are widened to bf16 (every E4M3 value is exact in bf16:
// the upper half of its fp32 form) and fed to the bf16 matrix cores, so the
// products are exact; the scale multiplies the row's score (s >= 0).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(f32x2_t f) {
  return (__float_as_uint(f.x) >> 16) | (__float_as_uint(f.y) & 0xFFFF0000u);
}
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint2 v) {
  return make_uint4(bf16_pair(__builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, false)),
                    bf16_pair(__builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, true)),
                    bf16_pair(__builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, false)),
                    bf16_pair(__builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, true)));
}
// Bytes per key row: bf16 (KF 0), fp8 rows (1), MXFP4 rows (2).
__device__ __forceinline__ int64_t key_row_bytes(const IndexParams& a, int kf) {
  return kf == 1 ? (int64_t)a.dI + 8 : kf == 2 ? (int64_t)a.dI / 2 + 8 : (int64_t)a.dI * 2;
}
// The 8 dims lane group grp feeds k-step ks of a 16x16x32 product.  bf16
// rows: dims 32*ks + 8*grp ..; fp8 rows: lane group grp takes the KS*8
// consecutive dims from KS*8*grp (one 16-byte load per two k-steps) -- the
// contraction runs over every dim once either way, and the query operand
// uses the same order.
template <int KS>
__device__ __forceinline__ int key_dim(int ks, int grp, bool fp8) {
  return fp8 ? (KS * grp + ks) * 8 : ks * 32 + grp * 8;
}
// MXFP4 rows: lane group grp's KS words of 8 E2M1 nibbles (its KS*8
// consecutive channels) and the E8M0 scale of each word's 32-channel block.
template <int KS>
__device__ __forceinline__ void load_mx_slices(const char* row, int grp, int dI, uint32_t (&w)[KS], float (&sc)[KS]) {
  const uint32_t* nib = reinterpret_cast<const uint32_t*>(row + grp * KS * 4);
  const uint8_t* scales = reinterpret_cast<const uint8_t*>(row + dI / 2);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    w[ks] = nib[ks];
    sc[ks] = e8m0_value(scales[(grp * KS * 8 + ks * 8) >> 5]);
  }
}
// Eight E2M1 nibbles (channel c at bits 4c) times the block scale s as bf16:
// gfx950's scaled FP4 conversion takes the two nibbles of one byte (low
// nibble first) per call; an E2M1 value times a power of two is exact in bf16.
__device__ __forceinline__ uint32_t e2m1x2_to_bf16x2(uint32_t w, float s, int byte) {
  switch (byte) {
    case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0));
    case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1));
    case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2));
    default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3));
  }
}
__device__ __forceinline__ uint4 e2m1x8_to_bf16x8(uint32_t w, float s) {
  return make_uint4(e2m1x2_to_bf16x2(w, s, 0), e2m1x2_to_bf16x2(w, s, 1), e2m1x2_to_bf16x2(w, s, 2),
                    e2m1x2_to_bf16x2(w, s, 3));
}

// Lane group grp's KS slices of 8 E4M3 bytes of one fp8 row, in 16-byte loads
// (rows are d_I + 8 bytes: 8-byte aligned, which the dword loads accept).
template <int KS>
__device__ __forceinline__ void load_fp8_slices(const char* row, int grp, uint2 (&out)[KS]) {
  const char* base = row + grp * KS * 8;
  if constexpr (KS == 1) {
    out[0] = *reinterpret_cast<const uint2*>(base);
  } else {
#pragma unroll
    for (int i = 0; i < KS / 2; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(base + 16 * i);
      out[2 * i] = make_uint2(v.x, v.y);
      out[2 * i + 1] = make_uint2(v.z, v.w);
    }
  }
}

// ------------------------------------------------------------------ scores

// Block 0 of each row's scores zeroes the row's list counters, which the
// filter that follows fills.
__device__ __forceinline__ void clear_row_state(const IndexParams& a, int r) {
  if (threadIdx.x == 0) {
    a.ctr[r] = 0;
    a.done[r] = 0;
  }
}

__device__ __forceinline__ void hist_add(uint32_t* h, float s) {
  atomicAdd(&h[score_key(s) >> 21], 1u);
}

__device__ __forceinline__ void hist_flush(const uint32_t* lh, uint32_t* gh) {
  for (int bin = threadIdx.x; bin < kHistBins; bin += blockDim.x) {
    uint32_t c = lh[bin];
    if (c) atomicAdd(&gh[bin], c);
  }
}

// bf16, matrix cores.  KS = dI / 32 k-steps.  Block (cx, r) scores the
// entries [cx*chunk, min((cx+1)*chunk, lim)) of row r; lh: kHistBins words
// of LDS.  KF: key rows 0 bf16, 1 fp8 (widened to bf16 in registers, score
// times the row's scale), 2 MXFP4 (widened with their block scales).
template <int KS, int KF = 0>
__device__ __forceinline__ void score_chunk_mfma(const IndexParams& a, int r, int cx, int64_t lim, uint32_t* lh) {
  const int b = r / a.Tq;
  // the sequence's entry range and the row's position, requested together
  const int64_t e_base = a.csa_off[b];
  const int64_t e_end = a.csa_off[b + 1];
  const int qi = a.q_pos[r];
  // (an empty use of the three values here keeps the compiler from sinking
  // one load below the division that needs the other: one wait for both)
  asm volatile("" : : "s"(e_base), "s"(e_end), "s"(qi));
  int64_t nv = n_windows((int64_t)qi + 1, a.m, a.w);
  nv = min(min(nv, e_end - e_base), a.max_entries);  // as row_visible
  const int64_t c0 = (int64_t)cx * a.chunk;
  const int64_t c1 = min(min(c0 + a.chunk, nv), lim);
  if (cx == 0) clear_row_state(a, r);
  if (c0 >= c1) return;
  const bool do_hist = nv > a.k && !a.no_hist;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const char* K = reinterpret_cast<const char*>(a.ikey);
  const int64_t rowb = key_row_bytes(a, KF);
  float* S = a.scores + (int64_t)r * a.max_entries;
  constexpr int U = 8;  // tiles in flight per wave
  const int64_t ntile = (c1 - c0 + 15) / 16;
  const int nw = (int)(blockDim.x >> 6);
  // The key rows of a batch of U tiles (16 entries each; lane (col, grp)
  // takes entry col's slices for lane group grp).  The wave's first batch is
  // requested right after the query operand and the head weights, before the
  // LDS histogram is cleared and the block synchronises, so that its memory
  // latency overlaps them.
  uint4 kv[U][KS];
  uint2 k8[U][KS];
  float sc[U];
  uint32_t k4[U][KS];
  float ms[U][KS];
  auto load_batch = [&](int64_t t0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t e = c0 + (t0 + u) * 16 + col;
      if (e >= c1) e = c1 - 1;  // clamp: stays inside the visible entries
      const char* row = K + (e_base + e) * rowb;
      if constexpr (KF == 1) {
        load_fp8_slices<KS>(row, grp, k8[u]);
        sc[u] = *reinterpret_cast<const float*>(row + a.dI);
      } else if constexpr (KF == 2) {
        load_mx_slices<KS>(row, grp, a.dI, k4[u], ms[u]);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kv[u][ks] = *reinterpret_cast<const uint4*>(row + (ks * 32 + grp * 8) * 2);
      }
    }
  };
  // A operand: head `col` (zero beyond HI), dims 32*ks + 8*grp .. +7
  bf16x8_t A[KS];
  {
    const uint16_t* P = reinterpret_cast<const uint16_t*>(a.p) + (int64_t)r * a.HI * a.dI;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (col < a.HI) v = *reinterpret_cast<const uint4*>(P + col * a.dI + key_dim<KS>(ks, grp, KF != 0));
      A[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  // head weights of the accumulator rows this lane holds: rows 4*grp + i
  float om[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = grp * 4 + i;
    om[i] = h < a.HI ? a.omega[(int64_t)r * a.HI + h] : 0.f;
  }
  int64_t t0 = wave * U;
  if (t0 < ntile) load_batch(t0);
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) lh[i] = 0;
  __syncthreads();

  while (t0 < ntile) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // C[head][entry] = P[head][:] . K[entry][:]; lane (col, grp) holds the
      // entry `col` against heads 4*grp .. 4*grp+3
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (KF == 1) kv[u][ks] = fp8x8_to_bf16x8(k8[u][ks]);
        if constexpr (KF == 2) kv[u][ks] = e2m1x8_to_bf16x8(k4[u][ks], ms[u][ks]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[ks], __builtin_bit_cast(bf16x8_t, kv[u][ks]), acc, 0, 0, 0);
      }
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) part = fmaf(om[i], fmaxf(acc[i], 0.f), part);
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      if constexpr (KF == 1) part *= sc[u];
      const int64_t e = c0 + (t0 + u) * 16 + col;
      if (grp == 0 && t0 + u < ntile && e < c1) {
        S[e] = part;
        if (do_hist) hist_add(lh, part);
      }
    }
    t0 += nw * U;
    if (t0 < ntile) load_batch(t0);
  }
  __syncthreads();
  if (do_hist) hist_flush(lh, a.hist + ((int64_t)r * a.nstripe + cx % a.nstripe) * kHistBins);
}

// Several query rows of one sequence (a decode step with Tq > 1, as when a
// draft token is verified beside the main one): block (cx, b) scores entries
// [cx*chunk, ...) for all Tq rows of sequence b from one read of the keys.
// The rows share the matrix-core A operand: row q's head h is A row q*HI + h
// (Tq * HI <= 16, so they fit the 16 rows that one head set pads to).  Each
// accumulator lane adds the weighted ReLU terms of its four A rows into the
// partial of the row they belong to; the partials are summed over the four
// lane groups and lane group q stores row q's score.  lh: TQ * kHistBins
// words of LDS, one histogram per row.  KF as score_chunk_mfma.
template <int KS, int TQ, int KF = 0>
__device__ __forceinline__ void score_chunk_multi(const IndexParams& a, int b, int cx, int64_t lim, uint32_t* lh) {
  static_assert(TQ >= 2 && TQ <= 4, "2 to 4 rows per block");
  const int nq = a.Tq;  // <= TQ, nq * HI <= 16 (checked by the host)
  const int r0 = b * a.Tq;
  const int64_t e_base = a.csa_off[b];
  const int64_t nseq = a.csa_off[b + 1] - e_base;
  const int64_t c0 = (int64_t)cx * a.chunk;
  int64_t c1q[TQ];
  bool hq[TQ];
  int64_t c1 = c0;
#pragma unroll
  for (int q = 0; q < TQ; ++q) {
    const int64_t nv = q < nq ? row_visible(a, r0 + q, nseq) : 0;
    c1q[q] = min(min(c0 + a.chunk, nv), lim);
    hq[q] = q < nq && nv > a.k && !a.no_hist;
    c1 = max(c1, c1q[q]);
  }
  if (cx == 0)
    for (int q = 0; q < nq; ++q) clear_row_state(a, r0 + q);
  if (c0 >= c1) return;
  for (int i = threadIdx.x; i < TQ * kHistBins; i += blockDim.x) lh[i] = 0;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int nrow = nq * a.HI;  // A rows in use
  // A operand: A row `col` = (row col / HI, head col % HI), zero beyond nrow
  bf16x8_t A[KS];
  {
    const uint16_t* P = reinterpret_cast<const uint16_t*>(a.p) + (int64_t)r0 * a.HI * a.dI;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (col < nrow) v = *reinterpret_cast<const uint4*>(P + col * a.dI + key_dim<KS>(ks, grp, KF != 0));
      A[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  // weights of the accumulator rows this lane holds (A rows 4*grp + i),
  // sorted by the query row they belong to
  float om[TQ][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = grp * 4 + i;
    const float wgt = m < nrow ? a.omega[(int64_t)r0 * a.HI + m] : 0.f;
    const int qm = m / a.HI;
#pragma unroll
    for (int q = 0; q < TQ; ++q) om[q][i] = qm == q ? wgt : 0.f;
  }
  __syncthreads();

  const char* K = reinterpret_cast<const char*>(a.ikey);
  const int64_t rowb = key_row_bytes(a, KF);
  constexpr int U = 8;  // tiles in flight per wave
  const int64_t ntile = (c1 - c0 + 15) / 16;
  const int nw = (int)(blockDim.x >> 6);
  for (int64_t t0 = wave * U; t0 < ntile; t0 += nw * U) {
    uint4 kv[U][KS];
    uint2 k8[U][KS];
    float sc[U];
    uint32_t k4[U][KS];
    float ms[U][KS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t e = c0 + (t0 + u) * 16 + col;
      if (e >= c1) e = c1 - 1;  // clamp: stays inside the visible entries
      const char* row = K + (e_base + e) * rowb;
      if constexpr (KF == 1) {
        load_fp8_slices<KS>(row, grp, k8[u]);
        sc[u] = *reinterpret_cast<const float*>(row + a.dI);
      } else if constexpr (KF == 2) {
        load_mx_slices<KS>(row, grp, a.dI, k4[u], ms[u]);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kv[u][ks] = *reinterpret_cast<const uint4*>(row + (ks * 32 + grp * 8) * 2);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (KF == 1) kv[u][ks] = fp8x8_to_bf16x8(k8[u][ks]);
        if constexpr (KF == 2) kv[u][ks] = e2m1x8_to_bf16x8(k4[u][ks], ms[u][ks]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[ks], __builtin_bit_cast(bf16x8_t, kv[u][ks]), acc, 0, 0, 0);
      }
      const int64_t e = c0 + (t0 + u) * 16 + col;
#pragma unroll
      for (int q = 0; q < TQ; ++q) {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) part = fmaf(om[q][i], fmaxf(acc[i], 0.f), part);
        part += __shfl_xor(part, 16, 64);
        part += __shfl_xor(part, 32, 64);
        if constexpr (KF == 1) part *= sc[u];
        if (grp == q && t0 + u < ntile && e < c1q[q]) {
          a.scores[(int64_t)(r0 + q) * a.max_entries + e] = part;
          if (hq[q]) hist_add(lh + q * kHistBins, part);
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < TQ; ++q)
    if (hq[q]) hist_flush(lh + q * kHistBins, a.hist + ((int64_t)(r0 + q) * a.nstripe + cx % a.nstripe) * kHistBins);
}

// ------------------------------------------------------------------ score + append
// One decode launch that also appends the entries the new tokens complete:
//   blocks [0, ncb):             the compression blocks of the other streams
//                                (KV entries that only the attention reads);
//   blocks [ncb, ncb + B):       per sequence, pool each new indexer key,
//                                store it, and score it against the indexer
//                                query of each of the sequence's rows that
//                                sees it (adding it to that row's histogram);
//   blocks [ncb + B, ... + nsb): scores of the entries that existed before
//                                the tokens (as index_score_mfma, or
//                                index_score_multi for Tq > 1 rows).
// Blocks are dispatched in index order, so the few long compression blocks
// start first and overlap the scoring.  No block reads what another block of
// the launch writes.
struct AppendIdx {
  CompressStreamDev s;      // the indexer-key stream (out is the key cache)
  const int64_t* tok_off;
  const int64_t* done_len;
  int ncb;                  // compression blocks
  int nsb;                  // score blocks
  int nsx;                  // score blocks per sequence
  int B;
  float eps;
};

// Sum over aligned groups of n lanes, n in {4, 8, 16, 32} (uniform).
__device__ __forceinline__ float group_sum_n(float v, int n) {
  switch (n) {
    case 4: return lane_group_sum<4>(v);
    case 8: return lane_group_sum<8>(v);
    case 16: return lane_group_sum<16>(v);
    default: return lane_group_sum<32>(v);
  }
}

template <int KF>
__device__ void append_and_score(const IndexParams& a, const AppendIdx& ap, int b) {
  constexpr int VE = 8;                    // bf16 channels per 16-byte vector
  const CompressStreamDev& s = ap.s;
  const int G = s.C / VE;                  // lanes per entry (4 .. 32)
  const int RG = (int)blockDim.x / G;
  const int rg = threadIdx.x / G, li = threadIdx.x % G;
  const int64_t t0 = ap.tok_off[b];
  const int64_t e_base = a.csa_off[b];
  const int64_t nseq = a.csa_off[b + 1] - e_base;
  // every entry the tokens complete is appended (as the compression kernel
  // does); each of the sequence's query rows scores the ones it sees
  const int64_t n_hi = n_windows(ap.tok_off[b + 1] - t0, s.m, s.w);
  const int64_t n_lo = n_windows(ap.done_len[b], s.m, s.w);
  const int64_t rb = (int64_t)s.C * 2;
  const char* src = reinterpret_cast<const char*>(s.src) + t0 * rb;
  const char* lg = reinterpret_cast<const char*>(s.logits) + (s.per_channel ? t0 * rb : t0 * 2);
  // the dual-stream form reads a window's second half from the second stream
  const char* src2 = s.src2 ? reinterpret_cast<const char*>(s.src2) + t0 * rb : src;
  const char* lg2 = s.src2 ? reinterpret_cast<const char*>(s.logits2) + (s.per_channel ? t0 * rb : t0 * 2) : lg;
  const int ch0 = li * VE;
  for (int64_t j0 = n_lo; j0 < n_hi; j0 += RG) {
    const int64_t j = j0 + rg;
    const bool on = j < n_hi;              // uniform over a row group
    // the same arithmetic, in the same order, as the small-window walk of
    // the compression kernel: each m-token segment pooled on its own, two
    // adjacent segments merged when w = 2m
    const int64_t tb = (on ? j : n_lo) * s.m;
    PoolState<VE> st[2];
    const int nseg = s.w == s.m ? 1 : 2;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      st[q].reset();
      if (q >= nseg) continue;
      const char* sq = q ? src2 : src;
      const char* lq = q ? lg2 : lg;
      for (int t = q * s.m; t < (q + 1) * s.m; ++t) {
        float x[VE], z[VE];
        BF16::unpack(ldg16(sq, (tb + t) * rb + ch0 * 2), x);
        if (s.per_channel) {
          BF16::unpack(ldg16(lq, (tb + t) * rb + ch0 * 2), z);
        } else {
          const float zs = BF16::load1(lq, tb + t);
#pragma unroll
          for (int e = 0; e < VE; ++e) z[e] = zs;
        }
        st[q].add(z, x);
      }
    }
    if (nseg == 2) st[0].merge(st[1]);
    float key[VE];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      key[e] = st[0].sn[e] / st[0].se[e];
      ss = fmaf(key[e], key[e], ss);
    }
    if (s.rmsnorm) {
      ss = wave_sum(ss, G);
      const float inv = 1.0f / sqrtf(ss / (float)s.C + ap.eps);
#pragma unroll
      for (int e = 0; e < VE; ++e) key[e] *= inv;
    }
    // the stored (rounded) key is the one scored
    float row_scale = 1.f;
    if constexpr (KF == 2) {
      // an MXFP4 key row (as the compression kernel writes it), scored as
      // its elements' values times their block scales
      char* row = reinterpret_cast<char*>(s.out) + (e_base + j) * (int64_t)(s.C / 2 + 8);
      float bs;
      const uint32_t w = store_mx_row(key, G, li, row, s.C, on, &bs);
      unpack_e2m1x8(w, bs, key);
    } else if constexpr (KF == 1) {
      // an fp8 key row (as the compression kernel writes it): E4M3 bytes of
      // value / scale, scale = amax / 448 over the row's lanes; scored as the
      // bytes' values, times the scale
      float am = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) am = fmaxf(am, fabsf(key[e]));
      am = wave_max(am, G);
      const float sc = am / 448.0f;
      const uint2 q = sc > 0.f ? pack_fp8x8(key, sc) : make_uint2(0u, 0u);
      if (on) {
        char* row = reinterpret_cast<char*>(s.out) + (e_base + j) * (int64_t)(s.C + 8);
        *reinterpret_cast<uint2*>(row + ch0) = q;
        if (li == 0) *reinterpret_cast<uint2*>(row + s.C) = make_uint2(__float_as_uint(sc), 0u);
      }
      unpack_fp8x8(q, key);
      row_scale = sc;
    } else {
      const uint4 kq = BF16::pack(key);
      if (on) stg16(s.out, (e_base + j) * rb + ch0 * 2, kq);
      BF16::unpack(kq, key);
    }
    for (int q = 0; q < a.Tq; ++q) {
      const int r = b * a.Tq + q;
      const int64_t nv = row_visible(a, r, nseq);
      const bool do_hist = nv > a.k && !a.no_hist;
      // indexer query of row r for this lane's channels, all heads
      const uint16_t* P = reinterpret_cast<const uint16_t*>(a.p) + (int64_t)r * a.HI * a.dI;
      float score = 0.f;
      for (int h = 0; h < a.HI; ++h) {
        float pv[VE];
        BF16::unpack(*reinterpret_cast<const uint4*>(P + h * a.dI + ch0), pv);
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) d = fmaf(pv[e], key[e], d);
        d = group_sum_n(d, G);
        score = fmaf(a.omega[(int64_t)r * a.HI + h], fmaxf(d, 0.f), score);
      }
      if constexpr (KF == 1) score *= row_scale;
      if (on && j < nv && li == 0) {
        a.scores[(int64_t)r * a.max_entries + j] = score;
        if (do_hist)
          atomicAdd(&a.hist[((int64_t)r * a.nstripe + (int)(j % a.nstripe)) * kHistBins + (score_key(score) >> 21)],
                    1u);
      }
    }
  }
}

}  // namespace lca
