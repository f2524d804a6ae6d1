// Lightning-indexer scores over the visible CSA entries and an exact
// top-k selection.
//
// Pages: "DeepSeek-V4", Design overview (CSA applies V3.2's lightning indexer
// to the compressed entries) and Inference efficiency (the indexer QK path);
// "Why DeepSeek V4 Stands Apart", Core Architectural Innovations (top-1024
// entries per query for Pro, top-512 for Flash).
//
// Score of entry j for query row r:  s = sum_h omega[r,h] * max(0, p[r,h,:] . key_j).
//
// Kernel 1 (score): streams the indexer keys once (the dominant HBM stream of a
// decode step).  bf16: the contraction runs on the matrix cores as
// C[head][entry] = P[head][dim] * K^T[dim][entry] with v_mfma_f32_16x16x32_bf16
// (heads padded to 16 rows); the key tile is the B operand, read straight from
// global memory with one 16-byte load per lane and k-step.  It also builds a
// 2048-bin histogram of the top 11 bits of an order-preserving integer key of
// every score (LDS, then one global atomic per non-empty bin).
//
// Kernel 2 (filter): every block derives the threshold bin T from the
// histogram (the highest bin whose suffix count reaches k), and appends the
// entries of its chunk above T to a per-row "selected" list and those inside T
// (the candidates) to a per-row candidate list, reserving space with one
// 64-bit atomic per block.  No block waits for another.
//
// Kernel 3 (finalize, one block per row): the exact selection of lca_topk.h
// -- the candidates counted per next-11-bit bin in LDS, radix passes only
// inside the threshold bin of that count, a bitmap of the chosen entries
// written out in ascending index order -- then zeroes the first histogram for
// the next call.  (The sparse-attention kernel can run the same selection in
// its own blocks instead.)  The score kernels zero the counters.
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
  const int64_t e_base = a.csa_off[b];
  const int64_t nv = row_visible(a, r, a.csa_off[b + 1] - e_base);
  const int64_t c0 = (int64_t)cx * a.chunk;
  const int64_t c1 = min(min(c0 + a.chunk, nv), lim);
  if (cx == 0) clear_row_state(a, r);
  if (c0 >= c1) return;
  const bool do_hist = nv > a.k && !a.no_hist;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) lh[i] = 0;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
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
  __syncthreads();

  const char* K = reinterpret_cast<const char*>(a.ikey);
  const int64_t rowb = key_row_bytes(a, KF);
  float* S = a.scores + (int64_t)r * a.max_entries;
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
  }
  __syncthreads();
  if (do_hist) hist_flush(lh, a.hist + ((int64_t)r * a.nstripe + cx % a.nstripe) * kHistBins);
}

template <int KS, int KF = 0>
__global__ __launch_bounds__(kIdxThreads) void index_score_mfma(IndexParams a) {
  __shared__ uint32_t lh[kHistBins];
  score_chunk_mfma<KS, KF>(a, blockIdx.y, blockIdx.x, INT64_MAX, lh);
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

template <int KS, int TQ, int KF = 0>
__global__ __launch_bounds__(kIdxThreads) void index_score_multi(IndexParams a) {
  __shared__ uint32_t lh[TQ * kHistBins];
  score_chunk_multi<KS, TQ, KF>(a, blockIdx.y, blockIdx.x, INT64_MAX, lh);
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
      for (int t = q * s.m; t < (q + 1) * s.m; ++t) {
        float x[VE], z[VE];
        BF16::unpack(ldg16(src, (tb + t) * rb + ch0 * 2), x);
        if (s.per_channel) {
          BF16::unpack(ldg16(lg, (tb + t) * rb + ch0 * 2), z);
        } else {
          const float zs = BF16::load1(lg, tb + t);
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

// TQ: query rows per sequence the score blocks take at once (1: one row;
// 2 or 4: all Tq <= TQ rows of a sequence, as score_chunk_multi).  KF (0, 1 fp8, 2 MXFP4): the
// indexer-key stream writes fp8 rows, which the score blocks read.
template <int KS, int TQ, int KF>
__global__ __launch_bounds__(kIdxThreads) void index_score_append(IndexParams a, AppendIdx ap, CompressParams cp) {
  extern __shared__ uint32_t dyn[];  // max(histograms, compression) words
  const int blk = blockIdx.x;
  if (blk < ap.ncb) {
    // 8-token batches and no prefetching keep the register budget of the
    // scoring blocks
    compress_block<BF16, 1, 8, false>(cp, blk, reinterpret_cast<float*>(dyn));
  } else if (blk < ap.ncb + ap.B) {
    append_and_score<KF>(a, ap, blk - ap.ncb);
  } else {
    const int sb = blk - ap.ncb - ap.B;
    const int b = sb / ap.nsx, cx = sb % ap.nsx;
    const int64_t lim = n_windows(ap.done_len[b], a.m, a.w);
    if constexpr (TQ == 1)
      score_chunk_mfma<KS, KF>(a, b, cx, lim, dyn);
    else
      score_chunk_multi<KS, TQ, KF>(a, b, cx, lim, dyn);
  }
}

// Generic path (fp32, or bf16 shapes the matrix-core kernel does not take):
// one thread per entry.
template <typename ET>
__global__ __launch_bounds__(kIdxThreads) void index_score_valu(IndexParams a) {
  __shared__ uint32_t lh[kHistBins];
  __shared__ float sp[1024];
  __shared__ float sw[16];
  const int r = blockIdx.y;
  const int b = r / a.Tq;
  const int64_t e_base = a.csa_off[b];
  const int64_t nv = row_visible(a, r, a.csa_off[b + 1] - e_base);
  const int64_t c0 = (int64_t)blockIdx.x * a.chunk;
  if (blockIdx.x == 0) clear_row_state(a, r);
  if (c0 >= nv) return;
  const int64_t c1 = min(c0 + a.chunk, nv);
  const bool do_hist = nv > a.k && !a.no_hist;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) lh[i] = 0;
  const int nq = a.HI * a.dI;
  for (int i = threadIdx.x; i < nq; i += blockDim.x) sp[i] = ET::load1(a.p, (int64_t)r * nq + i);
  for (int i = threadIdx.x; i < a.HI; i += blockDim.x) sw[i] = a.omega[(int64_t)r * a.HI + i];
  __syncthreads();
  float* S = a.scores + (int64_t)r * a.max_entries;
  for (int64_t e = c0 + threadIdx.x; e < c1; e += blockDim.x) {
    const int64_t kb = (e_base + e) * a.dI;
    float s = 0.f;
    for (int h = 0; h < a.HI; ++h) {
      float d = 0.f;
      for (int c = 0; c < a.dI; ++c) d = fmaf(sp[h * a.dI + c], ET::load1(a.ikey, kb + c), d);
      s = fmaf(sw[h], fmaxf(d, 0.f), s);
    }
    S[e] = s;
    if (do_hist) hist_add(lh, s);
  }
  __syncthreads();
  if (do_hist) hist_flush(lh, a.hist + ((int64_t)r * a.nstripe + blockIdx.x % a.nstripe) * kHistBins);
}

// ------------------------------------------------------------------ many rows
// Prefill chunks and other calls with many query rows per sequence: the
// scores as a row-tiled matrix product, so that a block reuses every key it
// loads for 32 query rows.  Block (entry tile, row group): 32 consecutive
// rows of one sequence x 1024 entries, each wave 256 of them in 16-entry
// blocks.  The A operand packs (row, head) pairs: with HI heads, an MFMA row
// block holds 16 / HI query rows, and the accumulator lane (col, grp) holds
// heads 4*grp .. 4*grp+3 of entry col -- 4 / HI whole query rows, so the
// weighted ReLU sum over the heads stays inside the lane.  No histogram: the
// selection of these calls runs one block per row (topk_rows).
constexpr int kRowsPerBlock = 32;
constexpr int kRowsEntriesPerWave = 256;
constexpr int kRowMaxEntries = 98304;  // entries per row the one-block selection takes

static bool rows_mode(int Tq, int64_t maxN) { return Tq >= kRowsPerBlock && maxN <= kRowMaxEntries; }
// the rows of a sequence share one score block (score_chunk_multi)
static bool multi_rows_ok(int Tq, int HI) { return Tq >= 2 && Tq <= 4 && Tq * HI <= 16; }

template <int KS, int HI, int KF = 0>
__global__ __launch_bounds__(256) void index_score_rows(IndexParams a) {
  constexpr int QR = 16 / HI;                // query rows per MFMA row block
  constexpr int RB = kRowsPerBlock / QR;     // MFMA row blocks per block
  constexpr int RPL = 4 / HI;                // query rows per accumulator lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int gps = (a.Tq + kRowsPerBlock - 1) / kRowsPerBlock;  // row groups per sequence
  const int b = blockIdx.y / gps;
  const int t0 = (blockIdx.y % gps) * kRowsPerBlock;
  const int nrows = min(kRowsPerBlock, a.Tq - t0);
  const int r0 = b * a.Tq + t0;
  const int64_t e_base = a.csa_off[b];
  const int64_t nseq = a.csa_off[b + 1] - e_base;
  // the most entries any row of the group sees (lanes 0..31 one row each)
  int64_t nv_lane = 0;
  if (lane < nrows) nv_lane = row_visible(a, r0 + lane, nseq);
  int64_t nv_max = nv_lane;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int64_t x = __shfl_xor(nv_max, o, 64);
    nv_max = x > nv_max ? x : nv_max;
  }
  const int64_t w0 = (int64_t)blockIdx.x * (4 * kRowsEntriesPerWave) + (int64_t)wave * kRowsEntriesPerWave;
  if (w0 >= nv_max) return;  // uniform per wave
  // A operands: lane (col, grp) holds (row rb*QR + col/HI, head col%HI), dims 32*ks + 8*grp ..
  bf16x8_t A[RB][KS];
  float om[RB][4];
  const uint16_t* P = reinterpret_cast<const uint16_t*>(a.p);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int qr = rb * QR + col / HI;
    const bool ok = qr < nrows;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ok) v = *reinterpret_cast<const uint4*>(P + ((int64_t)(r0 + qr) * HI + col % HI) * a.dI + key_dim<KS>(ks, grp, KF != 0));
      A[rb][ks] = __builtin_bit_cast(bf16x8_t, v);
    }
    // weights of the accumulator rows 4*grp + i: (row rb*QR + (4*grp + i)/HI, head (4*grp + i)%HI)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * grp + i;
      const int q2 = rb * QR + m / HI;
      om[rb][i] = q2 < nrows ? a.omega[(int64_t)(r0 + q2) * HI + m % HI] : 0.f;
    }
  }
  const char* K = reinterpret_cast<const char*>(a.ikey);
  const int64_t rowb = key_row_bytes(a, KF);
  constexpr int EB = 4;  // 16-entry blocks in flight
  const int64_t wend = min(w0 + kRowsEntriesPerWave, min(nv_max, a.max_entries));
  for (int64_t e0 = w0; e0 < wend; e0 += 16 * EB) {
    uint4 kv[EB][KS];
    uint2 k8[EB][KS];
    float rscale[EB];
    uint32_t k4[EB][KS];
    float ms[EB][KS];
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      int64_t e = e0 + u * 16 + col;
      if (e >= nseq) e = nseq - 1;  // clamp: stays inside the sequence's keys
      const char* row = K + (e_base + e) * rowb;
      if constexpr (KF == 1) {
        load_fp8_slices<KS>(row, grp, k8[u]);
        rscale[u] = *reinterpret_cast<const float*>(row + a.dI);
      } else if constexpr (KF == 2) {
        load_mx_slices<KS>(row, grp, a.dI, k4[u], ms[u]);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kv[u][ks] = *reinterpret_cast<const uint4*>(row + (ks * 32 + grp * 8) * 2);
      }
    }
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      const int64_t e = e0 + u * 16 + col;
      const bool e_ok = e < wend;
      if constexpr (KF == 1) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kv[u][ks] = fp8x8_to_bf16x8(k8[u][ks]);
      } else if constexpr (KF == 2) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kv[u][ks] = e2m1x8_to_bf16x8(k4[u][ks], ms[u][ks]);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rb][ks], __builtin_bit_cast(bf16x8_t, kv[u][ks]), acc, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < RPL; ++q) {
          float sc = 0.f;
#pragma unroll
          for (int h = 0; h < HI; ++h) sc = fmaf(om[rb][q * HI + h], fmaxf(acc[q * HI + h], 0.f), sc);
          const int qr = rb * QR + (4 * grp) / HI + q;
          if constexpr (KF == 1) sc *= rscale[u];
          if (e_ok && qr < nrows) a.scores[(int64_t)(r0 + qr) * a.max_entries + e] = sc;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ select

__device__ __forceinline__ TopkWs topk_view(const IndexParams& a) {
  TopkWs w;
  w.scores = a.scores; w.hist = a.hist; w.nstripe = a.nstripe; w.ctr = a.ctr; w.done = a.done;
  w.sel = a.sel; w.cand = a.cand; w.max_entries = a.max_entries; w.k = a.k;
  return w;
}

__global__ __launch_bounds__(kSelThreads) void topk_filter(IndexParams a) {
  __shared__ FilterShared F;
  const int r = blockIdx.y;
  const int cb = blockIdx.x;
  const int b = r / a.Tq;
  const int64_t nv = row_visible(a, r, a.csa_off[b + 1] - a.csa_off[b]);
  if (nv <= a.k) return;  // the selection takes every visible entry
  if ((int64_t)cb * kSelChunk >= nv) return;
  const TopkWs w = topk_view(a);
  FilterPrefetch<kSelThreads, kSelPerThread> P;
  filter_prefetch(w, r, cb, 1, P);
  filter_chunk(w, r, nv, cb, 1, P, F);
}

constexpr int kFinThreads = 1024;

constexpr uint32_t kFinCandLds = 8192;  // candidates beyond the prefetched ones kept in LDS
__global__ __launch_bounds__(kFinThreads) void topk_finalize(IndexParams a) {
  __shared__ SelectLds L;
  __shared__ SelectShared S;
  __shared__ uint64_t cl[kFinCandLds];
  const int r = blockIdx.x;
  const int b = r / a.Tq;
  const int64_t nv = row_visible(a, r, a.csa_off[b + 1] - a.csa_off[b]);
  int32_t* out = a.idx + (int64_t)r * a.k;
  if (nv <= a.k) {
    for (int t = threadIdx.x; t < a.k; t += blockDim.x) out[t] = t < nv ? t : -1;
    return;
  }
  // the filter kernel has read the histogram: clear it for the next call
  uint32_t* gh = a.hist + (int64_t)r * a.nstripe * kHistBins;
  for (int i = threadIdx.x; i < a.nstripe * kHistBins; i += blockDim.x) gh[i] = 0;
  const TopkWs w = topk_view(a);
  SelectPrefetch<kFinThreads> P;
  topk_prefetch(w, r, P);
  auto emit = [&](uint32_t o, int32_t e) { out[o] = e; };
  const uint32_t got = nv <= kBitmapEntries ? topk_row_select<kFinThreads, true>(w, r, P, L, S, emit, cl, kFinCandLds)
                                            : topk_row_select<kFinThreads, false>(w, r, P, L, S, emit, cl, kFinCandLds);
  if (got == 0)
    for (int t = threadIdx.x; t < a.k; t += blockDim.x) out[t] = -1;
}

// The exact top-k of one row per block, for calls with many rows per
// sequence (scores from index_score_rows, at most kRowMaxEntries per row):
// an LDS histogram of the top 11 key bits of every visible score gives the
// threshold bin T; a second pass over the scores marks every entry above T in
// an LDS bitmap and lists the candidates inside T (packed as in lca_topk.h)
// in the row's workspace, counting them per next-11-bit bin; the second
// histogram's bin T2 and, inside it, a direct ranking (or radix passes when
// crowded) give the exact cut; the bitmap then yields the row in ascending
// index order.
constexpr int kRowThreads = 1024;
constexpr int kRowLoads = 8;    // score loads in flight per thread and pass
constexpr int kRowBitmapWords = kRowMaxEntries / 32;

__global__ __launch_bounds__(kRowThreads) void topk_rows(IndexParams a) {
  __shared__ uint32_t h1[4096];
  __shared__ uint32_t h2[kH2Bins];
  __shared__ uint32_t bitmap[kRowBitmapWords];
  __shared__ uint64_t bl[kBoundaryLds];
  __shared__ uint32_t sm[kRowThreads / 64];
  __shared__ int s_T;
  __shared__ uint32_t s_above, s_cnt, s_nc, s_nbl;
  __shared__ uint64_t s_vstar;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int b = r / a.Tq;
  const int64_t nv = row_visible(a, r, a.csa_off[b + 1] - a.csa_off[b]);
  const uint32_t k = (uint32_t)a.k;
  int32_t* out = a.idx + (int64_t)r * a.k;
  if (nv <= a.k) {
    for (int t = tid; t < a.k; t += kRowThreads) out[t] = t < nv ? t : -1;
    return;
  }
  const float* S = a.scores + (int64_t)r * a.max_entries;
  uint64_t* cand = a.cand + (int64_t)r * a.max_entries;
  for (int i = tid; i < kHistBins; i += kRowThreads) h1[i] = 0;
  for (int i = tid; i < kH2Bins; i += kRowThreads) h2[i] = 0;
  for (int i = tid; i < kRowBitmapWords; i += kRowThreads) bitmap[i] = 0;
  if (tid == 0) { s_nc = 0; s_nbl = 0; s_vstar = ~0ull; }
  __syncthreads();
  // both passes over the row's scores keep kRowLoads loads in flight per
  // thread (one at a time would leave each pass bound by memory latency)
  constexpr int U = kRowLoads;
  for (int64_t base = tid; base < nv; base += (int64_t)kRowThreads * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = base + (int64_t)u * kRowThreads;
      v[u] = e < nv ? S[e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + (int64_t)u * kRowThreads < nv) atomicAdd(&h1[score_key(v[u]) >> 21], 1u);
  }
  __syncthreads();
  find_threshold(h1, kHistBins, k, sm, &s_T, &s_above, &s_cnt);
  const uint32_t T = (uint32_t)s_T;
  const uint32_t need = k - s_above;
  for (int64_t base = tid; base < nv; base += (int64_t)kRowThreads * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = base + (int64_t)u * kRowThreads;
      v[u] = e < nv ? S[e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = base + (int64_t)u * kRowThreads;
      if (e >= nv) continue;
      const uint32_t key = score_key(v[u]);
      const uint32_t bin = key >> 21;
      if (bin > T) {
        atomicOr(&bitmap[e >> 5], 1u << (e & 31));
      } else if (bin == T) {
        cand[atomicAdd(&s_nc, 1u)] = ((uint64_t)(key & 0x1FFFFFu) << 24) | (uint64_t)(0xFFFFFFu - (uint32_t)e);
        lds_count(h2, (key >> 10) & (uint32_t)(kH2Bins - 1));
      }
    }
  }
  __syncthreads();  // the candidate list (global, this block's) and h2 are complete
  const uint32_t nc = s_nc;
  find_threshold(h2, kH2Bins, need, sm, &s_T, &s_above, &s_cnt);
  const uint32_t T2 = (uint32_t)s_T;
  const uint32_t need2 = need - s_above, cnt2 = s_cnt;
  uint64_t vstar = (uint64_t)T2 << 34;
  if (cnt2 != need2 && cnt2 <= (uint32_t)kBoundaryLds) {
    walk_loads<8>(cand, (uint32_t)tid, nc, (uint32_t)kRowThreads, [&](uint32_t, uint64_t v) {
      if ((uint32_t)(v >> 34) == T2) {
        const uint32_t slot = atomicAdd(&s_nbl, 1u);
        if (slot < (uint32_t)kBoundaryLds) bl[slot] = v;
      }
    });
    __syncthreads();
    const uint32_t nb = min(s_nbl, (uint32_t)kBoundaryLds);
    for (uint32_t i = tid; i < nb; i += kRowThreads) {
      const uint64_t v = bl[i];
      uint32_t gt = 0;
      for (uint32_t j = 0; j < nb; ++j) gt += bl[j] > v ? 1u : 0u;
      if (gt == need2 - 1) s_vstar = v;
    }
    __syncthreads();
    vstar = s_vstar;
  } else if (cnt2 != need2) {
    // a crowded bin (ties): radix passes over the low 34 bits inside it
    uint64_t prefix = vstar, mask = (uint64_t)(kH2Bins - 1) << 34;
    uint32_t nd = need2;
    const int shifts[3] = {23, 12, 0};
    const int widths[3] = {11, 11, 12};
    for (int pass = 0; pass < 3; ++pass) {
      const int sft = shifts[pass], nbins = 1 << widths[pass];
      for (int i = tid; i < nbins; i += kRowThreads) h1[i] = 0;
      __syncthreads();
      walk_loads<8>(cand, (uint32_t)tid, nc, (uint32_t)kRowThreads, [&](uint32_t, uint64_t v) {
        if ((v & mask) == prefix) lds_count(h1, (uint32_t)(v >> sft) & (uint32_t)(nbins - 1));
      });
      __syncthreads();
      find_threshold(h1, nbins, nd, sm, &s_T, &s_above, &s_cnt);
      prefix |= (uint64_t)(uint32_t)s_T << sft;
      mask |= (uint64_t)(nbins - 1) << sft;
      nd -= s_above;
      const bool done = s_cnt == nd;
      __syncthreads();
      if (done) break;
    }
    vstar = prefix;
  }
  walk_loads<8>(cand, (uint32_t)tid, nc, (uint32_t)kRowThreads, [&](uint32_t, uint64_t v) {
    if (v >= vstar) {
      const uint32_t e = 0xFFFFFFu - (uint32_t)(v & 0xFFFFFFu);
      atomicOr(&bitmap[e >> 5], 1u << (e & 31));
    }
  });
  __syncthreads();
  // ascending order: the chosen entries before each thread's words, then its bits
  constexpr int WPT = kRowBitmapWords / kRowThreads;
  uint32_t wv[WPT], c = 0;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    wv[i] = bitmap[tid * WPT + i];
    c += __popc(wv[i]);
  }
  uint32_t tot;
  uint32_t o = block_excl_scan(c, &tot, sm);
  if (tot != k) {  // inconsistent (cannot happen with a consistent histogram)
    for (int t = tid; t < a.k; t += kRowThreads) out[t] = -1;
    return;
  }
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    uint32_t x = wv[i];
    while (x) {
      const int bit = __ffs(x) - 1;
      x &= x - 1;
      out[o++] = (int32_t)((tid * WPT + i) * 32 + bit);
    }
  }
}

// ------------------------------------------------------------------ host

struct IndexWs {
  size_t scores, hist, ctr, done, sel, cand, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// entries per score block (>= 2 blocks per CU at decode) and histogram stripes
static int64_t score_chunk(int rows, int64_t maxN) {
  int64_t chunk = 512;
  while (chunk < 8192 && ((maxN + chunk - 1) / chunk) * (int64_t)rows > 4096) chunk *= 2;
  return chunk;
}
static int hist_stripes(int rows, int64_t maxN) {
  const int64_t blocks = (maxN + score_chunk(rows, maxN) - 1) / score_chunk(rows, maxN);
  return blocks >= 8 ? 8 : (int)blocks;
}

static IndexWs index_ws_layout(int rows, int64_t maxN, int k) {
  IndexWs w{};
  size_t o = 0;
  w.hist = o;     o = align256(o + (size_t)rows * hist_stripes(rows, maxN) * kHistBins * 4);
  w.ctr = o;      o = align256(o + (size_t)rows * 8);
  w.done = o;     o = align256(o + (size_t)rows * 4);
  w.scores = o;   o = align256(o + (size_t)rows * maxN * 4);
  w.sel = o;      o = align256(o + (size_t)rows * k * 4);
  w.cand = o;     o = align256(o + (size_t)rows * maxN * 8);
  w.total = o;
  return w;
}

size_t index_topk_workspace(int rows, int64_t maxN, int k) { return index_ws_layout(rows, maxN, k).total; }

static IndexParams make_params(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                               const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w,
                               int64_t maxN, int32_t* idx, const float* scores, void* ws) {
  const int rows = B * Tq;
  IndexWs L = index_ws_layout(rows, maxN, k);
  char* base = reinterpret_cast<char*>(ws);
  IndexParams a{};
  a.p = p; a.omega = omega; a.ikey = ikey; a.csa_off = csa_off; a.q_pos = q_pos;
  a.Tq = Tq; a.HI = HI; a.dI = dI; a.k = k; a.m = m; a.w = w; a.max_entries = maxN;
  a.scores = scores ? const_cast<float*>(scores) : reinterpret_cast<float*>(base + L.scores);
  a.hist = reinterpret_cast<uint32_t*>(base + L.hist);
  a.ctr = reinterpret_cast<unsigned long long*>(base + L.ctr);
  a.done = reinterpret_cast<uint32_t*>(base + L.done);
  a.sel = reinterpret_cast<int32_t*>(base + L.sel);
  a.cand = reinterpret_cast<uint64_t*>(base + L.cand);
  a.idx = idx;
  a.chunk = (int)score_chunk(rows, maxN);
  a.nstripe = hist_stripes(rows, maxN);
  a.no_hist = rows_mode(Tq, maxN) ? 1 : 0;
  return a;
}

int launch_index_score(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                       const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w, int64_t maxN,
                       float* scores, void* ws, int dtype, hipStream_t stream) {
  IndexParams a = make_params(p, omega, ikey, csa_off, q_pos, B, Tq, HI, dI, k, m, w, maxN, nullptr, scores, ws);
  const int rows = B * Tq;
  dim3 g1((unsigned)((maxN + a.chunk - 1) / a.chunk), (unsigned)rows);
  // key rows: 0 bf16/fp32, 1 fp8, 2 MXFP4
  const int kf = dtype == LCA_BF16_FP8KEY ? 1 : dtype == LCA_BF16_MXFP4KEY ? 2 : 0;
  const bool mfma = (dtype == LCA_BF16 || kf) && HI <= 16 && (dI % 32) == 0 && dI <= 256;
  if (kf && !mfma) {
    set_error("csa_index_score: fp8 / MXFP4 key rows are scored for H_I <= 16 and d_I in {32, 64, 128, 256}");
    return LCA_ERR_UNSUPPORTED;
  }
  if (mfma && a.no_hist && (HI == 1 || HI == 2 || HI == 4)) {
    // many rows per sequence: the row-tiled kernel
    const int gps = (Tq + kRowsPerBlock - 1) / kRowsPerBlock;
    dim3 g((unsigned)((maxN + 4 * kRowsEntriesPerWave - 1) / (4 * kRowsEntriesPerWave)), (unsigned)(B * gps));
#define LCA_ROWS2(KSv, F8)                                                                                 \
  switch (HI) {                                                                                            \
    case 1: hipLaunchKernelGGL((index_score_rows<KSv, 1, F8>), g, dim3(256), 0, stream, a); break;       \
    case 2: hipLaunchKernelGGL((index_score_rows<KSv, 2, F8>), g, dim3(256), 0, stream, a); break;       \
    default: hipLaunchKernelGGL((index_score_rows<KSv, 4, F8>), g, dim3(256), 0, stream, a); break;      \
  }
#define LCA_ROWS(KSv)      \
  if (kf == 1) {           \
    LCA_ROWS2(KSv, 1)      \
  } else if (kf == 2) {    \
    LCA_ROWS2(KSv, 2)      \
  } else {                 \
    LCA_ROWS2(KSv, 0)      \
  }
    switch (dI / 32) {
      case 1: LCA_ROWS(1) break;
      case 2: LCA_ROWS(2) break;
      case 4: LCA_ROWS(4) break;
      default: LCA_ROWS(8) break;
    }
#undef LCA_ROWS
#undef LCA_ROWS2
    return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
  }
  if (mfma && multi_rows_ok(Tq, HI) && !a.no_hist) {
    // a few rows per sequence: all of them from one read of the keys
    dim3 g((unsigned)((maxN + a.chunk - 1) / a.chunk), (unsigned)B);
#define LCA_MULTI2(KSv, KFv)                                                                                   \
  if (Tq == 2) hipLaunchKernelGGL((index_score_multi<KSv, 2, KFv>), g, dim3(kIdxThreads), 0, stream, a);       \
  else hipLaunchKernelGGL((index_score_multi<KSv, 4, KFv>), g, dim3(kIdxThreads), 0, stream, a);
#define LCA_MULTI(KSv)                                                                                         \
  if (kf == 1) {                                                                                               \
    LCA_MULTI2(KSv, 1)                                                                                         \
  } else if (kf == 2) {                                                                                        \
    LCA_MULTI2(KSv, 2)                                                                                         \
  } else {                                                                                                     \
    LCA_MULTI2(KSv, 0)                                                                                         \
  }
    switch (dI / 32) {
      case 1: LCA_MULTI(1) break;
      case 2: LCA_MULTI(2) break;
      case 4: LCA_MULTI(4) break;
      default: LCA_MULTI(8) break;
    }
#undef LCA_MULTI
#undef LCA_MULTI2
    return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
  }
  if (mfma && kf) {
#define LCA_KEYROWS(KFv)                                                                                  \
  switch (dI / 32) {                                                                                      \
    case 1: hipLaunchKernelGGL((index_score_mfma<1, KFv>), g1, dim3(kIdxThreads), 0, stream, a); break;   \
    case 2: hipLaunchKernelGGL((index_score_mfma<2, KFv>), g1, dim3(kIdxThreads), 0, stream, a); break;   \
    case 4: hipLaunchKernelGGL((index_score_mfma<4, KFv>), g1, dim3(kIdxThreads), 0, stream, a); break;   \
    default: hipLaunchKernelGGL((index_score_mfma<8, KFv>), g1, dim3(kIdxThreads), 0, stream, a); break;  \
  }
    if (kf == 1) {
      LCA_KEYROWS(1)
    } else {
      LCA_KEYROWS(2)
    }
#undef LCA_KEYROWS
  } else if (mfma) {
    switch (dI / 32) {
      case 1: hipLaunchKernelGGL((index_score_mfma<1>), g1, dim3(kIdxThreads), 0, stream, a); break;
      case 2: hipLaunchKernelGGL((index_score_mfma<2>), g1, dim3(kIdxThreads), 0, stream, a); break;
      case 4: hipLaunchKernelGGL((index_score_mfma<4>), g1, dim3(kIdxThreads), 0, stream, a); break;
      case 8: hipLaunchKernelGGL((index_score_mfma<8>), g1, dim3(kIdxThreads), 0, stream, a); break;
      default: hipLaunchKernelGGL((index_score_valu<BF16>), g1, dim3(kIdxThreads), 0, stream, a);
    }
  } else if (dtype == LCA_BF16) {
    hipLaunchKernelGGL((index_score_valu<BF16>), g1, dim3(kIdxThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL((index_score_valu<F32>), g1, dim3(kIdxThreads), 0, stream, a);
  }
  return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
}

int launch_compress(const lca_compress_stream* streams, int n, const int64_t* tok_off, const int64_t* done_len,
                    int B, float eps, int dtype, hipStream_t stream);

int launch_index_score_append(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                              const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w, int64_t maxN,
                              const lca_compress_stream* idx_stream, const lca_compress_stream* kv_streams, int n_kv,
                              const int64_t* tok_off, const int64_t* done_len, float eps, float* scores, void* ws,
                              int dtype, hipStream_t stream) {
  // the fused launch: bf16 matrix-core scores, one query row per sequence or
  // a few sharing a score block, KV streams of at most 512 bf16 channels;
  // anything else runs as the two launches it stands for
  // dtype LCA_BF16_FP8KEY / LCA_BF16_MXFP4KEY: bf16 inputs, the indexer-key
  // stream writes (and the scores read) fp8 / MXFP4 key rows
  const int kf = dtype == LCA_BF16_FP8KEY ? 1 : dtype == LCA_BF16_MXFP4KEY ? 2 : 0;
  const int in_dtype = kf ? LCA_BF16 : dtype;
  const bool fused = in_dtype == LCA_BF16 && HI <= 16 && (dI == 32 || dI == 64 || dI == 128 || dI == 256) &&
                     idx_stream->C == dI && idx_stream->m == m && idx_stream->w == w &&
                     (w == m || w == 2 * m) && w <= 16 && (Tq == 1 || multi_rows_ok(Tq, HI));
  CompressParams cp{};
  int64_t cblocks = 0;
  size_t clds = 0;
  int nv = 1;
  if (fused && n_kv > 0) {
    const int rc = setup_compress(kv_streams, n_kv, tok_off, done_len, B, eps, in_dtype, kIdxThreads, &cp, &cblocks,
                                  &clds, &nv);
    if (rc != LCA_OK) return rc;
  }
  if (!fused || nv != 1) {
    lca_compress_stream all[5];
    int n = 0;
    all[n++] = *idx_stream;
    for (int i = 0; i < n_kv; ++i) all[n++] = kv_streams[i];
    // streams of one compression launch share the vector width: the indexer
    // keys go first, alone when they differ
    int rc = launch_compress(all, 1, tok_off, done_len, B, eps, in_dtype, stream);
    if (rc == LCA_OK && n_kv > 0) rc = launch_compress(all + 1, n_kv, tok_off, done_len, B, eps, in_dtype, stream);
    if (rc != LCA_OK) return rc;
    return launch_index_score(p, omega, ikey, csa_off, q_pos, B, Tq, HI, dI, k, m, w, maxN, scores, ws, dtype, stream);
  }
  IndexParams a = make_params(p, omega, ikey, csa_off, q_pos, B, Tq, HI, dI, k, m, w, maxN, nullptr, scores, ws);
  AppendIdx ap{};
  const lca_compress_stream& in = *idx_stream;
  ap.s.src = in.src; ap.s.logits = in.logits; ap.s.out = in.out; ap.s.ent_off = in.ent_off;
  ap.s.C = in.C; ap.s.m = in.m; ap.s.w = in.w; ap.s.per_channel = in.per_channel; ap.s.rmsnorm = in.rmsnorm;
  ap.s.key = in.out_key;
  ap.s.max_entries = in.max_entries;
  ap.tok_off = tok_off;
  ap.done_len = done_len;
  ap.nsx = (int)((maxN + a.chunk - 1) / a.chunk);
  ap.nsb = ap.nsx * B;
  ap.ncb = (int)cblocks;
  ap.B = B;
  ap.eps = eps;
  const int64_t blocks = (int64_t)ap.nsb + B + cblocks;
  if (blocks > 0x7FFFFFFF) {
    set_error("csa_index_score_append: grid too large (%lld blocks)", (long long)blocks);
    return LCA_ERR_UNSUPPORTED;
  }
  const int tq = Tq == 1 ? 1 : Tq == 2 ? 2 : 4;  // rows a score block takes
  const size_t hist_lds = (size_t)tq * kHistBins * 4;
  const size_t lds = clds > hist_lds ? clds : hist_lds;
  dim3 grid((unsigned)blocks);
#define LCA_APPEND2(KSv, F8)                                                                                     \
  switch (tq) {                                                                                                  \
    case 1: hipLaunchKernelGGL((index_score_append<KSv, 1, F8>), grid, dim3(kIdxThreads), lds, stream, a, ap, cp); break; \
    case 2: hipLaunchKernelGGL((index_score_append<KSv, 2, F8>), grid, dim3(kIdxThreads), lds, stream, a, ap, cp); break; \
    default: hipLaunchKernelGGL((index_score_append<KSv, 4, F8>), grid, dim3(kIdxThreads), lds, stream, a, ap, cp); break; \
  }
#define LCA_APPEND(KSv)        \
  if (kf == 1) {               \
    LCA_APPEND2(KSv, 1)        \
  } else if (kf == 2) {        \
    LCA_APPEND2(KSv, 2)        \
  } else {                     \
    LCA_APPEND2(KSv, 0)        \
  }
  switch (dI / 32) {
    case 1: LCA_APPEND(1) break;
    case 2: LCA_APPEND(2) break;
    case 4: LCA_APPEND(4) break;
    default: LCA_APPEND(8) break;
  }
#undef LCA_APPEND
#undef LCA_APPEND2
  return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
}

// The workspace views of the filter's lists, for the sparse-attention launch
// whose blocks run the exact selection.
void topk_ws_view(int rows, int64_t maxN, int k, const float* scores, void* ws, TopkWs* view) {
  IndexParams a = make_params(nullptr, nullptr, nullptr, nullptr, nullptr, rows, 1, 1, 8, k, 1, 1, maxN, nullptr,
                              scores, ws);
  view->scores = a.scores; view->hist = a.hist; view->nstripe = a.nstripe; view->ctr = a.ctr;
  view->done = a.done; view->sel = a.sel; view->cand = a.cand; view->max_entries = maxN; view->k = k;
}

int launch_topk_filter(const int64_t* csa_off, const int32_t* q_pos, int B, int Tq, int k, int m, int w,
                       int64_t maxN, const float* scores, void* ws, hipStream_t stream) {
  IndexParams a = make_params(nullptr, nullptr, nullptr, csa_off, q_pos, B, Tq, 1, 8, k, m, w, maxN, nullptr, scores,
                              ws);
  const int nblk = (int)((maxN + kSelChunk - 1) / kSelChunk);
  hipLaunchKernelGGL(topk_filter, dim3((unsigned)nblk, (unsigned)(B * Tq)), dim3(kSelThreads), 0, stream, a);
  return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
}

// The second launch of the selection alone (after the filter).
int launch_topk_finalize(const int64_t* csa_off, const int32_t* q_pos, int B, int Tq, int k, int m, int w,
                         int64_t maxN, int32_t* idx, const float* scores, void* ws, hipStream_t stream) {
  IndexParams a = make_params(nullptr, nullptr, nullptr, csa_off, q_pos, B, Tq, 1, 8, k, m, w, maxN, idx, scores, ws);
  hipLaunchKernelGGL(topk_finalize, dim3((unsigned)(B * Tq)), dim3(kFinThreads), 0, stream, a);
  return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
}

bool topk_rows_mode(int Tq, int64_t maxN) { return rows_mode(Tq, maxN); }

int launch_topk_select(const int64_t* csa_off, const int32_t* q_pos, int B, int Tq, int k, int m, int w,
                       int64_t maxN, int32_t* idx, const float* scores, void* ws, hipStream_t stream) {
  IndexParams a = make_params(nullptr, nullptr, nullptr, csa_off, q_pos, B, Tq, 1, 8, k, m, w, maxN, idx, scores, ws);
  if (a.no_hist) {
    // many rows per sequence: one block per row
    hipLaunchKernelGGL(topk_rows, dim3((unsigned)(B * Tq)), dim3(kRowThreads), 0, stream, a);
    return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
  }
  const int nblk = (int)((maxN + kSelChunk - 1) / kSelChunk);
  hipLaunchKernelGGL(topk_filter, dim3((unsigned)nblk, (unsigned)(B * Tq)), dim3(kSelThreads), 0, stream, a);
  hipLaunchKernelGGL(topk_finalize, dim3((unsigned)(B * Tq)), dim3(kFinThreads), 0, stream, a);
  return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
}

}  // namespace lca
