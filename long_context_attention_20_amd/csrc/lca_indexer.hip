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

#include <algorithm>
#include <mutex>

#include "lca_score.h"

namespace lca {

template <int KS, int KF = 0>
__global__ __launch_bounds__(kIdxThreads) void index_score_mfma(IndexParams a) {
  __shared__ uint32_t lh[kHistBins];
  warm_kernargs<sizeof(IndexParams)>();
  score_chunk_mfma<KS, KF>(a, blockIdx.y, blockIdx.x, INT64_MAX, lh);
}

template <int KS, int TQ, int KF = 0>
__global__ __launch_bounds__(kIdxThreads) void index_score_multi(IndexParams a) {
  warm_kernargs<sizeof(IndexParams)>();
  __shared__ uint32_t lh[TQ * kHistBins];
  score_chunk_multi<KS, TQ, KF>(a, blockIdx.y, blockIdx.x, INT64_MAX, lh);
}

// TQ: query rows per sequence the score blocks take at once (1: one row;
// 2 or 4: all Tq <= TQ rows of a sequence, as score_chunk_multi).  KF (0, 1 fp8, 2 MXFP4): the
// indexer-key stream writes fp8 rows, which the score blocks read.
template <int KS, int TQ, int KF>
__global__ __launch_bounds__(kIdxThreads) void index_score_append(IndexParams a, AppendIdx ap, CompressParams cp) {
  extern __shared__ uint32_t dyn[];  // max(histograms, compression) words
  warm_kernargs<sizeof(IndexParams) + sizeof(AppendIdx) + sizeof(CompressParams)>();
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
constexpr int kRowBitmapWords = kRowMaxEntries / 32;

static bool rows_mode(int Tq, int64_t maxN) { return Tq >= kRowsPerBlock && maxN <= kRowMaxEntries; }
// the rows of a sequence share one score block (score_chunk_multi)
static bool multi_rows_ok(int Tq, int HI) { return Tq >= 2 && Tq <= 4 && Tq * HI <= 16; }

// The raw key-row data of EB blocks of 16 entries from e0 in one lane: lane
// (col, grp) holds entry e0 + 16u + col, the 8 dims (bf16 rows) or bytes
// (fp8 / MXFP4 rows) lane group grp feeds each k-step.  Entries at or past
// nseq read the sequence's last key (their scores are not used).
template <int KS, int KF, int EB>
struct KeyRegs {
  uint4 kv[EB][KS];
  uint2 k8[EB][KS];
  float rscale[EB];
  uint32_t k4[EB][KS];
  float ms[EB][KS];

  __device__ __forceinline__ void load(const IndexParams& a, int64_t e_base, int64_t nseq, int64_t e0, int col,
                                       int grp) {
    const char* K = reinterpret_cast<const char*>(a.ikey);
    const int64_t rowb = key_row_bytes(a, KF);
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
  }

  // The same, with the row stride known at compile time (d_I = 32 KS) and
  // the addresses taken from the sequence's first row: entries from e0
  // (lane col: e0 + 16u + col), clamped below nseq only in a round that
  // reaches it.
  static constexpr int kRowBytes = KF == 1 ? KS * 32 + 8 : KF == 2 ? KS * 16 + 8 : KS * 64;
  __device__ __forceinline__ void load_rows(const char* seq, uint32_t e0, uint32_t nseq, int col, int grp) {
    const bool tail = e0 + EB * 16 > nseq;  // uniform
    const char* base = seq + (size_t)(e0 + (uint32_t)col) * kRowBytes;
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      const char* row = base + u * 16 * kRowBytes;
      if (tail) {
        uint32_t e = e0 + (uint32_t)(u * 16 + col);
        e = e < nseq ? e : nseq - 1;
        row = seq + (size_t)e * kRowBytes;
      }
      if constexpr (KF == 1) {
        load_fp8_slices<KS>(row, grp, k8[u]);
        rscale[u] = *reinterpret_cast<const float*>(row + KS * 32);
      } else if constexpr (KF == 2) {
        load_mx_slices<KS>(row, grp, KS * 32, k4[u], ms[u]);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kv[u][ks] = *reinterpret_cast<const uint4*>(row + (ks * 32 + grp * 8) * 2);
      }
    }
  }
};

// max(x, 0) as one integer max: a negative float's bit pattern is a negative
// integer (and -0 becomes +0); the same value as fmaxf(x, 0) for every
// non-NaN x, without the canonicalizing instruction fmaxf costs here
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// The row-tiled product's operands for NR consecutive query rows r0 ..
// r0 + nrows - 1 of one sequence: lane (col, grp) holds, for MFMA row block
// rb, the query dims of (row rb*QR + col/HI, head col%HI) and the weights of
// its accumulator rows 4*grp + i (rows past nrows weigh 0).
template <int KS, int HI, int KF, int NR>
struct RowTile {
  static constexpr int QR = 16 / HI;   // query rows per MFMA row block
  static constexpr int RB = NR / QR;   // MFMA row blocks
  static constexpr int RPL = 4 / HI;   // query rows per accumulator lane
  bf16x8_t A[RB][KS];
  float om[RB][4];

  // the query row (0 .. NR-1) of accumulator (rb, q) in lane group grp
  static __device__ __forceinline__ int row(int rb, int q, int grp) { return rb * QR + (4 * grp) / HI + q; }

  __device__ __forceinline__ void load(const IndexParams& a, int r0, int nrows, int col, int grp) {
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
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * grp + i;
        const int q2 = rb * QR + m / HI;
        om[rb][i] = q2 < nrows ? a.omega[(int64_t)(r0 + q2) * HI + m % HI] : 0.f;
      }
    }
  }

  // Scores of the loaded keys: sc[u][rb][q] is the score of entry
  // e0 + 16u + col for row(rb, q, grp).
  template <int EB>
  __device__ __forceinline__ void scores(KeyRegs<KS, KF, EB>& K, float (&sc)[EB][RB][RPL]) const {
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      uint4 kv[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (KF == 1) kv[ks] = fp8x8_to_bf16x8(K.k8[u][ks]);
        else if constexpr (KF == 2) kv[ks] = e2m1x8_to_bf16x8(K.k4[u][ks], K.ms[u][ks]);
        else kv[ks] = K.kv[u][ks];
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rb][ks], __builtin_bit_cast(bf16x8_t, kv[ks]), acc, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < RPL; ++q) {
          float s = 0.f;
#pragma unroll
          for (int h = 0; h < HI; ++h) s = fmaf(om[rb][q * HI + h], relu_bits(acc[q * HI + h]), s);
          if constexpr (KF == 1) s *= K.rscale[u];
          sc[u][rb][q] = s;
        }
      }
    }
  }
};

template <int KS, int HI, int KF = 0>
__global__ __launch_bounds__(256) void index_score_rows(IndexParams a) {
  warm_kernargs<sizeof(IndexParams)>();
  using Tile = RowTile<KS, HI, KF, kRowsPerBlock>;
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
  Tile T;
  T.load(a, r0, nrows, col, grp);
  constexpr int EB = 4;  // 16-entry blocks in flight
  const int64_t wend = min(w0 + kRowsEntriesPerWave, min(nv_max, a.max_entries));
  for (int64_t e0 = w0; e0 < wend; e0 += 16 * EB) {
    KeyRegs<KS, KF, EB> K;
    K.load(a, e_base, nseq, e0, col, grp);
    float sc[EB][Tile::RB][Tile::RPL];
    T.template scores<EB>(K, sc);
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      const int64_t e = e0 + u * 16 + col;
      const bool e_ok = e < wend;
#pragma unroll
      for (int rb = 0; rb < Tile::RB; ++rb)
#pragma unroll
        for (int q = 0; q < Tile::RPL; ++q) {
          const int qr = Tile::row(rb, q, grp);
          if (e_ok && qr < nrows) a.scores[(int64_t)(r0 + qr) * a.max_entries + e] = sc[u][rb][q];
        }
    }
  }
}

// ------------------------------------------------------------------ many rows, streaming selection
// Scores and the exact top-k of many rows per sequence in one launch, with
// no score stored: block = 16 consecutive query rows of one sequence x every
// entry they see, 8 waves.  The entries go by in rounds of 512 (each wave 64;
// 256 and 128 for d_I = 128 and 256), in the row-tiled product above (so the
// scores are bit-identical to index_score_rows'); each wave loads the keys of its next round before it
// scores the current one.  Each row keeps, in LDS, a list of candidates as
// 64-bit keys
//     score_key(s) << 32 | ~j
// (a total order: larger score first, then smaller entry), and a threshold
// tau: a key with at least k listed keys at or above it, so that an entry
// whose key is below tau cannot be among the row's k largest.  Every entry
// at or above tau is listed.  When a round's keys would overflow a list, a
// wave shrinks it first: histogram passes over the listed keys (256 equal bins of
// the current key range per pass) narrow down a bin edge T with at least k
// keys at or above it and at most k + k/4, the keys below T are dropped and T
// becomes tau.  At the end the same passes find the exact k-th key, and the
// chosen entries are sorted (bitonic, in LDS) and written in ascending
// order.  For k up to kStreamMaxK (the lists of 16 rows fill the LDS).
constexpr int kStreamRows = 16;
constexpr int kStreamWaves = 8;
// 16-entry blocks per wave and round (fewer for wide keys: the next round's
// keys are held in registers beside the current one's)
template <int KS>
constexpr int stream_eb() { return KS >= 8 ? 1 : KS >= 4 ? 2 : 4; }
constexpr int kStreamRound = kStreamWaves * 16 * 4;  // the largest round
constexpr int kStreamMaxK = 512;
constexpr int kStreamCap = kStreamMaxK + kStreamMaxK / 4 + kStreamRound;  // keys per row list

// f(L[j]) for this lane's j < n (j = lane, lane + 64, ...), four LDS reads in
// flight at a time.
template <class F>
__device__ __forceinline__ void lds_walk(const uint64_t* L, uint32_t n, F f) {
  const uint32_t lane = threadIdx.x & 63;
  for (uint32_t j = lane; j < n; j += 256) {
    uint64_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = j + 64 * i < n ? L[j + 64 * i] : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (j + 64 * i < n) f(v[i]);
  }
}

// 64-bit lane exchange within a 16-lane DPP row (lanes with no source read 0)
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const uint32_t lo = dpp_u32<CTRL, 0xF>((uint32_t)x), hi = dpp_u32<CTRL, 0xF>((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// One wave: a key T such that at least `need` of the n listed keys L[0..n)
// are >= T, and exactly `need` (exact) or at most need + slack.  Requires
// n >= need >= 1, distinct keys and lo <= every key <= hi.  h: the wave's
// 256 LDS bins.
__device__ __forceinline__ uint64_t wave_threshold(const uint64_t* L, uint32_t n, uint32_t need, uint32_t slack,
                                                   bool exact, uint32_t* h, uint64_t lo, uint64_t hi) {
  const int lane = threadIdx.x & 63;
  uint32_t rem = need;  // keys still needed from [lo, hi]
  for (int pass = 0; pass < 9; ++pass) {
    const uint64_t span = hi - lo;
    const int sft = span < 256 ? 0 : 56 - __builtin_clzll(span);  // (span >> sft) < 256
#pragma unroll
    for (int i = 0; i < 4; ++i) h[lane * 4 + i] = 0;
    wave_lds_sync();
    lds_walk(L, n, [&](uint64_t v) {
      if (v >= lo && v <= hi) atomicAdd(&h[(uint32_t)((v - lo) >> sft)], 1u);
    });
    wave_lds_sync();
    uint32_t c[4], mine = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = h[lane * 4 + i];
      mine += c[i];
    }
    const uint32_t incl = wave_incl_scan(mine);
    const uint32_t tot = __shfl(incl, 63, 64);
    const uint32_t above_mine = tot - incl;  // keys in the bins of the lanes after this one
    // the bin holding the rem-th largest key: its index, the keys above it, its count
    uint32_t pick = 0, above_b = 0, cnt_b = 0;
    if (above_mine < rem && above_mine + mine >= rem) {
      uint32_t acc = above_mine;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (acc < rem && acc + c[i] >= rem) {
          pick = (uint32_t)(lane * 4 + i);
          above_b = acc;
          cnt_b = c[i];
        }
        acc += c[i];
      }
    }
    const uint64_t who = __ballot(cnt_b != 0);
    const int src = who ? __ffsll((long long)who) - 1 : 0;
    pick = __shfl(pick, src, 64);
    above_b = __shfl(above_b, src, 64);
    cnt_b = __shfl(cnt_b, src, 64);
    rem -= above_b;
    const uint64_t edge = lo + ((uint64_t)pick << sft);
    if (cnt_b == rem || (!exact && cnt_b - rem <= slack) || sft == 0 || !who) return edge;
    lo = edge;
    const uint64_t top = edge + ((1ull << sft) - 1);
    hi = top < hi ? top : hi;
  }
  return lo;
}

// One wave: keeps the keys >= t of L[0..n) at the front of L, in order, and
// returns their number.  In place: four chunks of 64 are read before any of
// them is written, and the writes never pass the reads.
__device__ __forceinline__ uint32_t wave_compact(uint64_t* L, uint32_t n, uint64_t t) {
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t out = 0;
  for (uint32_t j = 0; j < n; j += 256) {
    uint64_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t jj = j + 64 * i + lane;
      v[i] = jj < n ? L[jj] : 0;
    }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t jj = j + 64 * i + lane;
      const bool kp = jj < n && v[i] >= t;
      const uint64_t bk = __ballot(kp);
      if (kp) L[out + __popcll(bk & below)] = v[i];
      out += (uint32_t)__popcll(bk);
    }
    wave_lds_sync();
  }
  return out;
}

template <int KS, int HI, int KF = 0>
__global__ __launch_bounds__(kStreamWaves * 64) void index_topk_rows(IndexParams a) {
  warm_kernargs<sizeof(IndexParams)>();
  using Tile = RowTile<KS, HI, KF, kStreamRows>;
  constexpr int RB = Tile::RB, RPL = Tile::RPL, EB = stream_eb<KS>();
  constexpr int ROUND = kStreamWaves * 16 * EB;  // entries per round
  __shared__ uint64_t s_list[kStreamRows][kStreamCap];
  __shared__ uint32_t s_h[kStreamWaves][256];
  __shared__ uint64_t s_tau[kStreamRows];   // tau (every listed key is at or above it) ...
  __shared__ uint64_t s_max[kStreamRows];   // ... and the largest listed key
  __shared__ float s_tauf[kStreamRows];    // tau's score ...
  __shared__ uint32_t s_etau[kStreamRows]; // ... and the largest entry it admits at that score
  __shared__ uint32_t s_n[kStreamRows];     // listed keys
  __shared__ uint32_t s_add[kStreamRows];   // keys the round lists
  __shared__ uint32_t s_base[kStreamRows];  // where the round's keys go
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int gps = (a.Tq + kStreamRows - 1) / kStreamRows;  // row groups per sequence
  const int b = blockIdx.x / gps;
  const int t0 = (blockIdx.x % gps) * kStreamRows;
  const int nrows = min(kStreamRows, a.Tq - t0);
  const int r0 = b * a.Tq + t0;
  const int64_t e_base = a.csa_off[b];
  const int64_t nseq = a.csa_off[b + 1] - e_base;
  const uint32_t k = (uint32_t)a.k;
  if (threadIdx.x < kStreamRows) {
    s_tau[threadIdx.x] = 0;
    s_max[threadIdx.x] = 0;
    s_tauf[threadIdx.x] = -__builtin_inff();
    s_etau[threadIdx.x] = 0xFFFFFFFFu;
    s_n[threadIdx.x] = 0;
    s_add[threadIdx.x] = 0;
  }
  // visible entries of each row (rows past nrows see none); the block's most
  uint32_t nv_lane = 0;
  if (lane < nrows) nv_lane = (uint32_t)row_visible(a, r0 + lane, nseq);
  uint32_t nv_max = nv_lane;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nv_max = max(nv_max, (uint32_t)__shfl_xor(nv_max, o, 64));
  // this lane's rows: row(rb, q, grp)
  uint32_t nv_r[RB][RPL];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int q = 0; q < RPL; ++q) nv_r[rb][q] = (uint32_t)__shfl(nv_lane, Tile::row(rb, q, grp), 64);
  Tile T;
  T.load(a, r0, nrows, col, grp);
  const char* seq = reinterpret_cast<const char*>(a.ikey) + e_base * KeyRegs<KS, KF, EB>::kRowBytes;
  const uint32_t nseq32 = (uint32_t)nseq;
  // two key buffers: a round scores one while the next round's keys load into the other
  KeyRegs<KS, KF, EB> K0, K1;
  if (nv_max > 0) K0.load_rows(seq, (uint32_t)wave * 16 * EB, nseq32, col, grp);
  lds_barrier();
  // A round: score the current keys (the next round's load in flight),
  // count the keys to list per row (s_add), then -- after a barrier -- the
  // owner wave of each row shrinks its list if the round's keys would not fit,
  // and records where they go (s_base); after a second barrier every lane
  // writes its keys.  The keys are tested against tau as it stood when the
  // round began: a shrink in between may leave some of them below the new
  // tau (extra candidates, which the final selection drops).
  auto round = [&](KeyRegs<KS, KF, EB>& cur, KeyRegs<KS, KF, EB>& nxt, uint32_t base) {
    float tf[RB][RPL];
    uint32_t et[RB][RPL];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int q = 0; q < RPL; ++q) {
        tf[rb][q] = s_tauf[Tile::row(rb, q, grp)];
        et[rb][q] = s_etau[Tile::row(rb, q, grp)];
      }
    const uint32_t e0 = base + (uint32_t)wave * 16 * EB;
    // unconditional (the addresses are clamped into the sequence, and the
    // filter drops entries no row sees): branches here would make the
    // compiler wait for the loads in flight
    nxt.load_rows(seq, e0 + ROUND, nseq32, col, grp);
    float sc[EB][RB][RPL];
    T.template scores<EB>(cur, sc);
    // listed: keys >= tau, i.e. a score above tau's, or equal to it with an
    // entry at most tau's (NaN scores pass).  The float test !(s < tau's
    // score) passes a superset; the exact test runs only when a lane of the
    // wave passes it.  bits[rb][q]: the lane's listed entries u of row(rb, q).
    uint32_t bits[RB][RPL];
    bool pass_any = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int q = 0; q < RPL; ++q) {
        bits[rb][q] = 0;
#pragma unroll
        for (int u = 0; u < EB; ++u) pass_any |= !(sc[u][rb][q] < tf[rb][q]);
      }
    if (__ballot(pass_any)) {
#pragma unroll
      for (int u = 0; u < EB; ++u) {
        const uint32_t e = e0 + (uint32_t)(u * 16 + col);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int q = 0; q < RPL; ++q) {
            const float s = sc[u][rb][q];
            const bool keep = (!(s < tf[rb][q])) & ((s != tf[rb][q]) | (e <= et[rb][q])) & (e < nv_r[rb][q]);
            bits[rb][q] |= (uint32_t)keep << u;
          }
      }
    }
    uint32_t any = 0;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int q = 0; q < RPL; ++q) any |= bits[rb][q];
    const bool wave_any = __ballot(any != 0) != 0;
    // the lane's place among the round's keys of each of its rows (one LDS
    // atomic per row, all issued before any result is used)
    uint32_t slot[RB][RPL];
    if (wave_any) {
      // the 16 lanes of a lane group share their rows: a prefix over the
      // group (DPP within the 16-lane row) and one LDS atomic per group and
      // row (sixteen lanes adding to one word in one instruction serialise)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int q = 0; q < RPL; ++q) {
          const uint32_t c = (uint32_t)__popc(bits[rb][q]);
          uint32_t incl = c;
          incl += dpp_u32<0x111, 0xF>(incl);  // row_shr:1
          incl += dpp_u32<0x112, 0xF>(incl);  // row_shr:2
          incl += dpp_u32<0x114, 0xF>(incl);  // row_shr:4
          incl += dpp_u32<0x118, 0xF>(incl);  // row_shr:8
          // the group's last lane holds its total
          uint32_t at = 0;
          if (col == 15 && incl) at = atomicAdd(&s_add[Tile::row(rb, q, grp)], incl);
          const uint32_t a0 = __builtin_amdgcn_readlane(at, 15), a1 = __builtin_amdgcn_readlane(at, 31);
          const uint32_t a2 = __builtin_amdgcn_readlane(at, 47), a3 = __builtin_amdgcn_readlane(at, 63);
          slot[rb][q] = (grp & 2 ? (grp & 1 ? a3 : a2) : (grp & 1 ? a1 : a0)) + incl - c;
        }
    }
    lds_barrier();  // the round's counts are complete
    // a list is shrunk when the round's keys would overflow it, and every
    // 4th round when it is more than three quarters full (rows fill at
    // similar rates, so their shrinks tend to fall in the same rounds and the
    // waves wait for each other less)
    const bool trim = ((base / ROUND) & 3) == 3;
    for (int r = wave; r < nrows; r += kStreamWaves) {
      const uint32_t add = s_add[r];
      uint32_t n = s_n[r];
      if ((add != 0 && n + add > (uint32_t)kStreamCap) ||
          (trim && n > k + k / 4 && n + add > (uint32_t)(kStreamCap - ROUND / 2))) {
        uint64_t* L = s_list[r];
        uint64_t t = wave_threshold(L, n, k, k / 4, false, s_h[wave], s_tau[r], s_max[r]);
        // no key has the pattern of -0 (score_key maps it to +0's): the next key up admits the same set
        if ((uint32_t)(t >> 32) == 0x7FFFFFFFu) t = 0x8000000000000000ull;
        wave_lds_sync();
        n = wave_compact(L, n, t);
        if (lane == 0) {
          const uint32_t kt = (uint32_t)(t >> 32);
          s_tau[r] = t;
          s_tauf[r] = kt ? __uint_as_float((kt & 0x80000000u) ? (kt & 0x7FFFFFFFu) : ~kt) : -__builtin_inff();
          s_etau[r] = ~(uint32_t)t;
        }
      }
      if (lane == 0) {
        s_base[r] = n;
        s_n[r] = n + add;
        s_add[r] = 0;
      }
    }
    lds_barrier();  // lists shrunk, places of the round's keys known
    if (wave_any) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int q = 0; q < RPL; ++q) slot[rb][q] += s_base[Tile::row(rb, q, grp)];
      uint64_t kmax[RB][RPL];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int q = 0; q < RPL; ++q) kmax[rb][q] = 0;
#pragma unroll
      for (int u = 0; u < EB; ++u) {
        const uint32_t e = e0 + (uint32_t)(u * 16 + col);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int q = 0; q < RPL; ++q)
            if (bits[rb][q] & (1u << u)) {
              const int qr = Tile::row(rb, q, grp);
              const uint32_t sl = slot[rb][q] + (uint32_t)__popc(bits[rb][q] & ((1u << u) - 1u));
              const uint64_t key = ((uint64_t)score_key(sc[u][rb][q]) << 32) | (uint64_t)(~e);
              kmax[rb][q] = key > kmax[rb][q] ? key : kmax[rb][q];
              if (sl < (uint32_t)kStreamCap) s_list[qr][sl] = key;
            }
      }
      // the group's largest key of each row (a prefix maximum over the 16
      // lanes ends in the last one) and one LDS atomic per group and row
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int q = 0; q < RPL; ++q) {
          uint64_t m = kmax[rb][q];
          m = max_u64(m, dpp_u64<0x111>(m));  // row_shr:1
          m = max_u64(m, dpp_u64<0x112>(m));  // row_shr:2
          m = max_u64(m, dpp_u64<0x114>(m));  // row_shr:4
          m = max_u64(m, dpp_u64<0x118>(m));  // row_shr:8
          if (col == 15 && m) atomicMax(&s_max[Tile::row(rb, q, grp)], m);
        }
    }
  };
  for (uint32_t base = 0; base < nv_max; base += 2 * ROUND) {
    round(K0, K1, base);
    if (base + ROUND >= nv_max) break;
    round(K1, K0, base + ROUND);
  }
  lds_barrier();  // the last round's keys are listed
  // the exact k-th key of each row, the chosen entries sorted by entry
  for (int r = wave; r < nrows; r += kStreamWaves) {
    uint64_t* L = s_list[r];
    int32_t* out = a.idx + (int64_t)(r0 + r) * a.k;
    const uint32_t n = min(s_n[r], (uint32_t)kStreamCap);
    uint32_t nc = n;
    if (n > k) {
      const uint64_t t = wave_threshold(L, n, k, 0, true, s_h[wave], s_tau[r], s_max[r]);
      wave_lds_sync();
      nc = wave_compact(L, n, t);  // == k
    }
    wave_lds_sync();
    // entries of the chosen keys behind them in the same list, padded to a power of two, sorted
    uint32_t* E = reinterpret_cast<uint32_t*>(L + kStreamMaxK);
    uint32_t P = 1;
    while (P < nc) P <<= 1;
    for (uint32_t j = (uint32_t)lane; j < P; j += 64) E[j] = j < nc ? ~(uint32_t)L[j] : 0xFFFFFFFFu;
    for (uint32_t size = 2; size <= P; size <<= 1)
      for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
        wave_lds_sync();
        for (uint32_t i = (uint32_t)lane; i < P / 2; i += 64) {
          const uint32_t x0 = 2 * stride * (i / stride) + (i % stride), x1 = x0 + stride;
          const uint32_t va = E[x0], vb = E[x1];
          if ((va > vb) == ((x0 & size) == 0)) {
            E[x0] = vb;
            E[x1] = va;
          }
        }
      }
    wave_lds_sync();
    for (uint32_t j = (uint32_t)lane; j < k; j += 64) out[j] = j < nc ? (int32_t)E[j] : -1;
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
  warm_kernargs<sizeof(IndexParams)>();
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
  warm_kernargs<sizeof(IndexParams)>();
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
  if (got == 0) {
    // inconsistent lists (nothing was emitted): the exact selection from the
    // row's scores alone
    __syncthreads();
    topk_row_scan_select<kFinThreads>(a.scores + (int64_t)r * a.max_entries, nv, (uint32_t)a.k, L.h, S, emit);
  }
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

__global__ __launch_bounds__(kRowThreads) void topk_rows(IndexParams a) {
  warm_kernargs<sizeof(IndexParams)>();
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
  // (no workspace: the streaming selection, which reads none of these)
  auto at = [&](size_t off) { return base ? base + off : nullptr; };
  a.scores = scores ? const_cast<float*>(scores) : reinterpret_cast<float*>(at(L.scores));
  a.hist = reinterpret_cast<uint32_t*>(at(L.hist));
  a.ctr = reinterpret_cast<unsigned long long*>(at(L.ctr));
  a.done = reinterpret_cast<uint32_t*>(at(L.done));
  a.sel = reinterpret_cast<int32_t*>(at(L.sel));
  a.cand = reinterpret_cast<uint64_t*>(at(L.cand));
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

// The scores and the selection of lca_csa_index_topk in one launch for calls
// with many rows per sequence and no scores requested (index_topk_rows).
// Returns false, launching nothing, where that kernel does not apply.
bool index_topk_stream_applies(int B, int Tq, int HI, int dI, int k, int64_t maxN, int dtype) {
  const bool keys = dtype == LCA_BF16 || dtype == LCA_BF16_FP8KEY || dtype == LCA_BF16_MXFP4KEY;
  return keys && rows_mode(Tq, maxN) && k <= kStreamMaxK && (HI == 1 || HI == 2 || HI == 4) && dI % 32 == 0 &&
         dI <= 256 &&
         (int64_t)B * ((Tq + kStreamRows - 1) / kStreamRows) <= INT32_MAX;
}

int launch_index_topk_stream(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                             const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w, int64_t maxN,
                             int32_t* idx, void* ws, int dtype, hipStream_t stream) {
  IndexParams a = make_params(p, omega, ikey, csa_off, q_pos, B, Tq, HI, dI, k, m, w, maxN, idx, nullptr, ws);
  const int kf = dtype == LCA_BF16_FP8KEY ? 1 : dtype == LCA_BF16_MXFP4KEY ? 2 : 0;
  const dim3 g((unsigned)(B * ((Tq + kStreamRows - 1) / kStreamRows)));
  const dim3 blk(kStreamWaves * 64);
#define LCA_STREAM2(KSv, F8)                                                                      \
  switch (HI) {                                                                                   \
    case 1: hipLaunchKernelGGL((index_topk_rows<KSv, 1, F8>), g, blk, 0, stream, a); break;      \
    case 2: hipLaunchKernelGGL((index_topk_rows<KSv, 2, F8>), g, blk, 0, stream, a); break;      \
    default: hipLaunchKernelGGL((index_topk_rows<KSv, 4, F8>), g, blk, 0, stream, a); break;     \
  }
#define LCA_STREAM(KSv)    \
  if (kf == 1) {           \
    LCA_STREAM2(KSv, 1)    \
  } else if (kf == 2) {    \
    LCA_STREAM2(KSv, 2)    \
  } else {                 \
    LCA_STREAM2(KSv, 0)    \
  }
  switch (dI / 32) {
    case 1: LCA_STREAM(1) break;
    case 2: LCA_STREAM(2) break;
    case 4: LCA_STREAM(4) break;
    default: LCA_STREAM(8) break;
  }
#undef LCA_STREAM
#undef LCA_STREAM2
  return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
}

int launch_compress(const lca_compress_stream* streams, int n, const int64_t* tok_off, const int64_t* done_len,
                    int B, float eps, int dtype, hipStream_t stream);

// The parameters of a score + append launch (index_score_append, or the
// decode front launch): the score blocks take `chunk` entries each (0: the
// score kernels' own choice).
static void fill_append_params(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                               const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w,
                               int64_t maxN, const lca_compress_stream* idx_stream, const int64_t* tok_off,
                               const int64_t* done_len, float eps, float* scores, void* ws, int cblocks,
                               IndexParams* a, AppendIdx* ap, int64_t chunk = 0) {
  *a = make_params(p, omega, ikey, csa_off, q_pos, B, Tq, HI, dI, k, m, w, maxN, nullptr, scores, ws);
  if (chunk > 0) a->chunk = (int)chunk;
  *ap = AppendIdx{};
  const lca_compress_stream& in = *idx_stream;
  ap->s.src = in.src; ap->s.logits = in.logits; ap->s.out = in.out; ap->s.ent_off = in.ent_off;
  ap->s.C = in.C; ap->s.m = in.m; ap->s.w = in.w; ap->s.per_channel = in.per_channel; ap->s.rmsnorm = in.rmsnorm;
  ap->s.key = in.out_key;
  ap->s.rope = RopeTab{};  // indexer keys are not rotated (the call rejects a rotated indexer stream)
  ap->s.src2 = in.src2;
  ap->s.logits2 = in.logits2;
  ap->s.max_entries = in.max_entries;
  ap->tok_off = tok_off;
  ap->done_len = done_len;
  ap->nsx = (int)((maxN + a->chunk - 1) / a->chunk);
  ap->nsb = ap->nsx * B;
  ap->ncb = cblocks;
  ap->B = B;
  ap->eps = eps;
}

// Whether the score + append work of a decode step can run as blocks of one
// launch (bf16 matrix-core scores of one row per sequence, or a few rows
// sharing a block; an indexer-key stream pooled over the CSA windows).
bool index_append_fusable(int dtype, int Tq, int HI, int dI, int m, int w, const lca_compress_stream* idx_stream) {
  const int kf = dtype == LCA_BF16_FP8KEY ? 1 : dtype == LCA_BF16_MXFP4KEY ? 2 : 0;
  const int in_dtype = kf ? LCA_BF16 : dtype;
  return in_dtype == LCA_BF16 && HI <= 16 && (dI == 32 || dI == 64 || dI == 128 || dI == 256) &&
         idx_stream->C == dI && idx_stream->m == m && idx_stream->w == w && (w == m || w == 2 * m) && w <= 16 &&
         (Tq == 1 || multi_rows_ok(Tq, HI));
}

// The score + append part of the decode front launch, for blocks of
// `threads` threads whose score blocks take `chunk` entries: fills the
// parameters and returns the number of blocks, or a negative status (the
// KV streams need another vector width, or the grid is too large).
int setup_front_scores(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                       const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w, int64_t maxN,
                       const lca_compress_stream* idx_stream, const lca_compress_stream* kv_streams, int n_kv,
                       const int64_t* tok_off, const int64_t* done_len, float eps, float* scores, void* ws, int dtype,
                       int threads, int64_t chunk, IndexParams* a, AppendIdx* ap, CompressParams* cp,
                       size_t* lds, int64_t* blocks) {
  *cp = CompressParams{};
  int64_t cblocks = 0;
  size_t clds = 0;
  int nv = 1;
  const int in_dtype = (dtype == LCA_BF16_FP8KEY || dtype == LCA_BF16_MXFP4KEY) ? LCA_BF16 : dtype;
  if (n_kv > 0) {
    const int rc = setup_compress(kv_streams, n_kv, tok_off, done_len, B, eps, in_dtype, threads, cp, &cblocks, &clds,
                                  &nv);
    if (rc != LCA_OK) return rc;
    if (nv != 1) return LCA_ERR_UNSUPPORTED;
  }
  fill_append_params(p, omega, ikey, csa_off, q_pos, B, Tq, HI, dI, k, m, w, maxN, idx_stream, tok_off, done_len,
                     eps, scores, ws, (int)cblocks, a, ap, chunk);
  const int tq = Tq == 1 ? 1 : Tq == 2 ? 2 : 4;
  const size_t hist_lds = (size_t)tq * kHistBins * 4;
  *lds = clds > hist_lds ? clds : hist_lds;
  *blocks = (int64_t)ap->nsb + B + cblocks;
  return LCA_OK;
}

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
  const bool fused = index_append_fusable(dtype, Tq, HI, dI, m, w, idx_stream);
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
  IndexParams a;
  AppendIdx ap;
  fill_append_params(p, omega, ikey, csa_off, q_pos, B, Tq, HI, dI, k, m, w, maxN, idx_stream, tok_off, done_len, eps,
                     scores, ws, (int)cblocks, &a, &ap);
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

// ------------------------------------------------------------------ no allocation
// The index workspace of lca_csa_index_topk_noalloc: a file-scope device
// array (each GPU the library runs on holds its own copy until the process
// ends).  Host code never passes the array's name to a kernel: its device
// address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

size_t index_noalloc_max_bytes() { return kScratchBytes; }

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];          // device address of scratch, per device
uint64_t g_scratch_layout[kMaxDevices];    // layout of the last call on the device (0: none)
}  // namespace

__global__ __launch_bounds__(256) void zero_words(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

// lca_csa_index_topk with the workspace in `scratch`: the device's address of
// the array is looked up at the first call on a device (with that device
// current); the workspace is cleared by a fill kernel at the first call and
// whenever the layout (rows, max_entries, k) differs from the last call's on
// the device, since a call leaves zero only what its own layout needs.
int launch_index_topk_noalloc(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                              const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w,
                              int64_t maxN, int32_t* idx, float* scores, int dtype, hipStream_t stream) {
  // many rows and no scores requested: the streaming selection, which keeps
  // its state in LDS and needs no workspace
  if (!scores && index_topk_stream_applies(B, Tq, HI, dI, k, maxN, dtype))
    return launch_index_topk_stream(p, omega, ikey, csa_off, q_pos, B, Tq, HI, dI, k, m, w, maxN, idx, nullptr, dtype,
                                    stream);
  const int rows = B * Tq;
  const size_t need = index_topk_workspace(rows, maxN, k);
  if (need > kScratchBytes) {
    set_error("csa_index_topk_noalloc: %zu workspace bytes needed, the static workspace holds %zu", need,
              kScratchBytes);
    return LCA_ERR_WORKSPACE;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("csa_index_topk_noalloc: no current device (or more than %d devices)", kMaxDevices);
    return LCA_ERR_HIP;
  }
  void* ws = nullptr;
  bool clear = false;
  const uint64_t layout = ((uint64_t)(uint32_t)rows << 40) ^ ((uint64_t)maxN << 13) ^ (uint64_t)(uint32_t)k ^ 1ull;
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* ptr = nullptr;
      const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !ptr) {
        set_error("csa_index_topk_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
        return LCA_ERR_HIP;
      }
      g_scratch_ptr[dev] = ptr;
    }
    ws = g_scratch_ptr[dev];
    clear = g_scratch_layout[dev] != layout;
    g_scratch_layout[dev] = layout;
  }
  if (clear) {
    const int64_t words = (int64_t)((need + 3) / 4);
    hipLaunchKernelGGL(zero_words, dim3((unsigned)std::min<int64_t>(1024, (words + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t*>(ws), words);
    if (hipPeekAtLastError() != hipSuccess) return LCA_ERR_HIP;
  }
  if (!scores && index_topk_stream_applies(B, Tq, HI, dI, k, maxN, dtype))
    return launch_index_topk_stream(p, omega, ikey, csa_off, q_pos, B, Tq, HI, dI, k, m, w, maxN, idx, ws, dtype,
                                    stream);
  int rc = launch_index_score(p, omega, ikey, csa_off, q_pos, B, Tq, HI, dI, k, m, w, maxN, scores, ws, dtype, stream);
  if (rc != LCA_OK) return rc;
  return launch_topk_select(csa_off, q_pos, B, Tq, k, m, w, maxN, idx, scores, ws, stream);
}

}  // namespace lca
