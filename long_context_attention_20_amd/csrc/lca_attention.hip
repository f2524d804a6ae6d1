// Shared-KV attention partials and the log-sum-exp merge.
//
// Pages: "DeepSeek-V4", Inference efficiency (one KV head shared by all query
// heads), Core block and Provenance 17-18 (RMSNorm on queries and compressed
// KV entries; attention sinks); "Why DeepSeek V4 Stands Apart", Core
// Architectural Innovations (sparse attention over the selected compressed
// entries, dense attention over the 128:1 entries, a 128-token window).
//
// One kernel serves three key sources:
//   DENSE   entries [0, n_visible) of a compressed cache     (HCA)
//   GATHER  the entries listed in idx (-1 = unused)          (CSA sparse)
//   WINDOW  raw rows max(0, i-W+1) .. i, RMS-normalised and   (sliding window)
//           rounded to bf16 while they are staged in LDS
// A compressed entry is key and value (K = V).
//
// Matrix-core path (bf16, H a multiple of 16): a block holds one query row and
// 64 heads.  A wave keeps normalised query heads in registers as the B operand
// of S^T = K . Qhat^T (v_mfma_f32_16x16x32_bf16: 16 entries x 16 heads x 32
// dims per instruction), runs the online softmax on the S^T accumulator
// (lane = head, 8 entries per lane), and accumulates
// O^T = V^T . P^T, whose B operand is the S^T accumulator itself once rounded
// to bf16 (the contraction index is permuted identically in A and B).  The
// 32-entry KV tile sits in LDS once, row-major (rows padded against bank
// conflicts): S^T reads it with 16-byte row reads, and the V^T operand of
// O^T comes from the same rows through ds_read_b64_tr_b16, whose 16-lane
// transpose hands lane i column i of a 4-row x 16-column block.  The next
// tile's global loads are in flight while the current tile is computed.
#include "lca_topk.h"

namespace lca {

enum { SRC_DENSE = 0, SRC_GATHER = 1, SRC_WINDOW = 2, SRC_TOPK = 3 };

// One key source of a launch; its splits take blockIdx.x in
// [block_begin, block_begin + n_split).
struct AttnSrc {
  const void* kv;       // cache rows (DENSE, GATHER) or raw rows (WINDOW)
  const int64_t* off;   // [B+1] row offsets of kv
  const int32_t* idx;   // GATHER: [rows, k]
  int32_t* idx_out;     // TOPK: [rows, k] receives the selected entries
  int kind;             // SRC_*
  int k;                // GATHER / TOPK slots per row
  int m2, w2;           // DENSE / TOPK visibility
  int W;                // WINDOW length
  int n_split;
  int block_begin;
  float* o_part;        // [n_split, rows, H, D]
  float* lse;           // [n_split, rows, H]
};

constexpr int kMaxSrc = 3;

struct AttnParams {
  const void* q;        // [rows, H, D]
  const int32_t* q_pos; // [rows]
  int Tq, H, D, rows;
  float scale, eps;
  int n_src;
  int n_x;              // splits of all sources (blocks per row and head block)
  int n_hb;             // head blocks per row (matrix-core path)
  AttnSrc s[kMaxSrc];
  TopkWs tw;            // the index workspace of a TOPK source
  int filter;           // 1: the TOPK blocks filter the scores themselves
  int tbpr;             // TOPK blocks per row (n_split * n_hb)
  // row-tiled path: every block takes all sources (one split each) and
  // writes the merged output with the sink (bf16 [rows, H, D]) instead of
  // partials
  int merge;
  const float* sink;    // [H] or NULL
  void* out;
};

constexpr int kFilterPer = 8;  // scores per thread and filter chunk
constexpr uint32_t kMaxSpins = 1u << 22;

// Source of split column bx (uniform) and the split inside it.
__device__ __forceinline__ int attn_source(const AttnParams& a, int bx, int* split) {
  int si = 0;
#pragma unroll
  for (int k = 1; k < kMaxSrc; ++k)
    if (k < a.n_src && bx >= a.s[k].block_begin) si = k;
  *split = bx - a.s[si].block_begin;
  return si;
}

// Number of keys of query row r and its first row in kv -------------------
__device__ __forceinline__ int64_t attn_keys(const AttnParams& a, const AttnSrc& s, int r, int64_t* first,
                                             int64_t* nseq_out) {
  const int b = r / a.Tq;
  const int64_t base = s.off[b];
  const int64_t nseq = s.off[b + 1] - base;
  *first = base;
  *nseq_out = nseq;
  if (s.kind == SRC_GATHER || s.kind == SRC_TOPK) return s.k;
  const int64_t i = a.q_pos[r];
  if (s.kind == SRC_DENSE) {
    int64_t n = n_windows(i + 1, s.m2, s.w2);
    return n < nseq ? n : nseq;
  }
  int64_t lo = i - s.W + 1;
  if (lo < 0) lo = 0;
  int64_t hi = i < nseq - 1 ? i : nseq - 1;
  *first = base + lo;
  return hi >= lo ? hi - lo + 1 : 0;
}

// Global row of key t (or -1 when the slot is unused or out of range).
__device__ __forceinline__ int64_t attn_row(const AttnSrc& s, int r, int64_t first, int64_t nseq, int64_t t) {
  if (s.kind == SRC_GATHER) {
    const int32_t j = s.idx[(int64_t)r * s.k + t];
    return (j < 0 || j >= nseq) ? -1 : first + j;
  }
  return first + t;
}

// ============================================================ matrix cores

constexpr int kTile = 32;       // keys per tile
constexpr int kIdxLds = 2048;   // gathered indices staged per block

typedef short s4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4_t lds_s4_t;

__device__ __forceinline__ uint4 pack_tr(const s4_t lo, const s4_t hi) {
  uint4 v;
  v.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  v.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  v.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  v.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return v;
}

// Block: 8 waves = 2 teams x 4 waves, 32 query heads of one query row, one
// key source (chosen per block).  Team t takes the tiles t, t+2, ... of the
// block's key range; in a team, wave w owns heads 16*(w%2) .. +15 and the dim
// half (w/2) of D: it computes the S^T partial over its half of D, adds its
// partner's half through LDS (same order in both, so both hold identical
// logits), runs the online softmax and accumulates O^T for its D/2 dims.  At
// the end the two teams' softmax states meet in LDS, so a block emits one
// partial for twice the keys of one team.
//
// A round costs two block barriers: tiles are double-buffered per team (a
// buffer is rewritten two rounds after it was read, with both barriers of the
// round between), the key-validity mask comes from a ballot, and window rows
// are RMS-normalised in registers before they are stored (a wave's loads of
// one tile hold whole rows).
constexpr int kAttnThreads = 512;
constexpr int kTeamThreads = 256;
constexpr int kAttnHeads = 32;      // query heads per block

// FC: filter chunks a sparse block of a TOPK source loads at its start and
// filters in one pass (2 when the row's scores give a block more than one).
template <int D, bool TOPK, int FC = 1>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_mfma(AttnParams a) {
  constexpr int DH = D / 2;                 // dims per wave
  constexpr int KS = DH / 32;               // k-steps of the S partial
  constexpr int DB = DH / 16;               // 16-dim blocks of O per wave
  constexpr int PITCH = D + 8;              // bf16 elements per LDS row
  constexpr int VPR = D / 8;                // 16-byte vectors per row (a divisor of 64)
  constexpr int LOADS = kTile * VPR / kTeamThreads;
  static_assert(LOADS * kTeamThreads == kTile * VPR, "a tile must split evenly over a team");
  constexpr int KB = KS < 2 ? KS : 2;       // k-steps per operand batch
  constexpr int OB = DB < 4 ? DB : 4;       // dim blocks per operand batch
  constexpr int TILE_ELEMS = kTile * PITCH;
  // [team][buffer] tiles; with a TOPK source the same memory first holds the
  // selection's scratch
  constexpr size_t kTileBytes = 4 * (size_t)TILE_ELEMS * 2;
  constexpr size_t kLdsBytes = (TOPK && sizeof(SelectLds) > kTileBytes) ? sizeof(SelectLds) : kTileBytes;
  __shared__ __attribute__((aligned(16))) char lds_raw[kLdsBytes];
  static_assert(!TOPK || sizeof(FilterShared) <= kLdsBytes, "the filter's LDS lives in the tile memory");
  auto tiles = reinterpret_cast<uint16_t(*)[2][TILE_ELEMS]>(lds_raw);
  __shared__ SelectShared sel_sh;
  __shared__ int32_t sidx[kIdxLds];
  __shared__ float sx[2][4][8][64];         // S partial exchange, per team
  __shared__ float qss[2][4][16];           // query sum-of-squares exchange, per team
  // 1-D grid, XCD-aware: workgroups go to the 8 XCDs round-robin by linear
  // id, so the n_hb head blocks of one (row, split) unit take ids 8 apart and
  // share an XCD's L2 for the keys they all read
  const int xcd = blockIdx.x & 7;
  const int jj = blockIdx.x >> 3;
  const int hb = jj % a.n_hb;
  const int unit = (jj / a.n_hb) * 8 + xcd;
  if (unit >= a.rows * a.n_x) return;  // padding of the last group (uniform)
  const int r = unit / a.n_x;
  int split;
  const int si = attn_source(a, unit % a.n_x, &split);
  const AttnSrc& S = a.s[si];
  const int kind = S.kind;
  const bool gather = kind == SRC_GATHER || kind == SRC_TOPK;
  // a TOPK block's selection loads go out first: they need nothing but the row
  __shared__ uint32_t s_timeout;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int team = wave >> 2, wt = wave & 3;
  const int tt = threadIdx.x & (kTeamThreads - 1);  // thread index inside the team
  const int c16 = lane & 15, g = lane >> 4;
  const int hq = wt & 1, dh = wt >> 1;
  const int hbase = hb * kAttnHeads;
  const int h0 = hbase + hq * 16;
  const bool wave_on = h0 < a.H;  // H is a multiple of 16; uniform per wave pair
  const int h = h0 + c16;
  const int d0 = dh * DH;         // first dim of this wave

  int64_t first, nseq;
  const int64_t n = attn_keys(a, S, r, &first, &nseq);
  // a TOPK block's next loads (its filter chunk, or the filtered lists) need
  // nothing but the row: they go out right after the row's position, so that
  // waiting for the position does not wait for them
  const int32_t qpos_r = kind == SRC_TOPK ? a.q_pos[r] : 0;
  SelectPrefetch<kAttnThreads> pf;
  FilterPrefetch<kAttnThreads, kFilterPer, FC> fpf;
  if constexpr (TOPK) {
    if (kind == SRC_TOPK) {
      if (a.filter)
        filter_prefetch(a.tw, r, split * a.n_hb + hb, a.tbpr, fpf);
      else
        topk_prefetch(a.tw, r, pf);
    }
  }
  const int64_t ntiles = (n + kTile - 1) / kTile;
  const int64_t tps = (ntiles + S.n_split - 1) / S.n_split;
  const int64_t tb = (int64_t)split * tps;
  const int64_t te = min(ntiles, tb + tps);
  const int64_t kbase = tb * kTile;
  const int64_t rounds = (te > tb && nseq > 0) ? (te - tb + 1) / 2 : 0;  // uniform over the block

  // --- tile staging (per team): loads are unconditional (invalid keys read a
  // clamped valid row) and zeroed when stored
  uint4 stage[LOADS];
  uint32_t okbits = 0;
  const uint16_t* kvp = reinterpret_cast<const uint16_t*>(S.kv);
  auto key_ok = [&](int64_t key) -> bool {
    if (key >= n) return false;
    return !gather || sidx[key - kbase] >= 0;
  };
  auto load_tile = [&](int64_t t) {
    okbits = 0;
    if (t >= te) return;
#pragma unroll
    for (int v = 0; v < LOADS; ++v) {
      const int id = tt + kTeamThreads * v;
      const int row = id / VPR, vec = id % VPR;
      const int64_t key = t * kTile + row;
      bool ok = key < n;
      int64_t off;
      if (gather) {
        const int32_t j = ok ? sidx[key - kbase] : -1;
        ok = j >= 0;
        off = ok ? j : 0;
      } else {
        off = ok ? key : 0;
      }
      okbits |= (ok ? 1u : 0u) << v;
      stage[v] = *reinterpret_cast<const uint4*>(kvp + (first + off) * D + vec * 8);
    }
  };
  auto store_tile = [&](uint16_t* tile) {
    if (kind == SRC_WINDOW) {
      // RMS-normalise each row over D: the VPR lanes holding a row are
      // consecutive lanes of one wave
#pragma unroll
      for (int v = 0; v < LOADS; ++v) {
        float f[8];
        BF16::unpack(stage[v], f);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
        ss = lane_group_sum<VPR>(ss);
        const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] *= inv;
        stage[v] = BF16::pack(f);
      }
    }
#pragma unroll
    for (int v = 0; v < LOADS; ++v) {
      const int id = tt + kTeamThreads * v;
      const int row = id / VPR, vec = id % VPR;
      const bool ok = (okbits >> v) & 1u;
      *reinterpret_cast<uint4*>(&tile[row * PITCH + vec * 8]) = ok ? stage[v] : make_uint4(0, 0, 0, 0);
    }
  };

  // --- prologue: the query (and, for gathered keys, the block's indices) in
  // one memory round trip; dense and window keys do not depend on staged
  // indices, so their first tile is requested first
  if (!gather && rounds > 0) load_tile(tb + team);
  uint4 qraw[KS];
  if (wave_on) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)r * a.H + h) * D + d0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qraw[ks] = *reinterpret_cast<const uint4*>(qp + ks * 32 + g * 8);
  }
  if (kind == SRC_GATHER && rounds > 0) {
    const int64_t cnt = min((te - tb) * kTile, n - kbase);
    for (int i = threadIdx.x; i < cnt; i += kAttnThreads) {
      const int32_t j = S.idx[(int64_t)r * S.k + kbase + i];
      sidx[i] = (j < 0 || j >= nseq) ? -1 : j;
    }
  }
  if constexpr (TOPK) {
    const TopkWs& tw = a.tw;
    const int64_t nv = kind == SRC_TOPK ? topk_visible(qpos_r, S.m2, S.w2, nseq, tw.max_entries) : 0;
    const bool all = nv <= S.k;  // every visible entry, in order
    bool ready = true;
    if (kind == SRC_TOPK && a.filter && !all) {
      // every TOPK block of the row (slots or not) filters its share of the
      // row's scores, then counts itself done and waits for the others.  The
      // launch fits the machine at once, so they are all resident and the
      // wait ends (bounded all the same: a count that never completes leaves
      // the slots empty rather than hanging).
      // the block's chunks are tbi, tbi + tbpr, ...; the first FC of them had
      // their loads issued at the start and are filtered in one pass (one
      // threshold, one list reservation)
      const int tbi = split * a.n_hb + hb;
      constexpr int64_t CH = (int64_t)kAttnThreads * kFilterPer;
      for (int64_t cb = tbi; cb * CH < nv; cb += (int64_t)a.tbpr * FC) {
        if (cb != tbi) filter_prefetch(tw, r, (int)cb, a.tbpr, fpf);
        filter_chunk(tw, r, nv, (int)cb, a.tbpr, fpf, *reinterpret_cast<FilterShared*>(lds_raw));
        __syncthreads();
      }
      if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(&tw.done[r], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t spins = 0;
        while (__hip_atomic_load(&tw.done[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)a.tbpr &&
               ++spins < kMaxSpins)
          __builtin_amdgcn_s_sleep(1);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_timeout = spins >= kMaxSpins;
      }
      __syncthreads();
      ready = !s_timeout;
      topk_prefetch(tw, r, pf);  // the lists are complete now
    }
    if (kind == SRC_TOPK && te > tb) {  // the block owns slots (even of an empty row)
      // this block's slots [kbase, kbase + cnt) of the row's top k in
      // ascending entry order: every block of the row runs the same exact
      // selection from the filtered lists; the head-block-0 blocks also
      // write their slots to idx_out
      const int64_t cnt = min((te - tb) * kTile, n - kbase);
      if (split == 0 && hb == 0) {
        // every filter of the row has read the first histogram: clear it for
        // the next call
        uint32_t* gh = tw.hist + (int64_t)r * tw.nstripe * kHistBins;
        for (int i = threadIdx.x; i < tw.nstripe * kHistBins; i += kAttnThreads) gh[i] = 0;
      }
      for (int i = threadIdx.x; i < cnt; i += kAttnThreads) sidx[i] = (all && kbase + i < nv) ? (int32_t)(kbase + i) : -1;
      // the tile memory beyond the selection's scratch keeps candidates the
      // selection reads more than once (8192 of them at D = 512)
      constexpr uint32_t kCandLds = (uint32_t)((kLdsBytes - sizeof(SelectLds)) / sizeof(uint64_t));
      static_assert(sizeof(SelectLds) % sizeof(uint64_t) == 0, "the candidate area must be 8-byte aligned");
      if (!all && ready)
        topk_row_select<kAttnThreads, true>(tw, r, pf, *reinterpret_cast<SelectLds*>(lds_raw), sel_sh,
                                            [&](uint32_t o, int32_t e) {
                                              const int64_t j = (int64_t)o - kbase;
                                              if (j >= 0 && j < cnt) sidx[j] = e;
                                            },
                                            reinterpret_cast<uint64_t*>(lds_raw + sizeof(SelectLds)), kCandLds);
      __syncthreads();  // sidx complete; the selection's scratch is free
      if (hb == 0 && S.idx_out)
        for (int i = threadIdx.x; i < cnt; i += kAttnThreads) S.idx_out[(int64_t)r * S.k + kbase + i] = sidx[i];
    }
  }
  {
    float ss = 0.f;
    if (wave_on) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float f[8];
        BF16::unpack(qraw[ks], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
      }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    if (g == 0) qss[team][wt][c16] = ss;
  }
  __syncthreads();  // sidx and qss ready
  if (gather && rounds > 0) load_tile(tb + team);
  bf16x8_t qb[KS];
  if (wave_on) {
    const float ss = qss[team][hq][c16] + qss[team][hq + 2][c16];
    const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.eps);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float f[8];
      BF16::unpack(qraw[ks], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= inv;
      qb[ks] = __builtin_bit_cast(bf16x8_t, BF16::pack(f));
    }
  }

  f32x4 O[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) O[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;

  for (int64_t rd = 0; rd < rounds; ++rd) {
    const int64_t t = tb + 2 * rd + team;   // this team's tile (may be past te)
    const bool active = t < te;
    uint16_t* tile = tiles[team][rd & 1];
    store_tile(tile);
    // validity of the tile's 32 keys, one per lane of the low half-wave
    const uint64_t vm = __ballot(lane < kTile && active && key_ok(t * kTile + lane));
    __syncthreads();  // A: tile in LDS
    load_tile(t + 2);
    // ---- S^T partial over this wave's dims, entries 0-15 (s0) and 16-31 (s1)
    f32x4 s0a = {0.f, 0.f, 0.f, 0.f}, s0b = s0a, s1a = s0a, s1b = s0a;
    if (wave_on && active) {
      const uint16_t* krow0 = &tile[c16 * PITCH + d0 + g * 8];
      const uint16_t* krow1 = krow0 + 16 * PITCH;
      uint4 kbuf[2][KB][2];
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        kbuf[0][j][0] = *reinterpret_cast<const uint4*>(krow0 + j * 32);
        kbuf[0][j][1] = *reinterpret_cast<const uint4*>(krow1 + j * 32);
      }
#pragma unroll
      for (int bi = 0; bi < KS / KB; ++bi) {
        const int cur = bi & 1;
        if (bi + 1 < KS / KB) {
#pragma unroll
          for (int j = 0; j < KB; ++j) {
            kbuf[cur ^ 1][j][0] = *reinterpret_cast<const uint4*>(krow0 + ((bi + 1) * KB + j) * 32);
            kbuf[cur ^ 1][j][1] = *reinterpret_cast<const uint4*>(krow1 + ((bi + 1) * KB + j) * 32);
          }
        }
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          const int ks = bi * KB + j;
          if (j & 1) {
            s0b = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kbuf[cur][j][0]), qb[ks], s0b, 0, 0, 0);
            s1b = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kbuf[cur][j][1]), qb[ks], s1b, 0, 0, 0);
          } else {
            s0a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kbuf[cur][j][0]), qb[ks], s0a, 0, 0, 0);
            s1a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kbuf[cur][j][1]), qb[ks], s1a, 0, 0, 0);
          }
        }
      }
    }
    const f32x4 p0 = s0a + s0b, p1 = s1a + s1b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sx[team][wt][i][lane] = p0[i];
      sx[team][wt][4 + i][lane] = p1[i];
    }
    __syncthreads();  // B: S partials exchanged
    if (wave_on && active) {
      float lg[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s0 = sx[team][hq][i][lane] + sx[team][hq + 2][i][lane];
        const float s1 = sx[team][hq][4 + i][lane] + sx[team][hq + 2][4 + i][lane];
        lg[i] = ((vm >> (4 * g + i)) & 1u) ? s0 * sl2 : -INFINITY;
        lg[4 + i] = ((vm >> (16 + 4 * g + i)) & 1u) ? s1 * sl2 : -INFINITY;
      }
      float tmax = lg[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, lg[i]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      if (tmax != -INFINITY) {  // uniform: masks do not depend on the head
        // the reference max moves only when a logit exceeds it by more than
        // 8 (log2 units): p <= 256, and the rescale of O is rare
        const bool move = tmax > m_run + 8.0f;  // true on the first valid tile
        const float alpha = move ? exp2f(m_run - tmax) : 1.0f;
        const float m_ref = move ? tmax : m_run;
        float p[8], psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = exp2f(lg[i] - m_ref);
          psum += p[i];
        }
        l_run = l_run * alpha + psum;
        m_run = m_ref;
        if (__ballot(alpha != 1.0f)) {
#pragma unroll
          for (int db = 0; db < DB; ++db) O[db] = O[db] * alpha;
        }
        uint4 pb;
        pb.x = pack_bf16x2(p[0], p[1]);
        pb.y = pack_bf16x2(p[2], p[3]);
        pb.z = pack_bf16x2(p[4], p[5]);
        pb.w = pack_bf16x2(p[6], p[7]);
        const bf16x8_t pt = __builtin_bit_cast(bf16x8_t, pb);
        // ---- O^T += V^T . P^T over this wave's dims; the V^T operand of lane
        // c16 in group g holds entries 4g..4g+3 and 16+4g..16+4g+3 at dim
        // d0 + 16*db + c16: it addresses row 4g + c16/4 (and 16 + ...) at
        // columns d0 + 16*db + 4*(c16%4); the transpose read returns its column.
        const uint16_t* trow0 = &tile[(4 * g + (c16 >> 2)) * PITCH + d0 + 4 * (c16 & 3)];
        const uint16_t* trow1 = trow0 + 16 * PITCH;
        s4_t vbuf[2][OB][2];
#pragma unroll
        for (int j = 0; j < OB; ++j) {
          vbuf[0][j][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t*)(trow0 + j * 16));
          vbuf[0][j][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t*)(trow1 + j * 16));
        }
#pragma unroll
        for (int bi = 0; bi < DB / OB; ++bi) {
          const int cur = bi & 1;
          if (bi + 1 < DB / OB) {
#pragma unroll
            for (int j = 0; j < OB; ++j) {
              vbuf[cur ^ 1][j][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t*)(trow0 + ((bi + 1) * OB + j) * 16));
              vbuf[cur ^ 1][j][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t*)(trow1 + ((bi + 1) * OB + j) * 16));
            }
          }
#pragma unroll
          for (int j = 0; j < OB; ++j) {
            const int db = bi * OB + j;
            O[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, pack_tr(vbuf[cur][j][0], vbuf[cur][j][1])), pt, O[db], 0, 0, 0);
          }
        }
      }
    }
  }

  // --- epilogue: the teams' softmax states meet in LDS; each wave writes its
  // O scaled by its team's weight into a per-team [head][dim] buffer (in the
  // free tile memory), and the block stores the sum of the two as one
  // contiguous run of 32 heads x D floats
  __shared__ float st_m[2][2][16], st_l[2][2][16];
  __syncthreads();  // every wave has left the last round: tiles and sx are free
  {
    float lg = l_run + __shfl_xor(l_run, 16, 64);
    lg += __shfl_xor(lg, 32, 64);
    if (dh == 0 && g == 0) {
      st_m[team][hq][c16] = m_run;
      st_l[team][hq][c16] = lg;
    }
  }
  __syncthreads();
  constexpr int XP = D + 4;  // floats per head row of the exchange buffers
  static_assert(2 * kAttnHeads * XP * 4 <= 4 * TILE_ELEMS * 2, "epilogue buffers exceed the tile memory");
  float* ox = reinterpret_cast<float*>(&tiles[0][0][0]);  // [team][32 heads][XP]
  auto head_state = [&](int hh, float* M, float* f0, float* f1, float* lsum) {
    const int q2 = hh >> 4, c = hh & 15;
    const float m0 = st_m[0][q2][c], m1 = st_m[1][q2][c];
    *M = fmaxf(m0, m1);
    *f0 = *M == -INFINITY ? 0.f : exp2f(m0 - *M);
    *f1 = *M == -INFINITY ? 0.f : exp2f(m1 - *M);
    *lsum = st_l[0][q2][c] * *f0 + st_l[1][q2][c] * *f1;
  };
  {
    float M, f0, f1, lsum;
    head_state(hq * 16 + c16, &M, &f0, &f1, &lsum);
    const float w = lsum > 0.f ? (team ? f1 : f0) / lsum : 0.f;
    float* xp = ox + (team * kAttnHeads + hq * 16 + c16) * XP + d0 + 4 * g;
    // lane (head c16, g) holds dims d0 + 16*db + 4g .. +3
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<float4*>(xp + db * 16) = make_float4(O[db][0] * w, O[db][1] * w, O[db][2] * w, O[db][3] * w);
  }
  __syncthreads();
  const int nh = min(kAttnHeads, a.H - hbase);
  float* op = S.o_part + (((int64_t)split * a.rows + r) * a.H + hbase) * D;
  for (int i = threadIdx.x; i < nh * (D / 4); i += kAttnThreads) {
    const int hh = i / (D / 4), d = (i % (D / 4)) * 4;
    const float4 u = *reinterpret_cast<const float4*>(ox + hh * XP + d);
    const float4 v = *reinterpret_cast<const float4*>(ox + (kAttnHeads + hh) * XP + d);
    *reinterpret_cast<float4*>(op + (int64_t)i * 4) = make_float4(u.x + v.x, u.y + v.y, u.z + v.z, u.w + v.w);
  }
  if (threadIdx.x < nh) {
    float M, f0, f1, lsum;
    head_state(threadIdx.x, &M, &f0, &f1, &lsum);
    S.lse[((int64_t)split * a.rows + r) * a.H + hbase + threadIdx.x] =
        lsum > 0.f ? (M + __log2f(lsum)) * kLn2 : -INFINITY;
  }
}

// ============================================================ many query rows
// Attention for calls with many query rows per sequence (prefill chunks),
// D = 512, bf16: a block holds 128 (query, head) rows -- 8 waves of 16 heads
// of one query each, 128 / H queries -- and streams one source's keys through
// LDS in 32-key tiles (double-buffered, one barrier per tile, the next tile's
// key rows moved straight from global memory into LDS while the current one
// is computed).  A wave keeps its 16 normalised query rows over all of D in
// registers as the B operand of S^T = K . Qhat^T, runs the online softmax on
// the S^T accumulator and accumulates O^T = V^T . P^T for all of D (V^T
// through ds_read_b64_tr_b16, the P^T operand the rounded accumulator itself,
// as in attn_mfma), so no logits are exchanged between waves.  The block's
// queries share the tiles of a dense source (the union of what they see) and
// of a window source (the union of their windows, each row RMS-normalised in
// LDS by the wave that loaded it); a gathered source gives every query its
// own stream of tiles (two streams at most: H = 64 or 128).  Each wave masks
// the keys its own query does not see.  A source's splits cut the block's key
// range into n_split parts, one partial each.
constexpr int kRowsThreads = 512;
constexpr int kRowsTile = 32;
constexpr int kRowsBlockRows = 128;  // (query, head) rows per block
constexpr int kRowsStreams = 2;      // gathered streams (queries) per block at most
constexpr int kRowsIdx = 1024;       // gathered slots per stream and split

// LDS rows of the row-tiled kernel are 1 KiB with no padding; the 16-byte
// chunk c of tile row r sits at chunk c ^ rows_swz(r).  The swizzle keeps
// both read patterns free of bank conflicts, for 32 banks (8 lanes per cycle
// of a 16-byte read, 16 of an 8-byte one) and for 64 (16 and 32): the K-row
// reads (16 rows, one chunk each) see rows_swz(r) distinct mod 16 over 16
// consecutive rows and mod 8 over 8 aligned ones; the transposed V reads (4 or
// 8 rows, two neighbouring chunks each) see rows_swz(r) >> 1 distinct over 4
// or 8 aligned rows.
// One wave moves 64 x 16 bytes from global memory straight into LDS: lane
// l's 16 bytes at its own address gsrc land at LDS byte offset lds + 16 l
// (lds uniform).  Issued as assembly so that the compiler does not make later
// LDS reads of the other tile buffer wait for it; the caller waits for the
// load (s_waitcnt vmcnt) and synchronises the block before the data is read
// or overwritten.  The instruction has no register result.
__device__ __forceinline__ void lds_dma16(const void* gsrc, const void* lds_dst) {
  const uint32_t lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_dst);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gsrc), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ int rows_swz(int r) {
  return (((r >> 2) & 1) << 3) | ((r & 3) << 1) | (((r >> 2) ^ (r >> 3)) & 1);
}

// Wave-uniform 64-bit value in scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <bool MERGE>
__global__ __launch_bounds__(kRowsThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_rows_mfma(AttnParams a) {
  constexpr int D = 512;
  constexpr int KS = D / 32;      // k-steps of S over D
  constexpr int DB = D / 16;      // 16-dim blocks of O
  constexpr int PITCH = D;        // bf16 elements per LDS row (chunks swizzled, no padding)
  constexpr int TILE_ELEMS = kRowsTile * PITCH;
  __shared__ __attribute__((aligned(16))) uint16_t tiles[kRowsStreams][2][TILE_ELEMS];
  __shared__ int32_t sidx[kRowsStreams][kRowsIdx];
  __shared__ int64_t s_lo[kRowsThreads / 64], s_hi[kRowsThreads / 64];
  const int lane = threadIdx.x & 63;
  // the wave index in a scalar register: everything derived from it (rows,
  // key ranges, addresses) stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  // block -> (sequence b, row tile, source split), or (b, row tile) with
  // every source in turn when the block also merges; a sequence's rows are
  // (t, h) -> t*H + h
  const int64_t rows_seq = (int64_t)a.Tq * a.H;
  const int64_t tiles_seq = (rows_seq + kRowsBlockRows - 1) / kRowsBlockRows;
  const int bx = MERGE ? 0 : (int)(blockIdx.x % a.n_x);
  const int64_t rest = MERGE ? (int64_t)blockIdx.x : (int64_t)(blockIdx.x / a.n_x);
  const int b = (int)(rest / tiles_seq);
  const int64_t rt = rest % tiles_seq;
  const int64_t rr = rt * kRowsBlockRows + wave * 16;  // this wave's first row
  const bool wave_on = rr < rows_seq;                  // uniform per wave (H divides 128)
  const int t = wave_on ? (int)(rr / a.H) : 0;
  const int h0 = (int)(rr % a.H);
  const int r = b * a.Tq + t;
  const int nq = kRowsBlockRows / a.H;                 // queries per block

  // the query rows, RMS-normalised over D and rounded to bf16: lane (c16, g)
  // holds head h0 + c16, dims 32*ks + 8*g .. +7
  bf16x8_t qb[KS];
  {
    uint4 qraw[KS];
    if (wave_on) {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)r * a.H + h0 + c16) * D + g * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qraw[ks] = *reinterpret_cast<const uint4*>(qp + ks * 32);
    }
    float ss = 0.f;
    if (wave_on) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float f[8];
        BF16::unpack(qraw[ks], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
      }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.eps);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float f[8];
      BF16::unpack(qraw[ks], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= inv;
      qb[ks] = __builtin_bit_cast(bf16x8_t, BF16::pack(f));
    }
  }

  // one online softmax over every key the block's sources give (one source,
  // or all of them in turn when the block merges)
  f32x4 O[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) O[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;
  int split = 0, si = 0;
  for (int sl = 0; sl < (MERGE ? a.n_src : 1); ++sl) {
    if (MERGE)
      si = sl;
    else
      si = attn_source(a, bx, &split);
    const AttnSrc& S = a.s[si];
    const int kind = S.kind;
    const int streams = kind == SRC_GATHER ? nq : 1;
    const int stream = kind == SRC_GATHER ? (wave * 16) / a.H : 0;
    const int wps = (kRowsThreads / 64) / streams;       // waves per stream
    const int wis = wave % wps;                          // this wave's place in its stream
    const int64_t first = S.off[b];
    const int64_t nseq = S.off[b + 1] - first;
    // this wave's visible key range [lo, hi) in the source's key coordinates:
    // entries (dense), token positions (window), slots (gathered)
    int64_t lo = 0, hi = 0;
    if (wave_on) {
      if (kind == SRC_DENSE) {
        const int64_t nh = n_windows((int64_t)a.q_pos[r] + 1, S.m2, S.w2);
        hi = nh < nseq ? nh : nseq;
      } else if (kind == SRC_WINDOW) {
        const int64_t i = a.q_pos[r];
        lo = i - S.W + 1 > 0 ? i - S.W + 1 : 0;
        hi = (i < nseq - 1 ? i : nseq - 1) + 1;
        if (hi < lo) hi = lo;
      } else {
        hi = nseq > 0 ? S.k : 0;
      }
    }
    // the previous source's readers of s_lo / s_hi, sidx and the tiles are done
    __syncthreads();
    lo = uniform64(lo);
    hi = uniform64(hi);
    if (lane == 0) {
      // an empty range adds nothing to the block's union (a window past the
      // sequence's last token has hi == lo > nseq)
      s_lo[wave] = wave_on && hi > lo ? lo : INT64_MAX;
      s_hi[wave] = wave_on && hi > lo ? hi : 0;
    }
    __syncthreads();  // s_lo, s_hi
    // the block's key range (per stream for gathered keys: every stream has k slots)
    int64_t blo = INT64_MAX, bhi = 0;
#pragma unroll
    for (int w = 0; w < kRowsThreads / 64; ++w) {
      blo = s_lo[w] < blo ? s_lo[w] : blo;
      bhi = s_hi[w] > bhi ? s_hi[w] : bhi;
    }
    if (blo > bhi) blo = bhi;  // nothing visible
    const int64_t ntiles = (bhi - blo + kRowsTile - 1) / kRowsTile;
    const int64_t tps = (ntiles + S.n_split - 1) / S.n_split;
    const int64_t tb = (int64_t)split * tps;
    const int64_t te = min(ntiles, tb + tps);
    const int64_t kbase = blo + tb * kRowsTile;  // key coordinate of the split's first tile row
    if (kind == SRC_GATHER && te > tb) {
      // every stream's slots of this split, -1 for unused or out-of-range entries
      const int64_t cnt = min((te - tb) * kRowsTile, bhi - kbase);
      const int q0 = (int)((rt * kRowsBlockRows) / a.H);
      for (int i = threadIdx.x; i < streams * kRowsIdx; i += kRowsThreads) {
        const int st = i / kRowsIdx, j = i % kRowsIdx;
        const int tq = q0 + st;
        int32_t e = -1;
        if (j < cnt && tq < a.Tq) {
          e = S.idx[(int64_t)(b * a.Tq + tq) * S.k + kbase + j];
          if (e < 0 || e >= nseq) e = -1;
        }
        sidx[st][j] = e;
      }
    }

    __syncthreads();  // sidx

    // tile staging: one wave instruction moves one 1 KiB key row straight into
    // LDS; wave w loads rows wis*rpw .. of its stream's tile.  Rows without a
    // visible key load a clamped valid row (their logits are masked, so they
    // weigh nothing).
    const uint16_t* kvp = reinterpret_cast<const uint16_t*>(S.kv);
    const int rpw = kRowsTile / wps;  // rows per wave: 4 (one stream) or 8 (two)
    auto load_tile = [&](int64_t tt) {
      if (tt >= te) return;
      uint16_t* tile = tiles[stream][(tt - tb) & 1];
      for (int v = 0; v < rpw; ++v) {  // uniform
        const int row = wis * rpw + v;
        const int64_t kc = blo + tt * kRowsTile + row;
        int64_t ent;
        if (kind == SRC_GATHER) {
          const int32_t e = sidx[stream][kc - kbase];
          ent = e >= 0 ? e : 0;
        } else {
          ent = kc < bhi ? kc : blo;
        }
        // lane l fills LDS chunk l with the row's chunk l ^ rows_swz(row)
        const uint16_t* src = kvp + (first + ent) * D + ((lane ^ rows_swz(row)) * 8);
        lds_dma16(src, tile + row * PITCH);
      }
    };
    // window rows: RMS over D of the raw row, rounded to bf16, in place (the
    // wave that loaded a row normalises it once its loads have landed; the
    // chunk order within the row does not matter here)
    auto norm_rows = [&](int64_t tt) {
      uint16_t* tile = tiles[0][(tt - tb) & 1];
      for (int v = 0; v < rpw; ++v) {
        uint16_t* rowp = tile + (wis * rpw + v) * PITCH + lane * 8;
        uint4 x = *reinterpret_cast<const uint4*>(rowp);
        float f[8];
        BF16::unpack(x, f);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
        ss = lane_group_sum<64>(ss);
        const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] *= inv;
        *reinterpret_cast<uint4*>(rowp) = BF16::pack(f);
      }
    };

    load_tile(tb);
    for (int64_t tt = tb; tt < te; ++tt) {
      __builtin_amdgcn_s_waitcnt(0);  // this wave's rows of the tile have landed
      if (kind == SRC_WINDOW) norm_rows(tt);
      // tile in LDS; every wave has left the previous tile, whose buffer the
      // next loads overwrite
      __syncthreads();
      load_tile(tt + 1);
      const uint16_t* tile = tiles[stream][(tt - tb) & 1];
      const int64_t k0 = blo + tt * kRowsTile;  // key coordinate of the tile's first row
      // the tile's rows this wave sees, one per lane of the low half-wave
      const int64_t kl = k0 + lane;
      const uint64_t vm = __ballot(lane < kRowsTile && kl >= lo && kl < hi &&
                                   (kind != SRC_GATHER || sidx[stream][kl - kbase] >= 0));
      if (wave_on && vm != 0) {  // uniform per wave
        // ---- S^T for tile rows 0..15 (p0) and 16..31 (p1)
        f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0;
        // rows c16 and 16 + c16 (same swizzle), logical chunk 4 ks + g: with
        // ks = 4j + i the physical chunk is 16j + ((4i + g) ^ swz), four
        // per-lane offsets and an immediate.  The swizzle goes through an empty
        // asm so that the offsets are formed here, not held over the loop.
        int sk = rows_swz(c16);
        asm volatile("" : "+v"(sk));
        int koff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) koff[i] = c16 * PITCH + ((4 * i + g) ^ sk) * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint16_t* k0p = tile + koff[ks & 3] + (ks >> 2) * 128;
          const uint4 a0 = *reinterpret_cast<const uint4*>(k0p);
          const uint4 a1 = *reinterpret_cast<const uint4*>(k0p + 16 * PITCH);
          p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0), qb[ks], p0, 0, 0, 0);
          p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1), qb[ks], p1, 0, 0, 0);
        }
        // ---- online softmax: lane (c16 = head, g) holds tile rows 4g+i and 16+4g+i
        float lg[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lg[i] = ((vm >> (4 * g + i)) & 1u) ? p0[i] * sl2 : -INFINITY;
          lg[4 + i] = ((vm >> (16 + 4 * g + i)) & 1u) ? p1[i] * sl2 : -INFINITY;
        }
        float tmax = lg[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, lg[i]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        if (tmax != -INFINITY) {  // uniform: the masks do not depend on the head
          const bool move = tmax > m_run + 8.0f;
          const float alpha = move ? exp2f(m_run - tmax) : 1.0f;
          const float m_ref = move ? tmax : m_run;
          float pr[8], psum = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            pr[i] = exp2f(lg[i] - m_ref);
            psum += pr[i];
          }
          l_run = l_run * alpha + psum;
          m_run = m_ref;
          if (__ballot(alpha != 1.0f)) {
#pragma unroll
            for (int db = 0; db < DB; ++db) O[db] = O[db] * alpha;
          }
          uint4 pb;
          pb.x = pack_bf16x2(pr[0], pr[1]);
          pb.y = pack_bf16x2(pr[2], pr[3]);
          pb.z = pack_bf16x2(pr[4], pr[5]);
          pb.w = pack_bf16x2(pr[6], pr[7]);
          const bf16x8_t pt = __builtin_bit_cast(bf16x8_t, pb);
          // ---- O^T += V^T . P^T: lane c16 of group g reads rows 4g + c16/4 (and
          // 16 + ...) at columns 16*db + 4*(c16%4); the transpose read returns
          // dim 16*db + c16 of tile rows 4g..4g+3 (and 16+4g..)
          // (logical chunk 2 db + bit 1 of c16, half c16 & 1; rows 4g + c16/4
          // and 16 + 4g + c16/4 share the swizzle)
          // (with db = 8j + i the physical chunk is 16j + ((2i + hh) ^ swz):
          // eight per-lane offsets and an immediate)
          const int tr_r = 4 * g + (c16 >> 2);
          int st = rows_swz(tr_r);
          asm volatile("" : "+v"(st));
          const int hh = (c16 >> 1) & 1;
          int toff[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) toff[i] = tr_r * PITCH + 4 * (c16 & 1) + ((2 * i + hh) ^ st) * 8;
#pragma unroll
          for (int db = 0; db < DB; db += 2) {
            const uint16_t* t0 = tile + toff[db & 7] + (db >> 3) * 128;
            const uint16_t* t1 = tile + toff[(db + 1) & 7] + ((db + 1) >> 3) * 128;
            const s4_t v00 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t*)t0);
            const s4_t v01 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t*)(t0 + 16 * PITCH));
            const s4_t v10 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t*)t1);
            const s4_t v11 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t*)(t1 + 16 * PITCH));
            O[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, pack_tr(v00, v01)), pt, O[db],
                                                            0, 0, 0);
            O[db + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, pack_tr(v10, v11)), pt,
                                                                O[db + 1], 0, 0, 0);
          }
        }
      }
    }

  }  // sources

  // ---- epilogue: lane (c16, g) holds dims 16*db + 4g .. +3 of head h0 + c16
  if (!wave_on) return;
  float lsum = l_run + __shfl_xor(l_run, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (MERGE) {
    // the sink (zero value) joins the denominator: out = O / (l + e^(sink - m))
    float den = lsum;
    if (a.sink && m_run != -INFINITY) den += exp2f(a.sink[h0 + c16] * kLog2e - m_run);
    const float w = den > 0.f ? 1.0f / den : 0.f;
    uint16_t* outp = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)r * a.H + h0 + c16) * D + 4 * g;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      uint2 pk;
      pk.x = pack_bf16x2(O[db][0] * w, O[db][1] * w);
      pk.y = pack_bf16x2(O[db][2] * w, O[db][3] * w);
      *reinterpret_cast<uint2*>(outp + db * 16) = pk;
    }
    return;
  }
  const AttnSrc& S = a.s[si];
  const float w = lsum > 0.f ? 1.0f / lsum : 0.f;
  const int64_t orow = ((int64_t)split * a.rows + r) * a.H + h0 + c16;
  float* op = S.o_part + orow * D + 4 * g;
#pragma unroll
  for (int db = 0; db < DB; ++db)
    *reinterpret_cast<float4*>(op + db * 16) = make_float4(O[db][0] * w, O[db][1] * w, O[db][2] * w, O[db][3] * w);
  if (g == 0) S.lse[orow] = lsum > 0.f ? (m_run + __log2f(lsum)) * kLn2 : -INFINITY;
}

// Row-tiled attention, two head groups per wave.  The same block shape and
// key staging as attn_rows_mfma (128 rows, 32-key tiles through swizzled LDS
// rows), but four waves of 32 rows each, one wave per SIMD with the whole
// register file: every K fragment read from LDS feeds the S^T products of both
// 16-head groups and every V^T fragment both O^T products, so a wave does
// twice the matrix work per LDS byte, and the accumulators of O^T (2 x 16 x D
// floats) live in the accumulation registers while the architectural ones
// hold the queries and the fragments in flight.
// ============================================================ generic path
// One wavefront per (query row, head, split); a lane owns D/64 dims.  Used for
// fp32 and for bf16 head counts that are not a multiple of 16.
template <typename ET, int DPL>
__global__ __launch_bounds__(64) void attn_valu(AttnParams a) {
  const int r = blockIdx.z;
  const int h = blockIdx.y;
  int split;
  const AttnSrc& S = a.s[attn_source(a, blockIdx.x, &split)];
  const int lane = threadIdx.x;
  const int D = a.D;
  int64_t first, nseq;
  const int64_t n = attn_keys(a, S, r, &first, &nseq);
  const int64_t per = (n + S.n_split - 1) / S.n_split;
  const int64_t kb = (int64_t)split * per;
  const int64_t ke = min(n, kb + per);

  float qh[DPL];
  {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      qh[i] = ET::load1(a.q, ((int64_t)r * a.H + h) * D + lane * DPL + i);
      ss = fmaf(qh[i], qh[i], ss);
    }
    ss = wave_sum(ss, 64);
    const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
    for (int i = 0; i < DPL; ++i) qh[i] = ET::round(qh[i] * inv);
  }
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  for (int64_t t = kb; t < ke; ++t) {
    const int64_t row = attn_row(S, r, first, nseq, t);
    if (row < 0) continue;
    float kv[DPL];
    float dot = 0.f, ss = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      kv[i] = ET::load1(S.kv, row * D + lane * DPL + i);
      ss = fmaf(kv[i], kv[i], ss);
    }
    if (S.kind == SRC_WINDOW) {
      ss = wave_sum(ss, 64);
      const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
      for (int i = 0; i < DPL; ++i) kv[i] = ET::round(kv[i] * inv);
    }
#pragma unroll
    for (int i = 0; i < DPL; ++i) dot = fmaf(qh[i], kv[i], dot);
    dot = wave_sum(dot, 64) * a.scale;
    const float m_new = fmaxf(m_run, dot);
    const float alpha = expf(m_run - m_new);
    const float p = expf(dot - m_new);
    l_run = l_run * alpha + p;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] = fmaf(o[i], alpha, p * kv[i]);
  }
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  float* op = S.o_part + (((int64_t)split * a.rows + r) * a.H + h) * D;
#pragma unroll
  for (int i = 0; i < DPL; ++i) op[lane * DPL + i] = o[i] * inv;
  if (lane == 0) S.lse[((int64_t)split * a.rows + r) * a.H + h] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
}

// ============================================================ merge
// out[r, h, :] = sum_s exp(lse_s - lse) * o_s,  lse = log(sum_s exp(lse_s) + exp(sink_h)).
// A block owns HPB (row, head) pairs; D/4 threads per pair, 4 dims each.  The
// slot weights of a pair are computed once into LDS.
constexpr int kMaxParts = 8;
constexpr int kMaxSlots = 512;
struct MergeParams {
  const float* o[kMaxParts];
  const float* lse[kMaxParts];
  int n_split[kMaxParts];
  int n_parts;
  int n_slots;
  const float* sink;
  int rows, H, D;
  void* out;
};

// One block per (row, head, 256-dim part): 256 threads = 4 slot groups x 64
// lanes; a lane owns 4 consecutive dims (or fewer for D = 64), a slot group
// every fourth slot.  The slots' addresses are resolved once, one thread per
// slot, into LDS; then every wave loads all the slots' lse values and its own
// slots' partials in one batch (one memory round trip), computes the slot
// weights itself, and the groups' sums meet in LDS.
constexpr int kMergeGroups = 4;
constexpr int kMergeSlotsPerWave = 32;  // partial loads in flight per lane and batch

template <typename ET, int DPL>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams a) {
  __shared__ float red[kMergeGroups][64 * DPL];
  __shared__ const float* s_o[kMaxSlots];
  __shared__ const float* s_l[kMaxSlots];
  const int lane = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int64_t RH = (int64_t)a.rows * a.H;
  const int parts_d = (a.D + 64 * DPL - 1) / (64 * DPL);
  const int64_t rh = blockIdx.x / parts_d;
  const int dpart = (blockIdx.x % parts_d) * 64 * DPL;
  const int h = (int)(rh % a.H);
  for (int i = threadIdx.x; i < a.n_slots; i += blockDim.x) {
    int p = 0, t = i;
    while (p + 1 < a.n_parts && t >= a.n_split[p]) { t -= a.n_split[p]; ++p; }
    s_o[i] = a.o[p] + ((int64_t)t * RH + rh) * a.D + dpart;
    s_l[i] = a.lse[p] + (int64_t)t * RH + rh;
  }
  __syncthreads();
  const int nmine = (a.n_slots - grp + kMergeGroups - 1) / kMergeGroups;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  float lse_tot = -INFINITY;
  for (int base = 0; base == 0 || base < nmine; base += kMergeSlotsPerWave) {
    // lse of every slot (lane l: slots l, l + 64, ...; first batch only) and
    // this group's partials, all in flight together
    float l_loc[kMaxSlots / 64];
    if (base == 0) {
#pragma unroll
      for (int i = 0; i < kMaxSlots / 64; ++i) {
        const int sidx = lane + 64 * i;
        l_loc[i] = sidx < a.n_slots ? *s_l[sidx] : -INFINITY;
      }
    }
    float v[kMergeSlotsPerWave][DPL];
    float lw[kMergeSlotsPerWave];
#pragma unroll
    for (int u = 0; u < kMergeSlotsPerWave; ++u) {
      const int j = base + u;
      const bool ok = j < nmine;
      const int sidx = ok ? grp + kMergeGroups * j : 0;
      lw[u] = ok ? *s_l[sidx] : -INFINITY;
      const float* op = (ok ? s_o[sidx] : s_o[0]) + lane * DPL;
      if constexpr (DPL == 4) {
        const float4 x = ok ? *reinterpret_cast<const float4*>(op) : make_float4(0.f, 0.f, 0.f, 0.f);
        v[u][0] = x.x; v[u][1] = x.y; v[u][2] = x.z; v[u][3] = x.w;
      } else {
#pragma unroll
        for (int i = 0; i < DPL; ++i) v[u][i] = ok ? op[i] : 0.f;
      }
    }
    if (base == 0) {
      // total log-sum-exp over every slot and the sink (each wave alike)
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < kMaxSlots / 64; ++i) mx = fmaxf(mx, l_loc[i]);
      mx = wave_max(mx, 64);
      if (a.sink) mx = fmaxf(mx, a.sink[h]);
      float den = 0.f;
      if (mx != -INFINITY) {
#pragma unroll
        for (int i = 0; i < kMaxSlots / 64; ++i) den += l_loc[i] == -INFINITY ? 0.f : expf(l_loc[i] - mx);
      }
      den = wave_sum(den, 64);
      if (a.sink && mx != -INFINITY) den += expf(a.sink[h] - mx);
      lse_tot = mx != -INFINITY ? mx + logf(den) : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < kMergeSlotsPerWave; ++u) {
      const bool use = lw[u] != -INFINITY && lse_tot != -INFINITY;
      const float wgt = use ? expf(lw[u] - lse_tot) : 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[i] = fmaf(wgt, v[u][i], acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < DPL; ++i) red[grp][lane * DPL + i] = acc[i];
  __syncthreads();
  const int d0 = dpart + lane * DPL;
  if (grp != 0 || d0 >= a.D) return;
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    float sum = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < kMergeGroups; ++g2) sum += red[g2][lane * DPL + i];
    acc[i] = sum;
  }
  const int64_t off = rh * a.D + d0;
  if constexpr (ET::kBytes == 2) {
    if constexpr (DPL == 4) {
      uint2 pk;
      pk.x = pack_bf16x2(acc[0], acc[1]);
      pk.y = pack_bf16x2(acc[2], acc[3]);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + off) = pk;
    } else {
      for (int i = 0; i < DPL; ++i) reinterpret_cast<uint16_t*>(a.out)[off + i] = (uint16_t)f32_to_bf16_bits(acc[i]);
    }
  } else {
    for (int i = 0; i < DPL; ++i) reinterpret_cast<float*>(a.out)[off + i] = acc[i];
  }
}

// Many rows, few partials (prefill chunks): one wave per (row, head), a lane
// owning DPL = D/64 consecutive dims; lane s holds slot s's lse, the slot
// weights come from wave reductions, and every slot's partial is requested
// before any is used.  At most kRowsSlots slots.
constexpr int kRowsSlots = 16;
constexpr int kRowsWaves = 4;  // (row, head) pairs per block

template <typename ET, int DPL>
__global__ __launch_bounds__(64 * kRowsWaves) void merge_rows_kernel(MergeParams a) {
  const int lane = threadIdx.x & 63;
  const int64_t RH = (int64_t)a.rows * a.H;
  const int64_t rh = (int64_t)blockIdx.x * kRowsWaves + (threadIdx.x >> 6);
  if (rh >= RH) return;  // uniform per wave
  const int h = (int)(rh % a.H);
  // slot -> (part, split): slots list the parts in order
  auto slot_part = [&](int s, int* t) {
    int p = 0;
    while (p + 1 < a.n_parts && s >= a.n_split[p]) { s -= a.n_split[p]; ++p; }
    *t = s;
    return p;
  };
  float v[kRowsSlots][DPL];
#pragma unroll
  for (int s = 0; s < kRowsSlots; ++s) {
    if (s < a.n_slots) {  // uniform
      int t;
      const int p = slot_part(s, &t);
      const float* op = a.o[p] + ((int64_t)t * RH + rh) * a.D + lane * DPL;
      if constexpr (DPL % 4 == 0) {
#pragma unroll
        for (int i = 0; i < DPL; i += 4) {
          const float4 x = *reinterpret_cast<const float4*>(op + i);
          v[s][i] = x.x; v[s][i + 1] = x.y; v[s][i + 2] = x.z; v[s][i + 3] = x.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < DPL; ++i) v[s][i] = op[i];
      }
    }
  }
  float l = -INFINITY;
  if (lane < a.n_slots) {
    int t;
    const int p = slot_part(lane, &t);
    l = a.lse[p][(int64_t)t * RH + rh];
  }
  float mx = wave_max(l, 64);
  const float sk = a.sink ? a.sink[h] : -INFINITY;
  mx = fmaxf(mx, sk);
  float den = (mx != -INFINITY && l != -INFINITY) ? expf(l - mx) : 0.f;
  den = wave_sum(den, 64);
  if (a.sink && mx != -INFINITY) den += expf(sk - mx);
  const float lse_tot = mx != -INFINITY ? mx + logf(den) : -INFINITY;
  const float w_lane = (l != -INFINITY && lse_tot != -INFINITY) ? expf(l - lse_tot) : 0.f;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
#pragma unroll
  for (int s = 0; s < kRowsSlots; ++s) {
    if (s < a.n_slots) {
      const float w = __shfl(w_lane, s, 64);
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[i] = fmaf(w, v[s][i], acc[i]);
    }
  }
  const int64_t off = rh * a.D + lane * DPL;
  if constexpr (ET::kBytes == 2) {
    uint32_t pk[DPL / 2];
#pragma unroll
    for (int i = 0; i < DPL / 2; ++i) pk[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + off;
    if constexpr (DPL == 8) {
      *reinterpret_cast<uint4*>(o) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    } else {
#pragma unroll
      for (int i = 0; i < DPL / 2; ++i) reinterpret_cast<uint32_t*>(o)[i] = pk[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < DPL; ++i) reinterpret_cast<float*>(a.out)[off + i] = acc[i];
  }
}

// ============================================================ host

void topk_ws_view(int rows, int64_t maxN, int k, const float* scores, void* ws, TopkWs* view);
bool topk_rows_mode(int Tq, int64_t maxN);
int launch_topk_filter(const int64_t* csa_off, const int32_t* q_pos, int B, int Tq, int k, int m, int w,
                       int64_t maxN, const float* scores, void* ws, hipStream_t stream);
int launch_topk_select(const int64_t* csa_off, const int32_t* q_pos, int B, int Tq, int k, int m, int w,
                       int64_t maxN, int32_t* idx, const float* scores, void* ws, hipStream_t stream);

// Blocks of attn_mfma<D, true, fc> the current device holds at once
// (compute units x blocks per unit), queried once per device, D and fc (2 is
// built for D = 512 only).
static int64_t resident_blocks(int D, int fc) {
  static int64_t cache[64][4][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int di = D == 64 ? 0 : D == 128 ? 1 : D == 256 ? 2 : 3;
  const int fi = fc == 2 && D == 512 ? 1 : 0;
  if (cache[dev][di][fi] == 0) {
    int cus = 0, per = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const void* fn = D == 64    ? reinterpret_cast<const void*>(&attn_mfma<64, true>)
                     : D == 128 ? reinterpret_cast<const void*>(&attn_mfma<128, true>)
                     : D == 256 ? reinterpret_cast<const void*>(&attn_mfma<256, true>)
                     : fi       ? reinterpret_cast<const void*>(&attn_mfma<512, true, 2>)
                                : reinterpret_cast<const void*>(&attn_mfma<512, true>);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, kAttnThreads, 0);
    cache[dev][di][fi] = (e == hipSuccess && cus > 0 && per > 0) ? (int64_t)cus * per : -1;
  }
  return cache[dev][di][fi];
}

// A merge to follow the attention (lca_hybrid_attn_merge): sink and output.
struct MergeReq {
  const float* sink;
  void* out;
};
static int launch_attention_sources(const lca_attn_source* srcs, int n_src, const void* q, const int32_t* q_pos,
                                    int B, int Tq, int H, int D, float scale, float eps, int dtype,
                                    hipStream_t stream);
int launch_merge(const lca_partial* parts, int n_parts, const float* win_o, const float* win_lse,
                 const float* sink, int rows, int H, int D, void* out, int dtype, hipStream_t stream);

// The merge of the sources' partials as its own launch.
static int merge_sources(const lca_attn_source* srcs, int n_src, int rows, int H, int D, const MergeReq* mr,
                         int dtype, hipStream_t stream) {
  lca_partial parts[kMaxSrc];
  for (int i = 0; i < n_src; ++i) {
    parts[i].o = srcs[i].o_part;
    parts[i].lse = srcs[i].lse;
    parts[i].n_split = srcs[i].n_split;
  }
  return launch_merge(parts, n_src, nullptr, nullptr, mr->sink, rows, H, D, mr->out, dtype, stream);
}
int launch_topk_select(const int64_t* csa_off, const int32_t* q_pos, int B, int Tq, int k, int m, int w,
                       int64_t maxN, int32_t* idx, const float* scores, void* ws, hipStream_t stream);

// Many query rows per sequence (D = 512, bf16, 128 divisible by H, at least
// kRowsMinTq queries and two blocks of rows): every source takes the
// row-tiled kernel, in one launch; a gathered source (or a top-k source,
// selected first) needs at most two queries per block (H >= 64) and at most
// kRowsIdx slots per split.  A few rows per sequence (a decode step checking
// drafted tokens) take the decode kernel: its blocks of 32 heads give the
// device four times the blocks of a row tile that holds all 128 heads of one
// query, and such a step's key ranges are too short to fill many row tiles.
constexpr int kRowsMinTq = 8;
static bool rows_launch(const lca_attn_source* srcs, int n_src, int Tq, int H, int D, int dtype) {
  if (dtype != LCA_BF16 || D != 512 || H % 16 != 0 || kRowsBlockRows % H != 0 || Tq < kRowsMinTq ||
      (int64_t)Tq * H < 2 * kRowsBlockRows)
    return false;
  for (int i = 0; i < n_src; ++i) {
    const lca_attn_source& in = srcs[i];
    if (in.kind == SRC_GATHER || in.kind == SRC_TOPK) {
      if (kRowsBlockRows / H > kRowsStreams) return false;
      if ((int64_t)((in.k + kRowsTile - 1) / kRowsTile + in.n_split - 1) / in.n_split * kRowsTile > kRowsIdx)
        return false;
    }
  }
  return true;
}

static int launch_attention_impl(const lca_attn_source* srcs, int n_src, const void* q, const int32_t* q_pos, int B,
                                 int Tq, int H, int D, float scale, float eps, int dtype, hipStream_t stream,
                                 const MergeReq* mr) {
  if (n_src < 1 || n_src > kMaxSrc) {
    set_error("attention: %d key sources, 1 to %d supported", n_src, kMaxSrc);
    return LCA_ERR_UNSUPPORTED;
  }
  if (!rows_launch(srcs, n_src, Tq, H, D, dtype)) {
    const int rc = launch_attention_sources(srcs, n_src, q, q_pos, B, Tq, H, D, scale, eps, dtype, stream);
    if (rc != LCA_OK || !mr) return rc;
    return merge_sources(srcs, n_src, B * Tq, H, D, mr, dtype, stream);
  }
  AttnParams a{};
  a.q = q; a.q_pos = q_pos; a.Tq = Tq; a.H = H; a.D = D; a.rows = B * Tq;
  a.scale = scale; a.eps = eps; a.n_src = n_src;
  int splits = 0, topk = -1;
  for (int i = 0; i < n_src; ++i) {
    const lca_attn_source& in = srcs[i];
    AttnSrc& d = a.s[i];
    d.kv = in.kv; d.off = in.off; d.idx = in.idx; d.kind = in.kind; d.k = in.k; d.m2 = in.m2; d.w2 = in.w2;
    d.W = in.W; d.n_split = in.n_split; d.o_part = in.o_part; d.lse = in.lse; d.idx_out = nullptr;
    d.block_begin = splits;
    splits += in.n_split;
    if (in.kind == SRC_TOPK) {
      // selected first (its own launches), then gathered
      topk = i;
      d.kind = SRC_GATHER;
      d.idx = in.idx_out;
    }
  }
  a.n_x = splits;
  // with one split per source the blocks also merge: each takes every source
  // for its rows and writes the output
  if (mr && splits == n_src) {
    a.merge = 1;
    a.sink = mr->sink;
    a.out = mr->out;
  }
  const int64_t tiles_seq = ((int64_t)Tq * H + kRowsBlockRows - 1) / kRowsBlockRows;
  const int64_t nblk = (int64_t)B * tiles_seq * (a.merge ? 1 : splits);
  if (nblk > 0x7FFFFFFF) {
    set_error("attention: %lld blocks exceed the grid limit", (long long)nblk);
    return LCA_ERR_UNSUPPORTED;
  }
  if (topk >= 0) {
    const lca_attn_source& in = srcs[topk];
    const int rc = launch_topk_select(in.off, q_pos, B, Tq, in.k, in.m2, in.w2, in.max_entries, in.idx_out, in.scores,
                                      in.ws, stream);
    if (rc != LCA_OK) return rc;
  }
  if (a.merge)
    hipLaunchKernelGGL(attn_rows_mfma<true>, dim3((unsigned)nblk), dim3(kRowsThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_rows_mfma<false>, dim3((unsigned)nblk), dim3(kRowsThreads), 0, stream, a);
  if (hipPeekAtLastError() != hipSuccess) return LCA_ERR_HIP;
  return (mr && !a.merge) ? merge_sources(srcs, n_src, B * Tq, H, D, mr, dtype, stream) : LCA_OK;
}

int launch_attention(const lca_attn_source* srcs, int n_src, const void* q, const int32_t* q_pos, int B, int Tq,
                     int H, int D, float scale, float eps, int dtype, hipStream_t stream) {
  return launch_attention_impl(srcs, n_src, q, q_pos, B, Tq, H, D, scale, eps, dtype, stream, nullptr);
}

// The attention of every source and the merge of their partials with the
// sink into out: one launch on the row-tiled path with one split per source,
// else the attention and then the merge.
int launch_attention_merge(const lca_attn_source* srcs, int n_src, const void* q, const int32_t* q_pos, int B,
                           int Tq, int H, int D, float scale, float eps, const float* sink, void* out, int dtype,
                           hipStream_t stream) {
  const MergeReq mr{sink, out};
  return launch_attention_impl(srcs, n_src, q, q_pos, B, Tq, H, D, scale, eps, dtype, stream, &mr);
}

static int launch_attention_sources(const lca_attn_source* srcs, int n_src, const void* q, const int32_t* q_pos,
                                    int B, int Tq, int H, int D, float scale, float eps, int dtype,
                                    hipStream_t stream) {
  AttnParams a{};
  a.q = q; a.q_pos = q_pos; a.Tq = Tq; a.H = H; a.D = D; a.rows = B * Tq;
  a.scale = scale; a.eps = eps; a.n_src = n_src;
  const bool mfma = dtype == LCA_BF16 && H % 16 == 0;
  int blocks = 0;
  int topk = -1;          // the TOPK source
  bool fused_topk = false;  // selected inside the attention blocks
  for (int i = 0; i < n_src; ++i) {
    const lca_attn_source& in = srcs[i];
    AttnSrc& d = a.s[i];
    d.kv = in.kv; d.off = in.off; d.idx = in.idx; d.kind = in.kind; d.k = in.k; d.m2 = in.m2; d.w2 = in.w2;
    d.W = in.W; d.n_split = in.n_split; d.o_part = in.o_part; d.lse = in.lse; d.idx_out = nullptr;
    d.block_begin = blocks;
    blocks += in.n_split;
    if (in.kind == SRC_TOPK) {
      topk = i;
      // (many rows per sequence are selected one block per row instead)
      fused_topk = mfma && in.max_entries <= kBitmapEntries && !topk_rows_mode(Tq, in.max_entries);
      if (fused_topk) {
        d.idx_out = in.idx_out;
      } else {
        // the selection's own launches, then the gathered source
        d.kind = SRC_GATHER;
        d.idx = in.idx_out;
      }
    }
    if (mfma && (d.kind == SRC_GATHER || d.kind == SRC_TOPK) &&
        (int64_t)((in.k + kTile - 1) / kTile + in.n_split - 1) / in.n_split * kTile > kIdxLds) {
      set_error("attention: n_split=%d leaves more than %d gathered slots per block (k=%d)", in.n_split, kIdxLds,
                in.k);
      return LCA_ERR_UNSUPPORTED;
    }
  }
  const int rows = B * Tq;
  a.n_x = blocks;
  a.n_hb = (H + kAttnHeads - 1) / kAttnHeads;
  if (mfma) {
    // units of (row, split) in groups of 8 (one per XCD), each with n_hb head blocks
    const int64_t units = (int64_t)rows * blocks;
    const int64_t nblk = (units + 7) / 8 * 8 * a.n_hb;
    if (nblk > 0x7FFFFFFF) {
      set_error("attention: %lld blocks exceed the grid limit", (long long)nblk);
      return LCA_ERR_UNSUPPORTED;
    }
    if (D != 64 && D != 128 && D != 256 && D != 512) {
      set_error("attention: D=%d not supported", D);
      return LCA_ERR_UNSUPPORTED;
    }
  }
  int fc = 1;  // filter chunks per sparse block and pass (attn_mfma's FC)
  if (topk >= 0) {
    // the sparse blocks select from the filtered lists themselves: they also
    // filter the scores when the whole launch is resident at once (else the
    // filter kernel runs first); elsewhere the selection's own launches write
    // idx_out first
    const lca_attn_source& in = srcs[topk];
    int rc = LCA_OK;
    if (fused_topk) {
      topk_ws_view(B * Tq, in.max_entries, in.k, in.scores, in.ws, &a.tw);
      const int64_t units = (int64_t)rows * blocks;
      const int64_t nblk = (units + 7) / 8 * 8 * a.n_hb;
      a.tbpr = in.n_split * a.n_hb;
      // two chunks per sparse block at once when the row's scores give a
      // block more than one
      fc = D == 512 && (int64_t)a.tbpr * kAttnThreads * kFilterPer < in.max_entries ? 2 : 1;
      a.filter = nblk <= resident_blocks(D, fc) ? 1 : 0;
      if (!a.filter)
        rc = launch_topk_filter(in.off, q_pos, B, Tq, in.k, in.m2, in.w2, in.max_entries, in.scores, in.ws, stream);
    } else {
      rc = launch_topk_select(in.off, q_pos, B, Tq, in.k, in.m2, in.w2, in.max_entries, in.idx_out, in.scores,
                              in.ws, stream);
    }
    if (rc != LCA_OK) return rc;
  }
  if (mfma) {
    const int64_t units = (int64_t)rows * blocks;
    dim3 grid((unsigned)((units + 7) / 8 * 8 * a.n_hb));
#define LCA_MFMA(DD)                                                                                      \
  if (fused_topk) hipLaunchKernelGGL((attn_mfma<DD, true>), grid, dim3(kAttnThreads), 0, stream, a);       \
  else hipLaunchKernelGGL((attn_mfma<DD, false>), grid, dim3(kAttnThreads), 0, stream, a);
    switch (D) {
      case 64: LCA_MFMA(64) break;
      case 128: LCA_MFMA(128) break;
      case 256: LCA_MFMA(256) break;
      default:
        if (fused_topk && fc == 2)
          hipLaunchKernelGGL((attn_mfma<512, true, 2>), grid, dim3(kAttnThreads), 0, stream, a);
        else
          LCA_MFMA(512)
        break;
    }
#undef LCA_MFMA
  } else {
    dim3 grid((unsigned)blocks, (unsigned)H, (unsigned)rows);
#define LCA_VALU(ETy)                                                                      \
  switch (D) {                                                                             \
    case 64: hipLaunchKernelGGL((attn_valu<ETy, 1>), grid, dim3(64), 0, stream, a); break; \
    case 128: hipLaunchKernelGGL((attn_valu<ETy, 2>), grid, dim3(64), 0, stream, a); break; \
    case 256: hipLaunchKernelGGL((attn_valu<ETy, 4>), grid, dim3(64), 0, stream, a); break; \
    case 512: hipLaunchKernelGGL((attn_valu<ETy, 8>), grid, dim3(64), 0, stream, a); break; \
    default: set_error("attention: D=%d not supported", D); return LCA_ERR_UNSUPPORTED;   \
  }
    if (dtype == LCA_BF16) { LCA_VALU(BF16) } else { LCA_VALU(F32) }
#undef LCA_VALU
  }
  return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
}

int launch_merge(const lca_partial* parts, int n_parts, const float* win_o, const float* win_lse,
                 const float* sink, int rows, int H, int D, void* out, int dtype, hipStream_t stream) {
  MergeParams a{};
  int np = 0, ns = 0;
  for (int p = 0; p < n_parts; ++p) {
    a.o[np] = parts[p].o; a.lse[np] = parts[p].lse; a.n_split[np] = parts[p].n_split; ns += parts[p].n_split; ++np;
  }
  if (win_o) { a.o[np] = win_o; a.lse[np] = win_lse; a.n_split[np] = 1; ns += 1; ++np; }
  if (ns > kMaxSlots) {
    set_error("merge: %d partial slots, at most %d", ns, kMaxSlots);
    return LCA_ERR_UNSUPPORTED;
  }
  a.n_parts = np;
  a.n_slots = ns;
  a.sink = sink; a.rows = rows; a.H = H; a.D = D; a.out = out;
  if (ns <= kRowsSlots && (int64_t)rows * H >= 1024 && D >= 128) {
    // many rows, few partials: one wave per (row, head)
    const int64_t nblk = ((int64_t)rows * H + kRowsWaves - 1) / kRowsWaves;
    if (nblk > 0x7FFFFFFF) {
      set_error("merge: %lld blocks exceed the grid limit", (long long)nblk);
      return LCA_ERR_UNSUPPORTED;
    }
    dim3 grid((unsigned)nblk);
#define LCA_MERGE_ROWS(ETy)                                                                                  \
  switch (D) {                                                                                               \
    case 128: hipLaunchKernelGGL((merge_rows_kernel<ETy, 2>), grid, dim3(64 * kRowsWaves), 0, stream, a); break; \
    case 256: hipLaunchKernelGGL((merge_rows_kernel<ETy, 4>), grid, dim3(64 * kRowsWaves), 0, stream, a); break; \
    default: hipLaunchKernelGGL((merge_rows_kernel<ETy, 8>), grid, dim3(64 * kRowsWaves), 0, stream, a); break;  \
  }
    if (dtype == LCA_BF16) { LCA_MERGE_ROWS(BF16) } else { LCA_MERGE_ROWS(F32) }
#undef LCA_MERGE_ROWS
    return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
  }
  // (row, head) pairs x 256-dim parts
  const int64_t nblk = (int64_t)rows * H * (D > 256 ? D / 256 : 1);
  if (nblk > 0x7FFFFFFF) {
    set_error("merge: %lld blocks exceed the grid limit", (long long)nblk);
    return LCA_ERR_UNSUPPORTED;
  }
  dim3 grid((unsigned)nblk);
#define LCA_MERGE(ETy)                                                                            \
  switch (D) {                                                                                    \
    case 64: hipLaunchKernelGGL((merge_kernel<ETy, 1>), grid, dim3(256), 0, stream, a); break;   \
    case 128: hipLaunchKernelGGL((merge_kernel<ETy, 2>), grid, dim3(256), 0, stream, a); break;  \
    case 256:                                                                                     \
    case 512: hipLaunchKernelGGL((merge_kernel<ETy, 4>), grid, dim3(256), 0, stream, a); break;  \
    default: set_error("merge: D=%d not supported", D); return LCA_ERR_UNSUPPORTED;             \
  }
  if (dtype == LCA_BF16) { LCA_MERGE(BF16) } else { LCA_MERGE(F32) }
#undef LCA_MERGE
  return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
}

}  // namespace lca
