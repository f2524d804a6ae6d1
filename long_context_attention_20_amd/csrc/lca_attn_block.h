// One block of the shared-KV attention for few query rows per sequence (a
// decode step): the source descriptors and launch parameters, and the block
// itself as a device function, so that the attention kernel and the decode
// front launch (index scores, appends and attention blocks in one grid) run
// the same code.
//
// Pages: "DeepSeek-V4", Inference efficiency (one KV head shared by all query
// heads), Core block and Provenance 17-18 (RMSNorm on queries and compressed
// KV entries; attention sinks); "Why DeepSeek V4 Stands Apart", Core
// Architectural Innovations (sparse attention over the selected compressed
// entries, dense attention over the 128:1 entries, a 128-token window).
//
// Key sources (one per block):
//   DENSE   entries [0, n_visible) of a compressed cache     (HCA), or the
//           part of them completed before / after a given length
//   GATHER  the entries listed in idx (-1 = unused)          (CSA sparse)
//   TOPK    GATHER over the exact top-k the block selects itself
//   WINDOW  raw rows max(0, i-W+1) .. i, RMS-normalised and   (sliding window)
//           rounded to bf16 while they are staged in LDS
// A compressed entry is key and value (K = V).
//
// Matrix-core path (bf16, H a multiple of 16): a block of 8 waves holds one
// query row and 32 query heads; the waves form 2 teams of 4, a team taking
// every other 32-key tile of the block's key range.  In a team, a wave keeps
// 16 normalised query heads over half of D in registers as the B operand of
// S^T = K . Qhat^T (v_mfma_f32_16x16x32_bf16: 16 entries x 16 heads x 32 dims
// per instruction), adds its partner's half of S^T through LDS, runs the
// online softmax on the accumulator (lane = head, 8 entries per lane) and
// accumulates O^T = V^T . P^T for its half of D, whose B operand is the S^T
// accumulator itself once rounded to bf16 (the contraction index is permuted
// identically in A and B).  A 32-entry KV tile sits in LDS once, row-major
// (rows padded by 8 elements against bank conflicts): S^T reads it with
// 16-byte row reads, and the V^T operand comes from the same rows through
// ds_read_b64_tr_b16, whose 16-lane transpose hands lane i column i of a
// 4-row x 16-column block.  Tiles are double-buffered per team, the next
// tile's global loads in flight while the current one is computed.
#pragma once
#include <atomic>

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
  float* o_part;        // [n_split, rows, H, D], fp32 (fp16 with o_half)
  float* lse;           // [n_split, rows, H]
  // DENSE: part 1 keeps the entries complete within the first done_len[b]
  // tokens of sequence b, part 2 the entries completed after them (0: all)
  const int64_t* done_len;
  int part;
  int tps;              // > 0: 32-key tiles per split (a fixed partition); 0: from n_split
  const void* v;        // values, rows laid out as kv; null: the keys are the values
  int o_half;           // 1: o_part holds fp16 values
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
  int topk_src;         // the TOPK source (selected inside the blocks), or -1
  int tbpr;             // TOPK blocks per row (n_split * n_hb)
  // row-tiled path: every block takes all sources (one split each) and
  // writes the merged output with the sink (bf16 [rows, H, D]) instead of
  // partials
  int merge;
  const float* sink;    // [H] or NULL
  void* out;
  // the rotary embedding of the call: the last rope.dims dims of each head
  // (0: none); queries turn by their position, window rows by theirs,
  // partials and outputs by minus the query's
  RopeTab rope;
  // the in-launch top-k wait: it waits for tbpr + wait_extra filter shares
  // (wait_extra > 0 only as a diagnostic: the wait then always gives up) for
  // at most wait_ticks of the 100 MHz constant clock
  uint32_t wait_extra;
  uint32_t wait_ticks;
  // dense and window blocks start this many ticks of the 100 MHz clock late
  // (a launch whose sparse blocks filter the scores: their loads go first)
  uint32_t hold_ticks;
  // diagnostics: per-block phase stamps (kTraceWords per block), or NULL
  uint64_t* trace;
  int64_t trace_words;
};

constexpr int kFilterPer = 8;  // scores per thread and filter chunk
constexpr uint32_t kDefaultWaitTicks = 10000;  // 100 us of the 100 MHz clock

// Phase stamps of a block (diagnostics): s_memrealtime (100 MHz) at
//   0 block start, 1 filter done, 2 wait done, 3 selection done,
//   4 prologue done (query normalised, first tile requested), 5 key loop
//   done, 6 partial stored;
// word 7: source kind | wait gave up << 2 | fallback selection << 3 |
//   owns top-k slots << 4 | XCC id << 8 | query row << 12 (20 bits) |
//   HW_ID register << 32;
// words 8..15, the top-k steps (last filter chunk / the selection): 8
//   histogram summed, 9 threshold found, 10 list space reserved, 11 own
//   share counted (before the wait), 12 lists loaded (selection starts),
//   13 second-level threshold found, 14 cut found, 15 filter loads issued.
constexpr int kTraceWords = 16;
__device__ __forceinline__ void trace_stamp(const AttnParams& a, int phase) {
  if (a.trace && threadIdx.x == 0 && (int64_t)(blockIdx.x + 1) * kTraceWords <= a.trace_words)
    a.trace[(int64_t)blockIdx.x * kTraceWords + phase] = __builtin_amdgcn_s_memrealtime();
}
__device__ __forceinline__ void trace_flags(const AttnParams& a, uint32_t flags) {
  if (a.trace && threadIdx.x == 0 && (int64_t)(blockIdx.x + 1) * kTraceWords <= a.trace_words) {
    uint32_t hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    a.trace[(int64_t)blockIdx.x * kTraceWords + 7] = ((uint64_t)hw << 32) | ((xcc & 0xFu) << 8) | flags;
    // (flags carries the row in bits 12..31)
  }
}

// A load of a block-uniform value through the scalar cache (the constant
// address space: memory this kernel does not write).
template <typename T>
__device__ __forceinline__ T scalar_load(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

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
    n = n < nseq ? n : nseq;
    if (s.part != 0) {
      const int64_t nd = n_windows(s.done_len[b], s.m2, s.w2);
      if (s.part == 1) return n < nd ? n : nd;
      *first = base + nd;
      return n > nd ? n - nd : 0;
    }
    return n;
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
// Options of a kernel variant (the OPT template argument): the rotary
// embedding, separate values.  Their code stays out of the plain kernel,
// whose register budget it would strain.
constexpr int kOptRope = 1;
constexpr int kQRotPairs = 64;  // rotated pairs of the query-angle table
constexpr int kOptValues = 2;

// LDS of the block (besides a few small arrays it declares itself): the
// tiles, or with a TOPK source the selection's scratch when that is larger.
template <int D, bool TOPK>
struct AttnLds {
  static constexpr size_t kTileBytes = 4 * (size_t)kTile * (D + 8) * 2;
  static constexpr size_t kBytes = (TOPK && sizeof(SelectLds) > kTileBytes) ? sizeof(SelectLds) : kTileBytes;
};

// One block of the attention: bid is the block's number in the attention
// grid (1-D, XCD-aware numbering below), lds_raw AttnLds<D, TOPK>::kBytes of
// LDS.  Called by the attention kernel, and by the decode front launch for
// its attention blocks.
template <int D, bool TOPK, int FC = 1, int OPT = 0>
__device__ __forceinline__ void attn_block(const AttnParams& a, const int bid, char* lds_raw) {
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
  constexpr size_t kLdsBytes = AttnLds<D, TOPK>::kBytes;
  static_assert(AttnLds<D, TOPK>::kTileBytes == 4 * (size_t)TILE_ELEMS * 2, "tile memory");
  static_assert(!TOPK || sizeof(FilterShared) <= kLdsBytes, "the filter's LDS lives in the tile memory");
  auto tiles = reinterpret_cast<uint16_t(*)[2][TILE_ELEMS]>(lds_raw);
  __shared__ SelectShared sel_sh;
  __shared__ int32_t sidx[kIdxLds];
  __shared__ float sx[2][4][8][64];         // S partial exchange, per team
  __shared__ float qss[2][4][16];           // query sum-of-squares exchange, per team
  // rotary embedding of a window block's rows: the angles of its first
  // token's position and the turns per position, per pair (rope_turn_near)
  __shared__ float2 s_rot[(OPT & kOptRope) ? D / 2 : 1];
  __shared__ float s_turns[(OPT & kOptRope) ? D / 2 : 1];
  // the query position's angles, cosine and sine per rotated pair (for
  // rotations over at most 2 * kQRotPairs dims): the query turns by them and
  // the partial turns back by their conjugates
  __shared__ float2 s_qrot[(OPT & kOptRope) ? kQRotPairs : 1];
  // 1-D grid, XCD-aware: workgroups go to the 8 XCDs round-robin by linear
  // id, so the n_hb head blocks of one (row, split) unit take ids 8 apart and
  // share an XCD's L2 for the keys they all read
  const int xcd = bid & 7;
  const int jj = bid >> 3;
  const int hb = jj % a.n_hb;
  const int unit = (jj / a.n_hb) * 8 + xcd;
  if (unit >= a.rows * a.n_x) return;  // padding of the last group (uniform)
  trace_stamp(a, 0);
  const int r = unit / a.n_x;
  int split;
  const int si = attn_source(a, unit % a.n_x, &split);
  // the block's source by value: every source's descriptor is read from the
  // kernel arguments in one batch (indexing them by si would make each read
  // wait for si, and every later read for the one before)
  AttnSrc S = a.s[0];
#pragma unroll
  for (int k = 1; k < kMaxSrc; ++k)
    if (si == k) S = a.s[k];
  const int kind = S.kind;
  const bool gather = kind == SRC_GATHER || kind == SRC_TOPK;
  // a TOPK block's filter (or selection) inputs first: they depend on the
  // kernel arguments alone, and the block's critical path starts with them
  SelectPrefetch<kAttnThreads> pf;
  FilterPrefetch<kAttnThreads, kFilterPer, FC> fpf;
  if constexpr (TOPK) {
    if (si == a.topk_src) {  // (kind == SRC_TOPK, from the kernel arguments alone)
      if (a.filter)
        filter_prefetch(a.tw, r, split * a.n_hb + hb, a.tbpr, fpf);
      else
        topk_prefetch(a.tw, r, pf);
      trace_stamp(a, 15);
    }
    if (a.hold_ticks && (kind == SRC_DENSE || kind == SRC_WINDOW)) {  // (a bounded wait)
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__builtin_amdgcn_s_memrealtime() - t0 < a.hold_ticks) __builtin_amdgcn_s_sleep(2);
    }
  }
  uint32_t tflags = (uint32_t)kind | ((uint32_t)(r & 0xFFFFF) << 12);
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

  // --- every load that needs only the row, issued in one batch before any
  // of them is waited for: the sequence's offsets and the row's position
  // (which give the key count), the query, a gathered block's slots, and a
  // TOPK block's filter or selection inputs
  // (each load is unconditional, from a valid stand-in address when its
  // value is not needed, so that no branch makes the compiler wait for it)
  // The block-uniform values are scalar loads (their own counter: waiting for
  // them does not wait for the vector loads behind them).
  // (r through an empty assembly statement: the row-only loads below then
  // cannot be hoisted above a TOPK block's prefetch, whose loads would wait
  // behind them)
  int r_row = r;
  asm volatile("" : "+s"(r_row));
  const int b = r_row / a.Tq;
  const int64_t* offp = S.off + b;
  const int64_t off0 = scalar_load(offp), off1 = scalar_load(offp + 1);
  const int32_t* qpp = a.q_pos ? a.q_pos + r_row : reinterpret_cast<const int32_t*>(offp);
  const int32_t qpos_ld = scalar_load(qpp);
  const int64_t* dlp = S.done_len ? S.done_len + b : offp;
  const int64_t dlen_ld = scalar_load(dlp);
  uint4 qraw[KS];
  {
    // (a wave beyond H loads head c16 instead and never uses it)
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)r * a.H + (wave_on ? h : c16)) * D + d0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qraw[ks] = *reinterpret_cast<const uint4*>(qp + ks * 32 + g * 8);
  }
  // gathered keys: the key count is k, so the block's slots are known now
  constexpr int kIdxPer = kIdxLds / kAttnThreads;
  int32_t jraw[kIdxPer];
  int64_t gcnt = 0, gkbase = 0;
  if (gather) {
    const int64_t gt = (S.k + kTile - 1) / kTile;
    const int64_t gps = S.tps > 0 ? (int64_t)S.tps : (gt + S.n_split - 1) / S.n_split;
    const int64_t gtb = (int64_t)split * gps;
    const int64_t gte = (S.tps > 0 && split == S.n_split - 1) ? gt : min(gt, gtb + gps);
    gkbase = gtb * kTile;
    gcnt = gte > gtb ? min((gte - gtb) * kTile, (int64_t)S.k - gkbase) : 0;
  }
  {
    // (unconditional loads: a slot beyond the block's reads its last one, a
    // block without listed slots reads a stand-in; the values are not used)
    const int32_t* ip = (kind == SRC_GATHER && gcnt > 0) ? S.idx + (int64_t)r * S.k + gkbase
                                                          : reinterpret_cast<const int32_t*>(offp);
    const int64_t last = (kind == SRC_GATHER && gcnt > 0) ? gcnt - 1 : 0;
#pragma unroll
    for (int u = 0; u < kIdxPer; ++u) {
      const int64_t i = (int64_t)threadIdx.x + u * kAttnThreads;
      jraw[u] = ip[i < last ? i : last];
    }
  }
  // --- the key count and the block's key range
  const int32_t qpos_r = ((kind != SRC_GATHER || ((OPT & kOptRope) && a.rope.dims)) && a.q_pos) ? qpos_ld : 0;
  const bool qtab = (OPT & kOptRope) && a.rope.dims > 0 && a.rope.dims <= 2 * kQRotPairs;  // uniform
  if constexpr ((OPT & kOptRope) != 0) {
    // (read after the barriers that precede the query's normalisation)
    if (qtab && (int)threadIdx.x < a.rope.dims / 2) {
      float sn, cs;
      rope_sincos((double)qpos_r, threadIdx.x, a.rope, &sn, &cs);
      s_qrot[threadIdx.x] = make_float2(cs, sn);
    }
  }
  const int64_t dlen = (kind == SRC_DENSE && S.part != 0) ? dlen_ld : 0;
  const int64_t nseq = off1 - off0;
  int64_t first = off0;
  int64_t n;
  if (gather) {
    n = S.k;
  } else if (kind == SRC_DENSE) {
    n = n_windows((int64_t)qpos_r + 1, S.m2, S.w2);
    n = n < nseq ? n : nseq;
    if (S.part != 0) {
      const int64_t nd = n_windows(dlen, S.m2, S.w2);
      if (S.part == 1) {
        n = n < nd ? n : nd;
      } else {
        first = off0 + nd;
        n = n > nd ? n - nd : 0;
      }
    }
  } else {  // window
    int64_t lo = (int64_t)qpos_r - S.W + 1;
    if (lo < 0) lo = 0;
    const int64_t hi = qpos_r < nseq - 1 ? (int64_t)qpos_r : nseq - 1;
    first = off0 + lo;
    n = hi >= lo ? hi - lo + 1 : 0;
  }
  const int64_t ntiles = (n + kTile - 1) / kTile;
  const int64_t tps = S.tps > 0 ? (int64_t)S.tps : (ntiles + S.n_split - 1) / S.n_split;
  const int64_t tb = (int64_t)split * tps;
  // (a fixed partition's last split takes whatever the others leave)
  const int64_t te = (S.tps > 0 && split == S.n_split - 1) ? ntiles : min(ntiles, tb + tps);
  const int64_t kbase = tb * kTile;
  const int64_t rounds = (te > tb && nseq > 0) ? (te - tb + 1) / 2 : 0;  // uniform over the block

  // --- tile staging (per team): loads are unconditional (invalid keys read a
  // clamped valid row) and zeroed when stored
  uint4 stage[LOADS];
  uint4 vstage[(OPT & kOptValues) ? LOADS : 1];  // the value rows beside the keys (separate values)
  const bool sv = (OPT & kOptValues) && S.v != nullptr;  // uniform over the block
  uint32_t okbits = 0;
  int64_t stage_t = 0;               // tile index of the staged loads (window rows' positions)
  const int64_t kpos0 = first - off0;  // window: position of key 0 (the window's first token)
  const uint16_t* kvp = reinterpret_cast<const uint16_t*>(S.kv);
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(sv ? S.v : S.kv);
  auto key_ok = [&](int64_t key) -> bool {
    if (key >= n) return false;
    return !gather || sidx[key - kbase] >= 0;
  };
  auto load_tile = [&](int64_t t) {
    okbits = 0;
    stage_t = t;
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
      if constexpr ((OPT & kOptValues) != 0)
        if (sv) vstage[v] = *reinterpret_cast<const uint4*>(vp + (first + off) * D + vec * 8);
    }
  };
  // raw window rows: RMS-normalised over D (the VPR lanes holding a row are
  // consecutive lanes of one wave), turned by the token's position, rounded
  auto norm_rows = [&](uint4 (&rows)[LOADS]) {
#pragma unroll
    for (int v = 0; v < LOADS; ++v) {
      float f[8];
      BF16::unpack(rows[v], f);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
      ss = lane_group_sum<VPR>(ss);
      const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= inv;
      if ((OPT & kOptRope) && a.rope.dims) {
        // (the block's first token at kpos0; its rows are a few thousand
        // positions from it at most)
        const int id = tt + kTeamThreads * v;
        rope_turn_near<8>(f, (id % VPR) * 8, D, a.rope.dims, s_rot, s_turns, (float)(stage_t * kTile + id / VPR));
      }
      rows[v] = BF16::pack(f);
    }
  };
  auto store_tile = [&](uint16_t* tile, uint16_t* vtile) {
    if (kind == SRC_WINDOW) {
      norm_rows(stage);
      if constexpr ((OPT & kOptValues) != 0)
        if (sv) norm_rows(vstage);
    }
#pragma unroll
    for (int v = 0; v < LOADS; ++v) {
      const int id = tt + kTeamThreads * v;
      const int row = id / VPR, vec = id % VPR;
      const bool ok = (okbits >> v) & 1u;
      *reinterpret_cast<uint4*>(&tile[row * PITCH + vec * 8]) = ok ? stage[v] : make_uint4(0, 0, 0, 0);
      if constexpr ((OPT & kOptValues) != 0)
        if (sv) *reinterpret_cast<uint4*>(&vtile[row * PITCH + vec * 8]) = ok ? vstage[v] : make_uint4(0, 0, 0, 0);
    }
  };

  if constexpr ((OPT & kOptRope) != 0) {
    if (kind == SRC_WINDOW && a.rope.dims) {  // (block-uniform)
      for (int p = threadIdx.x; p < a.rope.dims / 2; p += kAttnThreads) {
        const double th = rope_theta(p, a.rope);
        double rev = (double)kpos0 * th * kInvTwoPi;
        rev -= rint(rev);
        float sn, cs;
        sincos_quarters((float)(rev * 4.0), &sn, &cs);
        s_rot[p] = make_float2(cs, sn);
        s_turns[p] = (float)(th * kInvTwoPi);
      }
      __syncthreads();
    }
  }
  // --- prologue: dense and window keys do not depend on staged indices, so
  // their first tile is requested first
  if (!gather && rounds > 0) load_tile(tb + team);
  if (kind == SRC_GATHER && rounds > 0) {
#pragma unroll
    for (int u = 0; u < kIdxPer; ++u) {
      const int i = (int)threadIdx.x + u * kAttnThreads;
      const int32_t j = jraw[u];
      if (i < gcnt) sidx[i] = (j < 0 || j >= nseq) ? -1 : j;  // (i < gcnt: a listed slot)
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
      // launch is sized to fit the machine at once, so normally they are all
      // resident and the wait ends; the wait is bounded all the same (other
      // work on the device can keep blocks of this launch from starting), and
      // a block that gives up selects from the scores alone (below), so the
      // result is the same either way.
      // the block's chunks are tbi, tbi + tbpr, ...; the first FC of them had
      // their loads issued at the start and are filtered in one pass (one
      // threshold, one list reservation)
      const int tbi = split * a.n_hb + hb;
      constexpr int64_t CH = (int64_t)kAttnThreads * kFilterPer;
      for (int64_t cb = tbi; cb * CH < nv; cb += (int64_t)a.tbpr * FC) {
        if (cb != tbi) filter_prefetch(tw, r, (int)cb, a.tbpr, fpf);
        filter_chunk(tw, r, nv, (int)cb, a.tbpr, fpf, *reinterpret_cast<FilterShared*>(lds_raw),
                     [&](int ph) { trace_stamp(a, ph); });
        __syncthreads();
      }
      trace_stamp(a, 1);
      if (threadIdx.x == 0) {
        // the block that completes the count knows that every filter of the
        // row has read the first histogram (each reads it before it counts
        // itself): it clears the histogram for the next score call
        const uint32_t before = __hip_atomic_fetch_add(&tw.done[r], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        trace_stamp(a, 11);
        s_timeout = before + 1 == (uint32_t)a.tbpr ? 2u : 0u;
        const uint32_t target = (uint32_t)a.tbpr + a.wait_extra;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__hip_atomic_load(&tw.done[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
          if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)a.wait_ticks) {
            s_timeout |= 1u;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
      __syncthreads();
      const uint32_t wst = s_timeout;
      ready = !(wst & 1u);
      tflags |= (wst & 1u) << 2;
      if (wst & 2u) {
        uint32_t* gh = tw.hist + (int64_t)r * tw.nstripe * kHistBins;
        for (int i = threadIdx.x; i < tw.nstripe * kHistBins; i += kAttnThreads) gh[i] = 0;
      }
      if (ready) topk_prefetch(tw, r, pf);  // the lists are complete now
    }
    trace_stamp(a, 2);
    if (kind == SRC_TOPK && te > tb) {  // the block owns slots (even of an empty row)
      tflags |= 1u << 4;
      // this block's slots [kbase, kbase + cnt) of the row's top k in
      // ascending entry order: every block of the row runs the same exact
      // selection from the filtered lists; the head-block-0 blocks also
      // write their slots to idx_out
      const int64_t cnt = min((te - tb) * kTile, n - kbase);
      if (!a.filter && split == 0 && hb == 0 && !all) {
        // the filter launch before this one has read the first histogram:
        // clear it for the next call
        uint32_t* gh = tw.hist + (int64_t)r * tw.nstripe * kHistBins;
        for (int i = threadIdx.x; i < tw.nstripe * kHistBins; i += kAttnThreads) gh[i] = 0;
      }
      for (int i = threadIdx.x; i < cnt; i += kAttnThreads) sidx[i] = (all && kbase + i < nv) ? (int32_t)(kbase + i) : -1;
      // the tile memory beyond the selection's scratch keeps candidates the
      // selection reads more than once (8192 of them at D = 512)
      constexpr uint32_t kCandLds = (uint32_t)((kLdsBytes - sizeof(SelectLds)) / sizeof(uint64_t));
      static_assert(sizeof(SelectLds) % sizeof(uint64_t) == 0, "the candidate area must be 8-byte aligned");
      static_assert(kHistBins * sizeof(uint32_t) <= kLdsBytes, "the fallback's histogram lives in the tile memory");
      auto emit = [&](uint32_t o, int32_t e) {
        const int64_t j = (int64_t)o - kbase;
        if (j >= 0 && j < cnt) sidx[j] = e;
      };
      bool got = false;
      if (!all && ready)
        got = topk_row_select<kAttnThreads, true>(tw, r, pf, *reinterpret_cast<SelectLds*>(lds_raw), sel_sh, emit,
                                                  reinterpret_cast<uint64_t*>(lds_raw + sizeof(SelectLds)),
                                                  kCandLds, [&](int ph) { trace_stamp(a, ph); }) != 0;
      if (!all && !got) {
        // the wait gave up or the lists are not consistent: the exact
        // selection from the row's scores alone (the score launch before
        // this one wrote every score); nothing was emitted above
        __syncthreads();
        topk_row_scan_select<kAttnThreads>(tw.scores + (int64_t)r * tw.max_entries, nv, (uint32_t)S.k,
                                           reinterpret_cast<uint32_t*>(lds_raw), sel_sh, emit);
        tflags |= 1u << 3;
      }
      __syncthreads();  // sidx complete; the selection's scratch is free
      if (hb == 0 && S.idx_out)
        for (int i = threadIdx.x; i < cnt; i += kAttnThreads) S.idx_out[(int64_t)r * S.k + kbase + i] = sidx[i];
    }
  }
  trace_stamp(a, 3);
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
      if ((OPT & kOptRope) && a.rope.dims) {
        if (qtab)
          rope_turn_tab<8>(f, d0 + ks * 32 + g * 8, D, a.rope.dims, s_qrot, false);
        else
          rope_turn<8>(f, d0 + ks * 32 + g * 8, D, a.rope, (double)qpos_r);
      }
      qb[ks] = __builtin_bit_cast(bf16x8_t, BF16::pack(f));
    }
  }

  f32x4 O[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) O[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;
  trace_stamp(a, 4);

  for (int64_t rd = 0; rd < rounds; ++rd) {
    const int64_t t = tb + 2 * rd + team;   // this team's tile (may be past te)
    const bool active = t < te;
    // keys and values share one tile with one vector per key; separate
    // values take the team's second buffer, so the tiles are single-buffered
    // (the register staging still prefetches the next tile) and every wave
    // leaves the previous round before they are overwritten
    uint16_t* tile = tiles[team][sv ? 0 : (rd & 1)];
    uint16_t* vtile = sv ? tiles[team][1] : tile;
    if (sv && rd > 0) __syncthreads();
    store_tile(tile, vtile);
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
        const uint16_t* trow0 = &vtile[(4 * g + (c16 >> 2)) * PITCH + d0 + 4 * (c16 & 3)];
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
  trace_stamp(a, 5);
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
    float o4[4] = {u.x + v.x, u.y + v.y, u.z + v.z, u.w + v.w};
    if ((OPT & kOptRope) && a.rope.dims) {  // -i on the output
      if (qtab)
        rope_turn_tab<4>(o4, d, D, a.rope.dims, s_qrot, true);
      else
        rope_turn<4>(o4, d, D, a.rope, -(double)qpos_r);
    }
    if (S.o_half) {
      // fp16 (round to nearest even), 8 bytes per lane
      const f16x4 hv = {(_Float16)o4[0], (_Float16)o4[1], (_Float16)o4[2], (_Float16)o4[3]};
      __builtin_nontemporal_store(hv, reinterpret_cast<f16x4*>(reinterpret_cast<_Float16*>(S.o_part) +
                                                               ((((int64_t)split * a.rows + r) * a.H + hbase) * D +
                                                                (int64_t)i * 4)));
    } else {
      __builtin_nontemporal_store(f32x4{o4[0], o4[1], o4[2], o4[3]}, reinterpret_cast<f32x4*>(op + (int64_t)i * 4));
    }
  }
  if (threadIdx.x < nh) {
    float M, f0, f1, lsum;
    head_state(threadIdx.x, &M, &f0, &f1, &lsum);
    __builtin_nontemporal_store(lsum > 0.f ? (M + __log2f(lsum)) * kLn2 : -INFINITY,
                                &S.lse[((int64_t)split * a.rows + r) * a.H + hbase + threadIdx.x]);
  }
  trace_stamp(a, 6);
  trace_flags(a, tflags);
}

}  // namespace lca
