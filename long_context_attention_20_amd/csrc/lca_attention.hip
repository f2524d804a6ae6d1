// Shared-KV attention partials and the log-sum-exp merge.
//
// Pages: "DeepSeek-V4", Inference efficiency (one KV head shared by all query
// heads), Core block and Provenance 17-18 (RMSNorm on queries and compressed
// KV entries; attention sinks); "Why DeepSeek V4 Stands Apart", Core
// Architectural Innovations (sparse attention over the selected compressed
// entries, dense attention over the 128:1 entries, a 128-token window).
//
// Kernels: attn_mfma (few query rows per sequence; the block is attn_block in
// lca_attn_block.h), attn_rows_mfma (many query rows per sequence: row tiles,
// optionally with the merge), attn_valu (generic path: fp32, or H not a
// multiple of 16), merge_kernel / merge_rows_kernel (sink and log-sum-exp
// merge of the partials), and their host-side launchers.
#include "lca_attn_block.h"

namespace lca {

// The attention kernel of few query rows per sequence (see attn_block);
// OPT: kOptRope (the call turns by a rotary embedding) and / or kOptValues
// (its sources may give values apart from their keys).
template <int D, bool TOPK, int FC = 1, int OPT = 0>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_mfma(AttnParams a) {
  __shared__ __attribute__((aligned(16))) char lds_raw[AttnLds<D, TOPK>::kBytes];
  warm_kernargs<sizeof(AttnParams)>();
  attn_block<D, TOPK, FC, OPT>(a, blockIdx.x, lds_raw);
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

// LDS rows of the row-tiled kernel: the 1 KiB key row in order, padded to
// 1056 bytes.  With the pad, consecutive rows start 32 bytes further along
// the banks, which keeps both read patterns free of bank conflicts on gfx950
// (measured: SQ_LDS_BANK_CONFLICT 0 per launch, against 1.8e8 cycles for 1 KiB
// rows with the 16-byte chunks XOR-swizzled per row): the K-row reads (16
// rows, one 16-byte chunk each) and the transposed V reads (4 or 8 rows, two
// neighbouring 8-byte halves each).
constexpr int kRowsPitch = 528;  // bf16 elements per LDS row
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

// Wave-uniform 64-bit value in scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ROPE: the call turns by a rotary embedding (a kernel of its own, to keep
// the plain one within its register budget).
template <bool MERGE, bool ROPE>
__global__ __launch_bounds__(kRowsThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_rows_mfma(AttnParams a) {
  warm_kernargs<sizeof(AttnParams)>();
  constexpr int D = 512;
  constexpr int KS = D / 32;      // k-steps of S over D
  constexpr int DB = D / 16;      // 16-dim blocks of O
  constexpr int PITCH = kRowsPitch;  // bf16 elements per LDS row (padded)
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
      if (ROPE) rope_turn<8>(f, 32 * ks + 8 * g, D, a.rope, (double)a.q_pos[r]);
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
    const int64_t tps = (ntiles + S.n_split - 1) / S.n_split;  // (tiles_per_split does not apply here)
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
        // lane l fills the row's chunk l
        const uint16_t* src = kvp + (first + ent) * D + lane * 8;
        lds_dma16(src, tile + row * PITCH);
      }
    };
    // window rows: RMS over D of the raw row, then the rotary turn by the
    // token's position, rounded to bf16, in place (the wave that loaded a row
    // normalises it once its loads have landed; lane l holds the row's
    // channels 8 l ..)
    auto norm_rows = [&](int64_t tt) {
      uint16_t* tile = tiles[0][(tt - tb) & 1];
      for (int v = 0; v < rpw; ++v) {
        const int row = wis * rpw + v;
        uint16_t* rowp = tile + row * PITCH + lane * 8;
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
        if (ROPE) {
          const int64_t kc = blo + tt * kRowsTile + row;  // the token position load_tile read
          rope_turn<8>(f, lane * 8, D, a.rope, (double)(kc < bhi ? kc : blo));
        }
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
        // rows c16 and 16 + c16, chunk 4 ks + g: one per-lane offset and an
        // immediate
        const uint16_t* kp = tile + c16 * PITCH + g * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint16_t* k0p = kp + ks * 32;
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
          // (chunk 2 db + bit 1 of c16, half c16 & 1: one per-lane offset and
          // an immediate)
          const uint16_t* vp = tile + (4 * g + (c16 >> 2)) * PITCH + 8 * ((c16 >> 1) & 1) + 4 * (c16 & 1);
#pragma unroll
          for (int db = 0; db < DB; db += 2) {
            const uint16_t* t0 = vp + db * 16;
            const uint16_t* t1 = vp + (db + 1) * 16;
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
      float o4[4] = {O[db][0] * w, O[db][1] * w, O[db][2] * w, O[db][3] * w};
      if (ROPE) rope_turn<4>(o4, 16 * db + 4 * g, D, a.rope, -(double)a.q_pos[r]);
      uint2 pk;
      pk.x = pack_bf16x2(o4[0], o4[1]);
      pk.y = pack_bf16x2(o4[2], o4[3]);
      *reinterpret_cast<uint2*>(outp + db * 16) = pk;
    }
    return;
  }
  const AttnSrc& S = a.s[si];
  const float w = lsum > 0.f ? 1.0f / lsum : 0.f;
  const int64_t orow = ((int64_t)split * a.rows + r) * a.H + h0 + c16;
  float* op = S.o_part + orow * D + 4 * g;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    float o4[4] = {O[db][0] * w, O[db][1] * w, O[db][2] * w, O[db][3] * w};
    // the turn back by the query position (it commutes with the merge, a sum
    // of partials scaled by the same query's weights)
    if (ROPE) rope_turn<4>(o4, 16 * db + 4 * g, D, a.rope, -(double)a.q_pos[r]);
    *reinterpret_cast<float4*>(op + db * 16) = make_float4(o4[0], o4[1], o4[2], o4[3]);
  }
  if (g == 0) S.lse[orow] = lsum > 0.f ? (m_run + __log2f(lsum)) * kLn2 : -INFINITY;
}

// ============================================================ generic path
// One wavefront per (query row, head, split); a lane owns D/64 dims.  Used for
// fp32 and for bf16 head counts that are not a multiple of 16.
// The rotary turn of the lane's DPL dims (dims lane*DPL ..); with one dim per
// lane the pair (2i, 2i+1) spans lanes 2i and 2i+1 (every lane active).
template <int DPL>
__device__ __forceinline__ void valu_turn(float (&v)[DPL], int lane, int D, const RopeTab& rope, double pos) {
  if constexpr (DPL >= 2) {
    rope_turn<DPL>(v, lane * DPL, D, rope, pos);
  } else {
    const float other = __shfl_xor(v[0], 1, 64);
    float pr[2] = {(lane & 1) ? other : v[0], (lane & 1) ? v[0] : other};
    rope_turn<2>(pr, lane & ~1, D, rope, pos);
    v[0] = (lane & 1) ? pr[1] : pr[0];
  }
}

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
  // positions for the rotary embedding: the query's, and the window's first token
  const double qpos = a.rope.dims ? (double)a.q_pos[r] : 0.0;
  const int64_t kpos0 = (a.rope.dims && S.kind == SRC_WINDOW) ? first - S.off[r / a.Tq] : 0;
  const int64_t per = S.tps > 0 ? (int64_t)S.tps * 32 : (n + S.n_split - 1) / S.n_split;
  const int64_t kb = (int64_t)split * per;
  const int64_t ke = (S.tps > 0 && split == S.n_split - 1) ? n : min(n, kb + per);

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
    for (int i = 0; i < DPL; ++i) qh[i] *= inv;
    if (a.rope.dims) valu_turn<DPL>(qh, lane, D, a.rope, qpos);
#pragma unroll
    for (int i = 0; i < DPL; ++i) qh[i] = ET::round(qh[i]);
  }
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  for (int64_t t = kb; t < ke; ++t) {
    const int64_t row = attn_row(S, r, first, nseq, t);
    if (row < 0) continue;
    // a key row (and the value row beside it, with separate values); raw
    // window rows are normalised, turned and rounded on load
    auto fetch = [&](const void* base, float (&x)[DPL]) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        x[i] = ET::load1(base, row * D + lane * DPL + i);
        ss = fmaf(x[i], x[i], ss);
      }
      if (S.kind == SRC_WINDOW) {
        ss = wave_sum(ss, 64);
        const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
        for (int i = 0; i < DPL; ++i) x[i] *= inv;
        if (a.rope.dims) valu_turn<DPL>(x, lane, D, a.rope, (double)(kpos0 + t));
#pragma unroll
        for (int i = 0; i < DPL; ++i) x[i] = ET::round(x[i]);
      }
    };
    float kv[DPL], vv[DPL];
    fetch(S.kv, kv);
    if (S.v) {
      fetch(S.v, vv);
    } else {
#pragma unroll
      for (int i = 0; i < DPL; ++i) vv[i] = kv[i];
    }
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) dot = fmaf(qh[i], kv[i], dot);
    dot = wave_sum(dot, 64) * a.scale;
    const float m_new = fmaxf(m_run, dot);
    const float alpha = expf(m_run - m_new);
    const float p = expf(dot - m_new);
    l_run = l_run * alpha + p;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] = fmaf(o[i], alpha, p * vv[i]);
  }
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  float* op = S.o_part + (((int64_t)split * a.rows + r) * a.H + h) * D;
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] *= inv;
  if (a.rope.dims) valu_turn<DPL>(o, lane, D, a.rope, -qpos);  // -i on the output
#pragma unroll
  for (int i = 0; i < DPL; ++i) op[lane * DPL + i] = o[i];
  if (lane == 0) S.lse[((int64_t)split * a.rows + r) * a.H + h] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
}

// ============================================================ merge
// out[r, h, :] = sum_s exp(lse_s - lse) * o_s,  lse = log(sum_s exp(lse_s) + exp(sink_h)).
// A block owns HPB (row, head) pairs; D/4 threads per pair, 4 dims each.  The
// slot weights of a pair are computed once into LDS.
constexpr int kMaxParts = 8;
constexpr int kMaxSlots = 512;
struct MergeParams {
  const void* o[kMaxParts];     // fp32, or fp16 where o_half
  const float* lse[kMaxParts];
  int n_split[kMaxParts];
  int o_half[kMaxParts];
  int n_parts;
  int n_slots;
  const float* sink;
  int rows, H, D;
  void* out;
};

// One block per (row, head, 256-dim part): 256 threads = 4 slot groups x 64
// lanes; a lane owns 4 consecutive dims (or fewer for D = 64), a slot group
// (wave) every fourth slot.  The block first resolves every slot's addresses
// (one thread per slot) into LDS tables; every later load is then a global
// one (the pointers are cast to the global address space: a generic load
// would count against the LDS wait, so that each table read would also wait
// for every partial requested before it).  Every wave reads all the slots'
// lse values and its own slots' partials and lse in one batch (one memory
// round trip), computes the slot weights itself, and the groups' sums meet
// in LDS.
constexpr int kMergeGroups = 4;

// The block's slot tables: slot s (slots list the parts in order, split t
// of part p) -> the address of its partial's (row, head) row at element
// `first` (bit 0 set for fp16 partials; addresses are at least 4-byte
// aligned) and of its lse.  The parts are walked with compile-time indices:
// a part chosen per thread would index the kernel arguments at run time,
// which the compiler serves from a copy in scratch memory.
template <int NT>  // threads of the block
__device__ __forceinline__ void merge_tables(const MergeParams& a, int64_t RH, int64_t rh, int first,
                                             uint64_t* s_o, const float** s_l) {
  int beg = 0;
#pragma unroll
  for (int p = 0; p < kMaxParts; ++p) {
    if (p < a.n_parts) {  // uniform
      const int n = a.n_split[p];
      const int esz = a.o_half[p] ? 2 : 4;
      for (int t = threadIdx.x; t < n; t += NT) {
        const int64_t e = (int64_t)t * RH + rh;
        s_o[beg + t] = (uint64_t)(uintptr_t)(static_cast<const char*>(a.o[p]) + (e * a.D + first) * esz) |
                       (uint64_t)(a.o_half[p] ? 1 : 0);
        s_l[beg + t] = a.lse[p] + e;
      }
      beg += n;
    }
  }
}

template <typename T>
__device__ __forceinline__ T gload(const T* p) {
  return *(const __attribute__((address_space(1))) T*)(p);
}

// PH: the partials' types -- 0 every part fp32, 1 every part fp16, 2 some
// of each (the type chosen per slot with a branch, which makes the compiler
// wait for each slot's load: for the rare mixed call only).
// SPW: slots per wave and batch (16 for calls of at most 64 slots, whose
// lse values then take one load per lane; else 32): every load of a batch is
// issued, whether its slot exists or not, so the batch fits the call.
template <typename ET, int DPL, int PH, int SPW>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams a) {
  warm_kernargs<sizeof(MergeParams)>();
  constexpr int LLOC = SPW == 16 ? 1 : kMaxSlots / 64;  // lse words per lane
  __shared__ float red[kMergeGroups][64 * DPL];
  __shared__ uint64_t s_o[kMaxSlots];
  __shared__ const float* s_l[kMaxSlots];
  const int lane = threadIdx.x & 63;
  const int grp = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t RH = (int64_t)a.rows * a.H;
  const int parts_d = (a.D + 64 * DPL - 1) / (64 * DPL);
  const int64_t rh = blockIdx.x / parts_d;
  const int dpart = (blockIdx.x % parts_d) * 64 * DPL;
  const int h = (int)(rh % a.H);
  const int ns = a.n_slots;
  merge_tables<256>(a, RH, rh, dpart, s_o, s_l);
  __syncthreads();
  // the lse of every slot (lane l: slots l, l + 64, ...); loads are
  // unconditional (a slot beyond the list reads slot 0 and is not used), so
  // that each batch is straight-line code with every load in flight at once
  float l_loc[LLOC];
#pragma unroll
  for (int i = 0; i < LLOC; ++i) {
    const int sl = lane + 64 * i;
    l_loc[i] = gload(s_l[sl < ns ? sl : 0]);
  }
  const int nmine = (ns - grp + kMergeGroups - 1) / kMergeGroups;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  float lse_tot = -INFINITY;
  // one batch of this wave's slots; the first is peeled off the loop (a
  // loop entered with the lse loads in flight would wait for them first)
  auto batch = [&](const int base) {
    // this wave's slots grp + 4 j: the lane's DPL elements, fp32 words or
    // fp16 pairs (converted where they are used)
    constexpr int WPL = PH == 1 ? (DPL + 1) / 2 : DPL;  // 4-byte words per lane and slot
    uint32_t w[SPW][WPL];
    float lw[SPW];
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int j = base + u;
      const int sidx = j < nmine ? grp + kMergeGroups * j : 0;
      const uint64_t ad = s_o[sidx];
      lw[u] = gload(s_l[sidx]);
      const char* bp = reinterpret_cast<const char*>((uintptr_t)(ad & ~(uint64_t)1));
      if constexpr (PH == 0) {
        if constexpr (DPL == 4) {
          const u32x4 x = gload(reinterpret_cast<const u32x4*>(bp + lane * 16));
          w[u][0] = x[0]; w[u][1] = x[1]; w[u][2] = x[2]; w[u][3] = x[3];
        } else {
#pragma unroll
          for (int i = 0; i < DPL; ++i) w[u][i] = gload(reinterpret_cast<const uint32_t*>(bp) + lane * DPL + i);
        }
      } else if constexpr (PH == 1) {
        if constexpr (DPL == 4) {
          const u32x2 x = gload(reinterpret_cast<const u32x2*>(bp + lane * 8));
          w[u][0] = x[0]; w[u][1] = x[1];
        } else {
          // DPL 1: the word holding the lane's element and its neighbour's
          w[u][0] = gload(reinterpret_cast<const uint32_t*>(bp + ((lane * DPL * 2) & ~3)));
        }
      } else {
        if (ad & 1) {
#pragma unroll
          for (int i = 0; i < DPL; ++i)
            w[u][i] = gload(reinterpret_cast<const uint16_t*>(bp) + lane * DPL + i);
        } else {
#pragma unroll
          for (int i = 0; i < DPL; ++i) w[u][i] = gload(reinterpret_cast<const uint32_t*>(bp) + lane * DPL + i);
        }
      }
    }
    if (base == 0) {
      // total log-sum-exp over every slot and the sink (each wave alike)
#pragma unroll
      for (int i = 0; i < LLOC; ++i)
        if (lane + 64 * i >= ns) l_loc[i] = -INFINITY;
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < LLOC; ++i) mx = fmaxf(mx, l_loc[i]);
      mx = wave_max(mx, 64);
      if (a.sink) mx = fmaxf(mx, a.sink[h]);
      float den = 0.f;
      if (mx != -INFINITY) {
#pragma unroll
        for (int i = 0; i < LLOC; ++i) den += l_loc[i] == -INFINITY ? 0.f : expf(l_loc[i] - mx);
      }
      den = wave_sum(den, 64);
      if (a.sink && mx != -INFINITY) den += expf(a.sink[h] - mx);
      lse_tot = mx != -INFINITY ? mx + logf(den) : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int j = base + u;
      if (j >= nmine) continue;  // uniform
      const bool use = lw[u] != -INFINITY && lse_tot != -INFINITY;
      const float wgt = use ? expf(lw[u] - lse_tot) : 0.f;
      float v[DPL];
      if constexpr (PH == 0) {
#pragma unroll
        for (int i = 0; i < DPL; ++i) v[i] = __uint_as_float(w[u][i]);
      } else if constexpr (PH == 1) {
        if constexpr (DPL == 1) {
          v[0] = (float)__builtin_bit_cast(f16x2_t, w[u][0])[lane & 1];
        } else {
#pragma unroll
          for (int i = 0; i < DPL; ++i) v[i] = (float)__builtin_bit_cast(f16x2_t, w[u][i / 2])[i & 1];
        }
      } else {
        const uint32_t sidx = grp + kMergeGroups * j;
        const bool hf = s_o[sidx] & 1;
#pragma unroll
        for (int i = 0; i < DPL; ++i)
          v[i] = hf ? (float)__builtin_bit_cast(_Float16, (uint16_t)w[u][i]) : __uint_as_float(w[u][i]);
      }
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[i] = fmaf(wgt, v[i], acc[i]);
    }
  };
  batch(0);
  for (int base = SPW; base < nmine; base += SPW) batch(base);
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
  warm_kernargs<sizeof(MergeParams)>();
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
      const int64_t e0 = ((int64_t)t * RH + rh) * a.D + lane * DPL;
      // fp32 or fp16 partials without a branch (as merge_kernel): fp16
      // elements are read as 4-byte words of pairs (the second half of the
      // lane's fp32-sized reads repeats the first)
      const bool hf = a.o_half[p] != 0;
      const uint32_t* wp = reinterpret_cast<const uint32_t*>(static_cast<const char*>(a.o[p]) + e0 * (hf ? 2 : 4));
      uint32_t w[DPL];
#pragma unroll
      for (int i = 0; i < DPL; ++i) w[i] = wp[hf ? (i % (DPL / 2)) : i];
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const f16x2_t hx = __builtin_bit_cast(f16x2_t, w[i / 2]);
        v[s][i] = hf ? (float)hx[i & 1] : __uint_as_float(w[i]);
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

// Blocks of attn_mfma<D, true, fc, opt> the current device holds at once
// (compute units x blocks per unit, from the occupancy query on the idle
// device), queried once per device, D, fc (2 is built for D = 512 without
// options only) and opt (0..3).
// The cache is read and written atomically: concurrent first calls may both
// query, and both store the same value.  Residency is what lets the sparse
// blocks wait for each other; it is not guaranteed while other work holds
// compute units, which is why their wait is bounded (and falls back to an
// exact selection of its own).
static int64_t resident_blocks(int D, int fc, int opt) {
  static std::atomic<int64_t> cache[64][4][5];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int di = D == 64 ? 0 : D == 128 ? 1 : D == 256 ? 2 : 3;
  const int fi = opt ? 1 + opt : (fc == 2 && D == 512 ? 1 : 0);
  int64_t v = cache[dev][di][fi].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0, per = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const void* fn;
#define LCA_OPT_FN(O)                                                                \
  (D == 64    ? reinterpret_cast<const void*>(&attn_mfma<64, true, 1, O>)                \
   : D == 128 ? reinterpret_cast<const void*>(&attn_mfma<128, true, 1, O>)               \
   : D == 256 ? reinterpret_cast<const void*>(&attn_mfma<256, true, 1, O>)               \
              : reinterpret_cast<const void*>(&attn_mfma<512, true, 1, O>))
    if (opt == 1)
      fn = LCA_OPT_FN(1);
    else if (opt == 2)
      fn = LCA_OPT_FN(2);
    else if (opt == 3)
      fn = LCA_OPT_FN(3);
    else
      fn = D == 64    ? reinterpret_cast<const void*>(&attn_mfma<64, true>)
           : D == 128 ? reinterpret_cast<const void*>(&attn_mfma<128, true>)
           : D == 256 ? reinterpret_cast<const void*>(&attn_mfma<256, true>)
           : fi       ? reinterpret_cast<const void*>(&attn_mfma<512, true, 2>)
                      : reinterpret_cast<const void*>(&attn_mfma<512, true>);
#undef LCA_OPT_FN
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, kAttnThreads, 0);
    v = (e == hipSuccess && cus > 0 && per > 0) ? (int64_t)cus * per : -1;
    cache[dev][di][fi].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Diagnostics set through lca_diag_*: a per-block phase trace of the
// attention launches, and a top-k wait that is made to give up.
static std::atomic<uint64_t*> g_trace{nullptr};
static std::atomic<int64_t> g_trace_words{0};
static std::atomic<uint32_t> g_wait_extra{0};
static std::atomic<uint32_t> g_wait_ticks{kDefaultWaitTicks};

void diag_set_trace(uint64_t* buf, int64_t words) {
  g_trace_words.store(buf ? words : 0);
  g_trace.store(buf);
}
void diag_set_topk_wait(uint32_t extra, uint32_t ticks) {
  g_wait_extra.store(extra);
  g_wait_ticks.store(ticks ? ticks : kDefaultWaitTicks);
}
// The start delay of the dense and window blocks of a launch whose sparse
// blocks filter the scores themselves (100 MHz ticks), for at most kHoldRows
// query rows.
constexpr uint32_t kHoldTicks = 125;
constexpr int kHoldRows = 8;
static void apply_diag(AttnParams* a) {
  a->wait_extra = g_wait_extra.load();
  a->wait_ticks = g_wait_ticks.load();
  a->trace = g_trace.load();
  a->trace_words = g_trace_words.load();
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
    parts[i].o_half = srcs[i].o_half;
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
    if (in.v) return false;  // separate values: the per-row kernel
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
  a.topk_src = -1;
  a.q = q; a.q_pos = q_pos; a.Tq = Tq; a.H = H; a.D = D; a.rows = B * Tq;
  a.scale = scale; a.eps = eps; a.n_src = n_src;
  a.rope = make_rope_tab(srcs[0].rope_dims, srcs[0].rope_base);
  apply_diag(&a);
  int splits = 0, topk = -1;
  for (int i = 0; i < n_src; ++i) {
    const lca_attn_source& in = srcs[i];
    if (in.o_half) {
      set_error("attention: fp16 partials (o_half) are written by the few-rows kernel only, not by the "
                "row-tiled one (%d query rows per sequence)", Tq);
      return LCA_ERR_UNSUPPORTED;
    }
    AttnSrc& d = a.s[i];
    d.kv = in.kv; d.off = in.off; d.idx = in.idx; d.kind = in.kind; d.k = in.k; d.m2 = in.m2; d.w2 = in.w2;
    d.W = in.W; d.n_split = in.n_split; d.o_part = static_cast<float*>(in.o_part); d.lse = in.lse;
    d.o_half = in.o_half; d.idx_out = nullptr;
    d.done_len = in.done_len; d.part = in.part; d.tps = in.tiles_per_split; d.v = in.v;
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
  const dim3 grid((unsigned)nblk), block(kRowsThreads);
  if (a.rope.dims) {
    if (a.merge) hipLaunchKernelGGL((attn_rows_mfma<true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_rows_mfma<false, true>), grid, block, 0, stream, a);
  } else {
    if (a.merge) hipLaunchKernelGGL((attn_rows_mfma<true, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_rows_mfma<false, false>), grid, block, 0, stream, a);
  }
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
  a.topk_src = -1;
  a.q = q; a.q_pos = q_pos; a.Tq = Tq; a.H = H; a.D = D; a.rows = B * Tq;
  a.scale = scale; a.eps = eps; a.n_src = n_src;
  a.rope = make_rope_tab(srcs[0].rope_dims, srcs[0].rope_base);
  apply_diag(&a);
  const bool mfma = dtype == LCA_BF16 && H % 16 == 0;
  for (int i = 0; i < n_src; ++i)
    if (srcs[i].o_half && !mfma) {
      set_error("attention: fp16 partials (o_half) need dtype bf16 and H a multiple of 16 (H=%d)", H);
      return LCA_ERR_UNSUPPORTED;
    }
  int blocks = 0;
  int topk = -1;          // the TOPK source
  bool fused_topk = false;  // selected inside the attention blocks
  int opt = a.rope.dims > 0 ? kOptRope : 0;  // | kOptValues: a source with separate values
  for (int i = 0; i < n_src; ++i) {
    const lca_attn_source& in = srcs[i];
    AttnSrc& d = a.s[i];
    d.kv = in.kv; d.off = in.off; d.idx = in.idx; d.kind = in.kind; d.k = in.k; d.m2 = in.m2; d.w2 = in.w2;
    d.W = in.W; d.n_split = in.n_split; d.o_part = static_cast<float*>(in.o_part); d.lse = in.lse;
    d.o_half = in.o_half; d.idx_out = nullptr;
    d.done_len = in.done_len; d.part = in.part; d.tps = in.tiles_per_split; d.v = in.v;
    if (in.v) opt |= kOptValues;
    d.block_begin = blocks;
    blocks += in.n_split;
    if (in.kind == SRC_TOPK) {
      topk = i;
      // (many rows per sequence are selected one block per row instead)
      fused_topk = mfma && in.max_entries <= kBitmapEntries && !topk_rows_mode(Tq, in.max_entries);
      if (fused_topk) {
        d.idx_out = in.idx_out;
        a.topk_src = i;
      } else {
        // the selection's own launches, then the gathered source
        d.kind = SRC_GATHER;
        d.idx = in.idx_out;
      }
    }
    if (mfma && (d.kind == SRC_GATHER || d.kind == SRC_TOPK) &&
        (in.tiles_per_split > 0 ? (int64_t)in.tiles_per_split * kTile
                                : (int64_t)((in.k + kTile - 1) / kTile + in.n_split - 1) / in.n_split * kTile) > kIdxLds) {
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
      fc = !opt && D == 512 && (int64_t)a.tbpr * kAttnThreads * kFilterPer < in.max_entries ? 2 : 1;
      a.filter = nblk <= resident_blocks(D, fc, opt) ? 1 : 0;
      // with few query rows, the dense and window blocks start their loads
      // a little after the sparse blocks' filter loads, which lead the
      // launch's critical path (measured: Pro 1M decode 46.2-46.7 -> 44.7-45.2
      // us per step at 1.0-1.5 us, Flash decode 8 x 128K 61.1-61.6 -> 59.5;
      // 64 rows of varlen decode lose 1-4 us, so they start at once)
      if (a.filter && rows <= kHoldRows) a.hold_ticks = kHoldTicks;
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
#define LCA_MFMA_T(DD, O)                                                                         \
  if (fused_topk) hipLaunchKernelGGL((attn_mfma<DD, true, 1, O>), grid, dim3(kAttnThreads), 0, stream, a); \
  else hipLaunchKernelGGL((attn_mfma<DD, false, 1, O>), grid, dim3(kAttnThreads), 0, stream, a);
#define LCA_MFMA(DD)                                \
  switch (opt) {                                    \
    case 1: LCA_MFMA_T(DD, 1) break;                \
    case 2: LCA_MFMA_T(DD, 2) break;                \
    case 3: LCA_MFMA_T(DD, 3) break;                \
    default: LCA_MFMA_T(DD, 0) break;               \
  }
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
#undef LCA_MFMA_T
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

// The attention part of the decode front launch: DENSE and WINDOW sources on
// the matrix-core path (bf16, D = 512, H a multiple of 16), whose blocks run
// beside the score and append blocks of the same grid.  Fills the parameters
// and the number of attention blocks (a multiple of 8, so that the blocks
// after them keep the XCD-aware numbering), or returns LCA_ERR_UNSUPPORTED.
int setup_attention_front(const lca_attn_source* srcs, int n_src, const void* q, const int32_t* q_pos, int B, int Tq,
                          int H, int D, float scale, float eps, AttnParams* a, int64_t* nblk) {
  if (D != 512 || H % 16 != 0 || n_src < 1 || n_src > kMaxSrc) return LCA_ERR_UNSUPPORTED;
  *a = AttnParams{};
  a->topk_src = -1;
  a->q = q; a->q_pos = q_pos; a->Tq = Tq; a->H = H; a->D = D; a->rows = B * Tq;
  a->scale = scale; a->eps = eps; a->n_src = n_src;
  a->rope = make_rope_tab(srcs[0].rope_dims, srcs[0].rope_base);
  apply_diag(a);
  int blocks = 0;
  for (int i = 0; i < n_src; ++i) {
    const lca_attn_source& in = srcs[i];
    if (in.kind != LCA_SRC_DENSE && in.kind != LCA_SRC_WINDOW) return LCA_ERR_UNSUPPORTED;
    AttnSrc& d = a->s[i];
    d.kv = in.kv; d.off = in.off; d.idx = nullptr; d.kind = in.kind; d.k = 0; d.m2 = in.m2; d.w2 = in.w2;
    d.W = in.W; d.n_split = in.n_split; d.o_part = static_cast<float*>(in.o_part); d.lse = in.lse;
    d.o_half = in.o_half; d.idx_out = nullptr;
    d.done_len = in.done_len; d.part = in.part; d.tps = in.tiles_per_split; d.v = nullptr;
    d.block_begin = blocks;
    blocks += in.n_split;
  }
  a->n_x = blocks;
  a->n_hb = (H + kAttnHeads - 1) / kAttnHeads;
  const int64_t units = (int64_t)a->rows * blocks;
  *nblk = (units + 7) / 8 * 8 * a->n_hb;
  return LCA_OK;
}

int launch_merge(const lca_partial* parts, int n_parts, const float* win_o, const float* win_lse,
                 const float* sink, int rows, int H, int D, void* out, int dtype, hipStream_t stream) {
  MergeParams a{};
  int np = 0, ns = 0;
  for (int p = 0; p < n_parts; ++p) {
    a.o[np] = parts[p].o; a.lse[np] = parts[p].lse; a.n_split[np] = parts[p].n_split;
    a.o_half[np] = parts[p].o_half;
    ns += parts[p].n_split; ++np;
  }
  if (win_o) { a.o[np] = win_o; a.lse[np] = win_lse; a.n_split[np] = 1; a.o_half[np] = 0; ns += 1; ++np; }
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
  int n_half = 0;
  for (int p = 0; p < np; ++p) n_half += a.o_half[p] ? 1 : 0;
  const int ph = n_half == 0 ? 0 : n_half == np ? 1 : 2;
  const bool few = ns <= 64;  // 16 slots per wave and batch
#define LCA_MERGE_PH(ETy, PH)                                                                             \
  switch (D) {                                                                                           \
    case 64: hipLaunchKernelGGL((merge_kernel<ETy, 1, PH, 32>), grid, dim3(256), 0, stream, a); break;   \
    case 128: hipLaunchKernelGGL((merge_kernel<ETy, 2, PH, 32>), grid, dim3(256), 0, stream, a); break;  \
    case 256:                                                                                            \
    case 512:                                                                                            \
      if (few) hipLaunchKernelGGL((merge_kernel<ETy, 4, PH, 16>), grid, dim3(256), 0, stream, a);        \
      else hipLaunchKernelGGL((merge_kernel<ETy, 4, PH, 32>), grid, dim3(256), 0, stream, a);            \
      break;                                                                                             \
    default: set_error("merge: D=%d not supported", D); return LCA_ERR_UNSUPPORTED;                    \
  }
#define LCA_MERGE(ETy)                                                         \
  if (ph == 0) { LCA_MERGE_PH(ETy, 0) } else if (ph == 1) { LCA_MERGE_PH(ETy, 1) } else { LCA_MERGE_PH(ETy, 2) }
  if (dtype == LCA_BF16) { LCA_MERGE(BF16) } else { LCA_MERGE(F32) }
#undef LCA_MERGE
#undef LCA_MERGE_PH
  return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
}

}  // namespace lca
