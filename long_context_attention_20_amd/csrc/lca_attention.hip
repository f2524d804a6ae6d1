// a4 / a5 / a6. Shared-KV attention partials and the log-sum-exp merge.
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
#include "lca_common.h"

namespace lca {

enum { SRC_DENSE = 0, SRC_GATHER = 1, SRC_WINDOW = 2 };

struct AttnParams {
  const void* q;        // [rows, H, D]
  const void* kv;       // cache rows or raw rows
  const int64_t* off;   // [B+1] row offsets of kv
  const int32_t* idx;   // GATHER: [rows, k]
  const int32_t* q_pos; // [rows]
  int src;
  int Tq, H, D;
  int k;                // GATHER slots per row
  int m2, w2;           // DENSE visibility
  int W;                // WINDOW length
  float scale, eps;
  int n_split;
  int rows;
  float* o_part;        // [n_split, rows, H, D]
  float* lse;           // [n_split, rows, H]
};

// Number of keys of query row r and its first raw row (WINDOW) -------------
__device__ __forceinline__ int64_t attn_keys(const AttnParams& a, int r, int64_t* first, int64_t* nseq_out) {
  const int b = r / a.Tq;
  const int64_t base = a.off[b];
  const int64_t nseq = a.off[b + 1] - base;
  *first = base;
  *nseq_out = nseq;
  if (a.src == SRC_GATHER) return a.k;
  const int64_t i = a.q_pos[r];
  if (a.src == SRC_DENSE) {
    int64_t n = n_windows(i + 1, a.m2, a.w2);
    return n < nseq ? n : nseq;
  }
  int64_t lo = i - a.W + 1;
  if (lo < 0) lo = 0;
  int64_t hi = i < nseq - 1 ? i : nseq - 1;
  *first = base + lo;
  return hi >= lo ? hi - lo + 1 : 0;
}

// Global row of key t (or -1 when the slot is unused or out of range).
__device__ __forceinline__ int64_t attn_row(const AttnParams& a, int r, int64_t first, int64_t nseq, int64_t t) {
  if (a.src == SRC_GATHER) {
    const int32_t j = a.idx[(int64_t)r * a.k + t];
    return (j < 0 || j >= nseq) ? -1 : first + j;
  }
  return first + t;
}

// ============================================================ matrix cores

constexpr int kTile = 32;       // keys per tile
constexpr int kIdxLds = 4096;   // gathered indices staged per block

template <int D>
struct MfmaCfg {
  static constexpr int KS = D / 32;                // k-steps of S (32 dims each)
  static constexpr int DB = D / 16;                // 16-dim blocks of O
  static constexpr int PITCH = D + 8;              // bf16 elements per LDS row
  static constexpr int VPR = D / 8;                // 16-byte vectors per row
  static constexpr int LOADS = kTile * VPR / 256;  // per thread per tile
  static constexpr int KB = KS < 4 ? KS : 4;       // k-steps per operand batch
  static constexpr int OB = DB < 4 ? DB : 4;       // dim blocks per operand batch
};

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

// Block: 4 waves, 32 query heads of one query row.  Wave w owns heads
// 16*(w%2) .. +15 and the dim half (w/2) of D: it computes the S^T partial over
// its half of D, adds its partner's half through LDS (same order in both, so
// both hold identical logits), runs the online softmax and accumulates O^T
// for its D/2 dims.  Halving the per-wave query and accumulator state lets
// two or three independent blocks share a CU, so that the latency-bound
// phases of one block (staging, exchange, softmax) overlap the matrix-core
// phases of another.
constexpr int kAttnThreads = 256;
constexpr int kAttnHeads = 32;      // query heads per block

template <int D, int SRC>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_mfma(AttnParams a) {
  constexpr int DH = D / 2;                 // dims per wave
  constexpr int KS = DH / 32;               // k-steps of the S partial
  constexpr int DB = DH / 16;               // 16-dim blocks of O per wave
  constexpr int PITCH = D + 8;              // bf16 elements per LDS row
  constexpr int VPR = D / 8;                // 16-byte vectors per row
  constexpr int LOADS = (kTile * VPR + kAttnThreads - 1) / kAttnThreads;
  constexpr bool PARTIAL = kTile * VPR < kAttnThreads;  // some threads stage nothing
  constexpr int KB = KS < 2 ? KS : 2;       // k-steps per operand batch
  constexpr int OB = DB < 4 ? DB : 4;       // dim blocks per operand batch
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTile * PITCH];
  __shared__ int32_t sidx[SRC == SRC_GATHER ? kIdxLds : 1];
  __shared__ float sx[4][8][64];            // S partial exchange
  __shared__ float qss[4][16];              // query sum-of-squares exchange
  __shared__ uint32_t tile_valid;
  const int r = blockIdx.z;
  const int split = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int hq = wave & 1, dh = wave >> 1;
  const int h0 = blockIdx.y * kAttnHeads + hq * 16;
  const bool wave_on = h0 < a.H;  // H is a multiple of 16; uniform per wave pair
  const int h = h0 + c16;
  const int d0 = dh * DH;         // first dim of this wave

  int64_t first, nseq;
  const int64_t n = attn_keys(a, r, &first, &nseq);
  const int64_t ntiles = (n + kTile - 1) / kTile;
  const int64_t tps = (ntiles + a.n_split - 1) / a.n_split;
  const int64_t tb = (int64_t)split * tps;
  const int64_t te = min(ntiles, tb + tps);
  const int64_t kbase = tb * kTile;

  if (SRC == SRC_GATHER) {
    const int64_t cnt = min((te - tb) * kTile, n - kbase);
    for (int i = threadIdx.x; i < cnt; i += kAttnThreads) {
      const int32_t j = a.idx[(int64_t)r * a.k + kbase + i];
      sidx[i] = (j < 0 || j >= nseq) ? -1 : j;
    }
  }


  // --- tile staging: loads are unconditional (invalid keys read a clamped
  // valid row) and masked when stored
  uint4 stage[LOADS];
  uint32_t okbits = 0;
  const uint16_t* kvp = reinterpret_cast<const uint16_t*>(a.kv);
  auto load_tile = [&](int64_t t) {
    okbits = 0;
#pragma unroll
    for (int v = 0; v < LOADS; ++v) {
      const int id = threadIdx.x + kAttnThreads * v;
      const int row = id / VPR, vec = id % VPR;
      if (PARTIAL && row >= kTile) break;
      const int64_t key = t * kTile + row;
      bool ok = key < n;
      int64_t off;
      if (SRC == SRC_GATHER) {
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
  auto store_tile = [&]() {
    uint32_t mask = 0;
#pragma unroll
    for (int v = 0; v < LOADS; ++v) {
      const int id = threadIdx.x + kAttnThreads * v;
      const int row = id / VPR, vec = id % VPR;
      if (PARTIAL && row >= kTile) break;
      const bool ok = (okbits >> v) & 1u;
      *reinterpret_cast<uint4*>(&tile[row * PITCH + vec * 8]) = ok ? stage[v] : make_uint4(0, 0, 0, 0);
      if (vec == 0 && ok) mask |= 1u << row;
    }
    if (threadIdx.x == 0) tile_valid = 0;
    __syncthreads();
    if (mask) atomicOr(&tile_valid, mask);
    if (SRC == SRC_WINDOW) {
      // RMS-normalise each row over D in place: TPR threads per row
      __syncthreads();
      constexpr int TPR = VPR < 16 ? VPR : 16;
      constexpr int PER = D / TPR;                     // elements per thread, a multiple of 8
      constexpr int RPP = kAttnThreads / TPR;          // rows per pass
      const int part = threadIdx.x % TPR;
#pragma unroll
      for (int row0 = 0; row0 < kTile; row0 += RPP) {
        const int row = row0 + threadIdx.x / TPR;
        uint4* rp = reinterpret_cast<uint4*>(&tile[(row < kTile ? row : 0) * PITCH + part * PER]);
        uint4 vals[PER / 8];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < PER / 8; ++i) {
          vals[i] = rp[i];
          float f[8];
          BF16::unpack(vals[i], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
        }
#pragma unroll
        for (int o = 1; o < TPR; o <<= 1) ss += __shfl_xor(ss, o, 64);
        const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
        if (row < kTile) {
#pragma unroll
          for (int i = 0; i < PER / 8; ++i) {
            float f[8];
            BF16::unpack(vals[i], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] *= inv;
            rp[i] = BF16::pack(f);
          }
        }
      }
    }
  };

  // dense and window keys do not depend on staged indices: request the first
  // tile before the query loads
  if (SRC != SRC_GATHER && tb < te && nseq > 0) load_tile(tb);

  // --- normalised query: this wave's heads, its half of D (B operand of S^T)
  bf16x8_t qb[KS];
  uint4 qraw[KS];
  {
    float ss = 0.f;
    if (wave_on) {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)r * a.H + h) * D + d0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qraw[ks] = *reinterpret_cast<const uint4*>(qp + ks * 32 + g * 8);
        float f[8];
        BF16::unpack(qraw[ks], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
      }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    if (g == 0) qss[wave][c16] = ss;
  }
  __syncthreads();  // sidx and qss ready
  if (wave_on) {
    const float ss = qss[hq][c16] + qss[hq + 2][c16];
    const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
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
  if (SRC == SRC_GATHER && tb < te && nseq > 0) load_tile(tb);
  for (int64_t t = tb; t < te && nseq > 0; ++t) {
    store_tile();
    __syncthreads();
    if (t + 1 < te) load_tile(t + 1);
    // ---- S^T partial over this wave's dims, entries 0-15 (s0) and 16-31 (s1)
    f32x4 s0a = {0.f, 0.f, 0.f, 0.f}, s0b = s0a, s1a = s0a, s1b = s0a;
    if (wave_on) {
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
      sx[wave][i][lane] = p0[i];
      sx[wave][4 + i][lane] = p1[i];
    }
    __syncthreads();
    if (wave_on) {
      const int wlo = hq;       // dims [0, D/2)
      const int whi = hq + 2;   // dims [D/2, D)
      float lg[8];
      const uint32_t vm = tile_valid;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s0 = sx[wlo][i][lane] + sx[whi][i][lane];
        const float s1 = sx[wlo][4 + i][lane] + sx[whi][4 + i][lane];
        lg[i] = ((vm >> (4 * g + i)) & 1u) ? s0 * sl2 : -INFINITY;
        lg[4 + i] = ((vm >> (16 + 4 * g + i)) & 1u) ? s1 * sl2 : -INFINITY;
      }
      float tmax = lg[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, lg[i]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run, tmax);
      if (m_new != -INFINITY) {  // uniform: masks do not depend on the head
        const float alpha = exp2f(m_run - m_new);
        float p[8], psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = exp2f(lg[i] - m_new);
          psum += p[i];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
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
    __syncthreads();
  }

  if (!wave_on) return;
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  float* op = a.o_part + (((int64_t)split * a.rows + r) * a.H + h) * D + d0;
  // lane (head c16, g) holds dims d0 + 16*db + 4g .. +3
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    float4 v = make_float4(O[db][0] * inv, O[db][1] * inv, O[db][2] * inv, O[db][3] * inv);
    *reinterpret_cast<float4*>(op + db * 16 + 4 * g) = v;
  }
  if (g == 0 && dh == 0) {
    const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    a.lse[((int64_t)split * a.rows + r) * a.H + h] = lse;
  }
}

// ============================================================ generic path
// One wavefront per (query row, head, split); a lane owns D/64 dims.  Used for
// fp32 and for bf16 head counts that are not a multiple of 16.
template <typename ET, int DPL>
__global__ __launch_bounds__(64) void attn_valu(AttnParams a) {
  const int r = blockIdx.z;
  const int h = blockIdx.y;
  const int split = blockIdx.x;
  const int lane = threadIdx.x;
  const int D = a.D;
  int64_t first, nseq;
  const int64_t n = attn_keys(a, r, &first, &nseq);
  const int64_t per = (n + a.n_split - 1) / a.n_split;
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
    const int64_t row = attn_row(a, r, first, nseq, t);
    if (row < 0) continue;
    float kv[DPL];
    float dot = 0.f, ss = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      kv[i] = ET::load1(a.kv, row * D + lane * DPL + i);
      ss = fmaf(kv[i], kv[i], ss);
    }
    if (a.src == SRC_WINDOW) {
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
  float* op = a.o_part + (((int64_t)split * a.rows + r) * a.H + h) * D;
#pragma unroll
  for (int i = 0; i < DPL; ++i) op[lane * DPL + i] = o[i] * inv;
  if (lane == 0) a.lse[((int64_t)split * a.rows + r) * a.H + h] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
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

// One block per (row, head): 256 threads = 4 slot groups x 64 lanes; a lane
// owns D/64 dims (float4 or narrower), a slot group a quarter of the slots,
// and the groups meet in LDS.  All of a thread's loads are issued together.
constexpr int kMergeGroups = 4;
constexpr int kMergeSlotsPerGroup = kMaxSlots / kMergeGroups;

template <typename ET, int DPL>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams a) {
  __shared__ float wts[kMaxSlots];
  __shared__ float red[kMergeGroups][64 * DPL];
  const int lane = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int64_t RH = (int64_t)a.rows * a.H;
  const int64_t rh = blockIdx.x;
  const int h = (int)(rh % a.H);
  // slot pointers (cheap: at most kMaxParts parts)
  auto slot_ptr = [&](int sidx, const float** lse_p, const float** o_p) {
    int p = 0, s = sidx;
    while (s >= a.n_split[p]) { s -= a.n_split[p]; ++p; }
    *lse_p = a.lse[p] + (int64_t)s * RH + rh;
    *o_p = a.o[p] + ((int64_t)s * RH + rh) * a.D;
  };
  // weights, by wave 0
  if (grp == 0) {
    float l_loc[kMaxSlots / 64];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxSlots / 64; ++i) {
      const int sidx = lane + 64 * i;
      l_loc[i] = -INFINITY;
      if (sidx < a.n_slots) {
        const float* lp; const float* op;
        slot_ptr(sidx, &lp, &op);
        l_loc[i] = *lp;
      }
      mx = fmaxf(mx, l_loc[i]);
    }
    mx = wave_max(mx, 64);
    if (a.sink) mx = fmaxf(mx, a.sink[h]);
    float den = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int i = 0; i < kMaxSlots / 64; ++i) den += l_loc[i] == -INFINITY ? 0.f : expf(l_loc[i] - mx);
    }
    den = wave_sum(den, 64);
    if (a.sink && mx != -INFINITY) den += expf(a.sink[h] - mx);
    const float lse = mx != -INFINITY ? mx + logf(den) : -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxSlots / 64; ++i) {
      const int sidx = lane + 64 * i;
      if (sidx < a.n_slots) wts[sidx] = (l_loc[i] != -INFINITY && lse != -INFINITY) ? expf(l_loc[i] - lse) : 0.f;
    }
  }
  // this group's slots: grp, grp + 4, ...
  const int nmine = (a.n_slots - grp + kMergeGroups - 1) / kMergeGroups;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  constexpr int U = 16;
  for (int base = 0; base < nmine; base += U) {
    float v[U][DPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u;
      const int sidx = grp + kMergeGroups * (j < nmine ? j : 0);
      const float* lp; const float* op;
      slot_ptr(sidx, &lp, &op);
      if constexpr (DPL == 8) {
        const float4 x0 = *reinterpret_cast<const float4*>(op + lane * 8);
        const float4 x1 = *reinterpret_cast<const float4*>(op + lane * 8 + 4);
        v[u][0] = x0.x; v[u][1] = x0.y; v[u][2] = x0.z; v[u][3] = x0.w;
        v[u][4] = x1.x; v[u][5] = x1.y; v[u][6] = x1.z; v[u][7] = x1.w;
      } else {
#pragma unroll
        for (int i = 0; i < DPL; ++i) v[u][i] = op[lane * DPL + i];
      }
    }
    if (base == 0) __syncthreads();  // weights ready (every thread reaches this once)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u;
      if (j >= nmine) break;
      const float wgt = wts[grp + kMergeGroups * j];
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[i] = fmaf(wgt, v[u][i], acc[i]);
    }
  }
  if (nmine <= 0) __syncthreads();
#pragma unroll
  for (int i = 0; i < DPL; ++i) red[grp][lane * DPL + i] = acc[i];
  __syncthreads();
  if (grp != 0) return;
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    float sum = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < kMergeGroups; ++g2) sum += red[g2][lane * DPL + i];
    acc[i] = sum;
  }
  const int64_t off = rh * a.D + lane * DPL;
  if constexpr (ET::kBytes == 2) {
    if constexpr (DPL == 8) {
      stg16(a.out, off * 2, BF16::pack(acc));
    } else {
      for (int i = 0; i < DPL; ++i) reinterpret_cast<uint16_t*>(a.out)[off + i] = (uint16_t)f32_to_bf16_bits(acc[i]);
    }
  } else {
    for (int i = 0; i < DPL; ++i) reinterpret_cast<float*>(a.out)[off + i] = acc[i];
  }
}

// ============================================================ host

int launch_attention(int src, const void* q, const void* kv, const int64_t* off, const int32_t* idx,
                     const int32_t* q_pos, int B, int Tq, int H, int D, int k, int m2, int w2, int W,
                     float scale, float eps, int n_split, float* o_part, float* lse, int dtype,
                     hipStream_t stream) {
  AttnParams a{};
  a.q = q; a.kv = kv; a.off = off; a.idx = idx; a.q_pos = q_pos; a.src = src;
  a.Tq = Tq; a.H = H; a.D = D; a.k = k; a.m2 = m2; a.w2 = w2; a.W = W;
  a.scale = scale; a.eps = eps; a.n_split = n_split; a.rows = B * Tq;
  a.o_part = o_part; a.lse = lse;
  const int rows = B * Tq;
  if (dtype == LCA_BF16 && H % 16 == 0) {
    if (src == SRC_GATHER && (int64_t)((k + kTile - 1) / kTile + n_split - 1) / n_split * kTile > kIdxLds) {
      set_error("attention: n_split=%d leaves more than %d gathered slots per block (k=%d)", n_split, kIdxLds, k);
      return LCA_ERR_UNSUPPORTED;
    }
    dim3 grid((unsigned)n_split, (unsigned)((H + kAttnHeads - 1) / kAttnHeads), (unsigned)rows);
#define LCA_ATTN(DD)                                                                                             \
  switch (src) {                                                                                                 \
    case SRC_DENSE: hipLaunchKernelGGL((attn_mfma<DD, SRC_DENSE>), grid, dim3(kAttnThreads), 0, stream, a); break;       \
    case SRC_GATHER: hipLaunchKernelGGL((attn_mfma<DD, SRC_GATHER>), grid, dim3(kAttnThreads), 0, stream, a); break;     \
    default: hipLaunchKernelGGL((attn_mfma<DD, SRC_WINDOW>), grid, dim3(kAttnThreads), 0, stream, a); break;             \
  }
    switch (D) {
      case 64: LCA_ATTN(64) break;
      case 128: LCA_ATTN(128) break;
      case 256: LCA_ATTN(256) break;
      case 512: LCA_ATTN(512) break;
      default: set_error("attention: D=%d not supported", D); return LCA_ERR_UNSUPPORTED;
    }
#undef LCA_ATTN
  } else {
    dim3 grid((unsigned)n_split, (unsigned)H, (unsigned)rows);
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
  dim3 grid((unsigned)((int64_t)rows * H));
#define LCA_MERGE(ETy)                                                                            \
  switch (D) {                                                                                    \
    case 64: hipLaunchKernelGGL((merge_kernel<ETy, 1>), grid, dim3(256), 0, stream, a); break;   \
    case 128: hipLaunchKernelGGL((merge_kernel<ETy, 2>), grid, dim3(256), 0, stream, a); break;  \
    case 256: hipLaunchKernelGGL((merge_kernel<ETy, 4>), grid, dim3(256), 0, stream, a); break;  \
    case 512: hipLaunchKernelGGL((merge_kernel<ETy, 8>), grid, dim3(256), 0, stream, a); break;  \
    default: set_error("merge: D=%d not supported", D); return LCA_ERR_UNSUPPORTED;             \
  }
  if (dtype == LCA_BF16) { LCA_MERGE(BF16) } else { LCA_MERGE(F32) }
#undef LCA_MERGE
  return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
}

}  // namespace lca
