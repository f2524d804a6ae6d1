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
// 64 heads (4 waves x 16 heads).  A wave keeps its 16 normalised query heads in
// registers as the B operand of S^T = K . Qhat^T (v_mfma_f32_16x16x32_bf16:
// 16 entries x 16 heads x 32 dims per instruction), runs the online softmax on
// the S^T accumulator (lane = head, 8 entries per lane), and accumulates
// O^T = V^T . P^T, whose B operand is the S^T accumulator itself once rounded
// to bf16 (the contraction index is permuted identically in A and B).  The
// 32-entry KV tile sits in LDS (rows padded to avoid bank conflicts); the next
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

constexpr int kTile = 32;  // keys per tile

template <int D>
struct MfmaCfg {
  static constexpr int KS = D / 32;           // k-steps of S (32 dims each)
  static constexpr int DB = D / 16;           // 16-dim blocks of O
  static constexpr int PITCH = D + 8;         // bf16 elements per LDS row
  static constexpr int VPR = D / 8;           // 16-byte vectors per row
  static constexpr int LOADS = kTile * VPR / 256;  // per thread per tile
};

template <int D>
__global__ __launch_bounds__(256) void attn_mfma(AttnParams a) {
  using Cfg = MfmaCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTile * Cfg::PITCH];
  const int r = blockIdx.z;
  const int split = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int h0 = blockIdx.y * 64 + wave * 16;
  const bool wave_on = h0 < a.H;  // H is a multiple of 16
  const int h = h0 + c16;

  int64_t first, nseq;
  const int64_t n = attn_keys(a, r, &first, &nseq);
  const int64_t ntiles = (n + kTile - 1) / kTile;
  const int64_t tps = (ntiles + a.n_split - 1) / a.n_split;
  const int64_t tb = (int64_t)split * tps;
  const int64_t te = min(ntiles, tb + tps);

  // --- normalised query heads in registers (B operand of S^T)
  bf16x8_t qb[Cfg::KS];
  if (wave_on) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)r * a.H + h) * D;
    uint4 raw[Cfg::KS];
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < Cfg::KS; ++ks) {
      raw[ks] = *reinterpret_cast<const uint4*>(qp + ks * 32 + g * 8);
      float f[8];
      BF16::unpack(raw[ks], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
    for (int ks = 0; ks < Cfg::KS; ++ks) {
      float f[8];
      BF16::unpack(raw[ks], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= inv;
      qb[ks] = __builtin_bit_cast(bf16x8_t, BF16::pack(f));
    }
  }

  f32x4 O[Cfg::DB];
#pragma unroll
  for (int d = 0; d < Cfg::DB; ++d) O[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;

  // --- tile staging: thread -> (row, 16-byte vector) pairs
  uint4 stage[Cfg::LOADS];
  auto load_tile = [&](int64_t t) {
#pragma unroll
    for (int v = 0; v < Cfg::LOADS; ++v) {
      const int id = threadIdx.x + 256 * v;
      const int row = id / Cfg::VPR, vec = id % Cfg::VPR;
      const int64_t key = t * kTile + row;
      int64_t grow = -1;
      if (key < n) grow = attn_row(a, r, first, nseq, key);
      stage[v] = grow >= 0 ? *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.kv) + grow * D + vec * 8)
                           : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&]() {
    if (a.src == SRC_WINDOW) {
      // RMS-normalise every row over D; a row spans VPR consecutive lanes
#pragma unroll
      for (int v = 0; v < Cfg::LOADS; ++v) {
        float f[8];
        BF16::unpack(stage[v], f);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
        ss = wave_sum(ss, Cfg::VPR < 64 ? Cfg::VPR : 64);
        const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] *= inv;
        stage[v] = BF16::pack(f);
      }
    }
#pragma unroll
    for (int v = 0; v < Cfg::LOADS; ++v) {
      const int id = threadIdx.x + 256 * v;
      const int row = id / Cfg::VPR, vec = id % Cfg::VPR;
      *reinterpret_cast<uint4*>(&tile[row * Cfg::PITCH + vec * 8]) = stage[v];
    }
  };

  if (tb < te) load_tile(tb);
  for (int64_t t = tb; t < te; ++t) {
    store_tile();
    __syncthreads();
    if (t + 1 < te) load_tile(t + 1);
    if (wave_on) {
      // S^T for entries 0-15 and 16-31 of the tile
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < Cfg::KS; ++ks) {
        const uint4 k0 = *reinterpret_cast<const uint4*>(&tile[c16 * Cfg::PITCH + ks * 32 + g * 8]);
        const uint4 k1 = *reinterpret_cast<const uint4*>(&tile[(16 + c16) * Cfg::PITCH + ks * 32 + g * 8]);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k0), qb[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k1), qb[ks], s1, 0, 0, 0);
      }
      // lane (c16 = head, g): s0[i] -> entry 4g+i, s1[i] -> entry 16+4g+i
      float lg[8];
      const int64_t kb = t * kTile;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t e0 = kb + 4 * g + i, e1 = kb + 16 + 4 * g + i;
        bool v0 = e0 < n, v1 = e1 < n;
        if (a.src == SRC_GATHER) {
          v0 = v0 && attn_row(a, r, first, nseq, e0) >= 0;
          v1 = v1 && attn_row(a, r, first, nseq, e1) >= 0;
        }
        lg[i] = v0 ? s0[i] * sl2 : -INFINITY;
        lg[4 + i] = v1 ? s1[i] * sl2 : -INFINITY;
      }
      float tmax = lg[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, lg[i]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run, tmax);
      if (m_new != -INFINITY) {
        const float alpha = exp2f(m_run - m_new);
        float p[8], psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = exp2f(lg[i] - m_new);
          psum += p[i];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        uint4 pb;
        pb.x = pack_bf16x2(p[0], p[1]);
        pb.y = pack_bf16x2(p[2], p[3]);
        pb.z = pack_bf16x2(p[4], p[5]);
        pb.w = pack_bf16x2(p[6], p[7]);
        const bf16x8_t pt = __builtin_bit_cast(bf16x8_t, pb);
        // V^T operand rows for this lane group: entries 4g..4g+3, 16+4g..16+4g+3
        const uint16_t* r0 = &tile[(4 * g) * Cfg::PITCH];
        const uint16_t* r1 = &tile[(16 + 4 * g) * Cfg::PITCH];
#pragma unroll
        for (int db = 0; db < Cfg::DB; ++db) {
          const int col = db * 16 + c16;
          uint4 vv;
          vv.x = (uint32_t)r0[col] | ((uint32_t)r0[Cfg::PITCH + col] << 16);
          vv.y = (uint32_t)r0[2 * Cfg::PITCH + col] | ((uint32_t)r0[3 * Cfg::PITCH + col] << 16);
          vv.z = (uint32_t)r1[col] | ((uint32_t)r1[Cfg::PITCH + col] << 16);
          vv.w = (uint32_t)r1[2 * Cfg::PITCH + col] | ((uint32_t)r1[3 * Cfg::PITCH + col] << 16);
          O[db] = O[db] * alpha;
          O[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vv), pt, O[db], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  if (!wave_on) return;
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  float* op = a.o_part + (((int64_t)split * a.rows + r) * a.H + h) * D;
  // lane (head c16, g) holds dims 16*db + 4g .. +3
#pragma unroll
  for (int db = 0; db < Cfg::DB; ++db) {
    float4 v = make_float4(O[db][0] * inv, O[db][1] * inv, O[db][2] * inv, O[db][3] * inv);
    *reinterpret_cast<float4*>(op + db * 16 + 4 * g) = v;
  }
  if (g == 0) {
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
// One wavefront per (row, head); a lane owns D/64 dims.
constexpr int kMaxParts = 8;
struct MergeParams {
  const float* o[kMaxParts];
  const float* lse[kMaxParts];
  int n_split[kMaxParts];
  int n_parts;
  const float* sink;
  int rows, H, D;
  void* out;
};

template <typename ET, int DPL>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rh = (int64_t)blockIdx.x * 4 + wave;
  if (rh >= (int64_t)a.rows * a.H) return;
  const int h = (int)(rh % a.H);
  float mx = a.sink ? a.sink[h] : -INFINITY;
  for (int p = 0; p < a.n_parts; ++p)
    for (int s = 0; s < a.n_split[p]; ++s) mx = fmaxf(mx, a.lse[p][(int64_t)s * a.rows * a.H + rh]);
  float den = 0.f;
  if (mx != -INFINITY) {
    if (a.sink) den = expf(a.sink[h] - mx);
    for (int p = 0; p < a.n_parts; ++p)
      for (int s = 0; s < a.n_split[p]; ++s) {
        const float l = a.lse[p][(int64_t)s * a.rows * a.H + rh];
        if (l != -INFINITY) den += expf(l - mx);
      }
  }
  const float lse = mx != -INFINITY ? mx + logf(den) : -INFINITY;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  if (lse != -INFINITY) {
    for (int p = 0; p < a.n_parts; ++p)
      for (int s = 0; s < a.n_split[p]; ++s) {
        const int64_t base = (int64_t)s * a.rows * a.H + rh;
        const float l = a.lse[p][base];
        if (l == -INFINITY) continue;
        const float wgt = expf(l - lse);
        const float* op = a.o[p] + base * a.D + lane * DPL;
        if constexpr (DPL % 4 == 0) {
#pragma unroll
          for (int i = 0; i < DPL; i += 4) {
            const float4 v = *reinterpret_cast<const float4*>(op + i);
            acc[i] = fmaf(wgt, v.x, acc[i]); acc[i + 1] = fmaf(wgt, v.y, acc[i + 1]);
            acc[i + 2] = fmaf(wgt, v.z, acc[i + 2]); acc[i + 3] = fmaf(wgt, v.w, acc[i + 3]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < DPL; ++i) acc[i] = fmaf(wgt, op[i], acc[i]);
        }
      }
  }
  if constexpr (ET::kBytes == 2 && DPL == 8) {
    stg16(a.out, (rh * a.D + lane * 8) * 2, BF16::pack(acc));
  } else {
    for (int i = 0; i < DPL; ++i) {
      const int64_t o = rh * a.D + lane * DPL + i;
      if (ET::kBytes == 2)
        reinterpret_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_bf16_bits(acc[i]);
      else
        reinterpret_cast<float*>(a.out)[o] = acc[i];
    }
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
    dim3 grid((unsigned)n_split, (unsigned)((H + 63) / 64), (unsigned)rows);
    switch (D) {
      case 64: hipLaunchKernelGGL((attn_mfma<64>), grid, dim3(256), 0, stream, a); break;
      case 128: hipLaunchKernelGGL((attn_mfma<128>), grid, dim3(256), 0, stream, a); break;
      case 256: hipLaunchKernelGGL((attn_mfma<256>), grid, dim3(256), 0, stream, a); break;
      case 512: hipLaunchKernelGGL((attn_mfma<512>), grid, dim3(256), 0, stream, a); break;
      default: set_error("attention: D=%d not supported", D); return LCA_ERR_UNSUPPORTED;
    }
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
  int np = 0;
  for (int p = 0; p < n_parts; ++p) {
    a.o[np] = parts[p].o; a.lse[np] = parts[p].lse; a.n_split[np] = parts[p].n_split; ++np;
  }
  if (win_o) { a.o[np] = win_o; a.lse[np] = win_lse; a.n_split[np] = 1; ++np; }
  a.n_parts = np;
  a.sink = sink; a.rows = rows; a.H = H; a.D = D; a.out = out;
  const int64_t waves = (int64_t)rows * H;
  dim3 grid((unsigned)((waves + 3) / 4));
#define LCA_MERGE(ETy)                                                                           \
  switch (D) {                                                                                   \
    case 64: hipLaunchKernelGGL((merge_kernel<ETy, 1>), grid, dim3(256), 0, stream, a); break;  \
    case 128: hipLaunchKernelGGL((merge_kernel<ETy, 2>), grid, dim3(256), 0, stream, a); break; \
    case 256: hipLaunchKernelGGL((merge_kernel<ETy, 4>), grid, dim3(256), 0, stream, a); break; \
    case 512: hipLaunchKernelGGL((merge_kernel<ETy, 8>), grid, dim3(256), 0, stream, a); break; \
    default: set_error("merge: D=%d not supported", D); return LCA_ERR_UNSUPPORTED;            \
  }
  if (dtype == LCA_BF16) { LCA_MERGE(BF16) } else { LCA_MERGE(F32) }
#undef LCA_MERGE
  return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
}

}  // namespace lca
