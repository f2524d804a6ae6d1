// a2 + a3. Lightning-indexer scores over the visible CSA entries and an exact
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
// Kernel 2 (select): every block derives the threshold bin T from the
// histogram (the highest bin whose suffix count reaches k), keeps the entries
// of its chunk above T and the candidates inside T, each in index order, in a
// private workspace region.  The last block of a row (atomic ticket) gathers
// them, radix-selects the missing candidates exactly on (low 21 key bits,
// inverted index) -- a total order, so ties go to the smaller index -- writes
// the row and zeroes the histogram and ticket for the next call.
#include "lca_common.h"

namespace lca {

constexpr int kIdxThreads = 256;
constexpr int kHistBins = 2048;
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
  int chunk;           // entries per score block
  float* scores;       // [rows][max_entries]
  uint32_t* hist;      // [rows][kHistBins]
  // select
  uint32_t* ticket;    // [rows]
  uint32_t* nsel;      // [rows][nblk]
  uint32_t* ncand;     // [rows][nblk]
  int32_t* sel;        // [rows][nblk][selcap]
  uint64_t* cand;      // [rows][nblk][kSelChunk]
  uint64_t* cand_all;  // [rows][max_entries]
  int nblk;
  int selcap;
  int32_t* idx;        // [rows][k]
};

__device__ __forceinline__ int64_t row_visible(const IndexParams& a, int r, int64_t n_seq) {
  const int i = a.q_pos[r];
  int64_t nv = n_windows((int64_t)i + 1, a.m, a.w);
  nv = nv < n_seq ? nv : n_seq;
  // never beyond the per-row capacity the workspace was sized for
  return nv < a.max_entries ? nv : a.max_entries;
}

// ------------------------------------------------------------------ scores

__device__ __forceinline__ void hist_add(uint32_t* h, float s) {
  atomicAdd(&h[score_key(s) >> 21], 1u);
}

__device__ __forceinline__ void hist_flush(const uint32_t* lh, uint32_t* gh) {
  for (int bin = threadIdx.x; bin < kHistBins; bin += blockDim.x) {
    uint32_t c = lh[bin];
    if (c) atomicAdd(&gh[bin], c);
  }
}

// bf16, matrix cores.  KS = dI / 32 k-steps.
template <int KS>
__global__ __launch_bounds__(kIdxThreads) void index_score_mfma(IndexParams a) {
  __shared__ uint32_t lh[kHistBins];
  const int r = blockIdx.y;
  const int b = r / a.Tq;
  const int64_t e_base = a.csa_off[b];
  const int64_t nv = row_visible(a, r, a.csa_off[b + 1] - e_base);
  const int64_t c0 = (int64_t)blockIdx.x * a.chunk;
  if (c0 >= nv) return;
  const int64_t c1 = min(c0 + a.chunk, nv);
  const bool do_hist = nv > a.k;
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
      if (col < a.HI) v = *reinterpret_cast<const uint4*>(P + col * a.dI + ks * 32 + grp * 8);
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

  const uint16_t* K = reinterpret_cast<const uint16_t*>(a.ikey) + e_base * a.dI;
  float* S = a.scores + (int64_t)r * a.max_entries;
  constexpr int U = 4;  // tiles in flight per wave
  const int64_t ntile = (c1 - c0 + 15) / 16;
  for (int64_t t0 = wave * U; t0 < ntile; t0 += 4 * U) {
    uint4 kv[U][KS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t e = c0 + (t0 + u) * 16 + col;
      if (e >= c1) e = c1 - 1;  // clamp: stays inside the visible entries
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kv[u][ks] = *reinterpret_cast<const uint4*>(K + e * a.dI + ks * 32 + grp * 8);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // C[head][entry] = P[head][:] . K[entry][:]; lane (col, grp) holds the
      // entry `col` against heads 4*grp .. 4*grp+3
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[ks], __builtin_bit_cast(bf16x8_t, kv[u][ks]), acc, 0, 0, 0);
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) part = fmaf(om[i], fmaxf(acc[i], 0.f), part);
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      const int64_t e = c0 + (t0 + u) * 16 + col;
      if (grp == 0 && t0 + u < ntile && e < c1) {
        S[e] = part;
        if (do_hist) hist_add(lh, part);
      }
    }
  }
  __syncthreads();
  if (do_hist) hist_flush(lh, a.hist + (int64_t)r * kHistBins);
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
  if (c0 >= nv) return;
  const int64_t c1 = min(c0 + a.chunk, nv);
  const bool do_hist = nv > a.k;
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
  if (do_hist) hist_flush(lh, a.hist + (int64_t)r * kHistBins);
}

// ------------------------------------------------------------------ select

// Exclusive prefix sum over the block (256 threads); returns the total in *tot.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tot, uint32_t* sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sm[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    if (w < wave) before += sm[w];
    all += sm[w];
  }
  __syncthreads();
  *tot = all;
  return before + x - v;
}

// Highest bin T with suffix count >= need over a histogram in LDS; returns T
// and the count strictly above T.
__device__ void find_threshold(const uint32_t* h, int nbins, uint32_t need, uint32_t* sm, int* T_out,
                               uint32_t* above_out) {
  const int per = nbins / kSelThreads;
  // thread t owns bins [t*per, (t+1)*per); suffix order = descending bins
  const int t = threadIdx.x;
  uint32_t mine = 0;
  for (int i = 0; i < per; ++i) mine += h[t * per + i];
  // exclusive scan in reversed thread order
  const int rt = kSelThreads - 1 - t;
  // do a scan where the "earlier" threads are those with higher bins
  uint32_t tot;
  // emulate by scanning over reversed index via LDS
  __shared__ uint32_t rev[kSelThreads];
  rev[rt] = mine;
  __syncthreads();
  uint32_t v = rev[t];
  __syncthreads();
  uint32_t ex = block_excl_scan(v, &tot, sm);  // ex = sum of rev[0..t) = bins above thread (kSelThreads-1-t)'s range
  rev[t] = ex;
  __syncthreads();
  uint32_t above_mine = rev[rt];  // count in bins above my range
  __syncthreads();
  if (above_mine < need && above_mine + mine >= need) {
    uint32_t acc = above_mine;
    for (int i = per - 1; i >= 0; --i) {
      uint32_t c = h[t * per + i];
      if (acc + c >= need) {
        *T_out = t * per + i;
        *above_out = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kSelThreads) void topk_select(IndexParams a) {
  __shared__ uint32_t sh[4096];
  __shared__ uint32_t sm[8];
  __shared__ int s_T;
  __shared__ uint32_t s_above, s_flag;
  const int r = blockIdx.y;
  const int cb = blockIdx.x;
  const int b = r / a.Tq;
  const int64_t nv = row_visible(a, r, a.csa_off[b + 1] - a.csa_off[b]);
  int32_t* out = a.idx + (int64_t)r * a.k;
  if (nv <= a.k) {
    if (cb == 0)
      for (int t = threadIdx.x; t < a.k; t += blockDim.x) out[t] = t < nv ? t : -1;
    return;
  }
  const int nblk = (int)((nv + kSelChunk - 1) / kSelChunk);
  if (cb >= nblk) return;

  // threshold bin from the histogram
  const uint32_t* gh = a.hist + (int64_t)r * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) sh[i] = gh[i];
  if (threadIdx.x == 0) { s_T = 0; s_above = 0; }
  __syncthreads();
  find_threshold(sh, kHistBins, (uint32_t)a.k, sm, &s_T, &s_above);
  const uint32_t T = (uint32_t)s_T;
  const uint32_t above = s_above;

  // filter this chunk, index order: thread t owns kSelPerThread consecutive entries
  const float* S = a.scores + (int64_t)r * a.max_entries;
  const int64_t e0 = (int64_t)cb * kSelChunk + (int64_t)threadIdx.x * kSelPerThread;
  uint32_t keys[kSelPerThread];
  uint32_t ns = 0, nc = 0;
#pragma unroll
  for (int i = 0; i < kSelPerThread; ++i) {
    const int64_t e = e0 + i;
    uint32_t key = 0;
    if (e < nv) key = score_key(S[e]);
    keys[i] = key;
    const uint32_t bin = key >> 21;
    if (e < nv) {
      ns += bin > T;
      nc += bin == T;
    }
  }
  uint32_t tot_s, tot_c;
  uint32_t ps = block_excl_scan(ns, &tot_s, sm);
  uint32_t pc = block_excl_scan(nc, &tot_c, sm);
  int32_t* selr = a.sel + ((int64_t)r * a.nblk + cb) * a.selcap;
  uint64_t* candr = a.cand + ((int64_t)r * a.nblk + cb) * kSelChunk;
#pragma unroll
  for (int i = 0; i < kSelPerThread; ++i) {
    const int64_t e = e0 + i;
    if (e >= nv) continue;
    const uint32_t bin = keys[i] >> 21;
    if (bin > T) {
      if (ps < (uint32_t)a.selcap) selr[ps] = (int32_t)e;
      ++ps;
    } else if (bin == T)
      candr[pc++] = ((uint64_t)(keys[i] & 0x1FFFFFu) << 24) | (uint64_t)(0xFFFFFFu - (uint32_t)e);
  }
  if (threadIdx.x == 0) {
    a.nsel[(int64_t)r * a.nblk + cb] = tot_s;
    a.ncand[(int64_t)r * a.nblk + cb] = tot_c;
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t prev = atomicAdd(&a.ticket[r], 1u);
    s_flag = (prev == (uint32_t)nblk - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_flag) return;
  __threadfence();

  // ---- last block of the row: gather selected and candidates in index order
  uint32_t sel_base = 0, cand_base = 0;
  uint64_t* call = a.cand_all + (int64_t)r * a.max_entries;
  for (int blk0 = 0; blk0 < nblk; blk0 += kSelThreads) {
    const int blk = blk0 + threadIdx.x;
    uint32_t cs = 0, cc = 0;
    if (blk < nblk) {
      cs = __atomic_load_n(&a.nsel[(int64_t)r * a.nblk + blk], __ATOMIC_RELAXED);
      cc = __atomic_load_n(&a.ncand[(int64_t)r * a.nblk + blk], __ATOMIC_RELAXED);
    }
    uint32_t ts, tc;
    uint32_t os = block_excl_scan(cs, &ts, sm) + sel_base;
    uint32_t oc = block_excl_scan(cc, &tc, sm) + cand_base;
    if (blk < nblk) {
      const int32_t* src = a.sel + ((int64_t)r * a.nblk + blk) * a.selcap;
      for (uint32_t i = 0; i < cs && i < (uint32_t)a.selcap && os + i < (uint32_t)a.k; ++i) out[os + i] = src[i];
      const uint64_t* srcc = a.cand + ((int64_t)r * a.nblk + blk) * kSelChunk;
      for (uint32_t i = 0; i < cc; ++i) call[oc + i] = srcc[i];
    }
    sel_base += ts;
    cand_base += tc;
  }
  __threadfence_block();
  __syncthreads();
  const uint32_t ncands = cand_base;
  // consistent histogram: above < k <= above + ncands
  if (above >= (uint32_t)a.k || above + ncands < (uint32_t)a.k) {
    for (int t = threadIdx.x; t < a.k; t += blockDim.x) out[t] = -1;
    goto cleanup;
  }
  {
  uint32_t need = (uint32_t)a.k - above;

  // radix select of the need-th largest packed value (all distinct)
  uint64_t prefix = 0, mask = 0;
  const int shifts[4] = {34, 23, 12, 0};
  const int widths[4] = {11, 11, 11, 12};
  for (int pass = 0; pass < 4; ++pass) {
    const int sft = shifts[pass], nb = 1 << widths[pass];
    for (int i = threadIdx.x; i < nb; i += blockDim.x) sh[i] = 0;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < ncands; i += blockDim.x) {
      const uint64_t v = call[i];
      if ((v & mask) == prefix) atomicAdd(&sh[(uint32_t)(v >> sft) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) { s_T = 0; s_above = 0; }
    __syncthreads();
    find_threshold(sh, nb, need, sm, &s_T, &s_above);
    prefix |= (uint64_t)s_T << sft;
    mask |= (uint64_t)(nb - 1) << sft;
    need -= s_above;
  }
  const uint64_t vstar = prefix;  // exactly (k - above) candidates are >= vstar

  // write the chosen candidates in list (index) order
  uint32_t wbase = above;
  for (uint32_t c0 = 0; c0 < ncands; c0 += kSelThreads * 8) {
    uint32_t cnt = 0;
    uint64_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t ci = c0 + threadIdx.x * 8 + i;
      v[i] = ci < ncands ? call[ci] : 0;
      cnt += (ci < ncands && v[i] >= vstar);
    }
    uint32_t tot;
    uint32_t o = block_excl_scan(cnt, &tot, sm) + wbase;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t ci = c0 + threadIdx.x * 8 + i;
      if (ci < ncands && v[i] >= vstar) {
        if (o < (uint32_t)a.k) out[o] = (int32_t)(0xFFFFFFu - (uint32_t)(v[i] & 0xFFFFFFu));
        ++o;
      }
    }
    wbase += tot;
  }
  }
cleanup:
  // leave the workspace clean for the next call
  uint32_t* ghw = a.hist + (int64_t)r * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) ghw[i] = 0;
  if (threadIdx.x == 0) a.ticket[r] = 0;
}

// ------------------------------------------------------------------ host

struct IndexWs {
  size_t scores, hist, ticket, nsel, ncand, sel, cand, cand_all, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static IndexWs index_ws_layout(int rows, int64_t maxN, int k) {
  IndexWs w{};
  const int64_t nblk = (maxN + kSelChunk - 1) / kSelChunk;
  const int64_t selcap = k < kSelChunk ? k : kSelChunk;
  size_t o = 0;
  w.hist = o;     o = align256(o + (size_t)rows * kHistBins * 4);
  w.ticket = o;   o = align256(o + (size_t)rows * 4);
  w.scores = o;   o = align256(o + (size_t)rows * maxN * 4);
  w.nsel = o;     o = align256(o + (size_t)rows * nblk * 4);
  w.ncand = o;    o = align256(o + (size_t)rows * nblk * 4);
  w.sel = o;      o = align256(o + (size_t)rows * nblk * selcap * 4);
  w.cand = o;     o = align256(o + (size_t)rows * nblk * kSelChunk * 8);
  w.cand_all = o; o = align256(o + (size_t)rows * maxN * 8);
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
  a.ticket = reinterpret_cast<uint32_t*>(base + L.ticket);
  a.nsel = reinterpret_cast<uint32_t*>(base + L.nsel);
  a.ncand = reinterpret_cast<uint32_t*>(base + L.ncand);
  a.sel = reinterpret_cast<int32_t*>(base + L.sel);
  a.cand = reinterpret_cast<uint64_t*>(base + L.cand);
  a.cand_all = reinterpret_cast<uint64_t*>(base + L.cand_all);
  a.nblk = (int)((maxN + kSelChunk - 1) / kSelChunk);
  a.selcap = k < kSelChunk ? k : kSelChunk;
  a.idx = idx;
  // score blocks: aim for >= 2 blocks per CU at decode
  int64_t chunk = 512;
  while (chunk < 8192 && ((maxN + chunk - 1) / chunk) * (int64_t)rows > 4096) chunk *= 2;
  a.chunk = (int)chunk;
  return a;
}

int launch_index_score(const void* p, const float* omega, const void* ikey, const int64_t* csa_off,
                       const int32_t* q_pos, int B, int Tq, int HI, int dI, int k, int m, int w, int64_t maxN,
                       float* scores, void* ws, int dtype, hipStream_t stream) {
  IndexParams a = make_params(p, omega, ikey, csa_off, q_pos, B, Tq, HI, dI, k, m, w, maxN, nullptr, scores, ws);
  const int rows = B * Tq;
  dim3 g1((unsigned)((maxN + a.chunk - 1) / a.chunk), (unsigned)rows);
  const bool mfma = dtype == LCA_BF16 && HI <= 16 && (dI % 32) == 0 && dI <= 256;
  if (mfma) {
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

int launch_topk_select(const int64_t* csa_off, const int32_t* q_pos, int B, int Tq, int k, int m, int w,
                       int64_t maxN, int32_t* idx, const float* scores, void* ws, hipStream_t stream) {
  IndexParams a = make_params(nullptr, nullptr, nullptr, csa_off, q_pos, B, Tq, 1, 8, k, m, w, maxN, idx, scores, ws);
  dim3 g2((unsigned)a.nblk, (unsigned)(B * Tq));
  hipLaunchKernelGGL(topk_select, g2, dim3(kSelThreads), 0, stream, a);
  return hipPeekAtLastError() == hipSuccess ? LCA_OK : LCA_ERR_HIP;
}

}  // namespace lca
