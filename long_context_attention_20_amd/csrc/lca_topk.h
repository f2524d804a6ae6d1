// Exact top-k selection from the state the index-score and filter kernels
// leave in the index workspace, shared by the top-k finalize kernel and the
// sparse-attention blocks that select their own entries.
//
// Pages: "DeepSeek-V4", Lightning indexer (the query attends to the k
// compressed entries of largest index score).  Ties go to the smaller entry
// index.
//
// Keys: score_key maps a float score to a 32-bit integer of the same order.
// The score kernels build a histogram of the top 11 key bits; the filter
// finds the bin T holding the k-th largest, appends every entry above T to a
// per-row list `sel` (exactly `above` entries) and every entry inside T to a
// candidate list as the packed value
//     (key & 0x1FFFFF) << 24 | (0xFFFFFF - entry)
// (a total order: larger key first, then smaller entry).  Selecting then
// needs the k - above largest packed candidates: the selection counts the
// candidates per next-11-bit bin (bits 20..10 of the key) in LDS, which gives
// their bin T2, and only the candidates inside T2 (usually very few) need
// the exact radix passes over their low 34 bits.
#pragma once
#include "lca_common.h"

namespace lca {

constexpr int kHistBins = 2048;   // first-level bins (top 11 key bits)
constexpr int kH2Bins = 2048;     // second-level bins (key bits 20..10)
constexpr int kBitmapWords = 8192;  // entries covered by the ordering bitmap / 32
constexpr int64_t kBitmapEntries = (int64_t)kBitmapWords * 32;

// Exclusive prefix sum over the block; returns the total in *tot.  sm holds
// one word per wave; the block may reuse it once this returns.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tot, uint32_t* sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) sm[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
  const int nw = (int)(blockDim.x >> 6);
  for (int w = 0; w < nw; ++w) {
    const uint32_t c = sm[w];
    before += w < wave ? c : 0u;
    all += c;
  }
  __syncthreads();
  *tot = all;
  return before + inc - v;
}

// Highest bin T whose suffix count reaches need, over a histogram in LDS
// (nbins a multiple of blockDim.x).  Writes T, the count strictly above T and
// the count of bin T (0, 0, 0 when the histogram holds fewer than need).
// The results are visible to the block on return; the histogram is no longer
// read, so the block may overwrite it.
__device__ inline void find_threshold(const uint32_t* h, int nbins, uint32_t need, uint32_t* sm, int* T_out,
                                      uint32_t* above_out, uint32_t* cnt_out) {
  const int per = nbins / (int)blockDim.x;
  const int t = threadIdx.x;
  uint32_t mine = 0;
  for (int i = 0; i < per; ++i) mine += h[t * per + i];
  if (t == 0) { *T_out = 0; *above_out = 0; *cnt_out = 0; }
  uint32_t tot;
  const uint32_t ex = block_excl_scan(mine, &tot, sm);
  const uint32_t above_mine = tot - ex - mine;  // bins of the threads after this one
  if (above_mine < need && above_mine + mine >= need) {
    uint32_t acc = above_mine;
    for (int i = per - 1; i >= 0; --i) {
      const uint32_t c = h[t * per + i];
      if (acc + c >= need) {
        *T_out = t * per + i;
        *above_out = acc;
        *cnt_out = c;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

// Per-row views of the index workspace.
struct TopkWs {
  const float* scores;           // [rows][max_entries]
  uint32_t* hist;                // [rows][nstripe][kHistBins]
  int nstripe;
  unsigned long long* ctr;       // [rows]: sel count | candidate count << 32
  uint32_t* done;                // [rows]: blocks that finished filtering the row
  int32_t* sel;                  // [rows][k]
  uint64_t* cand;                // [rows][max_entries]
  int64_t max_entries;
  int k;
};

// LDS of filter_chunk.
struct FilterShared {
  uint32_t h[kHistBins];
  uint32_t sm[16];
  int T;
  uint32_t above, cnt;
  unsigned long long base;
};

// The loads of NC filter chunks of a row (histogram stripes and the chunks'
// scores, clamped to the row's columns), issued together; a caller can start
// them before it knows how many of the scores are visible.  Chunk c is chunk
// number cb0 + c * stride of the row (NT * PER scores each).
template <int NT, int PER, int NC = 1>
struct FilterPrefetch {
  static constexpr int kMaxStripes = 8;
  static constexpr int HV = kHistBins / 4 / NT;  // uint4 per thread and stripe
  uint4 hs[kMaxStripes][HV];
  float sv[NC][PER];
};

template <int NT, int PER, int NC>
__device__ __forceinline__ void filter_prefetch(const TopkWs& w, int r, int cb0, int stride,
                                                FilterPrefetch<NT, PER, NC>& P) {
  using FP = FilterPrefetch<NT, PER, NC>;
  static_assert(FP::HV * 4 * NT == kHistBins, "the histogram must split evenly over the block");
  const uint4* gh = reinterpret_cast<const uint4*>(w.hist + (int64_t)r * w.nstripe * kHistBins);
#pragma unroll
  for (int st = 0; st < FP::kMaxStripes; ++st)
#pragma unroll
    for (int i = 0; i < FP::HV; ++i)
      P.hs[st][i] = st < w.nstripe ? gh[st * (kHistBins / 4) + threadIdx.x + i * NT] : make_uint4(0, 0, 0, 0);
  const float* S = w.scores + (int64_t)r * w.max_entries;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int64_t base = (int64_t)(cb0 + c * stride) * NT * PER;
    if (c > 0 && base >= w.max_entries) {  // past every row's columns: never visible (uniform)
#pragma unroll
      for (int i = 0; i < PER; ++i) P.sv[c][i] = 0.f;
      continue;
    }
    const int64_t e0 = base + (int64_t)threadIdx.x * PER;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int64_t e = e0 + i;
      P.sv[c][i] = S[e < w.max_entries ? e : w.max_entries - 1];
    }
  }
}

// A diagnostic hook (sub-phase stamps) that does nothing.
struct NoStamp {
  __device__ void operator()(int) const {}
};

// The filter of NC chunks of row r (k < nv; the first chunk starts below
// nv) from their prefetched loads: the threshold bin T from the row's
// histogram (summed over its stripes), then every entry of the chunks above T
// appended to sel and every entry inside T to the candidate list (packed as
// above).  The list space comes from one 64-bit atomic on ctr for all the
// chunks.  No per-candidate counting here: with many equal scores (a row
// whose head weights are all negative scores thousands of entries exactly 0)
// per-candidate atomics would all hit one word.  (stamp: a diagnostic hook
// called with sub-phase numbers.)

template <int NT, int PER, int NC, class Stamp = NoStamp>
__device__ void filter_chunk(const TopkWs& w, int r, int64_t nv, int cb0, int stride,
                             const FilterPrefetch<NT, PER, NC>& P, FilterShared& F, Stamp stamp = Stamp()) {
  using FP = FilterPrefetch<NT, PER, NC>;
#pragma unroll
  for (int i = 0; i < FP::HV; ++i) {
    uint4 v = P.hs[0][i];
#pragma unroll
    for (int st = 1; st < FP::kMaxStripes; ++st) {
      v.x += P.hs[st][i].x; v.y += P.hs[st][i].y; v.z += P.hs[st][i].z; v.w += P.hs[st][i].w;
    }
    reinterpret_cast<uint4*>(F.h)[threadIdx.x + i * NT] = v;
  }
  __syncthreads();
  stamp(8);
  find_threshold(F.h, kHistBins, (uint32_t)w.k, F.sm, &F.T, &F.above, &F.cnt);
  const uint32_t T = (uint32_t)F.T;
  stamp(9);

  uint32_t keys[NC][PER];
  uint32_t ns = 0, nc = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int64_t e0 = (int64_t)(cb0 + c * stride) * NT * PER + (int64_t)threadIdx.x * PER;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool in = e0 + i < nv;
      keys[c][i] = score_key(P.sv[c][i]);
      const uint32_t bin = keys[c][i] >> 21;
      ns += (in && bin > T) ? 1u : 0u;
      nc += (in && bin == T) ? 1u : 0u;
    }
  }
  uint32_t tot;
  const uint32_t pos = block_excl_scan(ns | (nc << 16), &tot, F.sm);  // both counts < 2^16
  if (threadIdx.x == 0)
    F.base = atomicAdd(&w.ctr[r], (unsigned long long)(tot & 0xFFFFu) | ((unsigned long long)(tot >> 16) << 32));
  __syncthreads();
  stamp(10);
  uint32_t ps = (uint32_t)(F.base & 0xFFFFFFFFull) + (pos & 0xFFFFu);
  uint32_t pc = (uint32_t)(F.base >> 32) + (pos >> 16);
  int32_t* selr = w.sel + (int64_t)r * w.k;
  uint64_t* candr = w.cand + (int64_t)r * w.max_entries;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int64_t e0 = (int64_t)(cb0 + c * stride) * NT * PER + (int64_t)threadIdx.x * PER;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int64_t e = e0 + i;
      if (e >= nv) continue;
      const uint32_t bin = keys[c][i] >> 21;
      if (bin > T) {
        if (ps < (uint32_t)w.k) selr[ps] = (int32_t)e;
        ++ps;
      } else if (bin == T) {
        if (pc < (uint32_t)w.max_entries)
          candr[pc] = ((uint64_t)(keys[c][i] & 0x1FFFFFu) << 24) | (uint64_t)(0xFFFFFFu - (uint32_t)e);
        ++pc;
      }
    }
  }
}

// Visible compressed entries of a query at position i (the entries whose
// window ends at or before i), capped by the sequence and the workspace rows.
__device__ __forceinline__ int64_t topk_visible(int64_t i, int m, int w, int64_t n_seq, int64_t max_entries) {
  int64_t nv = n_windows(i + 1, m, w);
  nv = nv < n_seq ? nv : n_seq;
  return nv < max_entries ? nv : max_entries;
}

constexpr int kBoundaryLds = 256;  // threshold-bin candidates ranked directly
constexpr int kSelLoads = 4;       // candidate loads in flight per thread in the selection's walks

// h[bin] += 1 for every active lane: when all active lanes of the wave count
// the same bin (equal scores, the crowded case) one lane adds their number,
// else each lane adds its own (LDS atomics on one word serialize).
__device__ __forceinline__ void lds_count(uint32_t* h, uint32_t bin) {
  const uint32_t first = __builtin_amdgcn_readfirstlane(bin);
  const uint64_t act = __ballot(1);
  if (__ballot(bin == first) == act) {
    if ((int)(threadIdx.x & 63) == __ffsll((long long)act) - 1) atomicAdd(&h[first], (uint32_t)__popcll(act));
  } else {
    atomicAdd(&h[bin], 1u);
  }
}

// f(ptr[j]) for j = j0, j0 + stride, ... below n, with U loads in flight per
// thread: a walk over a list in global memory is bound by load latency, and
// a crowded threshold bin (many equal scores) makes the candidate list long.
template <int U, typename T, typename F>
__device__ __forceinline__ void walk_loads(const T* ptr, uint32_t j0, uint32_t n, uint32_t stride, F f) {
  for (uint32_t j = j0; j < n; j += stride * U) {
    T v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t jj = j + u * stride;
      v[u] = jj < n ? ptr[jj] : T{};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j + u * stride < n) f(j + u * stride, v[u]);
  }
}

// LDS of topk_row_select (66 KB): radix histogram (for a crowded threshold
// bin), chosen-entry bitmap, chosen entries before each bitmap word, and the
// candidates of the threshold bin.
struct SelectLds {
  uint32_t h[4096];
  uint32_t bitmap[kBitmapWords];
  uint16_t prefix[kBitmapWords];
  uint64_t bl[kBoundaryLds];
};
struct SelectShared {
  uint32_t sm[16];
  int T;
  uint32_t above, cnt, fill, nbl;
  uint64_t vstar;
};

// The loads of topk_row_select whose addresses do not depend on the list
// counts (the counts, the selected list and the first candidates), issued together: a caller can start them before anything
// else it needs, and pass them in.
template <int NT>
struct SelectPrefetch {
  static constexpr int SPT = 4096 / NT;     // selected-list slots per thread (k <= 4096)
  static constexpr int CPT = 2048 / NT;     // candidates per thread before the count is known
  unsigned long long cnt;
  int32_t sv[SPT];
  uint64_t cv[CPT];
};

template <int NT>
__device__ __forceinline__ void topk_prefetch(const TopkWs& w, int r, SelectPrefetch<NT>& P) {
  const int tid = threadIdx.x;
  P.cnt = w.ctr[r];
  const int32_t* selr = w.sel + (int64_t)r * w.k;
#pragma unroll
  for (int i = 0; i < SelectPrefetch<NT>::SPT; ++i) {
    const int j = tid + i * NT;
    P.sv[i] = j < w.k ? selr[j] : -1;
  }
  const uint64_t* cg = w.cand + (int64_t)r * w.max_entries;
#pragma unroll
  for (int i = 0; i < SelectPrefetch<NT>::CPT; ++i) {
    const int64_t j = tid + i * NT;
    P.cv[i] = j < w.max_entries ? cg[j] : 0ull;
  }
}

// Exact top-k of one row straight from its scores, with nothing but a 2048-word
// LDS histogram h and the block scan's scratch: three radix passes over the
// score keys (bits 31..21, 20..10, 9..0) find the k-th largest key v and how
// many entries of key v are taken (the smallest indices among them); a fourth
// pass emits every chosen entry with its rank in ascending index order.  Used
// when the filtered lists cannot be trusted (a bounded wait gave up, or the
// lists are inconsistent); slower than the list selection (four reads of the
// row's scores) but it depends on no other block.  k < nv.
template <int NT, int U, class F>
__device__ __forceinline__ void for_row_keys(const float* S, int64_t nv, F f) {
  for (int64_t base = threadIdx.x; base < nv; base += (int64_t)NT * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = base + (int64_t)u * NT;
      v[u] = e < nv ? S[e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + (int64_t)u * NT < nv) f(score_key(v[u]));
  }
}

template <int NT, class Emit>
__device__ void topk_row_scan_select(const float* S, int64_t nv, uint32_t k, uint32_t* h, SelectShared& sh,
                                     Emit emit) {
  static_assert(kHistBins % NT == 0 && 1024 % NT == 0, "the bins must split evenly over the block");
  constexpr int U = 8;
  // level 1: the top 11 key bits
  for (int i = threadIdx.x; i < kHistBins; i += NT) h[i] = 0;
  __syncthreads();
  for_row_keys<NT, U>(S, nv, [&](uint32_t key) { lds_count(h, key >> 21); });
  __syncthreads();
  find_threshold(h, kHistBins, k, sh.sm, &sh.T, &sh.above, &sh.cnt);
  const uint32_t T1 = (uint32_t)sh.T;
  uint32_t need = k - sh.above;
  // level 2: bits 20..10 inside bin T1
  for (int i = threadIdx.x; i < kHistBins; i += NT) h[i] = 0;
  __syncthreads();
  for_row_keys<NT, U>(S, nv, [&](uint32_t key) {
    if ((key >> 21) == T1) lds_count(h, (key >> 10) & 0x7FFu);
  });
  __syncthreads();
  find_threshold(h, kHistBins, need, sh.sm, &sh.T, &sh.above, &sh.cnt);
  const uint32_t p2 = (T1 << 11) | (uint32_t)sh.T;
  need -= sh.above;
  // level 3: bits 9..0 inside that bin
  for (int i = threadIdx.x; i < 1024; i += NT) h[i] = 0;
  __syncthreads();
  for_row_keys<NT, U>(S, nv, [&](uint32_t key) {
    if ((key >> 10) == p2) lds_count(h, key & 0x3FFu);
  });
  __syncthreads();
  find_threshold(h, 1024, need, sh.sm, &sh.T, &sh.above, &sh.cnt);
  const uint32_t vkey = (p2 << 10) | (uint32_t)sh.T;
  const uint32_t neq = need - sh.above;  // entries of key vkey taken: the first neq in index order
  // emission: thread t takes P consecutive entries of each NT*P chunk; one
  // block scan of (entries above vkey, entries equal to vkey) per chunk
  constexpr int P = 8;
  uint32_t run_gt = 0, run_eq = 0;
  for (int64_t base = 0; base < nv; base += (int64_t)NT * P) {
    const int64_t e0 = base + (int64_t)threadIdx.x * P;
    uint32_t keys[P];
#pragma unroll
    for (int i = 0; i < P; ++i) keys[i] = e0 + i < nv ? score_key(S[e0 + i]) : 0u;
    uint32_t ngt = 0, nq = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const bool in = e0 + i < nv;
      ngt += (in && keys[i] > vkey) ? 1u : 0u;
      nq += (in && keys[i] == vkey) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t pre = block_excl_scan(ngt | (nq << 16), &tot, sh.sm);  // both < 2^16
    uint32_t eq = run_eq + (pre >> 16);
    uint32_t o = run_gt + (pre & 0xFFFFu) + min(eq, neq);
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (e0 + i >= nv) continue;
      if (keys[i] > vkey) {
        emit(o++, (int32_t)(e0 + i));
      } else if (keys[i] == vkey) {
        if (eq < neq) emit(o++, (int32_t)(e0 + i));
        ++eq;
      }
    }
    run_gt += tot & 0xFFFFu;
    run_eq += tot >> 16;
  }
}

template <int NT, bool ORDERED, class Emit, class Stamp = NoStamp>
__device__ uint32_t topk_row_select(const TopkWs& w, int r, const SelectPrefetch<NT>& P, SelectLds& L,
                                    SelectShared& S, Emit emit, uint64_t* cl, uint32_t ncl, Stamp stamp = Stamp()) {
  constexpr int NW = NT / 64;
  constexpr int SPT = SelectPrefetch<NT>::SPT, CPT = SelectPrefetch<NT>::CPT;
  constexpr int HPT = kH2Bins / NT;  // second-level bins per thread
  static_assert(HPT * NT == kH2Bins, "the second-level bins must split evenly over the block");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t k = (uint32_t)w.k;
  const uint64_t* cg = w.cand + (int64_t)r * w.max_entries;
  // every entry above the threshold bin is chosen and the k-th largest lies
  // inside it exactly when n_sel < k <= n_sel + ncands
  const uint32_t n_sel = (uint32_t)(P.cnt & 0xFFFFFFFFull);
  const uint32_t ncands = (uint32_t)(P.cnt >> 32);
  const bool consistent = n_sel < k && (uint64_t)n_sel + ncands >= k && ncands <= (uint64_t)w.max_entries;
  if (!consistent) return 0;
  const uint32_t need = k - n_sel;
  // this thread's candidates: the prefetched ones, then the rest from
  // global memory, which the first pass copies into cl (ncl of them fit, in
  // LDS) and later passes read from there
  const uint32_t nreg = (uint32_t)(CPT * NT);
  const uint32_t nlds = ncands > nreg ? min(ncands - nreg, ncl) : 0u;
  auto for_cands_staging = [&](auto f) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      if ((uint32_t)(tid + i * NT) < ncands) f(P.cv[i]);
    walk_loads<kSelLoads>(cg, (uint32_t)tid + nreg, ncands, (uint32_t)NT, [&](uint32_t j, uint64_t v) {
      if (j - nreg < nlds) cl[j - nreg] = v;
      f(v);
    });
  };
  auto for_cands = [&](auto f) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      if ((uint32_t)(tid + i * NT) < ncands) f(P.cv[i]);
    for (uint32_t j = tid; j < nlds; j += NT) f(cl[j]);
    walk_loads<kSelLoads>(cg, (uint32_t)tid + nreg + nlds, ncands, (uint32_t)NT, [&](uint32_t, uint64_t v) { f(v); });
  };

  // 1. the candidates per second-level bin (key bits 20..10, the top bits
  // of the packed value's low 34), counted in LDS; then the bin T2 whose
  // suffix count reaches need: one block scan (thread t holds bins t*HPT ..)
  for (int i = tid; i < kH2Bins; i += NT) L.h[i] = 0;
  if (tid == 0) { S.T = 0; S.above = 0; S.cnt = 0; S.fill = 0; S.nbl = 0; S.vstar = ~0ull; }
  if (ORDERED)
    for (int i = tid; i < kBitmapWords; i += NT) L.bitmap[i] = 0;
  __syncthreads();
  stamp(12);
  for_cands_staging([&](uint64_t v) { lds_count(L.h, (uint32_t)(v >> 34) & (uint32_t)(kH2Bins - 1)); });
  if (ORDERED) {
    // the selected list is chosen whole
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const uint32_t e = (uint32_t)P.sv[i];
      if ((uint32_t)(tid + i * NT) < n_sel && e < (uint32_t)kBitmapEntries) atomicOr(&L.bitmap[e >> 5], 1u << (e & 31));
    }
  }
  __syncthreads();
  uint32_t hv[HPT];
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < HPT; ++i) {
    hv[i] = L.h[tid * HPT + i];
    mine += hv[i];
  }
  const uint32_t inc = wave_incl_scan(mine);
  if (lane == 63) S.sm[wave] = inc;
  __syncthreads();
  {
    uint32_t later = 0;  // bins of the waves after this one
#pragma unroll
    for (int v = 0; v < NW; ++v) later += v > wave ? S.sm[v] : 0u;
    const uint32_t above_mine = later + (S.sm[wave] - inc);  // bins of the threads after this one
    if (above_mine < need && above_mine + mine >= need) {
      uint32_t acc = above_mine;
#pragma unroll
      for (int i = HPT - 1; i >= 0; --i) {
        const uint32_t c = hv[i];
        if (acc < need && acc + c >= need) {
          S.T = tid * HPT + i;
          S.above = acc;
          S.cnt = c;
        }
        acc += c;
      }
    }
  }
  __syncthreads();
  stamp(13);
  const uint32_t T2 = (uint32_t)S.T;
  const uint32_t need2 = need - S.above, cnt2 = S.cnt;

  // 2. the threshold value vstar: the chosen candidates are those >= vstar
  uint64_t vstar = (uint64_t)T2 << 34;  // every candidate of T2 chosen
  if (cnt2 != need2 && cnt2 <= (uint32_t)kBoundaryLds) {
    // few candidates in T2: rank them against each other (all distinct)
    for_cands([&](uint64_t v) {
      if ((uint32_t)(v >> 34) == T2) {
        const uint32_t slot = atomicAdd(&S.nbl, 1u);
        if (slot < (uint32_t)kBoundaryLds) L.bl[slot] = v;
      }
    });
    __syncthreads();
    // (a count other than cnt2 means an inconsistent candidate list: the
    // chosen total then differs from k and the row is rejected below)
    const uint32_t nb = min(S.nbl, (uint32_t)kBoundaryLds);
    for (uint32_t i = tid; i < nb; i += NT) {
      const uint64_t v = L.bl[i];
      uint32_t gt = 0;
      for (uint32_t j = 0; j < nb; ++j) gt += L.bl[j] > v ? 1u : 0u;
      if (gt == need2 - 1) S.vstar = v;
    }
    __syncthreads();
    vstar = S.vstar;
  } else if (cnt2 != need2) {
    // a crowded bin (ties): radix passes over the low 34 bits inside it
    uint64_t prefix = vstar, mask = (uint64_t)(kH2Bins - 1) << 34;
    uint32_t nd = need2;
    const int shifts[3] = {23, 12, 0};
    const int widths[3] = {11, 11, 12};
    for (int pass = 0; pass < 3; ++pass) {
      const int sft = shifts[pass], nb = 1 << widths[pass];
      for (int i = tid; i < nb; i += NT) L.h[i] = 0;
      __syncthreads();
      for_cands([&](uint64_t v) {
        if ((v & mask) == prefix) lds_count(L.h, (uint32_t)(v >> sft) & (uint32_t)(nb - 1));
      });
      __syncthreads();
      find_threshold(L.h, nb, nd, S.sm, &S.T, &S.above, &S.cnt);
      prefix |= (uint64_t)(uint32_t)S.T << sft;
      mask |= (uint64_t)(nb - 1) << sft;
      nd -= S.above;
      // every value left in the chosen bucket is needed: its lower bound
      // (prefix with zero low bits) is the threshold
      const bool done = S.cnt == nd;
      __syncthreads();
      if (done) break;
    }
    vstar = prefix;
  }

  if constexpr (!ORDERED) {
    // the selected list in its order, then the chosen candidates
#pragma unroll
    for (int i = 0; i < SPT; ++i)
      if ((uint32_t)(tid + i * NT) < n_sel) emit((uint32_t)(tid + i * NT), P.sv[i]);
    for_cands([&](uint64_t v) {
      if (v >= vstar) {
        const uint32_t o = n_sel + atomicAdd(&S.fill, 1u);
        if (o < k) emit(o, (int32_t)(0xFFFFFFu - (uint32_t)(v & 0xFFFFFFu)));
      }
    });
    return k;
  }

  // 3. the chosen candidates into the bitmap, the chosen entries before
  // each bitmap word, then every chosen entry's rank in ascending order
  stamp(14);
  for_cands([&](uint64_t v) {
    if (v >= vstar) {
      const uint32_t e = 0xFFFFFFu - (uint32_t)(v & 0xFFFFFFu);
      if (e < (uint32_t)kBitmapEntries) atomicOr(&L.bitmap[e >> 5], 1u << (e & 31));
    }
  });
  __syncthreads();
  constexpr int WPT = kBitmapWords / NT;
  uint32_t wc[WPT], c = 0;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    wc[i] = __popc(L.bitmap[tid * WPT + i]);
    c += wc[i];
  }
  uint32_t tot;
  uint32_t o = block_excl_scan(c, &tot, S.sm);
  if (tot != k) return 0;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    L.prefix[tid * WPT + i] = (uint16_t)o;
    o += wc[i];
  }
  __syncthreads();
  auto rank_of = [&](uint32_t e) -> uint32_t {
    return (uint32_t)L.prefix[e >> 5] + (uint32_t)__popc(L.bitmap[e >> 5] & ((1u << (e & 31)) - 1u));
  };
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const uint32_t e = (uint32_t)P.sv[i];
    if ((uint32_t)(tid + i * NT) < n_sel && e < (uint32_t)kBitmapEntries) emit(rank_of(e), (int32_t)e);
  }
  for_cands([&](uint64_t v) {
    if (v >= vstar) {
      const uint32_t e = 0xFFFFFFu - (uint32_t)(v & 0xFFFFFFu);
      if (e < (uint32_t)kBitmapEntries) emit(rank_of(e), (int32_t)e);
    }
  });
  return k;
}

}  // namespace lca
