// kvev_select_head.h -- exact victim threshold of each KV head from its
// complete 2048-bin histogram of the top 11 key bits (device code of
// select.hip; the fused path runs the same two kernels).
//
// Victims are the m smallest (key, slot) pairs among the candidate slots
// [0, nc): ties on the score evict the lower position first ([SNAP]
// "Tie-breaking").  Writing T for the key of the m-th pair and cut for its
// slot, slot s < nc is a victim iff key < T, or key == T and s <= cut.
//   collect (4096 slots of a head per 1024-thread workgroup): the bucket b
//           of rank m from the histogram (the keys are already in flight);
//           per 1024-slot chunk the count of keys below b (ballot counts);
//           the (key, slot) pairs of bucket b to this workgroup's region,
//           and the histogram of their key bits 20..10 added into the head's
//           second-level histogram.
//   refine  (one 1024-thread workgroup per head): the sub-bucket of the
//           remaining rank from the second-level histogram; one pass over
//           the bucket's pairs counts the pairs below the sub-bucket per
//           chunk and keeps the sub-bucket's pairs in LDS; a radix pass over
//           key bits 9..0 gives T and the rank of the m-th pair among the
//           keys equal to T; rank counting among those gives the cut slot;
//           per-chunk victim counts and their exclusive scan (each chunk's
//           first output index); T, cut and n_victims to the workspace; both
//           histograms are left zero for the next call.
// Concentrated score distributions put many pairs in one bucket; they are
// streamed once, with eight loads in flight per thread.  A sub-bucket with
// more pairs than LDS holds is re-read from the regions.
#pragma once

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

constexpr int kSelThreads = 1024;   // collect and refine workgroups
constexpr int kHeadCand = 4096;     // bucket pairs refine keeps in LDS
constexpr int kHeadTie = 2048;      // keys equal to T ranked in LDS

// Inclusive scan of v over the 64 lanes of a wave.

struct RankOut {
  uint32_t bin, below;
};

// cnt[idx] += 1 for every lane with pred, one LDS atomic per distinct idx
// among those lanes (pairs that sit next to each other mostly share a
// chunk, and per-lane atomics on one counter would serialise the wave).
// Every lane of the wave must call it.
__device__ __forceinline__ void wave_count_add(uint32_t *cnt, int idx, bool pred) {
  uint64_t pending = __ballot(pred);
  while (pending) {
    const int leader = __ffsll((unsigned long long)pending) - 1;
    const int lidx = __shfl(idx, leader);
    const uint64_t same = __ballot(pred && idx == lidx);
    if (lane_id() == leader) atomicAdd(&cnt[lidx], (uint32_t)__popcll(same));
    pending &= ~same;
  }
}

// Bin of h[0, NBINS) that holds the element of 1-based rank `rank`, and the
// number of elements in lower bins ({0, 0} if the total is below the rank).
// Wave 0 computes: lane l owns NBINS/64 consecutive bins, summed in a
// rotated order (the lanes spread over the LDS banks); the owning lane reads
// its bins into registers at once and finds the bin there.  Every thread of
// the workgroup calls it and leaves after one barrier.
template <int NBINS>
__device__ inline void wg_rank_bin(const uint32_t *h, uint32_t rank, RankOut *out) {
  constexpr int PER = NBINS / kWave;
  static_assert(PER >= 1 && (PER & (PER - 1)) == 0, "bins per lane: a power of two");
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int b0 = lane * PER;
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) mine += h[b0 + ((i + lane) & (PER - 1))];
    const uint32_t incl = wave_incl_scan(mine);
    const uint32_t excl = incl - mine;
    const bool own = excl < rank && rank <= incl;
    if (own) {
      uint32_t x[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) x[i] = h[b0 + i];
      uint32_t acc = excl, bin = (uint32_t)(b0 + PER - 1);
      bool found = false;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        if (!found && acc + x[i] >= rank) {
          bin = (uint32_t)(b0 + i);
          found = true;
        }
        if (!found) acc += x[i];
      }
      out->bin = bin;
      out->below = acc;
    }
    if (__ballot(own) == 0 && lane == 0) *out = RankOut{0, 0};
  }
  __syncthreads();
}

// ---------------------------------------------------------------- collect

struct CollectLds {
  uint32_t h[kSelectBins];
  uint32_t cb[kHistChunk / kSelectChunk];  // keys below the bucket per chunk
  RankOut r;
  uint32_t s_ncand;
};

// Workgroup c of head u: slots [c*4096, c*4096 + 4096) of [0, nc).
__device__ inline void collect_chunk(const SelHead &S, const float *row, const uint32_t *hist,
                                     int u, int c, int m, int nc, int max_slots, CollectLds &L) {
  constexpr int NT = kSelThreads;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
  const int s0 = c * kHistChunk;
  // the histogram first, then this thread's four keys (in flight meanwhile)
  uint32_t hv[kSelectBins / NT];
#pragma unroll
  for (int q = 0; q < kSelectBins / NT; ++q) hv[q] = hist[tid + q * NT];
  // 16-byte aligned rows of a multiple of 16 floats: the clamped float4 is
  // inside the row (slots past nc are masked below)
  const float4 v = *reinterpret_cast<const float4 *>(row + min(s0 + 4 * tid, max_slots - 4));
#pragma unroll
  for (int q = 0; q < kSelectBins / NT; ++q) L.h[tid + q * NT] = hv[q];
  if (tid < kHistChunk / kSelectChunk) L.cb[tid] = 0;
  if (tid == 0) L.s_ncand = 0;
  __syncthreads();
  wg_rank_bin<kSelectBins>(L.h, (uint32_t)m, &L.r);
  const uint32_t b = L.r.bin;
  if (c == 0 && tid == 0) {
    S.head_sel[u * 4 + 2] = b;
    S.head_sel[u * 4 + 3] = L.r.below;
  }
  // L.h becomes the histogram of key bits 20..10 over the bucket's pairs
#pragma unroll
  for (int q = 0; q < kSelectBins / NT; ++q) L.h[tid + q * NT] = 0;
  __syncthreads();
  // a wave covers 256 consecutive slots: one chunk
  const int s = s0 + 4 * tid;
  const float e4[4] = {v.x, v.y, v.z, v.w};
  uint32_t key[4];
  uint64_t msk[4];
  uint32_t below = 0, total = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool in = s + e < nc;
    key[e] = score_key(e4[e]);
    const uint32_t bk = key[e] >> 21;
    below += (uint32_t)__popcll(__ballot(in && bk < b));
    msk[e] = __ballot(in && bk == b);
    total += (uint32_t)__popcll(msk[e]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if ((msk[e] >> lane) & 1ull) atomicAdd(&L.h[(key[e] >> 10) & 2047u], 1u);
  uint32_t base = 0;
  if (lane == 0) {
    if (below) atomicAdd(&L.cb[wv / (kSelectChunk / 256)], below);
    if (total) base = atomicAdd(&L.s_ncand, total);
  }
  base = __builtin_amdgcn_readfirstlane(base);
  uint2 *cand = S.cand + ((size_t)u * S.nwg + c) * kHistChunk;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if ((msk[e] >> lane) & 1ull)
      cand[base + (uint32_t)ballot_prefix(msk[e])] = make_uint2(key[e], (uint32_t)(s + e));
    base += (uint32_t)__popcll(msk[e]);
  }
  __syncthreads();
  if (tid == 0) S.ccount[(size_t)u * S.nwg + c] = L.s_ncand;
  uint32_t *h2 = S.hist2 + (size_t)u * kSelectBins;
#pragma unroll
  for (int q = 0; q < kSelectBins / NT; ++q)
    if (L.h[tid + q * NT]) atomicAdd(&h2[tid + q * NT], L.h[tid + q * NT]);
  if (tid < kHistChunk / kSelectChunk) {
    const int ch = s0 / kSelectChunk + tid;
    if (ch * kSelectChunk < nc) S.chunk_below[(size_t)u * S.chunks + ch] = L.cb[tid];
  }
}

// ----------------------------------------------------------------- refine

struct RefineLds {
  uint32_t h[kSelectBins];
  uint32_t chunk_cnt[kSelectMaxChunks];
  uint32_t coff[kSelectMaxChunks / (kHistChunk / kSelectChunk) + 1];  // region offsets
  uint2 cand[kHeadCand];  // the sub-bucket's pairs
  RankOut r;
  uint32_t s_cut, s_nt, s_nsub;
};

// One workgroup per head, after collect.  Requires 0 < m < nc.
__device__ inline void refine_head(const SelHead &S, uint32_t *hist, int u, int m, int nc,
                                   RefineLds &L) {
  constexpr int NT = kSelThreads;
  constexpr int kBatch = 8;  // pair loads in flight per thread
  const int tid = threadIdx.x, lane = lane_id();
  const int live = (nc + kSelectChunk - 1) / kSelectChunk;  // chunks with candidates
  const int nw = (nc + kHistChunk - 1) / kHistChunk;        // collect regions written
  uint32_t *h2 = S.hist2 + (size_t)u * kSelectBins;
  uint32_t h2v[kSelectBins / NT];
#pragma unroll
  for (int q = 0; q < kSelectBins / NT; ++q) h2v[q] = h2[tid + q * NT];
  const uint32_t b = S.head_sel[u * 4 + 2];
  const uint32_t need = (uint32_t)m - S.head_sel[u * 4 + 3];  // rank inside bucket b
  const uint32_t *cc = S.ccount + (size_t)u * S.nwg;
  const uint2 *reg = S.cand + (size_t)u * S.nwg * kHistChunk;
  // counts: the chunks' below-bucket counts, the regions' pair counts
  for (int i = tid; i < live; i += NT) L.chunk_cnt[i] = S.chunk_below[(size_t)u * S.chunks + i];
  if (tid < kWave) {  // exclusive scan of the region counts (nw <= 256: 4 per lane)
    const int per = (nw + kWave - 1) / kWave;
    const int w0 = min(lane * per, nw), w1 = min(w0 + per, nw);
    uint32_t mine = 0;
    for (int w = w0; w < w1; ++w) mine += min(cc[w], (uint32_t)kHistChunk);
    uint32_t e = wave_incl_scan(mine) - mine;
    for (int w = w0; w < w1; ++w) {
      L.coff[w] = e;
      e += min(cc[w], (uint32_t)kHistChunk);
    }
    if (lane == kWave - 1) L.coff[nw] = e;
  }
#pragma unroll
  for (int q = 0; q < kSelectBins / NT; ++q) {
    L.h[tid + q * NT] = h2v[q];
    h2[tid + q * NT] = 0;  // state for the next call
  }
  if (tid == 0) L.s_nsub = 0;
  __syncthreads();
  const int ncand = (int)L.coff[nw];
  // the sub-bucket: key bits 20..10 of the pair of rank `need` in bucket b
  wg_rank_bin<kSelectBins>(L.h, need, &L.r);
  const uint32_t pre = (b << 11) | L.r.bin;  // key >> 10 of T
  const uint32_t need2 = need - L.r.below;

  // pair i: its region by binary search over the offsets, starting from the
  // region of this thread's previous pair (its indices only grow)
  auto pair_at = [&](int i, int &lo) -> uint2 {
    int hi = nw - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int)L.coff[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return reg[(size_t)lo * kHistChunk + (i - (int)L.coff[lo])];
  };
  // every pair of the bucket, kBatch loads in flight per thread
  auto for_all = [&](auto &&f) {
    int lo = 0;
    for (int i0 = 0; i0 < ncand; i0 += kBatch * NT) {
      uint2 t[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int i = i0 + q * NT + tid;
        t[q] = i < ncand ? pair_at(i, lo) : make_uint2(0u, 0u);
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q)
        if (i0 + q * NT + tid < ncand) f(t[q].x, (int)t[q].y);
    }
  };
  // ---- one pass over the bucket: pairs below the sub-bucket are victims
  // (counted per chunk); the sub-bucket's pairs go to LDS (wave-uniform
  // loop: the counts and appends are aggregated per wave)
  {
    int lo = 0;
    for (int i0 = 0; i0 < ncand; i0 += kBatch * NT) {
      uint2 t[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int i = i0 + q * NT + tid;
        t[q] = i < ncand ? pair_at(i, lo) : make_uint2(0u, 0u);
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const bool valid = i0 + q * NT + tid < ncand;
        const uint32_t p = t[q].x >> 10;
        wave_count_add(L.chunk_cnt, (int)t[q].y / kSelectChunk, valid && p < pre);
        const bool sub = valid && p == pre;
        const uint64_t sm = __ballot(sub);
        if (sm) {
          uint32_t base = 0;
          if (lane == 0) base = atomicAdd(&L.s_nsub, (uint32_t)__popcll(sm));
          base = __shfl(base, 0);
          const uint32_t j = base + (uint32_t)ballot_prefix(sm);
          if (sub && j < (uint32_t)kHeadCand) L.cand[j] = t[q];
        }
      }
    }
  }
  for (int i = tid; i < 1024; i += NT) L.h[i] = 0;
  __syncthreads();
  const int nsub = (int)L.s_nsub;
  const bool in_lds = nsub <= kHeadCand;
  auto for_sub = [&](auto &&f) {
    if (in_lds) {
      for (int i = tid; i < nsub; i += NT) f(L.cand[i].x, (int)L.cand[i].y);
    } else {
      for_all([&](uint32_t k, int s) {
        if ((k >> 10) == pre) f(k, s);
      });
    }
  };

  // ---- radix pass over the sub-bucket: key bits 9..0
  for_sub([&](uint32_t k, int) { atomicAdd(&L.h[k & 1023u], 1u); });
  __syncthreads();
  wg_rank_bin<1024>(L.h, need2, &L.r);
  const uint32_t T = (pre << 10) | L.r.bin;
  const uint32_t eT = need2 - L.r.below;  // keys equal to T that are victims
  const uint32_t cnt_t = L.h[L.r.bin];     // keys equal to T
  __syncthreads();

  // ---- cut slot: the eT-th smallest slot among the keys equal to T
  int cut = INT_MAX;
  if (eT < cnt_t) {
    if (cnt_t <= (uint32_t)kHeadTie) {
      int *tie = reinterpret_cast<int *>(L.h);
      if (tid == 0) L.s_nt = 0;
      __syncthreads();
      for_sub([&](uint32_t k, int s) {
        if (k == T) tie[atomicAdd(&L.s_nt, 1u)] = s;
      });
      __syncthreads();
      for (int i = tid; i < (int)cnt_t; i += NT) {
        const int si = tie[i];
        uint32_t r = 0;
        for (int j = 0; j < (int)cnt_t; ++j) r += tie[j] < si ? 1u : 0u;
        if (r == eT - 1) L.s_cut = (uint32_t)si;
      }
      __syncthreads();
      cut = (int)L.s_cut;
    } else {
      // many equal keys: radix over the slot bits (4 x 8)
      uint32_t sp = 0, sm = 0, rank = eT;
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < 256; i += NT) L.h[i] = 0;
        __syncthreads();
        for_sub([&](uint32_t k, int s) {
          if (k == T && ((uint32_t)s & sm) == sp) atomicAdd(&L.h[((uint32_t)s >> shift) & 255u], 1u);
        });
        __syncthreads();
        wg_rank_bin<256>(L.h, rank, &L.r);
        sp |= L.r.bin << shift;
        sm |= 255u << shift;
        rank -= L.r.below;
        __syncthreads();
      }
      cut = (int)sp;
    }
  }

  // ---- victims of the sub-bucket per chunk, the offsets, the threshold
  if (in_lds) {
    for (int i0 = 0; i0 < nsub; i0 += NT) {  // wave-uniform
      const int i = i0 + tid;
      const uint2 c2 = i < nsub ? L.cand[i] : make_uint2(0u, 0u);
      const bool v = i < nsub && (c2.x < T || (c2.x == T && (int)c2.y <= cut));
      wave_count_add(L.chunk_cnt, (int)c2.y / kSelectChunk, v);
    }
  } else {
    for_sub([&](uint32_t k, int s) {
      if (k < T || (k == T && s <= cut)) atomicAdd(&L.chunk_cnt[s / kSelectChunk], 1u);
    });
  }
  __syncthreads();
  if (tid < kWave) {  // one wave: exclusive scan of the chunk counts
    const int per = (live + kWave - 1) / kWave;
    const int c0 = min(lane * per, live), c1 = min(c0 + per, live);
    uint32_t mine = 0;
    for (int c = c0; c < c1; ++c) mine += L.chunk_cnt[c];
    uint32_t e = wave_incl_scan(mine) - mine;
    uint32_t *off = S.chunk_off + (size_t)u * S.chunks;
    for (int c = c0; c < c1; ++c) {
      off[c] = e;
      e += L.chunk_cnt[c];
    }
  }
  if (tid == 0) {
    S.head_sel[u * 4 + 0] = T;
    S.head_sel[u * 4 + 1] = (uint32_t)cut;
    S.n_victims[u] = m;
  }
  for (int i = tid; i < kSelectBins; i += NT) hist[i] = 0;
}

}  // namespace kvev
