// kvev_select_head.h -- exact victim threshold of one KV head, computed by a
// single workgroup once the head's 2048-bin histogram of the top 11 key bits
// is complete (a kernel boundary after the histogram's last atomic).
//
// Victims are the m smallest (key, slot) pairs among the candidate slots
// [0, nc): ties on the score evict the lower position first ([SNAP]
// "Tie-breaking").  Writing T for the key of the m-th pair and cut for its
// slot, slot s < nc is a victim iff key < T, or key == T and s <= cut.
//   1. bucket b of rank m from the histogram;
//   2. one pass over the keys: per 1024-slot chunk the count of keys below
//      bucket b, and the (key, slot) pairs of bucket b into LDS;
//   3. two radix passes over those pairs (key bits 20..10, then 9..0) give T
//      and the rank of the m-th pair among the keys equal to T;
//   4. the cut slot: rank counting among the keys equal to T;
//   5. per-chunk victim counts, their exclusive scan (the chunk's first
//      output index), T and cut to the workspace, n_victims; the histogram
//      is left zero for the next call.
// A bucket larger than the LDS list is re-read from the score row instead.
#pragma once

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

constexpr int kHeadCand = 4096;  // bucket pairs kept in LDS
constexpr int kHeadTie = 2048;   // keys equal to T ranked in LDS

struct HeadSelLds {
  uint32_t h[kSelectBins];
  uint32_t chunk_cnt[kSelectMaxChunks];
  uint2 cand[kHeadCand];
  uint32_t wave_tot[16];
  uint32_t s_ncand, s_bin, s_below, s_cut, s_nt;
};

// Inclusive scan of v over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Bin of h[0, nbins) that holds the element of 1-based rank `rank`, and the
// number of elements in lower bins (requires 1 <= rank <= total).  Every
// thread of the workgroup calls it; thread t owns a run of consecutive bins.
__device__ inline void wg_rank_bin(const uint32_t *h, int nbins, uint32_t rank, HeadSelLds &L) {
  const int NT = blockDim.x, tid = threadIdx.x, wv = tid / kWave, lane = lane_id();
  const int per = (nbins + NT - 1) / NT;
  const int b0 = min(tid * per, nbins), b1 = min(b0 + per, nbins);
  uint32_t mine = 0;
  for (int i = b0; i < b1; ++i) mine += h[i];
  uint32_t incl = wave_incl_scan(mine);
  if (tid == 0) {
    L.s_bin = 0;
    L.s_below = 0;
  }
  if (lane == kWave - 1) L.wave_tot[wv] = incl;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wv; ++w) before += L.wave_tot[w];
  incl += before;
  const uint32_t excl = incl - mine;
  if (excl < rank && rank <= incl) {
    uint32_t acc = excl;
    int i = b0;
    while (acc + h[i] < rank) acc += h[i++];
    L.s_bin = (uint32_t)i;
    L.s_below = acc;
  }
  __syncthreads();
}

struct HeadSel {
  const float *score;  // row of this head: score + u * max_slots
  uint32_t *hist;      // 2048 bins of this head (complete on entry)
  int u, m, nc, chunks;
};

// Requires 0 < m < nc.  Call with every thread of the workgroup; uses only
// the LDS it is given.
__device__ inline void head_select(const SelHead &S, const HeadSel &H, HeadSelLds &L) {
  const int NT = blockDim.x, tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
  const int nw = NT / kWave;
  const int nc = H.nc;
  const uint32_t m = (uint32_t)H.m;
  const float *row = H.score;
  const int live = (nc + kSelectChunk - 1) / kSelectChunk;  // chunks with candidates
  const bool al16 = (reinterpret_cast<uintptr_t>(row) & 15) == 0;

  // ---- 1. bucket of rank m
  for (int i = tid; i < kSelectBins; i += NT) L.h[i] = H.hist[i];
  for (int i = tid; i < live; i += NT) L.chunk_cnt[i] = 0;
  if (tid == 0) L.s_ncand = 0;
  __syncthreads();
  wg_rank_bin(L.h, kSelectBins, m, L);
  const uint32_t b = L.s_bin;
  const uint32_t need = m - L.s_below;  // rank of the m-th pair inside bucket b

  // ---- 2. keys below bucket b per chunk; bucket members to LDS.  A wave
  // takes 256 consecutive slots (4 per lane) per step, four steps per round
  // with every load issued first.
  for (int g0 = wv * 256; g0 < nc; g0 += 4 * nw * 256) {
    float4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int s = g0 + k * nw * 256 + lane * 4;
      if (al16 && s + 3 < nc) {
        v[k] = *reinterpret_cast<const float4 *>(row + s);
      } else {
        v[k].x = s + 0 < nc ? row[s + 0] : 0.f;
        v[k].y = s + 1 < nc ? row[s + 1] : 0.f;
        v[k].z = s + 2 < nc ? row[s + 2] : 0.f;
        v[k].w = s + 3 < nc ? row[s + 3] : 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int gs = g0 + k * nw * 256;
      if (gs >= nc) break;
      const int s = gs + lane * 4;
      const float e4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
      uint32_t key[4];
      uint64_t msk[4];
      int below = 0, tot = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = s + e < nc;
        key[e] = score_key(e4[e]);
        const uint32_t bk = key[e] >> 21;
        below += (in && bk < b) ? 1 : 0;
        msk[e] = __ballot(in && bk == b);
        tot += __popcll(msk[e]);
      }
#pragma unroll
      for (int o = kWave / 2; o >= 1; o >>= 1) below += __shfl_xor(below, o);
      uint32_t base = 0;
      if (lane == 0) {
        if (below) atomicAdd(&L.chunk_cnt[gs / kSelectChunk], (uint32_t)below);
        if (tot) base = atomicAdd(&L.s_ncand, (uint32_t)tot);
      }
      base = __shfl(base, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((msk[e] >> lane) & 1ull) {
          const uint32_t p = base + (uint32_t)ballot_prefix(msk[e]);
          if (p < (uint32_t)kHeadCand) L.cand[p] = make_uint2(key[e], (uint32_t)(s + e));
        }
        base += (uint32_t)__popcll(msk[e]);
      }
    }
  }
  __syncthreads();
  const int ncand = (int)L.s_ncand;
  const bool staged = ncand <= kHeadCand;
  // visits every (key, slot) of bucket b: from LDS, or from the score row
  auto for_cand = [&](auto &&f) {
    if (staged) {
      for (int i = tid; i < ncand; i += NT) {
        const uint2 c = L.cand[i];
        f(c.x, (int)c.y);
      }
    } else {
      for (int s = tid; s < nc; s += NT) {
        const uint32_t k = score_key(row[s]);
        if ((k >> 21) == b) f(k, s);
      }
    }
  };

  // ---- 3. radix passes over the bucket: bits 20..10, then 9..0
  for (int i = tid; i < kSelectBins; i += NT) L.h[i] = 0;
  __syncthreads();
  for_cand([&](uint32_t k, int) { atomicAdd(&L.h[(k >> 10) & 2047u], 1u); });
  __syncthreads();
  wg_rank_bin(L.h, 2048, need, L);
  const uint32_t pre = (b << 11) | L.s_bin;  // key >> 10 of T
  const uint32_t need2 = need - L.s_below;
  for (int i = tid; i < 1024; i += NT) L.h[i] = 0;
  __syncthreads();
  for_cand([&](uint32_t k, int) {
    if ((k >> 10) == pre) atomicAdd(&L.h[k & 1023u], 1u);
  });
  __syncthreads();
  wg_rank_bin(L.h, 1024, need2, L);
  const uint32_t T = (pre << 10) | L.s_bin;
  const uint32_t eT = need2 - L.s_below;  // keys equal to T that are victims
  const uint32_t cnt_t = L.h[L.s_bin];     // keys equal to T
  __syncthreads();

  // ---- 4. cut slot: the eT-th smallest slot among the keys equal to T
  int cut = INT_MAX;
  if (eT < cnt_t) {
    if (cnt_t <= (uint32_t)kHeadTie) {
      int *tie = reinterpret_cast<int *>(L.h);
      if (tid == 0) L.s_nt = 0;
      __syncthreads();
      for_cand([&](uint32_t k, int s) {
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
        for_cand([&](uint32_t k, int s) {
          if (k == T && ((uint32_t)s & sm) == sp) atomicAdd(&L.h[((uint32_t)s >> shift) & 255u], 1u);
        });
        __syncthreads();
        wg_rank_bin(L.h, 256, rank, L);
        sp |= L.s_bin << shift;
        sm |= 255u << shift;
        rank -= L.s_below;
        __syncthreads();
      }
      cut = (int)sp;
    }
  }

  // ---- 5. victims per chunk, their offsets, the head's threshold
  for_cand([&](uint32_t k, int s) {
    if (k < T || (k == T && s <= cut)) atomicAdd(&L.chunk_cnt[s / kSelectChunk], 1u);
  });
  __syncthreads();
  {
    const int per = (live + NT - 1) / NT;
    const int c0 = min(tid * per, live), c1 = min(c0 + per, live);
    uint32_t mine = 0;
    for (int c = c0; c < c1; ++c) mine += L.chunk_cnt[c];
    uint32_t incl = wave_incl_scan(mine);
    if (lane == kWave - 1) L.wave_tot[wv] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wv; ++w) before += L.wave_tot[w];
    uint32_t e = before + incl - mine;
    uint32_t *off = S.chunk_off + (size_t)H.u * H.chunks;
    for (int c = c0; c < c1; ++c) {
      off[c] = e;
      e += L.chunk_cnt[c];
    }
  }
  if (tid == 0) {
    S.head_sel[H.u * 4 + 0] = T;
    S.head_sel[H.u * 4 + 1] = (uint32_t)cut;
    S.n_victims[H.u] = H.m;
  }
  for (int i = tid; i < kSelectBins; i += NT) H.hist[i] = 0;
}

}  // namespace kvev
