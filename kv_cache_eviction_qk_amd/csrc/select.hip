// select.hip -- victims of each KV head under a budget (gfx950).
//
// Scores become order-preserving 32-bit keys (kvev::score_key).  With m
// victims among the candidate slots [0, nc), the victims are the keys below
// the m-th smallest key T, plus the lowest-slot keys equal to T ([SNAP]
// "Tie-breaking": equal scores evict the lower position).  Four launches,
// the heavy ones spread over 1024-slot chunks of every head:
//   hist    chunk: LDS histogram of the top 11 key bits, added into the
//           head's 2048-bin histogram (integer atomics: exact).
//   collect chunk: from the head histogram, the bucket b holding rank m;
//           each wave counts the keys below b in its 256 slots and writes
//           the (key, slot) pairs of bucket b to its own region.
//   refine  head: gathers the candidate regions (into LDS when they fit),
//           radix-selects T and the tie cut (the slot of the last evicted
//           key equal to T), the number of victims of every chunk and its
//           output offset; resets the histogram state for the next call.
//   emit    chunk: marks victims, prefix sums them, writes slot indices at
//           the chunk's offset: ascending order overall.
// Integer throughout: the result depends only on the score bits.
#include <hip/hip_runtime.h>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {
constexpr int kThreads = 256;
constexpr int kChunk = kSelectChunk;         // candidate slots per chunk workgroup
constexpr int kPerThread = kChunk / kThreads;
constexpr int kBins = kSelectBins;           // top 11 key bits
constexpr int kShift = 21;
constexpr int kRefineThreads = 1024;
constexpr int kMaxChunks = kSelectMaxChunks; // chunks per head the refine step indexes
constexpr int kStaged = 6144;                // candidates the refine step keeps in LDS

__device__ __forceinline__ bool head_params(const SelectArgs &P, int u, int &n, int &m, int &nc) {
  n = P.seq_len[u];
  if (n < 0 || n > P.max_slots) return false;
  m = max(0, n - P.budget);
  nc = max(0, n - P.recent);
  return true;
}

// Bucket of the element of 1-based rank `rank` in a 2048-bin histogram in
// LDS, and the count of elements in lower buckets.  Called by every thread
// of a workgroup of 256 or more threads; threads 0..255 own 8 bins each.
__device__ void find_bucket(const uint32_t *h, uint32_t rank, int *s_b, uint32_t *s_below,
                            uint32_t *wave_tot) {
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
  uint32_t mine = 0, incl = 0;
  if (tid < 256) {
#pragma unroll
    for (int i = 0; i < 8; ++i) mine += h[8 * tid + i];
    incl = mine;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) wave_tot[wv] = incl;
  }
  __syncthreads();
  if (tid < 256) {
    uint32_t before = 0;
    for (int w = 0; w < wv; ++w) before += wave_tot[w];
    incl += before;
    const uint32_t excl = incl - mine;
    if (excl < rank && rank <= incl) {
      uint32_t acc = excl;
      int b = 8 * tid;
      while (acc + h[b] < rank) acc += h[b++];
      *s_b = b;
      *s_below = acc;
    }
  }
  __syncthreads();
}

// Radix refinement: the digit at `shift` (bits of `digit_mask`) of the
// element of 1-based rank *rank among the values v with (v & pmask) == prefix;
// hist holds (digit_mask + 1) counters.  One wave finds the digit.
__device__ void pick_digit(const uint32_t *hist, int ndig, uint32_t rank, uint32_t *s_digit,
                           uint32_t *s_rank) {
  const int tid = threadIdx.x;
  if (tid < kWave) {
    const int per = ndig / kWave;  // 2 or 4 digits per lane
    uint32_t c[4] = {0, 0, 0, 0};
    uint32_t mine = 0;
    for (int i = 0; i < per; ++i) {
      c[i] = hist[per * tid + i];
      mine += c[i];
    }
    uint32_t incl = mine;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t t = __shfl_up(incl, o);
      if (tid >= o) incl += t;
    }
    const uint32_t before = incl - mine;
    if (before < rank && rank <= incl) {
      uint32_t r = rank - before;
      int i = 0;
      while (r > c[i]) r -= c[i++];
      *s_digit = (uint32_t)(per * tid + i);
      *s_rank = r;
    }
  }
}

__device__ int block_sum(int v, int *red) {
  const int lane = lane_id(), wv = threadIdx.x / kWave, nw = blockDim.x / kWave;
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) red[wv] = v;
  __syncthreads();
  int t = 0;
  for (int w = 0; w < nw; ++w) t += red[w];
  __syncthreads();
  return t;
}
}  // namespace

__global__ __launch_bounds__(kThreads) void select_hist_kernel(const SelectArgs P) {
  __shared__ uint32_t hl[kBins];
  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  int n, m, nc;
  if (!head_params(P, u, n, m, nc) || m == 0) return;
  const int s0 = c * kChunk;
  if (s0 >= nc) return;
  const int s1 = min(s0 + kChunk, nc);
  for (int i = tid; i < kBins; i += kThreads) hl[i] = 0;
  __syncthreads();
  const float *row = P.score + (size_t)u * P.max_slots;
  for (int s = s0 + tid; s < s1; s += kThreads) atomicAdd(&hl[score_key(row[s]) >> kShift], 1u);
  __syncthreads();
  uint32_t *hg = P.hist + (size_t)u * kBins;
  for (int i = tid; i < kBins; i += kThreads)
    if (hl[i]) atomicAdd(&hg[i], hl[i]);
}

__global__ __launch_bounds__(kThreads) void select_collect_kernel(const SelectArgs P) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t wave_tot[kThreads / kWave];
  __shared__ int s_b;
  __shared__ uint32_t s_below;
  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x, lane = lane_id();
  int n, m, nc;
  if (!head_params(P, u, n, m, nc) || m == 0) return;
  const int s0 = c * kChunk;
  if (s0 >= nc) return;
  const uint32_t *hg = P.hist + (size_t)u * kBins;
  for (int i = tid; i < kBins; i += kThreads) h[i] = hg[i];
  __syncthreads();
  find_bucket(h, (uint32_t)m, &s_b, &s_below, wave_tot);
  const uint32_t b = (uint32_t)s_b;
  // each wave owns a 256-slot sub-chunk and its own candidate region: no
  // atomics, no workgroup barrier
  const int wv = tid / kWave;
  const int subs = P.chunks * 4, sub = c * 4 + wv;
  const float *row = P.score + (size_t)u * P.max_slots;
  uint2 *cand = P.cand + ((size_t)u * subs + sub) * 256;
  const int w0 = s0 + wv * 256;
  uint32_t k = 0;
  int below = 0;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int s = w0 + it * kWave + lane;
    const bool valid = s < nc;
    const uint32_t key = valid ? score_key(row[s]) : 0xffffffffu;
    const uint32_t bk = key >> kShift;
    below += (valid && bk < b) ? 1 : 0;
    const bool take = valid && bk == b;
    const uint64_t mask = __ballot(take);
    if (take) cand[k + ballot_prefix(mask)] = make_uint2(key, (uint32_t)s);
    k += (uint32_t)__popcll(mask);
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) below += __shfl_xor(below, o);
  if (lane == 0) {
    P.cnt_lt[(size_t)u * subs + sub] = below;
    P.ccount[(size_t)u * subs + sub] = k;
  }
}

// One workgroup per head: exact threshold from the candidate lists.
__global__ __launch_bounds__(kRefineThreads) void select_refine_kernel(const SelectArgs P) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t wave_tot[kRefineThreads / kWave];
  __shared__ uint32_t s_digit, s_rank, s_below;
  __shared__ int s_b;
  __shared__ uint32_t chunk_cnt[kMaxChunks];
  __shared__ uint32_t soff[4 * kMaxChunks + 1];
  __shared__ uint2 cl[kStaged];
  const int u = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
  int n, m, nc;
  uint32_t *hg = P.hist + (size_t)u * kBins;
  if (!head_params(P, u, n, m, nc)) {
    if (tid == 0) P.n_victims[u] = -1;
    return;  // inconsistent head: its histogram was not touched
  }
  if (m == 0) {
    if (tid == 0) P.n_victims[u] = 0;
    return;
  }
  const int subs = P.chunks * 4;
  const int live = (nc + kChunk - 1) / kChunk;  // chunks collect wrote
  const int nsub = live * 4;
  const int chunks = P.chunks;
  // one round of independent loads: histogram, candidate counts and the
  // below-bucket counts of this thread's chunk
  uint32_t hv[2], v[4], below_c = 0;
#pragma unroll
  for (int q = 0; q < 2; ++q) hv[q] = hg[tid + q * kRefineThreads];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = tid * 4 + q;
    v[q] = i < nsub ? min(P.ccount[(size_t)u * subs + i], 256u) : 0u;
  }
  if (tid < live) {
#pragma unroll
    for (int q = 0; q < 4; ++q) below_c += (uint32_t)P.cnt_lt[(size_t)u * subs + tid * 4 + q];
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) h[tid + q * kRefineThreads] = hv[q];
  if (tid < chunks) chunk_cnt[tid] = below_c;
  // exclusive scan of the sub-chunk candidate counts (4 per thread)
  {
    uint32_t mine = v[0] + v[1] + v[2] + v[3];
    uint32_t incl = mine;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) wave_tot[wv] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wv; ++w) before += wave_tot[w];
    uint32_t e = before + incl - mine;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = tid * 4 + q;
      if (i < nsub) soff[i] = e;
      e += v[q];
    }
    if (tid == kRefineThreads - 1) soff[nsub] = e;  // total
    __syncthreads();
  }
  const int ncand = (int)soff[nsub];
  const uint2 *cand = P.cand + (size_t)u * subs * 256;
  // candidate i: sub-chunk by binary search over the offsets
  auto cand_at = [&](int i) -> uint2 {
    int lo = 0, hi = nsub - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int)soff[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return cand[(size_t)lo * 256 + (i - (int)soff[lo])];
  };
  const bool staged = ncand <= kStaged;
  if (staged) {
    uint2 t[kStaged / kRefineThreads];
#pragma unroll
    for (int q = 0; q < kStaged / kRefineThreads; ++q) {
      const int i = tid + q * kRefineThreads;
      if (i < ncand) t[q] = cand_at(i);
    }
#pragma unroll
    for (int q = 0; q < kStaged / kRefineThreads; ++q) {
      const int i = tid + q * kRefineThreads;
      if (i < ncand) cl[i] = t[q];
    }
  }
  auto get = [&](int i) -> uint2 { return staged ? cl[i] : cand_at(i); };
  __syncthreads();
  find_bucket(h, (uint32_t)m, &s_b, &s_below, wave_tot);
  const uint32_t bkt = (uint32_t)s_b;
  const uint32_t need = (uint32_t)m - s_below;  // rank of T inside bucket bkt, 1-based

  // radix select over the low 21 bits of the candidates' keys (7 + 7 + 7)
  uint32_t prefix = bkt << kShift, pmask = 0xffffffffu << kShift, rank = need, cnt_t = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = 14 - 7 * pass;
    if (tid < 128) h[tid] = 0;
    __syncthreads();
    for (int i = tid; i < ncand; i += kRefineThreads) {
      const uint32_t key = get(i).x;
      if ((key & pmask) == prefix) atomicAdd(&h[(key >> shift) & 127u], 1u);
    }
    __syncthreads();
    pick_digit(h, 128, rank, &s_digit, &s_rank);
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= 127u << shift;
    rank = s_rank;
    cnt_t = h[s_digit];  // after the last pass: the number of keys equal to T
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t eT = rank;  // keys equal to T that are evicted: the eT lowest slots

  // tie cut: the eT-th smallest slot among the candidates with key T (all of
  // them when every key equal to T is evicted)
  int tie_cut = INT_MAX;
  if (eT < cnt_t) {
    uint32_t sp = 0, sm = 0, srank = eT;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) h[tid] = 0;
      __syncthreads();
      for (int i = tid; i < ncand; i += kRefineThreads) {
        const uint2 cv = get(i);
        if (cv.x == T && (cv.y & sm) == sp) atomicAdd(&h[(cv.y >> shift) & 255u], 1u);
      }
      __syncthreads();
      pick_digit(h, 256, srank, &s_digit, &s_rank);
      __syncthreads();
      sp |= s_digit << shift;
      sm |= 255u << shift;
      srank = s_rank;
      __syncthreads();
    }
    tie_cut = (int)sp;
  }

  // victims per 1024-slot chunk: keys below bucket bkt (counted by collect)
  // plus the candidates below T and the evicted ties
  for (int i = tid; i < ncand; i += kRefineThreads) {
    const uint2 cv = get(i);
    if (cv.y < (uint32_t)nc && (cv.x < T || (cv.x == T && (int)cv.y <= tie_cut)))
      atomicAdd(&chunk_cnt[cv.y / kChunk], 1u);
  }
  __syncthreads();
  // exclusive scan of the chunk counts (chunks <= 1024: one per thread)
  {
    const uint32_t v = tid < chunks ? chunk_cnt[tid] : 0u;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) wave_tot[wv] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wv; ++w) before += wave_tot[w];
    if (tid < chunks) P.chunk_off[(size_t)u * chunks + tid] = before + incl - v;
  }
  if (tid == 0) {
    P.head_sel[u * 4 + 0] = T;
    P.head_sel[u * 4 + 1] = (uint32_t)tie_cut;
    P.n_victims[u] = m;
  }
  // leave the histogram zeroed for the next call
  for (int i = tid; i < kBins; i += kRefineThreads) hg[i] = 0;
}

__global__ __launch_bounds__(kThreads) void select_emit_kernel(const SelectArgs P) {
  __shared__ int wave_tot[kThreads / kWave];
  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  int n, m, nc;
  if (!head_params(P, u, n, m, nc) || m == 0) return;
  const int s0 = c * kChunk;
  if (s0 >= nc) return;
  const int s1 = min(s0 + kChunk, nc);
  const uint32_t T = P.head_sel[u * 4 + 0];
  const int tie_cut = (int)P.head_sel[u * 4 + 1];
  const uint32_t off = P.chunk_off[(size_t)u * P.chunks + c];
  const float *row = P.score + (size_t)u * P.max_slots;
  bool vic[kPerThread];
  int cnt = 0;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int s = s0 + tid * kPerThread + q;
    bool v = false;
    if (s < s1) {
      const uint32_t k = score_key(row[s]);
      v = k < T || (k == T && s <= tie_cut);
    }
    vic[q] = v;
    cnt += v ? 1 : 0;
  }
  const int lane = lane_id(), wv = tid / kWave;
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) wave_tot[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wv; ++w) before += wave_tot[w];
  uint32_t o = off + (uint32_t)(before + incl - cnt);
  int32_t *out = P.victims + (size_t)u * P.max_slots;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q)
    if (vic[q]) {
      if (o < (uint32_t)m) out[o] = s0 + tid * kPerThread + q;
      ++o;
    }
}

hipError_t launch_select(const SelectArgs &a, hipStream_t s) {
  const dim3 grid(a.chunks, a.units);
  hipLaunchKernelGGL(select_hist_kernel, grid, dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_collect_kernel, grid, dim3(kThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_refine_kernel, dim3(a.units), dim3(kRefineThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_emit_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvev
