// finish.hip -- selection and in-place compaction of the fused eviction pass,
// in one launch after the scoring pass (gfx950).
//
// The scoring pass has written every live slot's eviction score to a
// workspace row and added the top 11 bits of each candidate's order key to
// its head's histogram.  Each KV head then gets kh workgroups of 1024
// threads, parts k = 0 .. kh - 1.
//
//  1. Threshold.  From the histogram every workgroup of the head knows the
//     bucket b holding the m-th smallest key.  The key T and the cut slot of
//     the m-th smallest (key, slot) pair then come from the bucket's members:
//     the histogram of their key bits 20..10 gives the sub-bucket, a radix
//     pass over the last 10 bits gives T, rank counting among equal keys the
//     cut.  Victims are the candidates with key < T, or key == T and slot <=
//     cut: equal scores evict the lower position ([SNAP] "Tie-breaking").
//     A head of at most kRes groups (32768 slots) is selected locally: each
//     of its workgroups holds all its keys in registers and finds T, the cut
//     and the victims per 1024-slot chunk itself, with no exchange.  A longer
//     head shares the work in two rounds over each workgroup's share of the
//     slots: first the histogram of the bucket members' key bits 20..10 is
//     summed over the head (one arrival), which gives the sub-bucket; then
//     each workgroup publishes its chunks' victim counts (keys below b and
//     members below the sub-bucket) and the sub-bucket's keys, and after a
//     second arrival every workgroup reads them all.
//  2. Victim list.  Each workgroup writes the victims of its share's groups
//     at their offsets, in ascending slot order.
//  3. Compaction ([H2O] "PagedAttention Memory Integration"; [VTOK] section
//     3.3 stage 3: destinations filled in logical order).  Batches k, k + kh,
//     ... of 256 destination ranks.  A batch finds the kept slots of its
//     ranks, loads their K, V and pos, and then marks itself "read"; before
//     storing into its destination slots it waits for the marks of the
//     batches that read those slots.  A kept row only moves down (rank <=
//     slot), so those are this batch or lower ones.  Nothing is staged: only
//     the moved rows are read and written.
//  4. The last workgroup of a head appends its emptied tail blocks
//     [ceil(n'/16), ceil(n/16)) to the free list in (b, h, block) order and
//     clears their table entries ([VTOK] section 3.5, I2 and I4).  The last
//     workgroup of the launch sets seq_len, the free count and the stats,
//     and leaves the state words zero for the next call.
//
// Waits and hand-offs.  A workgroup waits only for workgroups of its own
// head: for the marks of lower batches, and, when the head shares its
// selection, twice at the head's arrival counter.  When every head is selected
// locally (max_slots <= 32768), a workgroup's head and part come from its
// index, so its loads go out at once and, as dispatch deals workgroups to the
// 8 XCDs round robin, a head's workgroups share one XCD's L2; its batches
// come from a per-head ticket taken before the compaction, so a batch waits
// only for batches that running workgroups have claimed.  Otherwise a
// launch-wide ticket, taken in dispatch order, names the head and part: when
// a workgroup of a later head is resident every workgroup of this head has
// been dispatched, and a head needs only kh workgroups at once.  Every wait
// ends (each also has a spin limit, status bit 8, so no wave can loop
// forever).  Published values are
// written with agent-scope atomic stores and read with agent-scope atomic
// loads (both bypass the per-XCD L2, which is not coherent across XCDs), and
// the arrival add is issued after s_waitcnt has seen every one of those
// stores complete; the reader issues its loads only after its poll of the
// counter has returned.  A release / acquire pair would order the same
// accesses through the memory model, but on gfx950 an agent-scope release
// writes back the whole L2: one per workgroup over 256 workgroups cost
// 9 us.  A batch's "read" mark carries no data: it is stored after the
// batch's loads have returned (s_waitcnt), so no store can reach a row
// before its reader holds it.
//
// A head whose length is out of range gets n_victims = -1 and is left alone
// (status bit 2).  A head where the scoring pass met a block id outside the
// pool gets its victim list but no compaction (status bit 1).  A head that
// loses nothing keeps its tokens.  The output score row receives the
// compacted scores [0, n') of every head that was scored.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kvev_device.h"
#include "kvev_kernels.h"
#include "kvev_select_head.h"

namespace kvev {

namespace {

constexpr int kFT = 1024;               // threads per workgroup
constexpr int kFW = kFT / kWave;        // waves
constexpr int kGrp = 4 * kFT;           // slots per group: 4 consecutive slots per thread
constexpr int kRes = 8;                 // groups of a share whose keys stay in registers
constexpr int kBatchRanks = 256;        // destination ranks per batch
constexpr int kMem = 4096;              // sub-bucket members kept in LDS
constexpr int kTie = 2048;              // keys equal to T ranked by counting
constexpr int kPreBlk = 2048;           // block ids held in LDS (a head of kRes groups: all)
constexpr unsigned kSpinLimit = 1u << 20;  // polls of a wait before it gives up (status bit 8)
constexpr int kMaxHeadParts = 128;      // workgroups of one head (see finish_parts)

constexpr int kChunk = kSelectChunk;    // victim offsets are kept per 1024-slot chunk
constexpr int kMaxChunks = kSelectMaxChunks;

struct FinLds {
  uint32_t h[kSelectBins];           // key histogram (top bits, then reused)
  uint32_t h2[kSelectBins];          // key bits 20..10 of the bucket's members
  uint32_t cv[kMaxChunks + 1];       // victims per chunk, then victims before each chunk
  uint2 sub[kMem];                   // the sub-bucket's members
  int32_t blk[kPreBlk];              // block ids of the batch's first source groups
  int32_t src[kBatchRanks];          // source slot of each rank of a batch
  int32_t sblk[kBatchRanks];         // source block id of each rank (-1: stays)
  int32_t dblk[kBatchRanks / kBlock];  // destination block ids of the batch
  int32_t wsum[2][kFW];              // chunk_scan's wave totals (two rows, alternating)
  int32_t rtot[kFW];                 // rank_bin_all's scan scratch
  RankOut r;
  uint32_t ticket, nsub, nt, cut;
  int32_t moved, at_risk, last;
  unsigned long long pre_w[2][kFW];   // freed_prefix's wave sums
};

__device__ __forceinline__ int blocks_of(int n) { return (n + kBlock - 1) / kBlock; }

__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint2 ld_agent2(const uint2 *p) {
  const unsigned long long v =
      __hip_atomic_load(reinterpret_cast<const unsigned long long *>(p), __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_AGENT);
  return make_uint2((uint32_t)v, (uint32_t)(v >> 32));
}
__device__ __forceinline__ void st_agent2(uint2 *p, uint2 v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long *>(p),
                     (unsigned long long)v.x | ((unsigned long long)v.y << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
// Every earlier memory access of this thread has completed.
__device__ __forceinline__ void wait_mem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Exclusive prefix sum of v over the threads of this thread's 1024-slot
// chunk of a group (4 slots a thread: a chunk is 4 waves, wave w in chunk
// w / 4): the wave's own prefix plus the totals of the chunk's earlier waves,
// through LDS with one barrier (every thread must call).  Consecutive calls
// alternate between the two rows of wsum (*parity flips), so a call never
// overwrites totals that a slower thread still reads from the previous one.
__device__ int chunk_scan(int v, int (*wsum)[kFW], int *parity) {
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  const int incl = (int)wave_incl_scan((uint32_t)v);
  int *row = wsum[*parity];
  *parity ^= 1;
  if (lane == kWave - 1) row[wv] = incl;
  __syncthreads();
  int before = incl - v;
#pragma unroll
  for (int w = 0; w < 3; ++w)
    if ((wv & ~3) + w < wv) before += row[(wv & ~3) + w];
  return before;
}

// The bin holding the rank-th smallest key (1-based) of a histogram of NBINS
// bins, and the count below it, by the whole workgroup: PER bins a thread,
// a wave scan, the waves' totals through LDS.  out = {0, 0} when no bin holds
// it (rank 0 or above the total).  Ends with a barrier.
template <int NBINS>
__device__ void rank_bin_all(const uint32_t *h, uint32_t rank, RankOut *out, int *wtot) {
  constexpr int PER = NBINS >= kFT ? NBINS / kFT : 1;
  static_assert(PER == 1 || PER == 2, "one or two bins a thread");
  // (the 2048-bin steps and the last 10 bits' 1024 bins; the tie ranks'
  // 256-bin steps stay on one wave)
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
  const bool act = tid * PER < NBINS;
  uint32_t x[PER], mine = 0;
  if constexpr (PER == 2) {
    const uint2 v = act ? *reinterpret_cast<const uint2 *>(h + 2 * tid) : make_uint2(0u, 0u);
    x[0] = v.x;
    x[1] = v.y;
  } else {
    x[0] = act ? h[tid] : 0u;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) mine += x[i];
  uint32_t incl = wave_incl_scan(mine);
  if (lane == kWave - 1) wtot[wv] = (int)incl;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kFW; ++w) {
    const uint32_t t = (uint32_t)wtot[w];
    before += w < wv ? t : 0u;
    total += t;
  }
  incl += before;
  const uint32_t excl = incl - mine;
  if (act && excl < rank && rank <= incl) {
    uint32_t acc = excl, bin = (uint32_t)(tid * PER + PER - 1);
    bool found = false;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (!found && acc + x[i] >= rank) {
        bin = (uint32_t)(tid * PER + i);
        found = true;
      }
      if (!found) acc += x[i];
    }
    out->bin = bin;
    out->below = acc;
  }
  if (tid == 0 && !(rank > 0 && rank <= total)) *out = RankOut{0, 0};
  __syncthreads();
}

// The (head, part) of a ticket.  With the heads a multiple of 8, ticket t
// goes to head (t % 8) * (units / 8) + (t / 8) / kh, part (t / 8) % kh: when
// tickets follow dispatch order, which deals workgroups to the 8 XCDs round
// robin, XCD x runs the heads [x * units/8, (x+1) * units/8), the heads whose
// tiles the score kernel ran there, so each head's scores and histogram are
// read from the L2 that took their writes.  A head's tickets lie within 8 * kh
// consecutive ones, and within a head the parts' tickets increase with the
// part, which is all the waits need.
__device__ __forceinline__ void ticket_head(int t, int units, int kh, int &u, int &k) {
  if (units % 8 == 0) {
    const int slot = t >> 3;
    u = (t & 7) * (units / 8) + slot / kh;
    k = slot % kh;
  } else {
    u = t / kh;
    k = t % kh;
  }
}

// Adds 1 to cv[c] for every lane with `take`: one atomic for the wave when its
// valid lanes share one chunk (members arrive in slot order, so they usually
// do), else one a lane.  Every lane of the wave calls it; lane 0 is valid
// whenever any lane is.
__device__ __forceinline__ void count_chunk(uint32_t *cv, bool valid, bool take, uint32_t c) {
  const uint32_t c0 = (uint32_t)__shfl((int)c, 0);
  const uint64_t t = __ballot(take);
  if (__all(!valid || c == c0)) {
    if (lane_id() == 0 && t) atomicAdd(&cv[c0], (uint32_t)__popcll(t));
  } else if (take) {
    atomicAdd(&cv[c], 1u);
  }
}

// Wave 0 polls *p until it reads at least `want` (the caller then barriers).
__device__ void wait_count(const uint32_t *p, uint32_t want, unsigned long long *acc) {
  if (threadIdx.x >= kWave) return;
  unsigned spins = 0;
  while (ld_agent(p) < want) {
    if (++spins > kSpinLimit) {
      if (threadIdx.x == 0) atomicOr(&acc[3], 8ull);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// The free-list offset of head u (blocks freed by the heads before it) and
// the total over all heads; a head frees blocks when its length is in range,
// it loses tokens and the scoring pass met no bad block id.  The loads are
// issued by freed_prefix_load; every thread calls both.
struct Prefix {
  long long b, t;
};
__device__ __forceinline__ int head_freed(const FinishArgs &P, int n, int e) {
  if (n < 0 || n > P.max_slots || e != 0) return 0;
  const int m = max(0, n - P.budget);
  return m > 0 ? blocks_of(n) - blocks_of(n - m) : 0;
}
// pn, pe: the length and error flag of head threadIdx.x, loaded earlier
// when there are at most kFT heads (one head a thread), else ignored.
__device__ Prefix freed_prefix_load(const FinishArgs &P, int u, int pn, int pe) {
  Prefix x{0, 0};
  if (P.units <= kFT) {
    const int i = threadIdx.x;
    const int fr = i < P.units ? head_freed(P, pn, pe) : 0;
    x.t = fr;
    x.b = i < u ? fr : 0;
    return x;
  }
  for (int i = threadIdx.x; i < P.units; i += kFT) {
    const int fr = head_freed(P, P.seq_len[i], P.head_err[i]);
    x.t += fr;
    x.b += i < u ? fr : 0;
  }
  return x;
}
// One barrier: per-wave sums through LDS.  Where units * max_blocks stays
// below 2^31 (every shape in practice) the wave sums are 32-bit prefix sums
// on DPP lane moves; otherwise 64-bit sums over lane shuffles, so that an
// inconsistent table (a total above the pool) cannot wrap around.
__device__ void freed_prefix(const FinishArgs &P, Prefix x, FinLds &L, long long &before,
                             long long &total) {
  const int wv = threadIdx.x / kWave;
  unsigned long long bw, tw;
  if ((long long)P.units * P.max_blocks < (1ll << 31)) {
    bw = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan((uint32_t)x.b), kWave - 1);
    tw = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan((uint32_t)x.t), kWave - 1);
  } else {
    long long b = x.b, t = x.t;
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) {
      b += __shfl_xor(b, o);
      t += __shfl_xor(t, o);
    }
    bw = (unsigned long long)b;
    tw = (unsigned long long)t;
  }
  if (lane_id() == 0) {
    L.pre_w[0][wv] = bw;
    L.pre_w[1][wv] = tw;
  }
  __syncthreads();
  unsigned long long sb = 0, st = 0;
#pragma unroll
  for (int w = 0; w < kFW; ++w) {
    sb += L.pre_w[0][w];
    st += L.pre_w[1][w];
  }
  before = (long long)sb;
  total = (long long)st;
}

// PR: 16-byte pieces of one K (or V) row (8, 16 or 32); SPEC: every head
// fits the local selection (PR <= 16 and max_slots <= kRes * kGrp), so a
// workgroup's head and part come from its index.
template <int PR, bool SPEC>
__global__ __launch_bounds__(kFT) void evict_finish_kernel(const FinishArgs P) {
  extern __shared__ __align__(16) uint8_t smem[];
  FinLds &L = *reinterpret_cast<FinLds *>(smem);
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;

  // Every head of at most kRes groups (the whole launch when max_slots
  // allows): the histogram and all keys of the head this workgroup's index
  // maps to are loaded before the ticket returns, and kept when the ticket
  // names the same head (the usual case), else loaded again.
  constexpr bool spec = SPEC;
  uint32_t kr[kRes][4];
  uint32_t hv[kSelectBins / kFT];
  auto load_head = [&](int uh) {
    // the histogram first: the first rank step needs only it, and loads
    // complete in order, so the keys stream in behind that step
    const uint32_t *hgh = P.hist + (size_t)uh * kSelectBins;
#pragma unroll
    for (int q = 0; q < kSelectBins / kFT; ++q) hv[q] = hgh[tid + q * kFT];
    // the raw score bits (turned into keys by keys_from_raw before their
    // first use, so that all the loads go out at once)
    const float *sch = P.sc + (size_t)uh * P.max_slots;
#pragma unroll
    for (int q = 0; q < kRes; ++q) {
      const int s = min(q * kGrp + 4 * tid, P.max_slots - 4);
      const uint4 v = *reinterpret_cast<const uint4 *>(sch + s);
      kr[q][0] = v.x;
      kr[q][1] = v.y;
      kr[q][2] = v.z;
      kr[q][3] = v.w;
    }
  };
  auto keys_from_raw = [&]() {
#pragma unroll
    for (int q = 0; q < kRes; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) kr[q][e] = score_key(__uint_as_float(kr[q][e]));
  };
  // Heads of at most kRes groups (every head, when max_slots allows) are
  // selected locally with no wait before the compaction: a workgroup's head
  // and part come from its index (so its loads go out at once, and with
  // round-robin dispatch a head's workgroups share an XCD), and the
  // compaction's batches are handed out by a per-head ticket.  Otherwise a
  // launch-wide ticket, taken in dispatch order, names the head and part:
  // the shared selection waits for every workgroup of the head.
  int u, k, ticket;
  if (spec) {
    ticket = (int)blockIdx.x;
    ticket_head(ticket, P.units, P.kh, u, k);
  } else {
    if (tid == 0) L.ticket = atomicAdd(&P.ctr[0], 1u);
    __syncthreads();
    ticket = (int)L.ticket;
    ticket_head(ticket, P.units, P.kh, u, k);
  }
  // the small loads first (loads complete in order: waiting for the length
  // must not wait for the keys), then the head's histogram and keys
  const size_t urow = (size_t)u * P.max_slots;
  const int n = P.seq_len[u];
  const int herr = P.head_err[u];
  // every head's length and error flag, for the free-list prefix at the end
  // (one head a thread when there are at most kFT; used only then)
  const int pi = min(tid, P.units - 1);
  const int pn = P.seq_len[pi];
  const int pe = P.head_err[pi];
  // the free count (only the launch's last workgroup writes it, at the end)
  const int fc0 = *P.free_count;
  if (spec) load_head(u);
  // the compaction's first batch: a per-head ticket, taken now so that its
  // round trip overlaps the selection (batches go out in ticket order, each
  // to a running workgroup, so a wait for a lower batch always ends)
  uint32_t ticket0 = 0;
  if (spec && tid == 0) ticket0 = atomicAdd(&P.bctr[u], 1u);
  // nothing that waits for a load moves above the last of them
  __builtin_amdgcn_sched_barrier(0);
  const bool consistent = n >= 0 && n <= P.max_slots;
  const int m = consistent ? max(0, n - P.budget) : 0;
  const int nc = consistent ? max(0, n - P.recent) : 0;
  const int n2 = n - m;
  const bool bad = consistent && herr != 0;
  const float *sc = P.sc + urow;
  float *so = P.score_out + urow;
  unsigned long long *acc = P.acc;

  if (!consistent) {
    if (k == 0 && tid == 0) {
      P.n_victims[u] = -1;
      atomicOr(&acc[3], 2ull);
    }
  } else if (m == 0) {
    // nothing to evict: the scores of [0, n) go to the output row as they are
    if (k == 0 && tid == 0) P.n_victims[u] = 0;
    const int share = ((n + P.kh - 1) / P.kh + 3) & ~3;
    const int s0 = k * share, s1 = min(n, s0 + share);
    for (int s = s0 + tid; s < s1; s += kFT) so[s] = sc[s];
  } else {
    // ------------------------------------------------------------ threshold
    const int ngrp = (nc + kGrp - 1) / kGrp;      // groups with candidates
    const int ngrp_all = (n + kGrp - 1) / kGrp;   // groups with live slots
    const int nch = (nc + kChunk - 1) / kChunk;   // chunks with candidates
    const int nch_all = (n + kChunk - 1) / kChunk;
    const int gpp = (ngrp + P.kh - 1) / P.kh;     // groups per share
    const int g_lo = min(k * gpp, ngrp), g_hi = min(g_lo + gpp, ngrp);
    // A head of at most kRes groups is selected locally: every workgroup of
    // the head holds all its keys in registers and finds the threshold
    // itself, with no exchange; longer heads share the work (each its share,
    // published and read back in two rounds).  Keys held in registers: the whole head, or
    // the share (not beside the widest rows' pieces).
    const bool local = PR <= 16 && ngrp_all <= kRes;
    const int r_lo = local ? 0 : g_lo, r_hi = local ? ngrp_all : g_hi;
    const bool res = PR <= 16 && r_hi - r_lo <= kRes;
    // this thread's 4 keys of group g (slots g*4096 + 4*tid + e)
    auto load4 = [&](int g, uint32_t (&o)[4]) {
      const int s = min(g * kGrp + 4 * tid, P.max_slots - 4);
      const float4 v = *reinterpret_cast<const float4 *>(sc + s);
      o[0] = score_key(v.x);
      o[1] = score_key(v.y);
      o[2] = score_key(v.z);
      o[3] = score_key(v.w);
    };
    auto keys_of = [&](int g, uint32_t (&o)[4]) {
      if (res && g >= r_lo && g < r_hi) {
#pragma unroll
        for (int q = 0; q < kRes; ++q)
          if (q == g - r_lo) {
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = kr[q][e];
          }
      } else {
        load4(g, o);
      }
    };
    if (!spec) {
      const uint32_t *hg = P.hist + (size_t)u * kSelectBins;
#pragma unroll
      for (int q = 0; q < kSelectBins / kFT; ++q) hv[q] = hg[tid + q * kFT];
    }
    // block ids of the share's first groups, where a batch's sources mostly
    // lie (batch k of a head usually draws on group k)
    const int32_t *btu = P.block_table + (size_t)u * P.max_blocks;
    const int pb0 = spec ? 0 : g_lo * (kGrp / kBlock);
    int pbid[kPreBlk / kFT];
#pragma unroll
    for (int q = 0; q < kPreBlk / kFT; ++q)
      pbid[q] = !bad && pb0 + tid + q * kFT < blocks_of(n) ? btu[pb0 + tid + q * kFT] : 0;
    // and the destination block ids of this workgroup's first batch
    const int pdid = !bad && tid < kBatchRanks / kBlock &&
                             k * (kBatchRanks / kBlock) + tid < blocks_of(n - m)
                         ? btu[k * (kBatchRanks / kBlock) + tid] : 0;
    if (res && !spec) {
#pragma unroll
      for (int q = 0; q < kRes; ++q)
        if (q < r_hi - r_lo) load4(r_lo + q, kr[q]);
    }
#pragma unroll
    for (int q = 0; q < kSelectBins / kFT; ++q) {
      L.h[tid + q * kFT] = hv[q];
      L.h2[tid + q * kFT] = 0;
    }
    for (int i = tid; i <= kMaxChunks; i += kFT) L.cv[i] = 0;
    if (tid == 0) {
      L.nsub = 0;
      L.moved = 0;
      L.at_risk = 0;
    }
    __syncthreads();
    rank_bin_all<kSelectBins>(L.h, (uint32_t)m, &L.r, L.rtot);
    const uint32_t bkt = L.r.bin;
    const uint32_t need = (uint32_t)m - L.r.below;  // rank inside the bucket
    uint32_t pre, need2;
    int nmem = 0;
    uint2 *gmem = P.mem + urow;
    if (spec) keys_from_raw();  // the loads went out before the first rank step
    if (local) {
      // ---- the whole head: keys below the bucket per chunk (a wave covers
      // 256 slots of a group: chunk = 4 g + wave / 4) and the histogram of
      // the bucket members' key bits 20..10
      // (groups in compile-time order: the keys stay in named registers)
#pragma unroll
      for (int g = 0; g < kRes; ++g) {
        if (g >= ngrp) break;
        const uint32_t(&kk)[4] = kr[g];
        uint32_t below = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = g * kGrp + 4 * tid + e;
          const bool in = s < nc;
          const uint32_t top = kk[e] >> 21;
          below += (uint32_t)__popcll(__ballot(in && top < bkt));
          if (in && top == bkt) atomicAdd(&L.h2[(kk[e] >> 10) & 2047u], 1u);
        }
        if (lane == 0 && below) atomicAdd(&L.cv[4 * g + wv / 4], below);
      }
      for (int i = tid; i < 1024; i += kFT) L.h[i] = 0;
      __syncthreads();
      rank_bin_all<kSelectBins>(L.h2, need, &L.r, L.rtot);
      pre = (bkt << 11) | L.r.bin;  // key >> 10 of T
      need2 = need - L.r.below;
      // the bucket's members below the sub-bucket are victims (per chunk);
      // the sub-bucket's keys get the histogram of their last 10 bits and go
      // to LDS (the first kMem of them)
#pragma unroll
      for (int g = 0; g < kRes; ++g) {
        if (g >= ngrp) break;
        const uint32_t(&kk)[4] = kr[g];
        uint32_t below = 0;  // the wave's 256 slots lie in one chunk
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = g * kGrp + 4 * tid + e;
          const bool mb = s < nc && (kk[e] >> 21) == bkt;
          const uint32_t p = kk[e] >> 10;
          below += (uint32_t)__popcll(__ballot(mb && p < pre));
          const bool sb = mb && p == pre;
          if (sb) atomicAdd(&L.h[kk[e] & 1023u], 1u);
          const uint64_t sm = __ballot(sb);
          if (sm) {
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&L.nsub, (uint32_t)__popcll(sm));
            base = __shfl(base, 0);
            const uint32_t j = base + (uint32_t)ballot_prefix(sm);
            if (sb && j < (uint32_t)kMem) L.sub[j] = make_uint2(kk[e], (uint32_t)s);
          }
        }
        if (lane == 0 && below) atomicAdd(&L.cv[4 * g + wv / 4], below);
      }
    } else {
      // ---- own share, first pass: keys below the bucket per chunk (a wave
      // covers 256 slots of a group: chunk = 4 g + wave / 4), and the
      // histogram of the bucket members' key bits 20..10, added to the head's
      uint32_t *gbel = P.gbelow + (size_t)u * P.chunks;
      for (int g = g_lo; g < g_hi; ++g) {
        uint32_t kk[4];
        keys_of(g, kk);
        uint32_t below = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = g * kGrp + 4 * tid + e;
          const bool in = s < nc;
          const uint32_t top = kk[e] >> 21;
          below += (uint32_t)__popcll(__ballot(in && top < bkt));
          if (in && top == bkt) atomicAdd(&L.h2[(kk[e] >> 10) & 2047u], 1u);
        }
        if (lane == 0 && below) atomicAdd(&L.cv[4 * g + wv / 4], below);
      }
      __syncthreads();
      uint32_t *h2g = P.hist2 + (size_t)u * kSelectBins;
#pragma unroll
      for (int q = 0; q < kSelectBins / kFT; ++q)
        if (L.h2[tid + q * kFT]) atomicAdd(&h2g[tid + q * kFT], L.h2[tid + q * kFT]);
      // ---- arrive, then wait for every workgroup of the head
      wait_mem();
      __syncthreads();
      if (tid == 0) atomicAdd(&P.arrive[u], 1u);
      wait_count(&P.arrive[u], (uint32_t)P.kh, acc);
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kSelectBins / kFT; ++q) hv[q] = ld_agent(&h2g[tid + q * kFT]);
#pragma unroll
      for (int q = 0; q < kSelectBins / kFT; ++q) L.h2[tid + q * kFT] = hv[q];
      for (int i = tid; i < 1024; i += kFT) L.h[i] = 0;
      __syncthreads();
      rank_bin_all<kSelectBins>(L.h2, need, &L.r, L.rtot);
      pre = (bkt << 11) | L.r.bin;  // key >> 10 of T
      need2 = need - L.r.below;
      // ---- own share, second pass: the bucket's members below the sub-bucket
      // join their chunk's victims, and the sub-bucket's keys are published
      // (each wave reserves its place with one atomic)
      for (int g = g_lo; g < g_hi; ++g) {
        uint32_t kk[4];
        keys_of(g, kk);
        uint32_t below = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = g * kGrp + 4 * tid + e;
          const bool mb = s < nc && (kk[e] >> 21) == bkt;
          const uint32_t p = kk[e] >> 10;
          below += (uint32_t)__popcll(__ballot(mb && p < pre));
          const bool sb = mb && p == pre;
          const uint64_t sm = __ballot(sb);
          if (sm) {
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&P.nmem[u], (uint32_t)__popcll(sm));
            base = __shfl(base, 0);
            if (sb) st_agent2(gmem + base + (uint32_t)ballot_prefix(sm), make_uint2(kk[e], (uint32_t)s));
          }
        }
        if (lane == 0 && below) atomicAdd(&L.cv[4 * g + wv / 4], below);
      }
      __syncthreads();
      for (int c = 4 * g_lo + tid; c < min(4 * g_hi, nch); c += kFT) st_agent(gbel + c, L.cv[c]);
      // ---- arrive again, then read every chunk's count and the sub-bucket
      wait_mem();
      __syncthreads();
      if (tid == 0) atomicAdd(&P.arrive[u], 1u);
      wait_count(&P.arrive[u], 2u * (uint32_t)P.kh, acc);
      __syncthreads();
      nmem = (int)ld_agent(&P.nmem[u]);  // the sub-bucket's keys, all workgroups
      for (int c = tid; c < nch; c += kFT) L.cv[c] = ld_agent(gbel + c);
      if (tid == 0) L.nsub = (uint32_t)nmem;
      // their last 10 bits' histogram, and the first kMem of them in LDS
      for (int i = tid; i < nmem; i += kFT) {
        const uint2 pk = ld_agent2(gmem + i);
        atomicAdd(&L.h[pk.x & 1023u], 1u);
        if (i < kMem) L.sub[i] = pk;
      }
    }
    __syncthreads();
    const int nsub = (int)L.nsub;
    const bool sub_lds = nsub <= kMem;
    // every key of the sub-bucket: from LDS, or (too many) streamed again
    auto for_sub = [&](auto &&f) {
      if (sub_lds) {
        for (int i = tid; i < nsub; i += kFT) f(L.sub[i].x, (int)L.sub[i].y);
      } else if (local) {
#pragma unroll
        for (int g = 0; g < kRes; ++g) {
          if (g >= ngrp) break;
          const uint32_t(&kk)[4] = kr[g];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int s = g * kGrp + 4 * tid + e;
            if (s < nc && (kk[e] >> 10) == pre) f(kk[e], s);
          }
        }
      } else {
        for (int i = tid; i < nmem; i += kFT) {
          const uint2 p = ld_agent2(gmem + i);
          if ((p.x >> 10) == pre) f(p.x, (int)p.y);
        }
      }
    };
    rank_bin_all<1024>(L.h, need2, &L.r, L.rtot);
    const uint32_t T = (pre << 10) | L.r.bin;
    const uint32_t eT = need2 - L.r.below;  // keys equal to T that are victims
    const uint32_t cnt_t = L.h[L.r.bin];
    __syncthreads();
    // the cut: the eT-th smallest slot among the keys equal to T
    int cut = INT_MAX;
    if (eT < cnt_t) {
      if (cnt_t <= (uint32_t)kTie) {
        int *tie = reinterpret_cast<int *>(L.h2);
        if (tid == 0) L.nt = 0;
        __syncthreads();
        for_sub([&](uint32_t key, int s) {
          if (key == T) tie[atomicAdd(&L.nt, 1u)] = s;
        });
        __syncthreads();
        for (int i = tid; i < (int)cnt_t; i += kFT) {
          const int si = tie[i];
          uint32_t r = 0;
          for (int j = 0; j < (int)cnt_t; ++j) r += tie[j] < si ? 1u : 0u;
          if (r == eT - 1) L.cut = (uint32_t)si;
        }
        __syncthreads();
        cut = (int)L.cut;
      } else {
        // many equal keys: radix over the slot bits (4 x 8)
        uint32_t sp = 0, smask = 0, rank = eT;
        for (int pass = 0; pass < 4; ++pass) {
          const int shift = 24 - 8 * pass;
          for (int i = tid; i < 256; i += kFT) L.h[i] = 0;
          __syncthreads();
          for_sub([&](uint32_t key, int s) {
            if (key == T && ((uint32_t)s & smask) == sp)
              atomicAdd(&L.h[((uint32_t)s >> shift) & 255u], 1u);
          });
          __syncthreads();
          wg_rank_bin<256>(L.h, rank, &L.r);
          sp |= L.r.bin << shift;
          smask |= 255u << shift;
          rank -= L.r.below;
          __syncthreads();
        }
        cut = (int)sp;
      }
    }
    // the sub-bucket's victims per chunk, then the chunks' offsets
    if (sub_lds) {
      for (int i = tid; i < nsub; i += kFT) {
        const uint2 p = L.sub[i];
        if (p.x < T || (p.x == T && (int)p.y <= cut)) atomicAdd(&L.cv[p.y / kChunk], 1u);
      }
    } else {
      for_sub([&](uint32_t key, int s) {
        if (key < T || (key == T && s <= cut)) atomicAdd(&L.cv[s / kChunk], 1u);
      });
    }
    __syncthreads();
    if (wv == 0) {  // exclusive scan of the chunk counts (at most 1024: 16 per lane)
      const int per = (nch_all + kWave - 1) / kWave;
      const int c0 = min(lane * per, nch_all), c1 = min(c0 + per, nch_all);
      uint32_t mine = 0;
      for (int c = c0; c < c1; ++c) mine += L.cv[c];
      uint32_t e = wave_incl_scan(mine) - mine;
      for (int c = c0; c < c1; ++c) {
        const uint32_t x = L.cv[c];
        L.cv[c] = e;
        e += x;
      }
      if (lane == kWave - 1) L.cv[nch_all] = e;  // == m
    }
    __syncthreads();

    // victim flags of a group's slots for this thread
    auto vic4 = [&](int g, const uint32_t (&kk)[4], bool (&v)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = g * kGrp + 4 * tid + e;
        v[e] = s < nc && (kk[e] < T || (kk[e] == T && s <= cut));
      }
    };

    // ------------------------------------------------------------ victim list
    int scan_parity = 0;  // chunk_scan's row
    if (k == 0 && tid == 0) P.n_victims[u] = m;
    int32_t *vout = P.victims + urow;
    for (int g = g_lo; g < g_hi; ++g) {
      uint32_t kk[4];
      keys_of(g, kk);
      bool v[4];
      vic4(g, kk, v);
      const int cnt = (int)v[0] + (int)v[1] + (int)v[2] + (int)v[3];
      // victims before the chunk, then before this thread within it
      int o = (int)L.cv[4 * g + wv / 4] + chunk_scan(cnt, L.wsum, &scan_parity);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (v[e]) {
          if (o < m) vout[o] = g * kGrp + 4 * tid + e;
          ++o;
        }
    }

    // ------------------------------------------------------------ compaction
    if (bad) {
      // no compaction: the scores of [0, n) go to the output row as they are
      const int share = ((n + P.kh - 1) / P.kh + 3) & ~3;
      const int s0 = k * share, s1 = min(n, s0 + share);
      for (int s = s0 + tid; s < s1; s += kFT) so[s] = sc[s];
    } else {
      const int nbatch = (n2 + kBatchRanks - 1) / kBatchRanks;
      const int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
      const int32_t *pos = P.pos + urow;
      uint32_t *marks = P.marks + (size_t)u * P.marks_per_head;
      constexpr int kRowPieces = kBatchRanks * PR;   // 16-byte pieces of K (or V) per batch
      constexpr int kPer = kRowPieces / kFT;         // per thread, per tensor
      const int row_bytes = PR * 16;
      // kept slots before chunk c: the chunk's start minus the victims before it
      auto kbc = [&](int c) { return c * kChunk - (int)L.cv[min(c, nch_all)]; };
      // the last chunk c with kbc(c) <= r (kbc does not decrease)
      auto chunk_of_rank = [&](int r) {
        int lo = 0, hi = nch_all - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (kbc(mid) <= r) lo = mid; else hi = mid - 1;
        }
        return lo;
      };
      int b0 = pb0;  // first block whose id L.blk holds
#pragma unroll
      for (int q = 0; q < kPreBlk / kFT; ++q) L.blk[tid + q * kFT] = pbid[q];
      // the first batch: the per-head ticket (local selection), else the part
      if (spec && tid == 0) L.ticket = ticket0;
      __syncthreads();
      const int kb = spec ? (int)L.ticket : k;
      for (int rho = kb; rho < nbatch; rho += P.kh) {
        const int R0 = rho * kBatchRanks, R1 = min(R0 + kBatchRanks, n2);
        const int gs = chunk_of_rank(R0) / 4;  // group of the first source
        // block ids: the destinations', and the first source groups' unless
        // the prefetched ones cover them (loads in flight while the groups
        // are ranked)
        const bool fresh = gs * (kGrp / kBlock) < b0 || gs * (kGrp / kBlock) >= b0 + kPreBlk;
        int bid[kPreBlk / kFT];
#pragma unroll
        for (int q = 0; q < kPreBlk / kFT; ++q) {
          const int bi = gs * (kGrp / kBlock) + tid + q * kFT;
          bid[q] = fresh && bi < blocks_of(n) ? bt[bi] : 0;
        }
        // (a head held whole in L.blk: every id from LDS)
        const int did = spec ? (tid < kBatchRanks / kBlock && R0 / kBlock + tid < blocks_of(n2)
                                    ? L.blk[R0 / kBlock + tid] : 0)
                        : rho == k ? pdid  // prefetched for batch k
                        : tid < kBatchRanks / kBlock && R0 / kBlock + tid < blocks_of(n2)
                            ? bt[R0 / kBlock + tid] : 0;
        // rank each kept slot of group g; record the sources of [R0, R1)
        for (int g = gs; g < ngrp_all && kbc(4 * g) < R1; ++g) {
          uint32_t kk[4];
          keys_of(g, kk);
          bool v[4];
          vic4(g, kk, v);
          int kc = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int s = g * kGrp + 4 * tid + e;
            kc += (s < n && !v[e]) ? 1 : 0;
          }
          // kept slots before the chunk, then before this thread within it
          int r = kbc(4 * g + wv / 4) + chunk_scan(kc, L.wsum, &scan_parity);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int s = g * kGrp + 4 * tid + e;
            if (s < n && !v[e]) {
              if (r >= R0 && r < R1) L.src[r - R0] = s;
              ++r;
            }
          }
        }
        if (fresh) {
          __syncthreads();  // the previous batch's readers of blk are done
#pragma unroll
          for (int q = 0; q < kPreBlk / kFT; ++q) L.blk[tid + q * kFT] = bid[q];
          b0 = gs * (kGrp / kBlock);
        }
        if (tid < kBatchRanks / kBlock) L.dblk[tid] = did;
        __syncthreads();
        // ---- loads: source block ids (prefetched, else loaded), K / V
        // pieces, pos and score
        const int nr = R1 - R0;
        if (tid < nr) {
          const int s = L.src[tid];
          const int lb = s / kBlock - b0;
          L.sblk[tid] = s == R0 + tid ? -1 : (lb < kPreBlk ? L.blk[lb] : bt[s / kBlock]);
        }
        __syncthreads();
        uint4 kv[kPer], vv[kPer];
        bool mv[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int idx = tid + j * kFT;
          const int r = idx / PR, part = idx % PR;
          const int blk = r < nr ? L.sblk[r] : -1;
          mv[j] = blk >= 0;
          const int s = mv[j] ? L.src[r] : 0;
          const size_t off =
              ((size_t)max(blk, 0) * kBlock + s % kBlock) * row_bytes + (size_t)part * 16;
          kv[j] = mv[j] ? ld16(P.k_pool + off) : make_uint4(0, 0, 0, 0);
          vv[j] = mv[j] ? ld16(P.v_pool + off) : make_uint4(0, 0, 0, 0);
        }
        int my_pos = 0;
        float my_sc = 0.f;
        if (tid < nr) {
          const int s = L.src[tid];
          my_pos = pos[s];
          my_sc = sc[s];
        }
        // every load of the batch has returned its data before the mark
        wait_mem();
        __syncthreads();
        if (tid == 0) st_agent(&marks[rho], 1u);
        // ---- wait for the batches that read this batch's destination
        // slots: they lie in chunk R0 / 1024, whose kept slots have the ranks
        // [kbc(c), kbc(c + 1)); only batches below this one need waiting for
        const int cd = R0 / kChunk;
        const int klo = kbc(cd), khi = kbc(cd + 1);
        const int lo = klo / kBatchRanks, hi = min((khi - 1) / kBatchRanks, rho - 1);
        if (wv == 0 && khi > klo && lo <= hi) {
          unsigned spins = 0;
          for (int c0 = lo; c0 <= hi; c0 += kWave) {
            const int bi = c0 + lane;
            bool done = bi > hi;
            for (;;) {
              if (!done) done = ld_agent(&marks[bi]) != 0;
              if (__all(done)) break;
              if (++spins > kSpinLimit) {
                if (lane == 0) atomicOr(&acc[3], 8ull);
                break;
              }
              __builtin_amdgcn_s_sleep(1);
            }
          }
        }
        __syncthreads();
        // ---- stores: K / V rows (nontemporal), pos, score
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int idx = tid + j * kFT;
          const int r = idx / PR, part = idx % PR;
          if (mv[j]) {
            const int d = R0 + r;
            const size_t off = ((size_t)L.dblk[r / kBlock] * kBlock + d % kBlock) * row_bytes +
                               (size_t)part * 16;
            st16_nt(P.k_pool + off, kv[j]);
            st16_nt(P.v_pool + off, vv[j]);
          }
        }
        if (tid < nr) {
          const int d = R0 + tid, s = L.src[tid];
          if (s != d) P.pos[urow + d] = my_pos;
          so[d] = my_sc;
          const bool moves = s != d;
          const uint64_t mb = __ballot(moves), rb = __ballot(moves && s < n2);
          if (lane == 0) {
            atomicAdd(&L.moved, __popcll(mb));
            atomicAdd(&L.at_risk, __popcll(rb));
          }
        }
        __syncthreads();
      }
      if (tid == 0 && L.moved) {
        atomicAdd(&acc[1], (unsigned long long)L.moved);
        atomicAdd(&acc[2], (unsigned long long)L.at_risk);
      }
    }
  }

  // ------------------------------------------------------------ arrivals
  __syncthreads();
  if (tid == 0) L.last = atomicAdd(&P.head_done[u], 1u) == (uint32_t)(P.kh - 1) ? 1 : 0;
  __syncthreads();
  long long before, total;
  // the head's free-list offset and the total, for the head's last workgroup
  freed_prefix(P, freed_prefix_load(P, u, pn, pe), L, before, total);
  const bool room = fc0 >= 0 && (long long)fc0 + total <= (long long)P.free_capacity;
  if (L.last) {
    if (consistent && m > 0) {
      if (bad) {
        if (tid == 0) atomicOr(&acc[3], 1ull);
      } else {
        const int lb0 = blocks_of(n2), lb1 = blocks_of(n);
        int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
        if (room) {
          int32_t *fl = P.free_list + fc0 + before;
          for (int i = tid; i < lb1 - lb0; i += kFT) {
            fl[i] = bt[lb0 + i];
            bt[lb0 + i] = -1;
          }
          if (tid == 0) atomicAdd(&acc[0], (unsigned long long)(lb1 - lb0));
        }
        const int nbatch = (n2 + kBatchRanks - 1) / kBatchRanks;
        uint32_t *marks = P.marks + (size_t)u * P.marks_per_head;
        for (int i = tid; i < nbatch; i += kFT) st_agent(&marks[i], 0u);
      }
      // the head's selection state for the next call
      for (int i = tid; i < kSelectBins; i += kFT) {
        st_agent(&P.hist[(size_t)u * kSelectBins + i], 0u);
        st_agent(&P.hist2[(size_t)u * kSelectBins + i], 0u);
      }
      if (tid == 0) {
        st_agent(&P.nmem[u], 0u);
        st_agent(&P.arrive[u], 0u);
      }
    }
    if (tid == 0) {
      st_agent(&P.head_done[u], 0u);
      st_agent(&P.bctr[u], 0u);
    }
  }
  __syncthreads();
  if (tid == 0)
    L.last = atomicAdd(&P.ctr[1], 1u) == (uint32_t)(P.units * P.kh - 1) ? 1 : 0;
  __syncthreads();
  if (!L.last) return;
  // ---- the last workgroup of the launch: lengths, free count, stats, state
  for (int i = tid; i < P.units; i += kFT) {
    // (at most kFT heads: this thread's length and flag were loaded at entry)
    const int ni = P.units <= kFT ? pn : P.seq_len[i];
    const int ei = P.units <= kFT ? pe : (int)P.head_err[i];
    if (ni >= 0 && ni <= P.max_slots && ei == 0) P.seq_len[i] = min(ni, P.budget);
    st_agent(&P.head_err[i], 0u);
  }
  if (tid == 0) {
    const unsigned long long freed = atomicExch(&acc[0], 0ull);
    const unsigned long long moved = atomicExch(&acc[1], 0ull);
    const unsigned long long risk = atomicExch(&acc[2], 0ull);
    unsigned long long status = atomicExch(&acc[3], 0ull);
    if (room) *P.free_count = (int)(fc0 + total);
    else status |= 4ull;
    P.stats[0] = (int64_t)freed;
    P.stats[1] = (int64_t)moved;
    P.stats[2] = (int64_t)(moved * 4ull * (unsigned long long)P.row_bytes);
    P.stats[3] = (int64_t)risk;
    P.stats[4] = (int64_t)status;
    st_agent(&P.ctr[0], 0u);
    st_agent(&P.ctr[1], 0u);
  }
}

}  // namespace

size_t finish_lds_bytes() { return sizeof(FinLds); }

int finish_parts(int units, int rows_cap) {
  // enough workgroups to cover the CUs twice, at most one per batch of ranks,
  // and at most kMaxHeadParts: a head that shares its selection waits until
  // all its workgroups have arrived, so they must fit on the chip at once.
  // The kernel runs one 1024-thread workgroup per CU (its registers), and
  // half of gfx950's 256 CUs keeps a head's workgroups resident even beside
  // a second launch of this kernel on another stream.
  const int batches = std::max(1, (rows_cap + kBatchRanks - 1) / kBatchRanks);
  const int want = std::max(1, (512 + units - 1) / units);
  return std::min({batches, want, kMaxHeadParts});
}

hipError_t launch_finish(const FinishArgs &a, hipStream_t s) {
  const size_t lds = sizeof(FinLds);
  const dim3 grid((unsigned)(a.units * a.kh));
  const bool spec = a.max_slots <= kRes * kGrp;  // with PR <= 16
  switch (a.row_bytes / 16) {
    case 8:
      if (spec) hipLaunchKernelGGL((evict_finish_kernel<8, true>), grid, dim3(kFT), lds, s, a);
      else hipLaunchKernelGGL((evict_finish_kernel<8, false>), grid, dim3(kFT), lds, s, a);
      break;
    case 16:
      if (spec) hipLaunchKernelGGL((evict_finish_kernel<16, true>), grid, dim3(kFT), lds, s, a);
      else hipLaunchKernelGGL((evict_finish_kernel<16, false>), grid, dim3(kFT), lds, s, a);
      break;
    case 32: hipLaunchKernelGGL((evict_finish_kernel<32, false>), grid, dim3(kFT), lds, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvev
