// compact.hip -- in-place, order-preserving compaction of each KV head (gfx950).
//
// Kept slot s of rank r moves to slot r (r <= s).  Done in parallel this has
// one hazard: a destination row r < n' may still be the source of another
// kept token.  Those sources are exactly the kept slots in [first victim, n')
// ("at risk"); they are copied to the workspace first, up to stage_rows of a
// head.  A head with more at-risk rows is moved by one workgroup in rank
// order instead, staging nothing: rounds of destination ranks in ascending
// order, every load of a round returned before any store (a source never
// lies below its destination, so no later round reads a slot an earlier one
// wrote, and within a round the loads precede the stores).  Three launches:
//   prep    (1024-slot chunk of one head per workgroup): finds the chunk's
//           victims, ranks the kept slots, records for each destination rank
//           its source (physical row, staged copy, or "stays") and the kept
//           pos / score values, and copies the at-risk rows to the workspace.
//           Reads the cache only.  Each chunk adds its counts into one 64-bit
//           word of the head (arrivals, chunks with errors, rows moved, rows
//           staged) with a single atomic, whose previous value also gives
//           the chunk's first staging row; the chunk that arrives last
//           records the head's totals, so no chunk reads another's memory.
//           The chunk's victims come from the caller's ascending victim list
//           (256 evenly spaced samples bracket them, one range load fetches
//           them).
//   gather  (persistent grid over (head, rank range) items): each thread
//           issues all of its 16-byte K and V loads before any store; the
//           moved rows are stored with the nontemporal hint, so they reach
//           HBM during this latency-bound step rather than being written
//           back from the Infinity Cache while a later pass streams.  The
//           first item of a head also appends the emptied tail blocks
//           [ceil(n'/16), ceil(n/16)) to the free list in (b, h, block)
//           order, clears their table entries, sets seq_len = n' and adds the
//           head's stats.
//   inorder (one 1024-thread workgroup per head): moves the rows of the
//           heads whose at-risk rows did not fit, in ascending rounds of
//           destination ranks; the other heads return at once.
// ([H2O] "PagedAttention Memory Integration"; [VTOK] section 3.3, stage 3
// and section 3.5, invariants I1, I2 and I4.)
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {
constexpr int kThreads = 256;
constexpr int kChunk = kCompactChunk;   // slots per prep workgroup
constexpr int kPerThread = kChunk / kThreads;
constexpr int kMaxUnits = kCompactMaxUnits;
constexpr int kRange = 4096;            // victims a prep workgroup stages in LDS
constexpr int kSeqThreads = 1024;       // in-order kernel: threads per head
constexpr int kSeqRows = 8;             // in-order kernel: rows per thread and round

struct PrepLds {
  int stage_s[kChunk];                   // at-risk slots, in staging order
  int blk_l[kChunk / kBlock];            // block ids of the chunk's logical blocks
  int wave_tot[kThreads / kWave];
  int r0s[kThreads / kWave], r1s[kThreads / kWave];
  int s_err, s_nstage, s_base;
};

// Exclusive prefix sum over a 256-thread workgroup.
__device__ int block_exclusive_scan(int v, int *wave_tot) {
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  const int incl = (int)wave_incl_scan((uint32_t)v);
  if (lane == kWave - 1) wave_tot[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wv; ++w) before += wave_tot[w];
  __syncthreads();
  return before + incl - v;
}

// Sums of a and b over a 256-thread workgroup (every thread gets them).
__device__ void block_sum2(int &a, int &b, PrepLds &S) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    a += __shfl_xor(a, o);
    b += __shfl_xor(b, o);
  }
  __syncthreads();
  if (lane_id() == 0) {
    S.r0s[threadIdx.x / kWave] = a;
    S.r1s[threadIdx.x / kWave] = b;
  }
  __syncthreads();
  a = 0;
  b = 0;
  for (int w = 0; w < kThreads / kWave; ++w) {
    a += S.r0s[w];
    b += S.r1s[w];
  }
}

// Lower bound of key in the ascending a[0, m): counts the bracket [base,
// base + len) after the samples placed it there (one more round of loads).
__device__ int bracket_count(const int32_t *a, int base, int len, int key) {
  int cnt = 0;
  for (int off = 0; off < len; off += kThreads)
    cnt += __syncthreads_count(off + threadIdx.x < len && a[base + off + threadIdx.x] < key);
  return base + cnt;
}

__device__ __forceinline__ int blocks_of(int n) { return (n + kBlock - 1) / kBlock; }

// Blocks a head frees: 0 unless it is consistent, error free and loses tokens.
__device__ __forceinline__ int head_freed(const CompactArgs &P, int n, int m, int err) {
  if (err || n < 0 || n > P.max_slots || m <= 0 || m > n) return 0;
  return blocks_of(n) - blocks_of(n - m);
}

// Heads that are inconsistent, or lose nothing, are settled by chunk 0 alone.
__device__ bool settle_trivial(const CompactArgs &P, int u, int c, int n, int m) {
  int err = 0;
  if (n < 0 || n > P.max_slots) err = 2;
  else if (m < 0 || m > n) err = 1;
  if (!err && m > 0) return false;
  if (c == 0 && threadIdx.x == 0) {
    int32_t *hi = P.head_info + (size_t)u * 8;
    hi[0] = n;
    hi[1] = m;
    hi[2] = err;
    hi[3] = 0;
    hi[4] = 0;
    hi[5] = 0;
    hi[6] = 0;
  }
  return true;
}

// A chunk's arrival (thread 0): its counts go into the head's 64-bit word
// (bits 0-10 chunks, 11-21 chunks with errors, 22-42 rows moved, 43-63 rows
// staged; each at most 2^20 per head).  The staged count before it is the
// chunk's first staging row.  The chunk that arrives last has the totals: it
// records the head's error state, freed blocks, counts and whether the head
// moves in rank order (more at-risk rows than stage_rows), and clears the
// word for the next call.  s_err must be final (its writes precede a
// barrier).
__device__ void arrive(const CompactArgs &P, int u, int n, int m, int moved, int staged,
                       PrepLds &S) {
  const unsigned long long mine = 1ull | ((unsigned long long)(S.s_err ? 1 : 0) << 11) |
                                  ((unsigned long long)moved << 22) |
                                  ((unsigned long long)staged << 43);
  const unsigned long long old = atomicAdd(&P.head_acc[u], mine);
  S.s_base = (int)(old >> 43);
  if ((old & 2047ull) != (unsigned long long)(P.chunks - 1)) return;
  const unsigned long long tot = old + mine;
  const int err = ((tot >> 11) & 2047ull) ? 1 : 0;
  int32_t *hi = P.head_info + (size_t)u * 8;
  hi[2] = err;
  hi[3] = err ? 0 : blocks_of(n) - blocks_of(n - m);
  hi[4] = (int)((tot >> 22) & 0x1fffffull);
  hi[5] = (int)(tot >> 43);
  hi[6] = (int)(tot >> 43) > P.stage_rows ? 1 : 0;
  atomicExch(&P.head_acc[u], 0ull);  // state for the next call
}

// Ranks the kept slots of the chunk [s0, s1) (thread t owns the slots
// s0 + 4t .. s0 + 4t + 3), records their sources and new pos / score, makes
// the chunk's arrival and copies the at-risk rows to the workspace when they
// fit.  j0: victims of the head before s0.  With victims_out, also writes
// the chunk's victims at their list positions.  The at-risk list is built
// first, so the staging loads are in flight while the rank records are
// stored.
__device__ void rank_and_stage(const CompactArgs &P, int u, int s0, int s1, int n, int m, int j0,
                               const bool (&vic)[kPerThread], const int (&posv)[kPerThread],
                               const float (&scv)[kPerThread], int32_t *victims_out, PrepLds &S) {
  const int n2 = n - m;
  const int tid = threadIdx.x;
  const size_t urow = (size_t)u * P.max_slots;
  int kept = 0;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int s = s0 + tid * kPerThread + q;
    kept += (s < s1 && !vic[q]) ? 1 : 0;
  }
  const int excl = block_exclusive_scan(kept, S.wave_tot);
  // classify: destination rank and source of each kept slot, list position
  // of each victim; at-risk slots to the staging list
  int r = (s0 - j0) + excl;  // kept slots before s0, plus those before mine in the chunk
  int jv = j0 + (min(tid * kPerThread, max(0, s1 - s0)) - excl);  // victims before mine
  int rq[kPerThread], srcq[kPerThread], rowq[kPerThread], jq[kPerThread];
  int my_err = 0, my_moved = 0, my_staged = 0;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int s = s0 + tid * kPerThread + q;
    rq[q] = -1;
    jq[q] = -1;
    srcq[q] = -1;
    rowq[q] = -1;
    if (s >= s1) continue;
    if (vic[q]) {
      if (jv >= 0 && jv < m) jq[q] = jv;
      else my_err = 1;
      ++jv;
      continue;
    }
    if (r < 0 || r >= n2) { my_err = 1; ++r; continue; }
    const int blk = S.blk_l[(s - s0) / kBlock];
    const int row = (blk >= 0 && blk < P.num_blocks) ? blk * kBlock + s % kBlock : 0;
    int src;
    if (r == s) {
      src = -1;                       // stays in place
    } else if (s < n2) {              // at risk: staged before the gather (local index)
      const int k = atomicAdd(&S.s_nstage, 1);
      src = -2 - k;
      ++my_staged;
      S.stage_s[k] = s;
    } else {                          // slots >= n' are never written: read in place
      src = row;
    }
    my_moved += src != -1 ? 1 : 0;
    rq[q] = r;
    srcq[q] = src;
    rowq[q] = src != -1 ? row : -1;
    ++r;
  }
  if (my_err) atomicOr(&S.s_err, 1);
  block_sum2(my_moved, my_staged, S);  // barriers: the list and s_err are complete
  if (tid == 0) arrive(P, u, n, m, my_moved, my_staged, S);
  __syncthreads();
  const int sbase = S.s_base;  // the chunk's first staging row
  const bool fits = sbase + S.s_nstage <= P.stage_rows;

  // staging copy of the at-risk K and V rows in 16-byte pieces, four K and
  // four V pieces per thread and round: indices past the end repeat the last
  // piece (the same bytes again), a block id outside the pool (flagged
  // above) reads block 0, so loads and stores need no branches
  const int pshift = __ffs(P.row_bytes / 16) - 1;  // 16-byte pieces per row: 8, 16 or 32
  const int total = fits ? S.s_nstage << pshift : 0;  // else the head moves in rank order
  uint4 kv[4], vv[4];
  size_t dst[4];
  auto stage_load = [&](int base) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = min(base + q * kThreads + tid, total - 1);
      const int k = idx >> pshift, part = idx & ((1 << pshift) - 1);
      const int s = S.stage_s[k];
      int blk = S.blk_l[(s - s0) / kBlock];
      blk = (blk >= 0 && blk < P.num_blocks) ? blk : 0;
      const size_t src = ((size_t)blk * kBlock + s % kBlock) * P.row_bytes + (size_t)part * 16;
      dst[q] = ((size_t)u * P.stage_rows + sbase + k) * P.row_bytes + (size_t)part * 16;
      kv[q] = ld16(P.k_pool + src);
      vv[q] = ld16(P.v_pool + src);
    }
  };
  auto stage_store = [&]() {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      st16(P.stage_k + dst[q], kv[q]);
      st16(P.stage_v + dst[q], vv[q]);
    }
  };
  if (total > 0) stage_load(0);
  // the rank records while the first staging loads are in flight
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int s = s0 + tid * kPerThread + q;
    if (victims_out && jq[q] >= 0) victims_out[urow + jq[q]] = s;
    if (rq[q] >= 0) {
      P.src_of[urow + rq[q]] = srcq[q] <= -2 ? -2 - (sbase + (-2 - srcq[q])) : srcq[q];
      P.src_row[urow + rq[q]] = rowq[q];
      P.new_pos[urow + rq[q]] = posv[q];
      if (P.score) P.new_score[urow + rq[q]] = scv[q];
    }
  }
  if (total > 0) stage_store();
  for (int base = 4 * kThreads; base < total; base += 4 * kThreads) {
    stage_load(base);
    stage_store();
  }
}

__device__ void prep_common_start(const CompactArgs &P, int u, int c) {
  if (u == 0 && c == 0 && threadIdx.x == 0) {
    *P.fc0 = *P.free_count;
    for (int i = 0; i < 5; ++i) P.stats[i] = 0;
  }
}
}  // namespace

// Prep from a caller's victim list.
__global__ __launch_bounds__(kThreads) void compact_prep_kernel(const CompactArgs P) {
  __shared__ PrepLds S;
  __shared__ uint8_t flag[kChunk];
  __shared__ int vr[kRange];

  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  prep_common_start(P, u, c);
  const int n = P.seq_len[u];
  const int m = P.n_victims[u];
  if (settle_trivial(P, u, c, n, m)) return;
  if (c == 0 && tid == 0) {
    P.head_info[(size_t)u * 8 + 0] = n;
    P.head_info[(size_t)u * 8 + 1] = m;
  }
  const int s0 = c * kChunk;
  const int32_t *vic = P.victims + (size_t)u * P.max_slots;
  const size_t urow = (size_t)u * P.max_slots;
  const int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  if (tid == 0) {
    S.s_err = 0;
    S.s_nstage = 0;
  }
  for (int i = tid; i < kChunk; i += kThreads) flag[i] = 0;

  // ---- one round of independent loads: the victim-list check of this
  // chunk's index share, the samples, the chunk's block ids, pos and score
  int bad = 0;
  {
    // index share of this chunk: at most ceil(m / chunks) <= 1024 entries, so
    // four per thread, all loads issued before any check
    const int i0 = (int)((int64_t)m * c / P.chunks), i1 = (int)((int64_t)m * (c + 1) / P.chunks);
    int va[4], vb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + tid + q * kThreads;
      va[q] = i < i1 ? vic[i] : 0;
      vb[q] = (i < i1 && i + 1 < m) ? vic[i + 1] : INT_MAX;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + tid + q * kThreads;
      if (i < i1 && (va[q] < 0 || va[q] >= n || vb[q] <= va[q])) bad = 1;
    }
    if (i1 - i0 > 4 * kThreads) bad = 1;  // cannot happen: m <= max_slots <= 1024 * chunks
  }
  const bool live_chunk = s0 < n;
  const int s1 = live_chunk ? min(s0 + kChunk, n) : s0;
  int posv[kPerThread];
  float scv[kPerThread];
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int s = s0 + tid * kPerThread + q;
    posv[q] = (s < s1) ? P.pos[urow + s] : 0;
    scv[q] = (s < s1 && P.score) ? P.score[urow + s] : 0.f;
  }
  if (tid < kChunk / kBlock) {
    const int lb = s0 / kBlock + tid;
    const int blk = lb < blocks_of(s1) ? bt[lb] : 0;
    if (blk < 0 || blk >= P.num_blocks) bad = 1;
    S.blk_l[tid] = blk;
  }
  const int SP = (m + kThreads - 1) / kThreads;  // sample spacing
  const int samp = (tid * SP < m) ? vic[tid * SP] : INT_MAX;
  const int c0 = __syncthreads_count(samp < s0);
  if (bad) atomicOr(&S.s_err, 1);  // after a barrier: s_err is initialised
  const int c1 = __syncthreads_count(samp < s1);
  if (live_chunk) {
    // victims before s0 lie in [lo0, hi0], victims before s1 in [lo1, hi1]
    const int lo0 = c0 ? (c0 - 1) * SP + 1 : 0, hi0 = min(c0 * SP, m);
    const int lo1 = c1 ? (c1 - 1) * SP + 1 : 0, hi1 = min(c1 * SP, m);
    int j0, j1;
    if (hi1 - lo0 <= kRange) {
      // ---- one range load covers both brackets and every victim in the
      // chunk (at most kRange entries: 16 per thread, all issued first)
      {
        const int len = hi1 - lo0;
        int t[kRange / kThreads];
#pragma unroll
        for (int q = 0; q < kRange / kThreads; ++q) {
          const int i = tid + q * kThreads;
          t[q] = i < len ? vic[lo0 + i] : 0;
        }
#pragma unroll
        for (int q = 0; q < kRange / kThreads; ++q) {
          const int i = tid + q * kThreads;
          if (i < len) vr[i] = t[q];
        }
      }
      __syncthreads();
      int cnt0 = 0, cnt1 = 0;
      for (int i = tid; i < hi1 - lo0; i += kThreads) {
        cnt0 += vr[i] < s0;
        cnt1 += vr[i] < s1;
      }
      block_sum2(cnt0, cnt1, S);
      j0 = lo0 + cnt0;
      j1 = lo0 + cnt1;
      for (int i = j0 - lo0 + tid; i < j1 - lo0; i += kThreads) {
        const int v = vr[i];
        if (v >= s0 && v < s1) flag[v - s0] = 1;
      }
    } else {
      // long brackets (very sparse victims): count them, then mark
      j0 = bracket_count(vic, lo0, hi0 - lo0, s0);
      j1 = bracket_count(vic, lo1, hi1 - lo1, s1);
      for (int j = j0 + tid; j < j1; j += kThreads) {
        const int v = vic[j];
        if (v >= s0 && v < s1) flag[v - s0] = 1;
      }
    }
    __syncthreads();
    bool vf[kPerThread];
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
      const int s = s0 + tid * kPerThread + q;
      vf[q] = s < s1 && flag[s - s0];
    }
    rank_and_stage(P, u, s0, s1, n, m, j0, vf, posv, scv, nullptr, S);
  } else if (tid == 0) {
    // a chunk past the head's length arrives with nothing (s_err is final:
    // its writes precede the sample counts' barrier)
    arrive(P, u, n, m, 0, 0, S);
  }
}

// Persistent grid over (head, row range) items.  A prefix pass reads each
// head's record once and keeps in LDS the item and free-list offsets of every
// head.  Item 0 of a head records its stats and seq_len; every item appends
// its share of the head's freed blocks and moves up to rows_per_item rows.
// A head that moves in rank order is one item that moves no rows (the
// in-order kernel after this one moves them).
__global__ __launch_bounds__(kThreads) void compact_gather_kernel(const CompactArgs P) {
  extern __shared__ int gsm[];
  const int U = P.units, RC = P.rows_per_item;
  int *item_start = gsm;            // [U + 1]
  int *free_start = gsm + U + 1;    // [U + 1]
  int *n2_l = gsm + 2 * (U + 1);    // [U]: rows kept, -1 = the head does not move
  int *seq_l = gsm + 3 * U + 2;     // [U]: 1 = the head moves in rank order
  __shared__ int wave_tot[kThreads / kWave];
  __shared__ int s_tot[2];
  const int tid = threadIdx.x;
  const int fc0 = *P.fc0;
  int base_items = 0, base_freed = 0;
  for (int b0 = 0; b0 < U; b0 += kThreads) {
    const int u = b0 + tid;
    int cnt = 0, fr = 0;
    if (u < U) {
      const int32_t *hi = P.head_info + (size_t)u * 8;
      const int n = hi[0], m = hi[1], err = hi[2];
      fr = head_freed(P, n, m, err);
      const bool moves = !err && n >= 0 && n <= P.max_slots && m > 0 && m <= n;
      const bool seq = moves && hi[6] != 0;
      cnt = moves && !seq ? max(1, (n - m + RC - 1) / RC) : 1;
      n2_l[u] = moves ? n - m : -1;
      seq_l[u] = seq ? 1 : 0;
    }
    const int ex_i = block_exclusive_scan(cnt, wave_tot);
    const int ex_f = block_exclusive_scan(fr, wave_tot);
    if (u < U) {
      item_start[u] = base_items + ex_i;
      free_start[u] = base_freed + ex_f;
    }
    if (tid == kThreads - 1) {
      s_tot[0] = base_items + ex_i + cnt;
      s_tot[1] = base_freed + ex_f + fr;
    }
    __syncthreads();
    base_items = s_tot[0];
    base_freed = s_tot[1];
    __syncthreads();
  }
  if (tid == 0) {
    item_start[U] = base_items;
    free_start[U] = base_freed;
  }
  __syncthreads();
  const int total_items = base_items, total_freed = base_freed;
  const bool room = fc0 >= 0 && (long long)fc0 + total_freed <= (long long)P.free_capacity;
  const int pshift = __ffs(P.row_bytes / 16) - 1;  // 16-byte pieces per row: 8, 16 or 32
  const int pool_rows = P.num_blocks * kBlock;

  for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
    int lo = 0, hi_u = U - 1;
    while (lo < hi_u) {
      const int mid = (lo + hi_u + 1) >> 1;
      if (item_start[mid] <= item) lo = mid; else hi_u = mid - 1;
    }
    const int u = lo, k = item - item_start[u];
    const int nitems = item_start[u + 1] - item_start[u];
    const int n2 = n2_l[u];
    const bool seq = seq_l[u] != 0;
    const int fr = room ? free_start[u + 1] - free_start[u] : 0;  // > 0 only if the head moves
    const int r0 = k * RC;
    const bool rows = !seq && n2 > 0 && r0 < n2;
    const int r1 = rows ? min(r0 + RC, n2) : 0;
    // this item's share of the head's emptied tail blocks [lb0, lb0 + fr)
    const int f0 = fr > 0 ? (int)((long long)fr * k / nitems) : 0;
    const int f1 = fr > 0 ? (int)((long long)fr * (k + 1) / nitems) : 0;
    const int lb0 = blocks_of(max(n2, 0));
    int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
    const size_t urow = (size_t)u * P.max_slots;
    // lane group of 2^pshift threads per row, one 16-byte piece each, so an
    // instruction covers whole rows; 4 rows per thread
    const int rpr = kThreads >> pshift;  // rows per round
    const int part = tid & ((1 << pshift) - 1);

    // ---- one round of loads: sources, destination blocks, pos and score of
    // the rows (past the item: its last row again), the first freed ids
    int rr[4], srcv[4], dblk[4], npos[4], fid[4];
    float nsc[4];
    if (rows) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rr[i] = min(r0 + i * rpr + (tid >> pshift), r1 - 1);
        srcv[i] = P.src_of[urow + rr[i]];
        dblk[i] = bt[rr[i] / kBlock];
        npos[i] = P.new_pos[urow + rr[i]];
        nsc[i] = P.new_score[urow + rr[i]];
      }
    }
    if (f1 > f0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) fid[q] = bt[lb0 + min(f0 + q * kThreads + tid, f1 - 1)];
    }

    if (k == 0 && tid == 0) {  // the head's record: stats, seq_len, free count
      const int32_t *hi = P.head_info + (size_t)u * 8;
      const int n = hi[0], m = hi[1], ev = hi[2];
      unsigned long long *st = reinterpret_cast<unsigned long long *>(P.stats);
      if (ev) {
        atomicOr(&st[4], (unsigned long long)ev);
      } else if (n2 >= 0) {
        P.seq_len[u] = n - m;
        const long long mv = hi[4], sg = hi[5];
        if (mv) {
          atomicAdd(&st[1], (unsigned long long)mv);
          atomicAdd(&st[2], (unsigned long long)mv * 4ull * (unsigned long long)P.row_bytes);
        }
        if (sg) atomicAdd(&st[3], (unsigned long long)sg);
      }
      if (fr) atomicAdd(&st[0], (unsigned long long)fr);
      if (u == U - 1) {
        if (room) *P.free_count = fc0 + total_freed;
        else atomicOr(&st[4], 4ull);
      }
    }

    if (rows) {
      // No branches between the K/V loads and stores (a branch there makes
      // every store wait for the previous one): a row that stays copies onto
      // itself (same bytes); a wave whose rows all stay skips the copy.
      size_t dsto[4];
      const uint8_t *ksrc[4], *vsrc[4];
      bool moving = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dsto[i] = ((size_t)dblk[i] * kBlock + rr[i] % kBlock) * P.row_bytes + ((size_t)part << 4);
        const int src = srcv[i];
        const int si = -2 - src;
        const bool staged = src <= -2 && si < P.stage_rows;
        const bool pooled = src >= 0 && src < pool_rows;
        moving |= staged || pooled;
        const size_t so = staged ? ((size_t)u * P.stage_rows + si) * P.row_bytes + ((size_t)part << 4)
                                 : pooled ? (size_t)src * P.row_bytes + ((size_t)part << 4) : dsto[i];
        ksrc[i] = (staged ? P.stage_k : P.k_pool) + so;
        vsrc[i] = (staged ? P.stage_v : P.v_pool) + so;
      }
      if (__any(moving)) {  // wave-uniform
        uint4 kv[4], vv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kv[i] = ld16(ksrc[i]);
          vv[i] = ld16(vsrc[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          st16_nt(P.k_pool + dsto[i], kv[i]);
          st16_nt(P.v_pool + dsto[i], vv[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) P.pos[urow + rr[i]] = npos[i];
        if (P.score) {
#pragma unroll
          for (int i = 0; i < 4; ++i) P.score[urow + rr[i]] = nsc[i];
        }
      }
    }

    if (f1 > f0) {  // freed ids to the free list, their table entries to -1
      int32_t *fl = P.free_list + fc0 + free_start[u];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = f0 + q * kThreads + tid;
        if (i < f1) {
          fl[i] = fid[q];
          bt[lb0 + i] = -1;
        }
      }
      for (int i0 = f0 + 4 * kThreads; i0 < f1; i0 += 4 * kThreads) {
#pragma unroll
        for (int q = 0; q < 4; ++q) fid[q] = bt[lb0 + min(i0 + q * kThreads + tid, f1 - 1)];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = i0 + q * kThreads + tid;
          if (i < f1) {
            fl[i] = fid[q];
            bt[lb0 + i] = -1;
          }
        }
      }
    }
  }
}

// The heads that move in rank order (more at-risk rows than the staging
// holds), one 1024-thread workgroup each, after the gather: ascending rounds
// of destination ranks, every load of a round returned before any of its
// stores.  A source never lies below its destination, so no round reads a
// slot that an earlier round wrote, and within a round the loads precede the
// stores.  Other heads return at once.
__global__ __launch_bounds__(kSeqThreads) void compact_inorder_kernel(const CompactArgs P) {
  const int u = blockIdx.x, tid = threadIdx.x;
  const int32_t *hi = P.head_info + (size_t)u * 8;
  const int n = hi[0], m = hi[1], err = hi[2], seq = hi[6];
  if (!seq || err || n < 0 || n > P.max_slots || m <= 0 || m > n) return;
  const int n2 = n - m;
  const int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  const size_t urow = (size_t)u * P.max_slots;
  const int pshift = __ffs(P.row_bytes / 16) - 1;  // 16-byte pieces per row: 8, 16 or 32
  const int rpr = kSeqThreads >> pshift;           // rows per step of a round
  const int part = tid & ((1 << pshift) - 1);
  const int pool_rows = P.num_blocks * kBlock;
  for (int rb = 0; rb < n2; rb += kSeqRows * rpr) {
    // the round's destinations (past the head: its last row again, the
    // same bytes), their sources' pool rows (-1: the row stays), blocks,
    // new pos and score
    int rq[kSeqRows], srow[kSeqRows], db[kSeqRows], npos[kSeqRows];
    float nsc[kSeqRows];
#pragma unroll
    for (int i = 0; i < kSeqRows; ++i) {
      rq[i] = min(rb + i * rpr + (tid >> pshift), n2 - 1);
      srow[i] = P.src_row[urow + rq[i]];
      db[i] = bt[rq[i] / kBlock];
      npos[i] = P.new_pos[urow + rq[i]];
      nsc[i] = P.score ? P.new_score[urow + rq[i]] : 0.f;
    }
    size_t dsto[kSeqRows];
    uint4 kv[kSeqRows], vv[kSeqRows];
#pragma unroll
    for (int i = 0; i < kSeqRows; ++i) {
      dsto[i] = ((size_t)db[i] * kBlock + rq[i] % kBlock) * P.row_bytes + ((size_t)part << 4);
      const bool pooled = srow[i] >= 0 && srow[i] < pool_rows;
      const size_t so = pooled ? (size_t)srow[i] * P.row_bytes + ((size_t)part << 4) : dsto[i];
      kv[i] = ld16(P.k_pool + so);
      vv[i] = ld16(P.v_pool + so);
    }
    // every load of the round has returned before any thread stores
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSeqRows; ++i) {
      st16_nt(P.k_pool + dsto[i], kv[i]);
      st16_nt(P.v_pool + dsto[i], vv[i]);
      P.pos[urow + rq[i]] = npos[i];
      if (P.score) P.score[urow + rq[i]] = nsc[i];
    }
  }
}

static hipError_t launch_gather(const CompactArgs &a, hipStream_t s) {
  // enough workgroups to cover every item of a full cache, capped
  // kept rows per head are at most rows_cap (the fused path: the budget)
  const long long items =
      (long long)a.units * std::max(1, (a.rows_cap + a.rows_per_item - 1) / a.rows_per_item);
  const int grid = (int)(items < 2048 ? (items > 0 ? items : 1) : 2048);
  const size_t lds = sizeof(int) * (4 * (size_t)a.units + 2);  // item / free offsets, rows kept, order
  hipLaunchKernelGGL(compact_gather_kernel, dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(compact_prep_kernel, dim3(a.chunks, a.units), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_gather(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_inorder_kernel, dim3(a.units), dim3(kSeqThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvev
