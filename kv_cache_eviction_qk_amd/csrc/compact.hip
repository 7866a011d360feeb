// compact.hip -- in-place, order-preserving compaction of each KV head (gfx950).
//
// Kept slot s of rank r moves to slot r (r <= s).  Done in parallel this has
// one hazard: a destination row r < n' may still be the source of another
// kept token.  Those sources are exactly the kept slots in [first victim, n')
// ("at risk"); they are copied to the workspace first.  Three launches:
//   prep     (1024-slot chunk of one head per workgroup): checks the victim
//            list and the block ids, finds the victims inside the chunk
//            (256 evenly spaced samples bracket them, one range load fetches
//            them), ranks the kept slots, records for each destination rank
//            its source (physical row, staged copy, or "stays") and the kept
//            pos / score values, and copies the at-risk rows to the
//            workspace.  Reads the cache only.
//   gather   (persistent grid over (head, rank range) items): each thread
//            issues all of its 16-byte K and V loads before any store.
//   finalize (256 logical blocks of one head per workgroup): appends the
//            emptied tail blocks [ceil(n'/16), ceil(n/16)) to the free list
//            in (b, h, block) order, clears their table entries, sets
//            seq_len = n', completes the stats and clears the head's error
//            word for the next call.
// ([H2O] "PagedAttention Memory Integration"; [VTOK] section 3.3, stage 3
// and section 3.5, invariants I1, I2 and I4.)
#include <hip/hip_runtime.h>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {
constexpr int kThreads = 256;
constexpr int kChunk = kCompactChunk;   // slots per prep workgroup
constexpr int kPerThread = kChunk / kThreads;
constexpr int kFinBlocks = 256;         // logical blocks per finalize workgroup
constexpr int kMaxUnits = kCompactMaxUnits;
constexpr int kRange = 4096;            // victims a prep workgroup stages in LDS

// Exclusive prefix sum over a 256-thread workgroup.
__device__ int block_exclusive_scan(int v, int *wave_tot) {
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) wave_tot[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wv; ++w) before += wave_tot[w];
  __syncthreads();
  return before + incl - v;
}

// Lower bound of key in the ascending a[0, m): counts the bracket [base,
// base + len) after the samples placed it there (one more round of loads).
__device__ int bracket_count(const int32_t *a, int base, int len, int key) {
  int cnt = 0;
  for (int off = 0; off < len; off += kThreads)
    cnt += __syncthreads_count(off + threadIdx.x < len && a[base + off + threadIdx.x] < key);
  return base + cnt;
}
}  // namespace

__global__ __launch_bounds__(kThreads) void compact_prep_kernel(const CompactArgs P) {
  __shared__ uint8_t flag[kChunk];
  __shared__ int vr[kRange];
  __shared__ int stage_s[kChunk], stage_i[kChunk];
  __shared__ int s_err, s_nstage;
  __shared__ int wave_tot[kThreads / kWave];
  __shared__ int r0s[kThreads / kWave], r1s[kThreads / kWave];

  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  if (u == 0 && c == 0 && tid == 0) {
    *P.fc0 = *P.free_count;
    for (int i = 0; i < 5; ++i) P.stats[i] = 0;
  }
  const int n = P.seq_len[u];
  const int m = P.n_victims[u];
  if (c == 0 && tid == 0) P.head_info[u * 4 + 0] = n;
  // n or m out of range: the gather sees it from seq_len / n_victims directly
  if (n < 0 || n > P.max_slots || m < 0 || m > n || m == 0) return;
  const int s0 = c * kChunk;
  const int32_t *vic = P.victims + (size_t)u * P.max_slots;
  const size_t urow = (size_t)u * P.max_slots;
  const int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  if (tid == 0) {
    s_err = 0;
    s_nstage = 0;
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
  for (int lb = s0 / kBlock + tid; lb < (s1 + kBlock - 1) / kBlock; lb += kThreads) {
    const int blk = bt[lb];
    if (blk < 0 || blk >= P.num_blocks) bad = 1;
  }
  const int S = (m + kThreads - 1) / kThreads;  // sample spacing
  const int samp = (tid * S < m) ? vic[tid * S] : INT_MAX;
  const int first = vic[0];
  if (bad) atomicOr(&s_err, 1);
  const int c0 = __syncthreads_count(samp < s0);
  const int c1 = __syncthreads_count(samp < s1);
  if (!live_chunk) {
    if (tid == 0 && s_err) atomicOr(&P.head_err[u], 1u);
    return;
  }
  // victims before s0 lie in [lo0, hi0], victims before s1 in [lo1, hi1]
  const int lo0 = c0 ? (c0 - 1) * S + 1 : 0, hi0 = min(c0 * S, m);
  const int lo1 = c1 ? (c1 - 1) * S + 1 : 0, hi1 = min(c1 * S, m);
  int j0, j1;
  if (hi1 - lo0 <= kRange) {
    // ---- one range load covers both brackets and every victim in the chunk
    // (at most kRange entries: 16 per thread, all issued before any store)
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
    // block sums of the per-thread counts
    {
      int a0 = cnt0, a1 = cnt1;
#pragma unroll
      for (int o = kWave / 2; o >= 1; o >>= 1) {
        a0 += __shfl_xor(a0, o);
        a1 += __shfl_xor(a1, o);
      }
      if (lane_id() == 0) {
        r0s[tid / kWave] = a0;
        r1s[tid / kWave] = a1;
      }
      __syncthreads();
      int t0 = 0, t1 = 0;
      for (int w = 0; w < kThreads / kWave; ++w) {
        t0 += r0s[w];
        t1 += r1s[w];
      }
      j0 = lo0 + t0;
      j1 = lo0 + t1;
    }
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

  int kept = 0;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int s = s0 + tid * kPerThread + q;
    kept += (s < s1 && !flag[s - s0]) ? 1 : 0;
  }
  const int excl = block_exclusive_scan(kept, wave_tot);
  const int n2 = n - m;
  int r = (s0 - j0) + excl;  // kept slots before s0, plus those before mine in the chunk
  int my_err = 0, my_moved = 0, my_staged = 0;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int s = s0 + tid * kPerThread + q;
    if (s >= s1 || flag[s - s0]) continue;
    if (r < 0 || r >= n2) { my_err = 1; ++r; continue; }
    int src;
    if (r == s) {
      src = -1;                       // stays in place
    } else if (s < n2) {              // at risk: staged before the gather
      const int si = r - first;
      if (si < 0 || si >= P.stage_rows) { my_err = 1; ++r; continue; }
      src = -2 - si;
      ++my_staged;
      const int k = atomicAdd(&s_nstage, 1);
      stage_s[k] = s;
      stage_i[k] = si;
    } else {                          // slots >= n' are never written: read in place
      const int blk = bt[s / kBlock];
      src = (blk >= 0 && blk < P.num_blocks) ? blk * kBlock + s % kBlock : 0;
    }
    my_moved += src != -1 ? 1 : 0;
    P.src_of[urow + r] = src;
    P.new_pos[urow + r] = posv[q];
    if (P.score) P.new_score[urow + r] = scv[q];
    ++r;
  }
  if (my_err) atomicOr(&s_err, 1);
  // per-chunk counts for the stats (summed per head by the finalize step)
  {
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) {
      my_moved += __shfl_xor(my_moved, o);
      my_staged += __shfl_xor(my_staged, o);
    }
    if (lane_id() == 0) {
      r0s[tid / kWave] = my_moved;
      r1s[tid / kWave] = my_staged;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int a0 = 0, a1 = 0;
    for (int w = 0; w < kThreads / kWave; ++w) {
      a0 += r0s[w];
      a1 += r1s[w];
    }
    P.chunk_mv[((size_t)u * P.chunks + c) * 2 + 0] = a0;
    P.chunk_mv[((size_t)u * P.chunks + c) * 2 + 1] = a1;
  }
  // staging copy of the at-risk K and V rows (16-byte pieces)
  const int pieces = P.row_bytes / 16;
  const int ns = s_nstage;
  for (int idx = tid; idx < ns * pieces; idx += kThreads) {
    const int k = idx / pieces, part = idx % pieces;
    const int s = stage_s[k];
    const int blk = bt[s / kBlock];
    if (blk < 0 || blk >= P.num_blocks) continue;  // flagged above
    const size_t src = ((size_t)blk * kBlock + s % kBlock) * P.row_bytes + (size_t)part * 16;
    const size_t dst = ((size_t)u * P.stage_rows + stage_i[k]) * P.row_bytes + (size_t)part * 16;
    st16(P.stage_k + dst, ld16(P.k_pool + src));
    st16(P.stage_v + dst, ld16(P.v_pool + src));
  }
  if (tid == 0 && s_err) atomicOr(&P.head_err[u], 1u);
}

// Persistent grid over (head, rank range) items; every head has at least one
// item, which records the head's error state and the blocks it frees.
__global__ __launch_bounds__(kThreads) void compact_gather_kernel(const CompactArgs P) {
  __shared__ int item_start[kMaxUnits + 1];
  __shared__ int wave_tot[kThreads / kWave];
  __shared__ int s_total;
  const int tid = threadIdx.x, lane = lane_id();
  const int U = P.units, RC = P.rows_per_item;
  int base_count = 0;
  for (int b0 = 0; b0 < U; b0 += kThreads) {
    const int u = b0 + tid;
    int cnt = 0;
    if (u < U) {
      const int n = P.seq_len[u];
      const int m = P.n_victims[u];
      const bool ok = n >= 0 && n <= P.max_slots && m > 0 && m <= n;
      cnt = ok ? max(1, (n - m + RC - 1) / RC) : 1;
    }
    const int ex = block_exclusive_scan(cnt, wave_tot);
    if (u < U) item_start[u] = base_count + ex;
    if (tid == kThreads - 1) s_total = base_count + ex + cnt;
    __syncthreads();
    base_count = s_total;
    __syncthreads();
  }
  const int total = base_count;
  const int pieces = P.row_bytes / 16;  // 16-byte pieces per row (8, 16 or 32)

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    int lo = 0, hi = U - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (item_start[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int u = lo, k = item - item_start[u];
    const int n = P.seq_len[u];
    const int m = P.n_victims[u];
    const uint32_t herr = P.head_err[u];
    int ev = (int)herr;
    if (n < 0 || n > P.max_slots) ev = 2;
    else if (m < 0 || m > n) ev = 1;
    if (k == 0 && tid == 0) {
      P.head_info[u * 4 + 2] = ev;
      P.head_info[u * 4 + 3] = (ev || m <= 0) ? 0 : (n + kBlock - 1) / kBlock - (n - m + kBlock - 1) / kBlock;
    }
    if (ev || m <= 0) continue;
    const int n2 = n - m;
    const int r0 = k * RC;
    if (r0 >= n2) continue;
    const int r1 = min(r0 + RC, n2);
    const size_t urow = (size_t)u * P.max_slots;
    // lane group of `pieces` threads per row, one 16-byte piece each, so an
    // instruction covers whole rows; 4 rows per thread, all loads first
    const int rpr = kThreads / pieces;  // rows per round
    const int part = tid % pieces;
    int rr[4], srcv[4], dblk[4], npos[4];
    float nsc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rr[i] = r0 + i * rpr + tid / pieces;
      const bool in = rr[i] < r1;
      srcv[i] = in ? P.src_of[urow + rr[i]] : -1;
      dblk[i] = in ? P.block_table[(size_t)u * P.max_blocks + rr[i] / kBlock] : 0;
      npos[i] = (in && part == 0) ? P.new_pos[urow + rr[i]] : 0;
      nsc[i] = (in && part == 0 && P.score) ? P.new_score[urow + rr[i]] : 0.f;
    }
    uint4 kv[4], vv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int src = srcv[i];
      if (src != -1) {
        const uint8_t *ks, *vs;
        if (src >= 0) {
          ks = P.k_pool + (size_t)src * P.row_bytes;
          vs = P.v_pool + (size_t)src * P.row_bytes;
        } else {
          const size_t so = ((size_t)u * P.stage_rows + (-2 - src)) * P.row_bytes;
          ks = P.stage_k + so;
          vs = P.stage_v + so;
        }
        kv[i] = ld16(ks + (size_t)part * 16);
        vv[i] = ld16(vs + (size_t)part * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (srcv[i] == -1) continue;
      const size_t dst = ((size_t)dblk[i] * kBlock + rr[i] % kBlock) * P.row_bytes + (size_t)part * 16;
      st16(P.k_pool + dst, kv[i]);
      st16(P.v_pool + dst, vv[i]);
      if (part == 0) {
        P.pos[urow + rr[i]] = npos[i];
        if (P.score) P.score[urow + rr[i]] = nsc[i];
      }
    }
  }
}

// Workgroup (k, u): logical blocks [ceil(n'/16) + 256k, ...) of head u.
__global__ __launch_bounds__(kThreads) void compact_finalize_kernel(const CompactArgs P) {
  __shared__ long long s_before, s_total, s_mv, s_st;
  const int k = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  if (tid == 0) {
    s_before = 0;
    s_total = 0;
    s_mv = 0;
    s_st = 0;
  }
  __syncthreads();
  long long before = 0, total = 0;
  for (int v = tid; v < P.units; v += kThreads) {
    const long long f = P.head_info[v * 4 + 3];
    total += f;
    if (v < u) before += f;
  }
  if (before) atomicAdd(reinterpret_cast<unsigned long long *>(&s_before), (unsigned long long)before);
  if (total) atomicAdd(reinterpret_cast<unsigned long long *>(&s_total), (unsigned long long)total);
  __syncthreads();
  const int fc0 = *P.fc0;
  const bool room = fc0 >= 0 && (long long)fc0 + s_total <= (long long)P.free_capacity;
  const int n = P.head_info[u * 4 + 0];
  const int err = P.head_info[u * 4 + 2];
  const int freed = room ? P.head_info[u * 4 + 3] : 0;
  // rows moved and staged of this head: the prep chunks' counts, summed in parallel
  long long mv = 0, st = 0;
  if (k == 0 && !err && n > 0 && n <= P.max_slots) {
    const int live = (n + kChunk - 1) / kChunk;  // chunks prep wrote
    for (int c = tid; c < live; c += kThreads) {
      mv += P.chunk_mv[((size_t)u * P.chunks + c) * 2 + 0];
      st += P.chunk_mv[((size_t)u * P.chunks + c) * 2 + 1];
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) {
      mv += __shfl_xor(mv, o);
      st += __shfl_xor(st, o);
    }
    if (lane_id() == 0 && (mv || st)) {
      atomicAdd(reinterpret_cast<unsigned long long *>(&s_mv), (unsigned long long)mv);
      atomicAdd(reinterpret_cast<unsigned long long *>(&s_st), (unsigned long long)st);
    }
  }
  __syncthreads();
  if (k == 0 && tid == 0) {
    P.head_err[u] = 0u;  // state for the next call
    if (err) {
      atomicOr(reinterpret_cast<unsigned long long *>(&P.stats[4]), (unsigned long long)err);
    } else {
      const int m = P.n_victims[u];
      if (m > 0) {
        P.seq_len[u] = n - m;
        const long long mv = s_mv, st = s_st;
        if (mv) {
          atomicAdd(reinterpret_cast<unsigned long long *>(&P.stats[1]), (unsigned long long)mv);
          atomicAdd(reinterpret_cast<unsigned long long *>(&P.stats[2]),
                    (unsigned long long)mv * 4ull * (unsigned long long)P.row_bytes);
        }
        if (st) atomicAdd(reinterpret_cast<unsigned long long *>(&P.stats[3]), (unsigned long long)st);
      }
      if (freed) atomicAdd(reinterpret_cast<unsigned long long *>(&P.stats[0]), (unsigned long long)freed);
    }
    if (u == P.units - 1) {
      if (room) *P.free_count = fc0 + (int)s_total;
      else atomicOr(reinterpret_cast<unsigned long long *>(&P.stats[4]), 4ull);
    }
  }
  if (err || freed == 0) return;
  const int n2 = n - P.n_victims[u];
  const int lb0 = (n2 + kBlock - 1) / kBlock;
  int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  const int i = k * kFinBlocks + tid;
  if (i < freed) {
    P.free_list[fc0 + s_before + i] = bt[lb0 + i];
    bt[lb0 + i] = -1;
  }
}

hipError_t launch_compact(const CompactArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(compact_prep_kernel, dim3(a.chunks, a.units), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // enough workgroups to cover every item of a full cache, capped
  const long long items =
      (long long)a.units * ((a.max_slots + a.rows_per_item - 1) / a.rows_per_item);
  const int grid = (int)(items < 2048 ? (items > 0 ? items : 1) : 2048);
  hipLaunchKernelGGL(compact_gather_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int fin_x = (a.max_blocks + kFinBlocks - 1) / kFinBlocks;
  hipLaunchKernelGGL(compact_finalize_kernel, dim3(fin_x, a.units), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvev
