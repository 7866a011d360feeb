// compact.hip -- in-place, order-preserving compaction of each KV head (gfx950).
//
// Kept slot s of rank r moves to slot r (r <= s).  Done in parallel this has
// one hazard: a destination row r < n' may still be the source of another
// kept token.  Those sources are exactly the kept slots in [first victim, n')
// ("at risk"); they are copied to the workspace first.  Three launches:
//   prep     (1024-slot chunk of one head per workgroup): checks the victim
//            list and the block ids, ranks the kept slots (a two-round
//            cooperative search gives the victims before the chunk), records
//            for each destination rank its source (physical row, staged
//            copy, or "stays"), the kept pos / score values, and copies the
//            at-risk rows to the workspace.  Reads the cache only.
//   gather   (persistent grid over (head, 64-rank) items): copies every
//            moving K and V row with 16-byte accesses, then pos and score;
//            the first item of each head also records the head's error
//            state and the number of blocks it frees.
//   finalize (256 logical blocks of one head per workgroup): appends the
//            emptied tail blocks [ceil(n'/16), ceil(n/16)) to the free list
//            in (b, h, block) order, clears their table entries, sets
//            seq_len = n' and completes the stats.
// ([H2O] "PagedAttention Memory Integration"; [VTOK] section 3.3, stage 3
// and section 3.5, invariants I1, I2 and I4.)
#include <hip/hip_runtime.h>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {
constexpr int kThreads = 256;
constexpr int kChunk = 1024;          // slots per prep workgroup
constexpr int kPerThread = kChunk / kThreads;
constexpr int kRankChunk = 64;        // destination ranks per gather item
constexpr int kFinBlocks = 256;       // logical blocks per finalize workgroup
constexpr int kMaxUnits = kCompactMaxUnits;  // heads a gather workgroup indexes in LDS

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

// Number of entries of the ascending array a[0, m) below key (lower bound),
// found by the whole workgroup in two rounds of independent loads: 256
// evenly spaced samples bracket the answer, then the bracket is counted.
__device__ int wg_lower_bound(const int32_t *a, int m, int key) {
  const int tid = threadIdx.x;
  const int S = (m + kThreads - 1) / kThreads;  // sample spacing, >= 1 when m > 0
  const int idx = tid * S;
  const int c = __syncthreads_count(idx < m && a[idx] < key);
  if (c == 0) return 0;
  // a[(c-1)*S] < key, and a[c*S] >= key (or c*S >= m)
  const int base = (c - 1) * S + 1;
  const int len = min(S - 1, m - base);
  int cnt = 0;
  for (int off = 0; off < len; off += kThreads)
    cnt += __syncthreads_count(off + tid < len && a[base + off + tid] < key);
  return base + cnt;
}
}  // namespace

__global__ __launch_bounds__(kThreads) void compact_prep_kernel(const CompactArgs P) {
  __shared__ uint8_t flag[kChunk];
  __shared__ int stage_s[kChunk], stage_i[kChunk];
  __shared__ int s_err, s_nstage;
  __shared__ int wave_tot[kThreads / kWave];

  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  if (u == 0 && c == 0 && tid == 0) {
    *P.fc0 = *P.free_count;
    for (int i = 0; i < 5; ++i) P.stats[i] = 0;
  }
  const int n = P.seq_len[u];
  const int m = P.n_victims[u];
  int err = 0;
  if (n < 0 || n > P.max_slots) err = 2;
  else if (m < 0 || m > n) err = 1;
  const int32_t *vic = P.victims + (size_t)u * P.max_slots;
  if (tid == 0) {
    s_err = 0;
    s_nstage = 0;
    if (c == 0) P.head_info[u * 4 + 0] = n;
  }
  __syncthreads();
  // the victim list must be strictly ascending inside [0, n): chunk c checks
  // the pairs starting at indices [m*c/chunks, m*(c+1)/chunks)
  if (!err && m > 0) {
    const int i0 = (int)((int64_t)m * c / P.chunks), i1 = (int)((int64_t)m * (c + 1) / P.chunks);
    int bad = 0;
    for (int i = i0 + tid; i < i1; i += kThreads) {
      const int v = vic[i];
      if (v < 0 || v >= n || (i + 1 < m && vic[i + 1] <= v)) bad = 1;
    }
    if (bad) atomicOr(&s_err, 1);
  }
  __syncthreads();
  err |= s_err;
  const int s0 = c * kChunk;
  if (err || m == 0 || s0 >= n) {
    if (tid == 0) P.chunk_err[(size_t)u * P.chunks + c] = err;
    return;
  }
  const int s1 = min(s0 + kChunk, n);
  const int j0 = wg_lower_bound(vic, m, s0);
  const int j1 = wg_lower_bound(vic, m, s1);
  for (int i = tid; i < kChunk; i += kThreads) flag[i] = 0;
  // every block holding a slot of this chunk must be a valid pool index
  const int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  for (int lb = s0 / kBlock + tid; lb < (s1 + kBlock - 1) / kBlock; lb += kThreads) {
    const int blk = bt[lb];
    if (blk < 0 || blk >= P.num_blocks) atomicOr(&s_err, 1);
  }
  __syncthreads();
  for (int j = j0 + tid; j < j1; j += kThreads) {
    const int v = vic[j];
    if (v >= s0 && v < s1) flag[v - s0] = 1;
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
  const int first = vic[0];
  int r = (s0 - j0) + excl;  // kept slots before s0, plus those before mine in the chunk
  const size_t urow = (size_t)u * P.max_slots;
  int my_err = 0;
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
      const int k = atomicAdd(&s_nstage, 1);
      stage_s[k] = s;
      stage_i[k] = si;
    } else {                          // slots >= n' are never written: read in place
      const int blk = bt[s / kBlock];
      src = (blk >= 0 && blk < P.num_blocks) ? blk * kBlock + s % kBlock : 0;
    }
    P.src_of[urow + r] = src;
    P.new_pos[urow + r] = P.pos[urow + s];
    if (P.score) P.new_score[urow + r] = P.score[urow + s];
    ++r;
  }
  if (my_err) atomicOr(&s_err, 1);
  __syncthreads();
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
  __syncthreads();
  if (tid == 0) P.chunk_err[(size_t)u * P.chunks + c] = err | s_err;
}

// Persistent grid: every workgroup indexes the per-head item counts in LDS.
__global__ __launch_bounds__(kThreads) void compact_gather_kernel(const CompactArgs P) {
  __shared__ int item_start[kMaxUnits + 1];
  __shared__ int wave_tot[kThreads / kWave];
  __shared__ int s_total;
  const int tid = threadIdx.x, lane = lane_id();
  const int U = P.units;
  // items per head: ceil(n'/64) row chunks, at least one (it records the head state)
  int base_count = 0;
  for (int b0 = 0; b0 < U; b0 += kThreads) {
    const int u = b0 + tid;
    int cnt = 0;
    if (u < U) {
      const int n = P.head_info[u * 4 + 0];
      const int m = P.n_victims[u];
      const bool ok = n >= 0 && n <= P.max_slots && m > 0 && m <= n;
      cnt = ok ? max(1, (n - m + kRankChunk - 1) / kRankChunk) : 1;
    }
    const int ex = block_exclusive_scan(cnt, wave_tot);
    if (u < U) item_start[u] = base_count + ex;
    if (tid == kThreads - 1) s_total = base_count + ex + cnt;
    __syncthreads();
    base_count = s_total;
    __syncthreads();
  }
  if (tid == 0) item_start[U] = base_count;
  __syncthreads();
  const int total = base_count;
  const int pieces = P.row_bytes / 16;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // head of this item: the last u with item_start[u] <= item
    int lo = 0, hi = U - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (item_start[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int u = lo, k = item - item_start[u];
    const int n = P.head_info[u * 4 + 0];
    const int m = P.n_victims[u];
    // head error: any prep chunk flag, or n / m out of range
    int e = 0;
    for (int c = lane; c < P.chunks; c += kWave) e |= P.chunk_err[(size_t)u * P.chunks + c];
    const bool nm_bad = n < 0 || n > P.max_slots || m < 0 || m > n;
    const bool head_bad = __any(e != 0) || nm_bad;
    if (k == 0 && tid == 0) {
      int ev = nm_bad ? ((n < 0 || n > P.max_slots) ? 2 : 1) : 0;
      for (int c = 0; c < P.chunks && !nm_bad; ++c) ev |= P.chunk_err[(size_t)u * P.chunks + c];
      P.head_info[u * 4 + 2] = ev;
      P.head_info[u * 4 + 3] = (ev || m <= 0) ? 0 : (n + kBlock - 1) / kBlock - (n - m + kBlock - 1) / kBlock;
    }
    if (head_bad || m <= 0) continue;
    const int n2 = n - m;
    const int r0 = k * kRankChunk;
    if (r0 >= n2) continue;
    const int r1 = min(r0 + kRankChunk, n2);
    const size_t urow = (size_t)u * P.max_slots;
    const int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
    for (int idx = tid; idx < (r1 - r0) * pieces; idx += kThreads) {
      const int r = r0 + idx / pieces, part = idx % pieces;
      const int src = P.src_of[urow + r];
      if (src == -1) continue;
      const size_t dst = ((size_t)bt[r / kBlock] * kBlock + r % kBlock) * P.row_bytes + (size_t)part * 16;
      uint4 kv, vv;
      if (src >= 0) {
        const size_t so = (size_t)src * P.row_bytes + (size_t)part * 16;
        kv = ld16(P.k_pool + so);
        vv = ld16(P.v_pool + so);
      } else {
        const size_t so = ((size_t)u * P.stage_rows + (-2 - src)) * P.row_bytes + (size_t)part * 16;
        kv = ld16(P.stage_k + so);
        vv = ld16(P.stage_v + so);
      }
      st16(P.k_pool + dst, kv);
      st16(P.v_pool + dst, vv);
    }
    int moved = 0, risk = 0;
    for (int r = r0 + tid; r < r1; r += kThreads) {
      const int src = P.src_of[urow + r];
      if (src == -1) continue;
      P.pos[urow + r] = P.new_pos[urow + r];
      if (P.score) P.score[urow + r] = P.new_score[urow + r];
      ++moved;
      risk += src <= -2 ? 1 : 0;
    }
    // one atomic per wave
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) {
      moved += __shfl_xor(moved, o);
      risk += __shfl_xor(risk, o);
    }
    if (lane == 0 && moved) {
      atomicAdd(reinterpret_cast<unsigned long long *>(&P.stats[1]), (unsigned long long)moved);
      atomicAdd(reinterpret_cast<unsigned long long *>(&P.stats[2]),
                (unsigned long long)moved * 4ull * (unsigned long long)P.row_bytes);
      if (risk) atomicAdd(reinterpret_cast<unsigned long long *>(&P.stats[3]), (unsigned long long)risk);
    }
  }
}

// Workgroup (k, u): logical blocks [ceil(n'/16) + 256k, ...) of head u.
__global__ __launch_bounds__(kThreads) void compact_finalize_kernel(const CompactArgs P) {
  __shared__ long long s_before, s_total;
  const int k = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  if (tid == 0) {
    s_before = 0;
    s_total = 0;
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
  if (k == 0 && tid == 0) {
    if (err) {
      atomicOr(reinterpret_cast<unsigned long long *>(&P.stats[4]), (unsigned long long)err);
    } else {
      const int m = P.n_victims[u];
      if (m > 0) P.seq_len[u] = n - m;
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
  // enough workgroups to cover every 64-rank item of a full cache, capped
  const long long items = (long long)a.units * ((a.max_slots + kRankChunk - 1) / kRankChunk);
  const int grid = (int)(items < 2048 ? (items > 0 ? items : 1) : 2048);
  hipLaunchKernelGGL(compact_gather_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int fin_x = (a.max_blocks + kFinBlocks - 1) / kFinBlocks;
  hipLaunchKernelGGL(compact_finalize_kernel, dim3(fin_x, a.units), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvev
