// compact.hip -- in-place, order-preserving compaction of each KV head (gfx950).
//
// Kept slot s of rank r moves to slot r (r <= s).  Done in parallel this has
// one hazard: a destination row r < n' may still be the source of another
// kept token.  Those sources are exactly the kept slots in [first victim, n')
// ("at risk"); they are copied to the workspace first.  Three launches:
//   prep     (slot chunk per workgroup): ranks from the sorted victim list,
//            the source of every destination rank, the kept pos / score
//            values, and the staging copy of the at-risk rows.  Reads the
//            cache only.
//   gather   (rank chunk per workgroup): every moving row is copied with
//            16-byte vector accesses from the pool (sources >= n', never
//            written in this launch) or from the staged copy.
//   finalize (one workgroup): emptied tail blocks [ceil(n'/16), ceil(n/16))
//            are appended to the free list in (b, h, block) order, their
//            table entries cleared, seq_len set to n', stats completed.
// ([H2O] "PagedAttention Memory Integration"; [VTOK] section 3.3, stage 3
// and section 3.5, invariants I1, I2 and I4.)
#include <hip/hip_runtime.h>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {
constexpr int kThreads = 256;
constexpr int kChunk = 1024;          // slots (prep) or ranks (gather) per workgroup
constexpr int kPerThread = kChunk / kThreads;
constexpr int kFinThreads = 1024;

// Exclusive prefix sum over the workgroup (any size that is a multiple of 64).
__device__ int block_exclusive_scan(int v, int *wave_tot) {
  const int lane = lane_id(), wv = threadIdx.x / kWave, nw = blockDim.x / kWave;
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
  (void)nw;
  return before + incl - v;
}

__device__ __forceinline__ int lower_bound(const int32_t *a, int n, int key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < key) lo = mid + 1; else hi = mid;
  }
  return lo;
}
}  // namespace

// head_info[u*4 + 0] = n before the call, [1] = first victim slot.
__global__ __launch_bounds__(kThreads) void compact_prep_kernel(const CompactArgs P) {
  __shared__ uint8_t flag[kChunk];
  __shared__ int stage_s[kChunk], stage_i[kChunk];
  __shared__ int s_j0, s_j1, s_err, s_nstage;
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
    if (c == 0) {
      P.head_info[u * 4 + 0] = n;
      P.head_info[u * 4 + 1] = (!err && m > 0) ? vic[0] : n;
    }
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
  if (tid == 0) {
    s_j0 = lower_bound(vic, m, s0);
    s_j1 = lower_bound(vic, m, s1);
  }
  for (int i = tid; i < kChunk; i += kThreads) flag[i] = 0;
  __syncthreads();
  const int j0 = s_j0, j1 = s_j1;
  for (int j = j0 + tid; j < j1; j += kThreads) {
    const int v = vic[j];
    if (v >= s0 && v < s1) flag[v - s0] = 1;
  }
  __syncthreads();

  // every block holding a slot of this chunk must be a valid pool index
  for (int lb = s0 / kBlock + tid; lb < (s1 + kBlock - 1) / kBlock; lb += kThreads) {
    const int blk = P.block_table[(size_t)u * P.max_blocks + lb];
    if (blk < 0 || blk >= P.num_blocks) atomicOr(&s_err, 1);
  }
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
  const int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
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
    } else {
      src = s;                        // read in place: slots >= n' are never written
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
    if (blk < 0 || blk >= P.num_blocks) { atomicOr(&s_err, 1); continue; }
    const size_t src = ((size_t)blk * kBlock + s % kBlock) * P.row_bytes + (size_t)part * 16;
    const size_t dst = ((size_t)u * P.stage_rows + stage_i[k]) * P.row_bytes + (size_t)part * 16;
    st16(P.stage_k + dst, ld16(P.k_pool + src));
    st16(P.stage_v + dst, ld16(P.v_pool + src));
  }
  __syncthreads();
  if (tid == 0) P.chunk_err[(size_t)u * P.chunks + c] = err | s_err;
}

__global__ __launch_bounds__(kThreads) void compact_gather_kernel(const CompactArgs P) {
  __shared__ int s_err, s_moved, s_risk;
  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  if (tid == 0) {
    s_err = 0;
    s_moved = 0;
    s_risk = 0;
  }
  __syncthreads();
  for (int i = tid; i < P.chunks; i += kThreads)
    if (P.chunk_err[(size_t)u * P.chunks + i]) atomicOr(&s_err, 1);
  __syncthreads();
  if (s_err) return;
  const int n = P.head_info[u * 4 + 0];
  const int m = P.n_victims[u];
  const int n2 = n - m;
  const int r0 = c * kChunk;
  if (m == 0 || r0 >= n2) return;
  const int r1 = min(r0 + kChunk, n2);
  const size_t urow = (size_t)u * P.max_slots;
  const int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  const int pieces = P.row_bytes / 16;
  for (int idx = tid; idx < (r1 - r0) * pieces; idx += kThreads) {
    const int r = r0 + idx / pieces, part = idx % pieces;
    const int src = P.src_of[urow + r];
    if (src == -1) continue;
    const int dblk = bt[r / kBlock];
    const size_t dst = ((size_t)dblk * kBlock + r % kBlock) * P.row_bytes + (size_t)part * 16;
    uint4 kv, vv;
    if (src >= 0) {
      const size_t so = ((size_t)bt[src / kBlock] * kBlock + src % kBlock) * P.row_bytes +
                        (size_t)part * 16;
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
  if (moved) atomicAdd(&s_moved, moved);
  if (risk) atomicAdd(&s_risk, risk);
  __syncthreads();
  if (tid == 0 && s_moved) {
    atomicAdd(reinterpret_cast<unsigned long long *>(&P.stats[1]), (unsigned long long)s_moved);
    atomicAdd(reinterpret_cast<unsigned long long *>(&P.stats[2]),
              (unsigned long long)s_moved * 4ull * (unsigned long long)P.row_bytes);
    atomicAdd(reinterpret_cast<unsigned long long *>(&P.stats[3]), (unsigned long long)s_risk);
  }
}

// One workgroup: free-list append in (b, h, logical block) order.
__global__ __launch_bounds__(kFinThreads) void compact_finalize_kernel(const CompactArgs P) {
  __shared__ int wave_tot[kFinThreads / kWave];
  __shared__ int s_head_off[kFinThreads], s_head_freed[kFinThreads], s_head_n2[kFinThreads];
  __shared__ long long s_total;
  __shared__ int s_status;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_total = 0;
    s_status = 0;
  }
  __syncthreads();
  // pass 1: blocks freed over all consistent heads
  auto head_state = [&](int u, int &freed, int &n2, int &err) {
    const int n = P.head_info[u * 4 + 0];
    const int m = P.n_victims[u];
    err = 0;
    for (int i = 0; i < P.chunks; ++i) err |= P.chunk_err[(size_t)u * P.chunks + i];
    if (n < 0 || n > P.max_slots) err |= 2;
    else if (m < 0 || m > n) err |= 1;
    freed = 0;
    n2 = n;
    if (!err) {
      n2 = n - m;
      freed = (n + kBlock - 1) / kBlock - (n2 + kBlock - 1) / kBlock;
    }
  };
  for (int base = 0; base < P.units; base += kFinThreads) {
    const int u = base + tid;
    int freed = 0, n2 = 0, err = 0;
    if (u < P.units) head_state(u, freed, n2, err);
    if (err) atomicOr(&s_status, err);
    if (freed) atomicAdd(reinterpret_cast<unsigned long long *>(&s_total), (unsigned long long)freed);
  }
  __syncthreads();
  const int fc0 = *P.fc0;
  const bool room = (long long)fc0 + s_total <= (long long)P.free_capacity && fc0 >= 0;
  // pass 2: offsets and appends, 1024 heads at a time
  long long running = 0;
  for (int base = 0; base < P.units; base += kFinThreads) {
    const int u = base + tid;
    int freed = 0, n2 = 0, err = 0;
    if (u < P.units) head_state(u, freed, n2, err);
    if (!room) freed = 0;
    const int off = block_exclusive_scan(freed, wave_tot);
    s_head_off[tid] = (int)running + off;
    s_head_freed[tid] = freed;
    s_head_n2[tid] = (u < P.units && !err) ? n2 : -1;
    __syncthreads();
    const int cnt = min(kFinThreads, P.units - base);
    for (int k = 0; k < cnt; ++k) {
      const int uu = base + k;
      const int f = s_head_freed[k];
      const int nn2 = s_head_n2[k];
      if (nn2 < 0) continue;
      int32_t *bt = P.block_table + (size_t)uu * P.max_blocks;
      const int lb0 = (nn2 + kBlock - 1) / kBlock;
      for (int i = tid; i < f; i += kFinThreads) {
        P.free_list[fc0 + s_head_off[k] + i] = bt[lb0 + i];
        bt[lb0 + i] = -1;
      }
      if (tid == 0) P.seq_len[uu] = nn2;
    }
    running = s_head_off[cnt - 1] + s_head_freed[cnt - 1];
    __syncthreads();
  }
  if (tid == 0) {
    if (room) *P.free_count = fc0 + (int)s_total;
    int st = s_status | (room ? 0 : 4);
    P.stats[0] = room ? s_total : 0;
    P.stats[4] |= st;
  }
}

hipError_t launch_compact(const CompactArgs &a, hipStream_t s) {
  dim3 grid(a.chunks, a.units);
  hipLaunchKernelGGL(compact_prep_kernel, grid, dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_gather_kernel, grid, dim3(kThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_finalize_kernel, dim3(1), dim3(kFinThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvev
