// vtoken.hip -- vToken liveness marks and lazy, threshold-gated reclamation
// of each KV head's blocks (gfx950).
//
// [VTOK] section 3.2: the token table of a head is its block list plus, per
// slot, the token's position and a liveness byte; evicting a token clears the
// byte and the live count of its block, and moves nothing.  Section 3.3,
// stages 1-3, and section 3.5 (I1, I2, I4): a head whose waste
// F = 1 - live / (16 * allocated blocks) exceeds theta_F packs the live tokens
// of its first non-full blocks (the growing tail block excluded) into
// ceil(T / 16) destination blocks from the top of the free list, filled
// completely in logical order, only when that frees strictly more blocks than
// it takes; heads that find no headroom are deferred.
//
// Reclamation is four launches, each a global step of the plan:
//   plan   (one workgroup per head): allocated blocks, live tokens, F, the
//          sources (ordered selection over the block list), T and D;
//   admit  (one workgroup): heads in (b, h) order take D destinations from
//          the top of the free list while enough remain (a sequential scan
//          over LDS); copies the destination ids to the workspace (the free
//          list's top is overwritten by the pushes later); push offsets of
//          the sources; every statistic; the new free count;
//   move   (a wave per source slot): each live source token's K and V row to
//          its destination row, its position and score staged by rank;
//   apply  (one workgroup per admitted head): the block list entries of the
//          sources, liveness, live counts, positions and scores of their
//          slots, and the sources appended to the free list.
// Destination rows are fresh blocks, so no copy reads what another writes;
// the per-slot table of the sources is rewritten only after every copy.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kvev_device.h"
#include "kvev_kernels.h"

namespace kvev {

namespace {
constexpr int kPlanThreads = 1024;
constexpr int kPlanPer = 4;   // logical blocks per plan thread and pass
constexpr int kAdmitThreads = 1024;
constexpr int kMoveWaves = 4;  // source blocks per move workgroup (a wave each)
constexpr size_t kNoRow = ~(size_t)0;

// Exclusive prefix sum over the workgroup (every thread calls it).
__device__ __forceinline__ int wg_excl_scan(int v, int *wave_tot) {
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
}  // namespace

// ------------------------------------------------------------------ marks

__global__ void vtok_zero_kernel(int32_t *status) { *status = 0; }

// The checks every pass makes of victim i of head u: false for a victim out
// of the head's length or in a block without an id.
__device__ __forceinline__ bool victim_slot(const VtokArgs &P, int u, int i, int &v) {
  v = P.victims[(size_t)u * P.max_slots + i];
  const int n = P.seq_len[u];
  return v >= 0 && v < n && v < P.max_slots &&
         P.block_table[(size_t)u * P.max_blocks + v / kBlock] >= 0;
}

// Marks take three passes of plain loads and stores (no atomics on the table,
// whose victims crowd into the same words and blocks):
//   claim: a victim that is invalid or already dead sets the status; a live
//          one writes its index into its slot's claim word;
//   clear: the victim whose index the claim word holds clears the byte;
//          another victim of the same slot is a repeat and sets the status;
//   count: the live count of every block holding a victim is recounted from
//          its 16 bytes (the same value from every such victim).
__global__ __launch_bounds__(256) void vtok_claim_kernel(const VtokArgs P) {
  const int u = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
  const int m = P.n_victims[u];
  if (i == 0 && m > P.max_slots) atomicOr(P.status, 1);  // the list holds max_slots entries
  if (i >= m || i >= P.max_slots) return;
  int v;
  const size_t row = (size_t)u * P.max_slots;
  if (!victim_slot(P, u, i, v) || P.live[row + v] == 0) {
    atomicOr(P.status, 1);
    return;
  }
  P.claim[row + v] = i;
}

__global__ __launch_bounds__(256) void vtok_clear_kernel(const VtokArgs P) {
  const int u = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
  if (i >= P.n_victims[u] || i >= P.max_slots) return;
  int v;
  if (!victim_slot(P, u, i, v)) return;
  const size_t at = (size_t)u * P.max_slots + v;
  // a victim that was dead before the call was flagged by the claim pass and
  // wrote no claim: whatever the word holds, clearing its byte changes nothing
  if (P.claim[at] == i) {
    P.live[at] = 0;
  } else {
    atomicOr(P.status, 1);
  }
}

__global__ __launch_bounds__(256) void vtok_count_kernel(const VtokArgs P) {
  const int u = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
  if (i >= P.n_victims[u] || i >= P.max_slots) return;
  int v;
  if (!victim_slot(P, u, i, v)) return;
  const int lb = v / kBlock;
  const uint4 b = ld16(P.live + (size_t)u * P.max_slots + (size_t)lb * kBlock);
  int c = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x = w == 0 ? b.x : w == 1 ? b.y : w == 2 ? b.z : b.w;
#pragma unroll
    for (int q = 0; q < 4; ++q) c += ((x >> (8 * q)) & 0xffu) ? 1 : 0;
  }
  P.block_live[(size_t)u * P.max_blocks + lb] = c;
}

hipError_t launch_vtok_evict(const VtokArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(vtok_zero_kernel, dim3(1), dim3(1), 0, s, a.status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.units == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.max_slots + 255) / 256), (unsigned)a.units);
  hipLaunchKernelGGL(vtok_claim_kernel, grid, dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vtok_clear_kernel, grid, dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vtok_count_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ----------------------------------------------------------- reclamation

// plan record per head: {kind, nsrc, T, D, alloc, live, status}; kind 0 skip
// (bad head), 1 left as it is, 2 wants a plan.  Each thread takes kPlanPer
// consecutive logical blocks per pass; one scan gives every thread the rank
// and token offset of its first candidate.
__global__ __launch_bounds__(kPlanThreads) void vtok_plan_kernel(const VtokArgs P) {
  __shared__ int wave_tot[kPlanThreads / kWave];
  __shared__ int s_alloc, s_live, s_bad, s_tot;
  const int u = blockIdx.x, tid = threadIdx.x;
  const int n = P.seq_len[u];
  int32_t *plan = P.plan + (size_t)u * 8;
  if (n < 0 || n > P.max_slots) {
    if (tid == 0) {
      plan[0] = 0;
      plan[6] = 2;  // status bit
    }
    return;
  }
  const int nb = (n + kBlock - 1) / kBlock;
  const int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  const int32_t *bl = P.block_live + (size_t)u * P.max_blocks;
  if (tid == 0) {
    s_alloc = 0;
    s_live = 0;
    s_bad = 0;
  }
  // the ordered selection of sources: the first max_sources allocated blocks
  // that are not full, the tail excluded
  int32_t *src = P.src + (size_t)u * P.max_sources;
  int32_t *srcoff = P.srcoff + (size_t)u * P.max_sources;
  int k_base = 0, t_base = 0;
  int my_alloc = 0, my_live = 0, my_bad = 0;
  for (int lb0 = 0; lb0 < nb; lb0 += kPlanThreads * kPlanPer) {
    const int first = lb0 + tid * kPlanPer;
    int e[kPlanPer], c[kPlanPer];
    int nc = 0, nt = 0;
#pragma unroll
    for (int q = 0; q < kPlanPer; ++q) {
      const int lb = first + q;
      e[q] = lb < nb ? bt[lb] : -1;
      c[q] = lb < nb ? bl[lb] : 0;
    }
#pragma unroll
    for (int q = 0; q < kPlanPer; ++q) {
      const int lb = first + q;
      if (e[q] >= 0) {
        ++my_alloc;
        my_live += c[q];
        if (e[q] >= P.num_blocks || c[q] < 0 || c[q] > kBlock) my_bad = 1;
      }
      const bool cand = lb < nb - 1 && e[q] >= 0 && c[q] < kBlock;
      nc += cand ? 1 : 0;
      nt += cand ? max(c[q], 0) : 0;
    }
    // candidates (< 2^13 per pass) and their tokens (< 2^16) in one scan
    const int packed = wg_excl_scan((nc << 16) | nt, wave_tot);
    int rank = k_base + (packed >> 16), toff = t_base + (packed & 0xffff);
#pragma unroll
    for (int q = 0; q < kPlanPer; ++q) {
      const int lb = first + q;
      const bool cand = lb < nb - 1 && e[q] >= 0 && c[q] < kBlock;
      if (cand) {
        if (rank < P.max_sources) {
          src[rank] = lb;
          srcoff[rank] = toff;
        }
        ++rank;
        toff += max(c[q], 0);
      }
    }
    if (tid == kPlanThreads - 1) s_tot = packed + ((nc << 16) | nt);  // the pass's totals
    __syncthreads();
    k_base += s_tot >> 16;
    t_base += s_tot & 0xffff;
    __syncthreads();
  }
  if (my_alloc) atomicAdd(&s_alloc, my_alloc);
  if (my_live) atomicAdd(&s_live, my_live);
  if (my_bad) atomicOr(&s_bad, 1);
  __syncthreads();
  if (tid != 0) return;
  const int k = min(k_base, P.max_sources);
  // T counts the first max_sources candidates only
  const int T = k_base > P.max_sources ? srcoff[k - 1] + bl[src[k - 1]] : t_base;
  const int D = (T + kBlock - 1) / kBlock;
  const int alloc = s_alloc, live = s_live;
  plan[4] = alloc;
  plan[5] = live;
  plan[6] = 0;
  if (s_bad) {
    plan[0] = 0;
    plan[6] = 4;
    return;
  }
  // Eq. 1 over the head, in double, against the threshold
  const double F = alloc > 0 ? 1.0 - (double)live / (16.0 * (double)alloc) : 0.0;
  if (!(F > P.theta_f) || k < 2 || D >= k) {
    plan[0] = 1;
    return;
  }
  plan[0] = 2;
  plan[1] = k;
  plan[2] = T;
  plan[3] = D;
}

__global__ __launch_bounds__(kAdmitThreads) void vtok_admit_kernel(const VtokArgs P) {
  extern __shared__ int adm[];  // [units] D (-1: no plan), then [units] destination offsets
  __shared__ int wave_tot[kAdmitThreads / kWave];
  __shared__ int s_tot, s_taken;
  const int U = P.units, tid = threadIdx.x;
  int *dl = adm, *doff = adm + U;
  const int fc = *P.free_count;
  // a list holds at most every block once
  const bool fc_ok = fc >= 0 && fc <= P.free_capacity && fc <= P.num_blocks;
  // D of every head that wants a plan, and its offset if every plan fits
  int dsum = 0;
  for (int u0 = 0; u0 < U; u0 += kAdmitThreads) {
    const int u = u0 + tid;
    int d = -1;
    if (u < U && P.plan[(size_t)u * 8] == 2) d = P.plan[(size_t)u * 8 + 3];
    const int dd = d > 0 ? d : 0;
    const int ex = wg_excl_scan(dd, wave_tot);
    if (u < U) {
      dl[u] = d;
      doff[u] = d >= 0 ? dsum + ex : -1;
    }
    if (tid == kAdmitThreads - 1) s_tot = dsum + ex + dd;
    __syncthreads();
    dsum = s_tot;
    __syncthreads();
  }
  if (tid == 0) {
    int taken = dsum;
    if (!fc_ok) {  // an unusable free count: every plan waits
      for (int u = 0; u < U; ++u)
        if (dl[u] >= 0) doff[u] = -2;
      taken = 0;
    } else if (dsum > fc) {  // first fit in (b, h) order; a head that does not fit is deferred
      taken = 0;
      for (int u = 0; u < U; ++u) {
        const int d = dl[u];
        if (d < 0) continue;
        if (taken + d > fc) {
          doff[u] = -2;
        } else {
          doff[u] = taken;
          taken += d;
        }
      }
    }
    s_taken = taken;
  }
  __syncthreads();
  const int taken = s_taken;
  // push offsets and statistics, heads in order
  long long st[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
  int status = fc_ok ? 0 : 8, pbase = 0;
  for (int u0 = 0; u0 < U; u0 += kAdmitThreads) {
    const int u = u0 + tid;
    int push = 0;
    if (u < U) {
      const int32_t *plan = P.plan + (size_t)u * 8;
      const int kind = plan[0];
      status |= plan[6];
      if (kind != 0) {
        st[6] += plan[5];
        st[7] += plan[4];
        st[8] += plan[4];
      }
      if (kind == 1) st[2] += 1;
      if (kind == 2) {
        if (doff[u] == -2) {
          st[1] += 1;
        } else {
          push = plan[1];
          st[0] += 1;
          st[3] += plan[1] - plan[3];
          st[4] += plan[2];
          st[8] -= plan[1] - plan[3];
        }
      }
      P.dst_off[u] = kind == 2 ? doff[u] : -1;
    }
    const int ex = wg_excl_scan(push, wave_tot);
    if (u < U) P.push_off[u] = pbase + ex;
    if (tid == kAdmitThreads - 1) s_tot = pbase + ex + push;  // running total
    __syncthreads();
    pbase = s_tot;
    __syncthreads();
  }
  // workgroup sums of the statistics (fixed order)
  __shared__ long long s_st[9][kAdmitThreads / kWave];
  __shared__ int s_status[kAdmitThreads / kWave];
#pragma unroll
  for (int c = 0; c < 9; ++c) {
    long long v = st[c];
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    if (lane_id() == 0) s_st[c][tid / kWave] = v;
  }
  int sv = status;
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) sv |= __shfl_xor(sv, o);
  if (lane_id() == 0) s_status[tid / kWave] = sv;
  __syncthreads();
  if (tid == 0) {
    long long tot[9];
    int stat = 0;
    for (int c = 0; c < 9; ++c) {
      tot[c] = 0;
      for (int w = 0; w < kAdmitThreads / kWave; ++w) tot[c] += s_st[c][w];
    }
    for (int w = 0; w < kAdmitThreads / kWave; ++w) stat |= s_status[w];
    // a list that cannot hold the returned sources (block ids shared between
    // the tables and the list): the pushes past its capacity are dropped
    const long long end = (long long)(fc_ok ? fc : 0) - taken + pbase;
    if (end > P.free_capacity) stat |= 8;
    for (int c = 0; c < 9; ++c) P.stats[c] = tot[c];
    P.stats[5] = tot[4] * 2 * P.row_bytes * 2;
    P.stats[9] = stat;
    P.misc[0] = fc_ok ? fc : 0;
    P.misc[1] = taken;
    if (fc_ok) *P.free_count = (int32_t)min(end, (long long)P.free_capacity);
  }
}

// A wave per source block: its live rows (K and V) go to consecutive rows of
// the destinations, destination d of a head being free_list[top - 1 - off - d]
// (nothing writes the list until the apply step); positions and scores are
// staged by their place among the moved tokens, and the wave of source
// position j < D records that position's destination id.
__global__ __launch_bounds__(kMoveWaves * kWave) void vtok_move_kernel(const VtokArgs P) {
  const int u = blockIdx.y;
  const int off = P.dst_off[u];
  if (off < 0) return;  // not reclaimed
  const int k = P.plan[(size_t)u * 8 + 1], T = P.plan[(size_t)u * 8 + 2];
  const int D = P.plan[(size_t)u * 8 + 3];
  const int l = lane_id(), pieces = P.row_bytes / 16;
  const size_t urow = (size_t)u * P.max_slots;
  const size_t tbase = (size_t)u * P.max_sources * kBlock;
  const int32_t *dst = P.free_list + (P.misc[0] - 1 - off);  // dst[-d]: destination d
  for (int j = blockIdx.x * kMoveWaves + (int)(threadIdx.x / kWave); j < k;
       j += (int)gridDim.x * kMoveWaves) {
    const int lb = P.src[(size_t)u * P.max_sources + j];
    const int i0 = P.srcoff[(size_t)u * P.max_sources + j];  // first moved index of this block
    const int from_blk = P.block_table[(size_t)u * P.max_blocks + lb];
    if (l == 0 && j < D) P.dstw[(size_t)u * P.max_sources + j] = dst[-j];
    const bool mine = l < kBlock && P.live[urow + (size_t)lb * kBlock + l] != 0;
    const uint64_t mask = __ballot(mine);
    const int c = __popcll(mask);
    const int rank = __popcll(mask & ((1ull << l) - 1));
    if (mine && i0 + rank < T) {  // (always, when the live counts match the marks)
      P.tpos[tbase + i0 + rank] = P.pos[urow + (size_t)lb * kBlock + l];
      if (P.score) P.tscore[tbase + i0 + rank] = P.score[urow + (size_t)lb * kBlock + l];
    }
    // lane r < c learns the offset of the r-th live slot
    const int o_of_rank = __builtin_amdgcn_ds_permute((mine ? rank : (l | 32)) * 4, l);
    const int n16 = c * pieces;  // 16-byte pieces per pool
    for (int t0 = 0; t0 < 2 * n16; t0 += 4 * kWave) {
      uint4 v[4];
      size_t to[4];
      uint8_t *pool[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + q * kWave + l;
        const int which = t >= n16 ? 1 : 0;
        const int rem = t - which * n16;
        const int r = rem / pieces, p = rem - r * pieces;
        const int o = __shfl(o_of_rank, r < kBlock ? r : 0);
        pool[q] = which ? P.v_pool : P.k_pool;
        to[q] = kNoRow;
        if (t < 2 * n16 && i0 + r < T) {
          const int i = i0 + r;
          const int to_blk = dst[-(i / kBlock)];
          to[q] = (((size_t)to_blk * kBlock + i % kBlock) * P.row_bytes) + (size_t)p * 16;
          v[q] = ld16(pool[q] + ((size_t)from_blk * kBlock + o) * P.row_bytes + (size_t)p * 16);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (to[q] != kNoRow) st16_nt(pool[q] + to[q], v[q]);
    }
  }
}

// The per-slot table and the block list of the source positions; the sources
// go to the free list.  Runs after every copy, so no slot is read after it is
// rewritten.  A thread takes four consecutive slots of one source position.
__global__ __launch_bounds__(256) void vtok_apply_kernel(const VtokArgs P) {
  const int u = blockIdx.y;
  const int off = P.dst_off[u];
  if (off < 0) return;
  const int32_t *plan = P.plan + (size_t)u * 8;
  const int k = plan[1], T = plan[2], D = plan[3];
  const size_t urow = (size_t)u * P.max_slots;
  const size_t tbase = (size_t)u * P.max_sources * kBlock;
  int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  const int32_t *src = P.src + (size_t)u * P.max_sources;
  const int base = P.misc[0] - P.misc[1] + P.push_off[u];  // where this head's sources go
  for (int x = blockIdx.x * 256 + (int)threadIdx.x; x < k * (kBlock / 4);
       x += (int)gridDim.x * 256) {
    const int j = x / (kBlock / 4), o4 = (x % (kBlock / 4)) * 4;
    const int lb = src[j];
    // the first D source positions take the moved tokens in order
    const int cnt = j < D ? min(kBlock, T - kBlock * j) : 0;
    const size_t s = urow + (size_t)lb * kBlock + o4;
    uint32_t lw = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) lw |= (o4 + q < cnt ? 1u : 0u) << (8 * q);
    *reinterpret_cast<uint32_t *>(P.live + s) = lw;
    const size_t t = tbase + (size_t)kBlock * j + o4;
    if (o4 + 4 <= cnt) {
      *reinterpret_cast<int4 *>(P.pos + s) = *reinterpret_cast<const int4 *>(P.tpos + t);
      if (P.score)
        *reinterpret_cast<float4 *>(P.score + s) = *reinterpret_cast<const float4 *>(P.tscore + t);
    } else {
      for (int q = 0; q < 4 && o4 + q < cnt; ++q) {
        P.pos[s + q] = P.tpos[t + q];
        if (P.score) P.score[s + q] = P.tscore[t + q];
      }
    }
    if (o4 == 0) {
      if (base + j < P.free_capacity) P.free_list[base + j] = bt[lb];
      bt[lb] = j < D ? P.dstw[(size_t)u * P.max_sources + j] : -1;
      P.block_live[(size_t)u * P.max_blocks + lb] = cnt;
    }
  }
}

hipError_t launch_vtok_reclaim(const VtokArgs &a, hipStream_t s) {
  if (a.units == 0) return hipSuccess;
  hipLaunchKernelGGL(vtok_plan_kernel, dim3((unsigned)a.units), dim3(kPlanThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t adm_lds = (size_t)a.units * 2 * sizeof(int);
  if (adm_lds > 49152) {  // idempotent: set on every such launch, no cached state
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(vtok_admit_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)adm_lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(vtok_admit_kernel, dim3(1), dim3(kAdmitThreads), adm_lds, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // source blocks of a head: a wave each, striding when there are many
  const unsigned move_x = (unsigned)std::min((a.max_sources + kMoveWaves - 1) / kMoveWaves, 256);
  hipLaunchKernelGGL(vtok_move_kernel, dim3(move_x, (unsigned)a.units), dim3(kMoveWaves * kWave), 0,
                     s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned apply_x = (unsigned)std::min((a.max_sources * (kBlock / 4) + 255) / 256, 64);
  hipLaunchKernelGGL(vtok_apply_kernel, dim3(apply_x, (unsigned)a.units), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------- sync_new_tokens and slot mapping

// [VTOK] section 3.2, sync_new_tokens: the slots [seq_len, new_len) of a head
// become live at sequential positions; each block's live count grows by its
// new slots.  One workgroup per head.
__global__ __launch_bounds__(256) void vtok_sync_kernel(const VtokArgs P) {
  __shared__ int s_bad;
  const int u = blockIdx.x, b = u / P.Hkv, tid = threadIdx.x;
  const int n = P.seq_len[u], m = P.new_len[u];
  if (n < 0 || m < n || m > P.max_slots) {
    if (tid == 0) P.status[u] = -2;
    return;
  }
  const int32_t *bt = P.block_table + (size_t)u * P.max_blocks;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  const int lb0 = n / kBlock, lb1 = (m + kBlock - 1) / kBlock;  // blocks touched
  for (int lb = lb0 + tid; lb < lb1; lb += 256) {
    const int e = bt[lb];
    if (e < 0 || e >= P.num_blocks) s_bad = 1;
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0) P.status[u] = -4;
    return;
  }
  const size_t urow = (size_t)u * P.max_slots;
  const int p0 = P.pos0[b];
  for (int s = n + tid; s < m; s += 256) {
    P.live[urow + s] = 1;
    P.pos[urow + s] = p0 + (s - n);
  }
  for (int lb = lb0 + tid; lb < lb1; lb += 256)
    P.block_live[(size_t)u * P.max_blocks + lb] += min(m, (lb + 1) * kBlock) - max(n, lb * kBlock);
  if (tid == 0) {
    P.seq_len[u] = m;
    P.status[u] = 0;
  }
}

hipError_t launch_vtok_sync(const VtokArgs &a, hipStream_t s) {
  if (a.units == 0) return hipSuccess;
  hipLaunchKernelGGL(vtok_sync_kernel, dim3((unsigned)a.units), dim3(256), 0, s, a);
  return hipGetLastError();
}

// [VTOK] Algorithm 1, step 4, and Eq. 2: every live token's physical slot
// (block id * 16 + offset) and position, in logical order.  Two launches over
// chunks of kMapChunk slots of every head: the live count of each chunk, then
// each chunk's offset (the counts before it) and block-wide scans that rank
// its live slots, 1024 at a time.
constexpr int kMapThreads = 1024;
constexpr int kMapChunk = 4 * kMapThreads;

__device__ __forceinline__ bool map_live(const VtokArgs &P, int u, int s, int n, int &e) {
  e = -1;
  if (s >= n) return false;
  e = P.block_table[(size_t)u * P.max_blocks + s / kBlock];
  return e >= 0 && e < P.num_blocks && P.live[(size_t)u * P.max_slots + s] != 0;
}

__global__ __launch_bounds__(kMapThreads) void vtok_map_count_kernel(const VtokArgs P) {
  __shared__ int s_cnt[kMapThreads / kWave];
  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int n = P.seq_len[u];
  if (n < 0 || n > P.max_slots || c * kMapChunk >= n) return;
  int w = 0;
#pragma unroll
  for (int q = 0; q < kMapChunk / kMapThreads; ++q) {
    int e;
    w += __popcll(__ballot(map_live(P, u, c * kMapChunk + q * kMapThreads + tid, n, e)));
  }
  if (lane_id() == 0) s_cnt[tid / kWave] = w;
  __syncthreads();
  if (tid == 0) {
    int t = 0;
    for (int q = 0; q < kMapThreads / kWave; ++q) t += s_cnt[q];
    P.map_chunk[(size_t)u * P.map_chunks + c] = t;
  }
}

__global__ __launch_bounds__(kMapThreads) void vtok_map_write_kernel(const VtokArgs P) {
  __shared__ int wave_tot[kMapThreads / kWave];
  __shared__ int s_tot;
  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int n = P.seq_len[u];
  if (n < 0 || n > P.max_slots) {
    if (c == 0 && tid == 0) P.map_count[u] = -1;
    return;
  }
  const int chunks = (n + kMapChunk - 1) / kMapChunk;
  if (n == 0 && c == 0 && tid == 0) P.map_count[u] = 0;
  if (c >= chunks) return;
  // the live slots of the chunks before this one: a strided sum, reduced
  // over the workgroup
  const int32_t *cnt = P.map_chunk + (size_t)u * P.map_chunks;
  int own = 0;
  for (int q = tid; q < c; q += kMapThreads) own += cnt[q];
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) own += __shfl_xor(own, o);
  if (lane_id() == 0) wave_tot[tid / kWave] = own;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < kMapThreads / kWave; ++w) base += wave_tot[w];
  __syncthreads();  // wave_tot is the scans' next
  const size_t urow = (size_t)u * P.max_slots;
  for (int q = 0; q < kMapChunk / kMapThreads; ++q) {
    int e;
    const int s = c * kMapChunk + q * kMapThreads + tid;
    const bool ok = map_live(P, u, s, n, e);
    const int rank = wg_excl_scan(ok ? 1 : 0, wave_tot);
    if (ok) {
      P.map_slots[urow + base + rank] = e * kBlock + s % kBlock;  // Eq. 2
      P.map_pos[urow + base + rank] = P.pos[urow + s];
    }
    if (tid == kMapThreads - 1) s_tot = base + rank + (ok ? 1 : 0);
    __syncthreads();
    base = s_tot;
    __syncthreads();
  }
  if (c == chunks - 1 && tid == 0) P.map_count[u] = base;
}

hipError_t launch_vtok_slot_mapping(const VtokArgs &a, hipStream_t s) {
  if (a.units == 0) return hipSuccess;
  const dim3 grid((unsigned)a.map_chunks, (unsigned)a.units);
  hipLaunchKernelGGL(vtok_map_count_kernel, grid, dim3(kMapThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vtok_map_write_kernel, grid, dim3(kMapThreads), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------- online checks (I1, I2)

namespace {
constexpr uint64_t kGold = 0x9E3779B97F4A7C15ull;

// MurmurHash3's 64-bit finalizer (Appleby): xor-shift 33, multiply, twice.
__device__ __forceinline__ uint64_t fmix64(uint64_t k) {
  k ^= k >> 33;
  k *= 0xff51afd7ed558ccdull;
  k ^= k >> 33;
  k *= 0xc4ceb9fe1a85ec53ull;
  k ^= k >> 33;
  return k;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) v += (uint64_t)__shfl_xor((unsigned long long)v, o);
  return v;
}
}  // namespace

// Waves stride over a head's logical blocks.  Per block: the live slots'
// ranks by ballot, then four live tokens at a time, 16 lanes each; a lane
// finalizes its share of the token's 64-bit words (K words keyed 2i+1, V
// words 2i+2, times the golden-ratio constant), the 16 lanes sum, and the
// token's finalized sum joins the head's digest, a commutative integer sum
// (any order gives the same value).  One atomic per workgroup: a head's
// workgroups are few, so its digest word sees few atomics.
constexpr int kDigestWaves = 8;
constexpr int kDigestParts = 64;  // workgroups per head at most
__global__ __launch_bounds__(kDigestWaves * kWave) void vtok_digest_kernel(const VtokArgs P,
                                                                         uint64_t *digest) {
  __shared__ uint64_t part[kDigestWaves];
  const int u = blockIdx.y, l = lane_id(), wv = (int)(threadIdx.x / kWave);
  const int n = min(max(P.seq_len[u], 0), P.max_slots);
  const int nb = (n + kBlock - 1) / kBlock;
  const size_t urow = (size_t)u * P.max_slots;
  const int nw = P.row_bytes / 8, g = l / 16, gl = l % 16;
  uint64_t acc = 0;
  for (int lb = blockIdx.x * kDigestWaves + wv; lb < nb; lb += (int)gridDim.x * kDigestWaves) {
    const int e = P.block_table[(size_t)u * P.max_blocks + lb];
    if (e < 0 || e >= P.num_blocks) continue;
    const int slot = lb * kBlock + l;
    const bool mine = l < kBlock && slot < n && P.live[urow + slot] != 0;
    const uint64_t mask = __ballot(mine);
    const int c = __popcll(mask);
    const int rank = __popcll(mask & ((1ull << l) - 1));
    const int o_of_rank = __builtin_amdgcn_ds_permute((mine ? rank : (l | 32)) * 4, l);
    for (int r0 = 0; r0 < c; r0 += 4) {
      const int r = r0 + g;
      const int o = __shfl(o_of_rank, r < kBlock ? r : 0);
      uint64_t t = 0;
      if (r < c) {
        const size_t row = ((size_t)e * kBlock + o) * P.row_bytes;
        for (int w = gl; w < 2 * nw; w += 16) {
          const bool is_k = w < nw;
          const int i = is_k ? w : w - nw;
          const uint64_t x =
              *reinterpret_cast<const uint64_t *>((is_k ? P.k_pool : P.v_pool) + row + (size_t)i * 8);
          t += fmix64(x ^ ((uint64_t)(is_k ? 2 * i + 1 : 2 * i + 2) * kGold));
        }
      }
#pragma unroll
      for (int x = 8; x >= 1; x >>= 1) t += (uint64_t)__shfl_xor((unsigned long long)t, x);
      if (gl == 0 && r < c)
        acc += fmix64(t + fmix64((uint64_t)(uint32_t)P.pos[urow + lb * kBlock + o] ^ kGold));
    }
  }
  acc = wave_sum_u64(acc);
  if (l == 0) part[wv] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t sum = 0;
    for (int w = 0; w < kDigestWaves; ++w) sum += part[w];
    if (sum != 0) atomicAdd((unsigned long long *)(digest + u), (unsigned long long)sum);
  }
}

__global__ void vtok_fill_kernel(uint64_t *p, size_t n64) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n64;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

hipError_t launch_vtok_digest(const VtokArgs &a, uint64_t *digest, hipStream_t s) {
  hipLaunchKernelGGL(vtok_fill_kernel, dim3((unsigned)std::min((a.units + 255) / 256, 1024)),
                     dim3(256), 0, s, digest, (size_t)a.units);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.units == 0) return e;
  const int parts = std::min((a.max_blocks + kDigestWaves - 1) / kDigestWaves, kDigestParts);
  hipLaunchKernelGGL(vtok_digest_kernel, dim3((unsigned)parts, (unsigned)a.units),
                     dim3(kDigestWaves * kWave), 0, s, a, digest);
  return hipGetLastError();
}

// I2 and the live counts: every table entry and free-list entry adds one to
// its block's holder count (integer atomics); then a pass over the pool.
// out[4] = {held more than once, held by nobody, out of range, count
// mismatches}.
__global__ __launch_bounds__(256) void vtok_check_table_kernel(const VtokArgs P, int32_t *held,
                                                               int64_t *out) {
  const int u = blockIdx.y, lb = blockIdx.x * 256 + threadIdx.x;
  int bad = 0, mis = 0;
  if (lb < P.max_blocks) {
    const int e = P.block_table[(size_t)u * P.max_blocks + lb];
    if (e >= 0) {
      if (e < P.num_blocks) {
        atomicAdd(held + e, 1);
      } else {
        bad = 1;
      }
      const uint4 b = ld16(P.live + (size_t)u * P.max_slots + (size_t)lb * kBlock);
      int c = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = w == 0 ? b.x : w == 1 ? b.y : w == 2 ? b.z : b.w;
#pragma unroll
        for (int q = 0; q < 4; ++q) c += ((x >> (8 * q)) & 0xffu) ? 1 : 0;
      }
      mis = c != P.block_live[(size_t)u * P.max_blocks + lb] ? 1 : 0;
    }
  }
  const uint64_t bb = __ballot(bad), mm = __ballot(mis);
  if (lane_id() == 0) {
    if (bb) atomicAdd((unsigned long long *)(out + 2), (unsigned long long)__popcll(bb));
    if (mm) atomicAdd((unsigned long long *)(out + 3), (unsigned long long)__popcll(mm));
  }
}

__global__ __launch_bounds__(256) void vtok_check_list_kernel(const VtokArgs P, int32_t *held,
                                                              int64_t *out) {
  const int fc_raw = *P.free_count;
  const int fc = min(max(fc_raw, 0), P.free_capacity);
  const int i = blockIdx.x * 256 + threadIdx.x;
  int bad = 0;
  if (i < fc) {
    const int e = P.free_list[i];
    if (e >= 0 && e < P.num_blocks) {
      atomicAdd(held + e, 1);
    } else {
      bad = 1;
    }
  }
  if (i == 0 && fc != fc_raw) bad = 1;  // a count outside [0, capacity]
  const uint64_t bb = __ballot(bad);
  if (lane_id() == 0 && bb)
    atomicAdd((unsigned long long *)(out + 2), (unsigned long long)__popcll(bb));
}

__global__ __launch_bounds__(256) void vtok_check_pool_kernel(const VtokArgs P,
                                                              const int32_t *held, int64_t *out) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  const int h = b < P.num_blocks ? held[b] : 1;
  const uint64_t twice = __ballot(h > 1), none = __ballot(h == 0);
  if (lane_id() == 0) {
    if (twice) atomicAdd((unsigned long long *)(out + 0), (unsigned long long)__popcll(twice));
    if (none) atomicAdd((unsigned long long *)(out + 1), (unsigned long long)__popcll(none));
  }
}

hipError_t launch_vtok_check(const VtokArgs &a, int32_t *held, int64_t *out, hipStream_t s) {
  hipLaunchKernelGGL(vtok_fill_kernel, dim3(1), dim3(64), 0, s, reinterpret_cast<uint64_t *>(out),
                     (size_t)4);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n64 = ((size_t)a.num_blocks + 1) / 2;  // the holder counts, as 64-bit words
  hipLaunchKernelGGL(vtok_fill_kernel, dim3((unsigned)std::min<size_t>((n64 + 255) / 256, 4096)),
                     dim3(256), 0, s, reinterpret_cast<uint64_t *>(held), n64);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vtok_check_table_kernel,
                     dim3((unsigned)((a.max_blocks + 255) / 256), (unsigned)a.units), dim3(256), 0,
                     s, a, held, out);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vtok_check_list_kernel, dim3((unsigned)((a.free_capacity + 255) / 256)),
                     dim3(256), 0, s, a, held, out);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vtok_check_pool_kernel, dim3((unsigned)((a.num_blocks + 255) / 256)),
                     dim3(256), 0, s, a, held, out);
  return hipGetLastError();
}

}  // namespace kvev
